// Single-token grouped-query decode over a contiguous or paged KV cache, for
// gfx950.
//
// What is computed ("Grouped Query Attention (GQA)" glossary, sections "Cómo
// funciona GQA" and "Por qué GQA reduce la caché KV"): each sequence's new
// query token attends, head by head, to every valid cached key/value of its
// KV group.  The whole valid cache is read once per token, so the kernel is
// bound by HBM bandwidth and its traffic scales with Hkv, not Hq.
//
// With a RoPE theta the split pass first rotates each query head at position
// len - 1 (the same device code as the stand-alone RoPE kernel, so the fused
// and unfused paths agree bit for bit), saving a launch per decode step.
// Split pass: the launch has a fixed budget of workgroups (about two per
// compute unit when there are many (sequence, KV head [, 16-head slice])
// groups, fewer and longer streams when there are few).  Every workgroup reads
// the batch's lengths and derives the same split: each group of n 32-token
// sub-tiles gets ceil(n / U) workgroups, with U the smallest size (at least
// 16) that keeps the total within the budget, so ragged batches give
// workgroups of nearly equal work and all of them run at once.  Sub-tile j of
// a group goes to its workgroup j % nwg and, inside it, to wave (j / nwg) % 4,
// so a group's workgroups read one contiguous front of the cache.  Each byte
// of K and V is read once and serves all G query heads of the group.
// Per sub-tile:
//   * K rows are loaded straight from HBM into matrix-core operand registers
//     (16-byte loads; a wave instruction covers 16 rows x 64 contiguous bytes)
//     and S^T = K Q^T is one 16x16x32 bf16 product per 16 tokens x 32 dims,
//     with the group's query heads (padded to 16) as the N dimension;
//   * V rows are copied (16-byte loads, whole rows per lane group) into the
//     wave's own LDS slot and read back with the LDS transpose read as the A
//     operand of O^T = V^T P^T, P taken from registers as bf16.  These copies
//     carry the non-temporal cache policy: V bytes are read once per step, and
//     the hint lifts the stream rate by 7 to 9% on MI355X (K loads with the
//     same hint are slower, so they keep the default policy);
//   * the softmax is online in fp32 (exp2 domain), one query head per lane.
// The four waves then merge in LDS.  A sequence with a single split workgroup
// writes its bf16 output right there.  Otherwise each workgroup writes one
// unnormalised partial (max, sum, o[D]) per head to the fp32 workspace and
// tags it; a workgroup that finds every partial of its (sequence, KV head,
// head slice) tagged by this call combines them (log-sum-exp rescaling) and
// writes the output, so one launch does the whole step.  That merge ends the
// launch, so it is built for latency: a block of partials costs one memory
// round trip, and each head's statistics come from DPP row reductions rather
// than chained lane shuffles.  Cache slots at or past a
// sequence's length never reach the result: loads of rows past it re-read the
// last valid row (row 0 of an empty sequence) and their scores are masked.
//
// Paged caches (same glossary, section "GQA y técnicas relacionadas":
// PagedAttention's fixed-size blocks, and sliding-window attention) use the
// same kernel, instantiated with PAGED: a sub-tile's 32 rows never straddle a
// page (page sizes are multiples of 32), so only the row base changes, taken
// from the sequence's block-table entry, which each wave fetches one sub-tile
// ahead so the lookup's latency stays off the load path.  A window of w tokens
// starts the sequence's sub-tiles at the one holding token len - w and masks
// the keys before it; the split counts only the sub-tiles a query sees.  The
// contiguous instantiation compiles all of this out.
#include <algorithm>
#include <chrono>

#include "../../include/attn.h"
#include "common.hpp"
#include "kernels.hpp"

// Scratch of the allocation-free decode entry point (attn_decode_noalloc): the
// split pass's partial results, call tags and epochs, in a static array that
// each device holds from the library's load to the end of the process.  Host
// code never uses its name as an address (on the host it names a stand-in,
// not device memory): the device address is looked up per device with
// hipGetSymbolAddress and passed to the kernel as its workspace.
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_SCRATCH_BYTES];

namespace attn {

namespace {

constexpr int DC_NW = 4;      // waves per split workgroup
constexpr int DC_SUB = 32;    // tokens per wave sub-tile
constexpr int DC_HEADS = 16;  // query heads per split workgroup (MFMA N)
constexpr int DC_V_POLICY = 2;  // cache policy of the V copies: nt (non-temporal)

// Smallest number of sub-tiles one split workgroup is given: it bounds the
// split workgroups (partial results) of a group, ceil(n_sub / DC_UMIN), and so
// the workspace.
constexpr int DC_UMIN = 16;

__host__ __device__ inline int decode_max_partials(int max_len) {
    return max(1, ceil_div(ceil_div(max_len, DC_SUB), DC_UMIN));
}

// ceil(n / u) for 0 <= n < 2^30, 0 < u, given r ~ 1/u in float: the float
// quotient is within a few units of the answer, and integer steps settle it.
__device__ inline int ceil_div_est(int n, int u, float r) {
    int q = (int)((float)n * r);
    while ((long long)q * u < n) ++q;
    while (q > 0 && (long long)(q - 1) * u >= n) --q;
    return q;
}

// Wave-wide integer sum and inclusive prefix sum with data-parallel
// primitives (lane moves inside 16-lane rows, then row swaps or row
// broadcasts), avoiding the LDS round trips of general shuffles.
// dpp_add(x, ctrl, rows): x plus the lane value `ctrl` selects, in the rows
// of the `rows` mask (other rows add nothing).
template <int CTRL, int ROWS = 0xF>
__device__ inline int dpp_add(int x) {
    return x + __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, false);
}
__device__ inline int wave_sum(int x) {
    x = dpp_add<0xB1>(x);   // quad permutation: + lane ^ 1
    x = dpp_add<0x4E>(x);   // quad permutation: + lane ^ 2 (quad totals)
    x = dpp_add<0x124>(x);  // row rotate by 4: + a neighbouring quad
    x = dpp_add<0x128>(x);  // row rotate by 8: row totals
    const auto a = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    x = (int)(a[0] + a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return (int)(b[0] + b[1]);
}
// Max and sum over each 16-lane row (every lane of the row gets the result);
// all lanes of the wave must be active.
template <int CTRL>
__device__ inline float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ inline float row16_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));
    x = fmaxf(x, dpp_f<0x4E>(x));
    x = fmaxf(x, dpp_f<0x124>(x));
    return fmaxf(x, dpp_f<0x128>(x));
}
__device__ inline float row16_sum(float x) {
    x += dpp_f<0xB1>(x);
    x += dpp_f<0x4E>(x);
    x += dpp_f<0x124>(x);
    return x + dpp_f<0x128>(x);
}
__device__ inline int wave_inclusive_scan(int x) {
    x = dpp_add<0x111>(x);  // row shift right by 1, 2, 4, 8: prefix sums within rows
    x = dpp_add<0x112>(x);
    x = dpp_add<0x114>(x);
    x = dpp_add<0x118>(x);
    x = dpp_add<0x142, 0xA>(x);  // lane 15 of rows 0 and 2 into rows 1 and 3
    x = dpp_add<0x143, 0xC>(x);  // lane 31 into rows 2 and 3
    return x;
}

// Device-coherent (agent-scope) float accesses for the split partials.
__device__ inline void store_agent(float* p, float x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float load_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte device-coherent load and store (sc1: the per-XCD L2's non-coherent
// lines are bypassed) through a buffer resource, one instruction where 8- or
// 4-byte atomic accesses would take two or four
__device__ inline f32x4_t load4_coherent(__amdgpu_buffer_rsrc_t rs, int byte_off) {
    return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 16));
}
__device__ inline void store4_coherent(f32x4_t x, __amdgpu_buffer_rsrc_t rs, int byte_off) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), rs, byte_off, 0, 16);
}

template <int D>
struct DecodeSmem {
    // one V sub-tile slot per wave, in each of two arrays
    static constexpr int kSlots = DC_NW * DC_SUB * D * 2;
};

// Where the cached keys/values live.  Contiguous: k, v [B, Hkv, S_cap, D].
// Paged: k, v [num_pages, Hkv, page, D], and token t of sequence b is row
// t % page of page table[b * max_pages + t / page] ("GQA y técnicas
// relacionadas": PagedAttention's fixed-size blocks).  window > 0 limits each
// query to the last `window` tokens (sliding-window attention, same section).
struct DecodeCache {
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* table;
    int S_cap;
    int page, max_pages, num_pages;
    int window;
};

// First token a query of a sequence of len tokens sees, and the number of
// 32-token sub-tiles from the one holding it to the end.
__device__ inline int decode_first_token(int len, int window) {
    return window > 0 ? max(0, len - window) : 0;
}
__device__ inline int decode_subtiles(int len, int window) {
    return ceil_div(len, DC_SUB) - decode_first_token(len, window) / DC_SUB;
}

// s_waitcnt immediates: vmcnt(n) alone, and lgkmcnt(0) alone
constexpr int wait_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }
constexpr int kWaitLgkm0 = 0xC07F;

template <int D, bool PAGED>
__global__ __launch_bounds__(DC_NW * 64, 2) void decode_split_kernel(
    const uint16_t* __restrict__ q, DecodeCache cache, const int32_t* __restrict__ seqlens,
    float* __restrict__ ws_o, float* __restrict__ ws_ml, unsigned long long* __restrict__ ws_tag,
    unsigned long long* __restrict__ ws_epoch, uint16_t* __restrict__ o, int Hq, int Hkv, int max_len, int NC, float c, int n_hchunk,
    int rope, RopeFreqs fr, unsigned long long tag, int B, int budget) {
    constexpr int KSTEPS = D / 32, DT = D / 16;
    constexpr int ROW = D * 2;                 // bytes per cache row
    constexpr int VSUB = DC_SUB * ROW;         // bytes of one V sub-tile
    constexpr int VINST = VSUB / 1024;         // 1 KiB LDS-DMA instructions per sub-tile
    constexpr int RPI = 1024 / ROW;            // rows per DMA instruction
    // V slots: two arrays (the compiler then sees that the slot being filled is
    // not the one being read); after the loop the first holds the waves'
    // partial o vectors and, in the final merge, the partials' factors and sums.
    __shared__ __attribute__((aligned(1024))) char vs0[DecodeSmem<D>::kSlots];
    __shared__ __attribute__((aligned(1024))) char vs1[DecodeSmem<D>::kSlots];
    __shared__ float sstat[2 * DC_NW * DC_HEADS];  // waves' max and sum; then running stats

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int window = PAGED ? cache.window : 0;  // the contiguous entry point has none

    // ---- this workgroup's (sequence b, group gi, split chunk of nwg).  Groups
    // are numbered b-major (GPB per sequence), their workgroups consecutively.
    const int GPB = Hkv * n_hchunk;
    int b, gi, chunk, nwg, len;
    if ((long long)B * GPB >= budget) {  // one workgroup per group fills the budget
        b = (int)blockIdx.x / GPB;
        gi = (int)blockIdx.x % GPB;
        chunk = 0;
        nwg = 1;
        if (b >= B) return;
        len = min(max(seqlens[b], 0), max_len);
    } else {
        // B < budget: each wave stages the sequences' lengths in its own
        // second V slot, which only it fills later (an empty sequence still
        // gets one workgroup, which writes its zero rows)
        int* const ls = (int*)(vs1 + w * VSUB);
        for (int i = lane; i < B; i += 64) ls[i] = min(max(seqlens[i], 0), max_len);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        auto ns = [&](int i) { return decode_subtiles(ls[i], window); };
        // every wave finds the same U, a size whose workgroup count fits the
        // budget.  With T = GPB * sum(n), count(U) is about T / U + GPB * B / 2
        // (half a workgroup of rounding per group); start there and grow U
        // until the count fits (at n_sub_max it is B * GPB < budget).
        auto count = [&](int U) {
            const float r = 1.f / (float)U;
            int n = 0;
            for (int i = lane; i < B; i += 64) n += max(1, ceil_div_est(ns(i), U, r));
            return wave_sum(n) * GPB;
        };
        int tot = 0;  // the cache holds every counted token, so this fits
        for (int i = lane; i < B; i += 64) tot += ns(i);
        const long long T = (long long)wave_sum(tot) * GPB;
        const int n_sub_max = max(DC_UMIN, ceil_div(max_len, DC_SUB));
        const long long room = budget - (long long)GPB * B / 2;  // > budget / 2
        int U = (int)min<long long>(n_sub_max, max<long long>(DC_UMIN, ceil_div(T, room)));
        while (U < n_sub_max && count(U) > budget) U = min(n_sub_max, U + max(1, U >> 3));
        // locate this workgroup: prefix sums of the sequences' workgroup counts
        b = -1;
        int first = 0;  // first workgroup of sequence b
        const float rU = 1.f / (float)U;
        for (int i0 = 0, base = 0; i0 < B; i0 += 64) {
            const int i = i0 + lane;
            const int v = i < B ? GPB * max(1, ceil_div_est(ns(i), U, rU)) : 0;
            const int incl = wave_inclusive_scan(v);
            const int p = (int)blockIdx.x - base;
            const unsigned long long hit = __ballot(v > 0 && p >= incl - v && p < incl);
            if (hit) {
                const int l = __builtin_ctzll(hit);
                b = i0 + l;
                first = base + __builtin_amdgcn_readlane(incl - v, l);
                break;
            }
            base += __builtin_amdgcn_readlane(incl, 63);
        }
        if (b < 0) return;  // past the last group's workgroups (uniform)
        len = ls[b];
        nwg = max(1, ceil_div_est(decode_subtiles(len, window), U, rU));
        const int off = (int)blockIdx.x - first;
        gi = off / nwg;
        chunk = off % nwg;
    }
    b = __builtin_amdgcn_readfirstlane(b);
    gi = __builtin_amdgcn_readfirstlane(gi);
    chunk = __builtin_amdgcn_readfirstlane(chunk);
    nwg = __builtin_amdgcn_readfirstlane(nwg);
    len = __builtin_amdgcn_readfirstlane(len);
    const int kvh = gi / n_hchunk, hc = gi % n_hchunk;
    const int G = Hq / Hkv;
    const int h0 = kvh * G + hc * DC_HEADS;
    const int GH = min(DC_HEADS, G - hc * DC_HEADS);
    const int n_sub = ceil_div(len, DC_SUB);  // 32-token sub-tiles of this sequence
    const int w0 = decode_first_token(len, window);  // first token the query sees
    const int s0 = w0 / DC_SUB;                             // and its sub-tile

    const int lr = lane & 15, lg = lane >> 4;

    const size_t kvb = PAGED ? 0 : (size_t)(b * Hkv + kvh) * cache.S_cap * D;
    const uint16_t* const kg = cache.k + kvb;
    const uint16_t* const vg = cache.v + kvb;
    char* const slot0 = vs0 + w * VSUB;  // this wave's two V slots
    char* const slot1 = vs1 + w * VSUB;

    // The V sub-tile goes straight from HBM into this wave's LDS slot (no
    // registers): DMA instruction u puts lane l's 16 bytes at byte
    // u*1024 + 16l of the slot, i.e. row RPI*u + l/(ROW/16), physical chunk
    // l % (ROW/16) of the swz_v layout; the lane fetches the logical chunk that
    // belongs there.  Rows past the valid range re-read the last valid row:
    // their probabilities are exactly zero, and nothing past a sequence's
    // length is ever read.
    int vrow[VINST], vcol[VINST];
#pragma unroll
    for (int u = 0; u < VINST; ++u) {
        const int r = RPI * u + lane / (ROW / 16);
        const int pc = lane % (ROW / 16);
        vrow[u] = r;
        vcol[u] = (swz_v<D>(r, pc) - r * ROW) >> 4;  // XOR swizzle is an involution
    }
    int voff[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) voff[dt] = v_frag_off<D>(dt, lane);

    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4_t{0, 0, 0, 0};

    // Sub-tile j of the sequence belongs to workgroup j % nwg, wave (j / nwg) % 4:
    // at any moment the running workgroups read one contiguous front of the
    // cache, which keeps HBM streaming like a plain copy.  Each wave keeps two
    // sub-tiles in flight: the next one's K loads (registers) and V DMA (the
    // other LDS slot) are issued before the current one is computed.
    const int we = max(len, 1);  // rows at or past we - 1 re-read row we - 1 (row 0 if empty)
    const int jstep = nwg * DC_NW;
    // Page holding sub-tile j (paged cache).  A page holds whole sub-tiles,
    // and rows past the length re-read row we - 1 of the same sub-tile, so one
    // page serves a sub-tile.  Out-of-range table entries are clamped so that
    // no read leaves the page pool.  Each wave looks up the page of the
    // sub-tile after next while the current one streams, so the table read
    // never delays a prefetch.
    auto page_of = [&](int j) __attribute__((always_inline)) {
        if constexpr (!PAGED) return 0;
        const int pi = min(j * DC_SUB, we - 1) / cache.page;
        return min(max(cache.table[(size_t)b * cache.max_pages + pi], 0), cache.num_pages - 1);
    };
    auto issue = [&](int j, int pg, char* slot, bf16x8_t (&kd)[2][KSTEPS]) {
        const int t0 = j * DC_SUB;
        // rows of this sub-tile: token tok sits at base + (tok - r0) * D
        const uint16_t* kb = kg;
        const uint16_t* vb = vg;
        int r0 = 0;
        if constexpr (PAGED) {
            const size_t off = ((size_t)pg * Hkv + kvh) * (size_t)cache.page * D;
            kb += off;
            vb += off;
            r0 = min(t0, we - 1) / cache.page * cache.page;
        }
        // rows before the window's first token (only in the sub-tile holding
        // it, which lies in one page) re-read that token's row, as rows past
        // the length re-read the last one: every row read is one the query
        // sees, so a non-finite value outside the window never meets a zero
        // probability in the product
        auto row_tok = [&](int t) __attribute__((always_inline)) {
            if constexpr (PAGED) t = max(t, w0);
            return min(t, we - 1);
        };
#pragma unroll
        for (int u = 0; u < VINST; ++u) {
            const int tok = row_tok(t0 + vrow[u]);
            __builtin_amdgcn_global_load_lds((const void*)(vb + (size_t)(tok - r0) * D + vcol[u] * 8),
                                             (__attribute__((address_space(3))) void*)(slot + u * 1024),
                                             16, 0, DC_V_POLICY);
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int tok = row_tok(t0 + 16 * mt + lr);
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s)
                kd[mt][s] = *(const bf16x8_t*)(kb + (size_t)(tok - r0) * D + 32 * s + 8 * lg);
        }
    };

    // Q^T fragments (B operand, N = head): head h0 + lr (zero past the group),
    // dims 32s + 8lg.  The raw query and this lane's RoPE frequency are loaded
    // first, then the first sub-tile's cache loads are issued, and the query
    // is rotated while those are in flight.  All heads share the new token's
    // position, so each lane forms the cosine and sine of one channel pair
    // (lane % (D/2)) and the rotation fetches them from the lane holding them.
    // (unconditional loads, lanes past the group re-read its last head and are
    // zeroed afterwards, so the compiler can leave the cache loads in flight)
    u32x4_t xq[KSTEPS];
    const uint16_t* const qrow = q + (size_t)(b * Hq + h0 + min(lr, GH - 1)) * D + 8 * lg;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) xq[s] = *(const u32x4_t*)(qrow + 32 * s);
    const double freq = fr.f[lane % (D / 2)];  // loaded unconditionally, like the query

    bf16x8_t kA[2][KSTEPS], kB[2][KSTEPS];  // K fragments, double-buffered like V
    int j = s0 + chunk + nwg * w;
    // unconditional, like every prefetch below, so the number of loads in
    // flight is the same on every path (a wave with no sub-tile re-reads a
    // valid row and never uses it)
    int pg_this = page_of(j), pg_next = page_of(j + jstep);  // pages of sub-tiles j, j + jstep
    issue(j, pg_this, slot0, kA);

    bf16x8_t qf[KSTEPS];
    float cs_l = 1.f, sn_l = 0.f;
    if (rope) rope_cos_sin((long long)len - 1, freq, cs_l, sn_l);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
        u32x4_t x = lr < GH ? xq[s] : u32x4_t{0, 0, 0, 0};
        if (rope) {
            // word e of x holds channel pair 16s + 4lg + e
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int pr = 16 * s + 4 * lg + e;
                const float cs = __shfl(cs_l, pr, 64), sn = __shfl(sn_l, pr, 64);
                float y0, y1;
                rope_rotate(bf16_lo(x[e]), bf16_hi(x[e]), cs, sn, y0, y1);
                x[e] = pack_bf16x2(y0, y1);
            }
        }
        qf[s] = __builtin_bit_cast(bf16x8_t, x);
    }

    // One sub-tile: its V was DMA'd into vcur one step earlier and its K sits
    // in kf; the next sub-tile's loads go to vnext / kn first.
    auto body = [&](int jj, const char* vcur, char* vnext, const bf16x8_t (&kf)[2][KSTEPS],
                    bf16x8_t (&kn)[2][KSTEPS]) __attribute__((always_inline)) {
        const int t0 = jj * DC_SUB;
        const bool more = jj + jstep < n_sub;
        // Always prefetch (the last sub-tile re-fetches itself, an L2 hit) so the
        // number of loads in flight is the same on every path and the waits
        // can leave the prefetch outstanding.
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // vnext was read by the previous step's PV
        issue(more ? jj + jstep : jj, more ? pg_next : pg_this, vnext, kn);
        if (PAGED) {  // the next step's sub-tile and the one after it
            pg_this = more ? pg_next : pg_this;
            pg_next = page_of(jj + 2 * jstep);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the products
        // this sub-tile's K and V were loaded before the prefetch's
        // VINST + 2*KSTEPS operations, and vector memory completes in order
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(VINST + 2 * KSTEPS));
        __builtin_amdgcn_sched_barrier(0);  // ... and the products after the wait

        // S^T = K Q^T; lane holds head lr, tokens t0 + 16mt + 4lg + i
        f32x4_t sacc[2] = {f32x4_t{0, 0, 0, 0}, f32x4_t{0, 0, 0, 0}};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            sacc[0] = mfma16(kf[0][s], qf[s], sacc[0]);
            sacc[1] = mfma16(kf[1][s], qf[s], sacc[1]);
        }
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tk = t0 + 16 * mt + 4 * lg + i;
                if (tk >= len || (PAGED && tk < w0)) sacc[mt][i] = -INFINITY;
                mx = __builtin_elementwise_maximum(mx, sacc[mt][i]);
            }
        mx = __builtin_elementwise_maximum(mx, xor_shfl(mx, 16));
        mx = __builtin_elementwise_maximum(mx, xor_shfl(mx, 32));
        const float mnew = __builtin_elementwise_maximum(m_run, mx);
        const float mref = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f((m_run - mref) * c);
        const float mc = mref * c;
        float ls = 0.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sacc[mt][i], c, -mc));
                sacc[mt][i] = p;
                ls += p;
            }
        l_run = fmaf(l_run, alpha, ls);
        m_run = mnew;
        u32x4_t pw;
        pw[0] = pack_bf16x2(sacc[0][0], sacc[0][1]);
        pw[1] = pack_bf16x2(sacc[0][2], sacc[0][3]);
        pw[2] = pack_bf16x2(sacc[1][0], sacc[1][1]);
        pw[3] = pack_bf16x2(sacc[1][2], sacc[1][3]);
        const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pw);

#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            oacc[dt] = mfma16(v_frag_at<D>(vcur + voff[dt]), pf, oacc[dt] * alpha);
    };
    // Unrolled by two so each step names its V slots and K registers
    // statically, with no exit between the two steps (the compiler would
    // otherwise sink the first step's K prefetch past it, next to its use).
    for (; j + jstep < n_sub; j += 2 * jstep) {
        body(j, slot0, slot1, kA, kB);
        body(j + jstep, slot1, slot0, kB, kA);
    }
    if (j < n_sub) body(j, slot0, slot1, kA, kB);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): the last prefetch landed

    // ---- merge the four waves in LDS
    l_run += xor_shfl(l_run, 16);
    l_run += xor_shfl(l_run, 32);
    __syncthreads();  // all V staging reads are done
    float* const cm = sstat;
    float* const cl = sstat + DC_NW * DC_HEADS;
    float* const co = (float*)vs0;  // [wave][head][D]
    constexpr int OS = D;
    if (lg == 0) {
        cm[w * DC_HEADS + lr] = m_run;
        cl[w * DC_HEADS + lr] = l_run;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        *(f32x4_t*)(co + (w * DC_HEADS + lr) * OS + 16 * dt + 4 * lg) = oacc[dt];
    __syncthreads();
    if (nwg == 1) {
        // the sequence's only workgroup: normalise and write the output here
        for (int e = tid; e < GH * (D / 2); e += DC_NW * 64) {
            const int hd = e / (D / 2), d = 2 * (e % (D / 2));
            float M = -INFINITY;
#pragma unroll
            for (int ww = 0; ww < DC_NW; ++ww) M = fmaxf(M, cm[ww * DC_HEADS + hd]);
            float L = 0.f, O0 = 0.f, O1 = 0.f;
#pragma unroll
            for (int ww = 0; ww < DC_NW; ++ww) {
                const float mw = cm[ww * DC_HEADS + hd];
                const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((mw - M) * c);
                L += f * cl[ww * DC_HEADS + hd];
                O0 += f * co[(ww * DC_HEADS + hd) * OS + d];
                O1 += f * co[(ww * DC_HEADS + hd) * OS + d + 1];
            }
            const float inv = L > 0.f ? 1.f / L : 0.f;  // L == 0 only for an empty sequence
            *(unsigned*)(o + (size_t)(b * Hq + h0 + hd) * D + d) = pack_bf16x2(O0 * inv, O1 * inv);
        }
        return;
    }
    // This call's tag for the group: the host's call tag mixed with the
    // group's epoch word, which the group's merging workgroup advances (below).
    // Every workgroup of the group reads the epoch before it publishes
    // anything, and the epoch only moves once all of them have published, so
    // they all use the same tag.  Successive calls see successive epochs, so
    // the tag changes even when a captured graph replays a launch with the
    // same host tag.  The load is issued here, ahead of the partial stores,
    // so its latency overlaps theirs.
    const size_t grp = ((size_t)b * Hkv + kvh) * (size_t)n_hchunk + (size_t)hc;
    const unsigned long long epoch =
        __hip_atomic_load(ws_epoch + grp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long ctag = tag ^ (epoch * 0x9E3779B97F4A7C15ull);
    {
        // this workgroup's partial o vectors, 16 bytes (4 dims of a head) per store
        const __amdgpu_buffer_rsrc_t ors =
            buffer_rsrc(ws_o + (size_t)(b * Hq + h0) * NC * D, GH * NC * D * 4);
        for (int e = tid; e < GH * (D / 4); e += DC_NW * 64) {
            const int hd = e / (D / 4), d = 4 * (e % (D / 4));
            float M = -INFINITY;
#pragma unroll
            for (int ww = 0; ww < DC_NW; ++ww) M = fmaxf(M, cm[ww * DC_HEADS + hd]);
            float L = 0.f;
            f32x4_t O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ww = 0; ww < DC_NW; ++ww) {
                const float mw = cm[ww * DC_HEADS + hd];
                const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((mw - M) * c);
                L += f * cl[ww * DC_HEADS + hd];
                O += f * *(const f32x4_t*)(co + (ww * DC_HEADS + hd) * OS + d);
            }
            store4_coherent(O, ors, ((hd * NC + chunk) * D + d) * 4);
            if (d == 0) {
                const size_t slot = (size_t)(b * Hq + h0 + hd) * NC + chunk;
                store_agent(ws_ml + slot * 2, M);
                store_agent(ws_ml + slot * 2 + 1, L);
            }
        }
    }

    // ---- publish the partial, then look for the others.  Each partial slot of
    // a (sequence, KV head, head slice) carries the tag of the call that wrote
    // it, stored once the partial itself is complete.  A workgroup that, after
    // its own tag store has completed, finds this call's tag in every slot
    // merges all of them.  At least one workgroup always does: of two
    // workgroups that finish together, the one whose tag store completes last
    // sees the other's tag.  Two may both merge (identical results, written
    // twice).  Slots written by other calls, or holding anything at all, carry
    // another tag, so the workspace needs no clearing between calls.
    //
    // Why completed device-scope accesses suffice, with no fence.  In the
    // AMDGPU memory model of LLVM's AMDGPU backend documentation (the GFX942
    // section, which GFX950 follows), agent-scope atomic loads and stores are
    // plain loads and stores with the SC1 bit, the device scope of the CDNA3
    // instruction set's memory-scope bits: such a store writes through the
    // issuing XCD's L2, and such a load misses in any L1 or L2 line that is not
    // coherent at device scope, so it returns what completed device-scope
    // stores from any XCD left in memory.  The same document's agent-scope
    // release is an L2 write-back followed by a wait for vmcnt(0), and its
    // acquire an L1/L2 invalidate; the write-back exists for earlier stores
    // made without SC1 and the invalidate for later loads made without it.
    // Here every store that is published (partials, their (max, sum) pairs and
    // the tag) and every load that consumes them carries SC1 (the relaxed
    // agent-scope atomics, and the 16-byte buffer accesses with cache policy
    // bit 4, SC1), so the release reduces to the vmcnt(0) waits below, before
    // the tag store, and the acquire to nothing: the partial loads are issued
    // only after the barrier whose outcome depends on the tag loads.  A device-
    // wide fence (L2 write-back and invalidate) measured 50% slower, because it
    // stalls the workgroups still streaming the cache.
    unsigned long long* const tags = ws_tag + grp * (size_t)NC;
    __builtin_amdgcn_s_waitcnt(0x0070);  // this thread's partial stores (and epoch load) completed
    __syncthreads();
    if (tid == 0) {
        __hip_atomic_store(tags + chunk, ctag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0x0070);  // the tag store completed
    }
    __syncthreads();
    int mine = 1;
    for (int ch = tid; ch < nwg; ch += DC_NW * 64)
        mine &= __hip_atomic_load(tags + ch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ctag;
    if (!__syncthreads_and(mine)) return;
    // every workgroup of the group has read the epoch (each did before its tag
    // store): advance it for the group's next call (a store, so two merging
    // workgroups leave the same value)
    if (tid == 0)
        __hip_atomic_store(ws_epoch + grp, epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // ---- merge (log-sum-exp over the nwg partials).  Each thread folds one or
    // two items (a head and 4 consecutive dims each).  Partials are taken in
    // blocks: every thread first issues the loads of its items' o vectors for
    // the whole block (NSLOT 16-byte loads: 24 partials of one item, or 12 of
    // two), then the block's (max, sum) pairs, so a block costs one memory
    // round trip.  The pairs go to LDS, where one 16-lane row per head forms
    // its running max, factors and sum with row reductions, and the threads
    // fold their o vectors with those factors.
    constexpr int NSLOT = 24, EPI = 4, MBX = NSLOT;
    constexpr int NITEM = DC_HEADS * D / EPI / (DC_NW * 64);  // items per thread, at most
    static_assert(NITEM >= 1 && NITEM <= 2 && NSLOT % NITEM == 0, "merge slots");
    static_assert(2 * DC_HEADS * MBX * 4 <= DecodeSmem<D>::kSlots, "merge tables fit one V slot array");
    const int ipt = GH * (D / EPI) > DC_NW * 64 ? 2 : 1;  // items this workgroup's threads fold
    const int MB = NSLOT / ipt;                           // partials per block
    float* const bm = (float*)vs0;          // [DC_HEADS][MBX] max, then factor
    float* const bl = bm + DC_HEADS * MBX;  // [DC_HEADS][MBX] sum
    float* const run = sstat;  // [DC_HEADS] running max, [DC_HEADS] alpha, [DC_HEADS] L
    if (tid < DC_HEADS) {
        run[tid] = -INFINITY;
        run[2 * DC_HEADS + tid] = 0.f;
    }
    float acc[NITEM][EPI];
#pragma unroll
    for (int it = 0; it < NITEM; ++it)
#pragma unroll
        for (int e = 0; e < EPI; ++e) acc[it][e] = 0.f;
    constexpr int NML = ceil_div(DC_HEADS * MBX, DC_NW * 64);  // (max, sum) pairs per thread
    // the group's partial o vectors [GH][NC][D]
    const __amdgpu_buffer_rsrc_t ors = buffer_rsrc(ws_o + (size_t)(b * Hq + h0) * NC * D, GH * NC * D * 4);
    for (int c0 = 0; c0 < nwg; c0 += MB) {
        const int nb = min(MB, nwg - c0);
        // slot k: item k / MB, partial c0 + k % MB
        f32x4_t oc[NSLOT];
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) {
            const int it = (NITEM > 1 && k >= MB) ? 1 : 0, u = k - it * MB;
            const int item = tid + it * DC_NW * 64;
            const bool ok = it < ipt && item < GH * (D / EPI) && u < nb;
            const int hd = ok ? item / (D / EPI) : 0, d = EPI * (item % (D / EPI));
            oc[k] = ok ? load4_coherent(ors, ((hd * NC + c0 + u) * D + d) * 4)
                       : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        float pm[NML], pl[NML];
#pragma unroll
        for (int r = 0; r < NML; ++r) {
            const int e = tid + r * DC_NW * 64;
            pm[r] = pl[r] = 0.f;
            if (e < GH * nb) {
                const size_t sl = (size_t)(b * Hq + h0 + e / nb) * NC + c0 + e % nb;
                pm[r] = load_agent(ws_ml + sl * 2);
                pl[r] = load_agent(ws_ml + sl * 2 + 1);
            }
        }
        __syncthreads();  // the previous block's factors have been used
#pragma unroll
        for (int r = 0; r < NML; ++r) {
            const int e = tid + r * DC_NW * 64;
            if (e < GH * nb) {
                bm[(e / nb) * MBX + e % nb] = pm[r];
                bl[(e / nb) * MBX + e % nb] = pl[r];
            }
        }
        __syncthreads();
        {  // one 16-lane row per head: running max, rescale, factors, sum
            static_assert(DC_HEADS == 4 * DC_NW && MBX <= 32, "a row per head, two partials per lane");
            const int j = lane & 15, hd = 4 * w + (lane >> 4);
            const bool hv = hd < GH;
            const int r = hv ? hd : 0;
            const bool v0 = hv && j < nb, v1 = hv && j + 16 < nb && j + 16 < MBX;
            const float m0 = v0 ? bm[r * MBX + j] : -INFINITY;
            const float m1 = v1 ? bm[r * MBX + j + 16] : -INFINITY;
            const float l0 = v0 ? bl[r * MBX + j] : 0.f;
            const float l1 = v1 ? bl[r * MBX + j + 16] : 0.f;
            const float mprev = run[r];
            const float mx = row16_max(fmaxf(fmaxf(m0, m1), mprev));
            const float mref = (mx == -INFINITY) ? 0.f : mx;
            const float alpha = (mprev == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((mprev - mref) * c);
            const float f0 = (m0 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m0 - mref) * c);
            const float f1 = (m1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m1 - mref) * c);
            const float ls = row16_sum(fmaf(f0, l0, f1 * l1));
            if (v0) bm[r * MBX + j] = f0;
            if (v1) bm[r * MBX + j + 16] = f1;
            if (hv && j == 0) {
                run[r] = mx;
                run[DC_HEADS + r] = alpha;
                run[2 * DC_HEADS + r] = fmaf(run[2 * DC_HEADS + r], alpha, ls);
            }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < NITEM; ++it) {
            const int item = tid + it * DC_NW * 64;
            if (it >= ipt || item >= GH * (D / EPI)) break;
            const int hd = item / (D / EPI);
            const float alpha = run[DC_HEADS + hd];
#pragma unroll
            for (int e = 0; e < EPI; ++e) acc[it][e] *= alpha;
        }
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) {  // branch-free, so the factor reads batch up
            const int it = (NITEM > 1 && k >= MB) ? 1 : 0, u = k - it * MB;
            const int item = tid + it * DC_NW * 64;
            const bool ok = it < ipt && item < GH * (D / EPI) && u < nb;
            const float fr = bm[min(item / (D / EPI), DC_HEADS - 1) * MBX + u];
            const float f = ok ? fr : 0.f;
#pragma unroll
            for (int e = 0; e < EPI; ++e) acc[it][e] = fmaf(f, oc[k][e], acc[it][e]);
        }
    }
#pragma unroll
    for (int it = 0; it < NITEM; ++it) {
        const int item = tid + it * DC_NW * 64;
        if (item >= GH * (D / EPI)) break;
        const int hd = item / (D / EPI), d = EPI * (item % (D / EPI));
        const float L = run[2 * DC_HEADS + hd];
        const float inv = L > 0.f ? 1.f / L : 0.f;
        u32x2_t wv;
        wv[0] = pack_bf16x2(acc[it][0] * inv, acc[it][1] * inv);
        wv[1] = pack_bf16x2(acc[it][2] * inv, acc[it][3] * inv);
        *(u32x2_t*)(o + (size_t)(b * Hq + h0 + hd) * D + d) = wv;
    }
}

// Workgroup budget of a launch over `groups` (sequence, KV head, head slice)
// groups: about two per compute unit when there are many groups; with few
// groups (a handful of long sequences) about 72% of the units, since on this
// part fewer, longer streams per cache region read HBM faster.  At most the
// number of lengths a wave can stage.
#ifndef DC_MANY_PCT
#define DC_MANY_PCT 200
#endif
#ifndef DC_FEW_PCT
#define DC_FEW_PCT 72
#endif
int decode_budget(long long groups, int D) {
    const long long cus = device_cus();
    const long long budget = groups * 4 >= cus ? std::max(1ll, cus * DC_MANY_PCT / 100)
                                               : std::max(1ll, cus * DC_FEW_PCT / 100);
    const long long cap = (long long)(DC_SUB * D * 2) / 4;  // lengths one V slot holds
    return (int)std::min(budget, cap);
}

unsigned long long next_decode_tag();

template <int D, bool PAGED>
hipError_t launch_decode_d(void* o, const void* q, const DecodeCache& cache, int B, int Hq, int Hkv,
                           const int32_t* seqlens, int max_len, float c, double rope_theta,
                           void* workspace, unsigned long long tag, hipStream_t st) {
    const int NC = decode_num_chunks(B, Hkv, max_len);  // partial slots per (sequence, head)
    const int G = Hq / Hkv;
    const int n_hchunk = ceil_div(G, DC_HEADS);
    const long long groups = (long long)B * Hkv * n_hchunk;
    const int budget = decode_budget(groups, D);
    const long long nblocks = std::max<long long>(budget, groups);
    if (nblocks > INT32_MAX) return hipErrorInvalidValue;
    float* const ws_o = (float*)workspace;
    float* const ws_ml = ws_o + (size_t)B * Hq * NC * D;
    unsigned long long* const ws_tag = (unsigned long long*)(ws_ml + (size_t)B * Hq * NC * 2);
    unsigned long long* const ws_epoch = ws_tag + (size_t)groups * NC;
    hipLaunchKernelGGL((decode_split_kernel<D, PAGED>), dim3((unsigned)nblocks), dim3(DC_NW * 64), 0,
                       st, (const uint16_t*)q, cache, seqlens, ws_o, ws_ml, ws_tag, ws_epoch,
                       (uint16_t*)o, Hq,
                       Hkv, max_len, NC, c, n_hchunk, rope_theta > 0 ? 1 : 0,
                       rope_freqs(rope_theta > 0 ? rope_theta : 1.0, D), tag, B, budget);
    return hipGetLastError();
}

template <bool PAGED>
hipError_t launch_decode_any(void* o, const void* q, const DecodeCache& cache, int B, int Hq,
                             int Hkv, int D, const int32_t* seqlens, int max_len, float scale,
                             double rope_theta, void* workspace, hipStream_t st) {
    const float c = scale * kLog2e;
    const unsigned long long tag = next_decode_tag();
    return D == 64 ? launch_decode_d<64, PAGED>(o, q, cache, B, Hq, Hkv, seqlens, max_len, c,
                                                rope_theta, workspace, tag, st)
                   : launch_decode_d<128, PAGED>(o, q, cache, B, Hq, Hkv, seqlens, max_len, c,
                                                 rope_theta, workspace, tag, st);
}

// Call tags for the partial slots: distinct for every call in the process
// (40 bits, never zero), starting from a value that differs between processes.
unsigned long long next_decode_tag() {
    static std::atomic<unsigned long long> seq{
        (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count() * 0x9E3779B97F4A7C15ull};
    constexpr unsigned long long kMask = (1ull << 40) - 1;
    unsigned long long t;
    do {
        t = seq.fetch_add(1, std::memory_order_relaxed) & kMask;
    } while (t == 0);
    return t;
}

}  // namespace

int decode_num_chunks(int B, int Hkv, int max_len) {
    // workspace slots per (sequence, head): the most split workgroups a group can get
    return decode_max_partials(max_len);
}

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int max_len, int D) {
    // fp32 partials (o[D], max, sum) per (sequence, query head, split workgroup),
    // then one 64-bit call tag per (sequence, KV head, head slice, split
    // workgroup), then one 64-bit epoch per (sequence, KV head, head slice)
    const size_t NC = (size_t)decode_num_chunks(B, Hkv, max_len);
    const size_t n_hchunk = (size_t)ceil_div(Hq / Hkv, DC_HEADS);
    return (size_t)B * Hq * NC * (size_t)(D + 2) * sizeof(float) +
           (size_t)B * Hkv * n_hchunk * (NC + 1) * sizeof(unsigned long long);
}

hipError_t launch_decode(void* o, const void* q, const void* k_cache, const void* v_cache, int B,
                         int Hq, int Hkv, int S_cap, int D, const int32_t* seqlens, int max_len,
                         float scale, double rope_theta, void* workspace, hipStream_t st) {
    const DecodeCache cache{(const uint16_t*)k_cache, (const uint16_t*)v_cache, nullptr, S_cap, 0, 0, 0, 0};
    return launch_decode_any<false>(o, q, cache, B, Hq, Hkv, D, seqlens, max_len, scale, rope_theta,
                                    workspace, st);
}

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of `scratch` on device dev, looked up once per device with
// that device current (each device holds its own copy of the array).
hipError_t scratch_address(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}
}  // namespace

hipError_t launch_decode_noalloc(void* o, const void* q, const void* k_cache, const void* v_cache,
                                 int B, int Hq, int Hkv, int S_cap, int D, const int32_t* seqlens,
                                 int max_len, float scale, double rope_theta, hipStream_t st) {
    int dev = 0;
    hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    void* ws = nullptr;
    if ((e = scratch_address(dev, &ws)) != hipSuccess) return e;
    return launch_decode(o, q, k_cache, v_cache, B, Hq, Hkv, S_cap, D, seqlens, max_len, scale,
                         rope_theta, ws, st);
}

hipError_t launch_decode_paged(void* o, const void* q, const void* k_pages, const void* v_pages,
                               int B, int Hq, int Hkv, int page_size, int D, int num_pages,
                               const int32_t* block_table, int max_pages, const int32_t* seqlens,
                               int max_len, int window, float scale, double rope_theta,
                               void* workspace, hipStream_t st) {
    const DecodeCache cache{(const uint16_t*)k_pages, (const uint16_t*)v_pages, block_table, 0,
                            page_size, max_pages, num_pages, window};
    return launch_decode_any<true>(o, q, cache, B, Hq, Hkv, D, seqlens, max_len, scale, rope_theta,
                                   workspace, st);
}

}  // namespace attn
