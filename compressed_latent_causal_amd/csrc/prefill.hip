// Causal grouped-query attention prefill for gfx950.
//
// What is computed ("Grouped Query Attention (GQA)" glossary, section "Cómo
// funciona GQA"): per query head h, unchanged causal scaled dot-product
// attention against key/value head h / G, G = Hq / Hkv.  The "Compressed
// Convolutional Attention" summary ("Methodologie", CCGQA paragraph) runs the
// same operation in a compressed latent with small head dims (64 here).
//
// bf16 kernel design (flash-style, exact up to rounding):
//  * One workgroup = 4 waves = HPW query heads of one KV group x a block of
//    queries.  Each wave owns one head and 32 consecutive queries; two
//    workgroups share a CU, so while one waits on its barrier, its tile loads
//    or LDS, the other issues.  (A SIMD issues matrix and vector
//    instructions one after the other: vector work is never hidden behind
//    the matrix core, so the softmax is kept to the exponentials.)  The K and V
//    tile (64 keys x D) is loaded once into LDS and serves every head of the
//    workgroup, so a KV group's key/value bytes are fetched once per query block
//    rather than once per query head.
//  * Scores are formed transposed, S^T = K Q^T, with the 16x16x32 bf16 matrix
//    core: each lane ends up holding one query and 4 keys per 16x16 tile, so the
//    softmax row statistics are per-lane scalars (plus a 4-lane reduction).
//  * Online softmax in fp32 in the exp2 domain.  Q enters the score products
//    exactly (a copy pre-scaled by scale * log2 e and rounded to bf16 again
//    would move each score by up to 2^-9 of its terms, which peaked softmaxes
//    do not tolerate); one FMA per score then forms the exponent
//    c s - reference, and one exp2 the probability.  The reference moves only
//    when a tile's probabilities would sum past 2^16, so almost every tile
//    skips rescaling O (the normalisation at the end is exact for any
//    reference).  P is rounded to bf16 and fed straight from registers as the
//    B operand of O^T = V^T P^T.  The A operand (V^T) comes from the row-major
//    V tile through the LDS transpose read, so V is never transposed in memory.
//  * K/V tiles are double-buffered in LDS and loaded with buffer loads that
//    write LDS directly (no staging registers, no LDS store instructions, no
//    address arithmetic per tile: the tile start is a scalar offset).  The
//    load of tile t + 1 is issued right after the barrier that opens tile t
//    and lands while tile t is computed.  LDS rows are XOR-swizzled in
//    16-byte chunks, with one permutation for K and another for V, each
//    conflict-free for its read pattern; the swizzle is applied by choosing
//    each lane's source chunk.  Per-lane operand offsets are computed once, so
//    the tile loop addresses LDS with immediate offsets.
//  * Row statistics are combined across the four lanes that share a query
//    with the cross-row lane swap instructions, not through LDS.
//  * Work order: heaviest (last) query blocks are dispatched first, and
//    consecutive workgroup ids walk (batch, KV head) fastest so a KV group's
//    blocks share an XCD (and its L2) when B*Hkv is a multiple of 8.
//  * Only tiles at or left of the diagonal are visited; only diagonal tiles
//    pay the elementwise mask.
//
// fp32 kernel: plain fp32 VALU arithmetic (accuracy target 1e-5), the same
// work split idea with K/V tiles of 32 keys in LDS shared by up to 4 heads.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

#ifndef ATTN_PF_WAVES
#define ATTN_PF_WAVES 4
#endif
constexpr int PF_BN = 64;                 // keys per K/V tile
// Query tiles of 16 per wave (NQ): every K and V operand fragment read from
// LDS feeds NQ products, so LDS bytes per product fall as 1 / NQ.
#ifndef PF_NQ64
#define PF_NQ64 2
#endif
#ifndef PF_NQ128
#define PF_NQ128 2
#endif
constexpr int PF_NW = ATTN_PF_WAVES;      // waves per workgroup
constexpr int PF_THREADS = PF_NW * 64;

// Workgroup order.  Workgroups go to the 8 XCDs (each with its own L2) in
// turn, so workgroup i runs on XCD i % 8.  With per = (sequence, KV head,
// head chunk) combinations a multiple of 8, XCD x serves the combinations
// rem = x (mod 8) for every query block; in plain order it runs them
// interleaved, heaviest query blocks first, and the K/V of per/8 KV heads
// compete for its L2.  Here each XCD takes its combinations one after the
// other, each from its heaviest query block down, so the workgroups resident
// on an XCD mostly share one KV head's K/V.  Every XCD keeps the same work.
// Other shapes keep the plain order.  Returns the query-block rank qbi (0 =
// heaviest) and the combination rem.
__device__ inline void xcd_block_order(int i, int per, int n_qblk, int& qbi, int& rem) {
    if (per % 8 == 0) {
        const int j = i / 8, m = j / n_qblk;  // m-th combination of this XCD
        qbi = j % n_qblk;
        rem = (i % 8) + 8 * m;
    } else {
        qbi = i / per;
        rem = i % per;
    }
}

// LDS operand fragments read ahead of the products that use them
#ifndef PF_PD
#define PF_PD 2
#endif
// Issue priority of a wave's matrix-core phases over its softmax (experiment)
#ifndef PF_PRIO
#define PF_PRIO 0
#endif
__device__ __attribute__((always_inline)) inline void pf_prio_hi() {
    if constexpr (PF_PRIO) __builtin_amdgcn_s_setprio(PF_PRIO);
}
__device__ __attribute__((always_inline)) inline void pf_prio_lo() {
    if constexpr (PF_PRIO) __builtin_amdgcn_s_setprio(0);
}

// The online softmax keeps a per-row reference (a past tile maximum) and only
// moves it when a tile's probabilities relative to it sum to more than this:
// every accumulated probability is then at most 2^16 (exact in the final
// normalisation, far from fp32 and bf16 overflow), and most tiles need neither
// a maximum nor a rescale of O.
constexpr float PF_SUM_LIMIT = 65536.f;

template <int D, int HPW, int NQ>
__global__ __launch_bounds__(PF_THREADS, (D == 64 || NQ == 2) ? 2 : 1) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int B, int Hq, int Hkv, int S, float c,
    int n_qblk, int n_hchunk, int rope, RopeFreqs fr) {
    constexpr int KSTEPS = D / 32;              // k-steps of S^T = K Q^T
    constexpr int DT = D / 16;                  // d tiles of O^T
    constexpr int PF_QW = 16 * NQ;              // queries per wave
    constexpr int QPB = (PF_NW / HPW) * PF_QW;  // queries per head per workgroup
    constexpr int ROW = D * 2;                  // bytes per LDS row
    constexpr int TILE = PF_BN * ROW;
    constexpr int RPI = 1024 / ROW;             // rows per 1 KiB (one wave-wide 16-byte load)
    constexpr int NI = TILE / 1024 / PF_NW;     // such loads per wave per tile, for K and for V
    static_assert(NI >= 1 && TILE % (1024 * PF_NW) == 0, "tile split");
    static_assert(HPW <= PF_NW && PF_NW % HPW == 0, "one head per wave at most");

    // Two K and two V tile buffers as separate objects, so the compiler can
    // tell the buffer being filled from the one being read.
    __shared__ __attribute__((aligned(1024))) char k0[TILE];
    __shared__ __attribute__((aligned(1024))) char k1[TILE];
    __shared__ __attribute__((aligned(1024))) char v0[TILE];
    __shared__ __attribute__((aligned(1024))) char v1[TILE];

    const int G = Hq / Hkv;
    const int per = B * Hkv * n_hchunk;
    int qbi, rem;
    xcd_block_order((int)blockIdx.x, per, n_qblk, qbi, rem);
    const int qb = n_qblk - 1 - qbi;  // heaviest query blocks first
    const int bkv = rem % (B * Hkv), hc = rem / (B * Hkv);
    const int b = bkv / Hkv, kvh = bkv % Hkv;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;  // row-in-tile / lane group
    const int h = kvh * G + hc * HPW + (w % HPW);
    const int q0 = qb * QPB;
    const int qw0 = q0 + (w / HPW) * PF_QW;

    const uint16_t* const kg = k + (size_t)(b * Hkv + kvh) * S * D;
    const uint16_t* const vg = v + (size_t)(b * Hkv + kvh) * S * D;
    const size_t qo_base = (size_t)(b * Hq + h) * S * D;

    // With the query RoPE fused, the cosines and sines of the workgroup's query
    // positions are formed once into a table shared by its heads (rows 0..31
    // in the not yet used k1, rows 32..63 in v1: 32 rows x D/2 pairs x 8 bytes
    // fill one tile buffer).  Workgroups of 128 queries (one head each) form
    // them per lane instead.  A lane reads the 4 pairs it rotates as two
    // 16-byte units; unit u of row r is stored at u ^ swz(r) with the swz_v
    // row permutation, so the 16 rows one lane group reads fall in distinct
    // banks (unswizzled, rows 256 or 512 bytes apart share them all).
    constexpr bool kRopeTable = QPB <= 64;
    auto rope_slot = [&](int r, int u) __attribute__((always_inline)) {
        return (r < 32 ? k1 : v1) + (r & 31) * (4 * D) + 16 * (u ^ (((r & 7) << 1) | ((r >> 3) & 1)));
    };
    if (rope && kRopeTable) {
        for (int idx = tid; idx < QPB * (D / 2); idx += PF_THREADS) {
            const int r = idx / (D / 2), pr = idx % (D / 2);
            float cs, sn;
            rope_cos_sin(q0 + r, fr.f[pr], cs, sn);
            *(float2*)(rope_slot(r, pr >> 1) + 8 * (pr & 1)) = float2{cs, sn};
        }
        __syncthreads();
    }

    // Q^T fragments (B operand): query qw0 + 16n + lr, dims 32s + 8lg .. +7.
    bf16x8_t qf[NQ][KSTEPS];
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
        const int row = qw0 + 16 * n + lr;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            u32x4_t x = {0, 0, 0, 0};
            if (row < S) x = *(const u32x4_t*)(q + qo_base + (size_t)row * D + 32 * s + 8 * lg);
            if (rope) {
                // query `row` sits at position row; word e of x holds channel
                // pair 16s + 4lg + e (the same arithmetic as the RoPE kernel)
                f32x4_t tu[2];
                if constexpr (kRopeTable) {
                    const int tr = (w / HPW) * PF_QW + 16 * n + lr;  // table row
#pragma unroll
                    for (int hu = 0; hu < 2; ++hu)
                        tu[hu] = *(const f32x4_t*)rope_slot(tr, 8 * s + 2 * lg + hu);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int pr = 16 * s + 4 * lg + e;
                    float cs, sn, y0, y1;
                    if constexpr (kRopeTable) {
                        cs = tu[e >> 1][2 * (e & 1)];
                        sn = tu[e >> 1][2 * (e & 1) + 1];
                    } else {
                        rope_cos_sin(row, fr.f[pr], cs, sn);
                    }
                    rope_rotate(bf16_lo(x[e]), bf16_hi(x[e]), cs, sn, y0, y1);
                    x[e] = pack_bf16x2(y0, y1);
                }
            }
            // q enters the products exactly as given (or as rotated): a
            // pre-scaled copy, rounded to bf16 once more, would move each
            // score by up to 2^-9 of its terms, too much for peaked softmaxes
            qf[n][s] = __builtin_bit_cast(bf16x8_t, x);
        }
    }

    // Per-lane LDS offsets, fixed for the whole loop: the K operand of k-step s
    // (rows 16mt + lr add the constant 16mt * ROW) and the V operand of d tile dt.
    int koff[KSTEPS], voff[DT];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) koff[s] = swz_k<D>(lr, 4 * s + lg);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) voff[dt] = v_frag_off<D>(dt, lane);

    // Tiles go from global memory straight into LDS (buffer loads with the LDS
    // destination: no registers, no LDS store instructions).  Such a load puts
    // lane l's 16 bytes at byte 16 l of a 1 KiB destination, so the swizzled
    // layout is produced by choosing the source: the lane landing on physical
    // chunk p of row r fetches logical chunk p ^ f(r) (each swizzle is an
    // XOR, its own inverse).  Offsets are relative to the tile's first row;
    // the tile start is the scalar offset.  Rows past the sequence fall outside
    // the buffer resource and arrive as zeros (those keys are masked anyway).
    int kvo[NI], vvo[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int r = (w * NI + i) * RPI + lane / (ROW / 16), pc = lane % (ROW / 16);
        kvo[i] = r * ROW + ((swz_k<D>(r, pc) - r * ROW) & ~15);
        vvo[i] = r * ROW + ((swz_v<D>(r, pc) - r * ROW) & ~15);
    }
    const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(kg, S * ROW);
    const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(vg, S * ROW);
    auto issue = [&](int t, char* kb, char* vb) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            dma16(krs, kb + (w * NI + i) * 1024, kvo[i], t * TILE);
            dma16(vrs, vb + (w * NI + i) * 1024, vvo[i], t * TILE);
        }
    };

    const int kv_end = min(q0 + QPB, S);
    const int ntiles = ceil_div(kv_end, PF_BN);
    // last tile this wave needs (-1: none, the wave's queries are all past S)
    const int last = qw0 < S ? min(ntiles - 1, (qw0 + PF_QW - 1) / PF_BN) : -1;

    f32x4_t oacc[DT][NQ];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int n = 0; n < NQ; ++n) oacc[dt][n] = f32x4_t{0, 0, 0, 0};
    // Running reference of each row in the exp2 domain (-inf before the first
    // tile; 0 stands in for it until the first tile sets it).
    float m_run[NQ], mref[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
        m_run[n] = -INFINITY;
        mref[n] = 0.f;
    }
    // Row sums of P, formed on the matrix core: a tile of ones times P^T puts
    // each query's sum over the tile's keys in every element of its lane (no
    // lane reduction), and it sums exactly the bf16 values the P V product
    // weights.  Four products per tile cost less than 32 vector adds, since
    // vector and matrix instructions share a SIMD's issue.
    float lacc[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) lacc[n] = 0.f;
    const bf16x8_t kOnes = __builtin_bit_cast(
        bf16x8_t, u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});  // bf16 1.0

    auto compute = [&](int t, const char* ks, const char* vs) __attribute__((always_inline)) {
        const int kv0 = t * PF_BN;
        // ---- S^T = K Q^T : tile mt covers keys kv0 + 16mt .. +15.  Operand f
        // (k-step f / 4, key tile f % 4) is read PF_PD operands ahead of its
        // products, so the LDS latency hides behind them.
        constexpr int NKF = 4 * KSTEPS;
        auto kfrag = [&](int f) __attribute__((always_inline)) {
            return *(const bf16x8_t*)(ks + koff[f / 4] + 16 * (f % 4) * ROW);
        };
        f32x4_t sacc[4][NQ];
        bf16x8_t kf[NKF];
        pf_prio_hi();
#pragma unroll
        for (int f = 0; f < PF_PD && f < NKF; ++f) kf[f] = kfrag(f);
#pragma unroll
        for (int f = 0; f < NKF; ++f) {
            if (f + PF_PD < NKF) kf[f + PF_PD] = kfrag(f + PF_PD);
            __builtin_amdgcn_sched_barrier(0);
            const int s = f / 4, mt = f % 4;
#pragma unroll
            for (int n = 0; n < NQ; ++n)
                sacc[mt][n] = mfma16(kf[f], qf[n][s], s == 0 ? f32x4_t{0, 0, 0, 0} : sacc[mt][n]);
            __builtin_amdgcn_sched_barrier(0);
        }
        pf_prio_lo();
        // into the exp2 domain relative to the reference: c s - reference,
        // one FMA per score
#pragma unroll
        for (int n = 0; n < NQ; ++n)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) sacc[mt][n][i] = fmaf(sacc[mt][n][i], c, -mref[n]);

        // ---- online softmax; lane holds query qw0 + 16n + lr and keys kv0 + 16mt + 4lg + i
        if (t == last && kv0 + PF_BN - 1 > qw0) {  // the diagonal tile: mask future keys
#pragma unroll
            for (int n = 0; n < NQ; ++n) {
                const int lim = qw0 + 16 * n + lr - kv0 - 4 * lg;  // key offsets above lim are masked
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (16 * mt + i > lim) sacc[mt][n][i] = -INFINITY;
            }
        }
        // ---- sacc = c * s - reference.  P = exp2(sacc) as bf16 fragments and
        // its row sums lt for this tile.
        bf16x8_t pf[NQ][2];
        f32x4_t lt[NQ];
        auto exp_pack = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int n = 0; n < NQ; ++n) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    u32x4_t pw;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const f32x4_t& x = sacc[2 * kk + h][n];
                        pw[2 * h] = pack_bf16x2(__builtin_amdgcn_exp2f(x[0]), __builtin_amdgcn_exp2f(x[1]));
                        pw[2 * h + 1] = pack_bf16x2(__builtin_amdgcn_exp2f(x[2]), __builtin_amdgcn_exp2f(x[3]));
                    }
                    pf[n][kk] = __builtin_bit_cast(bf16x8_t, pw);
                }
                lt[n] = mfma16(kOnes, pf[n][0], f32x4_t{0, 0, 0, 0});
                lt[n] = mfma16(kOnes, pf[n][1], lt[n]);
            }
        };
        exp_pack();
        // The reference moves to the row's tile maximum on the row's first
        // tile, and when the tile's sum exceeds PF_SUM_LIMIT (or is not
        // finite); then O and the sums are rescaled and the tile is redone
        // (wave-uniform branch, taken on few tiles).
        bool redo = false;
#pragma unroll
        for (int n = 0; n < NQ; ++n) redo |= (m_run[n] == -INFINITY) | !(lt[n][0] <= PF_SUM_LIMIT);
        if (__any(redo)) {
#pragma unroll
            for (int n = 0; n < NQ; ++n) {
                // NaN-propagating maximum: one 3-input instruction per pair
                float m = sacc[0][n][0];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) m = __builtin_elementwise_maximum(m, sacc[mt][n][i]);
                const float mx = group4_max(m);
                const bool up = (mx > -INFINITY) & ((m_run[n] == -INFINITY) | !(lt[n][0] <= PF_SUM_LIMIT));
                const float d = up ? mx : 0.f;  // the shift of the reference
                // nothing is accumulated before the first tile
                const float alpha = (m_run[n] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(-d);
                if (up) m_run[n] = (m_run[n] == -INFINITY ? 0.f : m_run[n]) + d;
                mref[n] = m_run[n] == -INFINITY ? 0.f : m_run[n];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) sacc[mt][n] -= d;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) oacc[dt][n] *= alpha;
                lacc[n] *= alpha;
            }
            exp_pack();
        }
#pragma unroll
        for (int n = 0; n < NQ; ++n) lacc[n] += lt[n][0];

        // ---- O^T += V^T P^T, operand f = (d tile f / 2, key half f % 2) read
        // PF_PD operands ahead
        constexpr int NVF = 2 * DT;
        auto vfrag = [&](int f) __attribute__((always_inline)) {
            return v_frag_at<D>(vs + voff[f / 2] + 32 * (f % 2) * ROW);
        };
        bf16x8_t vf[NVF];
        pf_prio_hi();
#pragma unroll
        for (int f = 0; f < PF_PD && f < NVF; ++f) vf[f] = vfrag(f);
#pragma unroll
        for (int f = 0; f < NVF; ++f) {
            if (f + PF_PD < NVF) vf[f + PF_PD] = vfrag(f + PF_PD);
            __builtin_amdgcn_sched_barrier(0);
            const int dt = f / 2, kk = f % 2;
#pragma unroll
            for (int n = 0; n < NQ; ++n) oacc[dt][n] = mfma16(vf[f], pf[n][kk], oacc[dt][n]);
            __builtin_amdgcn_sched_barrier(0);
        }
        pf_prio_lo();
    };

    // Tile t sits in buffer t & 1.  Each step waits for its own share of tile
    // t, meets the other waves (so all of tile t has landed and everyone has
    // finished reading tile t - 1), starts loading tile t + 1 into the buffer
    // tile t - 1 used, and computes on tile t while that load is in flight.
    auto step = [&](int t, const char* ks, const char* vs, char* kn, char* vn)
                    __attribute__((always_inline)) {
        // vmcnt(0) lgkmcnt(0) (expcnt left alone), as the builtin so the
        // compiler's own wait bookkeeping sees it
        __builtin_amdgcn_s_waitcnt(0x0070);
        __builtin_amdgcn_s_barrier();
        if (t + 1 < ntiles) issue(t + 1, kn, vn);
        if (t <= last) compute(t, ks, vs);
    };
    issue(0, k0, v0);
    for (int t = 0; t < ntiles; t += 2) {
        step(t, k0, v0, k1, v1);
        if (t + 1 >= ntiles) break;
        step(t + 1, k1, v1, k0, v0);
    }

    // ---- epilogue: O = O^T / l, lane holds query qw0 + 16n + lr, dims 16dt + 4lg .. +3.
    // The row's probabilities are exp2(c s - m_run) / l, so its log-normaliser
    // (natural log, of the scaled scores) is ln 2 * (m_run + log2 l).
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
        const float lt = lacc[n];
        const int qi = qw0 + 16 * n + lr;
        if (qi >= S) continue;
        if (lse && lg == 0) lse[(size_t)(b * Hq + h) * S + qi] = (m_run[n] + log2f(lt)) * 0.69314718055994531f;
        const float inv = 1.f / lt;
        uint16_t* const orow = o + qo_base + (size_t)qi * D + 4 * lg;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            u32x2_t wv;
            wv[0] = pack_bf16x2(oacc[dt][n][0] * inv, oacc[dt][n][1] * inv);
            wv[1] = pack_bf16x2(oacc[dt][n][2] * inv, oacc[dt][n][3] * inv);
            *(u32x2_t*)(orow + 16 * dt) = wv;
        }
    }
}

// ------------------------------------------------------------------ fp32
constexpr int PF32_TK = 32;  // keys per tile

template <int D>
__global__ __launch_bounds__(256) void prefill_f32_kernel(const float* __restrict__ q,
                                                          const float* __restrict__ k,
                                                          const float* __restrict__ v,
                                                          float* __restrict__ o, int B, int Hq,
                                                          int Hkv, int S, float c, int HPW,
                                                          int n_qblk, int n_hchunk, int rope,
                                                          RopeFreqs fr) {
    constexpr int DP = D / 4;  // dims per thread (4 threads per query row)
    __shared__ float ks[PF32_TK][D];
    __shared__ float vs[PF32_TK][D];

    const int G = Hq / Hkv;
    const int QPH = 64 / HPW;  // queries per head per workgroup
    const int per = B * Hkv * n_hchunk;
    const int qb = n_qblk - 1 - (int)blockIdx.x / per;
    const int rem = (int)blockIdx.x % per;
    const int bkv = rem % (B * Hkv), hc = rem / (B * Hkv);
    const int b = bkv / Hkv, kvh = bkv % Hkv;

    const int tid = threadIdx.x, slot = tid >> 2, part = tid & 3;
    const int h = kvh * G + hc * HPW + slot / QPH;
    const int qi = qb * QPH + slot % QPH;
    const size_t qo = ((size_t)(b * Hq + h) * S + qi) * D + part * DP;
    const float* const kg = k + (size_t)(b * Hkv + kvh) * S * D;
    const float* const vg = v + (size_t)(b * Hkv + kvh) * S * D;

    float qr[DP], acc[DP];
#pragma unroll
    for (int e = 0; e < DP; ++e) {
        qr[e] = qi < S ? q[qo + e] : 0.f;
        acc[e] = 0.f;
    }
    if (rope) {  // dims part*DP .. +DP-1 are whole channel pairs of query qi at position qi
#pragma unroll
        for (int e = 0; e < DP; e += 2) {
            float cs, sn, y0, y1;
            rope_cos_sin(qi, fr.f[(part * DP + e) / 2], cs, sn);
            rope_rotate(qr[e], qr[e + 1], cs, sn, y0, y1);
            qr[e] = y0;
            qr[e + 1] = y1;
        }
    }
    float m_run = -INFINITY, l_run = 0.f;

    const int kv_end = min(qb * QPH + QPH, S);
    const int ntiles = ceil_div(kv_end, PF32_TK);
    for (int t = 0; t < ntiles; ++t) {
        const int kv0 = t * PF32_TK;
        __syncthreads();
        for (int e = tid; e < PF32_TK * D; e += 256) {
            const int r = e / D, d = e % D, key = kv0 + r;
            ks[r][d] = key < S ? kg[(size_t)key * D + d] : 0.f;
            vs[r][d] = key < S ? vg[(size_t)key * D + d] : 0.f;
        }
        __syncthreads();
        for (int j = 0; j < PF32_TK; ++j) {
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < DP; ++e) dot = fmaf(qr[e], ks[j][part * DP + e], dot);
            dot += __shfl_xor(dot, 1, 64);
            dot += __shfl_xor(dot, 2, 64);
            if (kv0 + j <= qi) {
                const float mnew = fmaxf(m_run, dot);
                const float alpha = exp2f((m_run - mnew) * c);
                const float p = exp2f((dot - mnew) * c);
                l_run = l_run * alpha + p;
#pragma unroll
                for (int e = 0; e < DP; ++e) acc[e] = fmaf(p, vs[j][part * DP + e], acc[e] * alpha);
                m_run = mnew;
            }
        }
    }
    if (qi < S) {
        const float inv = 1.f / l_run;
#pragma unroll
        for (int e = 0; e < DP; ++e) o[qo + e] = acc[e] * inv;
    }
}

int largest_pow2_divisor(int g, int cap) {
    int hp = 1;
    while (hp * 2 <= cap && g % (hp * 2) == 0) hp *= 2;
    return hp;
}

template <int D, int HPW>
hipError_t launch_bf16(void* o, float* lse, const void* q, const void* k, const void* v, int B,
                       int Hq, int Hkv, int S, float c, double rope_theta, hipStream_t st) {
    constexpr int NQ = D == 64 ? PF_NQ64 : PF_NQ128;
    constexpr int QPB = (PF_NW / HPW) * 16 * NQ;
    const int G = Hq / Hkv;
    const int n_qblk = ceil_div(S, QPB), n_hchunk = G / HPW;
    const long long nblk = (long long)n_qblk * B * Hkv * n_hchunk;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, HPW, NQ>), dim3((unsigned)nblk), dim3(PF_THREADS), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse,
                       B, Hq, Hkv, S, c, n_qblk, n_hchunk, rope_theta > 0 ? 1 : 0,
                       rope_freqs(rope_theta > 0 ? rope_theta : 1.0, D));
    return hipGetLastError();
}

template <int D>
hipError_t launch_bf16_d(void* o, float* lse, const void* q, const void* k, const void* v, int B,
                         int Hq, int Hkv, int S, float c, double th, hipStream_t st) {
    // heads per workgroup: the largest power of two dividing G, at most one per wave
    const int hpw = largest_pow2_divisor(Hq / Hkv, PF_NW);
    if constexpr (PF_NW >= 8)
        if (hpw == 8) return launch_bf16<D, 8>(o, lse, q, k, v, B, Hq, Hkv, S, c, th, st);
    if (hpw >= 4) return launch_bf16<D, 4>(o, lse, q, k, v, B, Hq, Hkv, S, c, th, st);
    if (hpw == 2) return launch_bf16<D, 2>(o, lse, q, k, v, B, Hq, Hkv, S, c, th, st);
    return launch_bf16<D, 1>(o, lse, q, k, v, B, Hq, Hkv, S, c, th, st);
}

template <int D>
hipError_t launch_f32(void* o, const void* q, const void* k, const void* v, int B, int Hq, int Hkv,
                      int S, float c, double th, hipStream_t st) {
    const int G = Hq / Hkv;
    const int HPW = largest_pow2_divisor(G, 4);
    const int QPH = 64 / HPW;
    const int n_qblk = ceil_div(S, QPH), n_hchunk = G / HPW;
    const long long nblk = (long long)n_qblk * B * Hkv * n_hchunk;
    hipLaunchKernelGGL((prefill_f32_kernel<D>), dim3((unsigned)nblk), dim3(256), 0, st,
                       (const float*)q, (const float*)k, (const float*)v, (float*)o, B, Hq, Hkv, S,
                       c, HPW, n_qblk, n_hchunk, th > 0 ? 1 : 0, rope_freqs(th > 0 ? th : 1.0, D));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(void* o, float* lse, const void* q, const void* k, const void* v, int dtype,
                          int B, int Hq, int Hkv, int S, int D, float scale, double th,
                          hipStream_t st) {
    const float c = scale * kLog2e;
    if (dtype == kBF16)
        return D == 64 ? launch_bf16_d<64>(o, lse, q, k, v, B, Hq, Hkv, S, c, th, st)
                       : launch_bf16_d<128>(o, lse, q, k, v, B, Hq, Hkv, S, c, th, st);
    return D == 64 ? launch_f32<64>(o, q, k, v, B, Hq, Hkv, S, c, th, st)
                   : launch_f32<128>(o, q, k, v, B, Hq, Hkv, S, c, th, st);
}

}  // namespace attn
