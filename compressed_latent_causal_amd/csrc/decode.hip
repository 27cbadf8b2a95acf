// Single-token grouped-query decode over a contiguous KV cache, for gfx950.
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
// Split pass: per (sequence, KV head [, 16-head slice]) as many workgroups as
// the sequence's length needs (each covers at most 4 x 32 sub-tiles of 32
// tokens).  Sub-tile j goes to workgroup j % nwg and, inside it, to wave
// (j / nwg) % 4, so the running workgroups always read one contiguous front of
// the cache (HBM streams as for a plain copy) and ragged batches stay balanced.  Each
// byte of K and V is read once and serves all G query heads of the group.
// Per sub-tile:
//   * K rows are loaded straight from HBM into matrix-core operand registers
//     (16-byte loads; a wave instruction covers 16 rows x 64 contiguous bytes)
//     and S^T = K Q^T is one 16x16x32 bf16 product per 16 tokens x 32 dims,
//     with the group's query heads (padded to 16) as the N dimension;
//   * V rows are copied (16-byte loads, whole rows per lane group) into the
//     wave's own LDS slot and read back with the LDS transpose read as the A
//     operand of O^T = V^T P^T, P taken from registers as bf16;
//   * the softmax is online in fp32 (exp2 domain), one query head per lane.
// The four waves then merge in LDS and write one unnormalised partial
// (max, sum, o[D]) per (sequence, head, workgroup) to the fp32 workspace.
// Merge pass: one workgroup per (head, sequence) combines the chunk partials
// (log-sum-exp rescaling) and writes the bf16 output.  Cache slots at or past
// a sequence's length are never loaded.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr int DC_NW = 4;      // waves per split workgroup
constexpr int DC_SUB = 32;    // tokens per wave sub-tile
constexpr int DC_HEADS = 16;  // query heads per split workgroup (MFMA N)

#ifndef ATTN_DC_SUBS_PER_WAVE
#define ATTN_DC_SUBS_PER_WAVE 32
#endif
// Sub-tiles one split workgroup covers at most: each of its waves walks about
// ATTN_DC_SUBS_PER_WAVE sub-tiles, so a sequence of n_sub sub-tiles gets
// ceil(n_sub / DC_SUBS_PER_WG) workgroups (partials) and no workgroup's work
// exceeds that bound, whatever the mix of lengths.
constexpr int DC_SUBS_PER_WG = DC_NW * ATTN_DC_SUBS_PER_WAVE;

__host__ __device__ inline int decode_partials(int len) {
    return ceil_div(ceil_div(len, DC_SUB), DC_SUBS_PER_WG);
}

template <int D>
struct DecodeSmem {
    static constexpr int kStage = 2 * DC_NW * DC_SUB * D * 2;          // V staging, 2 slots per wave
    static constexpr int kOStride = D + 4;                             // padded row (floats)
    static constexpr int kMerge = (2 * DC_NW * DC_HEADS + DC_NW * DC_HEADS * kOStride) * 4;
    static constexpr int kBytes = kStage > kMerge ? kStage : kMerge;
};

template <int D>
__global__ __launch_bounds__(DC_NW * 64, 2) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ seqlens, float* __restrict__ ws_o, float* __restrict__ ws_ml, int Hq,
    int Hkv, int S_cap, int max_len, int NC, float c, int n_hchunk, int rope, RopeFreqs fr) {
    constexpr int KSTEPS = D / 32, DT = D / 16;
    constexpr int ROW = D * 2;                 // bytes per cache row
    constexpr int VSUB = DC_SUB * ROW;         // bytes of one V sub-tile
    constexpr int VINST = VSUB / 1024;         // 1 KiB LDS-DMA instructions per sub-tile
    constexpr int RPI = 1024 / ROW;            // rows per DMA instruction
    __shared__ __attribute__((aligned(16))) char smem[DecodeSmem<D>::kBytes];

    const int chunk = blockIdx.x, b = blockIdx.z;
    const int kvh = (int)blockIdx.y / n_hchunk, hc = (int)blockIdx.y % n_hchunk;
    const int G = Hq / Hkv;
    const int h0 = kvh * G + hc * DC_HEADS;
    const int GH = min(DC_HEADS, G - hc * DC_HEADS);
    const int len = min(max(seqlens[b], 0), max_len);
    const int n_sub = ceil_div(len, DC_SUB);  // 32-token sub-tiles of this sequence
    const int nwg = decode_partials(len);     // split workgroups of this sequence
    if (chunk >= nwg) return;  // uniform: the merge pass never reads this partial

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;

    // Q^T fragments (B operand, N = head): head h0 + lr (zero past the group), dims 32s + 8lg.
    bf16x8_t qf[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
        u32x4_t x = {0, 0, 0, 0};
        if (lr < GH) x = *(const u32x4_t*)(q + (size_t)(b * Hq + h0 + lr) * D + 32 * s + 8 * lg);
        if (rope) {
            // the new token sits at position len - 1; word e of x holds channel
            // pair 16s + 4lg + e
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float cs, sn, y0, y1;
                rope_cos_sin((long long)len - 1, fr.f[16 * s + 4 * lg + e], cs, sn);
                rope_rotate(bf16_lo(x[e]), bf16_hi(x[e]), cs, sn, y0, y1);
                x[e] = pack_bf16x2(y0, y1);
            }
        }
        qf[s] = __builtin_bit_cast(bf16x8_t, x);
    }

    const size_t kvb = (size_t)(b * Hkv + kvh) * S_cap * D;
    const uint16_t* const kg = kc + kvb;
    const uint16_t* const vg = vc + kvb;
    char* const vst = smem + w * 2 * VSUB;  // this wave's two V slots

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
    const int we = len;
    const int jstep = nwg * DC_NW;
    auto issue = [&](int j, char* slot, bf16x8_t (&kd)[2][KSTEPS]) {
        const int t0 = j * DC_SUB;
#pragma unroll
        for (int u = 0; u < VINST; ++u) {
            const int tok = min(t0 + vrow[u], we - 1);
            __builtin_amdgcn_global_load_lds((const void*)(vg + (size_t)tok * D + vcol[u] * 8),
                                             (__attribute__((address_space(3))) void*)(slot + u * 1024),
                                             16, 0, 0);
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int tok = min(t0 + 16 * mt + lr, we - 1);
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s)
                kd[mt][s] = *(const bf16x8_t*)(kg + (size_t)tok * D + 32 * s + 8 * lg);
        }
    };

    bf16x8_t kf[2][KSTEPS];
    int j = chunk + nwg * w;
    int cur = 0;
    if (j < n_sub) issue(j, vst, kf);
    for (; j < n_sub; j += jstep, cur ^= 1) {
        const int t0 = j * DC_SUB;
        const bool more = j + jstep < n_sub;
        // Always prefetch (the last sub-tile re-fetches itself, an L2 hit) so the
        // number of loads in flight is the same on every path and the waits
        // below can leave the prefetch outstanding.
        bf16x8_t kn[2][KSTEPS];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the slot was read by the previous PV
        issue(more ? j + jstep : j, vst + (cur ^ 1) * VSUB, kn);

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
                if (t0 + 16 * mt + 4 * lg + i >= we) sacc[mt][i] = -INFINITY;
                mx = fmaxf(mx, sacc[mt][i]);
            }
        mx = fmaxf(mx, xor_shfl(mx, 16));
        mx = fmaxf(mx, xor_shfl(mx, 32));
        const float mnew = fmaxf(m_run, mx);
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

        // this sub-tile's V DMA was issued before the prefetch's VINST + 2*KSTEPS
        // loads, and vector memory operations complete in order
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VINST + 2 * KSTEPS) : "memory");
        const char* const vcur = vst + cur * VSUB;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            oacc[dt] = mfma16(v_frag_at<D>(vcur + voff[dt]), pf, oacc[dt] * alpha);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) kf[mt][s] = kn[mt][s];
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the last (redundant) prefetch landed

    // ---- merge the four waves in LDS
    l_run += xor_shfl(l_run, 16);
    l_run += xor_shfl(l_run, 32);
    __syncthreads();  // all V staging reads are done
    float* const cm = (float*)smem;
    float* const cl = cm + DC_NW * DC_HEADS;
    float* const co = cl + DC_NW * DC_HEADS;
    constexpr int OS = DecodeSmem<D>::kOStride;
    if (lg == 0) {
        cm[w * DC_HEADS + lr] = m_run;
        cl[w * DC_HEADS + lr] = l_run;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        *(f32x4_t*)(co + (w * DC_HEADS + lr) * OS + 16 * dt + 4 * lg) = oacc[dt];
    __syncthreads();
    for (int e = tid; e < GH * D; e += DC_NW * 64) {
        const int hd = e / D, d = e % D;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < DC_NW; ++ww) M = fmaxf(M, cm[ww * DC_HEADS + hd]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int ww = 0; ww < DC_NW; ++ww) {
            const float mw = cm[ww * DC_HEADS + hd];
            const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((mw - M) * c);
            L += f * cl[ww * DC_HEADS + hd];
            O += f * co[(ww * DC_HEADS + hd) * OS + d];
        }
        const size_t slot = (size_t)(b * Hq + h0 + hd) * NC + chunk;
        ws_o[slot * D + d] = O;
        if (d == 0) {
            ws_ml[slot * 2] = M;
            ws_ml[slot * 2 + 1] = L;
        }
    }
}

constexpr int MG_NW = 16;  // waves per merge workgroup
constexpr int MG_UNROLL = 8;

template <int D>
__global__ __launch_bounds__(MG_NW * 64) void decode_merge_kernel(const float* __restrict__ ws_o,
                                                                 const float* __restrict__ ws_ml,
                                                                 const int32_t* __restrict__ seqlens,
                                                                 uint16_t* __restrict__ o, int Hq,
                                                                 int max_len, int NC, float c) {
    constexpr int EPL = D / 64;  // output dims per lane
    __shared__ float sm[MG_NW], sl[MG_NW];
    __shared__ float so[MG_NW][D];
    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int len = min(max(seqlens[b], 0), max_len);
    const int nc = decode_partials(len);  // partials the split pass wrote (<= NC)
    const size_t base = (size_t)(b * Hq + h) * NC;

    // wave w folds chunks w, w + 16, ...; MG_UNROLL independent loads in flight
    float M = -INFINITY, L = 0.f, acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    for (int ch0 = w; ch0 < nc; ch0 += MG_NW * MG_UNROLL) {
        float mc[MG_UNROLL], lc[MG_UNROLL], oc[MG_UNROLL][EPL];
#pragma unroll
        for (int u = 0; u < MG_UNROLL; ++u) {
            const int ch = ch0 + u * MG_NW;
            mc[u] = -INFINITY;
            lc[u] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) oc[u][e] = 0.f;
            if (ch < nc) {
                mc[u] = ws_ml[(base + ch) * 2];
                lc[u] = ws_ml[(base + ch) * 2 + 1];
#pragma unroll
                for (int e = 0; e < EPL; ++e) oc[u][e] = ws_o[(base + ch) * D + lane * EPL + e];
            }
        }
#pragma unroll
        for (int u = 0; u < MG_UNROLL; ++u) {
            if (mc[u] == -INFINITY) continue;
            const float Mn = fmaxf(M, mc[u]);
            const float a = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((M - Mn) * c);
            const float f = __builtin_amdgcn_exp2f((mc[u] - Mn) * c);
            L = L * a + lc[u] * f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] = acc[e] * a + f * oc[u][e];
            M = Mn;
        }
    }
    if (lane == 0) {
        sm[w] = M;
        sl[w] = L;
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) so[w][lane * EPL + e] = acc[e];
    __syncthreads();
    if (w != 0) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < MG_NW; ++ww) Mt = fmaxf(Mt, sm[ww]);
    float Lt = 0.f, out[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[e] = 0.f;
#pragma unroll
    for (int ww = 0; ww < MG_NW; ++ww) {
        const float f = (sm[ww] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((sm[ww] - Mt) * c);
        Lt += f * sl[ww];
#pragma unroll
        for (int e = 0; e < EPL; ++e) out[e] += f * so[ww][lane * EPL + e];
    }
    const float inv = (len > 0) ? 1.f / Lt : 0.f;
    uint16_t* const dst = o + (size_t)(b * Hq + h) * D + lane * EPL;
    if constexpr (EPL == 2) {
        *(unsigned*)dst = pack_bf16x2(out[0] * inv, out[1] * inv);
    } else {
        dst[0] = (uint16_t)(pack_bf16x2(out[0] * inv, 0.f) & 0xffffu);
    }
}

template <int D>
hipError_t launch_decode_d(void* o, const void* q, const void* k_cache, const void* v_cache, int B,
                           int Hq, int Hkv, int S_cap, const int32_t* seqlens, int max_len, float c,
                           double rope_theta, void* workspace, hipStream_t st) {
    const int NC = decode_num_chunks(B, Hkv, max_len);
    const int G = Hq / Hkv;
    const int n_hchunk = ceil_div(G, DC_HEADS);
    float* const ws_o = (float*)workspace;
    float* const ws_ml = ws_o + (size_t)B * Hq * NC * D;
    if (max_len > 0) {
        hipLaunchKernelGGL((decode_split_kernel<D>), dim3(NC, Hkv * n_hchunk, B), dim3(DC_NW * 64), 0,
                           st, (const uint16_t*)q, (const uint16_t*)k_cache,
                           (const uint16_t*)v_cache, seqlens, ws_o, ws_ml, Hq, Hkv, S_cap, max_len,
                           NC, c, n_hchunk, rope_theta > 0 ? 1 : 0,
                           rope_freqs(rope_theta > 0 ? rope_theta : 1.0, D));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(Hq, B), dim3(MG_NW * 64), 0, st, ws_o, ws_ml, seqlens,
                       (uint16_t*)o, Hq, max_len, NC, c);
    return hipGetLastError();
}

}  // namespace

int decode_num_chunks(int B, int Hkv, int max_len) {
    // workspace slots per (sequence, head): the partial count of the longest sequence
    return max(1, decode_partials(max_len));
}

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int max_len, int D) {
    const size_t NC = (size_t)decode_num_chunks(B, Hkv, max_len);
    return (size_t)B * Hq * NC * (size_t)(D + 2) * sizeof(float);
}

hipError_t launch_decode(void* o, const void* q, const void* k_cache, const void* v_cache, int B,
                         int Hq, int Hkv, int S_cap, int D, const int32_t* seqlens, int max_len,
                         float scale, double rope_theta, void* workspace, hipStream_t st) {
    const float c = scale * kLog2e;
    return D == 64 ? launch_decode_d<64>(o, q, k_cache, v_cache, B, Hq, Hkv, S_cap, seqlens, max_len,
                                         c, rope_theta, workspace, st)
                   : launch_decode_d<128>(o, q, k_cache, v_cache, B, Hq, Hkv, S_cap, seqlens, max_len,
                                          c, rope_theta, workspace, st);
}

}  // namespace attn
