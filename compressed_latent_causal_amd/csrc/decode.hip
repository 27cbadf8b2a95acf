// Single-token grouped-query decode over a contiguous KV cache, for gfx950.
//
// What is computed ("Grouped Query Attention (GQA)" glossary, sections "Cómo
// funciona GQA" and "Por qué GQA reduce la caché KV"): each sequence's new
// query token attends, head by head, to every valid cached key/value of its
// KV group.  The whole valid cache is read once per token, so the kernel is
// bound by HBM bandwidth and its traffic scales with Hkv, not Hq.
//
// Split pass: one workgroup per (key chunk, KV head [, 16-head slice], batch).
// It streams its chunk of K and V once and serves all G query heads of the
// group from the same bytes.  Four waves split the chunk; each walks 32-token
// sub-tiles:
//   * K rows are loaded straight from HBM into matrix-core operand registers
//     (16-byte loads; a wave instruction covers 16 rows x 64 contiguous bytes)
//     and S^T = K Q^T is one 16x16x32 bf16 product per 16 tokens x 32 dims,
//     with the group's query heads (padded to 16) as the N dimension;
//   * V rows are copied (16-byte loads, whole rows per lane group) into the
//     wave's own LDS slot and read back with the LDS transpose read as the A
//     operand of O^T = V^T P^T, P taken from registers as bf16;
//   * the softmax is online in fp32 (exp2 domain), one query head per lane.
// The four waves then merge in LDS and write one unnormalised partial
// (max, sum, o[D]) per (sequence, head, chunk) to the fp32 workspace.
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

template <int D>
struct DecodeSmem {
    static constexpr int kStage = DC_NW * DC_SUB * D * 2;              // V staging
    static constexpr int kOStride = D + 4;                             // padded row (floats)
    static constexpr int kMerge = (2 * DC_NW * DC_HEADS + DC_NW * DC_HEADS * kOStride) * 4;
    static constexpr int kBytes = kStage > kMerge ? kStage : kMerge;
};

template <int D>
__global__ __launch_bounds__(DC_NW * 64) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ seqlens, float* __restrict__ ws_o, float* __restrict__ ws_ml, int Hq,
    int Hkv, int S_cap, int max_len, int T, int NC, float c, int n_hchunk) {
    constexpr int CH = D / 8, KSTEPS = D / 32, DT = D / 16;
    constexpr int VSUB = DC_SUB * D * 2;
    constexpr int VCPL = DC_SUB * CH / 64;  // V chunks per lane per sub-tile
    __shared__ __attribute__((aligned(16))) char smem[DecodeSmem<D>::kBytes];

    const int chunk = blockIdx.x, b = blockIdx.z;
    const int kvh = (int)blockIdx.y / n_hchunk, hc = (int)blockIdx.y % n_hchunk;
    const int G = Hq / Hkv;
    const int h0 = kvh * G + hc * DC_HEADS;
    const int GH = min(DC_HEADS, G - hc * DC_HEADS);
    const int len = min(max(seqlens[b], 0), max_len);
    const int t_begin = chunk * T;
    if (t_begin >= len) return;  // uniform: the merge pass never reads this chunk
    const int t_end = min(t_begin + T, len);

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int TW = T / DC_NW;
    const int wb = t_begin + w * TW, we = min(wb + TW, t_end);

    // Q^T fragments (B operand, N = head): head h0 + lr (zero past the group), dims 32s + 8lg.
    bf16x8_t qf[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
        u32x4_t x = {0, 0, 0, 0};
        if (lr < GH) x = *(const u32x4_t*)(q + (size_t)(b * Hq + h0 + lr) * D + 32 * s + 8 * lg);
        qf[s] = __builtin_bit_cast(bf16x8_t, x);
    }

    const size_t kvb = (size_t)(b * Hkv + kvh) * S_cap * D;
    const uint16_t* const kg = kc + kvb;
    const uint16_t* const vg = vc + kvb;
    char* const vst = smem + w * VSUB;

    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4_t{0, 0, 0, 0};

    // K operand of a sub-tile: token t0 + 16mt + lr, dims 32s + 8lg .. +7 (zero
    // past the valid range).  V rows: chunk lane + 64u of the 32 x D sub-tile.
    bf16x8_t kf[2][KSTEPS];
    u32x4_t vr[VCPL];
    auto load_sub = [&](int t0, bf16x8_t (&kd)[2][KSTEPS], u32x4_t (&vd)[VCPL]) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int tok = t0 + 16 * mt + lr;
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                u32x4_t x = {0, 0, 0, 0};
                if (tok < we) x = *(const u32x4_t*)(kg + (size_t)tok * D + 32 * s + 8 * lg);
                kd[mt][s] = __builtin_bit_cast(bf16x8_t, x);
            }
        }
#pragma unroll
        for (int u = 0; u < VCPL; ++u) {
            const int ci = lane + 64 * u, r = ci / CH, cc = ci % CH;
            const int tok = t0 + r;
            vd[u] = u32x4_t{0, 0, 0, 0};
            if (tok < we) vd[u] = *(const u32x4_t*)(vg + (size_t)tok * D + cc * 8);
        }
    };
    if (wb < we) load_sub(wb, kf, vr);

    for (int t0 = wb; t0 < we; t0 += DC_SUB) {
        // the loads of the next sub-tile stay in flight while this one is computed
        bf16x8_t kn[2][KSTEPS];
        u32x4_t vn[VCPL];
        const bool more = t0 + DC_SUB < we;
        if (more) load_sub(t0 + DC_SUB, kn, vn);

        // the previous sub-tile's transpose reads must be done before overwriting
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int u = 0; u < VCPL; ++u) {
            const int ci = lane + 64 * u, r = ci / CH, cc = ci % CH;
            *(u32x4_t*)(vst + swz_v<D>(r, cc)) = vr[u];
        }

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
        l_run = l_run * alpha + ls;
        m_run = mnew;
        u32x4_t pw;
        pw[0] = pack_bf16x2(sacc[0][0], sacc[0][1]);
        pw[1] = pack_bf16x2(sacc[0][2], sacc[0][3]);
        pw[2] = pack_bf16x2(sacc[1][0], sacc[1][1]);
        pw[3] = pack_bf16x2(sacc[1][2], sacc[1][3]);
        const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pw);

        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // V rows are in LDS
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const bf16x8_t a = v_frag_at<D>(vst + v_frag_off<D>(dt, lane));
            oacc[dt] = mfma16(a, pf, oacc[dt] * alpha);
        }
        if (more) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int s = 0; s < KSTEPS; ++s) kf[mt][s] = kn[mt][s];
#pragma unroll
            for (int u = 0; u < VCPL; ++u) vr[u] = vn[u];
        }
    }

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
constexpr int MG_UNROLL = 4;

template <int D>
__global__ __launch_bounds__(MG_NW * 64) void decode_merge_kernel(const float* __restrict__ ws_o,
                                                                 const float* __restrict__ ws_ml,
                                                                 const int32_t* __restrict__ seqlens,
                                                                 uint16_t* __restrict__ o, int Hq,
                                                                 int max_len, int T, int NC, float c) {
    constexpr int EPL = D / 64;  // output dims per lane
    __shared__ float sm[MG_NW], sl[MG_NW];
    __shared__ float so[MG_NW][D];
    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int len = min(max(seqlens[b], 0), max_len);
    const int nc = ceil_div(len, T);
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
                           void* workspace, hipStream_t st) {
    const int T = decode_chunk_tokens(B, Hkv, max_len);
    const int NC = decode_num_chunks(B, Hkv, max_len);
    const int G = Hq / Hkv;
    const int n_hchunk = ceil_div(G, DC_HEADS);
    float* const ws_o = (float*)workspace;
    float* const ws_ml = ws_o + (size_t)B * Hq * NC * D;
    if (max_len > 0) {
        hipLaunchKernelGGL((decode_split_kernel<D>), dim3(NC, Hkv * n_hchunk, B), dim3(DC_NW * 64), 0,
                           st, (const uint16_t*)q, (const uint16_t*)k_cache,
                           (const uint16_t*)v_cache, seqlens, ws_o, ws_ml, Hq, Hkv, S_cap, max_len,
                           T, NC, c, n_hchunk);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(Hq, B), dim3(MG_NW * 64), 0, st, ws_o, ws_ml, seqlens,
                       (uint16_t*)o, Hq, max_len, T, NC, c);
    return hipGetLastError();
}

}  // namespace

int decode_chunk_tokens(int B, int Hkv, int max_len) {
    // Long enough to amortise the per-chunk partial (D+2 floats per head), short
    // enough to give the chip several waves of workgroups.
    int T = 512;
    while (T > 128 && (long long)B * Hkv * ceil_div(max_len, T) < 2048) T /= 2;
    return T;
}

int decode_num_chunks(int B, int Hkv, int max_len) {
    return max_len > 0 ? ceil_div(max_len, decode_chunk_tokens(B, Hkv, max_len)) : 1;
}

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int max_len, int D) {
    const size_t NC = (size_t)decode_num_chunks(B, Hkv, max_len);
    return (size_t)B * Hq * NC * (size_t)(D + 2) * sizeof(float);
}

hipError_t launch_decode(void* o, const void* q, const void* k_cache, const void* v_cache, int B,
                         int Hq, int Hkv, int S_cap, int D, const int32_t* seqlens, int max_len,
                         float scale, void* workspace, hipStream_t st) {
    const float c = scale * kLog2e;
    return D == 64 ? launch_decode_d<64>(o, q, k_cache, v_cache, B, Hq, Hkv, S_cap, seqlens, max_len,
                                         c, workspace, st)
                   : launch_decode_d<128>(o, q, k_cache, v_cache, B, Hq, Hkv, S_cap, seqlens, max_len,
                                          c, workspace, st);
}

}  // namespace attn
