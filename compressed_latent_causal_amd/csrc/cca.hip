// CCA pre-attention operations on the compressed q, k, v, for gfx950.
//
// What is computed ("Compressed Convolutional Attention" summary, section
// "Methodologie", items 2 to 4; the summary names the operations without
// their sizes, so each is taken in its plainest form):
//  * sequence mixing: a causal depthwise convolution of width W over the
//    sequence, per channel of every head, s[t,c] = sum_{i<W} w[h,c,i] x[t-i,c]
//    (tap i weighs the token i steps back; tokens before the first are zero);
//  * channel mixing within a head: a dense D x D map per head,
//    z[t,c] = sum_c' M[h,c,c'] s[t,c'] (row c of M is output channel c);
//  * QK-mean: the mean of a token's pre-convolution query and key, the query
//    heads of a KV group averaged first, m[t,j] = (mean_h q~[t,h] + k~[t,j]) / 2,
//    added to every convolved q head of the group and to its k head;
//  * RoPE of those q and k at absolute position pos_offset[b] + t (the same
//    device code as attn_rope);
//  * value shift: each head's value takes its first D/2 channels from the
//    current token and its last D/2 from the previous one (zero at t = 0).
//
// Design.  One workgroup = 4 waves = one (sequence, KV group, 64-token block);
// wave w owns 16 tokens and walks the group's G query heads and its key head.
// Per head and wave, the 16 x D result is one matrix-core product,
// Z^T = M S^T with the 16x16x32 bf16 instruction: the A operand is M, staged in
// LDS once per workgroup and head by buffer loads that write LDS directly
// (double-buffered across heads, so head n+1's matrix streams in while head n
// is computed); the B operand is S^T, the convolution's output, which each lane
// forms in fp32 for its token and 8 channels per k-step.  The convolution's
// earlier tokens come from the lanes below in the same 16-lane row (DPP row
// shifts), the W - 1 rows before the wave's first token from a second load of
// the previous 16 rows (DPP row rotates).  S is split into bf16 high and low
// parts and both are multiplied, so the product is accurate to about 2^-17 of
// its terms: the result is the fp32-accurate value, rounded once to bf16.
// In the result layout each lane holds 4 consecutive channels of one token,
// so the mean is added, channel pairs are rotated in registers and 8 bytes
// are stored per lane.  The next head's input rows are loaded while the
// current head is computed.  The kernel is bound by HBM (it reads and writes
// q, k and v once) and by the vector work of the convolution.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr int CM_NW = 4;               // waves per workgroup
constexpr int CM_TW = 16;              // tokens per wave
constexpr int CM_TB = CM_NW * CM_TW;   // tokens per workgroup
constexpr int CM_MAXW = 8;             // widest sequence convolution

// s_waitcnt immediate: vmcnt(n) and lgkmcnt(0)
constexpr int wait_vmcnt_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70; }

// x of the lane SH places lower in the same 16-lane row; lanes with none keep `low`
template <int SH>
__device__ inline unsigned row_shift_in(unsigned x, unsigned low) {
    return (unsigned)__builtin_amdgcn_update_dpp((int)low, (int)x, 0x110 + SH, 0xF, 0xF, false);
}
// x of the lane SH places lower in the same 16-lane row, cyclically
template <int SH>
__device__ inline unsigned row_rotate(unsigned x) {
    return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x120 + SH, 0xF, 0xF, false);
}


// Input rows of one head as one vector value (dword 4 s + e of k-step s), so
// they stay in registers across the head loop.
template <int N>
struct DwordVec {
    typedef unsigned type __attribute__((ext_vector_type(N)));
};
template <int D>
using RowsVec = typename DwordVec<D / 8>::type;

// Tap I of the sequence convolution for this lane's token t and channels
// 32 s + 8 g + e: y += w[I][c] x[t - I, c].  Row t - I sits in lane r - I of
// the same 16-lane row, or, for r < I, in lane r - I + 16 of the previous 16
// rows.
template <int D, int I>
__device__ __attribute__((always_inline)) inline void conv_tap(float (&y)[D / 32][8],
                                                               const RowsVec<D>& cur,
                                                               const RowsVec<D>& prv,
                                                               const float* wsm, int g) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
        u32x4_t x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (I == 0)
                x[e] = cur[4 * s + e];
            else
                x[e] = row_shift_in<I>(cur[4 * s + e], row_rotate<I>(prv[4 * s + e]));
        }
        const f32x4_t w0 = *(const f32x4_t*)(wsm + I * D + 32 * s + 8 * g);
        const f32x4_t w1 = *(const f32x4_t*)(wsm + I * D + 32 * s + 8 * g + 4);
        const float wv[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            y[s][2 * e] = fmaf(wv[2 * e], bf16_lo(x[e]), y[s][2 * e]);
            y[s][2 * e + 1] = fmaf(wv[2 * e + 1], bf16_hi(x[e]), y[s][2 * e + 1]);
        }
    }
}

template <int D>
__global__ __launch_bounds__(CM_NW * 64, 2) void cca_mix_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ qo, uint16_t* __restrict__ ko, uint16_t* __restrict__ vo,
    const uint16_t* __restrict__ conv_q, const uint16_t* __restrict__ conv_k, int W,
    const uint16_t* __restrict__ mix_q, const uint16_t* __restrict__ mix_k,
    const int32_t* __restrict__ pos_offset, int rope, RopeFreqs fr, int Hq, int Hkv, int S,
    int n_tblk) {
    constexpr int KS = D / 32;          // k-steps of Z^T = M S^T
    constexpr int MT = D / 16;          // 16-channel output tiles
    constexpr int ROW = D * 2;          // bytes per bf16 row
    constexpr int MBYTES = D * ROW;     // one head's mix matrix
    constexpr int MINST = MBYTES / 1024 / CM_NW;  // 1 KiB LDS-DMA instructions per wave
    static_assert(MINST >= 1, "mix matrix split");

    __shared__ __attribute__((aligned(1024))) char msm0[MBYTES];
    __shared__ __attribute__((aligned(1024))) char msm1[MBYTES];
    __shared__ float wsm0[CM_MAXW * D];  // conv taps as fp32, [tap][channel]
    __shared__ float wsm1[CM_MAXW * D];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int tblk = (int)blockIdx.x % n_tblk;
    const int bj = (int)blockIdx.x / n_tblk;
    const int b = bj / Hkv, j = bj % Hkv;
    const int G = Hq / Hkv;
    const int NH = G + 1;  // the group's query heads, then its key head
    const int t0w = tblk * CM_TB + w * CM_TW;  // the wave's first token
    const int t = t0w + r;                     // this lane's token

    auto head_rows = [&](int n) -> const uint16_t* {
        return n < G ? q + ((size_t)b * Hq + (size_t)j * G + n) * S * D
                     : k + ((size_t)b * Hkv + j) * S * D;
    };
    auto head_out = [&](int n) -> uint16_t* {
        return n < G ? qo + ((size_t)b * Hq + (size_t)j * G + n) * S * D
                     : ko + ((size_t)b * Hkv + j) * S * D;
    };
    auto head_mix = [&](int n) -> const uint16_t* {
        return n < G ? mix_q + ((size_t)j * G + n) * D * D : mix_k + (size_t)j * D * D;
    };
    auto head_conv = [&](int n) -> const uint16_t* {
        return n < G ? conv_q + ((size_t)j * G + n) * D * W : conv_k + (size_t)j * D * W;
    };

    // This head's input rows and taps, replaced by the next head's once consumed:
    // row t (this lane's token) and row t - 16 (rows before the wave's first
    // token), channels 32 s + 8 g .. +7, and 16 bytes of the head's conv taps
    // [D][W] (threads tid < D W / 8).
    RowsVec<D> in_cur, in_prv;
    u32x4_t in_wc;
    auto put = [&](RowsVec<D>& dst, int s, u32x4_t x) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[4 * s + e] = x[e];
    };
    // Loads of head n: this wave's share of the mix matrix straight into LDS
    // (swz_k layout: instruction u puts lane l's 16 bytes at physical chunk
    // 64 (w MINST + u) + l, i.e. row pr, chunk pc, which holds logical chunk
    // pc ^ f(pr)), the conv taps of channel tid, and the lane's input rows.
    auto issue_matrix = [&](int n, char* msm) __attribute__((always_inline)) {
        const uint16_t* const mx = head_mix(n);
#pragma unroll
        for (int u = 0; u < MINST; ++u) {
            const int P = (w * MINST + u) * 64 + lane;
            const int pr = P / (D / 8), pc = P % (D / 8);
            const int lc = (swz_k<D>(pr, pc) - pr * ROW) >> 4;  // the XOR swizzle is an involution
            __builtin_amdgcn_global_load_lds((const void*)(mx + (size_t)pr * D + lc * 8),
                                             (__attribute__((address_space(3))) void*)(msm + (w * MINST + u) * 1024),
                                             16, 0, 0);
        }
    };
    auto issue_rows = [&](int n) __attribute__((always_inline)) {
        // Every load below is issued by every lane (buffer loads: an offset
        // past the resource reads zeros), so the number of loads in flight is
        // fixed and the waits can count them.  The taps come as raw bf16, 16
        // bytes per thread (threads past D W / 8 read zeros), and are unpacked
        // once they have landed.
        const __amdgpu_buffer_rsrc_t crs = buffer_rsrc(head_conv(n), D * W * 2);
        in_wc = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, 16 * tid, 0, 0));
        const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(head_rows(n), S * ROW);
        // rows before the wave's first token: only the last W - 1 lanes of a
        // row supply them, and none before the sequence's first token
        const bool use_prv = t0w > 0 && r >= CM_TW - (W - 1);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int cb = (32 * s + 8 * g) * 2;
            put(in_cur, s, __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xrs, t * ROW + cb, 0, 0)));
            put(in_prv, s, __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xrs, use_prv ? (t - CM_TW) * ROW + cb : -16, 0, 0)));
        }
    };

    // Loads of the value shift, issued during the last head: the workgroup's
    // 64 rows x D/8 chunks, KS per thread (zero for the row before the first)
    constexpr int CPR = D / 8;  // 16-byte chunks per row
    static_assert(CM_TB * CPR == KS * CM_NW * 64, "value chunks per thread");
    u32x4_t vsh[KS];
    auto issue_vshift = [&]() __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(v + ((size_t)b * Hkv + j) * S * D, S * ROW);
#pragma unroll
        for (int u = 0; u < KS; ++u) {
            const int e = tid + u * CM_NW * 64;
            const int tt = tblk * CM_TB + e / CPR, c = e % CPR;
            const int src = c < CPR / 2 ? tt : tt - 1;  // row -1 lies outside: zeros
            vsh[u] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vrs, src >= 0 ? (src * D + 8 * c) * 2 : -16, 0, 0));
        }
    };

    // ---- the token's QK-mean (result layout: channels 16 mt + 4 g + i) and,
    // with RoPE, the cosines and sines of its channel pairs
    f32x4_t mean[MT];
    {
        f32x4_t qs[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) qs[mt] = f32x4_t{0, 0, 0, 0};
        // query heads four at a time, all loads of a batch issued before any
        // is used (heads past G re-read the last one and weigh nothing)
        const size_t trow = (size_t)min(t, S - 1) * D + 4 * g;
        for (int h0 = 0; h0 < G; h0 += 4) {
            u32x2_t x[4][MT];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint16_t* const xr = head_rows(min(h0 + u, G - 1)) + trow;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) x[u][mt] = *(const u32x2_t*)(xr + 16 * mt);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float f = h0 + u < G ? 1.f : 0.f;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    qs[mt] += f * f32x4_t{bf16_lo(x[u][mt][0]), bf16_hi(x[u][mt][0]),
                                          bf16_lo(x[u][mt][1]), bf16_hi(x[u][mt][1])};
            }
        }
        const float inv_g = 1.f / (float)G;
        const uint16_t* const kr = head_rows(G) + trow;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const u32x2_t x = *(const u32x2_t*)(kr + 16 * mt);
            const f32x4_t kv = {bf16_lo(x[0]), bf16_hi(x[0]), bf16_lo(x[1]), bf16_hi(x[1])};
            mean[mt] = 0.5f * (qs[mt] * inv_g + kv);
        }
    }
    float cs[MT][2], sn[MT][2];
    if (rope) {
        const long long p = (long long)(pos_offset ? pos_offset[b] : 0) + t;
        double fq[MT][2];  // gathered first, so the loads overlap
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e) fq[mt][e] = fr.f[8 * mt + 2 * g + e];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e) rope_cos_sin(p, fq[mt][e], cs[mt][e], sn[mt][e]);
    }

    // ---- one head: convolution, channel mix, mean, RoPE, store
    auto body = [&](int n, const char* msm, float* wsm, char* msm_next) __attribute__((always_inline)) {
        // This head's loads were issued before the previous head's MT result
        // stores, the last vector-memory operations before this point (the
        // stores are unconditional buffer stores, so their number is fixed);
        // the first head waits for everything.
        __builtin_amdgcn_sched_barrier(0);
        if (n == 0)
            __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
        else
            __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(MT));
        __builtin_amdgcn_sched_barrier(0);
        if (tid < D * W / 8) {
            // taps element e of the thread's 8: channel (8 tid + e) / W, tap (8 tid + e) % W
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int idx = 8 * tid + e;
                const unsigned wd = in_wc[e / 2];
                wsm[(idx % W) * D + idx / W] = (e & 1) ? bf16_hi(wd) : bf16_lo(wd);
            }
        }
        // every wave's share of the matrix and the taps are in LDS, and every
        // wave is done with head n - 1 (whose buffers the next loads reuse)
        __syncthreads();
        if (n + 1 < NH) issue_matrix(n + 1, msm_next);
        __builtin_amdgcn_sched_barrier(0);  // the copy stays ahead of this head's work

        // S^T fragments: y[s][e] = channel 32 s + 8 g + e of token t
        float y[KS][8];
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) y[s][e] = 0.f;
        conv_tap<D, 0>(y, in_cur, in_prv, wsm, g);
        if (W > 1) conv_tap<D, 1>(y, in_cur, in_prv, wsm, g);
        if (W > 2) conv_tap<D, 2>(y, in_cur, in_prv, wsm, g);
        if (W > 3) conv_tap<D, 3>(y, in_cur, in_prv, wsm, g);
        if (W > 4) conv_tap<D, 4>(y, in_cur, in_prv, wsm, g);
        if (W > 5) conv_tap<D, 5>(y, in_cur, in_prv, wsm, g);
        if (W > 6) conv_tap<D, 6>(y, in_cur, in_prv, wsm, g);
        if (W > 7) conv_tap<D, 7>(y, in_cur, in_prv, wsm, g);
        // bf16 high and low parts of S^T
        bf16x8_t yh[KS], yl[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4_t h4, l4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h4[e] = pack_bf16x2(y[s][2 * e], y[s][2 * e + 1]);
                l4[e] = pack_bf16x2(y[s][2 * e] - bf16_lo(h4[e]), y[s][2 * e + 1] - bf16_hi(h4[e]));
            }
            yh[s] = __builtin_bit_cast(bf16x8_t, h4);
            yl[s] = __builtin_bit_cast(bf16x8_t, l4);
        }
        // the input registers are consumed: load the next head's rows (or,
        // after the last head, the value shift's) while this head's products run
        __builtin_amdgcn_sched_barrier(0);
        if (n + 1 < NH)
            issue_rows(n + 1);
        else
            issue_vshift();
        __builtin_amdgcn_sched_barrier(0);
        // Z^T = M S^T; lane gets channels 16 mt + 4 g + i of token t.  Stores
        // go through a buffer resource over the head's rows, which drops those
        // of tokens past the end, so every lane issues every store.
        const __amdgpu_buffer_rsrc_t ors = buffer_rsrc(head_out(n), S * ROW);
        const int obyte = (t * D + 4 * g) * 2;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f32x4_t acc = {0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const bf16x8_t a = *(const bf16x8_t*)(msm + swz_k<D>(16 * mt + r, 4 * s + g));
                acc = mfma16(a, yh[s], acc);
                acc = mfma16(a, yl[s], acc);
            }
            acc += mean[mt];
            if (rope) {
                float y0, y1, y2, y3;
                rope_rotate(acc[0], acc[1], cs[mt][0], sn[mt][0], y0, y1);
                rope_rotate(acc[2], acc[3], cs[mt][1], sn[mt][1], y2, y3);
                acc = f32x4_t{y0, y1, y2, y3};
            }
            __builtin_amdgcn_raw_buffer_store_b64(
                u32x2_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])}, ors,
                obyte + 32 * mt, 0, 0);
        }
    };

    issue_matrix(0, msm0);
    issue_rows(0);
    __builtin_amdgcn_sched_barrier(0);
    int n = 0;
    // unrolled by two so each step names its LDS buffers statically
    for (; n + 1 < NH; n += 2) {
        body(n, msm0, wsm0, msm1);
        body(n + 1, msm1, wsm1, msm0);
    }
    if (n < NH) body(n, msm0, wsm0, msm1);

    // ---- value shift of the block's rows: chunk c of row tt comes from row
    // tt for channels below D/2 and from row tt - 1 above (stores past the
    // end are dropped by the buffer resource)
    const __amdgpu_buffer_rsrc_t vws = buffer_rsrc(vo + ((size_t)b * Hkv + j) * S * D, S * ROW);
#pragma unroll
    for (int u = 0; u < KS; ++u) {
        const int e = tid + u * CM_NW * 64;
        const int tt = tblk * CM_TB + e / CPR, c = e % CPR;
        __builtin_amdgcn_raw_buffer_store_b128(vsh[u], vws, (tt * D + 8 * c) * 2, 0, 0);
    }

}

template <int D>
hipError_t launch_cca_mix_d(void* q_out, void* k_out, void* v_out, const void* q, const void* k,
                            const void* v, int B, int Hq, int Hkv, int S, const void* conv_q,
                            const void* conv_k, int W, const void* mix_q, const void* mix_k,
                            const int32_t* pos_offset, double rope_theta, hipStream_t st) {
    const int n_tblk = ceil_div(S, CM_TB);
    const long long nblocks = (long long)n_tblk * B * Hkv;
    if (nblocks > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((cca_mix_kernel<D>), dim3((unsigned)nblocks), dim3(CM_NW * 64), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)q_out,
                       (uint16_t*)k_out, (uint16_t*)v_out, (const uint16_t*)conv_q,
                       (const uint16_t*)conv_k, W, (const uint16_t*)mix_q, (const uint16_t*)mix_k,
                       pos_offset, rope_theta > 0 ? 1 : 0,
                       rope_freqs(rope_theta > 0 ? rope_theta : 1.0, D), Hq, Hkv, S, n_tblk);
    return hipGetLastError();
}

}  // namespace

int cca_max_width() { return CM_MAXW; }

hipError_t launch_cca_mix(void* q_out, void* k_out, void* v_out, const void* q, const void* k,
                          const void* v, int B, int Hq, int Hkv, int S, int D, const void* conv_q,
                          const void* conv_k, int W, const void* mix_q, const void* mix_k,
                          const int32_t* pos_offset, double rope_theta, hipStream_t st) {
    return D == 64 ? launch_cca_mix_d<64>(q_out, k_out, v_out, q, k, v, B, Hq, Hkv, S, conv_q,
                                          conv_k, W, mix_q, mix_k, pos_offset, rope_theta, st)
                   : launch_cca_mix_d<128>(q_out, k_out, v_out, q, k, v, B, Hq, Hkv, S, conv_q,
                                           conv_k, W, mix_q, mix_k, pos_offset, rope_theta, st);
}

}  // namespace attn
