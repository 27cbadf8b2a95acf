// CCA pre-attention operations on the compressed q, k, v, for gfx950.
//
// What is computed ("Compressed Convolutional Attention" summary, section
// "Methodologie", items 2 to 4; the summary names the operations without
// their sizes, so each is taken in its plainest form):
//  * sequence mixing: a causal depthwise convolution of width W over the
//    sequence, per channel of every head, s[t,c] = sum_{i<W} w[h,i,c] x[t-i,c]
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
// Z^T = M S^T with the 16x16x32 bf16 instruction: the A operand is M, the B
// operand S^T, the convolution's output, which each lane forms in fp32 for its
// token and 8 channels per k-step.  Everything a head reads arrives by buffer
// loads that write LDS directly, double-buffered across heads, so head n+1's
// data streams in while head n is computed and no input lives in registers:
// the mix matrix (swizzled for the operand reads), the conv taps, and the
// block's 64 rows plus the 8 before them (swizzled so that 16 lanes reading 16
// consecutive rows hit distinct banks; the waves split the copies).  Every
// load is issued by every lane of its wave (a buffer resource turns reads past
// a tensor into zeros), so each wave waits for its own loads by count and one
// barrier per head publishes them.  S is
// split into bf16 high and low parts and both are multiplied, so the product is
// accurate to about 2^-17 of its terms: the result is the fp32-accurate value,
// rounded once to bf16.  In the result layout each lane holds 4 consecutive
// channels of one token, so the mean is added, channel pairs are rotated in
// registers and 8 bytes are stored per lane (buffer stores, which drop tokens
// past the end, so their number is fixed too).  The kernel is bound by HBM (it
// reads and writes q, k and v once) and by the vector work of the convolution.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr int CM_NW = 4;               // waves per workgroup
constexpr int CM_TW = 16;              // tokens per wave
constexpr int CM_TB = CM_NW * CM_TW;   // tokens per workgroup
constexpr int CM_MAXW = 8;             // widest sequence convolution
constexpr int CM_PREV = 8;             // rows kept before a block's first token (CM_MAXW - 1 needed)

// s_waitcnt immediate: vmcnt(n) and lgkmcnt(0)
constexpr int wait_vmcnt_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70; }

template <int D>
struct CcaLayout {
    static constexpr int ROW = D * 2;                        // bytes per bf16 row
    static constexpr int MBYTES = D * ROW;                   // one head's mix matrix
    static constexpr int MINST = MBYTES / 1024 / CM_NW;      // its 1 KiB copies per wave
    static constexpr int XBYTES = (CM_TB + CM_PREV) * ROW;   // the block's input rows
    static constexpr int XINST = XBYTES / 1024;              // their 1 KiB copies
    static constexpr int XPW = (XINST + CM_NW - 1) / CM_NW;  // copies per wave, at most
    static constexpr int CBYTES = CM_MAXW * ROW;             // one head's taps, at most
    static constexpr int CINST = CBYTES / 1024;              // copies (one per wave)
    static_assert(MINST >= 1 && XBYTES % 1024 == 0 && CBYTES % 1024 == 0 && CINST <= CM_NW,
                  "copy split");
};

// Tap I of the sequence convolution for this lane's token (row CM_PREV + r of
// the block's rows) and channels 32 s + 8 g + e: y += w[I][c] x[t - I, c], with
// the taps [W][D] and the rows (swz_k layout) in LDS.
template <int D, int I>
__device__ __attribute__((always_inline)) inline void conv_tap(float (&y)[D / 32][8], const char* xs,
                                                               const char* cs, int r, int g) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
        const u32x4_t x = *(const u32x4_t*)(xs + swz_k<D>(CM_PREV + r - I, 4 * s + g));
        const u32x4_t wv = *(const u32x4_t*)(cs + (I * D + 32 * s + 8 * g) * 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            y[s][2 * e] = fmaf(bf16_lo(wv[e]), bf16_lo(x[e]), y[s][2 * e]);
            y[s][2 * e + 1] = fmaf(bf16_hi(wv[e]), bf16_hi(x[e]), y[s][2 * e + 1]);
        }
    }
}

// Four workgroups share a CU at D = 64 (36 KiB of LDS each), so a launch over
// 1024 blocks runs in one round.
template <int D>
constexpr int cca_waves_per_simd() { return D == 64 ? 4 : 1; }

template <int D>
__global__ __launch_bounds__(CM_NW * 64, cca_waves_per_simd<D>()) void cca_mix_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ qo, uint16_t* __restrict__ ko, uint16_t* __restrict__ vo,
    const uint16_t* __restrict__ conv_q, const uint16_t* __restrict__ conv_k, int W,
    const uint16_t* __restrict__ mix_q, const uint16_t* __restrict__ mix_k,
    const int32_t* __restrict__ pos_offset, int rope, RopeFreqs fr, int Hq, int Hkv, int S,
    int n_tblk) {
    using L = CcaLayout<D>;
    constexpr int KS = D / 32;  // k-steps of Z^T = M S^T
    constexpr int MT = D / 16;  // 16-channel output tiles
    constexpr int ROW = L::ROW;

    // two of each buffer (head n and head n + 1), as separate objects so the
    // compiler can tell the buffer being filled from the one being read
    __shared__ __attribute__((aligned(1024))) char msm0[L::MBYTES];
    __shared__ __attribute__((aligned(1024))) char msm1[L::MBYTES];
    __shared__ __attribute__((aligned(1024))) char xsm0[L::XBYTES];
    __shared__ __attribute__((aligned(1024))) char xsm1[L::XBYTES];
    __shared__ __attribute__((aligned(1024))) char csm0[L::CBYTES];
    __shared__ __attribute__((aligned(1024))) char csm1[L::CBYTES];
    // destination of the copies a wave issues only so that every wave issues
    // the same number (they read past their buffer: zeros, no memory access)
    __shared__ __attribute__((aligned(1024))) char dummy[1024];

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
        return n < G ? conv_q + ((size_t)j * G + n) * W * D : conv_k + (size_t)j * W * D;
    };

    // Per-lane source offsets of the copies, the same for every head.  A copy
    // puts lane l's 16 bytes at byte 16 l of a 1 KiB destination, i.e. at
    // physical chunk pc of row pr; the swizzle is produced by fetching the
    // logical chunk that belongs there (the XOR swizzle is its own inverse).
    int moff[L::MINST], xoff[L::XPW];
#pragma unroll
    for (int u = 0; u < L::MINST; ++u) {
        const int P = (w * L::MINST + u) * 64 + lane;
        const int pr = P / (D / 8), pc = P % (D / 8);
        moff[u] = swz_k<D>(pr, pc);
    }
#pragma unroll
    for (int u = 0; u < L::XPW; ++u) {  // copy w + CM_NW u of the block's rows
        const int P = (w + CM_NW * u) * 64 + lane;
        const int pr = P / (D / 8), pc = P % (D / 8);
        const int tok = tblk * CM_TB - CM_PREV + pr;  // rows before the first token read zeros
        xoff[u] = tok >= 0 ? tok * ROW + (swz_k<D>(pr, pc) - pr * ROW) : -16;
    }

    // ---- the copies of head n into the given buffers
    auto issue = [&](int n, char* msm, char* xsm, char* csm) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t mrs = buffer_rsrc(head_mix(n), L::MBYTES);
#pragma unroll
        for (int u = 0; u < L::MINST; ++u) dma16(mrs, msm + (w * L::MINST + u) * 1024, moff[u], 0);
        const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(head_rows(n), S * ROW);
#pragma unroll
        for (int u = 0; u < L::XPW; ++u) {
            const bool real = w + CM_NW * u < L::XINST;  // wave-uniform: a select, not a branch
            dma16(xrs, real ? xsm + (w + CM_NW * u) * 1024 : dummy, real ? xoff[u] : -16, 0);
        }
        // the taps [W][D] (past W * D they read zeros), CINST copies
        const __amdgpu_buffer_rsrc_t crs = buffer_rsrc(head_conv(n), W * D * 2);
        const bool tap = w < L::CINST;
        dma16(crs, tap ? csm + w * 1024 : dummy, tap ? lane * 16 : -16, tap ? w * 1024 : 0);
    };
    // the value shift's loads (issued during the last head): the workgroup's
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

    // ---- prologue.  Loads in this order: the RoPE frequencies and the
    // position, the first head's copies, the mean's rows; every one issued by
    // every lane, so the count behind each is fixed and the angle arithmetic
    // waits only for the frequencies, running while the rest is in flight.
    double fq[MT][2];  // frequencies of the token's channel pairs 8 mt + 2 g + e
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 2; ++e) fq[mt][e] = fr.f[8 * mt + 2 * g + e];
    const long long p = (long long)(pos_offset ? pos_offset[b] : 0) + t;

    issue(0, msm0, xsm0, csm0);

    // the token's rows of the group's first four query heads and of its key
    // head (result layout: channels 16 mt + 4 g + i; heads past G re-read the
    // last one and weigh nothing)
    const size_t trow = (size_t)min(t, S - 1) * D + 4 * g;
    u32x2_t xq[4][MT], xk[MT];
    auto load_q = [&](int h0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint16_t* const xr = head_rows(min(h0 + u, G - 1)) + trow;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) xq[u][mt] = *(const u32x2_t*)(xr + 16 * mt);
        }
    };
    load_q(0);
    {
        const uint16_t* const kr = head_rows(G) + trow;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) xk[mt] = *(const u32x2_t*)(kr + 16 * mt);
    }

    // with RoPE, the cosines and sines of the token's channel pairs
    float cs[MT][2], sn[MT][2];
    if (rope) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e) rope_cos_sin(p, fq[mt][e], cs[mt][e], sn[mt][e]);
    }

    // the QK-mean
    f32x4_t mean[MT];
    {
        auto widen = [](u32x2_t x) {
            return f32x4_t{bf16_lo(x[0]), bf16_hi(x[0]), bf16_lo(x[1]), bf16_hi(x[1])};
        };
        f32x4_t qs[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) qs[mt] = f32x4_t{0, 0, 0, 0};
        for (int h0 = 0;;) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float f = h0 + u < G ? 1.f : 0.f;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) qs[mt] += f * widen(xq[u][mt]);
            }
            h0 += 4;
            if (h0 >= G) break;
            load_q(h0);  // groups of more than four query heads
        }
        const float inv_g = 1.f / (float)G;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) mean[mt] = 0.5f * (qs[mt] * inv_g + widen(xk[mt]));
    }

    // ---- one head: convolution, channel mix, mean, RoPE, store
    auto body = [&](int n, const char* msm, const char* xsm, const char* csm, char* msm_next,
                    char* xsm_next, char* csm_next) __attribute__((always_inline)) {
        // This head's copies were issued before the previous head's MT result
        // stores, the last vector-memory operations of each wave before this
        // point; the first head waits for everything.  The barrier then
        // publishes every wave's copies and frees the other buffers.
        __builtin_amdgcn_sched_barrier(0);
        if (n == 0)
            __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
        else
            __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(MT));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (n + 1 < NH)
            issue(n + 1, msm_next, xsm_next, csm_next);
        else
            issue_vshift();
        __builtin_amdgcn_sched_barrier(0);  // the loads stay ahead of this head's work

        // S^T fragments: y[s][e] = channel 32 s + 8 g + e of token t
        const char* const xs = xsm;
        const int rb = CM_TW * w + r;  // the token's row among the block's
        float y[KS][8];
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) y[s][e] = 0.f;
        conv_tap<D, 0>(y, xs, csm, rb, g);
        if (W > 1) conv_tap<D, 1>(y, xs, csm, rb, g);
        if (W > 2) conv_tap<D, 2>(y, xs, csm, rb, g);
        if (W > 3) conv_tap<D, 3>(y, xs, csm, rb, g);
        if (W > 4) conv_tap<D, 4>(y, xs, csm, rb, g);
        if (W > 5) conv_tap<D, 5>(y, xs, csm, rb, g);
        if (W > 6) conv_tap<D, 6>(y, xs, csm, rb, g);
        if (W > 7) conv_tap<D, 7>(y, xs, csm, rb, g);
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

    int n = 0;
    // unrolled by two so each step names its buffers statically
    for (; n + 1 < NH; n += 2) {
        body(n, msm0, xsm0, csm0, msm1, xsm1, csm1);
        body(n + 1, msm1, xsm1, csm1, msm0, xsm0, csm0);
    }
    if (n < NH) body(n, msm0, xsm0, csm0, msm1, xsm1, csm1);

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

// ---------------------------------------------------------------- decode step
// The same operations for one new token per sequence (token index t[b] of its
// sequence, RoPE position pos_offset[b] + t[b]), with the earlier tokens the
// convolution reaches kept as state: the last W - 1 pre-convolution rows of
// every q and k head, token u in ring slot u mod (W - 1), and the previous
// token's v row.  The step reads the state, then writes this token's rows
// into it, so the next step finds them.  Its output equals row t of the
// prefill pass over the sequence.
//
// One workgroup per (sequence, KV group): first each thread convolves (head,
// channel) pairs in fp32 into LDS, forms the group's mean, shifts v and
// updates the state; then each thread takes (head, output channel pair)
// items: the row of the mix matrix times the convolved vector in fp32, plus
// the mean, rotated, rounded once to bf16.  A decode step moves a few
// kilobytes per head, so the kernel is kept simple: its time is launch and
// latency, far below the attention's cache read.
constexpr int CD_THREADS = 256;

template <int D>
__global__ __launch_bounds__(CD_THREADS) void cca_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ qo, uint16_t* __restrict__ ko, uint16_t* __restrict__ vo,
    const uint16_t* __restrict__ conv_q, const uint16_t* __restrict__ conv_k, int W,
    const uint16_t* __restrict__ mix_q, const uint16_t* __restrict__ mix_k,
    uint16_t* __restrict__ q_state, uint16_t* __restrict__ k_state, uint16_t* __restrict__ v_state,
    const int32_t* __restrict__ tok, const int32_t* __restrict__ pos_offset, int rope,
    RopeFreqs fr, int Hq, int Hkv) {
    extern __shared__ __attribute__((aligned(16))) float sm[];  // [NH][D] convolved, then [D] mean
    const int tid = threadIdx.x;
    const int b = (int)blockIdx.x / Hkv, j = (int)blockIdx.x % Hkv;
    const int G = Hq / Hkv, NH = G + 1;
    const int t = max(tok[b], 0);  // a negative index (a caller error) is taken as 0
    const int R = W - 1;  // state rows per head
    float* const mean = sm + NH * D;

    // head n of the group: its input row, state rows, taps and output row
    auto in_row = [&](int n) -> const uint16_t* {
        return n < G ? q + ((size_t)b * Hq + (size_t)j * G + n) * D : k + ((size_t)b * Hkv + j) * D;
    };
    auto state_rows = [&](int n) -> uint16_t* {
        return n < G ? q_state + ((size_t)b * Hq + (size_t)j * G + n) * R * D
                     : k_state + ((size_t)b * Hkv + j) * R * D;
    };
    auto taps = [&](int n) -> const uint16_t* {
        return n < G ? conv_q + ((size_t)j * G + n) * W * D : conv_k + (size_t)j * W * D;
    };
    auto bf = [](uint16_t x) { return __uint_as_float((unsigned)x << 16); };

    // ---- convolution of every (head, channel) and the state update.  Each
    // element of the state is read and then rewritten by the same thread.
    for (int e = tid; e < NH * D; e += CD_THREADS) {
        const int n = e / D, c = e % D;
        const uint16_t* const w = taps(n);
        uint16_t* const st = state_rows(n);
        const uint16_t x0 = in_row(n)[c];
        float y = bf(w[c]) * bf(x0);
        for (int i = 1; i < W; ++i)  // tap i: token t - i, none before the first
            if (t - i >= 0) y = fmaf(bf(w[(size_t)i * D + c]), bf(st[(size_t)((t - i) % R) * D + c]), y);
        if (R > 0) st[(size_t)(t % R) * D + c] = x0;
        sm[e] = y;
    }
    // ---- the mean and the value shift (first half from this token, second
    // half from the previous one, zero at t = 0)
    const float inv_g = 1.f / (float)G;
    for (int c = tid; c < D; c += CD_THREADS) {
        float sq = 0.f;
        for (int n = 0; n < G; ++n) sq += bf(in_row(n)[c]);
        mean[c] = 0.5f * (sq * inv_g + bf(in_row(G)[c]));
        const size_t vr = ((size_t)b * Hkv + j) * D + c;
        const uint16_t cur = v[vr];
        vo[vr] = c < D / 2 ? cur : (t >= 1 ? v_state[vr] : (uint16_t)0);
        v_state[vr] = cur;
    }
    __syncthreads();

    // ---- channel mix, mean, RoPE: item (head n, channel pair cp)
    const long long p = (long long)(pos_offset ? pos_offset[b] : 0) + t;
    for (int e = tid; e < NH * (D / 2); e += CD_THREADS) {
        const int n = e / (D / 2), cp = e % (D / 2), c = 2 * cp;
        const uint16_t* const m = n < G ? mix_q + ((size_t)j * G + n) * D * D : mix_k + (size_t)j * D * D;
        const float* const sv = sm + n * D;
        float z0 = 0.f, z1 = 0.f;
        for (int c2 = 0; c2 < D; c2 += 8) {
            const u32x4_t r0 = *(const u32x4_t*)(m + (size_t)c * D + c2);
            const u32x4_t r1 = *(const u32x4_t*)(m + (size_t)(c + 1) * D + c2);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                z0 = fmaf(bf16_lo(r0[u]), sv[c2 + 2 * u], z0);
                z0 = fmaf(bf16_hi(r0[u]), sv[c2 + 2 * u + 1], z0);
                z1 = fmaf(bf16_lo(r1[u]), sv[c2 + 2 * u], z1);
                z1 = fmaf(bf16_hi(r1[u]), sv[c2 + 2 * u + 1], z1);
            }
        }
        z0 += mean[c];
        z1 += mean[c + 1];
        if (rope) {
            float cs, sn, y0, y1;
            rope_cos_sin(p, fr.f[cp], cs, sn);
            rope_rotate(z0, z1, cs, sn, y0, y1);
            z0 = y0;
            z1 = y1;
        }
        uint16_t* const out = n < G ? qo + ((size_t)b * Hq + (size_t)j * G + n) * D
                                    : ko + ((size_t)b * Hkv + j) * D;
        *(uint32_t*)(out + c) = pack_bf16x2(z0, z1);
    }
}

template <int D>
hipError_t launch_cca_decode_d(void* q_out, void* k_out, void* v_out, const void* q, const void* k,
                               const void* v, int B, int Hq, int Hkv, const void* conv_q,
                               const void* conv_k, int W, const void* mix_q, const void* mix_k,
                               void* q_state, void* k_state, void* v_state, const int32_t* tok,
                               const int32_t* pos_offset, double rope_theta, hipStream_t st) {
    const size_t lds = (size_t)(Hq / Hkv + 2) * D * sizeof(float);
    hipLaunchKernelGGL((cca_decode_kernel<D>), dim3((unsigned)(B * Hkv)), dim3(CD_THREADS), lds, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)q_out,
                       (uint16_t*)k_out, (uint16_t*)v_out, (const uint16_t*)conv_q,
                       (const uint16_t*)conv_k, W, (const uint16_t*)mix_q, (const uint16_t*)mix_k,
                       (uint16_t*)q_state, (uint16_t*)k_state, (uint16_t*)v_state, tok, pos_offset,
                       rope_theta > 0 ? 1 : 0, rope_freqs(rope_theta > 0 ? rope_theta : 1.0, D), Hq,
                       Hkv);
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

size_t cca_decode_lds_bytes(int G, int D) { return (size_t)(G + 2) * D * sizeof(float); }

hipError_t launch_cca_decode(void* q_out, void* k_out, void* v_out, const void* q, const void* k,
                             const void* v, int B, int Hq, int Hkv, int D, const void* conv_q,
                             const void* conv_k, int W, const void* mix_q, const void* mix_k,
                             void* q_state, void* k_state, void* v_state, const int32_t* tok,
                             const int32_t* pos_offset, double rope_theta, hipStream_t st) {
    return D == 64 ? launch_cca_decode_d<64>(q_out, k_out, v_out, q, k, v, B, Hq, Hkv, conv_q, conv_k,
                                             W, mix_q, mix_k, q_state, k_state, v_state, tok,
                                             pos_offset, rope_theta, st)
                   : launch_cca_decode_d<128>(q_out, k_out, v_out, q, k, v, B, Hq, Hkv, conv_q,
                                              conv_k, W, mix_q, mix_k, q_state, k_state, v_state,
                                              tok, pos_offset, rope_theta, st);
}

}  // namespace attn
