// Backward pass of causal grouped-query prefill for gfx950.
//
// What is computed: the gradients of sum <dout, o> for o = prefill(q, k, v)
// (the "Compressed Convolutional Attention" summary, "Resultaten", reports
// this backward pass for the same attention; the formulas are the chain rule
// through the forward's definition).  Per query row i of head h and key t <= i
// of its KV head:  p = exp(scale <q_i, k_t> - lse_i),  dp = <dout_i, v_t>,
// ds = p (dp - delta_i) with delta_i = <dout_i, o_i>;  dq_i = scale sum_t ds k_t,
// dk_t = scale sum ds q_i and dv_t = sum p dout_i, the last two over every
// query head of the group and every query i >= t.
//
// Three kernels (four for split launches, below), bf16 in and out with fp32
// accumulation:
//  * row statistics: per query row the log-normaliser in the exp2 domain and
//    delta = <dout, o> (from the forward's bf16 output), padded per head to
//    whole tiles plus one (padding rows give p = 0 and ds = 0);
//  * dK/dV: one workgroup per (key block, batch, KV head).  Each wave keeps its
//    16 NK keys' K and V rows in registers (as the matrix-core B operand) and
//    the fp32 dK^T, dV^T tiles as accumulators; Q and dO tiles of 64 queries of
//    every query head of the group stream through LDS (buffer loads straight to
//    LDS, double-buffered, as in the forward).  Per 32 queries: S = Q K^T and
//    dP - delta = dO V^T (the product starts from -delta), P and dS in fp32,
//    rounded to bf16, then dV^T += dO^T P and dK^T += Q^T dS, with the A operand
//    read transposed from the same LDS tiles.  The group's heads are summed in
//    the accumulators, so dK and dV are written once, with no atomics.
//    Workgroups that start at the first key blocks see every query and run
//    longest; when a launch would give the GPU fewer than three rounds of
//    workgroups, those few long ones decide its time.  Then the group's heads
//    are split over hs workgroups per key block (and at D = 64 each wave takes
//    32 keys), each writing its fp32 dK^T, dV^T partial sums to the workspace,
//    and a fourth kernel adds the hs partials and rounds them once to bf16.
//  * dQ: the forward's work split (one workgroup per query block and head
//    slice of a KV group, K/V tiles of 64 keys through LDS); per tile S^T =
//    K Q^T and dP^T - delta = V dO^T, dS^T in fp32 then bf16, and
//    dQ^T += K^T dS^T with K^T read transposed from the K tile.
// S and dP are formed in both the dK/dV and the dQ kernel (seven products per
// score tile instead of five): the price of writing every gradient once
// without atomics or an fp32 dQ buffer.

#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr int BW_BQ = 64;  // queries per Q/dO tile (dK/dV kernel)
constexpr int BW_BN = 64;  // keys per K/V tile (dQ kernel)
// LDS operand fragments read ahead of the products that use them
#ifndef BW_PD
#define BW_PD 4
#endif

// The 8-wide slice of each 32-wide k-step that lane group lg supplies to the
// products whose A operand is read directly from a swz_v tile.  The same
// permutation on both operands leaves a product unchanged.  The order
// (0, 2, 1, 3) removes the LDS bank conflicts of these reads at both head
// dims: measured over five layouts, a 16-byte-per-lane read is served in four
// passes whose lanes agree in (lane bit 3 xor bit 4, bit 5), i.e. lanes
// {0-7, 24-31}, {8-15, 16-23}, {32-39, 56-63}, {40-47, 48-55}; in the natural
// order two lanes of a pass share banks (2-way conflicts, a third more LDS
// cycles), in this order none do.
__device__ inline int kslice(int lg) {
    return ((lg & 1) << 1) | (lg >> 1);
}

// Rows of row statistics per head: whole Q tiles plus one (the stats of a tile
// are fetched 128 rows at a time).
__host__ __device__ inline int stats_rows(int S) { return ceil_div(S, BW_BQ) * BW_BQ + BW_BQ; }

// ------------------------------------------------------------------ row statistics
// stats[(b*Hq + h) * S_pad + i] = (lse * log2 e, <dout_i, o_i>) for i < S, and
// (+inf, 0) for the padding rows S <= i < S_pad.  LPR lanes per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_rowstats_kernel(const uint16_t* __restrict__ o,
                                                           const uint16_t* __restrict__ dout,
                                                           const float* __restrict__ lse,
                                                           float2* __restrict__ stats, int S,
                                                           int S_pad, long long n_pad_rows) {
    constexpr int LPR = D / 8;
    constexpr int RPB = 256 / LPR;
    const long long rp = (long long)blockIdx.x * RPB + threadIdx.x / LPR;  // padded row
    const int part = threadIdx.x % LPR;
    const long long bh = rp / S_pad;
    const int i = (int)(rp % S_pad);
    const bool valid = rp < n_pad_rows && i < S;
    const long long r = bh * S + i;  // unpadded row
    float acc = 0.f;
    if (valid) {
        const u32x4_t a = *(const u32x4_t*)(o + r * D + part * 8);
        const u32x4_t g = *(const u32x4_t*)(dout + r * D + part * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = fmaf(bf16_lo(a[e]), bf16_lo(g[e]), acc);
            acc = fmaf(bf16_hi(a[e]), bf16_hi(g[e]), acc);
        }
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if (rp < n_pad_rows && part == 0)
        stats[rp] = valid ? float2{lse[r] * kLog2e, acc} : float2{INFINITY, 0.f};
}

// ------------------------------------------------------------------ dK, dV
template <int D, int NK, int NW>
__global__ __launch_bounds__(NW * 64, ((NK == 1 || D == 64) && NW == 4) ? 2 : 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float2* __restrict__ stats, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, float* __restrict__ part, int B, int Hq, int Hkv, int S, int S_pad,
    float c, float scale, int hsplit) {
    constexpr int KSTEPS = D / 32;  // k-steps of S = Q K^T
    constexpr int DT = D / 16;      // d tiles of dK^T, dV^T
    constexpr int ROW = D * 2;
    constexpr int TILE = BW_BQ * ROW;
    constexpr int BK = 16 * NK * NW;  // keys per workgroup
    constexpr int RPI = 1024 / ROW;
    constexpr int NI = TILE / 1024 / NW;  // wave-wide loads per wave per tile, for Q and for dO
    static_assert(NI >= 1 && TILE % (1024 * NW) == 0, "tile split");

    __shared__ __attribute__((aligned(1024))) char q0s[TILE];
    __shared__ __attribute__((aligned(1024))) char q1s[TILE];
    __shared__ __attribute__((aligned(1024))) char g0s[TILE];
    __shared__ __attribute__((aligned(1024))) char g1s[TILE];
    __shared__ __attribute__((aligned(1024))) char st0[1024];
    __shared__ __attribute__((aligned(1024))) char st1[1024];

    const int G = Hq / Hkv;
    const int per = B * Hkv;
    // workgroup = (key block, head slice, batch and KV head); the first key
    // blocks see the most queries: dispatched first
    const int kb = (int)blockIdx.x / (per * hsplit);
    const int hs = (int)blockIdx.x / per % hsplit;
    const int bkv = (int)blockIdx.x % per;
    const int b = bkv / Hkv, kvh = bkv % Hkv;
    const int Gs = G / hsplit;  // query heads of this workgroup: kvh G + hs Gs ..
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int k0 = kb * BK;
    const int kw0 = k0 + w * 16 * NK;  // first key of this wave

    // K and V rows of the wave's keys as B operands: key kw0 + 16nk + lr, dims
    // 32s + 8 kslice(lg) .. +7
    const size_t kv_base = (size_t)(b * Hkv + kvh) * S * D;
    const int ks8 = 8 * kslice(lg);
    bf16x8_t kf[NK][KSTEPS], vf[NK][KSTEPS];
#pragma unroll
    for (int nk = 0; nk < NK; ++nk) {
        const int row = kw0 + 16 * nk + lr;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            u32x4_t xk = {0, 0, 0, 0}, xv = {0, 0, 0, 0};
            if (row < S) {
                xk = *(const u32x4_t*)(k + kv_base + (size_t)row * D + 32 * s + ks8);
                xv = *(const u32x4_t*)(v + kv_base + (size_t)row * D + 32 * s + ks8);
            }
            kf[nk][s] = __builtin_bit_cast(bf16x8_t, xk);
            vf[nk][s] = __builtin_bit_cast(bf16x8_t, xv);
        }
    }

    f32x4_t dka[DT][NK], dva[DT][NK];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int nk = 0; nk < NK; ++nk) dka[dt][nk] = dva[dt][nk] = f32x4_t{0, 0, 0, 0};

    // LDS operand offsets (tiles in the swz_v layout): direct reads of rows
    // 16i + lr, chunk 4s + lg (the A operand of S and dP), and transposed reads
    // of d tile dt (the A operand of dV^T and dK^T).
    int aoff[KSTEPS], toff[DT];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) aoff[s] = swz_v<D>(lr, 4 * s + kslice(lg));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) toff[dt] = v_frag_off<D>(dt, lane);
    int vo[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int r = (w * NI + i) * RPI + lane / (ROW / 16), pc = lane % (ROW / 16);
        vo[i] = r * ROW + ((swz_v<D>(r, pc) - r * ROW) & ~15);
    }

    // Work items: (query head of the slice, Q tile), tiles from the one holding
    // the workgroup's first key to the end of the sequence.
    const int t0 = k0 / BW_BQ;
    const int nt = ceil_div(S, BW_BQ) - t0;
    const int n_it = nt > 0 ? Gs * nt : 0;
    auto issue = [&](int it, char* qb, char* gb, char* sb) __attribute__((always_inline)) {
        const int h = kvh * G + hs * Gs + it / nt, t = t0 + it % nt;
        const size_t hb = (size_t)(b * Hq + h);
        const __amdgpu_buffer_rsrc_t qrs = buffer_rsrc(q + hb * S * D, S * ROW);
        const __amdgpu_buffer_rsrc_t grs = buffer_rsrc(dout + hb * S * D, S * ROW);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            dma16(qrs, qb + (w * NI + i) * 1024, vo[i], t * TILE);
            dma16(grs, gb + (w * NI + i) * 1024, vo[i], t * TILE);
        }
        if (w == 0) {  // 128 rows of (log2-domain lse, delta): the tile's 64 and the next 64
            const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(stats + hb * S_pad, S_pad * 8);
            dma16(srs, sb, lane * 16, t * BW_BQ * 8);
        }
    };

    auto compute = [&](int it, const char* qs, const char* gs, const char* ss)
                       __attribute__((always_inline)) {
        const int q0 = (t0 + it % nt) * BW_BQ;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int qh0 = q0 + 32 * hh;
            // every query of the half precedes every key of the wave, or the half is past S
            if (qh0 + 31 < kw0 || qh0 >= S) continue;
            // this lane's queries qh0 + 16i + 4lg + r: log2-domain lse and delta
            f32x4_t l2[2], dl[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const f32x4_t a = *(const f32x4_t*)(ss + (32 * hh + 16 * i + 4 * lg) * 8);
                const f32x4_t e = *(const f32x4_t*)(ss + (32 * hh + 16 * i + 4 * lg) * 8 + 16);
                l2[i] = f32x4_t{a[0], a[2], e[0], e[2]};
                dl[i] = f32x4_t{-a[1], -a[3], -e[1], -e[3]};
            }
            // S = Q K^T and dP - delta = dO V^T; lane holds key kw0 + 16nk + lr,
            // queries qh0 + 16i + 4lg + r
            f32x4_t sacc[2][NK], pacc[2][NK];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int nk = 0; nk < NK; ++nk) {
                    sacc[i][nk] = f32x4_t{0, 0, 0, 0};
                    pacc[i][nk] = dl[i];
                }
            // operand f = (k-step f / 4, sub-tile (f / 2) % 2, Q or dO by f % 2),
            // read BW_PD operands ahead of the products that use it
            constexpr int NAF = 4 * KSTEPS;
            auto afrag = [&](int f) __attribute__((always_inline)) {
                const char* base = (f % 2) ? gs : qs;
                return *(const bf16x8_t*)(base + aoff[f / 4] + (32 * hh + 16 * ((f / 2) % 2)) * ROW);
            };
            bf16x8_t af[NAF];
#pragma unroll
            for (int f = 0; f < BW_PD && f < NAF; ++f) af[f] = afrag(f);
#pragma unroll
            for (int f = 0; f < NAF; ++f) {
                if (f + BW_PD < NAF) af[f + BW_PD] = afrag(f + BW_PD);
                __builtin_amdgcn_sched_barrier(0);
                const int s = f / 4, i = (f / 2) % 2;
#pragma unroll
                for (int nk = 0; nk < NK; ++nk) {
                    if (f % 2) pacc[i][nk] = mfma16(af[f], vf[nk][s], pacc[i][nk]);
                    else sacc[i][nk] = mfma16(af[f], kf[nk][s], sacc[i][nk]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // P = exp2(c s - lse2), dS = P (dP - delta); zero where the query
            // precedes the key or lies past the sequence
            const bool edge = (qh0 < kw0 + 16 * NK) || (qh0 + 32 > S);
            bf16x8_t pb[NK], sb[NK];
#pragma unroll
            for (int nk = 0; nk < NK; ++nk) {
                float p[2][4], d[2][4];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float pv = __builtin_amdgcn_exp2f(fmaf(sacc[i][nk][r], c, -l2[i][r]));
                        float dv_ = pv * pacc[i][nk][r];
                        if (edge) {
                            const int qi = qh0 + 16 * i + 4 * lg + r, key = kw0 + 16 * nk + lr;
                            if (qi < key || qi >= S) pv = dv_ = 0.f;
                        }
                        p[i][r] = pv;
                        d[i][r] = dv_;
                    }
                u32x4_t pw, dw;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    pw[2 * i] = pack_bf16x2(p[i][0], p[i][1]);
                    pw[2 * i + 1] = pack_bf16x2(p[i][2], p[i][3]);
                    dw[2 * i] = pack_bf16x2(d[i][0], d[i][1]);
                    dw[2 * i + 1] = pack_bf16x2(d[i][2], d[i][3]);
                }
                pb[nk] = __builtin_bit_cast(bf16x8_t, pw);
                sb[nk] = __builtin_bit_cast(bf16x8_t, dw);
            }
            // dV^T += dO^T P and dK^T += Q^T dS: the A operands are the half's 32
            // rows read transposed, in the row order the P and dS packing uses
            // operand f = (d tile f / 2, dO^T or Q^T by f % 2), read BW_PD ahead
            constexpr int NTF = 2 * DT;
            auto tfrag = [&](int f) __attribute__((always_inline)) {
                return v_frag_at<D>(((f % 2) ? qs : gs) + toff[f / 2] + 32 * hh * ROW);
            };
            bf16x8_t tf[NTF];
#pragma unroll
            for (int f = 0; f < BW_PD && f < NTF; ++f) tf[f] = tfrag(f);
#pragma unroll
            for (int f = 0; f < NTF; ++f) {
                if (f + BW_PD < NTF) tf[f + BW_PD] = tfrag(f + BW_PD);
                __builtin_amdgcn_sched_barrier(0);
                const int dt = f / 2;
#pragma unroll
                for (int nk = 0; nk < NK; ++nk) {
                    if (f % 2) dka[dt][nk] = mfma16(tf[f], sb[nk], dka[dt][nk]);
                    else dva[dt][nk] = mfma16(tf[f], pb[nk], dva[dt][nk]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    auto step = [&](int it, const char* qs, const char* gs, const char* ss, char* qn, char* gn,
                    char* sn) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        if (it + 1 < n_it) issue(it + 1, qn, gn, sn);
        compute(it, qs, gs, ss);
    };
    if (n_it > 0) issue(0, q0s, g0s, st0);
    for (int it = 0; it < n_it; it += 2) {
        step(it, q0s, g0s, st0, q1s, g1s, st1);
        if (it + 1 >= n_it) break;
        step(it + 1, q1s, g1s, st1, q0s, g0s, st0);
    }

    // ---- dK = scale dK^T, dV = dV^T; lane holds key kw0 + 16nk + lr, dims 16dt + 4lg .. +3
    if (hsplit > 1) {  // this slice's fp32 partial sums: part[hs][K or V][b, kvh, key, d]
        const size_t plane = (size_t)B * Hkv * S * D;
        float* const pk = part + (size_t)hs * 2 * plane + kv_base;
        float* const pv = pk + plane;
#pragma unroll
        for (int nk = 0; nk < NK; ++nk) {
            const int key = kw0 + 16 * nk + lr;
            if (key >= S) continue;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                *(f32x4_t*)(pk + (size_t)key * D + 16 * dt + 4 * lg) = dka[dt][nk];
                *(f32x4_t*)(pv + (size_t)key * D + 16 * dt + 4 * lg) = dva[dt][nk];
            }
        }
        return;
    }
#pragma unroll
    for (int nk = 0; nk < NK; ++nk) {
        const int key = kw0 + 16 * nk + lr;
        if (key >= S) continue;
        uint16_t* const krow = dk + kv_base + (size_t)key * D + 4 * lg;
        uint16_t* const vrow = dv + kv_base + (size_t)key * D + 4 * lg;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            u32x2_t a, e;
            a[0] = pack_bf16x2(dka[dt][nk][0] * scale, dka[dt][nk][1] * scale);
            a[1] = pack_bf16x2(dka[dt][nk][2] * scale, dka[dt][nk][3] * scale);
            e[0] = pack_bf16x2(dva[dt][nk][0], dva[dt][nk][1]);
            e[1] = pack_bf16x2(dva[dt][nk][2], dva[dt][nk][3]);
            *(u32x2_t*)(krow + 16 * dt) = a;
            *(u32x2_t*)(vrow + 16 * dt) = e;
        }
    }
}

// dk = scale sum_hs part[hs][K], dv = sum_hs part[hs][V], rounded once to bf16;
// one thread per 8 consecutive elements of the [B, Hkv, S, D] planes.
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(const float* __restrict__ part,
                                                              uint16_t* __restrict__ dk,
                                                              uint16_t* __restrict__ dv,
                                                              long long plane, int hsplit,
                                                              float scale) {
    const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i >= plane) return;
    f32x4_t ka = {0, 0, 0, 0}, kb = {0, 0, 0, 0}, va = {0, 0, 0, 0}, vb = {0, 0, 0, 0};
    for (int hs = 0; hs < hsplit; ++hs) {
        const float* const pk = part + (size_t)hs * 2 * plane + i;
        const float* const pv = pk + plane;
        ka += *(const f32x4_t*)pk;
        kb += *(const f32x4_t*)(pk + 4);
        va += *(const f32x4_t*)pv;
        vb += *(const f32x4_t*)(pv + 4);
    }
    u32x4_t ko, vo;
    ko[0] = pack_bf16x2(ka[0] * scale, ka[1] * scale);
    ko[1] = pack_bf16x2(ka[2] * scale, ka[3] * scale);
    ko[2] = pack_bf16x2(kb[0] * scale, kb[1] * scale);
    ko[3] = pack_bf16x2(kb[2] * scale, kb[3] * scale);
    vo[0] = pack_bf16x2(va[0], va[1]);
    vo[1] = pack_bf16x2(va[2], va[3]);
    vo[2] = pack_bf16x2(vb[0], vb[1]);
    vo[3] = pack_bf16x2(vb[2], vb[3]);
    *(u32x4_t*)(dk + i) = ko;
    *(u32x4_t*)(dv + i) = vo;
}

// ------------------------------------------------------------------ dQ
template <int D, int HPW>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float2* __restrict__ stats, uint16_t* __restrict__ dq,
    int B, int Hq, int Hkv, int S, int S_pad, float c, float scale, int n_qblk, int n_hchunk) {
    constexpr int NW = 4;
    constexpr int KSTEPS = D / 32;
    constexpr int DT = D / 16;
    constexpr int QPB = (NW / HPW) * 32;  // queries per head per workgroup
    constexpr int ROW = D * 2;
    constexpr int TILE = BW_BN * ROW;
    constexpr int RPI = 1024 / ROW;
    constexpr int NI = TILE / 1024 / NW;
    static_assert(NI >= 1 && TILE % (1024 * NW) == 0, "tile split");

    __shared__ __attribute__((aligned(1024))) char k0s[TILE];
    __shared__ __attribute__((aligned(1024))) char k1s[TILE];
    __shared__ __attribute__((aligned(1024))) char v0s[TILE];
    __shared__ __attribute__((aligned(1024))) char v1s[TILE];

    const int G = Hq / Hkv;
    const int per = B * Hkv * n_hchunk;
    const int qb = n_qblk - 1 - (int)blockIdx.x / per;  // heaviest query blocks first
    const int rem = (int)blockIdx.x % per;
    const int bkv = rem % (B * Hkv), hc = rem / (B * Hkv);
    const int b = bkv / Hkv, kvh = bkv % Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int h = kvh * G + hc * HPW + (w % HPW);
    const int q0 = qb * QPB;
    const int qw0 = q0 + (w / HPW) * 32;
    const size_t kv_base = (size_t)(b * Hkv + kvh) * S * D;
    const size_t qo_base = (size_t)(b * Hq + h) * S * D;

    // Q^T and dO^T fragments (B operands): query qw0 + 16n + lr, dims 32s + 8lg .. +7;
    // this lane's query's log2-domain lse and -delta
    bf16x8_t qf[2][KSTEPS], gf[2][KSTEPS];
    float l2[2], nd[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int row = qw0 + 16 * n + lr;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            u32x4_t xq = {0, 0, 0, 0}, xg = {0, 0, 0, 0};
            if (row < S) {  // Q^T in the k order of the K tile's direct reads
                xq = *(const u32x4_t*)(q + qo_base + (size_t)row * D + 32 * s + 8 * kslice(lg));
                xg = *(const u32x4_t*)(dout + qo_base + (size_t)row * D + 32 * s + 8 * lg);
            }
            qf[n][s] = __builtin_bit_cast(bf16x8_t, xq);
            gf[n][s] = __builtin_bit_cast(bf16x8_t, xg);
        }
        const float2 st = stats[(size_t)(b * Hq + h) * S_pad + min(row, S_pad - 1)];
        l2[n] = st.x;
        nd[n] = -st.y;
    }

    // K tiles in the swz_v layout (read directly for S^T and transposed for
    // dQ^T), V tiles in the swz_k layout (read directly for dP^T)
    int koff[KSTEPS], voff[KSTEPS], toff[DT];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
        koff[s] = swz_v<D>(lr, 4 * s + kslice(lg));
        voff[s] = swz_k<D>(lr, 4 * s + lg);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) toff[dt] = v_frag_off<D>(dt, lane);
    int kvo[NI], vvo[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int r = (w * NI + i) * RPI + lane / (ROW / 16), pc = lane % (ROW / 16);
        kvo[i] = r * ROW + ((swz_v<D>(r, pc) - r * ROW) & ~15);
        vvo[i] = r * ROW + ((swz_k<D>(r, pc) - r * ROW) & ~15);
    }
    const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(k + kv_base, S * ROW);
    const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(v + kv_base, S * ROW);
    auto issue = [&](int t, char* kb, char* vb) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            dma16(krs, kb + (w * NI + i) * 1024, kvo[i], t * TILE);
            dma16(vrs, vb + (w * NI + i) * 1024, vvo[i], t * TILE);
        }
    };

    const int kv_end = min(q0 + QPB, S);
    const int ntiles = ceil_div(kv_end, BW_BN);
    const int last = qw0 < S ? min(ntiles - 1, (qw0 + 31) / BW_BN) : -1;

    f32x4_t qa[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) qa[dt][0] = qa[dt][1] = f32x4_t{0, 0, 0, 0};

    auto compute = [&](int t, const char* ks, const char* vs) __attribute__((always_inline)) {
        const int kv0 = t * BW_BN;
        const bool diag = t == last && kv0 + BW_BN - 1 > qw0;  // mask keys above the diagonal
        // the tile's keys in two halves of 32 (fewer live score registers)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            // S^T = K Q^T and dP^T - delta = V dO^T; lane holds query qw0 + 16n + lr,
            // keys kv0 + 32kk + 16hf + 4lg + r
            f32x4_t sacc[2][2], pacc[2][2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    sacc[hf][n] = f32x4_t{0, 0, 0, 0};
                    pacc[hf][n] = f32x4_t{nd[n], nd[n], nd[n], nd[n]};
                }
            // operand f = (k-step f / 4, key tile 2kk + (f / 2) % 2, K or V by f % 2),
            // read BW_PD operands ahead of its two products
            constexpr int NAF = 4 * KSTEPS;
            auto afrag = [&](int f) __attribute__((always_inline)) {
                const int mt = 2 * kk + (f / 2) % 2;
                return (f % 2) ? *(const bf16x8_t*)(vs + voff[f / 4] + 16 * mt * ROW)
                               : *(const bf16x8_t*)(ks + koff[f / 4] + 16 * mt * ROW);
            };
            bf16x8_t af[NAF];
#pragma unroll
            for (int f = 0; f < BW_PD && f < NAF; ++f) af[f] = afrag(f);
#pragma unroll
            for (int f = 0; f < NAF; ++f) {
                if (f + BW_PD < NAF) af[f + BW_PD] = afrag(f + BW_PD);
                __builtin_amdgcn_sched_barrier(0);
                const int s = f / 4, hf = (f / 2) % 2;
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    if (f % 2) pacc[hf][n] = mfma16(af[f], gf[n][s], pacc[hf][n]);
                    else sacc[hf][n] = mfma16(af[f], qf[n][s], sacc[hf][n]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // dS^T = P^T (dP^T - delta), zero above the diagonal, packed as the
            // B operand (keys 4lg + r of both 16-key tiles)
            bf16x8_t sb[2];
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int qi = qw0 + 16 * n + lr;
                u32x4_t dw;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    float d[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[hf][n][r], c, -l2[n]));
                        d[r] = p * pacc[hf][n][r];
                        if (diag && kv0 + 32 * kk + 16 * hf + 4 * lg + r > qi) d[r] = 0.f;
                    }
                    dw[2 * hf] = pack_bf16x2(d[0], d[1]);
                    dw[2 * hf + 1] = pack_bf16x2(d[2], d[3]);
                }
                sb[n] = __builtin_bit_cast(bf16x8_t, dw);
            }
            // dQ^T += K^T dS^T, the K^T operand of d tile dt read BW_PD / 2 ahead
            constexpr int TPD = BW_PD / 2 > 0 ? BW_PD / 2 : 1;
            auto tfrag = [&](int dt) __attribute__((always_inline)) {
                return v_frag_at<D>(ks + toff[dt] + 32 * kk * ROW);
            };
            bf16x8_t tf[DT];
#pragma unroll
            for (int dt = 0; dt < TPD && dt < DT; ++dt) tf[dt] = tfrag(dt);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                if (dt + TPD < DT) tf[dt + TPD] = tfrag(dt + TPD);
                __builtin_amdgcn_sched_barrier(0);
                qa[dt][0] = mfma16(tf[dt], sb[0], qa[dt][0]);
                qa[dt][1] = mfma16(tf[dt], sb[1], qa[dt][1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    auto step = [&](int t, const char* ks, const char* vs, char* kn, char* vn)
                    __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0070);
        __builtin_amdgcn_s_barrier();
        if (t + 1 < ntiles) issue(t + 1, kn, vn);
        if (t <= last) compute(t, ks, vs);
    };
    issue(0, k0s, v0s);
    for (int t = 0; t < ntiles; t += 2) {
        step(t, k0s, v0s, k1s, v1s);
        if (t + 1 >= ntiles) break;
        step(t + 1, k1s, v1s, k0s, v0s);
    }

    // ---- dQ = scale dQ^T; lane holds query qw0 + 16n + lr, dims 16dt + 4lg .. +3
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int qi = qw0 + 16 * n + lr;
        if (qi >= S) continue;
        uint16_t* const row = dq + qo_base + (size_t)qi * D + 4 * lg;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            u32x2_t a;
            a[0] = pack_bf16x2(qa[dt][n][0] * scale, qa[dt][n][1] * scale);
            a[1] = pack_bf16x2(qa[dt][n][2] * scale, qa[dt][n][3] * scale);
            *(u32x2_t*)(row + 16 * dt) = a;
        }
    }
}

int pow2_divisor(int g, int cap) {
    int hp = 1;
    while (hp * 2 <= cap && g % (hp * 2) == 0) hp *= 2;
    return hp;
}

#ifndef BW_NW
#define BW_NW 4
#endif

template <int D, int NK>
int dkdv_blocks_per_cu() {
    static const int n = [] {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, bwd_dkdv_kernel<D, NK, BW_NW>,
                                                         BW_NW * 64, 0) != hipSuccess || b < 1)
            b = 1;
        return b;
    }();
    return n;
}

// How the dK/dV kernel is launched: keys of 16 per wave (nk) and head slices
// per key block (hs).  One slice and 16 keys while the launch fills the GPU
// at least three times over (the heaviest-first order then balances it);
// otherwise the fewest slices (1, 2 or 4, dividing G) that reach three rounds,
// with 32 keys per wave at D = 64, where each LDS operand then feeds two
// products.
struct BwdPlan {
    int nk, hs;
};
template <int D>
BwdPlan bwd_plan(int B, int Hq, int Hkv, int S) {
    const int G = Hq / Hkv;
    const long long cus = device_cus();
    const long long nblk1 = (long long)ceil_div(S, 16 * BW_NW) * B * Hkv;
    if (G == 1 || nblk1 >= 3 * cus * dkdv_blocks_per_cu<D, 1>()) return {1, 1};
    constexpr int NK2 = D == 64 ? 2 : 1;
    const long long nblk = (long long)ceil_div(S, 16 * NK2 * BW_NW) * B * Hkv;
    const long long slots = cus * dkdv_blocks_per_cu<D, NK2>();
    int hs = 1;
    while (hs * 2 <= 4 && G % (hs * 2) == 0 && nblk * hs < 3 * slots) hs *= 2;
    if (hs == 1) return {1, 1};
    return {NK2, hs};
}

size_t stats_bytes(int B, int Hq, int S) {
    return ((size_t)B * Hq * stats_rows(S) * sizeof(float2) + 255) & ~(size_t)255;
}

template <int D>
size_t backward_workspace_d(int B, int Hq, int Hkv, int S) {
    const BwdPlan pl = bwd_plan<D>(B, Hq, Hkv, S);
    const size_t part = pl.hs > 1 ? (size_t)pl.hs * 2 * B * Hkv * S * D * sizeof(float) : 0;
    return stats_bytes(B, Hq, S) + part;
}

template <int D>
hipError_t launch_backward_d(void* dq, void* dk, void* dv, const void* q, const void* k,
                             const void* v, const void* o, const void* dout, const float* lse,
                             int B, int Hq, int Hkv, int S, float scale, void* workspace,
                             hipStream_t st) {
    const float c = scale * kLog2e;
    const int S_pad = stats_rows(S);
    float2* const stats = (float2*)workspace;
    {
        const long long rows = (long long)B * Hq * S_pad;
        constexpr int RPB = 256 / (D / 8);
        hipLaunchKernelGGL(bwd_rowstats_kernel<D>, dim3((unsigned)ceil_div(rows, (long long)RPB)),
                           dim3(256), 0, st, (const uint16_t*)o, (const uint16_t*)dout, lse, stats,
                           S, S_pad, rows);
    }
    {
        const BwdPlan pl = bwd_plan<D>(B, Hq, Hkv, S);
        float* const part = pl.hs > 1 ? (float*)((char*)workspace + stats_bytes(B, Hq, S)) : nullptr;
        auto go = [&](auto kern, int bk) {
            const long long nblk = (long long)ceil_div(S, bk) * B * Hkv * pl.hs;
            hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(BW_NW * 64), 0, st,
                               (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                               (const uint16_t*)dout, (const float2*)stats, (uint16_t*)dk,
                               (uint16_t*)dv, part, B, Hq, Hkv, S, S_pad, c, scale, pl.hs);
        };
        constexpr int NK2 = D == 64 ? 2 : 1;
        if (pl.nk == NK2) go(bwd_dkdv_kernel<D, NK2, BW_NW>, 16 * NK2 * BW_NW);
        else go(bwd_dkdv_kernel<D, 1, BW_NW>, 16 * BW_NW);
        if (pl.hs > 1) {
            const long long plane = (long long)B * Hkv * S * D;
            hipLaunchKernelGGL(bwd_dkdv_reduce_kernel, dim3((unsigned)ceil_div(plane / 8, 256LL)),
                               dim3(256), 0, st, (const float*)part, (uint16_t*)dk, (uint16_t*)dv,
                               plane, pl.hs, scale);
        }
    }
    {
        const int G = Hq / Hkv;
        const int hpw = pow2_divisor(G, 4);
        const int QPB = (4 / hpw) * 32;
        const int n_qblk = ceil_div(S, QPB), n_hchunk = G / hpw;
        const long long nblk = (long long)n_qblk * B * Hkv * n_hchunk;
        auto go = [&](auto kern) {
            hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(256), 0, st, (const uint16_t*)q,
                               (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout,
                               (const float2*)stats, (uint16_t*)dq, B, Hq, Hkv, S, S_pad, c, scale,
                               n_qblk, n_hchunk);
        };
        if (hpw == 4) go(bwd_dq_kernel<D, 4>);
        else if (hpw == 2) go(bwd_dq_kernel<D, 2>);
        else go(bwd_dq_kernel<D, 1>);
    }
    return hipGetLastError();
}

}  // namespace

size_t prefill_backward_workspace_bytes(int B, int Hq, int Hkv, int S, int D) {
    return D == 64 ? backward_workspace_d<64>(B, Hq, Hkv, S) : backward_workspace_d<128>(B, Hq, Hkv, S);
}

hipError_t launch_prefill_backward(void* dq, void* dk, void* dv, const void* q, const void* k,
                                   const void* v, const void* o, const void* dout,
                                   const float* lse, int B, int Hq, int Hkv, int S, int D,
                                   float scale, void* workspace, hipStream_t st) {
    return D == 64 ? launch_backward_d<64>(dq, dk, dv, q, k, v, o, dout, lse, B, Hq, Hkv, S, scale,
                                           workspace, st)
                   : launch_backward_d<128>(dq, dk, dv, q, k, v, o, dout, lse, B, Hq, Hkv, S,
                                            scale, workspace, st);
}

}  // namespace attn
