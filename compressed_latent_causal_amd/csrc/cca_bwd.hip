// Backward pass of the CCA pre-attention operations for gfx950.
//
// What is computed ("Compressed Convolutional Attention" summary,
// "Resultaten" 2 reports a backward pass for CCA; the formulas are the chain
// rule through the forward operations of "Methodologie" items 2 to 4, in
// reverse order).  Given gq, gk (gradients with respect to the rotated q, k)
// and gv (with respect to the shifted v):
//   a = R_t^T g                      the transposed rotation (a = g without RoPE)
//   dm[t, j] = sum_{h in j} a_q[t, h] + a_k[t, j]        the mean's gradient
//   ds[t] = M^T a[t],  dM += a[t] s[t]^T                  the channel mix
//   dx[t] = sum_i w_i (.) ds[t + i] + dm[t] / (2G or 2)   the taps, forward in time
//   dw_i += ds[t] (.) x[t - i]                            the tap gradient
//   dv~[t] = (gv[t] first half, gv[t + 1] second half, zero at the last token)
// with s[t] = sum_i w_i (.) x[t - i] the forward's convolution output, formed
// again here.  Input gradients are rounded once to bf16; the weight gradients
// are fp32 sums over the batch and every token.
//
// Three kernels; the two D x D products per token and head (ds and dM) run on
// the matrix cores with fp32 values split into bf16 high and low parts, the
// rest is fp32 vector arithmetic:
//  * cca_bwd_mean_kernel: per token and KV group, the rotated-back gradients
//    of the group's query heads and key head summed into dm (fp32, in the
//    workspace), the value shift's gradient, and the rotation's (cos, sin)
//    per (sequence, token, channel pair) into the workspace for the next pass;
//  * cca_bwd_head_kernel<D, W>: one workgroup per (sequence, head, chunk of
//    256 tokens), walking the chunk in blocks of 32 tokens.  Per block the
//    rotated-back gradient rows (the block and the W - 1 tokens after it) and
//    the latent rows (the block and the W - 1 before it) are staged in LDS;
//    s is formed again, ds = M^T a for every staged gradient row, then dx,
//    and the workgroup's running sums of dM and of the tap gradient, which it
//    writes once per chunk into the workspace.  s and the tap gradient go
//    per channel over a run of consecutive tokens, the latent rows they reach
//    held in registers as a sliding window (W, the tap count, is a template
//    parameter so the window has fixed indices);
//  * cca_bwd_reduce_kernel: the per-chunk partial sums added up per weight.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr int CB_CHUNK = 256;    // tokens per workgroup
constexpr int CB_T = 32;         // tokens per block within it
constexpr int CB_MAXW = 8;       // convolution width at most
constexpr int CB_R = CB_T + CB_MAXW - 1;  // staged rows at most
constexpr int CB_THREADS = 256;

__device__ inline float bf16_at(const uint16_t* p, size_t i) { return __uint_as_float((unsigned)p[i] << 16); }

// dm[b, j, t, :] and the value gradient, one thread per (row, 8 channels)
template <int D>
__global__ __launch_bounds__(CB_THREADS) void cca_bwd_mean_kernel(
    float* __restrict__ dm, float* __restrict__ tab, uint16_t* __restrict__ dv, const uint16_t* __restrict__ gq,
    const uint16_t* __restrict__ gk, const uint16_t* __restrict__ gv, int B, int Hq, int Hkv, int S,
    const int32_t* __restrict__ pos_offset, int rope, RopeFreqs fr) {
    constexpr int C8 = D / 8;
    const long long rows = (long long)B * Hkv * S;
    const long long idx = (long long)blockIdx.x * CB_THREADS + threadIdx.x;
    if (idx >= rows * C8) return;
    const long long row = idx / C8;  // (b, j, t)
    const int c0 = 8 * (int)(idx % C8);
    const int t = (int)(row % S);
    const int j = (int)((row / S) % Hkv);
    const int b = (int)(row / ((long long)S * Hkv));
    const int G = Hq / Hkv;
    const long long p = (pos_offset ? (long long)pos_offset[b] : 0) + t;
    float cs[4] = {1.f, 1.f, 1.f, 1.f}, sn[4] = {0.f, 0.f, 0.f, 0.f};
    if (rope) {
#pragma unroll
        for (int e = 0; e < 4; ++e) rope_cos_sin(p, fr.f[c0 / 2 + e], cs[e], sn[e]);
        if (j == 0) {  // the (cos, sin) table of the per-head pass: [b, t, pair]
            float* const tp = tab + (((size_t)b * S + t) * (D / 2) + c0 / 2) * 2;
            *(f32x4_t*)tp = f32x4_t{cs[0], sn[0], cs[1], sn[1]};
            *(f32x4_t*)(tp + 4) = f32x4_t{cs[2], sn[2], cs[3], sn[3]};
        }
    }
    const size_t at = (size_t)row * D + c0;
    const u32x4_t kw = *(const u32x4_t*)(gk + at);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) rope_rotate(bf16_lo(kw[e]), bf16_hi(kw[e]), cs[e], -sn[e], acc[2 * e], acc[2 * e + 1]);
    for (int r = 0; r < G; ++r) {
        const u32x4_t qw = *(const u32x4_t*)(gq + (((size_t)b * Hq + (size_t)j * G + r) * S + t) * D + c0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float a0, a1;
            rope_rotate(bf16_lo(qw[e]), bf16_hi(qw[e]), cs[e], -sn[e], a0, a1);
            acc[2 * e] += a0;
            acc[2 * e + 1] += a1;
        }
    }
    *(f32x4_t*)(dm + at) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
    *(f32x4_t*)(dm + at + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
    // value shift: first half in place, second half from the next token
    u32x4_t vw = {0, 0, 0, 0};
    if (c0 < D / 2) vw = *(const u32x4_t*)(gv + at);
    else if (t + 1 < S) vw = *(const u32x4_t*)(gv + at + D);
    *(u32x4_t*)(dv + at) = vw;
}

// fp32 x as a bf16 high part (truncated) and the bf16 rounding of the rest:
// hi + lo carries about 16 bits of x, so products taken part by part with an
// exact bf16 (or a split) operand are fp32-accurate.
__device__ inline void split1(float x, unsigned& hi, unsigned& lo) {
    const unsigned b = __float_as_uint(x) & 0xffff0000u;
    hi = b >> 16;
    lo = pack_bf16x2(x - __uint_as_float(b), 0.f) & 0xffffu;
}

// 8 bf16 of column c0 + (lane % 16) of rows r0 .. r0 + 7 of a row-major bf16
// tile with rows of `ld` elements (two transpose reads of 4 rows each): the
// matrix-core operand whose k runs along the rows.
__device__ inline bf16x8_t col8(const uint16_t* tile, int ld, int r0, int c0, int lane) {
    const int L = lane & 15;
    const uint16_t* const p = tile + (r0 + L / 4) * ld + c0 + 4 * (L % 4);
    const bf16x4_t lo = lds_read_tr(p), hi = lds_read_tr(p + 4 * ld);
    const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
    return __builtin_bit_cast(bf16x8_t, u32x4_t{l2.x, l2.y, h2.x, h2.y});
}

// One workgroup per (chunk, head n of the Hq + Hkv, sequence b).  The two D x D
// products run on the matrix cores (v_mfma_f32_16x16x32_bf16) on operands
// stored in LDS as bf16 high and low parts: ds = M^T a (a split, M exact),
// read row-wise; dM += a s^T over the block's 32 tokens (hi hi + hi lo +
// lo hi), with a and s read down their token columns by transpose reads.
template <int D, int W>
__global__ __launch_bounds__(CB_THREADS, D == 64 ? 3 : 1) void cca_bwd_head_kernel(
    uint16_t* __restrict__ dq, uint16_t* __restrict__ dk, float* __restrict__ part_mix,
    float* __restrict__ part_conv, const float* __restrict__ dm, const float* __restrict__ tab,
    const uint16_t* __restrict__ gq, const uint16_t* __restrict__ gk, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ conv_q,
    const uint16_t* __restrict__ conv_k, const uint16_t* __restrict__ mix_q,
    const uint16_t* __restrict__ mix_k, int B, int Hq, int Hkv, int S, int rope) {
    static_assert(W >= 1 && W <= CB_MAXW, "convolution width");
    constexpr int NT = D / 16;      // 16-wide tiles of a D-long dimension
    constexpr int KS = D / 32;      // 32-deep k-steps over D
    constexpr int RM = 48;          // staged gradient rows, padded to 3 tiles of 16
    static_assert(RM >= CB_R, "row tiles");
    constexpr int DSN = 3 * NT;     // ds tiles
    constexpr int DMN = NT * NT;    // dM tiles
    constexpr int DMW = DMN / 4;    // dM tiles per wave

    // Rows are padded by 16 bytes (4 floats, 8 bf16) so that the reads of 16
    // rows at one column (the matrix-core operands, the convolution over
    // tokens) and the writes of the products' results fall in distinct banks.
    constexpr int DP = D + 4, AP = D + 8, MP = D + 8;
    __shared__ __attribute__((aligned(16))) uint16_t ah_s[RM * AP];  // a rows t0 .., bf16 high part, zeros after RA
    __shared__ __attribute__((aligned(16))) uint16_t al_s[RM * AP];  // low part
    __shared__ __attribute__((aligned(16))) uint16_t sh_s[CB_T * AP];  // s of the block, high part, zeros after T
    __shared__ __attribute__((aligned(16))) uint16_t sl_s[CB_T * AP];
    __shared__ __attribute__((aligned(16))) float ds_s[RM][DP];      // M^T a of the staged rows
    __shared__ __attribute__((aligned(16))) uint16_t x_s[CB_R * AP];  // x rows t0 - W + 1 .. t0 + T - 1 (bf16)
    __shared__ __attribute__((aligned(16))) float w_s[CB_MAXW][D];
    __shared__ __attribute__((aligned(16))) uint16_t mt_s[D * MP];   // M^T: mt_s[c' MP + c] = M[c][c']

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int nchunk = (S + CB_CHUNK - 1) / CB_CHUNK;
    const int chunk = (int)blockIdx.x % nchunk;
    const int n = (int)blockIdx.x / nchunk % (Hq + Hkv);
    const int b = (int)blockIdx.x / nchunk / (Hq + Hkv);
    const bool isq = n < Hq;
    const int h = isq ? n : n - Hq;
    const int H = isq ? Hq : Hkv;
    const int G = Hq / Hkv;
    const int j = isq ? h / G : h;
    const float mean_w = isq ? 0.5f / (float)G : 0.5f;
    const uint16_t* const g = isq ? gq : gk;
    const uint16_t* const x = isq ? q : k;
    uint16_t* const dx = isq ? dq : dk;
    const size_t row0 = ((size_t)b * H + h) * S;     // this head's first row
    const size_t mrow0 = ((size_t)b * Hkv + j) * S;  // its group's first dm row
    const float* const tab_b = tab + (size_t)b * S * D;  // (cos, sin) of the sequence's rows

    // weights of the head: M transposed into LDS, the taps in fp32
    {
        const uint16_t* const mw = (isq ? mix_q : mix_k) + (size_t)h * D * D;
        for (int e = tid; e < D * D; e += CB_THREADS) {
            const int c = e / D, c2 = e % D;  // coalesced read of row c
            mt_s[c2 * MP + c] = mw[e];
        }
    }
    for (int e = tid; e < W * D; e += CB_THREADS)
        w_s[e / D][e % D] = bf16_at(isq ? conv_q : conv_k, (size_t)h * W * D + e);

    // The convolution over tokens (s, formed again) and the tap gradient:
    // thread tid takes channel cc and the TPG consecutive tokens r0 .. of its
    // group, with the latent rows they reach held in registers (a sliding
    // window), so each staged value is read once per block.  Tap i meets the
    // row W - 1 - i after the token's own first reach; in the window that is
    // offset j = W - 1 - i, and the taps are kept in that order (wj[j] = w_i).
    constexpr int NG = CB_THREADS / D;        // token groups: 4 at D = 64, 2 at D = 128
    constexpr int TPG = CB_T / NG;            // tokens per group
    constexpr int XW = TPG + W - 1;           // window rows
    const int cc = tid % D, r0 = (tid / D) * TPG;

    // running sums of the weight gradients: the wave's dM tiles, and the
    // thread's tap sums (window offset j) over its groups' tokens
    f32x4_t dmacc[DMW];
#pragma unroll
    for (int u = 0; u < DMW; ++u) dmacc[u] = f32x4_t{0, 0, 0, 0};
    float conv_acc[W];
#pragma unroll
    for (int jj = 0; jj < W; ++jj) conv_acc[jj] = 0.f;
    // window rows r0 .. r0 + TPG + W - 2 of the staged latent rows (x_s row m
    // holds token t0 - W + 1 + m); rows past the staged ones are only reached
    // by tokens past the block
    auto load_window = [&](float (&xv)[XW]) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < XW; ++m) xv[m] = __uint_as_float((unsigned)x_s[(r0 + m) * AP + cc] << 16);
    };

    const int c_begin = chunk * CB_CHUNK, c_end = min(S, c_begin + CB_CHUNK);
    // A block's global loads (gradient rows, 8 channels per item; latent rows;
    // the mean's gradient) are issued while the previous block is computed.
    constexpr int AI = (RM * (D / 8) + CB_THREADS - 1) / CB_THREADS;
    constexpr int XI = (CB_R * (D / 8) + CB_THREADS - 1) / CB_THREADS;
    constexpr int DI = (CB_T * (D / 8) + CB_THREADS - 1) / CB_THREADS;
    u32x4_t gw[AI], xw[XI];
    f32x4_t tlo[AI], thi[AI];  // (cos, sin) of the 4 pairs of a gradient item
    f32x4_t mlo[DI], mhi[DI];
    auto load_block = [&](int tb) __attribute__((always_inline)) {
        const int Tb = min(CB_T, c_end - tb);
        const int RAb = min(Tb + W - 1, S - tb), RXb = Tb + W - 1;
#pragma unroll
        for (int u = 0; u < AI; ++u) {
            const int e = tid + u * CB_THREADS, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            gw[u] = u32x4_t{0, 0, 0, 0};
            tlo[u] = thi[u] = f32x4_t{1, 0, 1, 0};
            if (r < RAb) {
                gw[u] = *(const u32x4_t*)(g + (row0 + tb + r) * D + c0);
                if (rope) {
                    tlo[u] = *(const f32x4_t*)(tab_b + (size_t)(tb + r) * D + c0);
                    thi[u] = *(const f32x4_t*)(tab_b + (size_t)(tb + r) * D + c0 + 4);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < XI; ++u) {
            const int e = tid + u * CB_THREADS, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            const int tok = tb - (W - 1) + r;
            xw[u] = u32x4_t{0, 0, 0, 0};
            if (r < RXb && tok >= 0) xw[u] = *(const u32x4_t*)(x + (row0 + tok) * D + c0);
        }
#pragma unroll
        for (int u = 0; u < DI; ++u) {
            const int e = tid + u * CB_THREADS, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            mlo[u] = mhi[u] = f32x4_t{0, 0, 0, 0};
            if (r < Tb) {
                mlo[u] = *(const f32x4_t*)(dm + (mrow0 + tb + r) * D + c0);
                mhi[u] = *(const f32x4_t*)(dm + (mrow0 + tb + r) * D + c0 + 4);
            }
        }
    };
    load_block(c_begin);
    for (int t0 = c_begin; t0 < c_end; t0 += CB_T) {
        const int T = min(CB_T, c_end - t0);    // block tokens
        const int RA = min(T + W - 1, S - t0);  // gradient rows (tokens t0 .. t0 + RA - 1)
        __syncthreads();  // the previous block's reads are done
#pragma unroll
        for (int u = 0; u < AI; ++u) {
            const int e = tid + u * CB_THREADS, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            if (r < RM) {
                const float cs[4] = {tlo[u][0], tlo[u][2], thi[u][0], thi[u][2]};
                const float sn[4] = {tlo[u][1], tlo[u][3], thi[u][1], thi[u][3]};
                u32x4_t hw, lw;
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2) {  // a = R^T g (cos 1, sin 0 without RoPE)
                    float a0, a1;
                    rope_rotate(bf16_lo(gw[u][q2]), bf16_hi(gw[u][q2]), cs[q2], -sn[q2], a0, a1);
                    unsigned h0, l0, h1, l1;
                    split1(a0, h0, l0);
                    split1(a1, h1, l1);
                    hw[q2] = h0 | (h1 << 16);
                    lw[q2] = l0 | (l1 << 16);
                }
                *(u32x4_t*)(ah_s + r * AP + c0) = hw;
                *(u32x4_t*)(al_s + r * AP + c0) = lw;
            }
        }
#pragma unroll
        for (int u = 0; u < XI; ++u) {
            const int e = tid + u * CB_THREADS, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            // every staged row is written, zeros past the T + W - 1 the
            // block has (the windows of tokens past the block reach them)
            if (r < CB_R) *(u32x4_t*)(x_s + r * AP + c0) = xw[u];
        }
        f32x4_t cur_lo[DI], cur_hi[DI];  // this block's mean gradient
#pragma unroll
        for (int u = 0; u < DI; ++u) {
            cur_lo[u] = mlo[u];
            cur_hi[u] = mhi[u];
        }
        if (t0 + CB_T < c_end) load_block(t0 + CB_T);
        __syncthreads();
        // s of the block (the forward's convolution output) as bf16 parts,
        // zero past the block's tokens
        {
            float xv[XW], wj[W];
            load_window(xv);
#pragma unroll
            for (int jj = 0; jj < W; ++jj) wj[jj] = w_s[W - 1 - jj][cc];
#pragma unroll
            for (int kq = 0; kq < TPG; ++kq) {
                float sv = 0.f;
#pragma unroll
                for (int jj = W - 1; jj >= 0; --jj) sv = fmaf(wj[jj], xv[kq + jj], sv);  // taps i = 0 .. W - 1
                if (r0 + kq >= T) sv = 0.f;
                unsigned hs, ls;
                split1(sv, hs, ls);
                sh_s[(r0 + kq) * AP + cc] = (uint16_t)hs;
                sl_s[(r0 + kq) * AP + cc] = (uint16_t)ls;
            }
        }
        // ds = M^T a: tile (mt, nt) gives rows 16 mt + 4 lg + i, column 16 nt + lr
        for (int tt = w; tt < DSN; tt += 4) {
            const int mt = tt / NT, nt = tt % NT;
            f32x4_t acc = {0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int ao = (16 * mt + lr) * AP + 32 * ks + 8 * lg;
                const bf16x8_t ahi = *(const bf16x8_t*)(ah_s + ao), alo = *(const bf16x8_t*)(al_s + ao);
                const bf16x8_t bm = *(const bf16x8_t*)(mt_s + (16 * nt + lr) * MP + 32 * ks + 8 * lg);
                acc = mfma16(ahi, bm, acc);
                acc = mfma16(alo, bm, acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) ds_s[16 * mt + 4 * lg + i][16 * nt + lr] = acc[i];
        }
        __syncthreads();
        // dx of the block's tokens: the taps forward in time, plus the mean's
        // share; 8 channels per item
        {
#pragma unroll
            for (int u = 0; u < DI; ++u) {
                const int e = tid + u * CB_THREADS, r = e / (D / 8), c0 = 8 * (e % (D / 8));
                if (r < T) {
                    float v[8];
#pragma unroll
                    for (int z = 0; z < 4; ++z) {
                        v[z] = mean_w * cur_lo[u][z];
                        v[z + 4] = mean_w * cur_hi[u][z];
                    }
                    for (int i = 0; i < W && r + i < RA; ++i) {
                        const f32x4_t d0 = *(const f32x4_t*)&ds_s[r + i][c0];
                        const f32x4_t d1 = *(const f32x4_t*)&ds_s[r + i][c0 + 4];
                        const f32x4_t w0 = *(const f32x4_t*)&w_s[i][c0];
                        const f32x4_t w1 = *(const f32x4_t*)&w_s[i][c0 + 4];
#pragma unroll
                        for (int z = 0; z < 4; ++z) {
                            v[z] = fmaf(w0[z], d0[z], v[z]);
                            v[z + 4] = fmaf(w1[z], d1[z], v[z + 4]);
                        }
                    }
                    *(u32x4_t*)(dx + (row0 + t0 + r) * D + c0) =
                        u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
                }
            }
        }
        // tap gradient: dw_i[c] += sum over the block's tokens of ds[t] x[t - i]
        {
            float xv[XW];
            load_window(xv);
            float tacc[W];
#pragma unroll
            for (int jj = 0; jj < W; ++jj) tacc[jj] = 0.f;
#pragma unroll
            for (int kq = 0; kq < TPG; ++kq) {
                const float d = r0 + kq < T ? ds_s[r0 + kq][cc] : 0.f;
#pragma unroll
                for (int jj = 0; jj < W; ++jj) tacc[jj] = fmaf(d, xv[kq + jj], tacc[jj]);
            }
#pragma unroll
            for (int jj = 0; jj < W; ++jj) conv_acc[jj] += tacc[jj];
        }
        // dM += a s^T over the block: tile (mt, nt) of (c, c'), k = the 32 tokens
#pragma unroll
        for (int u = 0; u < DMW; ++u) {
            const int tt = w + 4 * u, mt = tt / NT, nt = tt % NT;
            // A[m = c][k = t] = a[t][c] and B[k = t][n = c'] = s[t][c']: token
            // columns of the row-major parts (rows 8 lg .. 8 lg + 7)
            const bf16x8_t ahi = col8(ah_s, AP, 8 * lg, 16 * mt, lane), alo = col8(al_s, AP, 8 * lg, 16 * mt, lane);
            const bf16x8_t shi = col8(sh_s, AP, 8 * lg, 16 * nt, lane), slo = col8(sl_s, AP, 8 * lg, 16 * nt, lane);
            dmacc[u] = mfma16(ahi, shi, dmacc[u]);
            dmacc[u] = mfma16(ahi, slo, dmacc[u]);
            dmacc[u] = mfma16(alo, shi, dmacc[u]);
        }
    }
    // this chunk's partial sums: part[(b, chunk)][n][...]
    const size_t pidx = ((size_t)b * nchunk + chunk) * (Hq + Hkv) + n;
    {
        float* const pm = part_mix + pidx * D * D;
#pragma unroll
        for (int u = 0; u < DMW; ++u) {
            const int tt = w + 4 * u, mt = tt / NT, nt = tt % NT;
#pragma unroll
            for (int i = 0; i < 4; ++i) pm[(size_t)(16 * mt + 4 * lg + i) * D + 16 * nt + lr] = dmacc[u][i];
        }
    }
    {
        // the token groups' tap sums added in group order through LDS (the
        // ds rows are free after the last block): row NG jj + group
        static_assert(NG * CB_MAXW <= RM, "tap-sum rows");
        __syncthreads();
#pragma unroll
        for (int jj = 0; jj < W; ++jj) ds_s[NG * jj + tid / D][cc] = conv_acc[jj];
        __syncthreads();
        float* const pc = part_conv + pidx * (size_t)W * D;
        for (int e = tid; e < W * D; e += CB_THREADS) {
            const int i = e / D, c = e % D, jj = W - 1 - i;
            float sum = 0.f;
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) sum += ds_s[NG * jj + gg][c];
            pc[e] = sum;
        }
    }
}

// Weight gradients: the sum of the P = B * nchunk partials of every weight
// element; element e of head n runs over dM (D D) then the taps (W D).  A
// workgroup takes 64 consecutive elements; its 4 waves each sum a quarter of
// the partials (8 loads in flight per lane), then the quarters are added
// through LDS, so the result does not depend on the launch.
__global__ __launch_bounds__(CB_THREADS) void cca_bwd_reduce_kernel(
    float* __restrict__ dconv_q, float* __restrict__ dconv_k, float* __restrict__ dmix_q,
    float* __restrict__ dmix_k, const float* __restrict__ part_mix, const float* __restrict__ part_conv,
    int Hq, int Hkv, int D, int W, int P) {
    __shared__ float red[4][64];
    const int per = D * D + W * D;
    const int NH = Hq + Hkv;
    const int lane = threadIdx.x & 63, qw = threadIdx.x >> 6;
    const long long idx = (long long)blockIdx.x * 64 + lane;
    const bool ok = idx < (long long)NH * per;
    const int n = ok ? (int)(idx / per) : 0, e = ok ? (int)(idx % per) : 0;
    const bool mix = e < D * D;
    const float* const base = mix ? part_mix + (size_t)n * D * D + e
                                  : part_conv + (size_t)n * W * D + (e - D * D);
    const size_t stride = mix ? (size_t)NH * D * D : (size_t)NH * W * D;
    const int p0 = qw * ((P + 3) / 4), p1 = min(P, p0 + (P + 3) / 4);
    float acc = 0.f;
    if (ok) {
        int p = p0;
        for (; p + 8 <= p1; p += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = base[(size_t)(p + u) * stride];
#pragma unroll
            for (int u = 0; u < 8; ++u) acc += v[u];
        }
        for (; p < p1; ++p) acc += base[(size_t)p * stride];
    }
    red[qw][lane] = acc;
    __syncthreads();
    if (qw == 0 && ok) {
        const float sum = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
        if (mix) {
            if (n < Hq) dmix_q[(size_t)n * D * D + e] = sum;
            else dmix_k[(size_t)(n - Hq) * D * D + e] = sum;
        } else {
            const int f = e - D * D;
            if (n < Hq) dconv_q[(size_t)n * W * D + f] = sum;
            else dconv_k[(size_t)(n - Hq) * W * D + f] = sum;
        }
    }
}

template <int D>
hipError_t launch_cca_bwd_d(void* dq, void* dk, void* dv, float* dconv_q, float* dconv_k,
                            float* dmix_q, float* dmix_k, const void* gq, const void* gk,
                            const void* gv, const void* q, const void* k, int B, int Hq, int Hkv,
                            int S, const void* conv_q, const void* conv_k, int W, const void* mix_q,
                            const void* mix_k, const int32_t* pos_offset, double rope_theta,
                            void* workspace, hipStream_t st) {
    const int rope = rope_theta > 0 ? 1 : 0;
    const RopeFreqs fr = rope_freqs(rope ? rope_theta : 1.0, D);
    const int nchunk = (S + CB_CHUNK - 1) / CB_CHUNK;
    const int P = B * nchunk;
    float* const dm = (float*)workspace;
    float* const tab = dm + (size_t)B * Hkv * S * D;  // [B, S, D / 2] (cos, sin)
    float* const part_mix = tab + (size_t)B * S * D;
    float* const part_conv = part_mix + (size_t)P * (Hq + Hkv) * D * D;
    if ((long long)B * S > 0) {
        const long long items = (long long)B * Hkv * S * (D / 8);
        hipLaunchKernelGGL(cca_bwd_mean_kernel<D>, dim3((unsigned)((items + CB_THREADS - 1) / CB_THREADS)),
                           dim3(CB_THREADS), 0, st, dm, tab, (uint16_t*)dv, (const uint16_t*)gq,
                           (const uint16_t*)gk, (const uint16_t*)gv, B, Hq, Hkv, S, pos_offset, rope, fr);
        auto head = [&](auto w_c) {
            hipLaunchKernelGGL((cca_bwd_head_kernel<D, decltype(w_c)::value>),
                               dim3((unsigned)((long long)B * (Hq + Hkv) * nchunk)), dim3(CB_THREADS), 0, st,
                               (uint16_t*)dq, (uint16_t*)dk, part_mix, part_conv, (const float*)dm,
                               (const float*)tab, (const uint16_t*)gq, (const uint16_t*)gk,
                               (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)conv_q,
                               (const uint16_t*)conv_k, (const uint16_t*)mix_q, (const uint16_t*)mix_k, B,
                               Hq, Hkv, S, rope);
        };
        static_assert(CB_MAXW == 8, "one instance per width");
        switch (W) {  // the width is checked (1 .. CB_MAXW) before the launch
            case 1: head(std::integral_constant<int, 1>{}); break;
            case 2: head(std::integral_constant<int, 2>{}); break;
            case 3: head(std::integral_constant<int, 3>{}); break;
            case 4: head(std::integral_constant<int, 4>{}); break;
            case 5: head(std::integral_constant<int, 5>{}); break;
            case 6: head(std::integral_constant<int, 6>{}); break;
            case 7: head(std::integral_constant<int, 7>{}); break;
            default: head(std::integral_constant<int, 8>{}); break;
        }
    }
    {
        const long long items = (long long)(Hq + Hkv) * (D * D + W * D);
        hipLaunchKernelGGL(cca_bwd_reduce_kernel, dim3((unsigned)((items + 63) / 64)),
                           dim3(CB_THREADS), 0, st, dconv_q, dconv_k, dmix_q, dmix_k,
                           (const float*)part_mix, (const float*)part_conv, Hq, Hkv, D, W, P);
    }
    return hipGetLastError();
}

}  // namespace

size_t cca_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D, int W) {
    const size_t nchunk = ((size_t)S + CB_CHUNK - 1) / CB_CHUNK;
    const size_t P = (size_t)B * nchunk;
    return sizeof(float) * ((size_t)B * Hkv * S * D + (size_t)B * S * D +
                            P * (Hq + Hkv) * ((size_t)D * D + (size_t)W * D));
}

int cca_bwd_max_width() { return CB_MAXW; }

hipError_t launch_cca_bwd(void* dq, void* dk, void* dv, float* dconv_q, float* dconv_k,
                          float* dmix_q, float* dmix_k, const void* gq, const void* gk,
                          const void* gv, const void* q, const void* k, int B, int Hq, int Hkv,
                          int S, int D, const void* conv_q, const void* conv_k, int W,
                          const void* mix_q, const void* mix_k, const int32_t* pos_offset,
                          double rope_theta, void* workspace, hipStream_t st) {
    return D == 64 ? launch_cca_bwd_d<64>(dq, dk, dv, dconv_q, dconv_k, dmix_q, dmix_k, gq, gk, gv,
                                          q, k, B, Hq, Hkv, S, conv_q, conv_k, W, mix_q, mix_k,
                                          pos_offset, rope_theta, workspace, st)
                   : launch_cca_bwd_d<128>(dq, dk, dv, dconv_q, dconv_k, dmix_q, dmix_k, gq, gk,
                                           gv, q, k, B, Hq, Hkv, S, conv_q, conv_k, W, mix_q,
                                           mix_k, pos_offset, rope_theta, workspace, st);
}

}  // namespace attn
