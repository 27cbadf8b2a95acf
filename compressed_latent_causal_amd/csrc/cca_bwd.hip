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
// Three kernels, all fp32 vector arithmetic (the pass moves a few bytes per
// flop; its products are small D x D maps per token):
//  * cca_bwd_mean_kernel: per token and KV group, the rotated-back gradients
//    of the group's query heads and key head summed into dm (fp32, in the
//    workspace), and the value shift's gradient;
//  * cca_bwd_head_kernel: one workgroup per (sequence, head, chunk of 256
//    tokens), walking the chunk in blocks of 32 tokens.  Per block the
//    rotated-back gradient rows (the block and the W - 1 tokens after it) and
//    the latent rows (the block and the W - 1 before it) are staged in LDS,
//    ds = M^T a is formed for every staged gradient row, then dx, s, and the
//    workgroup's running sums of dM and of the tap gradient, which it writes
//    once per chunk into the workspace;
//  * cca_bwd_reduce_kernel: the per-chunk partial sums added up per weight.
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

// a = R^T g for the channel pair (2i, 2i + 1) of one row at position p
__device__ inline void rope_back(float g0, float g1, long long p, double freq, int rope, float& a0, float& a1) {
    if (!rope) {
        a0 = g0;
        a1 = g1;
        return;
    }
    float cs, sn;
    rope_cos_sin(p, freq, cs, sn);
    rope_rotate(g0, g1, cs, -sn, a0, a1);
}

// dm[b, j, t, :] and the value gradient, one thread per (row, channel pair)
template <int D>
__global__ __launch_bounds__(CB_THREADS) void cca_bwd_mean_kernel(
    float* __restrict__ dm, uint16_t* __restrict__ dv, const uint16_t* __restrict__ gq,
    const uint16_t* __restrict__ gk, const uint16_t* __restrict__ gv, int B, int Hq, int Hkv, int S,
    const int32_t* __restrict__ pos_offset, int rope, RopeFreqs fr) {
    constexpr int P = D / 2;
    const long long rows = (long long)B * Hkv * S;
    const long long idx = (long long)blockIdx.x * CB_THREADS + threadIdx.x;
    if (idx >= rows * P) return;
    const long long row = idx / P;  // (b, j, t)
    const int i = (int)(idx % P);
    const int t = (int)(row % S);
    const int j = (int)((row / S) % Hkv);
    const int b = (int)(row / ((long long)S * Hkv));
    const int G = Hq / Hkv;
    const long long p = (pos_offset ? (long long)pos_offset[b] : 0) + t;
    float s0 = 0.f, s1 = 0.f;
    for (int r = 0; r < G; ++r) {
        const size_t at = (((size_t)b * Hq + (size_t)j * G + r) * S + t) * D + 2 * i;
        float a0, a1;
        rope_back(bf16_at(gq, at), bf16_at(gq, at + 1), p, fr.f[i], rope, a0, a1);
        s0 += a0;
        s1 += a1;
    }
    const size_t at = (size_t)row * D + 2 * i;
    float a0, a1;
    rope_back(bf16_at(gk, at), bf16_at(gk, at + 1), p, fr.f[i], rope, a0, a1);
    dm[at] = s0 + a0;
    dm[at + 1] = s1 + a1;
    // value shift: first half in place, second half from the next token
    unsigned w;
    if (2 * i < D / 2) w = *(const unsigned*)(gv + at);
    else w = t + 1 < S ? *(const unsigned*)(gv + at + D) : 0u;
    *(unsigned*)(dv + at) = w;
}

// One workgroup per (chunk, head n of the Hq + Hkv, sequence b).
template <int D>
__global__ __launch_bounds__(CB_THREADS) void cca_bwd_head_kernel(
    uint16_t* __restrict__ dq, uint16_t* __restrict__ dk, float* __restrict__ part_mix,
    float* __restrict__ part_conv, const float* __restrict__ dm, const uint16_t* __restrict__ gq,
    const uint16_t* __restrict__ gk, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ conv_q, const uint16_t* __restrict__ conv_k,
    const uint16_t* __restrict__ mix_q, const uint16_t* __restrict__ mix_k, int B, int Hq, int Hkv,
    int S, int W, const int32_t* __restrict__ pos_offset, int rope, RopeFreqs fr) {
    constexpr int CG = D / 4;                  // 4-column groups
    constexpr int RG = CB_THREADS / CG;        // row groups of the ds product
    constexpr int RPT = (CB_R + RG - 1) / RG;  // ds rows per thread
    constexpr int MB = D == 64 ? 4 : 8;        // dM block per thread: MB x MB
    constexpr int MG = D / MB;                 // dM column groups
    static_assert(MG * MG == CB_THREADS, "dM split");

    __shared__ __attribute__((aligned(16))) float a_s[CB_R][D];   // a rows t0 .. t0 + T + W - 2
    __shared__ __attribute__((aligned(16))) float ds_s[CB_R][D];  // M^T a of the same rows
    __shared__ __attribute__((aligned(16))) float x_s[CB_R][D];   // x rows t0 - W + 1 .. t0 + T - 1
    __shared__ __attribute__((aligned(16))) float s_s[CB_T][D];   // the forward's s of the block
    __shared__ __attribute__((aligned(16))) float w_s[CB_MAXW][D];
    __shared__ __attribute__((aligned(16))) uint16_t m_s[D * D];  // mix, row c = output channel

    const int tid = threadIdx.x;
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
    const long long pbase = pos_offset ? (long long)pos_offset[b] : 0;

    // weights of the head
    for (int e = tid; e < D * D / 8; e += CB_THREADS)
        *(u32x4_t*)(m_s + 8 * e) = *(const u32x4_t*)((isq ? mix_q : mix_k) + (size_t)h * D * D + 8 * e);
    for (int e = tid; e < W * D; e += CB_THREADS)
        w_s[e / D][e % D] = bf16_at(isq ? conv_q : conv_k, (size_t)h * W * D + e);

    // running sums of the weight gradients
    float mix_acc[MB][MB];
#pragma unroll
    for (int r = 0; r < MB; ++r)
#pragma unroll
        for (int c = 0; c < MB; ++c) mix_acc[r][c] = 0.f;
    // tap gradients: thread tid sums taps e = tid + 256 q4 (W D <= 1024)
    float conv_acc[4] = {0.f, 0.f, 0.f, 0.f};

    const int c_begin = chunk * CB_CHUNK, c_end = min(S, c_begin + CB_CHUNK);
    for (int t0 = c_begin; t0 < c_end; t0 += CB_T) {
        const int T = min(CB_T, c_end - t0);  // block tokens
        const int RA = min(T + W - 1, S - t0);  // gradient rows staged (tokens t0 .. t0 + RA - 1)
        const int RX = T + W - 1;               // latent rows staged (tokens t0 - W + 1 ..)
        __syncthreads();  // the previous block's reads are done
        for (int e = tid; e < RA * (D / 2); e += CB_THREADS) {
            const int r = e / (D / 2), i = e % (D / 2);
            const size_t at = (row0 + t0 + r) * D + 2 * i;
            float a0, a1;
            rope_back(bf16_at(g, at), bf16_at(g, at + 1), pbase + t0 + r, fr.f[i], rope, a0, a1);
            a_s[r][2 * i] = a0;
            a_s[r][2 * i + 1] = a1;
        }
        for (int e = tid; e < RX * D; e += CB_THREADS) {
            const int r = e / D, c = e % D;
            const int tok = t0 - (W - 1) + r;
            x_s[r][c] = tok >= 0 ? bf16_at(x, (row0 + tok) * D + c) : 0.f;
        }
        __syncthreads();
        // ds = M^T a: thread (column group cg, row group rg) forms rows rg + RG m, columns 4cg .. +3
        {
            const int cg = tid % CG, rg = tid / CG;
            float acc[RPT][4];
#pragma unroll
            for (int m = 0; m < RPT; ++m)
#pragma unroll
                for (int u = 0; u < 4; ++u) acc[m][u] = 0.f;
            for (int c = 0; c < D; ++c) {
                const u32x2_t mw = *(const u32x2_t*)(m_s + c * D + 4 * cg);
                const float m0 = bf16_lo(mw[0]), m1 = bf16_hi(mw[0]), m2 = bf16_lo(mw[1]), m3 = bf16_hi(mw[1]);
#pragma unroll
                for (int m = 0; m < RPT; ++m) {
                    const int r = rg + RG * m;
                    if (r < RA) {
                        const float av = a_s[r][c];
                        acc[m][0] = fmaf(m0, av, acc[m][0]);
                        acc[m][1] = fmaf(m1, av, acc[m][1]);
                        acc[m][2] = fmaf(m2, av, acc[m][2]);
                        acc[m][3] = fmaf(m3, av, acc[m][3]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const int r = rg + RG * m;
                if (r < RA) *(f32x4_t*)&ds_s[r][4 * cg] = f32x4_t{acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
            }
        }
        // s of the block (the forward's convolution output)
        for (int e = tid; e < T * D; e += CB_THREADS) {
            const int r = e / D, c = e % D;
            float acc = 0.f;
            for (int i = 0; i < W; ++i) acc = fmaf(w_s[i][c], x_s[r + W - 1 - i][c], acc);
            s_s[r][c] = acc;
        }
        __syncthreads();
        // dx of the block's tokens: the taps forward in time, plus the mean's share
        for (int e = tid; e < T * (D / 2); e += CB_THREADS) {
            const int r = e / (D / 2), c = 2 * (e % (D / 2));
            float v0 = 0.f, v1 = 0.f;
            for (int i = 0; i < W && r + i < RA; ++i) {
                v0 = fmaf(w_s[i][c], ds_s[r + i][c], v0);
                v1 = fmaf(w_s[i][c + 1], ds_s[r + i][c + 1], v1);
            }
            const float2 mm = *(const float2*)(dm + (mrow0 + t0 + r) * D + c);
            v0 = fmaf(mean_w, mm.x, v0);
            v1 = fmaf(mean_w, mm.y, v1);
            *(unsigned*)(dx + (row0 + t0 + r) * D + c) = pack_bf16x2(v0, v1);
        }
        // dM += a s^T over the block: thread owns rows MB (tid / MG) .., columns MB (tid % MG) ..
        {
            const int mr = MB * (tid / MG), mc = MB * (tid % MG);
            for (int r = 0; r < T; ++r) {
                float av[MB], sv[MB];
#pragma unroll
                for (int u = 0; u < MB; u += 4) {
                    const f32x4_t a4 = *(const f32x4_t*)&a_s[r][mr + u];
                    const f32x4_t s4 = *(const f32x4_t*)&s_s[r][mc + u];
#pragma unroll
                    for (int z = 0; z < 4; ++z) {
                        av[u + z] = a4[z];
                        sv[u + z] = s4[z];
                    }
                }
#pragma unroll
                for (int u = 0; u < MB; ++u)
#pragma unroll
                    for (int z = 0; z < MB; ++z) mix_acc[u][z] = fmaf(av[u], sv[z], mix_acc[u][z]);
            }
        }
        // tap gradient: dw_i[c] += sum over the block of ds[t] x[t - i]
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int e = tid + q4 * CB_THREADS;
            if (e < W * D) {
                const int i = e / D, c = e % D;
                float acc = 0.f;
                for (int r = 0; r < T; ++r) acc = fmaf(ds_s[r][c], x_s[r + W - 1 - i][c], acc);
                conv_acc[q4] += acc;
            }
        }
    }
    // this chunk's partial sums: part[(b, chunk)][n][...]
    const size_t pidx = ((size_t)b * nchunk + chunk) * (Hq + Hkv) + n;
    {
        const int mr = MB * (tid / MG), mc = MB * (tid % MG);
        float* const pm = part_mix + pidx * D * D;
#pragma unroll
        for (int u = 0; u < MB; ++u)
#pragma unroll
            for (int z = 0; z < MB; z += 4)
                *(f32x4_t*)(pm + (size_t)(mr + u) * D + mc + z) =
                    f32x4_t{mix_acc[u][z], mix_acc[u][z + 1], mix_acc[u][z + 2], mix_acc[u][z + 3]};
    }
    {
        float* const pc = part_conv + pidx * (size_t)W * D;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int e = tid + q4 * CB_THREADS;
            if (e < W * D) pc[e] = conv_acc[q4];
        }
    }
}

// Weight gradients: the sum of the P = B * nchunk partials of every weight
// element; element e of head n runs over dM (D D) then the taps (W D).
__global__ __launch_bounds__(CB_THREADS) void cca_bwd_reduce_kernel(
    float* __restrict__ dconv_q, float* __restrict__ dconv_k, float* __restrict__ dmix_q,
    float* __restrict__ dmix_k, const float* __restrict__ part_mix, const float* __restrict__ part_conv,
    int Hq, int Hkv, int D, int W, int P) {
    const int per = D * D + W * D;
    const long long idx = (long long)blockIdx.x * CB_THREADS + threadIdx.x;
    if (idx >= (long long)(Hq + Hkv) * per) return;
    const int n = (int)(idx / per), e = (int)(idx % per);
    const int NH = Hq + Hkv;
    float acc = 0.f;
    if (e < D * D) {
        for (int p = 0; p < P; ++p) acc += part_mix[((size_t)p * NH + n) * D * D + e];
        if (n < Hq) dmix_q[(size_t)n * D * D + e] = acc;
        else dmix_k[(size_t)(n - Hq) * D * D + e] = acc;
    } else {
        const int f = e - D * D;
        for (int p = 0; p < P; ++p) acc += part_conv[((size_t)p * NH + n) * W * D + f];
        if (n < Hq) dconv_q[(size_t)n * W * D + f] = acc;
        else dconv_k[(size_t)(n - Hq) * W * D + f] = acc;
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
    float* const part_mix = dm + (size_t)B * Hkv * S * D;
    float* const part_conv = part_mix + (size_t)P * (Hq + Hkv) * D * D;
    if ((long long)B * S > 0) {
        const long long items = (long long)B * Hkv * S * (D / 2);
        hipLaunchKernelGGL(cca_bwd_mean_kernel<D>, dim3((unsigned)((items + CB_THREADS - 1) / CB_THREADS)),
                           dim3(CB_THREADS), 0, st, dm, (uint16_t*)dv, (const uint16_t*)gq,
                           (const uint16_t*)gk, (const uint16_t*)gv, B, Hq, Hkv, S, pos_offset, rope, fr);
        hipLaunchKernelGGL(cca_bwd_head_kernel<D>, dim3((unsigned)((long long)B * (Hq + Hkv) * nchunk)),
                           dim3(CB_THREADS), 0, st, (uint16_t*)dq, (uint16_t*)dk, part_mix, part_conv,
                           (const float*)dm, (const uint16_t*)gq, (const uint16_t*)gk,
                           (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)conv_q,
                           (const uint16_t*)conv_k, (const uint16_t*)mix_q, (const uint16_t*)mix_k,
                           B, Hq, Hkv, S, W, pos_offset, rope, fr);
    }
    {
        const long long items = (long long)(Hq + Hkv) * (D * D + W * D);
        hipLaunchKernelGGL(cca_bwd_reduce_kernel, dim3((unsigned)((items + CB_THREADS - 1) / CB_THREADS)),
                           dim3(CB_THREADS), 0, st, dconv_q, dconv_k, dmix_q, dmix_k,
                           (const float*)part_mix, (const float*)part_conv, Hq, Hkv, D, W, P);
    }
    return hipGetLastError();
}

}  // namespace

size_t cca_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D, int W) {
    const size_t nchunk = ((size_t)S + CB_CHUNK - 1) / CB_CHUNK;
    const size_t P = (size_t)B * nchunk;
    return sizeof(float) * ((size_t)B * Hkv * S * D + P * (Hq + Hkv) * ((size_t)D * D + (size_t)W * D));
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
