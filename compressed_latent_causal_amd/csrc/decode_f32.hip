// fp32 accuracy path of single-token decode over a contiguous KV cache.
//
// What is computed ("Grouped Query Attention (GQA)" glossary, section "Por qué
// GQA reduce la caché KV"): the new query of every head attends to all len_b
// cached keys and values of its KV head, softmax(scale q.k) v, with the query
// rotated at position len_b - 1 when rope_theta > 0.  The same operation as
// the bf16 decode, for fp32 caches, in plain fp32 arithmetic: it is the
// accuracy path (results within 1e-5 of the fp64 definition), not a
// performance target.
//
// Two kernels.  The first splits each sequence into chunks of 512 keys: one
// workgroup per (chunk, sequence, KV head) stages 32 keys at a time in LDS,
// forms the scores of every query head of the group, keeps a running maximum
// and sum per head and accumulates its output, and writes the chunk's
// partial (o, max, sum) into the workspace.  The second combines a head's
// partials (log-sum-exp) and divides.  The workspace is the bf16 decode's
// (attn_decode_workspace_size), which holds ceil(max_len / 512) partials of
// D + 2 floats per (sequence, query head).
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr int DF_CHUNK = 512;   // keys per partial
constexpr int DF_SUB = 32;      // keys staged in LDS at a time
constexpr int DF_THREADS = 256;
constexpr int DF_MAX_GD = 4096;  // G * D at most: the output items a thread holds
constexpr int DF_IPT = DF_MAX_GD / DF_THREADS;

__device__ inline int clamp_len(const int32_t* seqlens, int b, int max_len) {
    return min(max(seqlens[b], 0), max_len);
}

template <int D>
__global__ __launch_bounds__(DF_THREADS) void decode_f32_partial_kernel(
    const float* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
    float* __restrict__ part, const int32_t* __restrict__ seqlens, int Hq, int Hkv, int S_cap,
    int max_len, int NC, float scale, int rope, RopeFreqs fr) {
    // LDS: q [G][D], k and v [DF_SUB][D], scores [G][DF_SUB], per head
    // (running max, running sum, rescale factor)
    extern __shared__ __attribute__((aligned(16))) float sm[];
    const int G = Hq / Hkv;
    float* const qs = sm;
    float* const ks = qs + G * D;
    float* const vs = ks + DF_SUB * D;
    float* const ss = vs + DF_SUB * D;
    float* const st = ss + G * DF_SUB;  // [G][3]

    const int tid = threadIdx.x;
    const int c = blockIdx.x;
    const int b = (int)blockIdx.y / Hkv, j = (int)blockIdx.y % Hkv;
    const int len = clamp_len(seqlens, b, max_len);
    const int t0 = c * DF_CHUNK;
    if (t0 >= len) return;  // no keys here; the merge reads ceil(len / 512) partials
    const int t1 = min(len, t0 + DF_CHUNK);

    // the group's queries, rotated at position len - 1 with RoPE
    for (int e = tid; e < G * (D / 2); e += DF_THREADS) {
        const int h = e / (D / 2), i = e % (D / 2);
        const float* const qr = q + ((size_t)b * Hq + (size_t)j * G + h) * D;
        float x0 = qr[2 * i], x1 = qr[2 * i + 1];
        if (rope) {
            float cs, sn, y0, y1;
            rope_cos_sin(len - 1, fr.f[i], cs, sn);
            rope_rotate(x0, x1, cs, sn, y0, y1);
            x0 = y0;
            x1 = y1;
        }
        qs[h * D + 2 * i] = x0;
        qs[h * D + 2 * i + 1] = x1;
    }
    for (int h = tid; h < G; h += DF_THREADS) {
        st[3 * h] = -INFINITY;
        st[3 * h + 1] = 0.f;
    }
    float oacc[DF_IPT];
#pragma unroll
    for (int u = 0; u < DF_IPT; ++u) oacc[u] = 0.f;

    const size_t kv_base = ((size_t)b * Hkv + j) * S_cap * D;
    for (int s0 = t0; s0 < t1; s0 += DF_SUB) {
        const int n = min(DF_SUB, t1 - s0);
        __syncthreads();  // the previous step's reads of k, v and the scores are done
        for (int e = tid; e < DF_SUB * D / 4; e += DF_THREADS) {
            const int r = e / (D / 4), c4 = e % (D / 4);
            f32x4_t kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
            if (r < n) {
                kx = *(const f32x4_t*)(kc + kv_base + (size_t)(s0 + r) * D + 4 * c4);
                vx = *(const f32x4_t*)(vc + kv_base + (size_t)(s0 + r) * D + 4 * c4);
            }
            *(f32x4_t*)(ks + r * D + 4 * c4) = kx;
            *(f32x4_t*)(vs + r * D + 4 * c4) = vx;
        }
        __syncthreads();
        // scores of every (head, key)
        for (int e = tid; e < G * DF_SUB; e += DF_THREADS) {
            const int h = e / DF_SUB, r = e % DF_SUB;
            float acc = 0.f;
            for (int d = 0; d < D; ++d) acc = fmaf(qs[h * D + d], ks[r * D + d], acc);
            ss[e] = r < n ? scale * acc : -INFINITY;
        }
        __syncthreads();
        // per head: the new running maximum, the rescale of what came before,
        // the probabilities and the running sum
        for (int h = tid; h < G; h += DF_THREADS) {
            float m = st[3 * h];
            for (int r = 0; r < n; ++r) m = fmaxf(m, ss[h * DF_SUB + r]);
            const float f = expf(st[3 * h] - m);  // 0 on the first step (max -inf)
            float l = 0.f;
            for (int r = 0; r < DF_SUB; ++r) {
                const float p = r < n ? expf(ss[h * DF_SUB + r] - m) : 0.f;
                ss[h * DF_SUB + r] = p;
                l += p;
            }
            st[3 * h] = m;
            st[3 * h + 1] = st[3 * h + 1] * f + l;
            st[3 * h + 2] = f;
        }
        __syncthreads();
        // o[h][d] = o[h][d] f + sum_r p[h][r] v[r][d]
#pragma unroll
        for (int u = 0; u < DF_IPT; ++u) {
            const int e = tid + u * DF_THREADS;
            if (e < G * D) {
                const int h = e / D, d = e % D;
                float acc = oacc[u] * st[3 * h + 2];
                for (int r = 0; r < n; ++r) acc = fmaf(ss[h * DF_SUB + r], vs[r * D + d], acc);
                oacc[u] = acc;
            }
        }
    }
    __syncthreads();
    // the chunk's partial: o[D], then (max, sum), per (sequence, query head, chunk)
#pragma unroll
    for (int u = 0; u < DF_IPT; ++u) {
        const int e = tid + u * DF_THREADS;
        if (e < G * D) {
            const int h = e / D, d = e % D;
            float* const pr = part + (((size_t)b * Hq + (size_t)j * G + h) * NC + c) * (D + 2);
            pr[d] = oacc[u];
            if (d == 0) {
                pr[D] = st[3 * h];
                pr[D + 1] = st[3 * h + 1];
            }
        }
    }
}

template <int D>
__global__ __launch_bounds__(D) void decode_f32_merge_kernel(float* __restrict__ o,
                                                            const float* __restrict__ part,
                                                            const int32_t* __restrict__ seqlens,
                                                            int Hq, int max_len, int NC) {
    const int b = (int)blockIdx.x / Hq, h = (int)blockIdx.x % Hq;
    const int d = threadIdx.x;
    const int len = clamp_len(seqlens, b, max_len);
    const int n = (len + DF_CHUNK - 1) / DF_CHUNK;
    const float* const pr = part + ((size_t)b * Hq + h) * NC * (D + 2);
    float M = -INFINITY;
    for (int c = 0; c < n; ++c) M = fmaxf(M, pr[(size_t)c * (D + 2) + D]);
    float L = 0.f, acc = 0.f;
    for (int c = 0; c < n; ++c) {
        const float w = expf(pr[(size_t)c * (D + 2) + D] - M);
        L = fmaf(pr[(size_t)c * (D + 2) + D + 1], w, L);
        acc = fmaf(pr[(size_t)c * (D + 2) + d], w, acc);
    }
    o[((size_t)b * Hq + h) * D + d] = n > 0 ? acc / L : 0.f;  // an empty sequence gives a zero row
}

template <int D>
hipError_t launch_decode_f32_d(void* o, const void* q, const void* k_cache, const void* v_cache,
                               int B, int Hq, int Hkv, int S_cap, const int32_t* seqlens,
                               int max_len, float scale, double rope_theta, void* workspace,
                               hipStream_t st) {
    const int NC = decode_num_chunks(B, Hkv, max_len);
    hipLaunchKernelGGL((decode_f32_partial_kernel<D>), dim3(NC, B * Hkv), dim3(DF_THREADS),
                       decode_f32_lds_bytes(Hq / Hkv, D), st, (const float*)q,
                       (const float*)k_cache, (const float*)v_cache, (float*)workspace, seqlens,
                       Hq, Hkv, S_cap, max_len, NC, scale, rope_theta > 0 ? 1 : 0,
                       rope_freqs(rope_theta > 0 ? rope_theta : 1.0, D));
    hipLaunchKernelGGL((decode_f32_merge_kernel<D>), dim3(B * Hq), dim3(D), 0, st, (float*)o,
                       (const float*)workspace, seqlens, Hq, max_len, NC);
    return hipGetLastError();
}

}  // namespace

bool decode_f32_supported(int G, int D) {
    return G * D <= DF_MAX_GD && decode_f32_lds_bytes(G, D) <= 64 * 1024;
}

size_t decode_f32_lds_bytes(int G, int D) {
    return ((size_t)G * D + 2 * DF_SUB * D + (size_t)G * DF_SUB + 3 * (size_t)G) * sizeof(float);
}

hipError_t launch_decode_f32(void* o, const void* q, const void* k_cache, const void* v_cache,
                             int B, int Hq, int Hkv, int S_cap, int D, const int32_t* seqlens,
                             int max_len, float scale, double rope_theta, void* workspace,
                             hipStream_t st) {
    return D == 64 ? launch_decode_f32_d<64>(o, q, k_cache, v_cache, B, Hq, Hkv, S_cap, seqlens,
                                             max_len, scale, rope_theta, workspace, st)
                   : launch_decode_f32_d<128>(o, q, k_cache, v_cache, B, Hq, Hkv, S_cap, seqlens,
                                              max_len, scale, rope_theta, workspace, st);
}

}  // namespace attn
