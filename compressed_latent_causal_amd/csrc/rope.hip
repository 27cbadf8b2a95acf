// Rotary position embedding on [B, H, S, D] for gfx950.
//
// What is rotated ("Compressed Convolutional Attention" summary, section
// "Methodologie", item 4: RoPE acts on the per-head q and k of the attention
// space; "Latent-Condensed Transformer" summary, section 2B: it is a function of
// the absolute position): channel pair (2i, 2i+1) of token position p turns by
// the angle p * theta^(-2i/D), the original rotary form.
//
// Design: the kernel streams x once (16-byte loads and stores, whole
// contiguous rows per head) and is meant to run at HBM speed.  A workgroup owns
// a block of tokens of one sequence and a block of heads; each thread owns one
// 16-byte chunk of a row (4 bf16 pairs or 2 fp32 pairs).  The angle of each
// (token, pair) is formed once per thread and reused for every head of the
// block:
//   * the frequencies theta^(-2i/D) come from the host in double precision,
//   * p * freq and its reduction to [-pi, pi] are done in double precision
//     from the exact integer position (so large positions lose nothing),
//   * sine and cosine of the reduced angle are evaluated in fp32.
// The rotation itself is two fp32 multiply/FMA pairs per channel pair and the
// result is rounded to the storage type once (round to nearest even).
//
// The same kernel applies the transpose of the rotation (the map that carries
// a gradient of the rotated tensor back to the unrotated one): the rotation by
// the negated angle, i.e. the same cosines with the sines negated.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void rope_kernel(T* out, const T* in, int H, int S, int HB,
                                                   const int32_t* __restrict__ pos_offset,
                                                   int pos_shift, RopeFreqs fr, int transpose) {
    constexpr int EPT = 16 / sizeof(T);  // elements per 16-byte chunk
    constexpr int PPT = EPT / 2;         // channel pairs per thread
    constexpr int CH = D / EPT;          // chunks per row
    constexpr int TS = 256 / CH;         // tokens per workgroup
    const int c = threadIdx.x % CH;
    const int s = blockIdx.x * TS + threadIdx.x / CH;
    const int b = blockIdx.y;
    const int h_begin = blockIdx.z * HB, h_end = min(H, h_begin + HB);
    if (s >= S) return;

    const size_t head_stride = (size_t)S * D;
    const size_t off = ((size_t)b * H * S + s) * D + (size_t)c * EPT;
    // Heads are processed in groups of eight whose loads are all issued before
    // any store, so the loads overlap; each thread touches only its own chunk
    // of each head, so this order is also correct when out == in.  The first
    // group's loads are issued before the angles are formed, so the sine and
    // cosine work overlaps their latency.
    constexpr int HG = 8;
    u32x4_t x[HG];
    auto load = [&](int h0) __attribute__((always_inline)) {
        // every lane issues all HG loads (heads past the block re-read its
        // last head and are not stored), so the loads' count is fixed and the
        // waits for them can be counted
#pragma unroll
        for (int u = 0; u < HG; ++u)
            x[u] = *(const u32x4_t*)(in + off + (size_t)min(h0 + u, h_end - 1) * head_stride);
    };
    // the frequencies and the position first: their loads then complete
    // before the data loads, and the angles need not wait for the data
    double fq[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) fq[j] = fr.f[c * PPT + j];
    const long long p = (long long)(pos_offset ? pos_offset[b] : 0) + pos_shift + s;
    load(h_begin);

    float cs[PPT], sn[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        rope_cos_sin(p, fq[j], cs[j], sn[j]);
        if (transpose) sn[j] = -sn[j];
    }

    for (int h0 = h_begin; h0 < h_end; h0 += HG) {
        if (h0 != h_begin) load(h0);
#pragma unroll
        for (int u = 0; u < HG; ++u) {
            if (h0 + u >= h_end) break;
            u32x4_t y;
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int j = 0; j < PPT; ++j) {
                    float y0, y1;
                    rope_rotate(bf16_lo(x[u][j]), bf16_hi(x[u][j]), cs[j], sn[j], y0, y1);
                    y[j] = pack_bf16x2(y0, y1);
                }
            } else {
#pragma unroll
                for (int j = 0; j < PPT; ++j) {
                    float y0, y1;
                    rope_rotate(__uint_as_float(x[u][2 * j]), __uint_as_float(x[u][2 * j + 1]),
                                cs[j], sn[j], y0, y1);
                    y[2 * j] = __float_as_uint(y0);
                    y[2 * j + 1] = __float_as_uint(y1);
                }
            }
            *(u32x4_t*)(out + off + (size_t)(h0 + u) * head_stride) = y;
        }
    }
}

template <typename T, int D>
hipError_t launch_rope_t(void* out, const void* in, int B, int H, int S, const int32_t* pos_offset,
                         int pos_shift, double theta, int transpose, hipStream_t st) {
    constexpr int TS = 256 / (D / (16 / sizeof(T)));
    const RopeFreqs fr = rope_freqs(theta, D);
    // Heads per workgroup: all of them when the token blocks alone fill the
    // chip (the angles are then formed once per token), fewer for short inputs
    // such as a decode step's single token.
    const long long tok_blocks = (long long)ceil_div(S, TS) * B;
    int HB = H;
    if (tok_blocks < 1024) HB = tok_blocks >= 256 ? 8 : 1;
    HB = min(HB, H);
    dim3 grid(ceil_div(S, TS), B, ceil_div(H, HB));
    hipLaunchKernelGGL((rope_kernel<T, D>), grid, dim3(256), 0, st, (T*)out, (const T*)in, H, S, HB,
                       pos_offset, pos_shift, fr, transpose);
    return hipGetLastError();
}

}  // namespace

RopeFreqs rope_freqs(double theta, int D) {
    RopeFreqs fr{};
    for (int i = 0; i < D / 2; ++i) fr.f[i] = pow(theta, -2.0 * i / D);
    return fr;
}

hipError_t launch_rope(void* out, const void* in, int dtype, int B, int H, int S, int D,
                       const int32_t* pos_offset, int pos_shift, double theta, int transpose,
                       hipStream_t st) {
    const int tr = transpose ? 1 : 0;
    if (dtype == kBF16)
        return D == 64 ? launch_rope_t<uint16_t, 64>(out, in, B, H, S, pos_offset, pos_shift, theta, tr, st)
                       : launch_rope_t<uint16_t, 128>(out, in, B, H, S, pos_offset, pos_shift, theta, tr, st);
    return D == 64 ? launch_rope_t<float, 64>(out, in, B, H, S, pos_offset, pos_shift, theta, tr, st)
                   : launch_rope_t<float, 128>(out, in, B, H, S, pos_offset, pos_shift, theta, tr, st);
}

}  // namespace attn
