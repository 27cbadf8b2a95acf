// Rotary position embedding on [B, H, S, D] for gfx950.
//
// What is rotated ("Compressed Convolutional Attention" summary, section
// "Methodologie", item 4: RoPE acts on the per-head q and k of the attention
// space; "Latent-Condensed Transformer" summary, section 2B: it is a function of
// the absolute position): channel pair (2i, 2i+1) of token position p turns by
// the angle p * theta^(-2i/D), the original rotary form.
//
// Design: a workgroup owns a block of tokens of one sequence and loops over all
// H heads.  Each thread owns one 16-byte chunk of a row (4 pairs of bf16 or 2
// pairs of fp32) and forms the cosines and sines of its pairs once, in double
// precision from the exact integer position, then reuses them for every head.
// The rotation is evaluated in double and rounded once to the storage type, so
// the result is the correctly rounded rotation up to the ~1e-16 error of the
// double-precision sine and cosine.  Memory traffic is one read and one write of
// x, fully coalesced (a workgroup reads whole contiguous rows of each head).
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

// double -> bf16 bits, round to nearest even, without double rounding: the
// first step rounds toward zero to binary32 and records inexactness in the
// lowest bit (round to odd), which the second, 16-bit RNE step then sees.
__device__ inline unsigned d2bf16(double y) {
    float f = __double2float_rz(y);
    unsigned u = __float_as_uint(f);
    if ((double)f != y && (u & 0x7fffffffu) < 0x7f800000u) u |= 1u;
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void rope_kernel(T* out, const T* in,
                                                   int H, int S, const int32_t* __restrict__ pos_offset,
                                                   int pos_shift, double log2_theta) {
    constexpr int EPT = 16 / sizeof(T);  // elements per 16-byte chunk
    constexpr int PPT = EPT / 2;         // channel pairs per thread
    constexpr int CH = D / EPT;          // chunks per row
    constexpr int TS = 256 / CH;         // tokens per workgroup
    const int c = threadIdx.x % CH;
    const int s = blockIdx.x * TS + threadIdx.x / CH;
    const int b = blockIdx.y;
    if (s >= S) return;

    const long long p = (long long)(pos_offset ? pos_offset[b] : 0) + pos_shift + s;
    const double two_pi_hi = 6.28318530717958623200;    // 2*pi rounded to double
    const double two_pi_lo = 2.44929359829470635445e-16;  // 2*pi - two_pi_hi
    double cs[PPT], sn[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int i = c * PPT + j;
        const double freq = exp2(-(2.0 * i / D) * log2_theta);
        const double ang = (double)p * freq;
        const double k = rint(ang * 0.15915494309189533577);  // ang / (2 pi)
        double r = fma(-k, two_pi_hi, ang);
        r = fma(-k, two_pi_lo, r);
        sincos(r, &sn[j], &cs[j]);
    }

    const size_t head_stride = (size_t)S * D;
    const size_t off = ((size_t)b * H * S + s) * D + (size_t)c * EPT;
    // Heads are processed in groups of four whose loads are all issued before
    // any store, so the loads overlap; each thread touches only its own chunk
    // of each head, so this order is also correct when out == in.
    constexpr int HG = 4;
    for (int h0 = 0; h0 < H; h0 += HG) {
        u32x4_t x[HG];
#pragma unroll
        for (int u = 0; u < HG; ++u)
            if (h0 + u < H) x[u] = *(const u32x4_t*)(in + off + (size_t)(h0 + u) * head_stride);
#pragma unroll
        for (int u = 0; u < HG; ++u) {
            if (h0 + u >= H) break;
            u32x4_t y;
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int j = 0; j < PPT; ++j) {
                    const double x0 = bf16_lo(x[u][j]), x1 = bf16_hi(x[u][j]);
                    const double y0 = x0 * cs[j] - x1 * sn[j];
                    const double y1 = x0 * sn[j] + x1 * cs[j];
                    y[j] = d2bf16(y0) | (d2bf16(y1) << 16);
                }
            } else {
#pragma unroll
                for (int j = 0; j < PPT; ++j) {
                    const double x0 = __uint_as_float(x[u][2 * j]);
                    const double x1 = __uint_as_float(x[u][2 * j + 1]);
                    y[2 * j] = __float_as_uint((float)(x0 * cs[j] - x1 * sn[j]));
                    y[2 * j + 1] = __float_as_uint((float)(x0 * sn[j] + x1 * cs[j]));
                }
            }
            *(u32x4_t*)(out + off + (size_t)(h0 + u) * head_stride) = y;
        }
    }
}

template <typename T, int D>
hipError_t launch_rope_t(void* out, const void* in, int B, int H, int S, const int32_t* pos_offset,
                         int pos_shift, double theta, hipStream_t st) {
    constexpr int TS = 256 / (D / (16 / sizeof(T)));
    dim3 grid(ceil_div(S, TS), B);
    hipLaunchKernelGGL((rope_kernel<T, D>), grid, dim3(256), 0, st, (T*)out, (const T*)in, H, S,
                       pos_offset, pos_shift, log2(theta));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(void* out, const void* in, int dtype, int B, int H, int S, int D,
                       const int32_t* pos_offset, int pos_shift, double theta, hipStream_t st) {
    if (dtype == kBF16)
        return D == 64 ? launch_rope_t<uint16_t, 64>(out, in, B, H, S, pos_offset, pos_shift, theta, st)
                       : launch_rope_t<uint16_t, 128>(out, in, B, H, S, pos_offset, pos_shift, theta, st);
    return D == 64 ? launch_rope_t<float, 64>(out, in, B, H, S, pos_offset, pos_shift, theta, st)
                   : launch_rope_t<float, 128>(out, in, B, H, S, pos_offset, pos_shift, theta, st);
}

}  // namespace attn
