// Device-side building blocks shared by the gfx950 attention kernels:
// vector types, bf16 conversions, the 16x16x32 bf16 matrix-core product,
// LDS transpose reads and the XOR swizzle used for K/V tiles in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace attn {

// ---------------------------------------------------------------- types
typedef short bf16x8_t __attribute__((__vector_size__(8 * sizeof(short))));  // 8 bf16 bit patterns
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr float kLog2e = 1.4426950408889634f;

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ constexpr long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- bf16
// bf16 -> fp32 is exact: the 16 bits are the top half of a binary32.
__device__ inline float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ inline unsigned pack_bf16x2(float lo, float hi) {
    f32x2_t f = {lo, hi};
    bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
    return __builtin_bit_cast(unsigned, b);
}

// ---------------------------------------------------------------- matrix core
// D = A * B + C for a 16x16 fp32 tile with K = 32 bf16.
// Lane l supplies A[m = l%16][k = 8*(l/16) .. +7] and B[k = 8*(l/16) .. +7][n = l%16]
// and receives D[m = 4*(l/16) + i][n = l%16] in element i.  Any fixed
// permutation of k applied to both A and B leaves the product unchanged.
__device__ inline f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- LDS
// Transpose read of 4 bf16 (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives element (i % 4) of the 8-byte chunks addressed by
// lanes 4*j + i/4 for j = 0..3.  If lane L of the group addresses
// row (r0 + L/4), columns (c0 + 4*(L%4)) .. +3 of a row-major tile, lane i
// receives column c0 + i of rows r0 .. r0+3.
__device__ inline bf16x4_t lds_read_tr(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p);
}

// LDS tile layouts.  Tiles are row-major (rows of D bf16, no padding) with the
// 16-byte chunks of each row XOR-permuted by bits of the row index.  Two
// permutations are used, one per read pattern (both measured free of bank
// conflicts on gfx950):
//  * swz_k: 16 consecutive lanes read one logical chunk of 16 consecutive rows
//    with ds_read_b128 (the matrix-core K operand): chunk c ^ (r & 15) for
//    D = 128, c ^ ((r >> 1) & 7) for D = 64;
//  * swz_v: the transpose read, where each 16-lane group reads 32 contiguous
//    bytes of 4 consecutive rows: chunk c ^ (((r & 7) << 1) | ((r >> 3) & 1))
//    for D = 128 and c ^ ((((r >> 1) & 3) << 1) | ((r >> 3) & 1)) for D = 64.
// A whole row is always written by 16 (or 8) consecutive lanes, which any
// in-row permutation keeps conflict-free.
template <int D>
__device__ inline int swz_k(int r, int c) {
    static_assert(D == 64 || D == 128, "head dim");
    if constexpr (D == 128)
        return r * 256 + ((c ^ (r & 15)) << 4);
    else
        return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
}

template <int D>
__device__ inline int swz_v(int r, int c) {
    static_assert(D == 64 || D == 128, "head dim");
    if constexpr (D == 128)
        return r * 256 + ((c ^ (((r & 7) << 1) | ((r >> 3) & 1))) << 4);
    else
        return r * 128 + ((c ^ ((((r >> 1) & 3) << 1) | ((r >> 3) & 1))) << 4);
}

// Per-lane byte offsets of the O^T = V^T P^T operand reads in a swz_v tile.
// For d tile dt, lane l reads V[key][d] for d = 16 dt + l%16 and the 8 keys
//   r0 + 4*(l/16) + {0,1,2,3}  and  r0 + 16 + 4*(l/16) + {0,1,2,3}
// (two transpose reads).  The keys match the rows that element i of the S^T =
// K Q^T tiles m and m+1 hold in lane group l/16.  Because the swizzle depends
// only on row bits 0..3, the offset of rows r0 = 32k (+16) is the dt offset
// plus the constant 32k * D * 2 (+ 16 * D * 2).
template <int D>
__device__ inline int v_frag_off(int dt, int lane) {
    const int g = lane >> 4, L = lane & 15;
    const int col = 16 * dt + 4 * (L & 3);  // first of the 4 columns this lane addresses
    return swz_v<D>(4 * g + (L >> 2), col >> 3) + (col & 7) * 2;
}

template <int D>
__device__ inline bf16x8_t v_frag_at(const char* p) {
    constexpr int kRow16 = 16 * D * 2;
    bf16x4_t lo = lds_read_tr(p);
    bf16x4_t hi = lds_read_tr(p + kRow16);
    u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
    u32x4_t w = {l2.x, l2.y, h2.x, h2.y};
    return __builtin_bit_cast(bf16x8_t, w);
}

// ---------------------------------------------------------------- RoPE
// Rotary embedding of channel pair (2i, 2i+1) at integer position p by the
// angle p * theta^(-2i/D).  The frequencies come from the host in double; the
// angle and its reduction to [-pi, pi] are formed in double from the exact
// position, sine and cosine of the reduced angle in fp32, and the rotation is
// one product and one FMA per output.  Every kernel that applies RoPE uses
// these two functions, so fused and stand-alone rotations agree bit for bit.
constexpr int kMaxPairs = 64;  // D / 2 for D = 128

struct RopeFreqs {
    double f[kMaxPairs];  // theta^(-2i/D), i < D/2
};

__device__ inline void rope_cos_sin(long long p, double freq, float& cs, float& sn) {
    const double two_pi_hi = 6.28318530717958623200;      // 2*pi rounded to double
    const double two_pi_lo = 2.44929359829470635445e-16;  // 2*pi - two_pi_hi
    const double ang = (double)p * freq;
    const double k = rint(ang * 0.15915494309189533577);  // ang / (2 pi)
    double r = fma(-k, two_pi_hi, ang);
    r = fma(-k, two_pi_lo, r);
    sincosf((float)r, &sn, &cs);
}

// (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos)
__device__ inline void rope_rotate(float x0, float x1, float cs, float sn, float& y0, float& y1) {
    y0 = fmaf(x0, cs, -x1 * sn);
    y1 = fmaf(x0, sn, x1 * cs);
}

// ---------------------------------------------------------------- cross-lane
__device__ inline float xor_shfl(float x, int m) { return __shfl_xor(x, m, 64); }

// Reductions over the four lanes l, l^16, l^32, l^48 (the lane groups that
// share a row of a 16x16 matrix-core result) with the cross-row swap
// instructions: each swap, given the same register twice, returns one copy
// holding the lanes' own rows and one holding the partner rows.
__device__ inline float group4_max(float x) {  // NaN-propagating maximum
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float group4_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Buffer resource over `bytes` bytes at `base` (raw addressing, no stride).
// Loads through it that fall past `bytes` return zeros instead of touching
// memory.  The last word selects 32-bit data format, as raw loads require.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
typedef __attribute__((address_space(3))) void lds_void_t;

// One wave-wide 16-byte-per-lane load from `rs` at byte voff + soff straight
// into LDS: lane l's data lands at lds + 16 l (lds must be wave-uniform).
__device__ __attribute__((always_inline)) inline void dma16(__amdgpu_buffer_rsrc_t rs, char* lds,
                                                            int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds, 16, voff, soff, 0, 0);
}

// Compute units of the current device (cached per device; 256 if the query
// fails).  Launch planning sizes grids and splits from it.
inline int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace attn
