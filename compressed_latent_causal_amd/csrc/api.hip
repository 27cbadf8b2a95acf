// C ABI of the attention library (declared in include/attn.h): argument
// validation on the host, then dispatch to the gfx950 kernels.  No HIP call is
// made before validation passes; the library allocates nothing.
#include <math.h>

#include "../../include/attn.h"
#include "kernels.hpp"

#define ATTN_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxGridYZ = 65535;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool supported_dim(int D) { return D == 64 || D == 128; }
bool known_dtype(int dt) { return dt == ATTN_F32 || dt == ATTN_BF16; }
bool good_scale(float s) { return isfinite(s) && s > 0.f; }

int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

}  // namespace

namespace {
int rope_call(void* out, const void* in, int dtype, int B, int H, int S, int D,
              const int32_t* pos_offset, int pos_shift, double theta, int transpose, void* stream) {
    if (B < 0 || S < 0 || H < 1) return ATTN_ERR_SHAPE;
    if (!known_dtype(dtype) || !supported_dim(D) || !(theta > 0.0) || !isfinite(theta))
        return ATTN_ERR_UNSUPPORTED;
    if (B > kMaxGridYZ || H > kMaxGridYZ) return ATTN_ERR_SHAPE;
    if (B == 0 || S == 0) return ATTN_OK;
    if (!out || !in) return ATTN_ERR_NULL;
    if (!aligned16(out) || !aligned16(in) || ((uintptr_t)pos_offset & 3u)) return ATTN_ERR_ALIGN;
    return hip_status(attn::launch_rope(out, in, dtype, B, H, S, D, pos_offset, pos_shift, theta,
                                        transpose, (hipStream_t)stream));
}
}  // namespace

ATTN_API int attn_rope(void* out, const void* in, int dtype, int B, int H, int S, int D,
                       const int32_t* pos_offset, int pos_shift, double theta, void* stream) {
    return rope_call(out, in, dtype, B, H, S, D, pos_offset, pos_shift, theta, 0, stream);
}

ATTN_API int attn_rope_backward(void* out, const void* in, int dtype, int B, int H, int S, int D,
                                const int32_t* pos_offset, int pos_shift, double theta,
                                void* stream) {
    return rope_call(out, in, dtype, B, H, S, D, pos_offset, pos_shift, theta, 1, stream);
}

ATTN_API int attn_prefill(void* o, const void* q, const void* k, const void* v, int dtype, int B,
                          int Hq, int Hkv, int S, int D, float scale, double rope_theta,
                          void* stream) {
    if (B < 0 || S < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
    if (!known_dtype(dtype) || !supported_dim(D) || !good_scale(scale)) return ATTN_ERR_UNSUPPORTED;
    if (!(rope_theta >= 0.0) || !isfinite(rope_theta)) return ATTN_ERR_UNSUPPORTED;
    if (B == 0 || S == 0) return ATTN_OK;
    // one workgroup per (query block, batch, KV head, head slice): stay in a 32-bit grid
    if ((long long)B * Hq * ((S + 31) / 32) >= (1ll << 31)) return ATTN_ERR_SHAPE;
    // one head's keys (or values) are addressed with 32-bit byte offsets
    if ((long long)S * D * (dtype == ATTN_BF16 ? 2 : 4) >= (1ll << 31)) return ATTN_ERR_SHAPE;
    if (!o || !q || !k || !v) return ATTN_ERR_NULL;
    if (!aligned16(o) || !aligned16(q) || !aligned16(k) || !aligned16(v)) return ATTN_ERR_ALIGN;
    return hip_status(attn::launch_prefill(o, nullptr, q, k, v, dtype, B, Hq, Hkv, S, D, scale,
                                           rope_theta, (hipStream_t)stream));
}

ATTN_API int attn_prefill_lse(void* o, float* lse, const void* q, const void* k, const void* v,
                              int dtype, int B, int Hq, int Hkv, int S, int D, float scale,
                              double rope_theta, void* stream) {
    if (B < 0 || S < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_BF16 || !supported_dim(D) || !good_scale(scale)) return ATTN_ERR_UNSUPPORTED;
    if (!(rope_theta >= 0.0) || !isfinite(rope_theta)) return ATTN_ERR_UNSUPPORTED;
    if (B == 0 || S == 0) return ATTN_OK;
    if ((long long)B * Hq * ((S + 31) / 32) >= (1ll << 31)) return ATTN_ERR_SHAPE;
    if ((long long)S * D * 2 >= (1ll << 31)) return ATTN_ERR_SHAPE;
    if (!o || !lse || !q || !k || !v) return ATTN_ERR_NULL;
    if (!aligned16(o) || !aligned16(q) || !aligned16(k) || !aligned16(v) || ((uintptr_t)lse & 3u))
        return ATTN_ERR_ALIGN;
    return hip_status(attn::launch_prefill(o, lse, q, k, v, dtype, B, Hq, Hkv, S, D, scale,
                                           rope_theta, (hipStream_t)stream));
}

ATTN_API size_t attn_prefill_backward_workspace_size(int B, int Hq, int Hkv, int S, int D) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || S < 1 || !supported_dim(D)) return 0;
    return attn::prefill_backward_workspace_bytes(B, Hq, Hkv, S, D);
}

ATTN_API int attn_prefill_backward(void* dq, void* dk, void* dv, const void* q, const void* k,
                                   const void* v, const void* o, const void* dout, const float* lse,
                                   int dtype, int B, int Hq, int Hkv, int S, int D, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 0 || S < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_BF16 || !supported_dim(D) || !good_scale(scale)) return ATTN_ERR_UNSUPPORTED;
    if (B == 0 || S == 0) return ATTN_OK;
    // grids of (key or query blocks) x B x Hq stay 32-bit; a head's rows and
    // its padded statistics are addressed with 32-bit byte offsets
    if ((long long)B * Hq * ((S + 31) / 32) >= (1ll << 31)) return ATTN_ERR_SHAPE;
    if ((long long)S * D * 2 >= (1ll << 31) || (long long)S + 128 >= (1ll << 28)) return ATTN_ERR_SHAPE;
    if (!dq || !dk || !dv || !q || !k || !v || !o || !dout || !lse) return ATTN_ERR_NULL;
    if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(q) || !aligned16(k) ||
        !aligned16(v) || !aligned16(o) || !aligned16(dout) || ((uintptr_t)lse & 3u))
        return ATTN_ERR_ALIGN;
    if (!workspace || workspace_bytes < attn::prefill_backward_workspace_bytes(B, Hq, Hkv, S, D))
        return ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
    return hip_status(attn::launch_prefill_backward(dq, dk, dv, q, k, v, o, dout, lse, B, Hq, Hkv,
                                                    S, D, scale, workspace, (hipStream_t)stream));
}

ATTN_API size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int max_len, int D) {
    if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_len < 0 || !supported_dim(D)) return 0;
    if (B == 0) return 0;
    return attn::decode_workspace_bytes(B, Hq, Hkv, max_len, D);
}

namespace {
// Checks shared by the contiguous decode entry points (everything but the
// workspace).  *empty is set when there is nothing to do.
int decode_checks(void* o, const void* q, const void* k_cache, const void* v_cache, int dtype,
                  int B, int Hq, int Hkv, int S_cap, int D, const int32_t* seqlens, int max_len,
                  float scale, double rope_theta, bool* empty, bool allow_f32 = false) {
    *empty = false;
    if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || S_cap < 1 || max_len < 0 || max_len > S_cap)
        return ATTN_ERR_SHAPE;
    const bool f32 = allow_f32 && dtype == ATTN_F32;
    if ((dtype != ATTN_BF16 && !f32) || !supported_dim(D) || !good_scale(scale))
        return ATTN_ERR_UNSUPPORTED;
    if (f32 && !attn::decode_f32_supported(Hq / Hkv, D)) return ATTN_ERR_UNSUPPORTED;
    if (!(rope_theta >= 0.0) || !isfinite(rope_theta)) return ATTN_ERR_UNSUPPORTED;
    if (B > kMaxGridYZ || (long long)Hkv * ((Hq / Hkv + 15) / 16) > kMaxGridYZ) return ATTN_ERR_SHAPE;
    if (f32 && (long long)B * Hkv > kMaxGridYZ) return ATTN_ERR_SHAPE;  // its grid's y extent
    // a group's partial results are addressed with 32-bit byte offsets
    if ((long long)max_len * D * (f32 ? 4 : 2) >= (1ll << 31)) return ATTN_ERR_SHAPE;
    if (B == 0) {
        *empty = true;
        return ATTN_OK;
    }
    if (!o || !q || !k_cache || !v_cache || !seqlens) return ATTN_ERR_NULL;
    if (!aligned16(o) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
        ((uintptr_t)seqlens & 3u))
        return ATTN_ERR_ALIGN;
    return ATTN_OK;
}
}  // namespace

ATTN_API int attn_decode(void* o, const void* q, const void* k_cache, const void* v_cache, int dtype,
                         int B, int Hq, int Hkv, int S_cap, int D, const int32_t* seqlens,
                         int max_len, float scale, double rope_theta, void* workspace,
                         size_t workspace_bytes, void* stream) {
    bool empty = false;
    const int rc = decode_checks(o, q, k_cache, v_cache, dtype, B, Hq, Hkv, S_cap, D, seqlens,
                                 max_len, scale, rope_theta, &empty, /*allow_f32=*/true);
    if (rc != ATTN_OK || empty) return rc;
    const size_t need = attn::decode_workspace_bytes(B, Hq, Hkv, max_len, D);
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
    if (dtype == ATTN_F32)
        return hip_status(attn::launch_decode_f32(o, q, k_cache, v_cache, B, Hq, Hkv, S_cap, D,
                                                  seqlens, max_len, scale, rope_theta, workspace,
                                                  (hipStream_t)stream));
    return hip_status(attn::launch_decode(o, q, k_cache, v_cache, B, Hq, Hkv, S_cap, D, seqlens,
                                          max_len, scale, rope_theta, workspace,
                                          (hipStream_t)stream));
}

ATTN_API int attn_decode_noalloc(void* o, const void* q, const void* k_cache, const void* v_cache,
                                 int dtype, int B, int Hq, int Hkv, int S_cap, int D,
                                 const int32_t* seqlens, int max_len, float scale,
                                 double rope_theta, void* stream) {
    bool empty = false;
    const int rc = decode_checks(o, q, k_cache, v_cache, dtype, B, Hq, Hkv, S_cap, D, seqlens,
                                 max_len, scale, rope_theta, &empty);
    if (rc != ATTN_OK || empty) return rc;
    if (attn::decode_workspace_bytes(B, Hq, Hkv, max_len, D) > (size_t)ATTN_DECODE_SCRATCH_BYTES)
        return ATTN_ERR_SCRATCH;
    return hip_status(attn::launch_decode_noalloc(o, q, k_cache, v_cache, B, Hq, Hkv, S_cap, D,
                                                  seqlens, max_len, scale, rope_theta,
                                                  (hipStream_t)stream));
}

ATTN_API int attn_decode_paged(void* o, const void* q, const void* k_pages, const void* v_pages,
                               int dtype, int B, int Hq, int Hkv, int page_size, int D,
                               int num_pages, const int32_t* block_table, int max_pages,
                               const int32_t* seqlens, int max_len, int window, float scale,
                               double rope_theta, void* workspace, size_t workspace_bytes,
                               void* stream) {
    if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || page_size < 32 || page_size % 32 != 0 ||
        num_pages < 1 || max_pages < 1 || max_len < 0 ||
        (long long)max_len > (long long)max_pages * page_size)
        return ATTN_ERR_SHAPE;
    if (dtype != ATTN_BF16 || !supported_dim(D) || !good_scale(scale)) return ATTN_ERR_UNSUPPORTED;
    if (!(rope_theta >= 0.0) || !isfinite(rope_theta)) return ATTN_ERR_UNSUPPORTED;
    if ((long long)B * max_pages > INT32_MAX) return ATTN_ERR_SHAPE;
    if ((long long)max_len * D * 2 >= (1ll << 31)) return ATTN_ERR_SHAPE;
    if (B == 0) return ATTN_OK;
    if (!o || !q || !k_pages || !v_pages || !block_table || !seqlens) return ATTN_ERR_NULL;
    if (!aligned16(o) || !aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) ||
        ((uintptr_t)block_table & 3u) || ((uintptr_t)seqlens & 3u))
        return ATTN_ERR_ALIGN;
    const size_t need = attn::decode_workspace_bytes(B, Hq, Hkv, max_len, D);
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
    return hip_status(attn::launch_decode_paged(o, q, k_pages, v_pages, B, Hq, Hkv, page_size, D,
                                                num_pages, block_table, max_pages, seqlens, max_len,
                                                window, scale, rope_theta, workspace,
                                                (hipStream_t)stream));
}

ATTN_API int attn_cca_mix(void* q_out, void* k_out, void* v_out, const void* q, const void* k,
                          const void* v, int dtype, int B, int Hq, int Hkv, int S, int D,
                          const void* conv_q, const void* conv_k, int conv_width,
                          const void* mix_q, const void* mix_k, const int32_t* pos_offset,
                          double rope_theta, void* stream) {
    if (B < 0 || S < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_BF16 || !supported_dim(D)) return ATTN_ERR_UNSUPPORTED;
    if (conv_width < 1 || conv_width > attn::cca_max_width()) return ATTN_ERR_UNSUPPORTED;
    if (!(rope_theta >= 0.0) || !isfinite(rope_theta)) return ATTN_ERR_UNSUPPORTED;
    if (B == 0 || S == 0) return ATTN_OK;
    // one workgroup per (64-token block, sequence, KV head); a head's rows
    // (plus a block past the end) are addressed with 32-bit byte offsets
    if ((long long)((S + 63) / 64) * B * Hkv >= (1ll << 31)) return ATTN_ERR_SHAPE;
    if ((long long)(S + 64) * D * 2 >= (1ll << 31)) return ATTN_ERR_SHAPE;
    if (!q_out || !k_out || !v_out || !q || !k || !v || !conv_q || !conv_k || !mix_q || !mix_k)
        return ATTN_ERR_NULL;
    if (!aligned16(q_out) || !aligned16(k_out) || !aligned16(v_out) || !aligned16(q) ||
        !aligned16(k) || !aligned16(v) || !aligned16(mix_q) || !aligned16(mix_k) ||
        !aligned16(conv_q) || !aligned16(conv_k) || ((uintptr_t)pos_offset & 3u))
        return ATTN_ERR_ALIGN;
    return hip_status(attn::launch_cca_mix(q_out, k_out, v_out, q, k, v, B, Hq, Hkv, S, D, conv_q,
                                           conv_k, conv_width, mix_q, mix_k, pos_offset,
                                           rope_theta, (hipStream_t)stream));
}

ATTN_API size_t attn_cca_mix_backward_workspace_size(int B, int Hq, int Hkv, int S, int D,
                                                     int conv_width) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || S < 1 || !supported_dim(D)) return 0;
    if (conv_width < 1 || conv_width > attn::cca_bwd_max_width()) return 0;
    return attn::cca_bwd_workspace_bytes(B, Hq, Hkv, S, D, conv_width);
}

ATTN_API int attn_cca_mix_backward(void* dq, void* dk, void* dv, float* dconv_q, float* dconv_k,
                                   float* dmix_q, float* dmix_k, const void* gq, const void* gk,
                                   const void* gv, const void* q, const void* k, int dtype, int B,
                                   int Hq, int Hkv, int S, int D, const void* conv_q,
                                   const void* conv_k, int conv_width, const void* mix_q,
                                   const void* mix_k, const int32_t* pos_offset,
                                   double rope_theta, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    if (B < 0 || S < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_BF16 || !supported_dim(D)) return ATTN_ERR_UNSUPPORTED;
    if (conv_width < 1 || conv_width > attn::cca_bwd_max_width()) return ATTN_ERR_UNSUPPORTED;
    if (!(rope_theta >= 0.0) || !isfinite(rope_theta)) return ATTN_ERR_UNSUPPORTED;
    // one workgroup per (sequence, head, 256-token chunk)
    if ((long long)B * (Hq + Hkv) * ((S + 255) / 256) >= (1ll << 31)) return ATTN_ERR_SHAPE;
    if (!dconv_q || !dconv_k || !dmix_q || !dmix_k) return ATTN_ERR_NULL;
    if (((uintptr_t)dconv_q & 3u) || ((uintptr_t)dconv_k & 3u) || ((uintptr_t)dmix_q & 3u) ||
        ((uintptr_t)dmix_k & 3u))
        return ATTN_ERR_ALIGN;
    if (B > 0 && S > 0) {
        if (!dq || !dk || !dv || !gq || !gk || !gv || !q || !k || !conv_q || !conv_k || !mix_q ||
            !mix_k)
            return ATTN_ERR_NULL;
        if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(gq) ||
            !aligned16(gk) || !aligned16(gv) || !aligned16(q) || !aligned16(k) ||
            !aligned16(mix_q) || !aligned16(mix_k) || ((uintptr_t)conv_q & 1u) ||
            ((uintptr_t)conv_k & 1u) || ((uintptr_t)pos_offset & 3u))
            return ATTN_ERR_ALIGN;
        if (!workspace ||
            workspace_bytes < attn::cca_bwd_workspace_bytes(B, Hq, Hkv, S, D, conv_width))
            return ATTN_ERR_WORKSPACE;
        if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
    }
    // with no token the weight gradients are zero (written by the reduce over
    // no partial sums); the input gradients are empty
    return hip_status(attn::launch_cca_bwd(dq, dk, dv, dconv_q, dconv_k, dmix_q, dmix_k, gq, gk,
                                           gv, q, k, B, Hq, Hkv, S, D, conv_q, conv_k, conv_width,
                                           mix_q, mix_k, pos_offset, rope_theta, workspace,
                                           (hipStream_t)stream));
}

ATTN_API int attn_cca_mix_decode(void* q_out, void* k_out, void* v_out, const void* q,
                                 const void* k, const void* v, int dtype, int B, int Hq, int Hkv,
                                 int D, const void* conv_q, const void* conv_k, int conv_width,
                                 const void* mix_q, const void* mix_k, void* q_state,
                                 void* k_state, void* v_state, const int32_t* t,
                                 const int32_t* pos_offset, double rope_theta, void* stream) {
    if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_BF16 || !supported_dim(D)) return ATTN_ERR_UNSUPPORTED;
    if (conv_width < 1 || conv_width > attn::cca_max_width()) return ATTN_ERR_UNSUPPORTED;
    if (!(rope_theta >= 0.0) || !isfinite(rope_theta)) return ATTN_ERR_UNSUPPORTED;
    // one workgroup per (sequence, KV group), the group's convolved rows in LDS
    if (attn::cca_decode_lds_bytes(Hq / Hkv, D) > 64 * 1024) return ATTN_ERR_UNSUPPORTED;
    if (B == 0) return ATTN_OK;
    if ((long long)B * Hkv >= (1ll << 31)) return ATTN_ERR_SHAPE;
    if (!q_out || !k_out || !v_out || !q || !k || !v || !conv_q || !conv_k || !mix_q || !mix_k ||
        !v_state || !t || (conv_width > 1 && (!q_state || !k_state)))
        return ATTN_ERR_NULL;
    if (!aligned16(q_out) || !aligned16(k_out) || !aligned16(v_out) || !aligned16(q) ||
        !aligned16(k) || !aligned16(v) || !aligned16(mix_q) || !aligned16(mix_k) ||
        !aligned16(conv_q) || !aligned16(conv_k) || !aligned16(q_state) || !aligned16(k_state) ||
        !aligned16(v_state) || ((uintptr_t)t & 3u) || ((uintptr_t)pos_offset & 3u))
        return ATTN_ERR_ALIGN;
    return hip_status(attn::launch_cca_decode(q_out, k_out, v_out, q, k, v, B, Hq, Hkv, D, conv_q,
                                              conv_k, conv_width, mix_q, mix_k, q_state, k_state,
                                              v_state, t, pos_offset, rope_theta,
                                              (hipStream_t)stream));
}

ATTN_API const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "invalid sizes (negative, Hq % Hkv != 0, max_len > S_cap, or too large)";
        case ATTN_ERR_UNSUPPORTED:
            return "unsupported argument (head dim not 64/128, dtype, theta or scale out of range, f32 decode or backward)";
        case ATTN_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
        case ATTN_ERR_HIP: return "kernel launch failed";
        case ATTN_ERR_SCRATCH:
            return "the problem needs more scratch than the allocation-free entry point holds "
                   "(ATTN_DECODE_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}
