// Host-side launchers of the gfx950 kernels (internal to the library).  Each
// enqueues its kernels on `st` and returns the launch status; arguments have
// already been validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

struct RopeFreqs;
// theta^(-2i/D) for i < D/2, in double (host side)
RopeFreqs rope_freqs(double theta, int D);

// transpose != 0 applies the transpose of the rotation (rotation by the
// negated angle), the map of gradients back through RoPE.
hipError_t launch_rope(void* out, const void* in, int dtype, int B, int H, int S, int D,
                       const int32_t* pos_offset, int pos_shift, double theta, int transpose,
                       hipStream_t st);

// rope_theta > 0 rotates each query at its token index on the fly (k must
// already be rotated); rope_theta == 0 takes q as given.  lse (bf16 only, may
// be NULL): fp32 [B, Hq, S] log-normaliser of each row's scaled scores.
hipError_t launch_prefill(void* o, float* lse, const void* q, const void* k, const void* v,
                          int dtype, int B, int Hq, int Hkv, int S, int D, float scale,
                          double rope_theta, hipStream_t st);

// Backward pass of causal grouped-query prefill (bf16): gradients dq, dk, dv
// of sum <dout, o>, from q, k, v, the forward output o, dout and the forward's
// lse.  workspace: prefill_backward_workspace_bytes(B, Hq, Hkv, S, D) bytes
// (row statistics, and the dK/dV partial sums when the launch splits the
// group's heads; sized for the current device).
size_t prefill_backward_workspace_bytes(int B, int Hq, int Hkv, int S, int D);
hipError_t launch_prefill_backward(void* dq, void* dk, void* dv, const void* q, const void* k,
                                   const void* v, const void* o, const void* dout,
                                   const float* lse, int B, int Hq, int Hkv, int S, int D,
                                   float scale, void* workspace, hipStream_t st);

// Split workgroups (partial results) per (sequence, KV head) and workspace
// bytes for these sizes.
int decode_num_chunks(int B, int Hkv, int max_len);
size_t decode_workspace_bytes(int B, int Hq, int Hkv, int max_len, int D);

// rope_theta > 0 rotates each query at position seqlens[b] - 1 on the fly;
// rope_theta == 0 takes q as already rotated.
hipError_t launch_decode(void* o, const void* q, const void* k_cache, const void* v_cache, int B,
                         int Hq, int Hkv, int S_cap, int D, const int32_t* seqlens, int max_len,
                         float scale, double rope_theta, void* workspace, hipStream_t st);

// launch_decode with the library's static per-device scratch as its workspace
// (the caller has checked that decode_workspace_bytes fits it).
hipError_t launch_decode_noalloc(void* o, const void* q, const void* k_cache, const void* v_cache,
                                 int B, int Hq, int Hkv, int S_cap, int D, const int32_t* seqlens,
                                 int max_len, float scale, double rope_theta, hipStream_t st);

// Decode over a paged cache (pages [num_pages, Hkv, page_size, D], page_size a
// multiple of 32, block_table [B, max_pages]); window > 0 limits each query to
// its sequence's last `window` tokens.
hipError_t launch_decode_paged(void* o, const void* q, const void* k_pages, const void* v_pages,
                               int B, int Hq, int Hkv, int page_size, int D, int num_pages,
                               const int32_t* block_table, int max_pages, const int32_t* seqlens,
                               int max_len, int window, float scale, double rope_theta,
                               void* workspace, hipStream_t st);

// fp32 decode over a contiguous cache (accuracy path): chunk partials into
// the decode workspace, then a merge; groups with G * D <= 4096.
bool decode_f32_supported(int G, int D);
size_t decode_f32_lds_bytes(int G, int D);
hipError_t launch_decode_f32(void* o, const void* q, const void* k_cache, const void* v_cache,
                             int B, int Hq, int Hkv, int S_cap, int D, const int32_t* seqlens,
                             int max_len, float scale, double rope_theta, void* workspace,
                             hipStream_t st);

// CCA pre-attention operations (bf16): causal depthwise sequence convolution
// of width W (conv_q [Hq, W, D], conv_k [Hkv, W, D]), channel mix per head
// (mix_q [Hq, D, D], mix_k [Hkv, D, D]), the group's pre-convolution
// query/key mean, RoPE when rope_theta > 0, and the value shift.
int cca_max_width();
hipError_t launch_cca_mix(void* q_out, void* k_out, void* v_out, const void* q, const void* k,
                          const void* v, int B, int Hq, int Hkv, int S, int D, const void* conv_q,
                          const void* conv_k, int W, const void* mix_q, const void* mix_k,
                          const int32_t* pos_offset, double rope_theta, hipStream_t st);
// The same for one new token per sequence, the convolution's reach kept as
// state (q_state [B, Hq, W-1, D], k_state [B, Hkv, W-1, D] rings, v_state
// [B, Hkv, D]); dynamic LDS of cca_decode_lds_bytes(G, D).
size_t cca_decode_lds_bytes(int G, int D);
hipError_t launch_cca_decode(void* q_out, void* k_out, void* v_out, const void* q, const void* k,
                             const void* v, int B, int Hq, int Hkv, int D, const void* conv_q,
                             const void* conv_k, int W, const void* mix_q, const void* mix_k,
                             void* q_state, void* k_state, void* v_state, const int32_t* tok,
                             const int32_t* pos_offset, double rope_theta, hipStream_t st);

// Backward of the CCA pre-attention operations (bf16 in, bf16 input gradients,
// fp32 weight gradients); workspace of cca_bwd_workspace_bytes bytes.
int cca_bwd_max_width();
size_t cca_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D, int W);
hipError_t launch_cca_bwd(void* dq, void* dk, void* dv, float* dconv_q, float* dconv_k,
                          float* dmix_q, float* dmix_k, const void* gq, const void* gk,
                          const void* gv, const void* q, const void* k, int B, int Hq, int Hkv,
                          int S, int D, const void* conv_q, const void* conv_k, int W,
                          const void* mix_q, const void* mix_k, const int32_t* pos_offset,
                          double rope_theta, void* workspace, hipStream_t st);

}  // namespace attn
