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

hipError_t launch_rope(void* out, const void* in, int dtype, int B, int H, int S, int D,
                       const int32_t* pos_offset, int pos_shift, double theta, hipStream_t st);

hipError_t launch_prefill(void* o, const void* q, const void* k, const void* v, int dtype, int B,
                          int Hq, int Hkv, int S, int D, float scale, hipStream_t st);

// Decode key-chunk length (tokens per split workgroup) for these sizes.
int decode_chunk_tokens(int B, int Hkv, int max_len);
// Number of key chunks and workspace bytes for these sizes.
int decode_num_chunks(int B, int Hkv, int max_len);
size_t decode_workspace_bytes(int B, int Hq, int Hkv, int max_len, int D);

hipError_t launch_decode(void* o, const void* q, const void* k_cache, const void* v_cache, int B,
                         int Hq, int Hkv, int S_cap, int D, const int32_t* seqlens, int max_len,
                         float scale, void* workspace, hipStream_t st);

}  // namespace attn
