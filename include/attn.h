/*
 * attn.h -- C ABI of the MI355X (gfx950) causal grouped-query attention
 * library: rotary position embedding, causal prefill (forward and backward),
 * single-token decode over a contiguous or a paged KV cache, and CCA's
 * pre-attention operations on the compressed q, k, v (prefill and decode step).
 *
 * What is computed (pages cited by title and section):
 *  - "Grouped Query Attention (GQA)" glossary, section "Cómo funciona GQA":
 *    query heads are split into Hkv consecutive groups of G = Hq / Hkv heads;
 *    every head of group j attends with its own queries to the one key head
 *    and one value head j, using unchanged scaled dot-product attention.  The
 *    page's example is causal, and equals multi-head attention with each
 *    key/value head repeated (interleaved) G times.  G = 1 is multi-head
 *    attention, Hkv = 1 multi-query attention.
 *  - same page, section "Por qué GQA reduce la caché KV": in generation the
 *    keys/values of all earlier tokens sit in a cache that is read in full for
 *    every new token; its size scales with Hkv, not Hq.
 *  - "Compressed Convolutional Attention" summary, section "Methodologie"
 *    (items 1 and 4, and the CCGQA paragraph): attention runs entirely inside
 *    a compressed latent of small per-head dims, with key/value heads shared by
 *    groups, and RoPE applied there directly to q and k.
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers, contiguous, innermost dim D (stride
 *    1), and 16-byte aligned.  Element type is given by `dtype`.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued on it; calls return without synchronising.  The caller keeps
 *    every buffer alive until that work completes.
 *  - The library allocates and frees nothing and keeps no state between calls
 *    (apart from a process-wide sequence number that tags each decode call and
 *    the static per-device scratch behind attn_decode_noalloc);
 *    calls on different streams may run concurrently on distinct buffers.
 *  - Arguments are validated on the host before any HIP call.  On a non-zero
 *    status nothing was enqueued.  ATTN_ERR_HIP reports a failed launch (the
 *    HIP error is consumed with hipGetLastError).
 *  - An empty problem (B == 0 or S == 0) returns ATTN_OK and enqueues nothing.
 *  - Supported head dims: D = 64 and D = 128.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_F32 = 0,   /* IEEE binary32 */
    ATTN_BF16 = 1   /* bfloat16 (top half of binary32), round to nearest even */
} attn_dtype;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,         /* a required pointer is NULL */
    ATTN_ERR_SHAPE = 2,        /* negative size, Hq/Hkv < 1, Hq % Hkv != 0, max_len > S_cap, ... */
    ATTN_ERR_UNSUPPORTED = 3,  /* D not 64/128, unknown dtype, theta/scale out of range, f32 decode/training */
    ATTN_ERR_ALIGN = 4,        /* a tensor pointer is not 16-byte aligned */
    ATTN_ERR_WORKSPACE = 5,    /* workspace missing or too small */
    ATTN_ERR_HIP = 6,          /* a kernel launch failed */
    ATTN_ERR_SCRATCH = 7       /* attn_decode_noalloc: the problem exceeds ATTN_DECODE_SCRATCH_BYTES */
} attn_status;

/* Bytes of the static per-device scratch behind attn_decode_noalloc. */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * Rotary position embedding of x [B, H, S, D] into out [B, H, S, D].
 *
 * Token s of sequence b sits at the integer position
 *     p = pos_offset[b] + pos_shift + s        (pos_offset NULL: offsets 0)
 * and for every head and channel pair i < D/2 the pair (x[2i], x[2i+1]) is
 * rotated by the angle p * theta^(-2i/D):
 *     out[2i]   = x[2i] cos(a) - x[2i+1] sin(a)
 *     out[2i+1] = x[2i] sin(a) + x[2i+1] cos(a).
 * The pages name RoPE ("Compressed Convolutional Attention", "Methodologie"
 * item 4; "Latent-Condensed Transformer", section 2B: a nonlinear function of
 * absolute position) without printing its formula; this is the original
 * rotary form with adjacent channel pairs.  Use it on Q and on K (never V).
 * For a decode query [B, Hq, 1, D] pass pos_offset = seqlens, pos_shift = -1.
 *
 * out == in is allowed (in place); other overlaps are undefined.
 * pos_offset: device int32[B] or NULL.  theta > 0.  dtype: F32 or BF16.
 * The angle is formed from the exact integer position in double precision.
 */
int attn_rope(void *out, const void *in, int dtype, int B, int H, int S, int D,
              const int32_t *pos_offset, int pos_shift, double theta, void *stream);

/*
 * Transpose of attn_rope, for gradients: out = R^T in, where R is the rotation
 * attn_rope applies with the same positions and theta.  Pair (2i, 2i+1) turns
 * by the negated angle:
 *     out[2i]   =  in[2i] cos(a) + in[2i+1] sin(a)
 *     out[2i+1] = -in[2i] sin(a) + in[2i+1] cos(a),   a = p * theta^(-2i/D).
 * Given the gradients attn_prefill_backward returns for the rotated q and k,
 * this yields the gradients of the unrotated ones.  Arguments, layout,
 * rounding and errors as attn_rope (out == in allowed).
 */
int attn_rope_backward(void *out, const void *in, int dtype, int B, int H, int S, int D,
                       const int32_t *pos_offset, int pos_shift, double theta, void *stream);

/*
 * Causal grouped-query attention over one sequence block ("prefill").
 *
 *   q, o: [B, Hq, S, D];  k, v: [B, Hkv, S, D];  Hq % Hkv == 0, G = Hq / Hkv.
 *   o[b,h,i,:] = sum_{t<=i} softmax_t(scale * <q[b,h,i,:], k[b,h/G,t,:]>) v[b,h/G,t,:]
 *
 * Queries and keys share positions (the page's is_causal example: query i sees
 * keys 0..i).  bf16 inputs use bf16 matrix-core products with fp32
 * accumulation and an fp32 softmax; the probabilities are rounded to bf16
 * before the product with V.  fp32 inputs are computed in fp32 throughout.
 * o must not overlap q, k or v.  scale > 0 and finite, usually 1/sqrt(D).
 * rope_theta > 0: q is taken unrotated and query i is rotated on the fly at
 * position i (bit for bit what attn_rope with pos_offset NULL, pos_shift 0
 * produces); k must already be rotated (attn_rope on K).  rope_theta == 0: q
 * is used as given.
 * One head's keys must span less than 2 GiB (S * D * element size < 2^31),
 * else ATTN_ERR_SHAPE.
 */
int attn_prefill(void *o, const void *q, const void *k, const void *v, int dtype,
                 int B, int Hq, int Hkv, int S, int D, float scale, double rope_theta,
                 void *stream);

/*
 * attn_prefill that also writes each row's log-normaliser, for training:
 *   lse[b,h,i] = log sum_{t<=i} exp(scale * <q[b,h,i,:], k[b,h/G,t,:]>)
 * (natural log; device fp32 [B, Hq, S], 4-byte aligned).  o and every other
 * argument as attn_prefill, bf16 only.  The forward's probabilities are the
 * exponentials of its scores minus lse, so lse is what attn_prefill_backward
 * needs to recompute them.
 */
int attn_prefill_lse(void *o, float *lse, const void *q, const void *k, const void *v,
                     int dtype, int B, int Hq, int Hkv, int S, int D, float scale,
                     double rope_theta, void *stream);

/*
 * Bytes of device workspace attn_prefill_backward needs for these sizes on the
 * current device (0 on invalid sizes): two fp32 row statistics per query row,
 * each head padded to whole 64-row tiles plus one, and, when the dk/dv pass
 * splits the group's query heads over hs = 2 or 4 workgroups per key block
 * (shapes that would not fill the device three times over), hs fp32 partial
 * sums of dk and dv ([hs][2][B, Hkv, S, D]).  The split depends on the
 * device's compute-unit count, so a workspace sized on one device is only
 * guaranteed for that device.
 */
size_t attn_prefill_backward_workspace_size(int B, int Hq, int Hkv, int S, int D);

/*
 * Backward pass of causal grouped-query prefill ("Compressed Convolutional
 * Attention" summary, "Resultaten", which reports this pass for the same
 * attention): the gradients of sum <dout, o> for o = attn_prefill(q, k, v),
 *   p_it = exp(scale <q_i, k_t> - lse_i),  ds_it = p_it (<dout_i, v_t> - <dout_i, o_i>)
 *   dq_i = scale sum_{t<=i} ds_it k_t
 *   dk_t = scale sum_{h in group} sum_{i>=t} ds_it q_i
 *   dv_t = sum_{h in group} sum_{i>=t} p_it dout_i
 * q, o, dout, dq: [B, Hq, S, D];  k, v, dk, dv: [B, Hkv, S, D];  lse: fp32
 * [B, Hq, S] from attn_prefill_lse on the same q, k, v, with o its output.
 * q and k are the tensors attention saw (already rotated); the gradients are
 * with respect to them (attn_rope_backward carries dq and dk back through the
 * rotation).  bf16 only: bf16 matrix-core products with fp32
 * accumulation, p and ds rounded to bf16 before their products, each
 * gradient rounded once to bf16.  Outputs must not overlap inputs.
 * workspace: at least attn_prefill_backward_workspace_size(B, Hq, Hkv, S, D)
 * bytes (ATTN_ERR_WORKSPACE otherwise), 16-byte aligned, contents on entry
 * irrelevant, not shared by calls that may overlap.  Three kernels are
 * enqueued (row statistics, dk/dv, dq); dk and dv sum the group's query heads
 * in registers and are written once, except for split launches, which write
 * fp32 partial sums to the workspace and add a fourth kernel that sums them
 * and rounds once to bf16.
 */
int attn_prefill_backward(void *dq, void *dk, void *dv, const void *q, const void *k,
                          const void *v, const void *o, const void *dout, const float *lse,
                          int dtype, int B, int Hq, int Hkv, int S, int D, float scale,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace attn_decode needs for these sizes (0 on invalid
 * sizes).  The workspace holds fp32 partial results (D + 2 floats) per
 * (sequence, query head, split workgroup), one 64-bit call tag per
 * (sequence, KV head, slice of up to 16 query heads, split workgroup) and one
 * 64-bit epoch per (sequence, KV head, slice).  A split workgroup covers at
 * least 16 x 32 cache tokens, so a sequence has at most ceil(max_len / 512)
 * of them.
 */
size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int max_len, int D);

/*
 * One new query token per sequence against a contiguous KV cache ("decode").
 *
 *   q, o: [B, Hq, D];  k_cache, v_cache: [B, Hkv, S_cap, D];
 *   seqlens: device int32[B], seqlens[b] = number of valid cached tokens of
 *   sequence b (the new token's key/value included), 0 <= seqlens[b] <= max_len.
 *   o[b,h,:] = sum_{t<len_b} softmax_t(scale * <q[b,h,:], k[b,h/G,t,:]>) v[b,h/G,t,:]
 *
 * Cache slots at or beyond seqlens[b] are never read into the result (they may
 * hold anything, NaN included).  A sequence with seqlens[b] == 0 gets a zero
 * row.  Out-of-contract lengths are clamped to [0, max_len] on the device.
 * max_len <= S_cap is a host-side upper bound of the lengths, and one head's
 * max_len keys must span less than 2 GiB (max_len * D * 2 < 2^31), else
 * ATTN_ERR_SHAPE.
 * rope_theta > 0: q is taken unrotated and each sequence's query is rotated
 * on the fly at position seqlens[b] - 1 (bit for bit what attn_rope with
 * pos_offset = seqlens, pos_shift = -1 produces); rope_theta == 0: q is used
 * as given (already rotated).  The cache holds keys already rotated.
 * workspace: device buffer of at least attn_decode_workspace_size(...) bytes,
 * 16-byte aligned; its contents on entry do not matter (each call tags the
 * partial results it writes with a host sequence number mixed with a per-group
 * epoch kept in the workspace and advanced on the device, so the tags also
 * differ between replays of one call captured in a HIP graph), and it must
 * not be shared by calls that may overlap.  The call enqueues no memset or
 * copy, so it may be captured in a graph.  scale > 0 and finite.
 * dtype BF16: one kernel is enqueued: its workgroups read the lengths and
 * split the batch's keys into nearly equal parts (a sequence's keys go to one
 * or more workgroups), and one that finds all partial results of its
 * (sequence, KV head) written merges them.
 * dtype F32: the accuracy path, fp32 throughout (within 1e-5 of the exact
 * result), not a performance path: two kernels, one writing the partial
 * result of every 512-key chunk into the same workspace, one merging them.
 * Groups with (Hq / Hkv) * D > 4096 return ATTN_ERR_UNSUPPORTED on this path.
 */
int attn_decode(void *o, const void *q, const void *k_cache, const void *v_cache, int dtype,
                int B, int Hq, int Hkv, int S_cap, int D, const int32_t *seqlens,
                int max_len, float scale, double rope_theta, void *workspace,
                size_t workspace_bytes, void *stream);

/*
 * attn_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments, results and errors are those of
 * attn_decode with dtype BF16 (F32 returns ATTN_ERR_UNSUPPORTED); the split
 * pass's partial results live instead in a static
 * array of ATTN_DECODE_SCRATCH_BYTES (16 MiB) that every device the library
 * runs on holds until the process ends.  The call allocates and frees nothing.
 * The problem must fit that array: attn_decode_workspace_size(B, Hq, Hkv,
 * max_len, D) <= ATTN_DECODE_SCRATCH_BYTES (both decode workloads of 32 x 8192
 * and 1 x 131072 tokens at D = 128 need about 8.5 MB), else ATTN_ERR_SCRATCH
 * with nothing enqueued.  All calls on one device share its array and find
 * the previous call's contents there, which, as for attn_decode, do not matter
 * (nothing needs to start at zero); calls that may overlap on one device (on
 * concurrent streams) race on it and must not be issued.  The first call on a
 * device looks up the array's device address (hipGetSymbolAddress, with that
 * device current), so make it outside graph capture.  The stream's device
 * (the current device for the null stream) selects the array.
 */
int attn_decode_noalloc(void *o, const void *q, const void *k_cache, const void *v_cache,
                        int dtype, int B, int Hq, int Hkv, int S_cap, int D,
                        const int32_t *seqlens, int max_len, float scale, double rope_theta,
                        void *stream);

/*
 * Decode over a paged KV cache, optionally limited to a sliding window.
 * "Grouped Query Attention (GQA)" glossary, section "GQA y técnicas
 * relacionadas": PagedAttention keeps the cache in fixed-size blocks, whatever
 * the number of heads, and sliding-window attention bounds the cached tokens
 * each query sees (Mistral 7B pairs it with GQA).
 *
 *   q, o: [B, Hq, D];  k_pages, v_pages: [num_pages, Hkv, page_size, D];
 *   block_table: device int32 [B, max_pages];  seqlens: device int32 [B].
 *   Token t of sequence b is row t % page_size of page
 *   block_table[b * max_pages + t / page_size].
 *   window > 0: the query of sequence b sees tokens max(0, len_b - window) ..
 *   len_b - 1;  window <= 0: all len_b tokens.
 *   o[b,h,:] = sum_{t seen} softmax_t(scale * <q[b,h,:], k_t>) v_t, with
 *   k_t, v_t the rows of head h / G.
 *
 * page_size: a positive multiple of 32.  0 <= seqlens[b] <= max_len <=
 * max_pages * page_size (lengths are clamped to [0, max_len] on the device),
 * and max_len * D * 2 < 2^31 as for attn_decode.
 * Table entries of the pages a query sees must lie in [0, num_pages); the
 * kernel clamps any other entry it reads into that range, so no read leaves
 * the page pool (the result is then unspecified).  Pages and rows that no
 * query sees are never read into a result.  A sequence that sees no token gets
 * a zero row.  rope_theta, scale, dtype (BF16 only) and the workspace are as
 * for attn_decode, with the same attn_decode_workspace_size(B, Hq, Hkv,
 * max_len, D).  One kernel is enqueued.
 */
int attn_decode_paged(void *o, const void *q, const void *k_pages, const void *v_pages,
                      int dtype, int B, int Hq, int Hkv, int page_size, int D, int num_pages,
                      const int32_t *block_table, int max_pages, const int32_t *seqlens,
                      int max_len, int window, float scale, double rope_theta,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * CCA pre-attention operations on the compressed q~, k~, v~ ("Compressed
 * Convolutional Attention" summary, "Methodologie", items 2 to 4; the summary
 * names the operations but not their sizes or exact form, so each is taken in
 * its plainest form):
 *   sequence mixing, a causal depthwise convolution of width W per channel:
 *     s[t,c] = sum_{i<W, t-i>=0} conv[h,i,c] x~[t-i,c]   (tap i: i tokens back)
 *   channel mixing within a head, a dense D x D map (row c = output channel c):
 *     z[t,c] = sum_c' mix[h,c,c'] s[t,c']
 *   QK-mean, the mean of the token's pre-convolution query (the group's query
 *   heads averaged) and key, added to every convolved q head of the KV group
 *   and to its k head:
 *     m[t,j] = ((1/G) sum_{h in group j} q~[t,h] + k~[t,j]) / 2
 *     q[t,h] = z_q[t,h] + m[t,h/G],   k[t,j] = z_k[t,j] + m[t,j]
 *   RoPE (item 4) of q and k at absolute position pos_offset[b] + t when
 *   rope_theta > 0 (the rotation of attn_rope; rope_theta == 0: none);
 *   value shift (item 3): v[t,c] = v~[t,c] for c < D/2, v~[t-1,c] for
 *   c >= D/2 (zero at t = 0).
 * q~, q_out: [B, Hq, S, D];  k~, v~, k_out, v_out: [B, Hkv, S, D];  conv_q
 * [Hq, W, D], conv_k [Hkv, W, D] (tap-major), mix_q [Hq, D, D], mix_k
 * [Hkv, D, D]; all
 * bf16 (dtype BF16 only), W = conv_width in 1..8, pos_offset device int32[B]
 * or NULL.  The outputs feed attn_prefill (rope_theta 0 there: q and k are
 * already rotated) and, as a cache, attn_decode.  The convolution and the
 * channel mix are evaluated in fp32 (the mix on the matrix cores, with the
 * convolution's output split into two bf16 parts) and each output is rounded
 * once to bf16.  Outputs must not overlap inputs.  Tensors are 16-byte
 * aligned; one head's rows must span less than 2 GiB ((S + 64) D 2 < 2^31),
 * else ATTN_ERR_SHAPE.  One kernel is enqueued.
 */
int attn_cca_mix(void *q_out, void *k_out, void *v_out, const void *q, const void *k,
                 const void *v, int dtype, int B, int Hq, int Hkv, int S, int D,
                 const void *conv_q, const void *conv_k, int conv_width, const void *mix_q,
                 const void *mix_k, const int32_t *pos_offset, double rope_theta, void *stream);

/*
 * The CCA pre-attention operations of attn_cca_mix for one new token per
 * sequence, as a decode step needs them ("Compressed Convolutional Attention"
 * summary, "Methodologie", items 2 to 4, in the same readings).  Token t[b]
 * (its index in sequence b, >= 0; a negative value, a caller error, is taken
 * as 0 on the device; RoPE position pos_offset[b] + t[b]) is
 * mixed with the tokens before it that the width-W convolution reaches,
 * which the caller keeps as state between steps:
 *   q_state [B, Hq, W-1, D], k_state [B, Hkv, W-1, D]: the pre-convolution
 *     q~ and k~ rows of the previous W - 1 tokens, token u in ring slot
 *     u mod (W - 1) (unused, and may be NULL, when W == 1);
 *   v_state [B, Hkv, D]: the previous token's v~ row.
 * State rows of tokens before the first (u < 0) are never read, so a new
 * sequence needs no initialisation; after a prefill of tokens 0 .. t - 1
 * through attn_cca_mix, the caller copies their last W - 1 q~ and k~ rows
 * into the rings and v~[t - 1] into v_state.  The call reads the state, then
 * writes token t's rows into it (q~[t], k~[t] into slot t mod (W - 1), v~[t]
 * into v_state), ready for token t + 1.
 * q~, q_out: [B, Hq, D];  k~, v~, k_out, v_out: [B, Hkv, D]; conv, mix,
 * conv_width and rope_theta as for attn_cca_mix; t and pos_offset device
 * int32[B] (pos_offset may be NULL).  Outputs equal row t of attn_cca_mix
 * over the sequence up to rounding: the convolution and the channel mix are
 * evaluated in fp32 (plain fp32 arithmetic here) and each output is rounded
 * once to bf16.  Outputs, inputs and state must not overlap.  bf16 only;
 * groups of more than (65536 / (4 D) - 2) query heads per KV head return
 * ATTN_ERR_UNSUPPORTED.  Tensors are 16-byte aligned.  One kernel is
 * enqueued.
 */
int attn_cca_mix_decode(void *q_out, void *k_out, void *v_out, const void *q, const void *k,
                        const void *v, int dtype, int B, int Hq, int Hkv, int D,
                        const void *conv_q, const void *conv_k, int conv_width, const void *mix_q,
                        const void *mix_k, void *q_state, void *k_state, void *v_state,
                        const int32_t *t, const int32_t *pos_offset, double rope_theta,
                        void *stream);

/*
 * Bytes of device workspace attn_cca_mix_backward needs (0 on invalid sizes):
 * the mean's fp32 gradient [B, Hkv, S, D], the rotation's fp32 (cos, sin) per
 * (sequence, token, channel pair), and fp32 partial weight gradients per
 * (sequence, 256-token chunk, head).
 */
size_t attn_cca_mix_backward_workspace_size(int B, int Hq, int Hkv, int S, int D, int conv_width);

/*
 * Backward pass of attn_cca_mix ("Compressed Convolutional Attention"
 * summary, "Resultaten" 2 reports a backward pass for CCA; the formulas are
 * the chain rule through the operations of "Methodologie" items 2 to 4, taken
 * in reverse order).  Given gq, gk, gv, the gradients of a loss with respect
 * to attn_cca_mix's outputs q, k (as rotated) and v, and the latent q~, k~ and
 * weights of that call, it returns the gradients with respect to q~, k~, v~
 * and the weights:
 *   a = R_t^T g (the transposed rotation at pos_offset[b] + t; a = g when
 *     rope_theta == 0);  dm[t,j] = sum_{h in group j} a_q[t,h] + a_k[t,j];
 *   ds[t] = M^T a[t];  dq~[t,h] = sum_{i < W, t+i < S} w_i (.) ds[t+i] + dm[t,j]/(2G),
 *     dk~[t,j] likewise with dm[t,j]/2;
 *   dmix[h] = sum_{b,t} a[t] s[t]^T (s the forward's convolution output);
 *   dconv[h,i] = sum_{b, t >= i} ds[t] (.) x~[t-i];
 *   dv~[t,c] = gv[t,c] for c < D/2, gv[t+1,c] for c >= D/2 (0 at t = S-1).
 * gq, dq: [B, Hq, S, D];  gk, gv, k~, dk, dv: [B, Hkv, S, D], bf16;  dconv_q
 * [Hq, W, D], dconv_k [Hkv, W, D], dmix_q [Hq, D, D], dmix_k [Hkv, D, D]:
 * fp32 device arrays (4-byte aligned), written (not accumulated into); with
 * B == 0 or S == 0 they are set to zero and nothing else is touched.  Other
 * arguments as for attn_cca_mix (W in 1..8).  Arithmetic is fp32; dq, dk, dv
 * are rounded once to bf16.  workspace: at least
 * attn_cca_mix_backward_workspace_size(B, Hq, Hkv, S, D, conv_width) bytes,
 * 16-byte aligned, contents on entry irrelevant, not shared by calls that may
 * overlap (ATTN_ERR_WORKSPACE otherwise).  Outputs must not overlap inputs.
 * Three kernels are enqueued (the mean's gradient and dv, the per-head pass,
 * the reduction of the weight gradients).
 */
int attn_cca_mix_backward(void *dq, void *dk, void *dv, float *dconv_q, float *dconv_k,
                          float *dmix_q, float *dmix_k, const void *gq, const void *gk,
                          const void *gv, const void *q, const void *k, int dtype, int B, int Hq,
                          int Hkv, int S, int D, const void *conv_q, const void *conv_k,
                          int conv_width, const void *mix_q, const void *mix_k,
                          const int32_t *pos_offset, double rope_theta, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
