"""MI355X-native causal grouped-query attention with RoPE.

Thin Python binding over the C ABI of ``libattn.so`` (``include/attn.h``):
argument marshalling only.  Every step runs in the library's gfx950 kernels;
PyTorch supplies device memory and the current stream.  There is no CPU
fallback: calling into the library without the built ``libattn.so`` raises.

    rope(x, theta, pos_offset=None, pos_shift=0, out=None)
    rope_backward(dy, theta, pos_offset=None, pos_shift=0, out=None)
    prefill(q, k, v, scale=None, out=None, rope_theta=0.0)
    prefill_lse(q, k, v, scale=None, out=None, lse=None, rope_theta=0.0)
    prefill_backward(q, k, v, o, dout, lse, scale=None, dq=None, dk=None, dv=None, workspace=None)
    prefill_backward_workspace_size(B, Hq, Hkv, S, D)
    decode(q, k_cache, v_cache, seqlens, max_len=None, scale=None, rope_theta=0.0, out=None,
           workspace=None)
    decode_noalloc(q, k_cache, v_cache, seqlens, out, max_len=None, scale=None, rope_theta=0.0)
    decode_workspace_size(B, Hq, Hkv, max_len, D)
    cca_mix(q, k, v, conv_q, conv_k, mix_q, mix_k, rope_theta=0.0, pos_offset=None,
            q_out=None, k_out=None, v_out=None)
    cca_mix_backward(gq, gk, gv, q, k, conv_q, conv_k, mix_q, mix_k, rope_theta=0.0,
                     pos_offset=None, workspace=None)
    cca_mix_backward_workspace_size(B, Hq, Hkv, S, D, W)
    cca_mix_decode(q, k, v, conv_q, conv_k, mix_q, mix_k, t, q_state, k_state, v_state,
                   rope_theta=0.0, pos_offset=None, q_out=None, k_out=None, v_out=None)

Shapes follow the C ABI: x [B,H,S,D]; q/o [B,Hq,S,D], k/v [B,Hkv,S,D];
decode q/o [B,Hq,D], caches [B,Hkv,S_cap,D], seqlens int32 [B] on the device.
"""
from __future__ import annotations

import math

from ._lib import (  # noqa: F401
    AttnError, lib, lib_path, DTYPE_CODES, STATUS, DECODE_SCRATCH_BYTES,
)

__all__ = ["rope", "rope_backward", "prefill", "prefill_lse", "prefill_backward", "prefill_backward_workspace_size",
           "decode", "decode_noalloc", "decode_paged", "decode_workspace_size", "AttnError",
           "lib_path", "DECODE_SCRATCH_BYTES", "cca_mix", "cca_mix_decode", "cca_mix_backward",
           "cca_mix_backward_workspace_size"]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    try:
        return DTYPE_CODES[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}; use float32 or bfloat16") from None


def _check_dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _call(fn, *args):
    rc = fn(*args)
    if rc != 0:
        raise AttnError(rc)


def rope(x, theta: float, pos_offset=None, pos_shift: int = 0, out=None):
    """Rotary embedding of x [B,H,S,D]: token s of sequence b is at position
    pos_offset[b] + pos_shift + s.  out may be x itself (in place)."""
    torch = _torch()
    if x.dim() != 4:
        raise ValueError("x must be [B, H, S, D]")
    B, H, S, D = x.shape
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x")
    _check_dev(x, out)
    po = 0
    if pos_offset is not None:
        if pos_offset.dtype != torch.int32 or pos_offset.shape != (B,):
            raise ValueError("pos_offset must be int32 [B]")
        _check_dev(pos_offset)
        po = pos_offset.data_ptr()
    _call(lib().attn_rope, out.data_ptr(), x.data_ptr(), _dtype_code(x), B, H, S, D, po,
          int(pos_shift), float(theta), _stream(x))
    return out


def rope_backward(dy, theta: float, pos_offset=None, pos_shift: int = 0, out=None):
    """Transpose of rope(): carries a gradient of the rotated tensor back to the
    unrotated one (same positions and theta).  out may be dy itself."""
    torch = _torch()
    if dy.dim() != 4:
        raise ValueError("dy must be [B, H, S, D]")
    B, H, S, D = dy.shape
    if out is None:
        out = torch.empty_like(dy)
    if out.shape != dy.shape or out.dtype != dy.dtype:
        raise ValueError("out must match dy")
    _check_dev(dy, out)
    po = 0
    if pos_offset is not None:
        if pos_offset.dtype != torch.int32 or pos_offset.shape != (B,):
            raise ValueError("pos_offset must be int32 [B]")
        _check_dev(pos_offset)
        po = pos_offset.data_ptr()
    _call(lib().attn_rope_backward, out.data_ptr(), dy.data_ptr(), _dtype_code(dy), B, H, S, D, po,
          int(pos_shift), float(theta), _stream(dy))
    return out


def prefill(q, k, v, scale: float | None = None, out=None, rope_theta: float = 0.0):
    """Causal GQA attention: q [B,Hq,S,D], k/v [B,Hkv,S,D] -> [B,Hq,S,D].

    rope_theta > 0 rotates query i at position i inside the kernel (k must
    already be rotated); 0 takes q as already rotated."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,Hq,S,D] and k, v [B,Hkv,S,D]")
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[2] != S or k.shape[3] != D:
        raise ValueError("k/v must be [B,Hkv,S,D] with q's B, S and D")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _check_dev(q, k, v, out)
    _call(lib().attn_prefill, out.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
          _dtype_code(q), B, Hq, Hkv, S, D, float(scale), float(rope_theta), _stream(q))
    return out


def _check_prefill_shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,Hq,S,D] and k, v [B,Hkv,S,D]")
    B, Hq, S, D = q.shape
    if k.shape[0] != B or k.shape[2] != S or k.shape[3] != D:
        raise ValueError("k/v must be [B,Hkv,S,D] with q's B, S and D")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    return B, Hq, k.shape[1], S, D


def prefill_lse(q, k, v, scale: float | None = None, out=None, lse=None, rope_theta: float = 0.0):
    """prefill() that also returns each row's log-normaliser (bf16 only):
    (o [B,Hq,S,D], lse float32 [B,Hq,S]), lse = log sum_t exp(scale <q_i, k_t>)."""
    torch = _torch()
    B, Hq, Hkv, S, D = _check_prefill_shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, Hq, S, dtype=torch.float32, device=q.device)
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, S):
        raise ValueError("lse must be float32 [B, Hq, S]")
    _check_dev(q, k, v, out, lse)
    _call(lib().attn_prefill_lse, out.data_ptr(), lse.data_ptr(), q.data_ptr(), k.data_ptr(),
          v.data_ptr(), _dtype_code(q), B, Hq, Hkv, S, D, float(scale), float(rope_theta),
          _stream(q))
    return out, lse


def prefill_backward_workspace_size(B: int, Hq: int, Hkv: int, S: int, D: int) -> int:
    return int(lib().attn_prefill_backward_workspace_size(B, Hq, Hkv, S, D))


def prefill_backward(q, k, v, o, dout, lse, scale: float | None = None, dq=None, dk=None, dv=None,
                     workspace=None):
    """Gradients (dq, dk, dv) of sum <dout, o> for o = prefill(q, k, v) (bf16).

    q, k as the forward attended with them (already rotated); o and lse from
    prefill_lse; dout like o."""
    torch = _torch()
    B, Hq, Hkv, S, D = _check_prefill_shapes(q, k, v)
    if o.shape != q.shape or dout.shape != q.shape or o.dtype != q.dtype or dout.dtype != q.dtype:
        raise ValueError("o and dout must match q")
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, S):
        raise ValueError("lse must be float32 [B, Hq, S]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("dq, dk, dv must match q, k, v")
    if workspace is None:
        workspace = torch.empty(max(1, prefill_backward_workspace_size(B, Hq, Hkv, S, D)),
                                dtype=torch.uint8, device=q.device)
    _check_dev(q, k, v, o, dout, lse, dq, dk, dv, workspace)
    _call(lib().attn_prefill_backward, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), q.data_ptr(),
          k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
          _dtype_code(q), B, Hq, Hkv, S, D, float(scale), workspace.data_ptr(),
          workspace.numel() * workspace.element_size(), _stream(q))
    return dq, dk, dv


def decode_workspace_size(B: int, Hq: int, Hkv: int, max_len: int, D: int) -> int:
    return int(lib().attn_decode_workspace_size(B, Hq, Hkv, max_len, D))


def decode(q, k_cache, v_cache, seqlens, max_len: int | None = None, scale: float | None = None,
           rope_theta: float = 0.0, out=None, workspace=None):
    """One query token per sequence over a contiguous cache.

    q [B,Hq,D]; caches [B,Hkv,S_cap,D]; seqlens device int32 [B] with
    0 <= seqlens[b] <= max_len <= S_cap (max_len defaults to S_cap, which needs
    no host synchronisation).  rope_theta > 0 rotates q at position
    seqlens[b] - 1 inside the kernel; 0 takes q as already rotated.
    Returns [B,Hq,D]."""
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B,Hq,D] and caches [B,Hkv,S_cap,D]")
    B, Hq, D = q.shape
    _, Hkv, S_cap, _ = k_cache.shape
    if k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("caches must be [B,Hkv,S_cap,D] with q's B and D")
    if seqlens.dtype != torch.int32 or seqlens.shape != (B,):
        raise ValueError("seqlens must be int32 [B]")
    if max_len is None:
        max_len = S_cap
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    need = decode_workspace_size(B, Hq, Hkv, max_len, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_dev(q, k_cache, v_cache, seqlens, out, workspace)
    _call(lib().attn_decode, out.data_ptr(), q.data_ptr(), k_cache.data_ptr(),
          v_cache.data_ptr(), _dtype_code(q), B, Hq, Hkv, S_cap, D, seqlens.data_ptr(),
          int(max_len), float(scale), float(rope_theta), workspace.data_ptr(),
          workspace.numel() * workspace.element_size(), _stream(q))
    return out


def decode_noalloc(q, k_cache, v_cache, seqlens, out, max_len: int | None = None,
                   scale: float | None = None, rope_theta: float = 0.0):
    """decode() through the allocation-free entry point: no workspace, the
    library's static per-device scratch instead (problems whose
    decode_workspace_size exceeds DECODE_SCRATCH_BYTES are rejected).  The
    caller passes the output buffer out [B,Hq,D]; nothing is allocated."""
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B,Hq,D] and caches [B,Hkv,S_cap,D]")
    B, Hq, D = q.shape
    _, Hkv, S_cap, _ = k_cache.shape
    if k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("caches must be [B,Hkv,S_cap,D] with q's B and D")
    if seqlens.dtype != torch.int32 or seqlens.shape != (B,):
        raise ValueError("seqlens must be int32 [B]")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if max_len is None:
        max_len = S_cap
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check_dev(q, k_cache, v_cache, seqlens, out)
    _call(lib().attn_decode_noalloc, out.data_ptr(), q.data_ptr(), k_cache.data_ptr(),
          v_cache.data_ptr(), _dtype_code(q), B, Hq, Hkv, S_cap, D, seqlens.data_ptr(),
          int(max_len), float(scale), float(rope_theta), _stream(q))
    return out


def decode_paged(q, k_pages, v_pages, block_table, seqlens, max_len: int | None = None,
                 window: int = 0, scale: float | None = None, rope_theta: float = 0.0,
                 out=None, workspace=None):
    """One query token per sequence over a paged cache.

    q [B,Hq,D]; pages [num_pages,Hkv,page_size,D] (page_size a multiple of
    32); block_table device int32 [B,max_pages]: token t of sequence b is row
    t % page_size of page block_table[b, t // page_size]; seqlens device int32
    [B] with 0 <= seqlens[b] <= max_len <= max_pages*page_size (max_len
    defaults to that product).  window > 0 limits each query to its
    sequence's last `window` tokens.  rope_theta as for decode.
    Returns [B,Hq,D]."""
    torch = _torch()
    if q.dim() != 3 or k_pages.dim() != 4 or v_pages.shape != k_pages.shape:
        raise ValueError("q must be [B,Hq,D] and pages [num_pages,Hkv,page_size,D]")
    B, Hq, D = q.shape
    num_pages, Hkv, page_size, _ = k_pages.shape
    if k_pages.shape[3] != D:
        raise ValueError("pages must have q's head dim")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages]")
    if seqlens.dtype != torch.int32 or seqlens.shape != (B,):
        raise ValueError("seqlens must be int32 [B]")
    max_pages = block_table.shape[1]
    if max_len is None:
        max_len = max_pages * page_size
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    need = decode_workspace_size(B, Hq, Hkv, max_len, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    block_table = block_table.contiguous()
    _check_dev(q, k_pages, v_pages, block_table, seqlens, out, workspace)
    _call(lib().attn_decode_paged, out.data_ptr(), q.data_ptr(), k_pages.data_ptr(),
          v_pages.data_ptr(), _dtype_code(q), B, Hq, Hkv, page_size, D, num_pages,
          block_table.data_ptr(), max_pages, seqlens.data_ptr(), int(max_len), int(window),
          float(scale), float(rope_theta), workspace.data_ptr(),
          workspace.numel() * workspace.element_size(), _stream(q))
    return out


def cca_mix(q, k, v, conv_q, conv_k, mix_q, mix_k, rope_theta: float = 0.0, pos_offset=None,
            q_out=None, k_out=None, v_out=None):
    """CCA pre-attention operations on the compressed q [B,Hq,S,D], k, v
    [B,Hkv,S,D] (bf16): causal depthwise sequence convolution (conv_q [Hq,W,D],
    conv_k [Hkv,W,D]; tap i weighs the token i steps back), channel mix per
    head (mix_q [Hq,D,D], mix_k [Hkv,D,D]; row c = output channel c), plus the
    group's pre-convolution query/key mean; RoPE at position pos_offset[b] + t
    when rope_theta > 0; value shift (last D/2 channels from the previous
    token).  Returns (q_out, k_out, v_out), ready for prefill(..., rope_theta=0)."""
    torch = _torch()
    B, Hq, Hkv, S, D = _check_prefill_shapes(q, k, v)
    W = conv_q.shape[1] if conv_q.dim() == 3 else -1
    if (conv_q.shape != (Hq, W, D) or conv_k.shape != (Hkv, W, D) or mix_q.shape != (Hq, D, D)
            or mix_k.shape != (Hkv, D, D)):
        raise ValueError("conv_q [Hq,W,D], conv_k [Hkv,W,D], mix_q [Hq,D,D], mix_k [Hkv,D,D]")
    if any(t.dtype != q.dtype for t in (conv_q, conv_k, mix_q, mix_k)):
        raise ValueError("weights must share the activations' dtype")
    q_out = torch.empty_like(q) if q_out is None else q_out
    k_out = torch.empty_like(k) if k_out is None else k_out
    v_out = torch.empty_like(v) if v_out is None else v_out
    if q_out.shape != q.shape or k_out.shape != k.shape or v_out.shape != v.shape:
        raise ValueError("outputs must match q, k, v")
    po = 0
    if pos_offset is not None:
        if pos_offset.dtype != torch.int32 or pos_offset.shape != (B,):
            raise ValueError("pos_offset must be int32 [B]")
        _check_dev(pos_offset)
        po = pos_offset.data_ptr()
    _check_dev(q, k, v, conv_q, conv_k, mix_q, mix_k, q_out, k_out, v_out)
    _call(lib().attn_cca_mix, q_out.data_ptr(), k_out.data_ptr(), v_out.data_ptr(), q.data_ptr(),
          k.data_ptr(), v.data_ptr(), _dtype_code(q), B, Hq, Hkv, S, D, conv_q.data_ptr(),
          conv_k.data_ptr(), W, mix_q.data_ptr(), mix_k.data_ptr(), po, float(rope_theta),
          _stream(q))
    return q_out, k_out, v_out


def cca_mix_backward_workspace_size(B: int, Hq: int, Hkv: int, S: int, D: int, W: int) -> int:
    return int(lib().attn_cca_mix_backward_workspace_size(B, Hq, Hkv, S, D, W))


def cca_mix_backward(gq, gk, gv, q, k, conv_q, conv_k, mix_q, mix_k, rope_theta: float = 0.0,
                     pos_offset=None, workspace=None):
    """Gradients of cca_mix: given gq [B,Hq,S,D], gk, gv [B,Hkv,S,D] (bf16), the
    gradients with respect to cca_mix's outputs (q and k as rotated), and the
    latent q, k and the weights of that call, returns (dq, dk, dv) (bf16, like
    the latent inputs) and (dconv_q, dconv_k, dmix_q, dmix_k) (fp32, like the
    weights' shapes), the weight gradients summed over the batch and tokens."""
    torch = _torch()
    B, Hq, Hkv, S, D = _check_prefill_shapes(q, k, k)
    W = conv_q.shape[1] if conv_q.dim() == 3 else -1
    if (conv_q.shape != (Hq, W, D) or conv_k.shape != (Hkv, W, D) or mix_q.shape != (Hq, D, D)
            or mix_k.shape != (Hkv, D, D)):
        raise ValueError("conv_q [Hq,W,D], conv_k [Hkv,W,D], mix_q [Hq,D,D], mix_k [Hkv,D,D]")
    if gq.shape != q.shape or gk.shape != k.shape or gv.shape != k.shape:
        raise ValueError("gq like q, gk and gv like k")
    if any(t.dtype != q.dtype for t in (gq, gk, gv, k, conv_q, conv_k, mix_q, mix_k)):
        raise ValueError("all tensors share one dtype")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
    f32 = dict(dtype=torch.float32, device=q.device)
    dcq, dck = torch.empty((Hq, W, D), **f32), torch.empty((Hkv, W, D), **f32)
    dmq, dmk = torch.empty((Hq, D, D), **f32), torch.empty((Hkv, D, D), **f32)
    po = 0
    if pos_offset is not None:
        if pos_offset.dtype != torch.int32 or pos_offset.shape != (B,):
            raise ValueError("pos_offset must be int32 [B]")
        _check_dev(pos_offset)
        po = pos_offset.data_ptr()
    if workspace is None:
        workspace = torch.empty(max(1, cca_mix_backward_workspace_size(B, Hq, Hkv, S, D, W)),
                                dtype=torch.uint8, device=q.device)
    _check_dev(gq, gk, gv, q, k, conv_q, conv_k, mix_q, mix_k, workspace)
    _call(lib().attn_cca_mix_backward, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
          dcq.data_ptr(), dck.data_ptr(), dmq.data_ptr(), dmk.data_ptr(), gq.data_ptr(),
          gk.data_ptr(), gv.data_ptr(), q.data_ptr(), k.data_ptr(), _dtype_code(q), B, Hq, Hkv, S,
          D, conv_q.data_ptr(), conv_k.data_ptr(), W, mix_q.data_ptr(), mix_k.data_ptr(), po,
          float(rope_theta), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
          _stream(q))
    return (dq, dk, dv), (dcq, dck, dmq, dmk)


def cca_mix_decode(q, k, v, conv_q, conv_k, mix_q, mix_k, t, q_state, k_state, v_state,
                   rope_theta: float = 0.0, pos_offset=None, q_out=None, k_out=None, v_out=None):
    """cca_mix for one new token per sequence (decode): q [B,Hq,D], k, v [B,Hkv,D]
    (bf16) of token t[b] (int32 [B]), with the convolution's reach as state:
    q_state [B,Hq,W-1,D] and k_state [B,Hkv,W-1,D] rings (token u in slot
    u mod (W-1)), v_state [B,Hkv,D] (the previous token's v).  The state is read,
    then updated in place with this token's rows.  Returns (q_out, k_out, v_out),
    row t of cca_mix over the sequence."""
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("q [B,Hq,D], k and v [B,Hkv,D]")
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[2] != D:
        raise ValueError("q [B,Hq,D], k and v [B,Hkv,D]")
    W = conv_q.shape[1] if conv_q.dim() == 3 else -1
    if (conv_q.shape != (Hq, W, D) or conv_k.shape != (Hkv, W, D) or mix_q.shape != (Hq, D, D)
            or mix_k.shape != (Hkv, D, D)):
        raise ValueError("conv_q [Hq,W,D], conv_k [Hkv,W,D], mix_q [Hq,D,D], mix_k [Hkv,D,D]")
    if any(x.dtype != q.dtype for x in (k, v, conv_q, conv_k, mix_q, mix_k, v_state)):
        raise ValueError("all tensors share one dtype")
    if v_state.shape != (B, Hkv, D):
        raise ValueError("v_state [B,Hkv,D]")
    qs = ks = 0
    if W > 1:
        if q_state.shape != (B, Hq, W - 1, D) or k_state.shape != (B, Hkv, W - 1, D):
            raise ValueError("q_state [B,Hq,W-1,D], k_state [B,Hkv,W-1,D]")
        if q_state.dtype != q.dtype or k_state.dtype != q.dtype:
            raise ValueError("all tensors share one dtype")
        _check_dev(q_state, k_state)
        qs, ks = q_state.data_ptr(), k_state.data_ptr()
    if t.dtype != torch.int32 or t.shape != (B,):
        raise ValueError("t must be int32 [B]")
    po = 0
    if pos_offset is not None:
        if pos_offset.dtype != torch.int32 or pos_offset.shape != (B,):
            raise ValueError("pos_offset must be int32 [B]")
        _check_dev(pos_offset)
        po = pos_offset.data_ptr()
    q_out = torch.empty_like(q) if q_out is None else q_out
    k_out = torch.empty_like(k) if k_out is None else k_out
    v_out = torch.empty_like(v) if v_out is None else v_out
    if q_out.shape != q.shape or k_out.shape != k.shape or v_out.shape != v.shape:
        raise ValueError("outputs must match q, k, v")
    _check_dev(q, k, v, conv_q, conv_k, mix_q, mix_k, v_state, t, q_out, k_out, v_out)
    _call(lib().attn_cca_mix_decode, q_out.data_ptr(), k_out.data_ptr(), v_out.data_ptr(),
          q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), B, Hq, Hkv, D,
          conv_q.data_ptr(), conv_k.data_ptr(), W, mix_q.data_ptr(), mix_k.data_ptr(), qs, ks,
          v_state.data_ptr(), t.data_ptr(), po, float(rope_theta), _stream(q))
    return q_out, k_out, v_out
