"""Plain fp64 CPU oracle for causal grouped-query attention with RoPE.

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use this package; the library under test
(``compressed_latent_causal_amd``) never imports it, and this package imports
nothing from the library.  The arithmetic lives in ``oracle.c`` (plain C, double
precision, computed row by row from the definition); this module only marshals
numpy arrays into it.

Inputs are numpy arrays: float64, float32, or uint16 holding raw bf16 bit
patterns (pass ``dtype="bf16"``).  Outputs are float64 arrays.

Pages cited (by title and section):
  * "Grouped Query Attention (GQA)" glossary, "Cómo funciona GQA": GQA is
    unchanged scaled dot-product attention per query head, with consecutive
    query heads sharing one key/value head; the example is causal.
  * same page, "Por qué GQA reduce la caché KV": the cache stores keys and
    values of every earlier token and is read in full per generated token; its
    size grows with the number of key/value heads.
  * "Compressed Convolutional Attention" summary, "Methodologie" item 4: RoPE is
    applied to q and k inside the attention space itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_DT_CODE = {"f64": 0, "f32": 1, "bf16": 2}


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (IEEE semantics, no FMA
    contraction, OpenMP over output rows)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = [
            "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
            "-fopenmp", "-shared", "-fPIC", "-Wall", _SRC, "-o", tmp, "-lm",
        ]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # ORACLE_LIB points the pins at a deliberately broken build of
            # oracle.c (the mutation test); normally the library is built here.
            path = os.environ.get("ORACLE_LIB") or build()
            lib = ctypes.CDLL(path)
            P = ctypes.c_void_p
            i = ctypes.c_int
            lib.oracle_rope.argtypes = [P, P, i, i, i, i, i, P, ctypes.c_double]
            lib.oracle_rope.restype = None
            lib.oracle_rope_transpose.argtypes = [P, P, i, i, i, i, i, P, ctypes.c_double]
            lib.oracle_rope_transpose.restype = None
            lib.oracle_prefill.argtypes = [P, P, P, P, i, i, i, i, i, i,
                                           ctypes.c_double, P, ctypes.c_int64]
            lib.oracle_prefill.restype = i
            lib.oracle_decode.argtypes = [P, P, P, P, i, i, i, i, i, i, P,
                                          ctypes.c_double]
            lib.oracle_decode.restype = i
            lib.oracle_decode_paged.argtypes = [P, P, P, P, i, i, i, i, i, i, i, P, i, P, i,
                                                ctypes.c_double]
            lib.oracle_decode_paged.restype = i
            lib.oracle_prefill_lse.argtypes = [P, P, P, i, i, i, i, i, i, ctypes.c_double, P,
                                               ctypes.c_int64]
            lib.oracle_prefill_lse.restype = i
            lib.oracle_prefill_backward.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, i,
                                                    ctypes.c_double, P, ctypes.c_int64, P,
                                                    ctypes.c_int64]
            lib.oracle_prefill_backward.restype = i
            lib.oracle_cca_mix.argtypes = [P, P, P, P, P, P, i, i, i, i, i, i, P, P, i, P, P, P,
                                           ctypes.c_double]
            lib.oracle_cca_mix.restype = i
            lib.oracle_cca_mix_backward.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, i, i, i, i,
                                                    i, i, P, P, i, P, P, P, ctypes.c_double]
            lib.oracle_cca_mix_backward.restype = i
            lib.oracle_round_bf16.argtypes = [P, P, ctypes.c_size_t]
            lib.oracle_round_bf16.restype = None
            lib.oracle_round_f32.argtypes = [P, P, ctypes.c_size_t]
            lib.oracle_round_f32.restype = None
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = i
            _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def _as_input(x: np.ndarray, dtype: str) -> np.ndarray:
    want = {"f64": np.float64, "f32": np.float32, "bf16": np.uint16}[dtype]
    x = np.ascontiguousarray(x)
    if x.dtype != want:
        raise TypeError(f"oracle input for dtype {dtype} must be {want}, got {x.dtype}")
    return x


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_of(x: np.ndarray) -> str:
    return {np.dtype(np.float64): "f64", np.dtype(np.float32): "f32",
            np.dtype(np.uint16): "bf16"}[x.dtype]


# ---------------------------------------------------------------------------
# rounding to storage types
# ---------------------------------------------------------------------------
def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_round_bf16(_ptr(out), _ptr(x), x.size)
    return out


def round_f32(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float32)
    _load().oracle_round_f32(_ptr(out), _ptr(x), x.size)
    return out


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the storage type `dtype` ("f32" or "bf16")."""
    if dtype == "f32":
        return round_f32(x)
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f64":
        return np.ascontiguousarray(x, dtype=np.float64)
    raise ValueError(dtype)


def widen(x: np.ndarray) -> np.ndarray:
    """Exact fp64 value of an f64/f32/bf16-bits array."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# ---------------------------------------------------------------------------
# RoPE, prefill, decode
# ---------------------------------------------------------------------------
def rope(x: np.ndarray, theta: float, pos_offset=None) -> np.ndarray:
    """Rotary embedding of x [B, H, S, D]; token s of sequence b at position
    pos_offset[b] + s.  Returns fp64 [B, H, S, D]."""
    dt = _dtype_of(x)
    x = _as_input(x, dt)
    B, H, S, D = x.shape
    if D % 2:
        raise ValueError("RoPE needs an even head dim")
    off = None
    if pos_offset is not None:
        off = np.ascontiguousarray(pos_offset, dtype=np.int32)
        if off.shape != (B,):
            raise ValueError("pos_offset must have shape [B]")
    out = np.empty(x.shape, dtype=np.float64)
    _load().oracle_rope(_ptr(out), _ptr(x), _DT_CODE[dt], B, H, S, D, _ptr(off),
                        float(theta))
    return out


def rope_transpose(dy: np.ndarray, theta: float, pos_offset=None) -> np.ndarray:
    """Transpose of the rotary embedding (the gradient map of rope): each pair
    of dy [B, H, S, D] turned back by its angle.  Returns fp64 [B, H, S, D]."""
    dt = _dtype_of(dy)
    dy = _as_input(dy, dt)
    B, H, S, D = dy.shape
    if D % 2:
        raise ValueError("RoPE needs an even head dim")
    off = None
    if pos_offset is not None:
        off = np.ascontiguousarray(pos_offset, dtype=np.int32)
        if off.shape != (B,):
            raise ValueError("pos_offset must have shape [B]")
    out = np.empty(dy.shape, dtype=np.float64)
    _load().oracle_rope_transpose(_ptr(out), _ptr(dy), _DT_CODE[dt], B, H, S, D, _ptr(off),
                                  float(theta))
    return out


def prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float | None = None,
            rows: np.ndarray | None = None) -> np.ndarray:
    """Causal GQA attention.  q [B,Hq,S,D], k/v [B,Hkv,S,D] of one dtype.
    rows=None: fp64 [B,Hq,S,D]; else rows are flat indices (b*Hq+h)*S+i and the
    result is fp64 [len(rows), D]."""
    dt = _dtype_of(q)
    q, k, v = (_as_input(t, dt) for t in (q, k, v))
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, S, D) or v.shape != k.shape or Hq % Hkv:
        raise ValueError("bad shapes")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if rows is None:
        out = np.empty((B, Hq, S, D), dtype=np.float64)
        r_ptr, n = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((rows.size, D), dtype=np.float64)
        r_ptr, n = _ptr(rows), rows.size
    rc = _load().oracle_prefill(_ptr(out), _ptr(q), _ptr(k), _ptr(v), _DT_CODE[dt], B,
                                Hq, Hkv, S, D, float(scale), r_ptr, n)
    if rc:
        raise RuntimeError(f"oracle_prefill failed ({rc})")
    return out


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, seqlens,
           scale: float | None = None) -> np.ndarray:
    """One new query token per sequence over a contiguous cache.
    q [B,Hq,D], caches [B,Hkv,S_cap,D], seqlens int [B].  Returns fp64 [B,Hq,D]."""
    dt = _dtype_of(q)
    q, k_cache, v_cache = (_as_input(t, dt) for t in (q, k_cache, v_cache))
    B, Hq, D = q.shape
    _, Hkv, S_cap, _ = k_cache.shape
    if k_cache.shape != (B, Hkv, S_cap, D) or v_cache.shape != k_cache.shape or Hq % Hkv:
        raise ValueError("bad shapes")
    lens = np.ascontiguousarray(seqlens, dtype=np.int32)
    if lens.shape != (B,) or (lens < 0).any() or (lens > S_cap).any():
        raise ValueError("seqlens must be [B] in [0, S_cap]")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, Hq, D), dtype=np.float64)
    rc = _load().oracle_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                               _DT_CODE[dt], B, Hq, Hkv, S_cap, D, _ptr(lens),
                               float(scale))
    if rc:
        raise RuntimeError(f"oracle_decode failed ({rc})")
    return out


def decode_paged(q: np.ndarray, k_pages: np.ndarray, v_pages: np.ndarray, block_table,
                 seqlens, window: int = 0, scale: float | None = None) -> np.ndarray:
    """One new query token per sequence over a paged cache ("GQA y técnicas
    relacionadas": PagedAttention, sliding-window attention).  q [B,Hq,D],
    pages [num_pages,Hkv,page_size,D], block_table int [B,max_pages] (token t
    of sequence b is row t % page_size of page block_table[b, t // page_size]),
    seqlens int [B]; window > 0 limits the query to the last `window` tokens.
    Returns fp64 [B,Hq,D]."""
    dt = _dtype_of(q)
    q, k_pages, v_pages = (_as_input(t, dt) for t in (q, k_pages, v_pages))
    B, Hq, D = q.shape
    num_pages, Hkv, page_size, _ = k_pages.shape
    if k_pages.shape != (num_pages, Hkv, page_size, D) or v_pages.shape != k_pages.shape or Hq % Hkv:
        raise ValueError("bad shapes")
    table = np.ascontiguousarray(block_table, dtype=np.int32)
    if table.ndim != 2 or table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    lens = np.ascontiguousarray(seqlens, dtype=np.int32)
    if lens.shape != (B,):
        raise ValueError("seqlens must be [B]")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, Hq, D), dtype=np.float64)
    rc = _load().oracle_decode_paged(_ptr(out), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                     _DT_CODE[dt], B, Hq, Hkv, page_size, D, num_pages,
                                     _ptr(table), table.shape[1], _ptr(lens), int(window),
                                     float(scale))
    if rc:
        raise RuntimeError(f"oracle_decode_paged failed ({rc})")
    return out


# ---------------------------------------------------------------------------
# KV-cache accounting ("Por qué GQA reduce la caché KV" and the worked example)
# ---------------------------------------------------------------------------
def kv_values_per_token(n_kv_heads: int, head_dim: int, n_layers: int = 1) -> int:
    """Cached scalars per token: one key and one value vector per KV head."""
    return n_layers * 2 * n_kv_heads * head_dim


def kv_cache_bytes(n_kv_heads: int, head_dim: int, n_tokens: int, n_layers: int = 1,
                   bytes_per_value: int = 2) -> int:
    return kv_values_per_token(n_kv_heads, head_dim, n_layers) * n_tokens * bytes_per_value


# ---------------------------------------------------------------------------
# training: log-normaliser and backward pass
# ---------------------------------------------------------------------------
def prefill_lse(q: np.ndarray, k: np.ndarray, scale: float | None = None,
                rows: np.ndarray | None = None) -> np.ndarray:
    """Log-normaliser of causal prefill rows, log sum_{t<=i} exp(scale <q_i, k_t>)
    (natural log).  rows=None: fp64 [B,Hq,S]; else fp64 [len(rows)] for flat
    row indices (b*Hq+h)*S+i."""
    dt = _dtype_of(q)
    q, k = (_as_input(t, dt) for t in (q, k))
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, S, D) or Hq % Hkv:
        raise ValueError("bad shapes")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if rows is None:
        out = np.empty((B, Hq, S), dtype=np.float64)
        r_ptr, n = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty(rows.size, dtype=np.float64)
        r_ptr, n = _ptr(rows), rows.size
    rc = _load().oracle_prefill_lse(_ptr(out), _ptr(q), _ptr(k), _DT_CODE[dt], B, Hq, Hkv, S,
                                    D, float(scale), r_ptr, n)
    if rc:
        raise RuntimeError(f"oracle_prefill_lse failed ({rc})")
    return out


def prefill_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
                     scale: float | None = None, q_rows: np.ndarray | None = None,
                     k_rows: np.ndarray | None = None, want_dq: bool = True,
                     want_dkv: bool = True):
    """Gradients (dq, dk, dv) of sum <dout, prefill(q, k, v)>, fp64.

    Full tensors by default ([B,Hq,S,D], [B,Hkv,S,D], [B,Hkv,S,D]); q_rows
    (flat (b*Hq+h)*S+i) or k_rows (flat (b*Hkv+j)*S+t) select rows instead, and
    want_dq / want_dkv skip a side (returned as None)."""
    dt = _dtype_of(q)
    q, k, v, dout = (_as_input(t, dt) for t in (q, k, v, dout))
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, S, D) or v.shape != k.shape or dout.shape != q.shape or Hq % Hkv:
        raise ValueError("bad shapes")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dq = dk = dv = None
    qr = kr = None
    nq = nk = 0
    if want_dq:
        if q_rows is None:
            dq = np.empty((B, Hq, S, D), dtype=np.float64)
        else:
            qr = np.ascontiguousarray(q_rows, dtype=np.int64)
            nq = qr.size
            dq = np.empty((nq, D), dtype=np.float64)
    if want_dkv:
        if k_rows is None:
            dk = np.empty((B, Hkv, S, D), dtype=np.float64)
        else:
            kr = np.ascontiguousarray(k_rows, dtype=np.int64)
            nk = kr.size
            dk = np.empty((nk, D), dtype=np.float64)
        dv = np.empty_like(dk)
    rc = _load().oracle_prefill_backward(_ptr(dq), _ptr(dk), _ptr(dv), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(dout), _DT_CODE[dt], B, Hq, Hkv, S, D, float(scale),
                                         _ptr(qr), nq, _ptr(kr), nk)
    if rc:
        raise RuntimeError(f"oracle_prefill_backward failed ({rc})")
    return dq, dk, dv


# ---------------------------------------------------------------------------
# CCA pre-attention operations ("Compressed Convolutional Attention",
# "Methodologie" items 2-4)
# ---------------------------------------------------------------------------
def cca_mix(q: np.ndarray, k: np.ndarray, v: np.ndarray, conv_q: np.ndarray, conv_k: np.ndarray,
            mix_q: np.ndarray, mix_k: np.ndarray, pos_offset=None, theta: float = 0.0):
    """The compressed q~ [B,Hq,S,D], k~, v~ [B,Hkv,S,D] through the CCA
    pre-attention operations (oracle.c, oracle_cca_mix): a causal depthwise
    sequence convolution of width W (conv_q [Hq,W,D], conv_k [Hkv,W,D]; tap i
    weighs the token i steps back), a dense channel mix per head (mix_q
    [Hq,D,D], mix_k [Hkv,D,D]; row c is output channel c), plus the group's
    pre-convolution query/key mean; RoPE of the result when theta > 0; and
    the value shift (second half of each head's channels from the previous
    token).  All inputs share one dtype.  Returns fp64 (q, k, v)."""
    dt = _dtype_of(q)
    q, k, v, conv_q, conv_k, mix_q, mix_k = (_as_input(t, dt) for t in
                                             (q, k, v, conv_q, conv_k, mix_q, mix_k))
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    W = conv_q.shape[1]
    if (k.shape != (B, Hkv, S, D) or v.shape != k.shape or Hq % Hkv or D % 2
            or conv_q.shape != (Hq, W, D) or conv_k.shape != (Hkv, W, D)
            or mix_q.shape != (Hq, D, D) or mix_k.shape != (Hkv, D, D)):
        raise ValueError("bad shapes")
    off = None
    if pos_offset is not None:
        off = np.ascontiguousarray(pos_offset, dtype=np.int32)
        if off.shape != (B,):
            raise ValueError("pos_offset must have shape [B]")
    qo = np.empty((B, Hq, S, D), dtype=np.float64)
    ko = np.empty((B, Hkv, S, D), dtype=np.float64)
    vo = np.empty((B, Hkv, S, D), dtype=np.float64)
    rc = _load().oracle_cca_mix(_ptr(qo), _ptr(ko), _ptr(vo), _ptr(q), _ptr(k), _ptr(v),
                                _DT_CODE[dt], B, Hq, Hkv, S, D, _ptr(conv_q), _ptr(conv_k), W,
                                _ptr(mix_q), _ptr(mix_k), _ptr(off), float(theta))
    if rc:
        raise RuntimeError(f"oracle_cca_mix failed ({rc})")
    return qo, ko, vo


def cca_mix_backward(gq: np.ndarray, gk: np.ndarray, gv: np.ndarray, q: np.ndarray, k: np.ndarray,
                     conv_q: np.ndarray, conv_k: np.ndarray, mix_q: np.ndarray, mix_k: np.ndarray,
                     pos_offset=None, theta: float = 0.0):
    """Gradients of the CCA pre-attention operations (oracle.c,
    oracle_cca_mix_backward): given gq [B,Hq,S,D], gk, gv [B,Hkv,S,D], the
    gradients of a loss with respect to cca_mix's outputs (q and k as rotated),
    and the latent q~, k~ and the weights that produced them, returns fp64
    (dq~, dk~, dv~, dconv_q, dconv_k, dmix_q, dmix_k); the weight gradients are
    summed over the batch and the tokens.  All inputs share one dtype."""
    dt = _dtype_of(gq)
    gq, gk, gv, q, k, conv_q, conv_k, mix_q, mix_k = (
        _as_input(t, dt) for t in (gq, gk, gv, q, k, conv_q, conv_k, mix_q, mix_k))
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    W = conv_q.shape[1]
    if (gq.shape != q.shape or k.shape != (B, Hkv, S, D) or gk.shape != k.shape
            or gv.shape != k.shape or Hq % Hkv or D % 2
            or conv_q.shape != (Hq, W, D) or conv_k.shape != (Hkv, W, D)
            or mix_q.shape != (Hq, D, D) or mix_k.shape != (Hkv, D, D)):
        raise ValueError("bad shapes")
    off = None
    if pos_offset is not None:
        off = np.ascontiguousarray(pos_offset, dtype=np.int32)
        if off.shape != (B,):
            raise ValueError("pos_offset must have shape [B]")
    dq = np.empty((B, Hq, S, D), dtype=np.float64)
    dk = np.empty((B, Hkv, S, D), dtype=np.float64)
    dv = np.empty((B, Hkv, S, D), dtype=np.float64)
    dcq = np.empty((Hq, W, D), dtype=np.float64)
    dck = np.empty((Hkv, W, D), dtype=np.float64)
    dmq = np.empty((Hq, D, D), dtype=np.float64)
    dmk = np.empty((Hkv, D, D), dtype=np.float64)
    rc = _load().oracle_cca_mix_backward(
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dcq), _ptr(dck), _ptr(dmq), _ptr(dmk), _ptr(gq),
        _ptr(gk), _ptr(gv), _ptr(q), _ptr(k), _DT_CODE[dt], B, Hq, Hkv, S, D, _ptr(conv_q),
        _ptr(conv_k), W, _ptr(mix_q), _ptr(mix_k), _ptr(off), float(theta))
    if rc:
        raise RuntimeError(f"oracle_cca_mix_backward failed ({rc})")
    return dq, dk, dv, dcq, dck, dmq, dmk
