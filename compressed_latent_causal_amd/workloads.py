"""Seeded synthetic workloads for causal GQA attention (no attention arithmetic).

This module only draws random inputs and describes shapes; it is shared by the
tests, the benchmark and the smoke check, which feed the very same bytes to the
GPU library and to the CPU oracle.

Generator recipe: a CPU ``torch.Generator`` seeded with ``seed`` draws, in this
order, q, k, v (then decode lengths) as float32 N(0, 1); bf16 workloads round
those float32 draws to bf16 (nearest even).  With seed 0 and the tiny shape
this reproduces the tensors of the PyTorch example on the "Grouped Query
Attention (GQA)" glossary page (section "Cómo funciona GQA"): ``manual_seed(0)``
then ``randn`` for q (1,8,16,64), k (1,2,16,64) and v (1,2,16,64).

The named workloads follow the head geometries the pages discuss: Llama 3.1 8B
(32 query heads, 8 KV heads of dim 128; "Por qué GQA reduce la caché KV"), and
the compressed-latent CCGQA setting of "Compressed Convolutional Attention"
("Methodologie"): hidden E = 2048 compressed by C = 4 into a 512-wide latent,
split into 8 query heads of 64 with 2 shared KV heads.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    dtype: str           # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    D: int
    S: int               # prefill: sequence length; decode: cache capacity S_cap
    theta: float
    len_lo: int = 0      # decode: per-sequence lengths uniform in [len_lo, len_hi]
    len_hi: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16}[self.dtype]


# Latent geometry of the CCGQA workload: E / C = 512 = Hq * D.
CCA_HIDDEN = 2048
CCA_COMPRESSION = 4

WORKLOADS = {
    "tiny_gqa": Workload("tiny_gqa", "prefill", "f32", 1, 8, 2, 64, 16, 1e4),
    "llama8b_prefill": Workload("llama8b_prefill", "prefill", "bf16", 4, 32, 8, 128, 4096,
                                5e5),
    "gqa_decode": Workload("gqa_decode", "decode", "bf16", 32, 32, 8, 128, 8192, 5e5,
                           1024, 8192),
    "ccgqa_prefill": Workload("ccgqa_prefill", "prefill", "bf16", 2, 8, 2, 64, 16384, 1e4),
    "long_decode": Workload("long_decode", "decode", "bf16", 1, 64, 8, 128, 131072, 5e5,
                            131072, 131072),
}


def _randn(g: torch.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def make_prefill(w: Workload, seed: int = 0):
    """q [B,Hq,S,D], k, v [B,Hkv,S,D] on the CPU, dtype of the workload."""
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, (w.B, w.Hq, w.S, w.D), w.torch_dtype)
    k = _randn(g, (w.B, w.Hkv, w.S, w.D), w.torch_dtype)
    v = _randn(g, (w.B, w.Hkv, w.S, w.D), w.torch_dtype)
    return q, k, v


def make_backward(w: Workload, seed: int = 0):
    """q, k, v as make_prefill (same draws), then the output gradient dout
    [B,Hq,S,D] drawn next from the same generator, N(0,1)."""
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, (w.B, w.Hq, w.S, w.D), w.torch_dtype)
    k = _randn(g, (w.B, w.Hkv, w.S, w.D), w.torch_dtype)
    v = _randn(g, (w.B, w.Hkv, w.S, w.D), w.torch_dtype)
    dout = _randn(g, (w.B, w.Hq, w.S, w.D), w.torch_dtype)
    return q, k, v, dout


def make_decode(w: Workload, seed: int = 0, poison_tail: bool = False):
    """q [B,Hq,D], k/v caches [B,Hkv,S_cap,D], seqlens int32 [B] (CPU).

    Lengths are integers drawn uniformly from [len_lo, len_hi] (both ends
    included).  The cache is filled to capacity with N(0,1); with poison_tail,
    every slot at or beyond a sequence's length holds NaN instead, so that a
    kernel reading past the length shows up in the output.
    """
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, (w.B, w.Hq, w.D), w.torch_dtype)
    k = _randn(g, (w.B, w.Hkv, w.S, w.D), w.torch_dtype)
    v = _randn(g, (w.B, w.Hkv, w.S, w.D), w.torch_dtype)
    if w.len_lo == w.len_hi:
        lens = torch.full((w.B,), w.len_hi, dtype=torch.int32)
    else:
        lens = torch.randint(w.len_lo, w.len_hi + 1, (w.B,), generator=g, dtype=torch.int32)
    if poison_tail:
        poison_cache_tail(k, lens)
        poison_cache_tail(v, lens)
    return q, k, v, lens


# Width of the causal sequence convolution of the CCA pre-attention operations
# (the summary gives none; 4 is a common short-convolution width).
CCA_CONV_WIDTH = 4


def make_cca(w: Workload, seed: int = 0, width: int = CCA_CONV_WIDTH):
    """Inputs of the CCA pre-attention operations (CPU, dtype of the workload):
    the compressed q~ [B,Hq,S,D], k~, v~ [B,Hkv,S,D] drawn as make_prefill
    draws q, k, v, then from the same generator the sequence-convolution taps
    conv_q [Hq,width,D], conv_k [Hkv,width,D] ~ N(0, 1/width) and the
    channel-mixing matrices mix_q [Hq,D,D], mix_k [Hkv,D,D] ~ N(0, 1/D), so
    the mixed vectors keep about unit scale."""
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, (w.B, w.Hq, w.S, w.D), w.torch_dtype)
    k = _randn(g, (w.B, w.Hkv, w.S, w.D), w.torch_dtype)
    v = _randn(g, (w.B, w.Hkv, w.S, w.D), w.torch_dtype)

    def scaled(shape, s):
        x = torch.randn(*shape, generator=g, dtype=torch.float32) * s
        return x if w.torch_dtype == torch.float32 else x.to(w.torch_dtype)

    conv_q = scaled((w.Hq, width, w.D), width ** -0.5)
    conv_k = scaled((w.Hkv, width, w.D), width ** -0.5)
    mix_q = scaled((w.Hq, w.D, w.D), w.D ** -0.5)
    mix_k = scaled((w.Hkv, w.D, w.D), w.D ** -0.5)
    return q, k, v, conv_q, conv_k, mix_q, mix_k


def make_cca_grads(w: Workload, seed: int = 0):
    """Gradients for the CCA backward (CPU, dtype of the workload): gq
    [B,Hq,S,D], gk, gv [B,Hkv,S,D] ~ N(0, 1), standing in for what the
    attention backward returns for the mixed q, k, v."""
    g = torch.Generator().manual_seed(seed)
    return (_randn(g, (w.B, w.Hq, w.S, w.D), w.torch_dtype),
            _randn(g, (w.B, w.Hkv, w.S, w.D), w.torch_dtype),
            _randn(g, (w.B, w.Hkv, w.S, w.D), w.torch_dtype))


def poison_cache_tail(cache: torch.Tensor, lens: torch.Tensor) -> None:
    """Write NaN into cache[b, :, t, :] for every t >= lens[b] (in place)."""
    for b in range(cache.shape[0]):
        n = int(lens[b])
        if n < cache.shape[2]:
            cache[b, :, n:, :] = float("nan")


def to_pages(k: torch.Tensor, v: torch.Tensor, lens: torch.Tensor, page_size: int, seed: int = 0,
             spare_pages: int = 3):
    """Lay a contiguous cache [B,Hkv,S,D] out as a paged one (CPU).

    Returns (k_pages, v_pages, block_table): pages [num_pages,Hkv,page_size,D]
    and table int32 [B, ceil(S/page_size)], where token t of sequence b is row
    t % page_size of page table[b, t // page_size].  Only the pages holding a
    sequence's first lens[b] tokens are kept, in a seeded random physical
    order, mixed with `spare_pages` NaN pages that no table entry names; table
    entries past a sequence's pages are -1.  Rows past a length inside its
    last page keep the contiguous cache's values."""
    B, Hkv, S, D = k.shape
    mp = -(-S // page_size)
    need = [-(-int(n) // page_size) for n in lens]
    total = sum(need) + spare_pages
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(total, generator=g)
    kp = torch.full((total, Hkv, page_size, D), float("nan"), dtype=k.dtype)
    vp = torch.full_like(kp, float("nan"))
    table = torch.full((B, mp), -1, dtype=torch.int32)
    slot = 0
    for b in range(B):
        for i in range(need[b]):
            pg = int(perm[slot])
            slot += 1
            lo, hi = i * page_size, min(S, (i + 1) * page_size)
            kp[pg, :, :hi - lo] = k[b, :, lo:hi]
            vp[pg, :, :hi - lo] = v[b, :, lo:hi]
            table[b, i] = pg
    return kp, vp, table


def custom(kind: str, dtype: str, B: int, Hq: int, Hkv: int, D: int, S: int,
           theta: float = 1e4, len_lo: int = 0, len_hi: int = 0) -> Workload:
    """An ad-hoc workload (tests sweep shapes and edge cases with it)."""
    return Workload(f"custom_{kind}", kind, dtype, B, Hq, Hkv, D, S, theta, len_lo, len_hi)


def to_numpy_bits(t: torch.Tensor):
    """CPU tensor -> numpy array in the oracle's input convention
    (float32/float64 as is, bf16 as uint16 bit patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


def from_numpy_bits(a, dtype: torch.dtype) -> torch.Tensor:
    """Inverse of to_numpy_bits for float32 / bf16."""
    import numpy as np
    if dtype == torch.bfloat16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype)
