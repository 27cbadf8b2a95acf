"""attn_decode_noalloc (the decode entry point that allocates nothing and keeps
its partial results in the library's static per-device scratch), called
through the C ABI, against attn_decode with a caller workspace on the same
inputs, and against the fp64 oracle (marker `gpu`)."""
import numpy as np
import pytest
import torch

import compressed_latent_causal_amd as attn
import oracle
from compressed_latent_causal_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"
BF16_MAX, BF16_MEAN = 2e-2, 2e-3


def _inputs(B, Hq, Hkv, S_cap, D, lens, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    kc = torch.randn(B, Hkv, S_cap, D, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, Hkv, S_cap, D, generator=g).to(torch.bfloat16)
    lt = torch.tensor(lens, dtype=torch.int32)
    wl.poison_cache_tail(kc, lt)
    wl.poison_cache_tail(vc, lt)
    return q, kc, vc, lt


def _check(case, seed, theta):
    B, Hq, Hkv, S_cap, D, lens = case
    print(f"[case] decode_noalloc {case[:5]} seed {seed}", flush=True)
    q, kc, vc, lt = _inputs(B, Hq, Hkv, S_cap, D, lens, seed)
    qd, kd, vd, ld = (t.to(DEV) for t in (q, kc, vc, lt))
    out = torch.empty_like(qd)
    got = attn.decode_noalloc(qd, kd, vd, ld, out, max_len=S_cap, rope_theta=theta)
    ref_ws = attn.decode(qd, kd, vd, ld, max_len=S_cap, rope_theta=theta)
    torch.cuda.synchronize()
    # the same kernel on the same split: identical to the workspace entry point
    assert torch.equal(got, ref_ws)
    qb = wl.to_numpy_bits(q)
    if theta > 0:
        qb = oracle.round_bf16(oracle.rope(qb[:, :, None, :], theta, lt.numpy() - 1))[:, :, 0]
    ref = oracle.decode(qb, wl.to_numpy_bits(kc), wl.to_numpy_bits(vc), lt.numpy())
    diff = np.abs(got.cpu().double().numpy() - ref)
    assert np.isfinite(diff).all()
    assert diff.max() <= BF16_MAX and diff.mean() <= BF16_MEAN, (diff.max(), diff.mean())


def test_decode_noalloc_two_calls_in_a_row_second_smaller():
    # several split workgroups per sequence, then a smaller batch whose
    # partials land in the same scratch over the first call's contents
    big = (6, 32, 8, 9000, 128, [9000, 4097, 1, 0, 7777, 513])
    small = (2, 16, 2, 3000, 64, [2999, 1200])
    _check(big, 11, 5e5)
    _check(small, 12, 0.0)
    # and back: the smaller call's leftovers do not disturb a larger one
    _check(big, 13, 0.0)


def test_decode_noalloc_long_sequence_many_partials():
    _check((1, 64, 8, 131072, 128, [131072]), 14, 5e5)


def test_decode_noalloc_rejects_problems_beyond_the_scratch():
    B, Hq, Hkv, S_cap, D = 128, 32, 1, 4096, 128
    assert attn.decode_workspace_size(B, Hq, Hkv, S_cap, D) > attn.DECODE_SCRATCH_BYTES
    q = torch.zeros(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(B, Hkv, S_cap, D, dtype=torch.bfloat16, device=DEV)
    lens = torch.ones(B, dtype=torch.int32, device=DEV)
    out = torch.full_like(q, 7.0)
    with pytest.raises(attn.AttnError) as e:
        attn.decode_noalloc(q, kc, kc, lens, out, max_len=S_cap)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert (out == 7.0).all()  # nothing was enqueued
