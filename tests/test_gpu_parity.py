"""GPU parity: the HIP library, called through its C ABI, against the fp64 CPU
oracle on the same seeded inputs (marker `gpu`; needs an MI355X).

Tolerances (the benchmark spec): bf16 attention max |err| <= 2e-2 and mean |err| <=
2e-3; fp32 attention max |err| <= 1e-5.  RoPE is checked bit for bit: the bf16
output must equal the oracle's fp64 rotation rounded to nearest even, except
where the exact value lies within the fp32 evaluation error of a rounding
midpoint (there it may be the neighbouring bf16 value), and each token's
rotation must match its own integer position better than any neighbouring
one.  No expected value comes from the
GPU; inputs come from compressed_latent_causal_amd.workloads.
"""
import math

import numpy as np
import pytest
import torch

import compressed_latent_causal_amd as attn
import oracle
from compressed_latent_causal_amd import workloads as wl

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, F32_MAX = 2e-2, 2e-3, 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    attn.lib()  # fail loudly if the library was not built


DEV = "cuda"


def say(msg):
    print(f"[case] {msg}", flush=True)


def bits(t):
    return wl.to_numpy_bits(t)


def dev(t):
    return t.to(DEV)


def host_f64(t):
    return t.detach().cpu().double().numpy()


def assert_close(got, ref, max_tol, mean_tol=None, what=""):
    diff = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    mx, mn = float(diff.max()), float(diff.mean())
    say(f"{what}: max {mx:.3e} mean {mn:.3e}")
    assert mx <= max_tol, f"{what}: max abs err {mx} > {max_tol}"
    if mean_tol is not None:
        assert mn <= mean_tol, f"{what}: mean abs err {mn} > {mean_tol}"


def rand_bf16(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g).to(torch.bfloat16)


# ============================================================== RoPE
def _rope_err_bound(x_bits):
    """Bound on |fp32-evaluated rotation - exact rotation| for every output
    element: cos/sin rounded to fp32 (2^-24 relative each), one rounded product
    and one FMA (2^-24 relative each), so 2^-21 (|x0| + |x1|) of its pair is
    generous."""
    x = oracle.widen(x_bits)
    pair = np.abs(x[..., 0::2]) + np.abs(x[..., 1::2])
    return np.repeat(pair, 2, axis=-1) * 2.0 ** -21


def _bf16_midpoint_distance(y):
    """Distance of each fp64 value to the nearest bf16 rounding midpoint."""
    a = np.abs(y)
    _, e = np.frexp(a)                 # a = m * 2**e, 0.5 <= m < 1
    ulp = np.ldexp(1.0, e - 8)         # bf16 keeps 8 significant bits
    frac = a / ulp - np.floor(a / ulp)
    return np.abs(frac - 0.5) * ulp


def assert_rope_rounding(got_bits, ref, x_bits):
    """The GPU output must be RNE of the exact rotation wherever the exact
    value is farther from a bf16 midpoint than the fp32 evaluation error; at
    the remaining elements it may be the other neighbour (one ulp away)."""
    want = oracle.round_bf16(ref)
    mism = got_bits != want
    n = int(mism.sum())
    say(f"rope: {n} of {got_bits.size} elements round the other way near a midpoint")
    if n:
        bound = _rope_err_bound(x_bits)[mism]
        near = _bf16_midpoint_distance(ref[mism]) <= bound
        assert near.all(), f"{int((~near).sum())} elements differ from RNE(oracle) away from a midpoint"
        # the output is RNE of a value within `bound` of the exact one (under
        # cancellation that can be more than one bf16 step from RNE(exact))
        got = oracle.widen(got_bits[mism])
        _, e = np.frexp(np.abs(got))
        assert (np.abs(got - ref[mism]) <= bound + np.ldexp(1.0, e - 9)).all()
    assert n <= max(2, got_bits.size // 1000)


@pytest.mark.parametrize("D,theta,B,H,S,offsets", [
    (128, 5e5, 2, 3, 37, [0, 131000]),
    (64, 1e4, 1, 8, 300, [5]),
    (128, 1e4, 3, 2, 16, [0, 1, 2_000_000]),
    (64, 5e5, 2, 1, 129, None),
    (128, 5e5, 4, 32, 64, None),              # all heads in one workgroup
    (128, 5e5, 3, 40, 1, [1, 8191, 131071]),  # decode-like: one token, head blocks
])
def test_rope_bf16_matches_rounded_oracle(D, theta, B, H, S, offsets):
    x = rand_bf16((B, H, S, D), 100 + S)
    off = None if offsets is None else torch.tensor(offsets, dtype=torch.int32)
    say(f"rope bf16 B={B} H={H} S={S} D={D} theta={theta} offsets={offsets}")
    y = attn.rope(dev(x), theta, None if off is None else dev(off))
    torch.cuda.synchronize()
    ref = oracle.rope(bits(x), theta, None if off is None else off.numpy())
    assert_rope_rounding(bits(y), ref, bits(x))


@pytest.mark.parametrize("D", [64, 128])
def test_rope_position_indexing_is_exact(D):
    """Every token's output is closest to the oracle at its own position, not a
    neighbouring one (checked over a window of +-3 positions)."""
    B, H, S = 2, 2, 64
    offsets = np.array([0, 131007], dtype=np.int32)
    x = rand_bf16((B, H, S, D), 7)
    say(f"rope indexing D={D}")
    y = host_f64(attn.rope(dev(x), 5e5, dev(torch.from_numpy(offsets))))
    dists = []
    for delta in range(-3, 4):
        r = oracle.widen(oracle.round_bf16(oracle.rope(bits(x), 5e5, offsets + delta)))
        dists.append(np.abs(y - r).sum(axis=-1))
    best = np.argmin(np.stack(dists), axis=0)
    assert (best == 3).all()


def test_rope_fp32_and_in_place():
    x = torch.randn(2, 4, 50, 128, generator=torch.Generator().manual_seed(3))
    offs = torch.tensor([7, 90000], dtype=torch.int32)
    say("rope fp32 out-of-place and in place")
    xd = dev(x)
    y = attn.rope(xd, 5e5, dev(offs))
    ref = oracle.rope(x.numpy(), 5e5, offs.numpy())
    assert_close(host_f64(y), ref, 2e-6, what="rope fp32")
    attn.rope(xd, 5e5, dev(offs), out=xd)
    assert torch.equal(xd, y)
    xb = dev(rand_bf16((1, 3, 20, 64), 4))
    yb = attn.rope(xb, 1e4)
    attn.rope(xb, 1e4, out=xb)
    assert torch.equal(xb, yb)


def test_rope_decode_positions_from_lengths():
    """pos_offset = seqlens and pos_shift = -1 put each decode query at len - 1."""
    lens = torch.tensor([1, 17, 8192, 131072], dtype=torch.int32)
    q = rand_bf16((4, 8, 1, 128), 11)
    say("rope decode positions")
    y = bits(attn.rope(dev(q), 5e5, dev(lens), pos_shift=-1))
    assert_rope_rounding(y, oracle.rope(bits(q), 5e5, lens.numpy() - 1), bits(q))


@pytest.mark.parametrize("D,theta,B,H,S,offsets", [
    (128, 5e5, 2, 3, 37, [0, 131000]),
    (64, 1e4, 1, 8, 300, [5]),
    (128, 5e5, 3, 40, 1, [1, 8191, 131071]),
])
def test_rope_backward_bf16_matches_rounded_oracle_transpose(D, theta, B, H, S, offsets):
    """The transpose carries the same rounding guarantee as the rotation: the
    same angles with negated sines, one product and one FMA per output."""
    g = rand_bf16((B, H, S, D), 200 + S)
    off = None if offsets is None else torch.tensor(offsets, dtype=torch.int32)
    say(f"rope_backward bf16 B={B} H={H} S={S} D={D} theta={theta} offsets={offsets}")
    y = attn.rope_backward(dev(g), theta, None if off is None else dev(off))
    torch.cuda.synchronize()
    ref = oracle.rope_transpose(bits(g), theta, None if off is None else off.numpy())
    assert_rope_rounding(bits(y), ref, bits(g))


def test_rope_backward_fp32_undoes_rope_and_works_in_place():
    x = torch.randn(2, 4, 50, 128, generator=torch.Generator().manual_seed(13))
    offs = torch.tensor([3, 70000], dtype=torch.int32)
    say("rope_backward fp32")
    xd, od = dev(x), dev(offs)
    y = attn.rope_backward(xd, 5e5, od)
    assert_close(host_f64(y), oracle.rope_transpose(x.numpy(), 5e5, offs.numpy()), 2e-6,
                 what="rope_backward fp32")
    back = attn.rope_backward(attn.rope(xd, 5e5, od), 5e5, od)
    assert_close(host_f64(back), x.double().numpy(), 2e-6, what="rope_backward(rope(x))")
    attn.rope_backward(xd, 5e5, od, out=xd)
    assert torch.equal(xd, y)


# ============================================================== prefill
def _oracle_prefill_e2e(q, k, v, theta, scale, dtype, rows=None):
    """Oracle pipeline: RoPE in fp64, rounded to the storage type (the dtype
    boundary between the two calls), then attention in fp64."""
    rq = oracle.round_to(oracle.rope(bits(q), theta), dtype)
    rk = oracle.round_to(oracle.rope(bits(k), theta), dtype)
    return oracle.prefill(rq, rk, bits(v), scale=scale, rows=rows)


def test_prefill_worked_example_fp32_end_to_end():
    """The GQA glossary's example geometry (8 query heads, 2 KV heads, 16
    tokens, dim 64, seed 0) with RoPE theta 1e4 and scale 1/8, in fp32."""
    w = wl.WORKLOADS["tiny_gqa"]
    q, k, v = wl.make_prefill(w, seed=0)
    say("tiny fp32 end to end")
    o = attn.prefill(attn.rope(dev(q), w.theta), attn.rope(dev(k), w.theta), dev(v), w.scale)
    ref = _oracle_prefill_e2e(q, k, v, w.theta, w.scale, "f32")
    assert tuple(o.shape) == (1, 8, 16, 64)
    assert_close(host_f64(o), ref, F32_MAX, what="tiny fp32")


def test_prefill_worked_example_fp32_fused_rope():
    """Same example with the query rotation done inside the prefill kernel."""
    w = wl.WORKLOADS["tiny_gqa"]
    q, k, v = wl.make_prefill(w, seed=0)
    say("tiny fp32 end to end, fused query RoPE")
    o = attn.prefill(dev(q), attn.rope(dev(k), w.theta), dev(v), w.scale, rope_theta=w.theta)
    ref = _oracle_prefill_e2e(q, k, v, w.theta, w.scale, "f32")
    assert_close(host_f64(o), ref, F32_MAX, what="tiny fp32 fused")


FUSED_ROPE_GEOMS = [  # B, Hq, Hkv, S, D, dtype, theta
    (1, 8, 2, 16, 64, "bf16", 1e4),
    (2, 8, 2, 257, 64, "bf16", 1e4),
    (2, 8, 2, 200, 128, "bf16", 5e5),
    (1, 32, 2, 70, 128, "bf16", 5e5),    # G = 16: two head slices
    (1, 12, 2, 90, 128, "bf16", 1e4),    # G = 6
    (1, 8, 2, 100, 64, "f32", 1e4),
    (1, 4, 4, 70, 128, "f32", 5e5),
]


@pytest.mark.parametrize("geom", FUSED_ROPE_GEOMS)
def test_prefill_fused_rope_equals_separate_rope(geom):
    """rope_theta > 0 rotates q in the prefill kernel exactly as attn_rope does."""
    B, Hq, Hkv, S, D, dt, theta = geom
    g = torch.Generator().manual_seed(S * 7 + D)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    q, k, v = (torch.randn(*shp, generator=g).to(dtype) for shp in
               ((B, Hq, S, D), (B, Hkv, S, D), (B, Hkv, S, D)))
    say(f"prefill fused vs separate RoPE {geom}")
    qd, kd, vd = dev(q), dev(k), dev(v)
    kr = attn.rope(kd, theta)
    sep = attn.prefill(attn.rope(qd, theta), kr, vd)
    fused = attn.prefill(qd, kr, vd, rope_theta=theta)
    assert torch.equal(sep, fused)


@pytest.mark.parametrize("seed", [0, 1])
def test_prefill_worked_example_gqa_equals_repeated_mha(seed):
    w = wl.WORKLOADS["tiny_gqa"]
    q, k, v = (dev(t) for t in wl.make_prefill(w, seed=seed))
    say(f"tiny GQA vs repeat-interleaved MHA seed {seed}")
    out = attn.prefill(q, k, v)
    ref = attn.prefill(q, k.repeat_interleave(4, dim=1).contiguous(),
                       v.repeat_interleave(4, dim=1).contiguous())
    assert torch.allclose(out, ref, atol=1e-6, rtol=0)


GEOMS = [  # B, Hq, Hkv, S, D
    (1, 8, 2, 1, 64),
    (1, 8, 2, 16, 64),
    (1, 8, 2, 63, 64),
    (1, 8, 2, 64, 64),
    (1, 8, 2, 65, 64),
    (1, 8, 2, 130, 64),
    (2, 8, 2, 257, 64),
    (2, 8, 2, 200, 128),
    (1, 4, 4, 300, 128),     # MHA
    (1, 8, 1, 150, 64),      # MQA, G = 8
    (1, 32, 2, 70, 128),     # G = 16: two head slices per KV group
    (2, 6, 2, 100, 64),      # G = 3
    (1, 12, 2, 90, 128),     # G = 6
    (3, 4, 2, 513, 128),
]


@pytest.mark.parametrize("geom", GEOMS)
def test_prefill_bf16_matches_oracle(geom):
    B, Hq, Hkv, S, D = geom
    q, k, v = rand_bf16((B, Hq, S, D), 1), rand_bf16((B, Hkv, S, D), 2), rand_bf16((B, Hkv, S, D), 3)
    say(f"prefill bf16 {geom}")
    o = attn.prefill(dev(q), dev(k), dev(v))
    ref = oracle.prefill(bits(q), bits(k), bits(v))
    assert_close(host_f64(o), ref, BF16_MAX, BF16_MEAN, what=f"prefill bf16 {geom}")


@pytest.mark.parametrize("geom", [(1, 8, 2, 1, 64), (1, 8, 2, 77, 64), (2, 4, 4, 100, 128),
                                  (1, 8, 1, 40, 128), (1, 6, 2, 33, 64)])
def test_prefill_fp32_matches_oracle(geom):
    B, Hq, Hkv, S, D = geom
    g = torch.Generator().manual_seed(5)
    q, k, v = (torch.randn(*s, generator=g) for s in [(B, Hq, S, D), (B, Hkv, S, D), (B, Hkv, S, D)])
    say(f"prefill fp32 {geom}")
    o = attn.prefill(dev(q), dev(k), dev(v))
    ref = oracle.prefill(q.numpy(), k.numpy(), v.numpy())
    assert_close(host_f64(o), ref, F32_MAX, what=f"prefill fp32 {geom}")


def test_prefill_gqa_equals_repeated_mha_bitwise():
    B, Hq, Hkv, S, D = 2, 8, 2, 333, 128
    q, k, v = (dev(rand_bf16(s, i)) for i, s in enumerate([(B, Hq, S, D), (B, Hkv, S, D), (B, Hkv, S, D)]))
    say("prefill GQA vs MHA bitwise")
    out = attn.prefill(q, k, v)
    mha = attn.prefill(q, k.repeat_interleave(Hq // Hkv, dim=1).contiguous(),
                       v.repeat_interleave(Hq // Hkv, dim=1).contiguous())
    assert torch.equal(out, mha)


def test_prefill_is_causal_on_gpu():
    B, Hq, Hkv, S, D = 1, 8, 2, 200, 64
    q, k, v = rand_bf16((B, Hq, S, D), 8), rand_bf16((B, Hkv, S, D), 9), rand_bf16((B, Hkv, S, D), 10)
    say("prefill causality")
    base = attn.prefill(dev(q), dev(k), dev(v))
    i = 120
    k2, v2 = k.clone(), v.clone()
    k2[:, :, i + 1:] = rand_bf16(k2[:, :, i + 1:].shape, 11)
    v2[:, :, i + 1:] = 1e3
    pert = attn.prefill(dev(q), dev(k2), dev(v2))
    assert torch.equal(pert[:, :, :i + 1], base[:, :, :i + 1])


def test_prefill_scale_and_errors():
    q, k, v = rand_bf16((1, 4, 40, 64), 12), rand_bf16((1, 2, 40, 64), 13), rand_bf16((1, 2, 40, 64), 14)
    say("prefill explicit scale")
    o = attn.prefill(dev(q), dev(k), dev(v), scale=0.3)
    assert_close(host_f64(o), oracle.prefill(bits(q), bits(k), bits(v), scale=0.3), BF16_MAX,
                 BF16_MEAN, what="scale 0.3")
    with pytest.raises(attn.AttnError) as e:
        attn.prefill(dev(rand_bf16((1, 4, 8, 96), 1)), dev(rand_bf16((1, 2, 8, 96), 2)),
                     dev(rand_bf16((1, 2, 8, 96), 3)))
    assert e.value.status == 3
    with pytest.raises(ValueError):
        attn.prefill(dev(q), dev(k).float(), dev(v))


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_scores_growing_along_the_keys(D):
    """Keys scaled up along the sequence (and queries aligned with them), so
    later tiles keep exceeding the row's reference by many exp2 units: the
    kernel's rescale path runs on most tiles, and some tiles' probabilities
    relative to a stale reference would overflow."""
    B, Hq, Hkv, S = 1, 4, 2, 700
    g = torch.Generator().manual_seed(77 + D)
    base = torch.randn(D, generator=g)
    q = (base + 0.3 * torch.randn(B, Hq, S, D, generator=g)).to(torch.bfloat16)
    growth = torch.linspace(0.2, 3.0, S).reshape(1, 1, S, 1)
    k = ((base + 0.3 * torch.randn(B, Hkv, S, D, generator=g)) * growth).to(torch.bfloat16)
    v = torch.randn(B, Hkv, S, D, generator=g).to(torch.bfloat16)
    say(f"prefill growing scores D={D}")
    o = attn.prefill(dev(q), dev(k), dev(v))
    assert_close(host_f64(o), oracle.prefill(bits(q), bits(k), bits(v)), BF16_MAX, BF16_MEAN,
                 what=f"growing scores D={D}")


PEAKED = [  # B, Hq, Hkv, S, D, sigma of q and k, fused RoPE theta (0: none)
    (1, 8, 2, 517, 64, 3.0, 0.0),
    (1, 8, 2, 517, 128, 3.0, 0.0),
    (2, 4, 1, 300, 64, 5.0, 1e4),
    (1, 4, 2, 1000, 128, 5.0, 5e5),
]


@pytest.mark.parametrize("case", PEAKED)
def test_prefill_peaked_softmax(case):
    """q and k ~ N(0, sigma^2), so the scaled scores have a standard deviation
    of sigma^2 (9 and 25): a row's weight sits on a few keys, and a score
    error of a few hundredths of an exp2 unit shows in the output.  bf16
    inputs must still meet the bf16 tolerance (the kernel multiplies the exact
    q, never a rounded pre-scaled copy)."""
    B, Hq, Hkv, S, D, sigma, theta = case
    g = torch.Generator().manual_seed(int(100 * sigma) + D + S)
    q = (torch.randn(B, Hq, S, D, generator=g) * sigma).to(torch.bfloat16)
    k = (torch.randn(B, Hkv, S, D, generator=g) * sigma).to(torch.bfloat16)
    v = torch.randn(B, Hkv, S, D, generator=g).to(torch.bfloat16)
    say(f"prefill peaked softmax {case}")
    o = attn.prefill(dev(q), dev(k), dev(v), rope_theta=theta)
    qb = bits(q) if theta == 0 else oracle.round_bf16(oracle.rope(bits(q), theta))
    ref = oracle.prefill(qb, bits(k), bits(v))
    assert_close(host_f64(o), ref, BF16_MAX, BF16_MEAN, what=f"peaked {case}")


@pytest.mark.parametrize("sigma", [3.0, 5.0])
def test_decode_peaked_softmax(sigma):
    B, Hq, Hkv, S_cap, D = 4, 16, 2, 3000, 128
    g = torch.Generator().manual_seed(int(10 * sigma))
    q = (torch.randn(B, Hq, D, generator=g) * sigma).to(torch.bfloat16)
    kc = (torch.randn(B, Hkv, S_cap, D, generator=g) * sigma).to(torch.bfloat16)
    vc = torch.randn(B, Hkv, S_cap, D, generator=g).to(torch.bfloat16)
    lens = torch.tensor([3000, 1700, 513, 31], dtype=torch.int32)
    say(f"decode peaked softmax sigma={sigma}")
    o = attn.decode(dev(q), dev(kc), dev(vc), dev(lens))
    ref = oracle.decode(bits(q), bits(kc), bits(vc), lens.numpy())
    assert_close(host_f64(o), ref, BF16_MAX, BF16_MEAN, what=f"decode peaked {sigma}")


def _sample_rows(B, Hq, S, n_random, seed):
    """Row indices (b*Hq + h)*S + i: both ends of every head, tile edges and
    random interior rows."""
    rng = np.random.default_rng(seed)
    edge = [0, 1, 31, 32, 63, 64, 65, S // 2, S - 65, S - 2, S - 1]
    rows = []
    for b in range(B):
        for h in range(Hq):
            if (b + h) % 3 == 0:
                rows += [(b * Hq + h) * S + i for i in edge]
    rows += list(rng.integers(0, B * Hq * S, n_random))
    return np.unique(np.array(rows, dtype=np.int64))


@pytest.mark.parametrize("name", ["llama8b_prefill", "ccgqa_prefill"])
def test_prefill_full_size_sampled_rows(name):
    """Full-size workloads in the launch configuration the benchmark times:
    RoPE on K, then prefill with the query rotation fused, end to end from the
    raw inputs; the oracle recomputes a sample of output rows."""
    w = wl.WORKLOADS[name]
    q, k, v = wl.make_prefill(w, seed=0)
    say(f"{name} full size: rope(K) + prefill with fused query RoPE")
    qd, kd, vd = dev(q), dev(k), dev(v)
    o = attn.prefill(qd, attn.rope(kd, w.theta), vd, w.scale, rope_theta=w.theta)
    torch.cuda.synchronize()
    rows = _sample_rows(w.B, w.Hq, w.S, 200, 42)
    got = o.reshape(-1, w.D)[torch.from_numpy(rows).to(DEV)].double().cpu().numpy()
    del o, qd, kd, vd
    # oracle: RoPE of the sampled query rows and of all keys, rounded to bf16
    rk = oracle.round_bf16(oracle.rope(bits(k), w.theta))
    qsel = bits(q).reshape(-1, w.D)[rows].reshape(-1, 1, 1, w.D)   # one "sequence" per row
    pos = (rows % w.S).astype(np.int32)                               # its token position
    rq_sel = oracle.round_bf16(oracle.rope(qsel, w.theta, pos))
    rq = np.zeros(w.B * w.Hq * w.S * w.D, dtype=np.uint16).reshape(-1, w.D)
    rq[rows] = rq_sel.reshape(-1, w.D)
    ref = oracle.prefill(rq.reshape(w.B, w.Hq, w.S, w.D), rk, bits(v), scale=w.scale, rows=rows)
    assert_close(got, ref, BF16_MAX, BF16_MEAN, what=f"{name} sampled rows")


# ============================================================== decode
def _decode_e2e(w, seed, poison=True, max_len=None):
    """Decode with the query's RoPE fused into the kernel (rope_theta), against
    the oracle pipeline: RoPE of q at position len - 1 in fp64, rounded to bf16,
    then decode in fp64."""
    q, kc, vc, lens = wl.make_decode(w, seed=seed, poison_tail=poison)
    say(f"decode {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} S_cap={w.S} D={w.D} "
        f"lens {int(lens.min())}..{int(lens.max())}")
    o = attn.decode(dev(q), dev(kc), dev(vc), dev(lens), max_len=max_len, scale=w.scale,
                    rope_theta=w.theta)
    torch.cuda.synchronize()
    rq = oracle.round_bf16(oracle.rope(bits(q)[:, :, None, :], w.theta, lens.numpy() - 1))[:, :, 0]
    ref = oracle.decode(rq, bits(kc), bits(vc), lens.numpy(), scale=w.scale)
    return host_f64(o), ref


def test_decode_fused_rope_equals_separate_rope():
    """rope_theta > 0 rotates q in the split kernel exactly as attn_rope does."""
    B, Hq, Hkv, S_cap, D = 5, 16, 2, 700, 128
    q, kc, vc = rand_bf16((B, Hq, D), 40), rand_bf16((B, Hkv, S_cap, D), 41), rand_bf16((B, Hkv, S_cap, D), 42)
    lens = torch.tensor([700, 1, 333, 64, 0], dtype=torch.int32)
    say("decode fused vs separate RoPE")
    ld = dev(lens)
    qr = attn.rope(dev(q).unsqueeze(2), 5e5, ld, pos_shift=-1).squeeze(2)
    sep = attn.decode(qr, dev(kc), dev(vc), ld)
    fused = attn.decode(dev(q), dev(kc), dev(vc), ld, rope_theta=5e5)
    assert torch.equal(sep, fused)


@pytest.mark.parametrize("name", ["gqa_decode", "long_decode"])
def test_decode_full_size_end_to_end(name):
    """Full-size decode workloads, every output checked; the gqa workload's
    cache tail past each length is NaN."""
    w = wl.WORKLOADS[name]
    got, ref = _decode_e2e(w, seed=0, poison=(name == "gqa_decode"))
    assert_close(got, ref, BF16_MAX, BF16_MEAN, what=name)


DECODE_CASES = [  # B, Hq, Hkv, S_cap, D, lengths
    (9, 8, 2, 1100, 128, [0, 1, 31, 32, 33, 511, 512, 513, 1100]),
    (4, 8, 8, 300, 64, [300, 1, 129, 64]),        # MHA, D = 64
    (3, 8, 1, 700, 128, [700, 350, 2]),           # MQA, G = 8
    (2, 32, 2, 260, 128, [260, 100]),             # G = 16
    (2, 64, 2, 100, 64, [100, 37]),               # G = 32: two head slices
    (2, 12, 4, 90, 128, [90, 45]),                # G = 3
    (1, 4, 1, 5000, 128, [4999]),
    # several split workgroups per sequence (merged by the last one to finish)
    # next to single-workgroup sequences in the same batch
    (3, 16, 2, 20000, 64, [20000, 4097, 1]),
    (2, 64, 2, 9000, 128, [9000, 8193]),          # two head slices, 3 partials each
    (1, 2, 1, 1100000, 64, [1100000]),            # > 256 partials: blocked final merge
    # more (sequence, KV head) groups than the launch budget (two workgroups
    # per compute unit): one workgroup per group
    (70, 8, 8, 200, 64, [(37 * i) % 201 for i in range(70)]),
    # over 64 ragged sequences under the budget: the split's prefix sums span
    # several 64-sequence passes
    (100, 4, 1, 3000, 64, [(997 * i) % 3001 for i in range(100)]),
]


@pytest.mark.parametrize("case", DECODE_CASES)
def test_decode_edge_cases(case):
    B, Hq, Hkv, S_cap, D, lens = case
    g = torch.Generator().manual_seed(B * 1000 + S_cap)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    kc = torch.randn(B, Hkv, S_cap, D, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, Hkv, S_cap, D, generator=g).to(torch.bfloat16)
    lt = torch.tensor(lens, dtype=torch.int32)
    wl.poison_cache_tail(kc, lt)
    wl.poison_cache_tail(vc, lt)
    say(f"decode edge {case}")
    o = attn.decode(dev(q), dev(kc), dev(vc), dev(lt), max_len=max(lens))
    ref = oracle.decode(bits(q), bits(kc), bits(vc), lt.numpy())
    got = host_f64(o)
    assert_close(got, ref, BF16_MAX, BF16_MEAN, what=f"decode {case}")
    for b, n in enumerate(lens):
        if n == 0:
            assert (got[b] == 0).all()


PAGED_CASES = [  # B, Hq, Hkv, S_cap, D, page_size, lengths, window
    (9, 8, 2, 1100, 128, 64, [0, 1, 31, 32, 33, 511, 512, 513, 1100], 0),
    (9, 8, 2, 1100, 128, 32, [0, 1, 31, 32, 33, 511, 512, 513, 1100], 0),
    (4, 8, 8, 300, 64, 256, [300, 1, 129, 64], 0),
    (3, 16, 2, 20000, 64, 128, [20000, 4097, 1], 0),   # several split workgroups
    (2, 64, 2, 9000, 128, 512, [9000, 8193], 0),       # two head slices
    (5, 8, 2, 3000, 128, 64, [3000, 1000, 64, 2, 0], 1),
    (5, 8, 2, 3000, 128, 64, [3000, 1000, 64, 2, 0], 31),
    (5, 8, 2, 3000, 128, 64, [3000, 1000, 64, 33, 0], 32),
    (5, 8, 2, 3000, 64, 32, [3000, 1000, 64, 33, 0], 33),
    (5, 8, 2, 3000, 128, 256, [3000, 1000, 64, 33, 0], 1024),
    (2, 16, 2, 20000, 128, 256, [20000, 12000], 4096),  # windows split over workgroups
    (70, 8, 8, 200, 64, 32, [(37 * i) % 201 for i in range(70)], 50),
    (3, 16, 1, 2000, 128, 64, [2000, 777, 5], 100),     # MQA
    (3, 8, 2, 500, 64, 64, [500, 100, 1], 4096),        # window wider than every length
]


@pytest.mark.parametrize("case", PAGED_CASES)
def test_decode_paged_matches_oracle(case):
    """Paged cache in shuffled page order with unreferenced NaN pages, table
    entries past each sequence set to -1, and an optional sliding window."""
    B, Hq, Hkv, S_cap, D, P, lens, window = case
    g = torch.Generator().manual_seed(B * 100 + P + window)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    kc = torch.randn(B, Hkv, S_cap, D, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, Hkv, S_cap, D, generator=g).to(torch.bfloat16)
    lt = torch.tensor(lens, dtype=torch.int32)
    kp, vp, table = wl.to_pages(kc, vc, lt, P, seed=B + P)
    say(f"decode paged B={B} Hq={Hq} Hkv={Hkv} S_cap={S_cap} D={D} page={P} window={window} "
        f"lens={lens if len(lens) < 12 else str(len(lens)) + ' ragged'}")
    o = attn.decode_paged(dev(q), dev(kp), dev(vp), dev(table), dev(lt), max_len=max(lens),
                          window=window)
    ref = oracle.decode_paged(bits(q), bits(kp), bits(vp),
                              np.maximum(table.numpy(), 0), lt.numpy(), window=window)
    got = host_f64(o)
    assert_close(got, ref, BF16_MAX, BF16_MEAN, what=f"decode paged {case[:6]} window {window}")
    for b, n in enumerate(lens):
        if n == 0:
            assert (got[b] == 0).all()


def test_decode_paged_window_never_reads_rows_before_the_window():
    """Rows before a sequence's window share a page (and a 32-token sub-tile)
    with the first row it sees; they hold NaN here, and must not reach the
    output (a zero probability times NaN would)."""
    B, Hq, Hkv, S_cap, D, P = 4, 8, 2, 2000, 128, 64
    lens, window = [2000, 1000, 77, 40], 50
    g = torch.Generator().manual_seed(77)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    kc = torch.randn(B, Hkv, S_cap, D, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, Hkv, S_cap, D, generator=g).to(torch.bfloat16)
    lt = torch.tensor(lens, dtype=torch.int32)
    for b, n in enumerate(lens):
        lo = max(0, n - window)
        kc[b, :, :lo] = float("nan")
        vc[b, :, :lo] = float("nan")
    kp, vp, table = wl.to_pages(kc, vc, lt, P, seed=3)
    say(f"decode paged window {window}, NaN before the window, lens={lens}")
    o = attn.decode_paged(dev(q), dev(kp), dev(vp), dev(table), dev(lt), max_len=max(lens),
                          window=window)
    ref = oracle.decode_paged(bits(q), bits(kp), bits(vp), np.maximum(table.numpy(), 0),
                              lt.numpy(), window=window)
    assert_close(host_f64(o), ref, BF16_MAX, BF16_MEAN, what="decode paged window NaN before")


GRAPH_CASES = [  # B, Hq, Hkv, S_cap, D, paged page size (0: contiguous), window
    (4, 32, 8, 6000, 128, 0, 0),      # few groups: several split workgroups each
    (32, 32, 8, 8192, 128, 0, 0),     # the gqa_decode geometry
    (3, 16, 2, 9000, 64, 256, 0),
    (3, 16, 2, 9000, 128, 128, 3000),
]


@pytest.mark.parametrize("case", GRAPH_CASES)
def test_decode_in_a_captured_graph_matches_oracle_on_every_replay(case):
    """One decode call captured in a HIP graph and replayed with new queries
    and lengths written into its input buffers between replays (and eager
    decode calls on the same workspace in between): every replay must match
    the oracle, and a replay on unchanged inputs must repeat its result."""
    B, Hq, Hkv, S_cap, D, P, window = case
    theta = 5e5
    g = torch.Generator().manual_seed(1000 + B + P)
    kc = torch.randn(B, Hkv, S_cap, D, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, Hkv, S_cap, D, generator=g).to(torch.bfloat16)
    full = torch.full((B,), S_cap, dtype=torch.int32)
    if P:
        kp, vp, table = wl.to_pages(kc, vc, full, P, seed=4)
        kd, vd, tb = dev(kp), dev(vp), dev(table)
    else:
        kd, vd = dev(kc), dev(vc)
    qd = torch.zeros(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    ld = torch.zeros(B, dtype=torch.int32, device=DEV)
    od = torch.zeros(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    ws = torch.full((attn.decode_workspace_size(B, Hq, Hkv, S_cap, D),), 0xA5, dtype=torch.uint8,
                    device=DEV)

    def call(q_, l_, out_):
        if P:
            return attn.decode_paged(q_, kd, vd, tb, l_, max_len=S_cap, window=window,
                                     rope_theta=theta, out=out_, workspace=ws)
        return attn.decode(q_, kd, vd, l_, max_len=S_cap, rope_theta=theta, out=out_,
                           workspace=ws)

    def expect(q, lens):
        rq = oracle.round_bf16(oracle.rope(bits(q)[:, :, None, :], theta, lens.numpy() - 1))[:, :, 0]
        if P:
            return oracle.decode_paged(rq, bits(kp), bits(vp), table.numpy(), lens.numpy(),
                                       window=window)
        return oracle.decode(rq, bits(kc), bits(vc), lens.numpy())

    say(f"decode graph capture {case}")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(qd, ld, od)
    torch.cuda.synchronize()
    prev = None
    for r in range(4):
        gg = torch.Generator().manual_seed(2000 + r)
        q = torch.randn(B, Hq, D, generator=gg).to(torch.bfloat16)
        lens = torch.randint(max(1, S_cap // 3), S_cap + 1, (B,), generator=gg, dtype=torch.int32)
        if r == 3:   # unchanged inputs: the replay must repeat the previous result
            q, lens = prev_q, prev_lens
        qd.copy_(dev(q))
        ld.copy_(dev(lens))
        graph.replay()
        torch.cuda.synchronize()
        got = od.clone()
        if r == 3:
            assert torch.equal(got, prev)
        else:
            assert_close(host_f64(got), expect(q, lens), BF16_MAX, BF16_MEAN,
                         what=f"graph replay {r} {case}")
        prev, prev_q, prev_lens = got, q, lens
        # eager work on the same workspace between replays, with other lengths
        eager_lens = torch.full((B,), S_cap - 7 * (r + 1), dtype=torch.int32)
        eager = call(dev(q), dev(eager_lens), torch.empty_like(od))
        torch.cuda.synchronize()
        if r == 0:
            assert_close(host_f64(eager), expect(q, eager_lens), BF16_MAX, BF16_MEAN,
                         what=f"eager between replays {case}")


def test_decode_paged_in_order_equals_contiguous_decode_bitwise():
    """The gqa_decode workload laid out as 256-token pages in order: the
    paged path reads the same rows in the same split, so it agrees bitwise."""
    w = wl.WORKLOADS["gqa_decode"]
    q, kc, vc, lens = wl.make_decode(w, seed=0)
    B, Hkv, S, D = kc.shape
    P = 256
    kp = kc.reshape(B, Hkv, S // P, P, D).permute(0, 2, 1, 3, 4).contiguous().reshape(-1, Hkv, P, D)
    vp = vc.reshape(B, Hkv, S // P, P, D).permute(0, 2, 1, 3, 4).contiguous().reshape(-1, Hkv, P, D)
    table = torch.arange(B * (S // P), dtype=torch.int32).reshape(B, S // P)
    say("decode paged in order vs contiguous, gqa_decode")
    ld = dev(lens)
    cont = attn.decode(dev(q), dev(kc), dev(vc), ld, rope_theta=w.theta)
    paged = attn.decode_paged(dev(q), dev(kp), dev(vp), dev(table), ld, rope_theta=w.theta)
    assert torch.equal(cont, paged)


def test_decode_paged_fused_rope_equals_separate_rope():
    B, Hq, Hkv, S_cap, D, P = 3, 16, 2, 700, 128, 64
    g = torch.Generator().manual_seed(5)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    kc = torch.randn(B, Hkv, S_cap, D, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, Hkv, S_cap, D, generator=g).to(torch.bfloat16)
    lt = torch.tensor([700, 65, 1], dtype=torch.int32)
    kp, vp, table = wl.to_pages(kc, vc, lt, P, seed=9)
    ld, tb = dev(lt), dev(table)
    say("decode paged fused RoPE vs separate, window 100")
    qr = attn.rope(dev(q).unsqueeze(2), 5e5, ld, pos_shift=-1).squeeze(2)
    sep = attn.decode_paged(qr, dev(kp), dev(vp), tb, ld, window=100)
    fused = attn.decode_paged(dev(q), dev(kp), dev(vp), tb, ld, window=100, rope_theta=5e5)
    assert torch.equal(sep, fused)


def test_decode_ignores_workspace_contents_and_default_max_len():
    B, Hq, Hkv, S_cap, D = 3, 8, 2, 600, 128
    q, kc, vc = rand_bf16((B, Hq, D), 20), rand_bf16((B, Hkv, S_cap, D), 21), rand_bf16((B, Hkv, S_cap, D), 22)
    lens = torch.tensor([600, 5, 300], dtype=torch.int32)
    need = attn.decode_workspace_size(B, Hq, Hkv, S_cap, D)
    ws = torch.full((need // 4,), float("nan"), device=DEV)
    say("decode NaN workspace")
    o1 = attn.decode(dev(q), dev(kc), dev(vc), dev(lens), workspace=ws)
    o2 = attn.decode(dev(q), dev(kc), dev(vc), dev(lens), max_len=600)
    assert torch.equal(o1, o2)
    ref = oracle.decode(bits(q), bits(kc), bits(vc), lens.numpy())
    assert_close(host_f64(o1), ref, BF16_MAX, BF16_MEAN, what="decode ws")


def test_decode_reuses_a_workspace_across_calls():
    """Completion counters left in the workspace by earlier calls (or any
    bytes at all) must not disturb a later call, including one with other
    lengths on the same buffer."""
    B, Hq, Hkv, S_cap, D = 3, 16, 4, 12000, 128
    q, kc, vc = rand_bf16((B, Hq, D), 50), rand_bf16((B, Hkv, S_cap, D), 51), rand_bf16((B, Hkv, S_cap, D), 52)
    lens_a = torch.tensor([12000, 4500, 700], dtype=torch.int32)
    lens_b = torch.tensor([9000, 12000, 4097], dtype=torch.int32)
    need = attn.decode_workspace_size(B, Hq, Hkv, S_cap, D)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    say("decode workspace reuse")
    qd, kd, vd = dev(q), dev(kc), dev(vc)
    outs_a, outs_b = [], []
    for _ in range(3):
        outs_a.append(attn.decode(qd, kd, vd, dev(lens_a), max_len=S_cap, workspace=ws))
        outs_b.append(attn.decode(qd, kd, vd, dev(lens_b), max_len=S_cap, workspace=ws))
    for o in outs_a[1:]:
        assert torch.equal(o, outs_a[0])
    for o in outs_b[1:]:
        assert torch.equal(o, outs_b[0])
    ref_a = oracle.decode(bits(q), bits(kc), bits(vc), lens_a.numpy())
    ref_b = oracle.decode(bits(q), bits(kc), bits(vc), lens_b.numpy())
    assert_close(host_f64(outs_a[0]), ref_a, BF16_MAX, BF16_MEAN, what="decode reuse a")
    assert_close(host_f64(outs_b[0]), ref_b, BF16_MAX, BF16_MEAN, what="decode reuse b")


def test_decode_matches_last_prefill_row():
    B, Hq, Hkv, S, D = 2, 8, 2, 777, 128
    q, k, v = rand_bf16((B, Hq, S, D), 30), rand_bf16((B, Hkv, S, D), 31), rand_bf16((B, Hkv, S, D), 32)
    say("decode vs prefill last row")
    pre = attn.prefill(dev(q), dev(k), dev(v))
    dec = attn.decode(dev(q[:, :, S - 1].contiguous()), dev(k), dev(v),
                      dev(torch.full((B,), S, dtype=torch.int32)))
    assert_close(host_f64(dec), host_f64(pre[:, :, S - 1]), BF16_MAX, BF16_MEAN, what="dec vs pre")


F32_DECODE_CASES = [  # B, Hq, Hkv, S_cap, D, lengths, theta
    (3, 8, 2, 1500, 128, [1500, 1, 700], 5e5),      # chunks of 512 with a ragged tail
    (2, 4, 4, 600, 64, [0, 513], 0.0),              # MHA, an empty sequence
    (1, 16, 1, 2049, 64, [2049], 1e4),              # MQA, five chunks
    (4, 32, 1, 100, 128, [1, 31, 32, 100], 5e5),    # G * D = 4096, the largest group
]


@pytest.mark.parametrize("case", F32_DECODE_CASES)
def test_decode_fp32_matches_oracle(case):
    """fp32 caches take the accuracy path (chunk partials and a merge, fp32
    throughout): within 1e-5 of the fp64 oracle, the query rotated at len - 1
    when theta > 0, a NaN-poisoned tail never read."""
    B, Hq, Hkv, S_cap, D, lens, theta = case
    g = torch.Generator().manual_seed(S_cap + D)
    q = torch.randn(B, Hq, D, generator=g)
    kc = torch.randn(B, Hkv, S_cap, D, generator=g)
    vc = torch.randn(B, Hkv, S_cap, D, generator=g)
    L = torch.tensor(lens, dtype=torch.int32)
    wl.poison_cache_tail(kc, L)
    wl.poison_cache_tail(vc, L)
    say(f"decode fp32 {case}")
    o = attn.decode(dev(q), dev(kc), dev(vc), dev(L), rope_theta=theta)
    qr = q.numpy().astype(np.float64)
    if theta > 0:
        qr = oracle.rope(q.numpy()[:, :, None, :], theta, (L.numpy() - 1))[:, :, 0, :]
    ref = oracle.decode(qr, kc.numpy().astype(np.float64), vc.numpy().astype(np.float64), L.numpy())
    got = host_f64(o)
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max()
    say(f"decode fp32 max err {err:.2e}")
    assert err <= 1e-5


def test_decode_rejects_large_fp32_groups_and_small_workspace():
    q = torch.zeros(1, 64, 128, device=DEV)
    kc = torch.zeros(1, 1, 16, 128, device=DEV)
    with pytest.raises(attn.AttnError) as e:  # G * D = 8192 is past the fp32 path
        attn.decode(q, kc, kc, torch.ones(1, dtype=torch.int32, device=DEV))
    assert e.value.status == 3
    qb, kb = q.bfloat16(), kc.bfloat16()
    with pytest.raises(attn.AttnError) as e:
        attn.decode(qb, kb, kb, torch.ones(1, dtype=torch.int32, device=DEV),
                    workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert e.value.status == 5
