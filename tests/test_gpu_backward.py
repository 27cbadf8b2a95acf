"""GPU parity of the training path: attn_prefill_lse and attn_prefill_backward,
called through the C ABI, against the fp64 CPU oracle on the same seeded bf16
inputs (marker `gpu`; needs an MI355X).

Tolerances.  The log-normaliser is checked against a per-row bound: the
forward's scores are fp32 sums of exact bf16 products (error <= 2^-16 scale
sum_d |q_d k_d| for D <= 128, with the exp2-domain FMA), and the row sum adds
bf16-rounded probabilities (relative error <= 2^-8); lse moves by no more
than the largest score error plus 2^-8.
Gradients: the GPU rounds p, ds and the forward's o (which enters delta) to
bf16, and each gradient is rounded once at the end; each is a relative error
<= 2^-8 on terms that add with random signs.  An element's error is
therefore a few 2^-8 of the size of its own gradient row (rows differ a lot in
size: a query that sees few keys has large gradients).  The bar: every
element within 2^-5 of max(rms of its row, rms of the tensor), and the mean
error within 2^-7 of the tensor's rms.  dq gets one more, separately derived allowance:
delta = <dout_i, o_i> uses the forward's bf16 o (each element within 2^-8 of
o's exact value), which moves every ds of row i by p times the same error and
so dq_i by scale |delta error| |sum_t p_t k_t|; that is at most
scale 2^-8 sum_d |dout_d o_d| |sum_t p_t k_td| per element (the p-weighted
key mean is the oracle's attention with the keys as values), and it dominates
the rows that see few keys (whose exact dq is small).  A dropped or misplaced term (wrong head, wrong
causal bound, missing delta) moves a short row by the order of its own size;
the parity cases include many short rows.
"""
import numpy as np
import pytest
import torch

import compressed_latent_causal_amd as attn
import oracle
from compressed_latent_causal_amd import workloads as wl

pytestmark = pytest.mark.gpu

GRAD_MAX, GRAD_MEAN = 2.0 ** -5, 2.0 ** -7


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    attn.lib()


def say(msg):
    print(f"[case] {msg}", flush=True)


def _bits(t):
    return wl.to_numpy_bits(t)


def _lse_bound(q, k, scale):
    """Per-row bound on |GPU lse - oracle lse| (see the module docstring)."""
    qf, kf = oracle.widen(q), oracle.widen(k)
    G = qf.shape[1] // kf.shape[1]
    kr = np.repeat(np.abs(kf), G, axis=1)
    a = np.einsum("bhid,bhtd->bhit", np.abs(qf), kr) * scale
    S = qf.shape[2]
    a = np.where(np.tril(np.ones((S, S), dtype=bool)), a, 0.0)
    return 2.0 ** -16 * a.max(axis=-1) + 2.0 ** -8 + 1e-5


def _dq_delta_allowance(q, k, v, dout, scale, rows=None):
    """Per-element bound on the dq error that the bf16 rounding of the forward's
    o brings in through delta (see the module docstring); q, k, v, dout are the
    bf16 bit arrays, rows optional flat query rows.  Shape of dq (or [rows, D])."""
    B, Hq, S, D = q.shape
    o = oracle.prefill(q, k, v, scale=scale, rows=rows)
    g = oracle.widen(dout).reshape(-1, D)
    full = rows is None
    if full:
        rows = np.arange(B * Hq * S)
        o = o.reshape(-1, D)
    g = g[rows]
    dmax = 2.0 ** -8 * np.abs(g * o).sum(-1, keepdims=True)
    kmean = oracle.prefill(q, k, k, scale=scale, rows=rows)  # sum_t p_t k_t of each row
    out = scale * dmax * np.abs(kmean.reshape(len(rows), D))
    return out.reshape(B, Hq, S, D) if full else out


def _assert_grad(got, ref, what, extra=None):
    """Elementwise error over max(row rms, tensor rms) after taking off an
    optional per-element allowance, mean error over the tensor rms (rows: the
    last axis)."""
    assert np.isfinite(got).all(), f"{what}: non-finite"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    row = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
    diff = np.abs(got - ref)
    if extra is not None:
        diff_c = np.maximum(diff - extra.reshape(diff.shape), 0.0)
    else:
        diff_c = diff
    rel = diff_c / np.maximum(row, rms)
    mx, mn = float(rel.max()), float(diff.mean()) / rms
    at = np.unravel_index(int(rel.argmax()), rel.shape)
    say(f"{what}: rms {rms:.3e}, worst err {mx:.3e} of its row scale at "
        f"{tuple(int(i) for i in at)} (row rms {float(row[at[:-1]][0]):.3e}), mean/rms {mn:.3e}")
    assert mx <= GRAD_MAX, f"{what}: element error {mx} of its row scale > {GRAD_MAX}"
    assert mn <= GRAD_MEAN, f"{what}: mean err {mn} rms units > {GRAD_MEAN}"


def _run(q, k, v, dout, scale):
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, dout))
    o, lse = attn.prefill_lse(qd, kd, vd, scale=scale)
    dq, dk, dv = attn.prefill_backward(qd, kd, vd, o, gd, lse, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu(), dq.cpu(), dk.cpu(), dv.cpu()


LSE_GEOMS = [(1, 8, 2, 200, 128), (2, 4, 1, 97, 64), (1, 4, 4, 64, 128)]


@pytest.mark.parametrize("geom", LSE_GEOMS)
def test_prefill_lse_matches_oracle(geom):
    B, Hq, Hkv, S, D = geom
    say(f"lse {geom}")
    w = wl.custom("prefill", "bf16", B, Hq, Hkv, D, S)
    q, k, v = wl.make_prefill(w, seed=11)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, lse = attn.prefill_lse(qd, kd, vd)
    o_plain = attn.prefill(qd, kd, vd)
    torch.cuda.synchronize()
    # the output is the plain forward's, bit for bit
    assert torch.equal(o.cpu(), o_plain.cpu())
    ref = oracle.prefill_lse(_bits(q), _bits(k))
    err = np.abs(lse.cpu().double().numpy() - ref)
    bound = _lse_bound(_bits(q), _bits(k), w.scale)
    say(f"lse max err {err.max():.3e}, largest bound {bound.max():.3e}, "
        f"worst err/bound {(err / bound).max():.3f}")
    assert (err <= bound).all()


BWD_GEOMS = [  # B, Hq, Hkv, S, D
    (1, 4, 2, 64, 128),
    (2, 8, 2, 100, 64),
    (1, 8, 8, 257, 128),   # MHA, ragged over several key blocks and Q tiles
    (1, 4, 1, 130, 64),    # MQA
    (2, 8, 2, 1, 128),     # one token: only dv moves
    (1, 4, 4, 17, 64),
    (1, 16, 2, 300, 128),  # G = 8
    (1, 6, 2, 96, 64),     # G = 3
    (1, 4, 2, 513, 128),   # 9 key blocks, a one-row tail
]


@pytest.mark.parametrize("geom", BWD_GEOMS)
def test_prefill_backward_matches_oracle(geom):
    B, Hq, Hkv, S, D = geom
    say(f"backward {geom}")
    w = wl.custom("prefill", "bf16", B, Hq, Hkv, D, S)
    q, k, v, dout = wl.make_backward(w, seed=12)
    _, _, dq, dk, dv = _run(q, k, v, dout, w.scale)
    rq, rk, rv = oracle.prefill_backward(_bits(q), _bits(k), _bits(v), _bits(dout))
    if S == 1:
        # p = 1 and ds = dp - delta = 0 exactly: what is left is the fp32
        # rounding of two D-term sums of the same products (<dout, v> on the
        # matrix core, <dout, o> from the forward's o = v), each within
        # D 2^-24 sum_d |dout_d v_d|; times scale |k| for dq and scale |q| for dk
        gd, vd = oracle.widen(_bits(dout)), oracle.widen(_bits(v))
        G = Hq // Hkv
        dsb = 2 * D * 2.0 ** -24 * (np.abs(gd) * np.abs(np.repeat(vd, G, axis=1))).sum(-1).max()
        assert dq.float().abs().max() <= w.scale * np.abs(oracle.widen(_bits(k))).max() * dsb
        assert dk.float().abs().max() <= G * w.scale * np.abs(oracle.widen(_bits(q))).max() * dsb
    else:
        bq, bk, bv, bg = (_bits(t) for t in (q, k, v, dout))
        _assert_grad(dq.double().numpy(), rq, "dq", _dq_delta_allowance(bq, bk, bv, bg, w.scale))
        _assert_grad(dk.double().numpy(), rk, "dk")
    _assert_grad(dv.double().numpy(), rv, "dv")


def test_prefill_backward_zero_dout_gives_zero_gradients():
    w = wl.custom("prefill", "bf16", 1, 8, 2, 64, 150)
    q, k, v, dout = wl.make_backward(w, seed=13)
    _, _, dq, dk, dv = _run(q, k, v, torch.zeros_like(dout), w.scale)
    for t in (dq, dk, dv):
        assert not t.float().abs().any()


def test_prefill_backward_is_deterministic():
    w = wl.custom("prefill", "bf16", 1, 8, 2, 128, 200)
    q, k, v, dout = wl.make_backward(w, seed=14)
    a = _run(q, k, v, dout, w.scale)
    b = _run(q, k, v, dout, w.scale)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_prefill_backward_full_size_sampled_rows():
    """llama8b_prefill (4 x 32/8 heads x 4096 x 128) in the launch
    configuration the benchmark times: dq on sampled query rows, dk/dv on
    sampled keys of two KV groups, against the oracle row by row."""
    w = wl.WORKLOADS["llama8b_prefill"]
    say("backward llama8b_prefill sampled rows")
    q, k, v, dout = wl.make_backward(w, seed=0)
    _, _, dq, dk, dv = _run(q, k, v, dout, w.scale)
    g = np.random.default_rng(3)
    S = w.S
    qr = np.concatenate([g.integers(0, w.B * w.Hq * S, 48),
                         np.array([0, S - 1, S, 64, 63, w.B * w.Hq * S - 1])])
    groups = [(0, 0), (w.B - 1, w.Hkv - 1)]
    kr = []
    for b, j in groups:
        base = (b * w.Hkv + j) * S
        kr += [base + t for t in (0, 1, 63, 64, S // 2, S - 65, S - 1)]
        kr += list(base + g.integers(0, S, 9))
    kr = np.array(kr)
    rq, rk, rv = oracle.prefill_backward(_bits(q), _bits(k), _bits(v), _bits(dout), q_rows=qr,
                                         k_rows=kr)
    allow = _dq_delta_allowance(_bits(q), _bits(k), _bits(v), _bits(dout), w.scale, rows=qr)
    _assert_grad(dq.reshape(-1, w.D)[qr].double().numpy(), rq, "dq rows", allow)
    _assert_grad(dk.reshape(-1, w.D)[kr].double().numpy(), rk, "dk rows")
    _assert_grad(dv.reshape(-1, w.D)[kr].double().numpy(), rv, "dv rows")


def test_prefill_backward_ccgqa_full_size_sampled_rows():
    """ccgqa_prefill (2 x 8/2 heads x 16384 x 64) in the launch configuration
    the benchmark times, where the dK/dV pass splits each group's 4 query heads
    over 4 workgroups per key block (32 keys per wave) and a fourth kernel sums
    their fp32 partials: sampled rows against the oracle."""
    w = wl.WORKLOADS["ccgqa_prefill"]
    say("backward ccgqa_prefill sampled rows")
    n_split = attn.prefill_backward_workspace_size(w.B, w.Hq, w.Hkv, w.S, w.D)
    stats = w.B * w.Hq * (-(-w.S // 64) * 64 + 64) * 8
    assert n_split == stats + 4 * 2 * w.B * w.Hkv * w.S * w.D * 4  # the split this test is for
    q, k, v, dout = wl.make_backward(w, seed=5)
    _, _, dq, dk, dv = _run(q, k, v, dout, w.scale)
    g = np.random.default_rng(4)
    S = w.S
    qr = np.concatenate([g.integers(0, w.B * w.Hq * S, 24),
                         np.array([0, S - 1, S, 127, 128, w.B * w.Hq * S - 1])])
    kr = []
    for b, j in [(0, 0), (w.B - 1, w.Hkv - 1)]:
        base = (b * w.Hkv + j) * S
        kr += [base + t for t in (0, 1, 127, 128, S // 2, S - 129, S - 1)]
        kr += list(base + g.integers(0, S, 5))
    kr = np.array(kr)
    rq, rk, rv = oracle.prefill_backward(_bits(q), _bits(k), _bits(v), _bits(dout), q_rows=qr,
                                         k_rows=kr)
    allow = _dq_delta_allowance(_bits(q), _bits(k), _bits(v), _bits(dout), w.scale, rows=qr)
    _assert_grad(dq.reshape(-1, w.D)[qr].double().numpy(), rq, "dq rows", allow)
    _assert_grad(dk.reshape(-1, w.D)[kr].double().numpy(), rk, "dk rows")
    _assert_grad(dv.reshape(-1, w.D)[kr].double().numpy(), rv, "dv rows")


def test_training_step_with_rope_end_to_end():
    """Forward with the query RoPE fused and K rotated by attn_rope, backward
    on the rotated q and k, then attn_rope_backward for dq and dk: the
    gradients of the unrotated q and k match the oracle's chain (its backward
    on its own rotations, then its transposed rotation)."""
    B, Hq, Hkv, S, D, theta = 1, 8, 2, 160, 128, 5e5
    w = wl.custom("prefill", "bf16", B, Hq, Hkv, D, S)
    q, k, v, dout = wl.make_backward(w, seed=15)
    say("training step with RoPE")
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, dout))
    kr = attn.rope(kd, theta)
    o, lse = attn.prefill_lse(qd, kr, vd, rope_theta=theta)
    qr = attn.rope(qd, theta)  # the rotated q the forward attended with
    dqr, dkr, dv = attn.prefill_backward(qr, kr, vd, o, gd, lse)
    dq = attn.rope_backward(dqr, theta)
    dk = attn.rope_backward(dkr, theta)
    torch.cuda.synchronize()
    # oracle chain: rotations rounded to bf16 at the same boundaries as the GPU's
    rq = oracle.round_bf16(oracle.rope(_bits(q), theta))
    rk = oracle.round_bf16(oracle.rope(_bits(k), theta))
    gq, gk, gv = oracle.prefill_backward(rq, rk, _bits(v), _bits(dout))
    ref_dq = oracle.rope_transpose(gq, theta)
    ref_dk = oracle.rope_transpose(gk, theta)
    allow = _dq_delta_allowance(rq, rk, _bits(v), _bits(dout), w.scale)
    # a rotation preserves each pair's length, so the dq allowance carries over pairwise
    pair = np.sqrt(allow[..., 0::2] ** 2 + allow[..., 1::2] ** 2)
    _assert_grad(dq.cpu().double().numpy(), ref_dq, "dq (unrotated)", np.repeat(pair, 2, axis=-1))
    _assert_grad(dk.cpu().double().numpy(), ref_dk, "dk (unrotated)")
    _assert_grad(dv.cpu().double().numpy(), gv, "dv")


def test_prefill_backward_ignores_workspace_contents():
    """The row statistics are rewritten on every call, padding rows included:
    a NaN-filled workspace and a reused one give the same gradients."""
    w = wl.custom("prefill", "bf16", 2, 8, 2, 64, 130)
    q, k, v, dout = (t.cuda() for t in wl.make_backward(w, seed=16))
    say("backward with a NaN-filled workspace")
    o, lse = attn.prefill_lse(q, k, v)
    n = attn.prefill_backward_workspace_size(w.B, w.Hq, w.Hkv, w.S, w.D)
    ws = torch.full((n // 4,), float("nan"), dtype=torch.float32, device="cuda")
    a = attn.prefill_backward(q, k, v, o, dout, lse, workspace=ws)
    b = attn.prefill_backward(q, k, v, o, dout, lse, workspace=ws)
    c = attn.prefill_backward(q, k, v, o, dout, lse)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.isfinite(x.float()).all()
        assert torch.equal(x, y) and torch.equal(x, z)


def test_prefill_lse_full_size_sampled_rows():
    """llama8b_prefill's log-normaliser on sampled rows (first, last and
    block-edge queries included) within the per-row rounding bound."""
    w = wl.WORKLOADS["llama8b_prefill"]
    say("lse llama8b_prefill sampled rows")
    q, k, v = wl.make_prefill(w, seed=0)
    _, lse = attn.prefill_lse(q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    g = np.random.default_rng(5)
    S = w.S
    rows = np.concatenate([g.integers(0, w.B * w.Hq * S, 40),
                           np.array([0, 31, 32, 63, 64, S - 1, w.B * w.Hq * S - 1])])
    ref = oracle.prefill_lse(_bits(q), _bits(k), rows=rows)
    got = lse.reshape(-1).cpu()[torch.from_numpy(rows)].double().numpy()
    qf = oracle.widen(_bits(q)).reshape(-1, w.D)[rows]
    G = w.Hq // w.Hkv
    bound = []
    for n, r in enumerate(rows):
        i, h, b = r % S, (r // S) % w.Hq, r // (S * w.Hq)
        kf = np.abs(oracle.widen(_bits(k[b, h // G, :i + 1])))
        bound.append(2.0 ** -8 * ((kf @ np.abs(qf[n])).max() * w.scale + 1.0) + 1e-5)
    err = np.abs(got - ref)
    say(f"lse rows: max err {err.max():.3e}, worst err/bound {(err / np.array(bound)).max():.3f}")
    assert (err <= np.array(bound)).all()
