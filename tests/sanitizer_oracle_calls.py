"""Every oracle entry point on small inputs, edge cases included (run as a
script by tests/test_sanitizers.py, in a process whose oracle library is an
AddressSanitizer + UndefinedBehaviorSanitizer build).  numpy only: the process
loads nothing else that allocates through the sanitizer's interposed malloc.
Correctness is the pins' business; this only drives every loop bound, index
and error path of oracle.c once."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import oracle  # noqa: E402

rng = np.random.default_rng(5)


def draw(shape, dt):
    x = rng.standard_normal(shape)
    if dt == "f64":
        return x
    if dt == "f32":
        return x.astype(np.float32)
    return oracle.round_bf16(x)


def expect_error(fn, *a, **kw):
    try:
        fn(*a, **kw)
    except RuntimeError:
        return
    raise AssertionError(f"{fn.__name__} accepted a bad input")


assert oracle.num_threads() >= 1

# rounding: specials, ties, subnormals, the overflow edge
special = np.array([0.0, -0.0, 1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -24, 2.0 ** -133,
                    2.0 ** -149, 2.0 ** -150, 3.5e38, 3.4028235677973366e38, -1e300, np.inf, -np.inf,
                    np.nan])
oracle.round_bf16(special)
oracle.round_f32(special)
oracle.round_bf16(np.zeros(0))

for dt in ("f64", "f32", "bf16"):
    for B, Hq, Hkv, S, D in [(2, 6, 2, 5, 64), (1, 2, 1, 1, 128), (1, 4, 4, 33, 64)]:
        q, k, v = draw((B, Hq, S, D), dt), draw((B, Hkv, S, D), dt), draw((B, Hkv, S, D), dt)
        off = rng.integers(0, 1000, B).astype(np.int32)
        oracle.rope(q, 1e4)
        oracle.rope(k, 5e5, pos_offset=off)
        oracle.rope_transpose(q, 1e4, pos_offset=off)
        oracle.prefill(q, k, v)
        oracle.prefill(q, k, v, scale=0.0)
        rows = np.array([0, B * Hq * S - 1, S // 2], dtype=np.int64)
        oracle.prefill(q, k, v, rows=rows)
        oracle.prefill_lse(q, k)
        oracle.prefill_lse(q, k, rows=rows)
        dout = draw((B, Hq, S, D), dt)
        oracle.prefill_backward(q, k, v, dout)
        oracle.prefill_backward(q, k, v, dout, q_rows=rows,
                                k_rows=np.array([0, B * Hkv * S - 1], dtype=np.int64))
        oracle.prefill_backward(q, k, v, dout, want_dq=False)
        oracle.prefill_backward(q, k, v, dout, want_dkv=False)

# decode over a contiguous cache: empty, one, full and ragged lengths
for dt in ("f32", "bf16"):
    B, Hq, Hkv, S_cap, D = 4, 8, 2, 40, 64
    q = draw((B, Hq, D), dt)
    kc, vc = draw((B, Hkv, S_cap, D), dt), draw((B, Hkv, S_cap, D), dt)
    oracle.decode(q, kc, vc, np.array([0, 1, S_cap, 17], dtype=np.int32))

# paged cache: tables with -1 past each sequence, windows, a bad entry
B, Hq, Hkv, P, D, NP = 3, 4, 2, 8, 64, 9
q = draw((B, Hq, D), "bf16")
kp, vp = draw((NP, Hkv, P, D), "bf16"), draw((NP, Hkv, P, D), "bf16")
table = np.full((B, 4), -1, dtype=np.int32)
table[0, :3] = [4, 0, 7]
table[1, :1] = [2]
table[2, :4] = [8, 1, 3, 5]
lens = np.array([20, 0, 32], dtype=np.int32)
for window in (0, 1, 3, 8, 100):
    oracle.decode_paged(q, kp, vp, table, lens, window=window)
bad = table.copy()
bad[2, 1] = NP
expect_error(oracle.decode_paged, q, kp, vp, bad, lens)

# CCA pre-attention operations: widths 1 to 8, with and without RoPE
for dt in ("f64", "bf16"):
    for B, Hq, Hkv, S, D, W in [(2, 6, 2, 9, 64, 4), (1, 2, 2, 1, 128, 8), (1, 4, 1, 3, 64, 1)]:
        q, k, v = draw((B, Hq, S, D), dt), draw((B, Hkv, S, D), dt), draw((B, Hkv, S, D), dt)
        cq, ck = draw((Hq, W, D), dt), draw((Hkv, W, D), dt)
        mq, mk = draw((Hq, D, D), dt), draw((Hkv, D, D), dt)
        oracle.cca_mix(q, k, v, cq, ck, mq, mk)
        oracle.cca_mix(q, k, v, cq, ck, mq, mk, pos_offset=np.arange(B, dtype=np.int32) * 7,
                       theta=1e4)
        # and its backward, with gradients drawn like the inputs
        gq, gk, gv = draw((B, Hq, S, D), dt), draw((B, Hkv, S, D), dt), draw((B, Hkv, S, D), dt)
        oracle.cca_mix_backward(gq, gk, gv, q, k, cq, ck, mq, mk)
        oracle.cca_mix_backward(gq, gk, gv, q, k, cq, ck, mq, mk,
                                pos_offset=np.arange(B, dtype=np.int32) * 7, theta=1e4)

print("all oracle calls done", flush=True)
