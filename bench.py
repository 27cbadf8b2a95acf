"""Benchmark of the causal GQA attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode]
                    [--no-backward]

Headline workload: the Llama-3.1-8B-shaped prefill layer (batch 4, 32 query
heads, 8 KV heads, head dim 128, 4096 tokens, bf16, RoPE theta 5e5).  One step
is one pass of the prefill hot path over that batch: RoPE on K, then causal GQA
attention with the queries' RoPE done inside the prefill kernel.  `value` is algorithmic prefill TFLOP/s over the whole
step (4*B*Hq*D*S(S+1)/2 flops: QK^T and PV over unmasked pairs only), inputs
resident in HBM.  The `roofline` object prices the prefill kernel alone, timed
with HIP events on the stream it runs on.  The `decode` object reports KV-cache
GB/s of the two decode workloads (one decode step over several layers' caches
back to back, caches evicted before each timed step), the `backward` object the
training backward pass of both prefill workloads, and `cpu_baseline` times
the fp64 CPU oracle on a bounded sample of the same prefill workload (and on
the gqa_decode batch, and the CCA pass and its backward on ccgqa_prefill).  `prefill_ccgqa` times the compressed-latent prefill
(batch 2, 8 query heads, 2 KV heads, head dim 64, 16384 tokens) the same way
as the headline step, and `ccgqa_cca_step` the same layer with the CCA
pre-attention pass (convolutions, QK-mean, RoPE, value shift) before it.  Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill attention TFLOP/s & decode KV GB/s (1 MI355X, % of roofline)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
COPY_BYTES = 256 << 20      # calibration copy: bytes read (and written) per launch

# HBM traffic of the prefill kernel comes from rocprofv3 counter runs whose
# summary is kept under profiles/; it is used only while the kernel source is
# the one those counters were taken on.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "prefill_bf16_kernel_llama8b_prefill_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "compressed_latent_causal_amd", "csrc", f)
                  for f in ("prefill.hip", "common.hpp")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_flops(B, Hq, S, D):
    """QK^T and PV over the S(S+1)/2 unmasked (query, key) pairs of each head."""
    return 4.0 * B * Hq * D * (S * (S + 1) / 2)


def min_prefill_bytes(w, elem_bytes=2):
    """Compulsory HBM bytes of one prefill launch: read Q, K, V once, write O."""
    return float(2 * w.B * w.Hq * w.S * w.D + 2 * w.B * w.Hkv * w.S * w.D) * elem_bytes


def decode_bytes(lens, Hkv, D, elem_bytes=2):
    """Valid K and V cache bytes read for one token of every sequence."""
    return float(sum(int(n) for n in lens)) * Hkv * D * 2 * elem_bytes


def kernel_source_digest():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profiled_traffic():
    """(bytes per launch, note) from the committed counter summary, or (None,
    reason) when there is none or the kernel source changed since."""
    import re
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None, "no counter summary"
    m_sha = re.search(r"^kernel_source_sha256: ([0-9a-f]{64})$", text, re.M)
    m_b = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
    if not (m_sha and m_b):
        return None, "counter summary unreadable"
    if m_sha.group(1) != kernel_source_digest():
        return None, "kernel changed since the counters were taken"
    return int(m_b.group(1)), os.path.relpath(TRAFFIC_PROFILE, ROOT)


def settle(fn, seconds=1.0):
    """Run `fn` untimed until the GPU has been busy for `seconds`: clocks ramp
    up from idle over a fraction of a second, and the timed steps should see
    the steady state."""
    import torch
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def bench_copy(iters=20):
    """Plain device copy of COPY_BYTES (the counter calibration kernel)."""
    import torch
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    settle(lambda: dst.copy_(src), 0.3)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / iters
    return {"workload": "copy", "bytes_read_per_launch": COPY_BYTES,
            "bytes_written_per_launch": COPY_BYTES, "ms_mean": round(ms, 5),
            "GB_per_s": round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 1)}


# ---------------------------------------------------------------------------
def bench_prefill(w, steps, warmup):
    import torch
    import compressed_latent_causal_amd as attn
    from compressed_latent_causal_amd import workloads as wl

    q, k, v = wl.make_prefill(w, seed=0)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    del q, k, v
    kr, o = torch.empty_like(kd), torch.empty_like(qd)
    stream = torch.cuda.current_stream()

    def step(ev=None):  # RoPE of the queries is fused into the prefill kernel
        attn.rope(kd, w.theta, out=kr)
        if ev is not None:
            ev[0].record(stream)
        attn.prefill(qd, kr, vd, w.scale, out=o, rope_theta=w.theta)
        if ev is not None:
            ev[1].record(stream)

    settle(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    return wall * 1e3 / steps, sum(kern_ms) / len(kern_ms), sorted(kern_ms)


def bench_decode(w, iters, warmup, layers, page_size=0):
    """One decode step of a `layers`-layer model: the same call on `layers`
    distinct KV caches back to back (as a serving step walks its layers), the
    whole group timed with HIP events.  Together the caches far exceed the
    L2 and memory-side caches, and a 1 GiB read before every timed group evicts
    them too, so every layer reads its cache from HBM.  page_size > 0 lays each
    cache out as pages of that many tokens in a shuffled physical order and
    runs the paged entry point."""
    import torch
    import compressed_latent_causal_amd as attn
    from compressed_latent_causal_amd import workloads as wl

    q, kc, vc, lens = wl.make_decode(w, seed=0)
    qd, ld = q.cuda(), lens.cuda()
    if page_size:
        kc, vc, table = wl.to_pages(kc, vc, lens, page_size, seed=1, spare_pages=0)
        tb = table.cuda()
    kcs = [kc.cuda() for _ in range(layers)]  # same values, distinct memory
    vcs = [vc.cuda() for _ in range(layers)]
    del kc, vc
    o = torch.empty(w.B, w.Hq, w.D, dtype=qd.dtype, device="cuda")
    ws = torch.empty(attn.decode_workspace_size(w.B, w.Hq, w.Hkv, w.S, w.D), dtype=torch.uint8,
                     device="cuda")
    # Reading 1 GiB evicts the caches with clean lines (a write flush would
    # leave dirty lines whose write-back would land inside the timed region).
    flush = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():  # RoPE of the new query is fused into the decode kernel
        for l in range(layers):
            if page_size:
                attn.decode_paged(qd, kcs[l], vcs[l], tb, ld, max_len=w.S, scale=w.scale,
                                  rope_theta=w.theta, out=o, workspace=ws)
            else:
                attn.decode(qd, kcs[l], vcs[l], ld, max_len=w.S, scale=w.scale,
                            rope_theta=w.theta, out=o, workspace=ws)

    settle(step, 0.5)
    for _ in range(warmup):
        step()
    ms = []
    for _ in range(iters):
        torch.cuda.synchronize()
        # The eviction read (about 0.27 ms of GPU work) stays queued ahead of
        # the timed group, so the host enqueues the group's calls while it
        # runs and the first decode launch does not wait on the host.
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b) / layers)
    ms.sort()
    med = ms[len(ms) // 2]
    nbytes = decode_bytes(lens.tolist(), w.Hkv, w.D)
    gbs = nbytes / (med * 1e-3) / 1e9
    return {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
            "head_dim": w.D, "cache_capacity": w.S,
            "cache": f"paged, {page_size}-token pages in shuffled order" if page_size else "contiguous",
            "sum_len": int(lens.sum()),
            "kv_bytes_per_layer": nbytes, "layers": layers, "ms_per_layer_median": round(med, 5),
            "ms_per_layer_min": round(ms[0], 5), "GB_per_s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "iters": iters,
            "step": "one fused decode launch per layer (query RoPE at len-1, split-K, merge)"}


def bench_backward(w, iters, warmup):
    """The backward pass of one prefill layer (attn_prefill_backward: row
    statistics, dK/dV and dQ kernels) on the forward's o and lse, inputs
    resident, each call timed with HIP events on its stream.  TFLOP/s counts
    the five products of the backward over unmasked pairs (2.5x the forward's
    count); the kernels execute seven (S and dP are formed in both the dK/dV
    and the dQ kernel)."""
    import torch
    import compressed_latent_causal_amd as attn
    from compressed_latent_causal_amd import workloads as wl

    q, k, v, dout = (t.cuda() for t in wl.make_backward(w, seed=0))
    o, lse = attn.prefill_lse(q, k, v, scale=w.scale)
    ws = torch.empty(attn.prefill_backward_workspace_size(w.B, w.Hq, w.Hkv, w.S, w.D), dtype=torch.uint8,
                     device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream()

    def step():
        attn.prefill_backward(q, k, v, o, dout, lse, scale=w.scale, dq=dq, dk=dk, dv=dv,
                              workspace=ws)

    settle(step, 0.5)
    for _ in range(warmup):
        step()
    # Calls run back to back, each between its own pair of events, with one
    # synchronisation at the end: the queue stays ahead of the GPU, so no
    # call's time includes the host's launch latency.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    ms.sort()
    med = ms[len(ms) // 2]
    flops = 2.5 * prefill_flops(w.B, w.Hq, w.S, w.D)
    tf = flops / (med * 1e-3) / 1e12
    return {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
            "head_dim": w.D, "seq_len": w.S, "ms_median": round(med, 5), "ms_min": round(ms[0], 5),
            "TFLOP_per_s": round(tf, 1), "frac_of_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "flop_counted": flops, "iters": iters,
            "step": "attn_prefill_backward: dq, dk, dv from q, k, v, o, dout, lse (bf16)"}


DECODE_LAYERS = {"gqa_decode": 4, "long_decode": 8}  # 4 GiB of caches either way
# (reported name, workload, page size): the paged line reads the gqa workload's
# cache through 256-token pages
DECODE_LINES = [("gqa_decode", "gqa_decode", 0), ("long_decode", "long_decode", 0),
                ("gqa_decode_paged256", "gqa_decode", 256)]


def prefill_line(w, steps, warmup):
    """The prefill step of workload w (RoPE of K, then the prefill kernel with
    the query RoPE fused), timed as the headline step is; reported beside it."""
    flops = prefill_flops(w.B, w.Hq, w.S, w.D)
    ms_step, ms_kern, kern_sorted = bench_prefill(w, steps, warmup)
    tk = flops / (ms_kern * 1e-3) / 1e12
    return {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
            "head_dim": w.D, "seq_len": w.S, "rope_theta": w.theta,
            "kernel": f"prefill_bf16_kernel<{w.D},4,2>", "flop_per_launch": flops,
            "kernel_ms_mean": round(ms_kern, 5), "kernel_ms_min": round(kern_sorted[0], 5),
            "TFLOP_per_s": round(tk, 1), "frac_of_mfma_peak": round(tk / PEAK_BF16_TFLOPS, 4),
            "ms_per_step": round(ms_step, 5),
            "step_TFLOP_per_s": round(flops / (ms_step * 1e-3) / 1e12, 1), "steps": steps,
            "step": "rope(K) + causal GQA prefill with the query RoPE fused"}


def cca_bytes(w):
    """Algorithmic HBM bytes of the CCA pre-attention pass: q, k and v read
    once and written once (bf16); the per-head weights are negligible."""
    return float(2 * 2 * w.B * w.S * w.D * (w.Hq + 2 * w.Hkv))


def cca_backward_bytes(w):
    """Algorithmic HBM bytes of the CCA backward: the gradients gq, gk, gv and
    the latent q~, k~ read once, dq~, dk~, dv~ written once (bf16); the
    weights and their fp32 gradients are negligible."""
    return float(2 * w.B * w.S * w.D * (2 * (w.Hq + 2 * w.Hkv) + w.Hq + w.Hkv))


def bench_cca_step(w, steps, warmup):
    """The compressed-latent layer's attention step: the CCA pre-attention
    pass (causal sequence convolution, channel mix, QK-mean, RoPE of q and k,
    value shift), then causal GQA prefill on its outputs.  Each kernel is
    timed with HIP events on the stream it runs on."""
    import torch
    import compressed_latent_causal_amd as attn
    from compressed_latent_causal_amd import workloads as wl

    ins = [t.cuda() for t in wl.make_cca(w, seed=0)]
    qo, ko, vo = torch.empty_like(ins[0]), torch.empty_like(ins[1]), torch.empty_like(ins[2])
    o = torch.empty_like(ins[0])
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        attn.cca_mix(*ins, rope_theta=w.theta, q_out=qo, k_out=ko, v_out=vo)
        if ev is not None:
            ev[1].record(stream)
        attn.prefill(qo, ko, vo, w.scale, out=o)
        if ev is not None:
            ev[2].record(stream)

    settle(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mix_ms = sum(a.elapsed_time(b) for a, b, _ in evs) / steps
    pre_ms = sum(b.elapsed_time(c) for _, b, c in evs) / steps
    flops = prefill_flops(w.B, w.Hq, w.S, w.D)
    gbs = cca_bytes(w) / (mix_ms * 1e-3) / 1e9
    ms_step = wall * 1e3 / steps

    # the decode step's counterpart: one new token for each of 32 sequences
    # of the same geometry, at token indices drawn from 1024..8192
    Bd, Wd = 32, wl.CCA_CONV_WIDTH
    g = torch.Generator().manual_seed(0)
    qd = torch.randn(Bd, w.Hq, w.D, generator=g).to(torch.bfloat16).cuda()
    kd = torch.randn(Bd, w.Hkv, w.D, generator=g).to(torch.bfloat16).cuda()
    vd = torch.randn(Bd, w.Hkv, w.D, generator=g).to(torch.bfloat16).cuda()
    tok = torch.randint(1024, 8193, (Bd,), generator=g, dtype=torch.int32).cuda()
    qs = torch.randn(Bd, w.Hq, Wd - 1, w.D, generator=g).to(torch.bfloat16).cuda()
    ks = torch.randn(Bd, w.Hkv, Wd - 1, w.D, generator=g).to(torch.bfloat16).cuda()
    vs = torch.randn(Bd, w.Hkv, w.D, generator=g).to(torch.bfloat16).cuda()
    douts = [torch.empty_like(x) for x in (qd, kd, vd)]

    def dstep():
        attn.cca_mix_decode(qd, kd, vd, *ins[3:], tok, qs, ks, vs, rope_theta=w.theta,
                            q_out=douts[0], k_out=douts[1], v_out=douts[2])

    # 100 steps captured in a HIP graph and replayed, so the time is the GPU's
    # and not the host's per-call overhead (the step itself is a few us)
    for _ in range(20):
        dstep()
    torch.cuda.synchronize()
    graph, gs = torch.cuda.CUDAGraph(), torch.cuda.Stream()
    with torch.cuda.stream(gs):
        with torch.cuda.graph(graph, stream=gs):
            for _ in range(100):
                dstep()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    dec_us = e0.elapsed_time(e1) / 100 * 1e3

    # the backward of the pass, given gradients of its outputs
    grads = [t.cuda() for t in wl.make_cca_grads(w, seed=1)]
    bws = torch.empty(attn.cca_mix_backward_workspace_size(w.B, w.Hq, w.Hkv, w.S, w.D,
                                                           wl.CCA_CONV_WIDTH),
                      dtype=torch.uint8, device="cuda")

    def bstep():
        attn.cca_mix_backward(*grads, ins[0], ins[1], *ins[3:], rope_theta=w.theta, workspace=bws)

    for _ in range(warmup + 2):
        bstep()
    torch.cuda.synchronize()
    bevs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(steps)]
    for i in range(steps):
        bevs[i][0].record(stream)
        bstep()
        bevs[i][1].record(stream)
    torch.cuda.synchronize()
    bwd_ms = sum(a.elapsed_time(b) for a, b in bevs) / steps
    bwd_gbs = cca_backward_bytes(w) / (bwd_ms * 1e-3) / 1e9

    # a whole training step of the attention block: the pass and the prefill
    # with its log-normaliser, then the prefill backward on a loss gradient
    # (N(0, 1), like the pass's output gradients above) and the pass's
    # backward on the gradients it returns
    dout = grads[0]
    lse = torch.empty(w.B, w.Hq, w.S, dtype=torch.float32, device="cuda")
    gqo, gko, gvo = torch.empty_like(qo), torch.empty_like(ko), torch.empty_like(vo)
    pws = torch.empty(max(1, attn.prefill_backward_workspace_size(w.B, w.Hq, w.Hkv, w.S, w.D)),
                      dtype=torch.uint8, device="cuda")

    def tstep():
        attn.cca_mix(*ins, rope_theta=w.theta, q_out=qo, k_out=ko, v_out=vo)
        attn.prefill_lse(qo, ko, vo, w.scale, out=o, lse=lse)
        attn.prefill_backward(qo, ko, vo, o, dout, lse, w.scale, dq=gqo, dk=gko, dv=gvo, workspace=pws)
        attn.cca_mix_backward(gqo, gko, gvo, ins[0], ins[1], *ins[3:], rope_theta=w.theta, workspace=bws)

    for _ in range(warmup + 2):
        tstep()
    torch.cuda.synchronize()
    tevs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(steps)]
    for i in range(steps):
        tevs[i][0].record(stream)
        tstep()
        tevs[i][1].record(stream)
    torch.cuda.synchronize()
    train_ms = sum(a.elapsed_time(b) for a, b in tevs) / steps
    # products of the step: QK^T and PV forward, five in the backward (S, dP,
    # dV, dK, dQ), each 2 D flop per unmasked pair
    train_flops = prefill_flops(w.B, w.Hq, w.S, w.D) * 7 / 2
    return {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
            "head_dim": w.D, "seq_len": w.S, "rope_theta": w.theta,
            "conv_width": wl.CCA_CONV_WIDTH,
            "cca_mix_ms_mean": round(mix_ms, 5), "cca_mix_bytes": cca_bytes(w),
            "cca_mix_GB_per_s": round(gbs, 1), "cca_mix_frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "prefill_ms_mean": round(pre_ms, 5),
            "prefill_TFLOP_per_s": round(flops / (pre_ms * 1e-3) / 1e12, 1),
            "ms_per_step": round(ms_step, 5),
            "step_TFLOP_per_s": round(flops / (ms_step * 1e-3) / 1e12, 1), "steps": steps,
            "step": "CCA pre-attention pass (conv, channel mix, QK-mean, RoPE, value shift) + "
                    "causal GQA prefill",
            "cca_backward_ms_mean": round(bwd_ms, 5), "cca_backward_bytes": cca_backward_bytes(w),
            "cca_backward_GB_per_s": round(bwd_gbs, 1),
            "cca_backward": "attn_cca_mix_backward: input gradients (bf16) and weight gradients "
                            "(fp32, summed over the batch and tokens) of the pass, three kernels",
            "train_step_ms_mean": round(train_ms, 5),
            "train_step_TFLOP_per_s": round(train_flops / (train_ms * 1e-3) / 1e12, 1),
            "train_step": "attn_cca_mix, attn_prefill_lse, attn_prefill_backward, attn_cca_mix_backward "
                          "(TFLOP/s of the 2 forward and 5 backward attention products)",
            "cca_decode_step_us": round(dec_us, 2),
            "cca_decode_step": f"attn_cca_mix_decode: one new token for each of {Bd} sequences "
                               f"(token indices 1024..8192), 100 steps replayed from a HIP graph"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_decode(w):
    """The oracle's decode (fp64 C, OpenMP over (sequence, head) rows) on the
    whole batch of a decode workload, in GB/s of the same KV-cache bytes the
    GPU line counts."""
    import oracle
    from compressed_latent_causal_amd import workloads as wl

    q, kc, vc, lens = wl.make_decode(w, seed=0)
    qb, kb, vb = (wl.to_numpy_bits(t) for t in (q, kc, vc))
    t0 = time.perf_counter()
    oracle.decode(qb, kb, vb, lens.numpy(), scale=w.scale)
    el = time.perf_counter() - t0
    nbytes = decode_bytes(lens.tolist(), w.Hkv, w.D)
    return {"value": nbytes / el / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"the whole {w.name} batch ({w.B} sequences, {int(lens.sum())} cached tokens), "
                      f"{el:.2f} s wall"}


def cpu_baseline_cca(w):
    """The oracle's CCA pre-attention pass and its backward (fp64 C, OpenMP
    over heads) on the whole workload, in GB/s of the same algorithmic bytes
    the GPU lines count."""
    import oracle
    from compressed_latent_causal_amd import workloads as wl

    ins = [wl.to_numpy_bits(t) for t in wl.make_cca(w, seed=0)]
    grads = [wl.to_numpy_bits(t) for t in wl.make_cca_grads(w, seed=1)]
    t0 = time.perf_counter()
    oracle.cca_mix(*ins, theta=w.theta)
    t1 = time.perf_counter()
    oracle.cca_mix_backward(*grads, ins[0], ins[1], *ins[3:], theta=w.theta)
    t2 = time.perf_counter()
    return {"pass": {"value": cca_bytes(w) / (t1 - t0) / 1e9, "unit": "GB/s"},
            "backward": {"value": cca_backward_bytes(w) / (t2 - t1) / 1e9, "unit": "GB/s"},
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the whole {w.name} workload, {t1 - t0:.2f} s and {t2 - t1:.2f} s wall"}


def cpu_baseline(w, budget_s=15.0):
    """The oracle (fp64 C, OpenMP) on a random sample of output rows of the
    same prefill workload: RoPE of all keys and of the sampled queries, then
    attention for those rows.  Rows are drawn without repetition in random
    order (so the sample's mean causal length is that of the whole job) until
    the time budget is spent or every row is done; throughput is reported in
    TFLOP/s of the same algorithmic count."""
    import numpy as np
    import oracle
    from compressed_latent_causal_amd import workloads as wl

    q, k, v = wl.make_prefill(w, seed=0)
    qb, kb, vb = (wl.to_numpy_bits(t) for t in (q, k, v))
    rng = np.random.default_rng(0)
    n_total = w.B * w.Hq * w.S
    order = rng.permutation(n_total)  # rows without repetition, in random order
    n_rows, flops, elapsed = 0, 0.0, 0.0
    batch = 64
    rq_full = np.zeros((n_total, w.D), dtype=np.uint16)
    t_start = time.perf_counter()
    rk = oracle.round_bf16(oracle.rope(kb, w.theta))
    while elapsed < budget_s and n_rows < n_total:
        rows = order[n_rows:n_rows + batch]
        batch = len(rows)
        qsel = qb.reshape(-1, w.D)[rows].reshape(-1, 1, 1, w.D)
        rq = oracle.round_bf16(oracle.rope(qsel, w.theta, (rows % w.S).astype(np.int32)))
        rq_full[rows] = rq.reshape(-1, w.D)
        oracle.prefill(rq_full.reshape(w.B, w.Hq, w.S, w.D), rk, vb, scale=w.scale, rows=rows)
        n_rows += batch
        flops += float(np.sum(4.0 * w.D * ((rows % w.S) + 1)))
        elapsed = time.perf_counter() - t_start
        batch = min(batch * 2, 4096)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{n_rows} randomly drawn distinct output rows of {w.name} (of {n_total}), "
                      f"RoPE of all keys included, {elapsed:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-iters", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--only", choices=["prefill", "gqa_decode", "long_decode", "gqa_decode_paged256",
                                       "ccgqa_prefill", "ccgqa_cca", "backward_llama8b_prefill",
                                       "backward_ccgqa_prefill", "copy"],
                    help="time one workload alone and print its line (profiling runs; `copy` is "
                         "the plain copy that calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the attention path is built and timed on a single "
              "MI355X (no sharding or collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import compressed_latent_causal_amd as attn
    from compressed_latent_causal_amd import workloads as wl

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    attn.lib()

    if args.only == "copy":
        print(json.dumps(bench_copy()), flush=True)
        return
    if args.only == "ccgqa_cca":
        print(json.dumps(bench_cca_step(wl.WORKLOADS["ccgqa_prefill"], args.steps, args.warmup)),
              flush=True)
        return
    if args.only and args.only.startswith("backward_"):
        b = bench_backward(wl.WORKLOADS[args.only[len("backward_"):]], args.steps, args.warmup)
        print(json.dumps(b), flush=True)
        return
    lines = {name: (wname, page) for name, wname, page in DECODE_LINES}
    if args.only in lines:
        wname, page = lines[args.only]
        d = bench_decode(wl.WORKLOADS[wname], args.decode_iters, args.warmup,
                         DECODE_LAYERS[wname], page)
        print(json.dumps(d), flush=True)
        return
    w = wl.WORKLOADS["ccgqa_prefill" if args.only == "ccgqa_prefill" else "llama8b_prefill"]
    flops = prefill_flops(w.B, w.Hq, w.S, w.D)
    log(f"prefill {w.name}: {flops:.4e} flop per step")
    ms_step, ms_kern, kern_sorted = bench_prefill(w, args.steps, args.warmup)
    tflops_step = flops / (ms_step * 1e-3) / 1e12
    tflops_kern = flops / (ms_kern * 1e-3) / 1e12
    log(f"step {ms_step:.4f} ms ({tflops_step:.1f} TFLOP/s); prefill kernel mean {ms_kern:.4f} ms "
        f"({tflops_kern:.1f} TFLOP/s), min {kern_sorted[0]:.4f} max {kern_sorted[-1]:.4f}")

    result = {
        "metric": METRIC, "value": round(tflops_step, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "seq_len": w.S, "rope_theta": w.theta, "causal": True,
                   "step": "rope(K) + causal GQA prefill with the query RoPE fused"},
        "roofline": {"bound": "mfma", "kernel": "prefill_bf16_kernel<128,4,2>",
                     "achieved": round(tflops_kern, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops_kern / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel_ms_mean": round(ms_kern, 5),
                     "flop_per_launch": flops},
    }
    if w.name == "llama8b_prefill":
        traffic, note = profiled_traffic()
        result["roofline"]["traffic"] = traffic
        result["roofline"]["traffic_source"] = note
        if traffic:
            result["roofline"]["traffic_over_min_bytes"] = round(traffic / min_prefill_bytes(w), 3)
    if args.only:
        print(json.dumps(result), flush=True)
        return
    # the compressed-latent prefill at 16k tokens, timed the same way
    cc = prefill_line(wl.WORKLOADS["ccgqa_prefill"], args.steps, args.warmup)
    log(f"prefill ccgqa_prefill: kernel mean {cc['kernel_ms_mean']:.4f} ms "
        f"({cc['TFLOP_per_s']:.1f} TFLOP/s), step {cc['ms_per_step']:.4f} ms")
    result["prefill_ccgqa"] = cc
    ca = bench_cca_step(wl.WORKLOADS["ccgqa_prefill"], args.steps, args.warmup)
    log(f"ccgqa with the CCA pass: mix {ca['cca_mix_ms_mean']:.4f} ms ({ca['cca_mix_GB_per_s']:.0f} GB/s), "
        f"prefill {ca['prefill_ms_mean']:.4f} ms, step {ca['ms_per_step']:.4f} ms; "
        f"decode step {ca['cca_decode_step_us']:.1f} us; backward {ca['cca_backward_ms_mean']:.4f} ms "
        f"({ca['cca_backward_GB_per_s']:.0f} GB/s); training step {ca['train_step_ms_mean']:.4f} ms "
        f"({ca['train_step_TFLOP_per_s']:.0f} TFLOP/s)")
    result["ccgqa_cca_step"] = ca
    if not args.no_decode:
        dec = {}
        for name, wname, page in DECODE_LINES:
            d = bench_decode(wl.WORKLOADS[wname], args.decode_iters, 3, DECODE_LAYERS[wname], page)
            log(f"decode {name}: {d['ms_per_layer_median']:.4f} ms per layer, {d['GB_per_s']:.0f} GB/s")
            dec[name] = d
        result["decode"] = dec
    if not args.no_backward:
        bwd = {}
        for name in ("llama8b_prefill", "ccgqa_prefill"):
            b = bench_backward(wl.WORKLOADS[name], args.steps, 3)
            log(f"backward {name}: {b['ms_median']:.4f} ms, {b['TFLOP_per_s']:.0f} TFLOP/s")
            bwd[name] = b
        result["backward"] = bwd
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
        if not args.no_decode:
            result["cpu_baseline"]["decode"] = cpu_baseline_decode(wl.WORKLOADS["gqa_decode"])
        result["cpu_baseline"]["cca"] = cpu_baseline_cca(wl.WORKLOADS["ccgqa_prefill"])
        log(f"cpu baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
