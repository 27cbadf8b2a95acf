"""Host-side logic of bench.py (CPU only): the one-GPU exit, the algorithmic
counting rules, the guard on the recorded HBM traffic, and the shape of the
CPU-baseline record."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from compressed_latent_causal_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("B,Hq,S,D", [(1, 1, 1, 64), (2, 3, 7, 128), (4, 32, 4096, 128)])
def test_prefill_flops_count_unmasked_pairs_only(B, Hq, S, D):
    pairs = sum(i + 1 for i in range(S))  # query i sees keys 0..i
    assert bench.prefill_flops(B, Hq, S, D) == 4.0 * B * Hq * D * pairs
    # the headline workload's count, as quoted in the design notes
    if S == 4096:
        assert bench.prefill_flops(B, Hq, S, D) == 549890031616.0


def test_decode_bytes_scale_with_kv_heads_not_query_heads():
    lens = [5, 0, 1024]
    assert bench.decode_bytes(lens, Hkv=8, D=128) == 1029 * 8 * 128 * 2 * 2
    assert bench.decode_bytes(lens, Hkv=1, D=64) == 1029 * 64 * 4


def test_min_prefill_bytes_reads_q_k_v_and_writes_o_once():
    w = wl.WORKLOADS["llama8b_prefill"]
    elems_q = w.B * w.Hq * w.S * w.D
    elems_kv = w.B * w.Hkv * w.S * w.D
    assert bench.min_prefill_bytes(w) == (2 * elems_q + 2 * elems_kv) * 2


def test_recorded_traffic_is_used_only_for_the_profiled_source(tmp_path, monkeypatch):
    traffic, note = bench.profiled_traffic()
    text = open(bench.TRAFFIC_PROFILE).read()
    if traffic is not None:  # the committed summary matches the current kernel source
        assert f"traffic_bytes_per_launch: {traffic}" in text
        assert note.startswith("profiles/")
    # any change to the kernel source invalidates the recorded figure
    changed = tmp_path / "prefill.hip"
    changed.write_text(open(bench.KERNEL_SOURCES[0]).read() + "\n// changed\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(changed)] + bench.KERNEL_SOURCES[1:])
    assert bench.profiled_traffic() == (None, "kernel changed since the counters were taken")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(tmp_path / "missing.md"))
    assert bench.profiled_traffic() == (None, "no counter summary")


def test_cpu_baseline_record_on_a_small_workload():
    w = wl.custom("prefill", "bf16", 1, 4, 2, 64, 96, theta=1e4)
    r = bench.cpu_baseline(w, budget_s=0.2)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1
    n = int(r["sample"].split()[0])
    assert 0 < n <= w.B * w.Hq * w.S
    assert r["cpu_model"] == bench.cpu_model() and r["cpu_model"]


def test_cpu_baseline_decode_record_on_a_small_workload():
    w = wl.custom("decode", "bf16", 3, 8, 2, 64, 200, theta=5e5, len_lo=1, len_hi=200)
    r = bench.cpu_baseline_decode(w)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s"
    assert r["value"] > 0 and r["cores"] >= 1
    assert "3 sequences" in r["sample"]


def test_cca_bytes_read_and_write_q_k_v_once():
    w = wl.WORKLOADS["ccgqa_prefill"]
    per_tensor = lambda H: w.B * H * w.S * w.D * 2
    assert bench.cca_bytes(w) == 2 * (per_tensor(w.Hq) + 2 * per_tensor(w.Hkv))
    assert bench.cca_bytes(w) == 96 * 2 ** 20
