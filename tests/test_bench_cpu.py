"""Host logic of bench.py (no GPU): the one-GPU rule, the algorithmic byte
counts behind the roofline entry, and when a committed counter summary is
taken as the step's measured traffic."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_step_bytes_135m_from_the_parameter_count():
    # The 135M shape holds 134,515,008 parameters: 134,479,872 in matrices
    # (the tied 49152 x 576 embedding once, 30 layers of q, k, v, o, w1, w3,
    # w2) and 35,136 norm gains.  One step at a 5-token context reads every
    # matrix once as bf16, the gains as fp32, one embedding row, the K/V rows
    # of positions 0..5 (30 layers x 2 x 3 groups x 64 fp32) and writes one
    # K/V row per layer and the 49152 fp32 logits.
    m = synth.M135
    mats, gains = 134_479_872, 35_136
    kv_row = 30 * 2 * 3 * 64 * 4
    want = 2 * mats + 4 * gains + 2 * 576 + 6 * kv_row + kv_row + 4 * 49152
    assert bench.step_bytes(m, np.array([5], np.int32)) == want == 269_620_608


def test_step_bytes_8b_untied_counts_the_head_not_the_embedding():
    # 8B shape, untied: the 32 layers' matrices (6144x4096 q/k/v, 4096x4096 o,
    # 2 x 14336x4096 w1/w3, 4096x14336 w2) and the 128256x4096 head, all bf16,
    # are 15,009,316,864 bytes; the embedding table is only gathered (one
    # 4096-element bf16 row).  Gains: 65 x 4096 fp32.  At 4096 cached
    # positions the step reads 4097 K/V rows of 32 x 2 x 8 x 128 fp32 and
    # writes one, and writes 128256 fp32 logits.
    m = synth.M8B
    assert m.tied_embeddings == 0
    kv_row = 32 * 2 * 8 * 128 * 4
    want = 15_009_316_864 + 65 * 4096 * 4 + 4096 * 2 + 4097 * kv_row + kv_row + 128256 * 4
    assert bench.step_bytes(m, np.array([4096], np.int32)) == want
    # about 16.09 GB, not the 17.14 GB the whole embedding table would add
    assert abs(want / 1e9 - 16.09) < 0.01


def test_kernel_bytes_8b():
    m = synth.M8B
    # W1 and W3: 2 x 14336 x 4096 bf16, plus the fp32 input row read twice
    # (norm and product) and the 14336-float h written
    assert bench.kernel_bytes(m, "w13", 1, 0) == 2 * 14336 * 4096 * 2 + 4096 * 4 * 2 + 14336 * 4
    # attention at 4096 cached positions: 8 groups x 128 dims x (K and V) fp32, and the queries
    assert bench.kernel_bytes(m, "attn", 1, 4096) == 2 * 8 * 128 * 4096 * 4 + 32 * 128 * 4


@pytest.mark.parametrize("kernel,workload", [("k_persist", "llama135m_p5"), ("k_attn_g", "llama135m_b64")])
def test_traffic_summary_follows_the_source_hash(monkeypatch, kernel, workload):
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    fields = dict(line.split(":", 1) for line in open(path) if line.startswith(("traffic_bytes", "kernel_sources")))
    h = fields["kernel_sources_sha256_16"].strip()
    monkeypatch.setattr(bench, "kernel_sources_hash", lambda *a: h)
    v, note = bench.measured_traffic(workload, kernel)
    assert v == float(fields["traffic_bytes_per_launch"]) and "FETCH_SIZE" in note
    monkeypatch.setattr(bench, "kernel_sources_hash", lambda *a: "0" * 16)
    assert bench.measured_traffic(workload, kernel) == (None, "kernel changed since the counters were taken")
    assert bench.measured_traffic("no_such_workload", kernel)[0] is None


def test_kernel_source_sets():
    # the single launch and the split-K attention are hashed over their own sources
    assert set(bench.KERNEL_SOURCES) == {"k_persist", "k_attn_g"}
    assert bench.kernel_sources_hash("k_persist") != bench.kernel_sources_hash("k_attn_g")
