"""Host-side pieces of bench.py's measurement contract (no GPU needed): the one-GPU guard,
the algorithmic byte and ALU-slot counts the roofline divides by, and the rule that a
counter-measured traffic figure is reported only while the kernel's sources are the ones it
was measured on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from gen import workload  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_forward_algorithmic_bytes():
    """x, Δraw, z in bf16 (2 bytes), y float32, B and C bf16, A, D, dt_bias float32."""
    w = workload("c2")
    B, L, D, N = w.batch, w.seqlen, w.dim, w.dstate
    want = 3 * B * L * D * 2 + B * L * D * 4 + 2 * B * N * L * 2 + D * N * 4 + 2 * D * 4
    assert bench.min_bytes(w, 2) == want == 840_278_016
    # a Δraw shared by the channels replaces its [B, D, L] read by [B, L]
    assert bench.min_bytes(w, 2, True) == want - B * L * D * 2 + B * L * 2


def test_alu_slot_counts():
    """118 slots per element for the gated bf16 forward at N = 16 with a general A (6 per
    state element plus 22 per element), 166 with the exact hold; with A = -(n+1) each Ā is one
    product of the previous one and e^{-δ} (4 per state element, 3 per element for e^{-δ}).
    The gated bf16 backward: 17 per state element (15 with A = -(n+1), plus e^{-δ}; 30 with the
    exact hold) plus 32 per element (18, the gate's 11, three bf16 widenings)."""
    c2, c3, c4 = workload("c2"), workload("c3"), workload("c4")
    assert bench.alu_slots_per_elem(c2) == 16 * 6 + 22 == 118
    assert bench.alu_slots_per_elem(c2, 1) == 16 * 9 + 22 == 166
    assert bench.alu_slots_per_elem(c3) == 16 * 4 + 3 + 13 == 80
    assert bench.alu_slots_per_elem(c4) == 16 * 4 + 3 + 22 == 89
    assert bench.bwd_alu_slots_per_elem(c4) == 15 * 16 + 3 + 32 == 275
    assert bench.bwd_alu_slots_per_elem(c4, 1) == 30 * 16 + 32 == 512
    assert bench.alu_slots_per_elem(c4) + bench.bwd_alu_slots_per_elem(c4) == 364
    assert bench.alu_slots_per_elem(c4, 1) + bench.bwd_alu_slots_per_elem(c4, 1) == 678


def test_traffic_only_for_the_measured_sources(monkeypatch):
    w = workload("c2")
    entry = dict(bench.MEASURED_TRAFFIC[("c2", 0)])
    want = bench.FETCH_SCALE * entry["fetch_kib"] * 1024 + bench.WRITE_SCALE * entry["write_kib"] * 1024
    # sources hashing to the recorded value: the figure is reported
    entry["sources_sha256"] = bench.sources_sha256(entry["sources"])
    monkeypatch.setitem(bench.MEASURED_TRAFFIC, ("c2", 0), entry)
    assert bench.measured_traffic(w) == pytest.approx(want)
    # any other source text: null
    stale = dict(entry, sources_sha256="0" * 64)
    monkeypatch.setitem(bench.MEASURED_TRAFFIC, ("c2", 0), stale)
    assert bench.measured_traffic(w) is None
    # no figure for a workload that was not measured, nor for a backward workload
    assert bench.measured_traffic(workload("c3")) is None
    assert bench.measured_traffic(workload("c4")) is None
