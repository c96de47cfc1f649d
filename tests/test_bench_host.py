"""Host-side checks of bench.py (no GPU): the FLOP conventions against brute
force, the roofline peaks, the committed profiles that `traffic` is read
from, and the refusal of more than one GPU."""
import os
import re
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from exact_attention_117_amd import inputs  # noqa: E402


def brute_pairs(N, causal, window):
    """(query, key) pairs with i - left <= j <= i + right (j <= i if causal),
    counted one by one; -1 leaves a side unbounded."""
    wl, wr = window
    n = 0
    for i in range(N):
        for j in range(N):
            if causal and j > i:
                continue
            if wl >= 0 and j < i - wl:
                continue
            if wr >= 0 and j > i + wr:
                continue
            n += 1
    return n


@pytest.mark.parametrize("N", [1, 2, 7, 64, 129])
@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (False, (-1, -1)), (True, (0, 0)),
                                           (True, (5, 0)), (False, (3, 9)), (False, (0, 200)),
                                           (False, (-1, 2))])
def test_visible_pairs_brute_force(N, causal, window):
    assert bench.visible_pairs(N, causal, window) == brute_pairs(N, causal, window)


def test_fwd_flop_convention():
    # 4 B H N^2 d, halved for causal; a window counts 4 d per visible pair
    assert bench.fwd_flops(2, 8, 3, 16, False) == 4 * 2 * 3 * 8 * 8 * 16
    assert bench.fwd_flops(2, 8, 3, 16, True) == 4 * 2 * 3 * 8 * 8 * 16 / 2
    assert bench.fwd_flops(1, 10, 2, 4, True, (3, 0)) == 4 * 2 * 4 * brute_pairs(10, True, (3, 0))
    # the headline's 549.8 GFLOP
    assert bench.fwd_flops(4, 4096, 32, 128, True) == 4 * 4 * 32 * 4096 ** 2 * 128 / 2


def test_roofline_peaks():
    # dense MFMA: 256 CUs at 2.4 GHz, 4096 bf16 and 8192 fp8 FLOP per clock and CU
    assert abs(bench.PEAK_BF16_TFLOPS - 256 * 2.4e9 * 4096 / 1e12) < 0.1
    assert abs(bench.PEAK_FP8_TFLOPS - 256 * 2.4e9 * 8192 / 1e12) < 0.1
    # FP8 forward: half of the FLOPs at each peak, so the time of the two halves
    t = 0.5 / bench.PEAK_FP8_TFLOPS + 0.5 / bench.PEAK_BF16_TFLOPS
    assert abs(bench.PEAK_FP8_MIXED_TFLOPS - 1.0 / t) < 1e-9
    assert bench.PEAK_BF16_TFLOPS < bench.PEAK_FP8_MIXED_TFLOPS < bench.PEAK_FP8_TFLOPS


def test_algorithmic_bytes_by_hand():
    # forward: q, k, v read and o written (16-bit), lse written (fp32)
    w = inputs.Workload("t", 0, 0, 2, 8, 3, 16, True)
    assert bench.algorithmic_bytes(w) == 2 * 8 * 3 * (4 * 16 * 2 + 4)
    # fp8: one byte per q, k, v element, bf16 o
    w8 = inputs.Workload("t", 0, 0, 2, 8, 3, 16, True, dtype="fp8")
    assert bench.algorithmic_bytes(w8) == 2 * 8 * 3 * (3 * 16 + 16 * 2 + 4)
    # backward: q, k, v, o, dO read and dq, dk, dv written (16-bit); lse read,
    # D written and read (fp32)
    wb = inputs.Workload("t", 0, 0, 2, 8, 3, 16, True, kind="bwd")
    assert bench.algorithmic_bytes(wb) == 2 * 8 * 3 * (8 * 16 * 2 + 3 * 4)
    # packed sequences count their rows
    wv = inputs.Workload("t", 0, 0, 3, 8, 3, 16, True, kind="varlen")
    assert bench.algorithmic_bytes(wv, [1, 5, 2]) == 8 * 3 * (4 * 16 * 2 + 4)


@pytest.mark.parametrize("name", sorted(bench.TRAFFIC_PROFILES))
def test_traffic_profiles_are_readable(name):
    path, sources = bench.TRAFFIC_PROFILES[name]
    text = open(os.path.join(ROOT, path)).read()
    assert re.search(r"sha256: `[0-9a-f]{64}`", text)
    m_tr = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
    m_al = re.search(r"^algorithmic_bytes_per_launch: (\d+)$", text, re.M)
    assert m_tr and m_al
    for f in sources:
        assert os.path.exists(os.path.join(ROOT, f)), f
    # the commands are those of this workload
    if name != "headline":
        assert "--workload %s " % name in text
    # the recorded algorithmic bytes are the ones bench.py computes
    w = inputs.WORKLOADS[name]
    lengths = None
    if w.kind in ("varlen", "bwd_varlen", "decode"):
        lengths = inputs.varlen_lengths(w, torch.Generator().manual_seed(w.seed))
    assert int(m_al.group(1)) == bench.algorithmic_bytes(w, lengths)
    # traffic is reported only while the sources are the profiled ones
    value, note = bench.profiled_traffic(name)
    assert value == int(m_tr.group(1)) or note == "kernel changed since the counters were taken"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
