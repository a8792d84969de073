"""Host logic of bench.py (no GPU): the algorithmic byte counts behind the
roofline figure, the traffic lookup that must go stale when the kernels change,
and the single-GPU guard."""
import os
import subprocess
import sys

import numpy as np

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _tiny():
    cols = [W.Column(W.HASH, W.SUM, W.F32, 100, 8, 0, 1 << 40),
            W.Column(W.BUCKET, W.MEAN, W.BF16, 70, 16, boundaries=np.arange(5, dtype=np.float32)),
            W.Column(W.IDENTITY, W.SUM, W.F32, 50, 4)]
    w = W.Workload("t", cols, 3, "fixed", 2, 2, opt=W.OPT_SGD, lr=0.1)
    off = np.array([0, 2, 4, 5, 6, 7, 8, 10, 10, 13], dtype=np.int32)
    b = W.Batch(off, np.zeros(13, np.int64), np.zeros(13, np.float32), np.zeros(13, bool),
                np.zeros(9, bool), 13)
    return w, b


def test_forward_bytes_closed_form():
    w, b = _tiny()
    valid, gathers = [4, 3, 5], [4, 3, 4]
    # ids: 8 B at the 4 + 6 hashed / identity positions, 4 B at the 3 float positions;
    # offsets 4 * (9 + 1); rows 4*8*4 + 3*16*2 + 4*4*4; Y 4 * 3 * 28; saved rows 4 * 12
    want = 8 * 10 + 4 * 3 + 4 * 10 + (128 + 96 + 64) + 4 * 3 * 28 + 4 * 12
    assert bench.fwd_bytes(w, b, valid, gathers, True) == want
    assert bench.fwd_bytes(w, b, valid, gathers, False) == want - 4 * 12


def test_backward_bytes_per_optimizer():
    w, _ = _tiny()
    uniq = [3, 2, 4]
    base = 4 * 12 + 4 * 3 * 28
    w.opt = W.OPT_EMIT
    assert bench.bwd_bytes(w, 12, uniq) == base + 3 * (4 + 32) + 2 * (4 + 64) + 4 * (4 + 16)
    w.opt = W.OPT_SGD
    assert bench.bwd_bytes(w, 12, uniq) == base + 3 * 64 + 2 * 64 + 4 * 32
    w.opt = W.OPT_ADAGRAD
    assert bench.bwd_bytes(w, 12, uniq) == base + 3 * (64 + 64) + 2 * (64 + 128) + 4 * (32 + 32)


def test_traffic_goes_stale_with_the_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    f = prof / "seg_apply_w_traffic.md"
    f.write_text(f"traffic_bytes_per_launch: 1234\n\nsource_sha256: {bench.source_hash()}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("seg_apply", "w") == 1234
    f.write_text("traffic_bytes_per_launch: 1234\n\nsource_sha256: " + "0" * 64 + "\n")
    assert bench.measured_traffic("seg_apply", "w") is None
    assert bench.measured_traffic("fwd_kernel", "w") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
