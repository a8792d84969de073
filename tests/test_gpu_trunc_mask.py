"""Sequence truncation and the per-position mask on the HIP path vs the oracle.

Both remove raw positions before the transform (RecIS Sec. 3.1 / Figure 2:
SeqTrunc is ordered before Hash): a removed position reads no row, does not
count in a mean and gets no gradient.  Parity as in the other GPU tests: rows,
bags and counts bit-exact, pooled outputs and updates within the
condition-aware tolerance.  The long-bag cases put the kept window of a bag in
another tile than the bag's start or end, so the kernel has to find both ends
outside its own tile."""
import numpy as np
import pytest

import workloads as W
from gpu_harness import run_dense_case, to_np

pytestmark = pytest.mark.gpu


def _truncate(w, seq_max, keep_last, every=1):
    for c, col in enumerate(w.cols):
        if c % every == 0:
            col.seq_max, col.seq_keep_last = seq_max, keep_last
    return w


@pytest.mark.parametrize("keep_last", [0, 1])
@pytest.mark.parametrize("seq_max", [1, 2, 5])
def test_truncation_front_end_sgd(seq_max, keep_last):
    # Poisson(3) bags; every other column truncated, so truncated and plain
    # columns share tiles
    w = _truncate(W.config(2, n_cols=24, batch=512, rows_range=(1e2, 1e4)), seq_max, keep_last, 2)
    run_dense_case(w, seed=5100 + seq_max, tile=128)


@pytest.mark.parametrize("keep_last", [0, 1])
@pytest.mark.parametrize("tile", [64, 256])
def test_truncation_long_bags_bf16_adagrad(keep_last, tile):
    # bags of 200..2000 positions cut to 300: the kept window and the bag's ends
    # fall in different tiles; mean over the kept positions only
    w = _truncate(W.config(4, n_cols=4, batch=24, rows=50_000), 300, keep_last)
    run_dense_case(w, seed=5200 + keep_last, tile=tile)


@pytest.mark.parametrize("keep", [0.0, 0.5, 0.9])
def test_mask_front_end_sgd(keep):
    w = W.config(2, n_cols=20, batch=400, rows_range=(1e2, 1e4))
    run_dense_case(w, seed=5300, tile=128, mask_keep=keep)


def test_mask_and_truncation_long_bags():
    w = _truncate(W.config(4, n_cols=4, batch=16, rows=50_000), 250, 1, 2)
    run_dense_case(w, seed=5400, tile=128, mask_keep=0.7)


@pytest.mark.parametrize("training", [False, True])
def test_mask_many_tiny_columns(training):
    # hashed and bucketized columns, forward only or with the backward
    w = _truncate(W.config(3, n_cols=60, batch=128, rows_range=(100, 3000), opt=W.OPT_SGD,
                           lr=0.01, training=training), 3, 0, 3)
    run_dense_case(w, seed=5500, tile=64, training=training, mask_keep=0.6)


def test_truncation_emit_and_segments_from_keys():
    w = _truncate(W.config(2, n_cols=16, batch=300, rows_range=(30, 3000), opt=W.OPT_EMIT), 2, 1)
    run_dense_case(w, seed=5600, tile=64)
    w = _truncate(W.config(2, n_cols=16, batch=300, rows_range=(30, 3000)), 2, 0)
    run_dense_case(w, seed=5601, tile=256, ask_unique=False)


def test_filtered_stats():
    """filtered = positions removed by truncation or the mask; dropped counts only
    the transform's own drops among the kept positions."""
    w = _truncate(W.config(2, n_cols=10, batch=200, rows_range=(100, 1000), opt=W.OPT_EMIT), 2, 1, 2)
    out = run_dense_case(w, seed=5700, tile=128, mask_keep=0.75)
    st, b, mask = out["step"], out["batch"], out["mask"]
    s = to_np(st.stats)
    _, _, bag_n, rows = out["ref"]
    C, B = len(w.cols), w.batch
    kept = mask.astype(bool).copy()
    for bag in range(C * B):
        col = w.cols[bag // B]
        a, e = int(b.offsets[bag]), int(b.offsets[bag + 1])
        if col.seq_max and e - a > col.seq_max:
            cut = np.ones(e - a, bool)
            if col.seq_keep_last:
                cut[e - a - col.seq_max:] = False
            else:
                cut[:col.seq_max] = False
            kept[a:e] &= ~cut
    assert s[0] == b.n
    assert s[10] == b.n - int(kept.sum())
    assert s[2] == int((b.invalid_mask & kept).sum())
    assert s[1] == int(kept.sum()) - s[2] == int((rows >= 0).sum())
    assert int(bag_n.sum()) == s[1]
