"""One-hot columns on the HIP path vs the oracle.

Every bag of a one-hot column holds exactly one position (the RECom explainer's
one-hot case, where the reduction is pointless).  The forward's general walk
already turns such a run into one row load and one output store per position,
so there is no separate path; these tests mix one-hot columns with ordinary
ones in the same tiles, and cover dropped IDs (zero output, or the default row),
mean pooling (n = 1), weights, bf16 tables and the backward."""
import pytest

import workloads as W
from gpu_harness import run_dense_case

pytestmark = pytest.mark.gpu


def _one_hot_workload(C=12, B=700, dtype=W.F32, opt=W.OPT_SGD, mixed=True):
    cols = []
    for c in range(C):
        cols.append(W.Column(W.HASH, (W.SUM, W.MEAN)[c % 2], dtype, 500 + 37 * c,
                             (4, 8, 16, 64)[c % 4], 0, W.ID_SPACE_40))
    w = W.Workload("one-hot", cols, B, "fixed", 1, 1, invalid_frac=0.05, id_dist="uniform",
                   opt=opt, lr=0.01, eps=1e-8)
    if mixed:
        # every third column gets bags of 1..4 instead (set per column by the generator)
        w.extra["lens"] = {c: (1, 4) for c in range(0, C, 3)}
    return w


@pytest.mark.parametrize("tile", [64, 256])
@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
def test_one_hot_sgd(tile, dtype):
    run_dense_case(_one_hot_workload(dtype=dtype), seed=8100 + tile, tile=tile)


def test_one_hot_emit_and_inference():
    run_dense_case(_one_hot_workload(opt=W.OPT_EMIT), seed=8200, tile=128)
    run_dense_case(_one_hot_workload(opt=W.OPT_EMIT), seed=8201, tile=128, training=False)


def test_one_hot_weights_and_default_rows():
    w = _one_hot_workload(opt=W.OPT_ADAGRAD)
    for c, col in enumerate(w.cols):
        if c % 2 == 1:
            col.default_row = c
    run_dense_case(w, seed=8300, tile=64, weighted=True, ask_unique=False)
