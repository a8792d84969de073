"""Default rows on the HIP path vs the oracle.

A column with a default row d fills every bag that has no valid position (empty,
all IDs dropped, truncated or masked away) with row d: the bag pools to E[d]
and d receives that bag's gradient with weight 1 (the RECom explainer's default
for a missing feature, merged into the lookup).  The forward adds one sort entry
per bag after the N positions; these tests run every backward path that reads
them (the unique-row list for EMIT / SGD / Adagrad, segments from the sorted
keys), with weights, truncation and masks, and with every bag empty."""
import numpy as np
import pytest

import workloads as W
from gpu_harness import run_dense_case

pytestmark = pytest.mark.gpu


def _defaults(w, every=2):
    for c, col in enumerate(w.cols):
        if c % every == 0:
            col.default_row = (7 * c + 3) % col.rows
    return w


@pytest.mark.parametrize("ask_unique", [True, False])
@pytest.mark.parametrize("tile", [64, 256])
def test_default_row_front_end_sgd(tile, ask_unique):
    # 5 % forced-empty bags, Poisson(3) lengths (more empty ones), 2 % invalid IDs
    w = _defaults(W.config(2, n_cols=24, batch=512, rows_range=(1e2, 1e4)))
    run_dense_case(w, seed=7100 + tile, tile=tile, ask_unique=ask_unique)


def test_default_row_emit_gradients():
    w = _defaults(W.config(2, n_cols=16, batch=300, rows_range=(30, 3000), opt=W.OPT_EMIT,
                           empty_frac=0.3), every=1)
    run_dense_case(w, seed=7200, tile=128)


@pytest.mark.parametrize("ask_unique", [True, False])
def test_default_row_adagrad_with_mask_weights_truncation(ask_unique):
    # a sparse mask empties many short bags; weights and truncation on top
    w = _defaults(W.config(2, n_cols=20, batch=256, rows_range=(1e2, 1e4), opt=W.OPT_ADAGRAD,
                           lr=0.05, eps=1e-8))
    for c, col in enumerate(w.cols):
        if c % 3 == 1:
            col.seq_max, col.seq_keep_last = 2, 1
    run_dense_case(w, seed=7300, tile=64, mask_keep=0.3, weighted=True, ask_unique=ask_unique)


def test_default_row_bf16_long_bags_masked_out():
    # long bf16 bags; a mask keeping 0.1 % of positions leaves most bags empty
    w = _defaults(W.config(4, n_cols=4, batch=24, rows=50_000), every=1)
    run_dense_case(w, seed=7400, tile=256, mask_keep=0.001)


@pytest.mark.parametrize("opt", [W.OPT_EMIT, W.OPT_SGD])
def test_default_row_every_bag_empty(opt):
    # no positions at all: every output is its column's default row (or zero)
    w = _defaults(W.config(2, n_cols=10, batch=64, rows_range=(50, 500), opt=opt, lr=0.01,
                           empty_frac=1.0))
    out = run_dense_case(w, seed=7500, tile=128)
    assert out["batch"].n == 0


def test_default_row_inference():
    w = _defaults(W.config(3, n_cols=40, batch=128, rows_range=(100, 3000), training=False))
    run_dense_case(w, seed=7600, tile=64, training=False, mask_keep=0.5)
