"""The distinct-row list on both sort paths vs the oracle.

When the distinct rows, their count or the counters are asked for (always for
EMIT), the backward needs one ascending run of valid keys (RecIS Sec. 3.2: the
backward merges the gradients of each distinct ID).  Columns that fit the
column sort are sorted per column and then compacted (valid keys of every
column first, dropped ones after); larger inputs take the global radix passes.
Both must give the same distinct rows (bit-exact), counts and gradients (within
the condition-aware tolerance) as the oracle."""
import pytest

import workloads as W
from gpu_harness import run_dense_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("keep", [0.0, 0.3, 1.0])
def test_emit_column_sort_with_dropped_columns(keep):
    # many small columns; with the mask some columns lose every position, and
    # keep = 0 leaves no valid key at all
    w = W.config(3, n_cols=40, batch=96, rows_range=(50, 5000), opt=W.OPT_EMIT, training=True)
    run_dense_case(w, seed=5800, tile=64, mask_keep=None if keep == 1.0 else keep)


def test_emit_column_sort_front_end_shape():
    w = W.config(2, n_cols=30, batch=1024, rows_range=(1e2, 1e5), opt=W.OPT_EMIT)
    run_dense_case(w, seed=5810, tile=256)


def test_emit_global_passes():
    # two columns of ~30000 positions each: above 12288 per column on average,
    # so the global radix passes sort them
    w = W.config(2, n_cols=2, batch=10000, rows_range=(1e3, 1e5), opt=W.OPT_EMIT)
    run_dense_case(w, seed=5820, tile=128)


@pytest.mark.parametrize("ncols", [3, 24])
def test_sgd_unique_list_asked(ncols):
    # SGD with the distinct rows asked for: the unique list drives the apply
    # (on the compacted column sort for 24 columns, the global passes for 3)
    w = W.config(2, n_cols=ncols, batch=2048 if ncols == 24 else 12000,
                 rows_range=(1e2, 1e4), opt=W.OPT_SGD)
    run_dense_case(w, seed=5830 + ncols, tile=128, ask_unique=True)


def test_emit_global_passes_many_blocks():
    # about 18 M positions: some 4400 radix blocks of 4096 keys, so the per-digit
    # scan of the block counts (4096 counts per round) takes two rounds; long
    # Zipf sequences as in the long-sequence workload, on smaller tables
    w = W.config(4, rows=200_000, batch=4096, opt=W.OPT_EMIT)
    out = run_dense_case(w, seed=5840, tile=256)
    assert out["batch"].n > 4096 * 4096
