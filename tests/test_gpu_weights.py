"""Per-position weights on the HIP path vs the oracle.

Each contributor r of a bag carries a weight v_r (RecIS Sec. 3.2, index-aware
segment reduction: the forward sums w_r E[i_r], the backward sends w_r G[s(r)]
to row i_r).  A sum bag uses w_r = v_r, a mean bag v_r / n.  The weighted
forward records the weights and lets the sort carry positions, so every
backward path is covered: the unique-row list (EMIT, SGD, Adagrad), segments
found from the sorted keys (column sort and global radix passes), bf16 tables,
and weights together with truncation and a mask.  Parity bar as in the other
GPU tests."""
import numpy as np
import pytest

import workloads as W
from gpu_harness import run_dense_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ask_unique", [True, False])
@pytest.mark.parametrize("tile", [64, 256])
def test_weighted_front_end_sgd(tile, ask_unique):
    w = W.config(2, n_cols=24, batch=512, rows_range=(1e2, 1e4))
    run_dense_case(w, seed=6100 + tile, tile=tile, weighted=True, ask_unique=ask_unique)


def test_weighted_emit_gradients():
    w = W.config(2, n_cols=16, batch=300, rows_range=(30, 3000), opt=W.OPT_EMIT)
    run_dense_case(w, seed=6200, tile=128, weighted=True)


@pytest.mark.parametrize("ask_unique", [True, False])
def test_weighted_long_bags_bf16_adagrad(ask_unique):
    # bags of 200..2000 positions (split over tiles), bf16 tables, mean, Adagrad
    w = W.config(4, n_cols=4, batch=24, rows=50_000)
    run_dense_case(w, seed=6300, tile=128, weighted=True, ask_unique=ask_unique)


@pytest.mark.parametrize("training", [False, True])
def test_weighted_many_tiny_columns(training):
    w = W.config(3, n_cols=60, batch=128, rows_range=(100, 3000), opt=W.OPT_SGD, lr=0.01,
                 training=training)
    run_dense_case(w, seed=6400, tile=64, training=training, weighted=True)


def test_weighted_global_radix_passes():
    # one column of 40000 positions: more than the column sort holds per column on
    # average, so the segments come from the global radix passes
    cols = [W.Column(W.IDENTITY, W.SUM, W.F32, 3000, 16)]
    w = W.Workload("one-column", cols, 8, "fixed", 5000, 5000, id_dist="uniform", id_space=3000,
                   opt=W.OPT_SGD, lr=0.01)
    run_dense_case(w, seed=6500, tile=256, weighted=True, ask_unique=False)


def test_weighted_with_truncation_and_mask():
    w = W.config(2, n_cols=20, batch=300, rows_range=(1e2, 1e4))
    for c, col in enumerate(w.cols):
        if c % 3 == 0:
            col.seq_max, col.seq_keep_last = 2, c % 2
    run_dense_case(w, seed=6600, tile=64, weighted=True, mask_keep=0.7)


def test_unit_weights_equal_the_plain_forward():
    """All-one weights through the extended forward give bit-identical outputs and
    updated tables to the plain forward."""
    import torch
    from gpu_harness import Step, to_np
    w = W.config(2, n_cols=12, batch=256, rows_range=(50, 2000))
    b = W.make_batch(w, seed=6700)
    G = W.make_grad(w, seed=6700, device="cpu")
    outs = []
    for pw in (None, np.ones(b.n, np.float32)):
        wts, sts = W.make_tables(w, seed=6700, device="cpu")
        st = Step(w, b, wts, sts, tile=128)
        Y = st.forward(training=True, pweights=pw)
        st.backward(G, ask_unique=False)
        torch.cuda.synchronize()
        outs.append((to_np(Y), [to_np(t) for t in st.gw]))
    assert np.array_equal(outs[0][0], outs[1][0])
    for x, y in zip(outs[0][1], outs[1][1]):
        assert np.array_equal(x, y)
