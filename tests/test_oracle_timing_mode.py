"""The oracle's timing mode (oracle_omp.c: columns spread over OpenMP threads, one
column per reference call) computes exactly what the single-threaded oracle does:
the benchmark's CPU baseline times the same arithmetic in both modes."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


@pytest.mark.parametrize("cfg,opt", [(2, W.OPT_SGD), (4, W.OPT_ADAGRAD), (3, None)])
def test_columns_over_threads_equal_the_reference(cfg, opt):
    if cfg == 2:
        w = W.config(2, n_cols=14, batch=64, rows_range=(100, 1000))
    elif cfg == 4:
        w = W.config(4, n_cols=4, batch=12, rows=5000)
    else:
        w = W.config(3, n_cols=40, batch=32, rows_range=(100, 1000))
    b = W.make_batch(w, seed=11 + cfg)
    wts, sts = W.make_tables(w, seed=11 + cfg)
    G = W.make_grad(w, seed=11 + cfg).numpy()
    ref = oracle.Columns(w.cols, [_host(t) for t in wts],
                         [None if s is None else _host(s) for s in sts])
    par = oracle.Columns(w.cols, [_host(t) for t in wts],
                         [None if s is None else _host(s) for s in sts])
    Y, _, _, _ = oracle.forward(ref, w.batch, b.offsets, b.ids, b.fvals)
    if w.training:
        oracle.backward(ref, w.batch, b.offsets, G, b.ids, b.fvals, opt=w.opt, lr=w.lr, eps=w.eps)
    cs = oracle.ColumnSteps(par, w.batch, G)
    used = cs.run(b.offsets, b.ids, b.fvals, training=w.training, opt=w.opt, lr=w.lr, eps=w.eps,
                  threads=4)
    assert used >= 1
    offs = np.concatenate([[0], np.cumsum([c.dim for c in w.cols])])
    for c in range(len(w.cols)):
        assert np.array_equal(Y[:, offs[c]:offs[c + 1]], cs.Y[c])
        assert np.array_equal(ref.weights[c], par.weights[c])
        if ref.states[c] is not None:
            assert np.array_equal(ref.states[c], par.states[c])
