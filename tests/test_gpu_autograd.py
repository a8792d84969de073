"""The stage under torch autograd: loss.backward() runs emb_backward.

Monolith Sec. 2.1 treats embedding lookups and their updates as native framework
operations; here the fused forward is an autograd node.  The gradient that
reaches it is captured with a hook and handed to the oracle, so each test checks
the wiring (what autograd passes in) and the result (what the library does with
it) separately: SGD and Adagrad rows updated in place, EMIT gradients as sparse
table gradients."""
import numpy as np
import pytest
import torch

import embedding_columns_amd as E
import oracle
import workloads as W
from gpu_harness import RTOL_F32, check_rows_adagrad, check_rows_sgd, to_np

pytestmark = pytest.mark.gpu


def _setup(w, seed, dev, tables_require_grad=False):
    b = W.make_batch(w, seed=seed)
    wts, sts = W.make_tables(w, seed=seed, device="cpu")
    gw = [t.to(dev).contiguous() for t in wts]
    gs = [None if s is None else s.to(dev).contiguous() for s in sts]
    if tables_require_grad:
        for t in gw:
            t.requires_grad_(True)
    cols = E.EmbeddingColumns(w.cols, gw, gs, batch=w.batch, max_ids=b.n, opt=w.opt, lr=w.lr,
                              eps=w.eps, device=dev)
    host_w = [to_np(t) for t in wts]
    host_s = [None if s is None else to_np(s) for s in sts]
    return b, cols, gw, gs, host_w, host_s


def _run(cols, b, dev, w):
    """Y through autograd, then a small dense head and a squared loss; returns the
    pooled output and the gradient autograd handed to the stage."""
    off = torch.from_numpy(b.offsets).to(dev)
    ids = torch.from_numpy(b.ids).to(dev)
    Y = cols(off, ids=ids)
    seen = []
    Y.register_hook(lambda g: seen.append(g.detach().clone()))
    head = torch.linspace(-1.0, 1.0, w.sum_dim * 3, device=dev).reshape(w.sum_dim, 3)
    loss = ((Y @ head) ** 2).sum() * 0.5
    loss.backward()
    torch.cuda.synchronize()
    assert len(seen) == 1
    return Y.detach(), seen[0]


def test_autograd_sgd_updates_rows_in_place():
    dev = torch.device("cuda")
    w = W.config(2, n_cols=16, batch=256, rows_range=(100, 2000))
    b, cols, gw, _, host_w, _ = _setup(w, 8100, dev)
    Y, G = _run(cols, b, dev, w)
    oc = oracle.Columns(w.cols, [x.copy() for x in host_w])
    Yr, Yb, _, _ = oracle.forward(oc, w.batch, b.offsets, b.ids)
    assert np.all(np.abs(to_np(Y).astype(np.float64) - Yr) <= RTOL_F32 * Yb)
    ucol, urow, ug, ub = oracle.backward(oc, w.batch, b.offsets, to_np(G), b.ids, opt=W.OPT_SGD,
                                         lr=w.lr)
    for c, col in enumerate(w.cols):
        sel = ucol == c
        check_rows_sgd(col, host_w[c], to_np(gw[c]), oc.weights[c], urow[sel],
                       ub[sel][:, :col.dim], w.lr)


def test_autograd_adagrad_bf16_long_bags():
    dev = torch.device("cuda")
    w = W.config(4, n_cols=4, batch=32, rows=20_000)
    b, cols, gw, gs, host_w, host_s = _setup(w, 8200, dev)
    Y, G = _run(cols, b, dev, w)
    oc = oracle.Columns(w.cols, [x.copy() for x in host_w], [s.copy() for s in host_s])
    Yr, Yb, _, _ = oracle.forward(oc, w.batch, b.offsets, b.ids)
    assert np.all(np.abs(to_np(Y).astype(np.float64) - Yr) <= RTOL_F32 * Yb)
    ucol, urow, ug, ub = oracle.backward(oc, w.batch, b.offsets, to_np(G), b.ids,
                                         opt=W.OPT_ADAGRAD, lr=w.lr, eps=w.eps)
    for c, col in enumerate(w.cols):
        sel = ucol == c
        check_rows_adagrad(col, host_w[c], host_s[c], to_np(gw[c]), to_np(gs[c]),
                           ug[sel][:, :col.dim], ub[sel][:, :col.dim], urow[sel], w.lr, w.eps)


def test_autograd_emit_sparse_table_grads():
    dev = torch.device("cuda")
    w = W.config(2, n_cols=12, batch=200, rows_range=(50, 3000), opt=W.OPT_EMIT)
    b, cols, gw, _, host_w, _ = _setup(w, 8300, dev, tables_require_grad=True)
    Y, G = _run(cols, b, dev, w)
    oc = oracle.Columns(w.cols, [x.copy() for x in host_w])
    ucol, urow, ug, ub = oracle.backward(oc, w.batch, b.offsets, to_np(G), b.ids, opt=W.OPT_EMIT)
    for c, col in enumerate(w.cols):
        assert np.array_equal(to_np(gw[c].detach()), host_w[c]), "EMIT must not touch tables"
        g = gw[c].grad
        assert g is not None and g.is_sparse
        g = g.coalesce()
        sel = ucol == c
        assert np.array_equal(g.indices()[0].cpu().numpy(), urow[sel]), "touched rows differ"
        d = np.abs(to_np(g.values()).astype(np.float64) - ug[sel][:, :col.dim])
        assert np.all(d <= RTOL_F32 * ub[sel][:, :col.dim])
    keys, grads, nu = cols.emitted
    assert int(nu.item()) == ucol.size


def test_no_grad_is_plain_inference():
    dev = torch.device("cuda")
    w = W.config(2, n_cols=8, batch=64, rows_range=(100, 1000))
    b, cols, gw, _, host_w, _ = _setup(w, 8400, dev)
    off = torch.from_numpy(b.offsets).to(dev)
    ids = torch.from_numpy(b.ids).to(dev)
    with torch.no_grad():
        Y = cols(off, ids=ids)
    assert not Y.requires_grad
    torch.cuda.synchronize()
    oc = oracle.Columns(w.cols, [x.copy() for x in host_w])
    Yr, Yb, _, _ = oracle.forward(oc, w.batch, b.offsets, b.ids)
    assert np.all(np.abs(to_np(Y).astype(np.float64) - Yr) <= RTOL_F32 * Yb)
    for c in range(len(w.cols)):
        assert np.array_equal(to_np(gw[c]), host_w[c])
