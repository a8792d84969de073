"""Parity at the workloads' full sizes, in the benchmark's launch configuration
(default tile; the benchmark's first batch, tables, upstream gradient and
prepopulated keyed table, from the same seeds).

The CPU oracle recomputes every pooled output and every touched row: the
training front end's SGD rows, all of the long sequences' touched Adagrad rows
and accumulators (a seeded sample of untouched rows must stay bit-identical),
and every row the keyed workload's step updated, on the full prepopulated
table."""
import numpy as np
import pytest
import torch

import embedding_columns_amd as E
import oracle
import workloads as W
from gpu_harness import (RTOL_F32, check_forward, check_rows_adagrad, check_rows_sgd,
                         check_unique, to_np)
from oracle.table import OracleTable

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gpu_step(w, b, weights, states, G):
    cols = E.EmbeddingColumns(w.cols, weights, states, batch=w.batch, max_ids=b.n, opt=w.opt,
                              lr=w.lr, eps=w.eps, device=DEV)
    off = torch.from_numpy(b.offsets).to(DEV)
    kinds = {c.kind for c in w.cols}
    ids = torch.from_numpy(b.ids).to(DEV) if kinds & {W.HASH, W.IDENTITY} else None
    fv = torch.from_numpy(b.fvals).to(DEV) if W.BUCKET in kinds else None
    Y = cols.forward(off, ids=ids, fvals=fv, training=w.training)
    # the backward's sort reuses the forward's key and bag arrays: copy them first
    ws = tuple(t.clone() for t in cols.workspace_view(b.n)) if w.training else None
    out = {"Y": Y, "ws": ws, "cols": cols}
    if w.training:
        # the unique-row list, from a dedup of its own (the apply is not run here)
        keys = torch.empty(b.n, dtype=torch.int32, device=DEV)
        nu = torch.zeros(1, dtype=torch.int64, device=DEV)
        E.emb_backward_dedup(cols.plan, cols.workspace, keys, nu, None)
        out["ukeys"], out["nu"] = keys, nu
        torch.cuda.synchronize()
        # then the benchmark's step: forward again, backward with nothing asked back
        cols.forward(off, ids=ids, fvals=fv, training=True)
        cols.backward(G, want_count=False)
    torch.cuda.synchronize()
    return out


def test_training_front_end_full():
    w = W.config(2)
    b = W.make_batch(w, seed=2000)
    wts, sts = W.make_tables(w, seed=2, device=DEV)
    G = W.make_grad(w, seed=2, device=DEV)
    host_w = [to_np(t) for t in wts]
    r = _gpu_step(w, b, wts, sts, G)
    oc = oracle.Columns(w.cols, [x.copy() for x in host_w])
    ref = oracle.forward(oc, w.batch, b.offsets, b.ids, b.fvals)
    check_forward(w, b, r["Y"], r["ws"], ref)
    ucol, urow, ug, ub = oracle.backward(oc, w.batch, b.offsets, to_np(G), b.ids, b.fvals,
                                         opt=w.opt, lr=w.lr)
    check_unique(w, r["ukeys"], r["nu"], ucol, urow)
    for c, col in enumerate(w.cols):
        sel = ucol == c
        check_rows_sgd(col, host_w[c], to_np(wts[c]), oc.weights[c], urow[sel],
                       ub[sel][:, :col.dim], w.lr)


def test_many_tiny_columns_full():
    w = W.config(3)
    b = W.make_batch(w, seed=3000)
    wts, sts = W.make_tables(w, seed=3, device=DEV)
    host_w = [to_np(t) for t in wts]
    r = _gpu_step(w, b, wts, sts, None)
    oc = oracle.Columns(w.cols, host_w)
    ref = oracle.forward(oc, w.batch, b.offsets, b.ids, b.fvals)
    check_forward(w, b, r["Y"], None, ref, training=False)


def test_long_sequences_full():
    w = W.config(4)
    b = W.make_batch(w, seed=4000)
    wts, sts = W.make_tables(w, seed=4, device=DEV)
    G = W.make_grad(w, seed=4, device=DEV)
    host_w = [to_np(t) for t in wts]
    host_s = [to_np(s) for s in sts]
    r = _gpu_step(w, b, wts, sts, G)
    oc = oracle.Columns(w.cols, [x.copy() for x in host_w], [s.copy() for s in host_s])
    ref = oracle.forward(oc, w.batch, b.offsets, b.ids, b.fvals)
    check_forward(w, b, r["Y"], r["ws"], ref)
    ucol, urow, ug, ub = oracle.backward(oc, w.batch, b.offsets, to_np(G), b.ids, b.fvals,
                                         opt=w.opt, lr=w.lr, eps=w.eps)
    check_unique(w, r["ukeys"], r["nu"], ucol, urow)
    rng = np.random.default_rng(44)
    for c, col in enumerate(w.cols):
        sel = np.flatnonzero(ucol == c)
        rows = urow[sel]
        gw = to_np(wts[c][torch.from_numpy(rows).to(DEV)])
        gs = to_np(sts[c][torch.from_numpy(rows).to(DEV)])
        # every touched row and accumulator, compared as a table whose rows are all touched
        sub = W.Column(col.kind, col.pool, col.dtype, rows.size, col.dim)
        check_rows_adagrad(sub, host_w[c][rows], host_s[c][rows], gw, gs, ug[sel][:, :col.dim],
                           ub[sel][:, :col.dim], np.arange(rows.size), w.lr, w.eps)
        # a sample of untouched rows stays bit-identical
        touched = np.zeros(col.rows, bool)
        touched[rows] = True
        r_ = rng.integers(0, col.rows, 200000)
        un = np.unique(r_[~touched[r_]])
        assert np.array_equal(to_np(wts[c][torch.from_numpy(un).to(DEV)]), host_w[c][un])
        assert np.array_equal(to_np(sts[c][torch.from_numpy(un).to(DEV)]), host_s[c][un])


def test_keyed_table_full_one_step():
    w = W.config(5)
    pk = W.prepop_keys(w.prepop)
    T = E.KeyedTable(w.capacity, w.row_capacity, 32, threshold=w.threshold, init_std=w.init_std,
                     device=DEV)
    # prepopulated in chunks of 10M keys with per-chunk seeds, as the benchmark does
    prows = torch.empty(w.prepop, 32, dtype=torch.float32, device=DEV)
    chunk = 10_000_000
    for s in range(0, w.prepop, chunk):
        e = min(s + chunk, w.prepop)
        prows[s:e] = W.make_prepop_rows(e - s, 32, w.init_std, seed=s, device=DEV)
        T.bulk_insert(torch.from_numpy(pk[s:e]).to(DEV), prows[s:e])
    torch.cuda.synchronize()
    O = OracleTable(w.capacity, 32, w.threshold, w.init_std, pk,
                    lambda idx: to_np(prows[torch.from_numpy(np.asarray(idx)).to(DEV)]))
    b = W.make_batch(w, seed=5000)
    G = W.make_grad(w, seed=5, device=DEV)
    keys = torch.from_numpy(b.ids).to(DEV)
    rows = T.lookup_or_insert(keys)
    cols = E.EmbeddingColumns(w.cols, [T.rows], batch=w.batch, max_ids=b.n, opt=W.OPT_SGD, lr=w.lr,
                              device=DEV)
    Y = cols.forward(torch.from_numpy(b.offsets).to(DEV), keyed_rows=rows, training=True)
    cols.backward(G)
    torch.cuda.synchronize()

    O.step(b.ids)
    krows, pool_keys, pool = O.resolve(b.ids)
    col = W.Column(W.KEYED, W.SUM, W.F32, max(pool.shape[0], 1), 32)
    oc = oracle.Columns([col], [pool.copy()])
    Yr, Yb, _, _ = oracle.forward(oc, w.batch, b.offsets, keyed_rows=krows)
    _, urow, _, ub = oracle.backward(oc, w.batch, b.offsets, to_np(G), keyed_rows=krows,
                                     opt=W.OPT_SGD, lr=w.lr)
    g_rows = to_np(rows)
    assert np.array_equal(g_rows == E.ROW_DEFAULT, krows == oracle.ROW_DEFAULT)
    assert np.array_equal(g_rows == E.ROW_DROPPED, krows == oracle.ROW_DROPPED)
    adm = g_rows >= 0
    pairs = np.unique(np.stack([b.ids[adm], g_rows[adm]]), axis=1)
    assert np.unique(pairs[0]).size == pairs.shape[1] == np.unique(pairs[1]).size
    err = np.abs(to_np(Y).astype(np.float64) - Yr)
    assert np.all(err <= RTOL_F32 * Yb), "pooled outputs differ"
    # every updated row, found by its key
    pick = np.arange(urow.size)
    sk = pool_keys[urow[pick]]
    grow, gcnt = T.find(torch.from_numpy(sk).to(DEV))
    grow = to_np(grow)
    assert np.all(grow >= 0)
    gvals = to_np(T.rows[torch.from_numpy(grow).long().to(DEV)]).astype(np.float64)
    ovals = oc.weights[0][urow[pick]].astype(np.float64)
    tol = w.lr * RTOL_F32 * ub[pick][:, :32] + 2.0 ** -22 * (np.abs(ovals) + np.abs(pool[urow[pick]])) + 1e-30
    assert np.all(np.abs(gvals - ovals) <= tol), "updated keyed rows differ"
    _, ocnt, _ = O.state(sk)
    assert np.array_equal(to_np(gcnt), ocnt), "occurrence counts differ"
