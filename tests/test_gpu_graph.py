"""The stage captured as a HIP graph.

emb_forward, emb_backward_dedup and emb_backward_apply only launch kernels on
the caller's stream (no allocation, copy or memset when the batch is not
empty), so one captured step replays to the results of the eager calls: the
same kernels on the same inputs, bit for bit (the sorted backward sums in a
fixed order).  Each check replays several times with other eager work of the
library and synchronisations in between, and compares every replay."""
import pytest
import torch

import embedding_columns_amd as E
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bufs(b):
    return dict(off=torch.from_numpy(b.offsets).to(DEV), ids=torch.from_numpy(b.ids).to(DEV),
                fv=torch.from_numpy(b.fvals).to(DEV), n=b.n)


def _step(plan, w, d, G, Y, out):
    kinds = {c.kind for c in w.cols}
    E.emb_forward(plan.plan, d["off"], d["ids"] if kinds & {0, 1} else None,
                  d["fv"] if 2 in kinds else None, None, d["n"], Y, plan.workspace, True)
    E.emb_backward_dedup(plan.plan, plan.workspace, out.get("ukeys"), out.get("nu"))
    E.emb_backward_apply(plan.plan, G, plan.workspace, out.get("ugrads"))


def _capture(fn):
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_graph_emit_replays_equal_eager():
    w = W.config(1)
    ba, bb = W.make_batch(w, seed=7100), W.make_batch(w, seed=7101)
    wts, sts = W.make_tables(w, seed=71, device=DEV)
    plan = E.EmbeddingColumns(w.cols, wts, sts, batch=w.batch, max_ids=max(ba.n, bb.n), opt=w.opt,
                              lr=w.lr, eps=w.eps, device=DEV)
    G = W.make_grad(w, seed=71, device=DEV)
    da, db = _bufs(ba), _bufs(bb)
    Y = torch.empty(w.batch, w.sum_dim, dtype=torch.float32, device=DEV)
    maxd = max(c.dim for c in w.cols)
    out = dict(ukeys=torch.empty(max(ba.n, bb.n), dtype=torch.int32, device=DEV),
               nu=torch.zeros(1, dtype=torch.int64, device=DEV),
               ugrads=torch.empty(max(ba.n, bb.n), maxd, dtype=torch.float32, device=DEV))
    _step(plan, w, da, G, Y, out)
    torch.cuda.synchronize()
    nu = int(out["nu"].item())
    assert nu > 0
    ref = (Y.clone(), out["ukeys"][:nu].clone(), out["ugrads"][:nu].clone())
    g = _capture(lambda: _step(plan, w, da, G, Y, out))
    for r in range(3):
        # other eager work of the library on the same workspace and outputs
        _step(plan, w, db, G, Y, out)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(out["nu"].item()) == nu, f"replay {r}: distinct-row count"
        assert torch.equal(Y, ref[0]), f"replay {r}: pooled output"
        assert torch.equal(out["ukeys"][:nu], ref[1]), f"replay {r}: distinct keys"
        assert torch.equal(out["ugrads"][:nu], ref[2]), f"replay {r}: row gradients"
    # the tables are left alone by EMIT
    w0, _ = W.make_tables(w, seed=71, device=DEV)
    for c in range(len(w.cols)):
        assert torch.equal(w0[c], wts[c])


@pytest.mark.parametrize("case", ["front-end-sgd", "long-seq-adagrad"])
def test_graph_update_replays_equal_eager(case):
    if case == "front-end-sgd":
        # hashed sum / mean columns with dropped IDs and empty bags; the column sort
        w = W.config(2, n_cols=12, batch=512, rows_range=(1e2, 1e4))
    else:
        # bf16 tables, Adagrad, columns above the column sort's capacity: the
        # global radix passes
        w = W.config(4, rows=50_000, batch=48)
    b = W.make_batch(w, seed=7200)
    G = W.make_grad(w, seed=72, device=DEV)
    d = _bufs(b)
    plans, tabs = [], []
    for _ in range(2):
        wts, sts = W.make_tables(w, seed=72, device=DEV)
        plans.append(E.EmbeddingColumns(w.cols, wts, sts, batch=w.batch, max_ids=b.n, opt=w.opt,
                                        lr=w.lr, eps=w.eps, device=DEV))
        tabs.append((wts, sts))
    Ye = torch.empty(w.batch, w.sum_dim, dtype=torch.float32, device=DEV)
    Yg = torch.empty_like(Ye)
    # the graph twin: captured once (capture runs nothing), then replayed per step
    g = _capture(lambda: _step(plans[1], w, d, G, Yg, {}))
    scratch = torch.empty(1 << 20, dtype=torch.float32, device=DEV)
    for step in range(3):
        _step(plans[0], w, d, G, Ye, {})
        torch.cuda.synchronize()
        scratch.normal_()                      # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Ye, Yg), f"step {step}: pooled output"
        for c in range(len(w.cols)):
            assert torch.equal(tabs[0][0][c], tabs[1][0][c]), f"step {step}: table {c}"
            if tabs[0][1][c] is not None:
                assert torch.equal(tabs[0][1][c], tabs[1][1][c]), f"step {step}: state {c}"
    # the steps did move the rows
    w0, _ = W.make_tables(w, seed=72, device=DEV)
    assert any(not torch.equal(w0[c], tabs[1][0][c]) for c in range(len(w.cols)))
