"""emb_forward_noalloc (the inference forward with the library's fixed scratch)
against emb_forward with a workspace: the same kernels over the same tiles, so
the pooled outputs must be identical, on two calls in a row (the second with a
smaller batch, which finds the first call's leftovers in the shared array), and
equal to the oracle within the parity tolerance.  A batch too large for the
array is refused before anything is launched."""
import numpy as np
import pytest
import torch

import embedding_columns_amd as E
import oracle
import workloads as W
from gpu_harness import RTOL_F32, to_np

pytestmark = pytest.mark.gpu


def _inputs(w, seed, dev):
    b = W.make_batch(w, seed=seed)
    return b, torch.from_numpy(b.offsets).to(dev), torch.from_numpy(b.ids).to(dev), \
        torch.from_numpy(b.fvals).to(dev)


def _both(cols, w, b, off, ids, fv, dev):
    kinds = {c.kind for c in w.cols}
    gi = ids if kinds & {W.HASH, W.IDENTITY} else None
    gf = fv if W.BUCKET in kinds else None
    y_ws = torch.full((w.batch, w.sum_dim), 7.0, dtype=torch.float32, device=dev)
    y_na = torch.full((w.batch, w.sum_dim), -7.0, dtype=torch.float32, device=dev)
    E.emb_forward(cols.plan, off, gi, gf, None, b.n, y_ws, cols.workspace, False)
    E.emb_forward_noalloc(cols.plan, off, gi, gf, None, b.n, y_na)
    torch.cuda.synchronize()
    return y_ws, y_na


@pytest.mark.parametrize("cfg", [3, 4])
def test_noalloc_equals_workspace_forward_twice(cfg):
    dev = torch.device("cuda")
    if cfg == 3:
        w = W.config(3, n_cols=200, batch=256, rows_range=(100, 5000))
        small = W.config(3, n_cols=200, batch=256, rows_range=(100, 5000), bag_hi=2)
    else:
        # bags of 200..2000 positions: most cross tile boundaries (partials + tickets)
        w = W.config(4, n_cols=4, batch=96, rows=40_000, training=False)
        small = W.config(4, n_cols=4, batch=96, rows=40_000, training=False, bag_lo=20, bag_hi=300)
    b1, off1, ids1, fv1 = _inputs(w, 5100 + cfg, dev)
    b2, off2, ids2, fv2 = _inputs(small, 5200 + cfg, dev)
    assert b2.n < b1.n
    wts, _ = W.make_tables(w, seed=5100 + cfg, device="cpu")
    gw = [t.to(dev) for t in wts]
    cols = E.EmbeddingColumns(w.cols, gw, batch=w.batch, max_ids=b1.n, opt=E.OPT_EMIT,
                              tile=128, device=dev)
    for b, off, ids, fv in ((b1, off1, ids1, fv1), (b2, off2, ids2, fv2)):
        y_ws, y_na = _both(cols, w, b, off, ids, fv, dev)
        assert torch.equal(y_ws, y_na), "the no-alloc forward differs from emb_forward"
        oc = oracle.Columns(w.cols, [to_np(t) for t in wts])
        Yr, Yb, _, _ = oracle.forward(oc, w.batch, b.offsets, b.ids, b.fvals)
        err = np.abs(to_np(y_na).astype(np.float64) - Yr)
        assert np.all(err <= RTOL_F32 * Yb), f"no-alloc forward vs oracle: {err.max()}"


def test_noalloc_refuses_a_batch_beyond_the_array():
    dev = torch.device("cuda")
    w = W.config(2, n_cols=2, batch=8, rows_range=(100, 200))
    for c in w.cols:
        c.dim = 256
    gw = [torch.zeros(c.rows, c.dim, device=dev) for c in w.cols]
    n = 40_000_000                     # 156250 tiles x 2 KiB of partials: far above 32 MiB
    cols = E.EmbeddingColumns(w.cols, gw, batch=w.batch, max_ids=n, opt=E.OPT_EMIT, device=dev)
    off = torch.zeros(len(w.cols) * w.batch + 1, dtype=torch.int32, device=dev)
    ids = torch.zeros(1, dtype=torch.int64, device=dev)
    y = torch.empty(w.batch, w.sum_dim, device=dev)
    with pytest.raises(E.EmbError) as ex:
        E.emb_forward_noalloc(cols.plan, off, ids, None, None, n, y)
    assert ex.value.status == 3 and "scratch" in str(ex.value)
