"""HIP path vs the CPU oracle, element by element, through the C ABI.

Integer results (transformed rows, bag of each position, valid counts per bag,
the distinct touched rows) must match bit-exactly; pooled outputs and gradients
within 1e-5 of sum |term| (fp32 accumulation in another order); updated rows
within the interval the oracle's update takes over that gradient error.
Sizes span many tiles with ragged tails; tiles of 64 positions force most bags
across tile boundaries (the split-bag combine)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_harness import (run_dense_case, Step, to_np, check_forward, check_rows_sgd, oracle_columns,
                         check_unique, check_emit)
import oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("tile", [64, 256])
def test_tiny_fused_bag_emit(tile):
    # 8 hashed columns, B=256, 1000 x 16 fp32 tables, bags of 1..4, EMIT of row grads
    run_dense_case(W.config(1), seed=1001, tile=tile)


@pytest.mark.parametrize("tile", [64, 192, 256])
def test_training_front_end_sgd(tile):
    # Poisson(3) bags, 5 % forced empty, 2 % invalid IDs, sum/mean, dims 8..64, SGD
    w = W.config(2, n_cols=24, batch=512, rows_range=(1e2, 1e4))
    run_dense_case(w, seed=2002, tile=tile)


def test_training_front_end_emit_mean_and_sum():
    w = W.config(2, n_cols=16, batch=300, rows_range=(30, 3000), opt=W.OPT_EMIT)
    run_dense_case(w, seed=2003, tile=128)


@pytest.mark.parametrize("training", [False, True])
def test_many_tiny_columns_inference(training):
    # 100 columns (70 hashed, 30 bucketized floats), dims 4..16, forward
    w = W.config(3, n_cols=100, batch=128, rows_range=(100, 1e4))
    run_dense_case(w, seed=3003, tile=256, training=training, check_bwd=False)


def test_many_tiny_columns_backward():
    w = W.config(3, n_cols=60, batch=96, rows_range=(100, 5000), opt=W.OPT_SGD, lr=0.01,
                 training=True)
    run_dense_case(w, seed=3004, tile=64)


@pytest.mark.parametrize("tile", [128, 256])
def test_long_sequences_bf16_adagrad(tile):
    # bags of 200..2000 IDs over 4 identity columns, bf16 tables, mean, Adagrad
    w = W.config(4, n_cols=4, batch=40, rows=100_000)
    run_dense_case(w, seed=4004, tile=tile)


@pytest.mark.parametrize("tile", [64, 256])
def test_training_front_end_sgd_segments_from_keys(tile):
    # the benchmark's backward: nothing asked back, segments found from the sorted keys
    w = W.config(2, n_cols=24, batch=512, rows_range=(1e2, 1e4))
    run_dense_case(w, seed=2012, tile=tile, ask_unique=False)


@pytest.mark.parametrize("tile", [64, 256])
def test_long_sequences_adagrad_segments_from_keys(tile):
    # hot rows: segments of thousands of contributors spanning many tiles
    w = W.config(4, n_cols=4, batch=40, rows=5_000)
    run_dense_case(w, seed=4014, tile=tile, ask_unique=False)


def test_many_tiny_columns_segments_from_keys():
    w = W.config(3, n_cols=60, batch=96, rows_range=(100, 5000), opt=W.OPT_SGD, lr=0.01,
                 training=True)
    run_dense_case(w, seed=3014, tile=64, ask_unique=False)


@pytest.mark.parametrize("ask_unique", [True, False])
def test_mixed_dtypes_sgd(ask_unique):
    # fp32 and bf16 columns in one plan, SGD (bf16 rows rounded to nearest even)
    w = W.config(2, n_cols=16, batch=300, rows_range=(100, 5000))
    for c, col in enumerate(w.cols):
        if c % 2:
            col.dtype = W.BF16
    run_dense_case(w, seed=2022, tile=128, ask_unique=ask_unique)


@pytest.mark.parametrize("ask_unique", [True, False])
def test_training_front_end_adagrad_fp32(ask_unique):
    # Adagrad on fp32 tables (the long-sequence workload has bf16 ones)
    w = W.config(2, n_cols=12, batch=256, rows_range=(100, 3000), opt=W.OPT_ADAGRAD, lr=0.05,
                 eps=1e-8)
    run_dense_case(w, seed=2032, tile=256, ask_unique=ask_unique)


def test_bucket_boundaries_beyond_lds():
    # more boundaries than the LDS stage holds: the search reads them from memory
    rng = np.random.default_rng(303)
    bnd = np.sort(rng.normal(size=300).astype(np.float32))
    cols = [W.Column(W.BUCKET, W.SUM, W.F32, 301, 8, boundaries=bnd),
            W.Column(W.BUCKET, W.MEAN, W.F32, 301, 16, boundaries=bnd[:200].copy())]
    lens = rng.integers(0, 6, size=2 * 120)
    n = int(lens.sum())
    fv = rng.normal(scale=1.5, size=n).astype(np.float32)
    fv[::17] = bnd[rng.integers(0, 200, size=fv[::17].size)]      # exact ties
    w, b = _custom(cols, lens, fvals=fv)
    _run_custom(w, b, 64)


def _atomic_sgd_case(w, b, seed, pweights=None):
    """The atomic-scatter SGD backward against the oracle's sorted sums.

    The row ends as E + sum_i t_i (t_i = -lr w_i g_i) added one term at a time in
    an unknown order.  Recursive fp32 summation of m terms onto E in any order is
    within (m + 2) u (|E| + sum |t_i|) of the exact sum (u = 2^-24; the extra 2 u
    cover the rounding of each t_i), on top of the sorted path's tolerance."""
    wts, sts = W.make_tables(w, seed=seed, device="cpu")
    G = W.make_grad(w, seed=seed, device="cpu")
    st = Step(w, b, wts, sts, tile=256)
    st.forward(training=True, pweights=pweights)
    st.cols.backward_atomic(G.to("cuda"))
    torch.cuda.synchronize()
    host_w = [to_np(t) for t in wts]
    oc = oracle_columns(w, [x.copy() for x in host_w])
    _, _, _, rows = oracle.forward(oc, w.batch, b.offsets, b.ids, b.fvals, pweights=pweights)
    ucol, urow, ug, ub = oracle.backward(oc, w.batch, b.offsets, G.numpy(), b.ids, b.fvals,
                                         opt=w.opt, lr=w.lr, pweights=pweights)
    from gpu_harness import positions_columns, as_f64
    _, pcol = positions_columns(b.offsets, len(w.cols), w.batch)
    for c, col in enumerate(w.cols):
        sel = ucol == c
        touched = urow[sel]
        m = np.bincount(rows[(pcol == c) & (rows >= 0)].astype(np.int64), minlength=col.rows)[touched]
        before, after, ref = host_w[c], to_np(st.gw[c]), oc.weights[c]
        untouched = np.setdiff1d(np.arange(col.rows), touched)
        assert np.array_equal(after[untouched], before[untouched]), "untouched rows changed"
        e0 = as_f64(col, before[touched])
        gb = ub[sel][:, :col.dim]
        tol = (w.lr * 1e-5 * gb + 2.0 ** -22 * (np.abs(ref[touched]) + np.abs(e0))
               + (m[:, None] + 2) * 2.0 ** -24 * (np.abs(e0) + w.lr * gb) + 1e-30)
        d = np.abs(as_f64(col, after[touched]) - ref[touched].astype(np.float64))
        assert np.all(d <= tol), f"rows differ: max {d.max()} tol {tol[d > tol][:3]}"


def test_atomic_backward_sgd():
    # the pages' backward (atomic adds, no sort) on the training front end's shape
    w = W.config(2, n_cols=24, batch=512, rows_range=(1e2, 1e4))
    _atomic_sgd_case(w, W.make_batch(w, seed=2042), 2042)


def test_atomic_backward_weighted():
    # per-position weights reach the atomic backward through the workspace
    w = W.config(2, n_cols=16, batch=400, rows_range=(1e2, 1e4))
    b = W.make_batch(w, seed=2043)
    _atomic_sgd_case(w, b, 2043, pweights=W.make_position_weights(b.n, 2043))


def test_atomic_backward_hot_row():
    # 5000 contributions to one row (mean bags): the unordered fp32 adds stay
    # inside the tolerance of the sorted sums
    cols = [W.Column(W.IDENTITY, W.MEAN, W.F32, 50, 32)]
    lens = [3, 2500, 0, 2500, 1, 4]
    n = sum(lens)
    ids = np.full(n, 7, dtype=np.int64)
    ids[:3] = [1, 2, 7]
    ids[-5:] = [49, 0, 7, 3, 3]
    w, b = _custom(cols, lens, ids=ids, opt=W.OPT_SGD, lr=0.01)
    _atomic_sgd_case(w, b, 12)


def test_deterministic_across_runs():
    w = W.config(2, n_cols=12, batch=256, rows_range=(50, 2000), opt=W.OPT_EMIT)
    a = run_dense_case(w, seed=5, tile=64)
    b = run_dense_case(w, seed=5, tile=64)
    assert torch.equal(a["Y"], b["Y"])
    n = int(a["nu"].item())
    assert torch.equal(a["ukeys"][:n], b["ukeys"][:n])
    # gradient rows are padded to the widest column; compare each row's own dims
    rb = np.concatenate([[0], np.cumsum([c.rows for c in w.cols])])
    keys = to_np(a["ukeys"][:n]).astype(np.int64)
    dims = np.array([c.dim for c in w.cols])[np.searchsorted(rb, keys, side="right") - 1]
    ga, gb = to_np(a["ugrads"][:n]), to_np(b["ugrads"][:n])
    for u in range(n):
        assert np.array_equal(ga[u, :dims[u]], gb[u, :dims[u]])


# ------------------------------------------------------------------ edges

def _custom(cols, lens, ids=None, fvals=None, B=None, opt=W.OPT_EMIT, lr=0.0):
    C = len(cols)
    B = B or len(lens) // C
    off = np.zeros(C * B + 1, dtype=np.int32)
    off[1:] = np.cumsum(lens)
    n = int(off[-1])
    rng = np.random.default_rng(n + C)
    ids = ids if ids is not None else rng.integers(0, 1 << 40, size=n, dtype=np.int64)
    fvals = fvals if fvals is not None else rng.normal(size=n).astype(np.float32)
    w = W.Workload("edge", cols, B, "fixed", opt=opt, lr=lr)
    b = W.Batch(off, ids, fvals, np.zeros(n, bool), np.zeros(C * B, bool), n)
    return w, b


def _run_custom(w, b, tile, seed=0):
    wts, sts = W.make_tables(w, seed=seed, device="cpu")
    G = W.make_grad(w, seed=seed, device="cpu")
    st = Step(w, b, wts, sts, tile=tile)
    Y = st.forward(training=True)
    ws = st.cols.workspace_view(max(b.n, 1))
    host_w = [to_np(t) for t in wts]
    oc = oracle_columns(w, [x.copy() for x in host_w])
    ref = oracle.forward(oc, w.batch, b.offsets, b.ids, b.fvals)
    torch.cuda.synchronize()
    check_forward(w, b, Y, (ws[0][:b.n], ws[1][:b.n], ws[2]), ref)
    ukeys, ugrads, nu = st.backward(G)
    torch.cuda.synchronize()
    ucol, urow, ug, ub = oracle.backward(oc, w.batch, b.offsets, G.numpy(), b.ids, b.fvals)
    n = int(nu.item())
    assert n == ucol.size
    rb = np.concatenate([[0], np.cumsum([c.rows for c in w.cols])])
    assert np.array_equal(to_np(ukeys[:n]).astype(np.int64), rb[ucol] + urow)
    # lanes past a column's width are not written: convert only the written ones
    g = to_np(ugrads[:n])
    for u in range(n):
        D = w.cols[ucol[u]].dim
        assert np.all(np.abs(g[u, :D].astype(np.float64) - ug[u, :D]) <= 1e-5 * ub[u, :D])
    return Y


def _hash_cols(n, dim=16, rows=97, pool=W.SUM):
    return [W.Column(W.HASH, pool, W.F32, rows, dim, 0, 1 << 40) for _ in range(n)]


def test_all_bags_empty():
    w, b = _custom(_hash_cols(3), [0] * 30)
    Y = _run_custom(w, b, 64)
    assert torch.count_nonzero(Y) == 0


@pytest.mark.parametrize("tile", [64, 256])
def test_one_bag_spanning_many_tiles(tile):
    # one 5000-position bag between empty bags: pieces from ~80 tiles combine
    lens = [0, 5000, 0, 3, 0, 0]
    w, b = _custom(_hash_cols(2, dim=32, pool=W.MEAN), lens)
    _run_custom(w, b, tile)


@pytest.mark.parametrize("tile", [64, 256])
def test_hot_row_segment_spanning_many_tiles_sgd(tile):
    # one row looked up 5000 times (plus a few others): with nothing asked back,
    # the segment's start and end tiles are found by searching the sorted keys
    cols = [W.Column(W.IDENTITY, W.MEAN, W.F32, 50, 32)]
    lens = [3, 2500, 0, 2500, 1, 4]
    n = sum(lens)
    ids = np.full(n, 7, dtype=np.int64)
    ids[:3] = [1, 2, 7]
    ids[-5:] = [49, 0, 7, 3, 3]
    w, b = _custom(cols, lens, ids=ids, opt=W.OPT_SGD, lr=0.01)
    wts, sts = W.make_tables(w, seed=11, device="cpu")
    G = W.make_grad(w, seed=11, device="cpu")
    st = Step(w, b, wts, sts, tile=tile)
    st.forward(training=True)
    st.backward(G, ask_unique=False)
    torch.cuda.synchronize()
    host_w = to_np(wts[0])
    oc = oracle_columns(w, [host_w.copy()])
    ucol, urow, ug, ub = oracle.backward(oc, w.batch, b.offsets, G.numpy(), b.ids, b.fvals,
                                         opt=w.opt, lr=w.lr)
    check_rows_sgd(cols[0], host_w, to_np(st.gw[0]), oc.weights[0], urow, ub[:, :32], w.lr)


@pytest.mark.parametrize("big", [12288, 12289, 20000, 40000])
def test_segments_from_keys_column_sort_capacity(big):
    # the column-local sort takes columns of up to 12288 positions; one larger
    # column sends the whole step to the global radix passes (behind the column
    # sort while n <= 3 * 12288, without it beyond)
    cols = [W.Column(W.HASH, W.SUM, W.F32, 300, 16, 0, 1 << 40),
            W.Column(W.IDENTITY, W.MEAN, W.F32, 5000, 8),
            W.Column(W.HASH, W.MEAN, W.F32, 40, 32, 0, 1 << 40)]
    B = 8
    lens = [5] * B + [0] * (B - 1) + [big] + [3, 0, 1, 700, 2, 2, 9, 4]
    n = sum(lens)
    rng = np.random.default_rng(big)
    ids = rng.integers(-3, 5200, size=n, dtype=np.int64)
    w, b = _custom(cols, lens, ids=ids, B=B, opt=W.OPT_SGD, lr=0.01)
    wts, sts = W.make_tables(w, seed=13, device="cpu")
    G = W.make_grad(w, seed=13, device="cpu")
    st = Step(w, b, wts, sts, tile=256)
    st.forward(training=True)
    st.backward(G, ask_unique=False)
    torch.cuda.synchronize()
    host_w = [to_np(x) for x in wts]
    oc = oracle_columns(w, [x.copy() for x in host_w])
    ucol, urow, ug, ub = oracle.backward(oc, w.batch, b.offsets, G.numpy(), b.ids, b.fvals,
                                         opt=w.opt, lr=w.lr)
    for c, col in enumerate(cols):
        sel = ucol == c
        check_rows_sgd(col, host_w[c], to_np(st.gw[c]), oc.weights[c], urow[sel], ub[sel][:, :col.dim], w.lr)


@pytest.mark.parametrize("mode", ["sgd_unique", "emit"])
@pytest.mark.parametrize("mid_rows", [5000, 20000])
@pytest.mark.parametrize("big", [12289, 20000])
def test_column_sort_oversized_column_with_unique_list(big, mid_rows, mode):
    # one column above the LDS capacity while the average column still fits: the
    # oversized column is sorted through global memory in 7-bit passes (2 for
    # 5000 rows, 3 for 20000: the result then ends in the other buffer), the
    # valid keys of every column are counted and compacted into one sorted run,
    # and the unique-row list is built from it
    cols = [W.Column(W.HASH, W.SUM, W.F32, 300, 16, 0, 1 << 40),
            W.Column(W.IDENTITY, W.MEAN, W.F32, mid_rows, 8),
            W.Column(W.HASH, W.MEAN, W.F32, 40, 32, 0, 1 << 40)]
    B = 8
    lens = [5] * B + [0] * (B - 1) + [big] + [3, 0, 1, 700, 2, 2, 9, 4]
    n = sum(lens)
    rng = np.random.default_rng(big + mid_rows)
    ids = rng.integers(-3, mid_rows + 200, size=n, dtype=np.int64)
    opt = W.OPT_EMIT if mode == "emit" else W.OPT_SGD
    w, b = _custom(cols, lens, ids=ids, B=B, opt=opt, lr=0.01)
    wts, sts = W.make_tables(w, seed=14, device="cpu")
    G = W.make_grad(w, seed=14, device="cpu")
    st = Step(w, b, wts, sts, tile=256)
    st.forward(training=True)
    ukeys, ugrads, nu = st.backward(G, ask_unique=True)
    torch.cuda.synchronize()
    host_w = [to_np(x) for x in wts]
    oc = oracle_columns(w, [x.copy() for x in host_w])
    ucol, urow, ug, ub = oracle.backward(oc, w.batch, b.offsets, G.numpy(), b.ids, b.fvals,
                                         opt=w.opt, lr=w.lr)
    check_unique(w, ukeys, nu, ucol, urow)
    if opt == W.OPT_EMIT:
        check_emit(w, ugrads, int(nu.item()), ucol, ug, ub)
        return
    for c, col in enumerate(cols):
        sel = ucol == c
        check_rows_sgd(col, host_w[c], to_np(st.gw[c]), oc.weights[c], urow[sel], ub[sel][:, :col.dim], w.lr)


def test_single_position_and_all_invalid():
    cols = _hash_cols(2, dim=8)
    w, b = _custom(cols, [1, 0, 0, 4], ids=np.array([5, -1, -7, 1 << 41, -2], dtype=np.int64))
    Y = _run_custom(w, b, 64)
    assert torch.count_nonzero(Y[1]) == 0


@pytest.mark.parametrize("dtype,dim", [(W.F32, 256), (W.F32, 4), (W.BF16, 256), (W.BF16, 8),
                                       (W.F32, 12), (W.BF16, 24)])
def test_dims_and_dtypes(dtype, dim):
    cols = [W.Column(W.IDENTITY, W.MEAN, dtype, 50, dim), W.Column(W.HASH, W.SUM, dtype, 31, dim, 0, 1 << 40)]
    rng = np.random.default_rng(dim)
    lens = rng.integers(0, 40, size=2 * 70)
    n = int(lens.sum())
    ids = rng.integers(-3, 60, size=n).astype(np.int64)
    w, b = _custom(cols, lens, ids=ids)
    _run_custom(w, b, 128)


def test_many_columns_tiny_batch():
    # 300 columns with B=1: a tile spans many column segments
    cols = [W.Column(W.HASH, W.SUM if c % 3 else W.MEAN, W.F32, 7 + c, 4 * (1 + c % 4), 0, 1 << 40)
            for c in range(300)]
    rng = np.random.default_rng(9)
    w, b = _custom(cols, rng.integers(0, 4, size=300), B=1)
    _run_custom(w, b, 64)


def test_bucket_edges():
    bnd = np.array([-1.0, 0.0, 0.0, 2.5], dtype=np.float32)
    cols = [W.Column(W.BUCKET, W.SUM, W.F32, 5, 8, boundaries=bnd),
            W.Column(W.BUCKET, W.MEAN, W.F32, 9, 4, boundaries=bnd)]
    fv = np.array([np.nan, -1.0, 0.0, -0.0, 2.5, np.inf, -np.inf, 1e-45, 3.0, -1.0000001, np.nan,
                   0.5], dtype=np.float32)
    w, b = _custom(cols, [3, 3, 0, 2, 4, 0], fvals=fv)
    _run_custom(w, b, 64)


def test_stats_counts():
    w = W.config(2, n_cols=10, batch=200, rows_range=(100, 1000), opt=W.OPT_EMIT)
    out = run_dense_case(w, seed=77, tile=128)
    st, b = out["step"], out["batch"]
    s = to_np(st.stats)
    assert s[0] == b.n
    assert s[2] == int(b.invalid_mask.sum())          # dropped = generator's invalid IDs
    assert s[1] == b.n - s[2]
    lens = np.diff(b.offsets)
    assert s[4] >= int((lens == 0).sum())             # at least the empty bags are zero
    assert s[5] == int(out["nu"].item())
