"""Keyed table on the GPU vs the oracle's table model (Monolith Sec. 2.1: a
collisionless key-value table whose IDs are admitted after a tunable number of
occurrences), through the C ABI.

Slot placement and row indices are the implementation's choice (several results
are correct), so the comparison is over what the method fixes: the exported key
set, each key's count and admission, the per-occurrence outcome (row / DEFAULT /
dropped), distinct rows for distinct admitted keys, new-row values (bit-exact),
and the pooled outputs and updated rows of a training step."""
import numpy as np
import pytest
import torch

import embedding_columns_amd as E
import oracle
import workloads as W
from gpu_harness import RTOL_F32, to_np
from oracle.table import OracleTable

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _keyed_workload(cap, prepop, batch, key_space):
    w = W.config(5, capacity=cap, row_capacity=cap, prepop=prepop, batch=batch)
    w.key_space = key_space
    return w


def _setup(w, seed):
    pk = W.prepop_keys(w.prepop)
    prows = W.make_prepop_rows(w.prepop, 32, 0.01, seed, device="cpu")
    T = E.KeyedTable(w.capacity, w.row_capacity, 32, threshold=w.threshold, init_std=0.01, device=DEV)
    stats = torch.zeros(E.STAT_COUNT, dtype=torch.int64, device=DEV)
    T.bulk_insert(torch.from_numpy(pk).to(DEV), prows.to(DEV), stats=stats)
    O = OracleTable(w.capacity, 32, w.threshold, 0.01, pk, prows.numpy())
    return T, O, stats


@pytest.mark.parametrize("key_space", [20_000, W.KEY_SPACE_63])
def test_keyed_training_steps(key_space):
    # small universe: many repeats, admissions across steps; full 2^63: mostly unseen keys
    w = _keyed_workload(1 << 16, 3000, 96, key_space)
    T, O, stats = _setup(w, seed=55)
    bound = {}            # key -> accumulated lr * sum |w G| (fp32 error scale of its row)
    seen = set()
    for step in range(3):
        b = W.make_batch(w, seed=5000 + step)
        G = W.make_grad(w, seed=5000 + step, device="cpu")
        keys = torch.from_numpy(b.ids).to(DEV)
        rows = T.lookup_or_insert(keys, stats=stats)
        cols = E.EmbeddingColumns(w.cols, [T.rows], batch=w.batch, max_ids=b.n, opt=W.OPT_SGD,
                                  lr=w.lr, device=DEV)
        off = torch.from_numpy(b.offsets).to(DEV)
        Y = cols.forward(off, keyed_rows=rows, training=True)
        cols.backward(G.to(DEV))
        torch.cuda.synchronize()

        # oracle: table step, forward, backward with SGD on its own rows
        O.step(b.ids)
        krows, pool_keys, pool = O.resolve(b.ids)
        col = W.Column(W.KEYED, W.SUM, W.F32, max(pool.shape[0], 1), 32)
        pool = pool if pool.shape[0] else np.zeros((1, 32), np.float32)
        oc = oracle.Columns([col], [pool.copy()])
        Yr, Yb, bag_n, _ = oracle.forward(oc, w.batch, b.offsets, keyed_rows=krows)
        ucol, urow, ug, ub = oracle.backward(oc, w.batch, b.offsets, G.numpy(), keyed_rows=krows,
                                             opt=W.OPT_SGD, lr=w.lr)
        O.store(pool_keys, oc.weights[0])
        for r, bb in zip(urow, ub):
            k = int(pool_keys[r])
            bound[k] = bound.get(k, 0.0) + w.lr * bb[:32]

        # per-occurrence outcome: same admitted / DEFAULT / dropped decisions
        g_rows = to_np(rows)
        assert np.array_equal(g_rows == E.ROW_DEFAULT, krows == oracle.ROW_DEFAULT)
        assert np.array_equal(g_rows == E.ROW_DROPPED, krows == oracle.ROW_DROPPED)
        # collisionless: one row per admitted key, distinct keys -> distinct rows
        adm = g_rows >= 0
        pairs = np.unique(np.stack([b.ids[adm], g_rows[adm]]), axis=1)
        assert np.unique(pairs[0]).size == pairs.shape[1] == np.unique(pairs[1]).size
        # rows updated in earlier steps carry their own fp32 error: add it per bag
        slack = np.zeros((b.n, 32))
        for p, k in enumerate(b.ids.tolist()):
            if k in bound and krows[p] >= 0:
                slack[p] = RTOL_F32 * (np.abs(pool[krows[p]]) + bound[k])
        lens = np.diff(b.offsets)
        bag_slack = np.zeros((w.batch, 32))
        nz = lens > 0
        bag_slack[nz] = np.add.reduceat(slack, b.offsets[:-1][nz], axis=0) if b.n else 0
        err = np.abs(to_np(Y).astype(np.float64) - Yr)
        assert np.all(err <= RTOL_F32 * Yb + bag_slack + 1e-12), "pooled outputs differ"
        seen.update(b.ids[b.ids >= 1].tolist())

    # table state after the steps: set equality, counts, admission, row values
    gk, gc, gr = (to_np(x) for x in T.export())
    assert np.unique(gk).size == gk.size, "a key occupies two slots"
    want = set(O.keys.tolist())
    assert set(gk.tolist()) == want
    order = np.argsort(gk)
    gk, gc, gr = gk[order], gc[order], gr[order]
    present, oc_cnt, oc_adm = O.state(gk)
    assert present.all()
    assert np.array_equal(gc, oc_cnt), "occurrence counts differ"
    assert np.array_equal(gr >= 0, oc_adm), "admitted sets differ"
    sk = np.array(sorted(seen), dtype=np.int64)
    _, _, adm_seen = O.state(sk)
    sk = sk[adm_seen]
    grow, gcnt = T.find(torch.from_numpy(sk).to(DEV))
    grow = to_np(grow)
    assert np.all(grow >= 0)
    gvals = to_np(T.rows[torch.from_numpy(grow).long().to(DEV)])
    ovals = O.row_values(sk)
    tol = np.array([RTOL_F32 * (np.abs(ovals[i]) + bound.get(int(k), 0.0)) + 1e-9
                    for i, k in enumerate(sk)])
    assert np.all(np.abs(gvals - ovals) <= tol), "row values differ"
    s = to_np(stats)
    assert s[E.STAT_NAMES.index("table_full")] == 0


def test_new_rows_bit_exact_and_threshold():
    T = E.KeyedTable(1 << 10, 1 << 10, 32, threshold=3, init_std=0.01, device=DEV)
    keys = torch.tensor([7, 7, 9, 9, 9, 11, 0, -5, 13, 13, 13, 13], dtype=torch.int64, device=DEV)
    rows = to_np(T.lookup_or_insert(keys))
    assert rows[0] == rows[1] == E.ROW_DEFAULT          # 2 < threshold
    assert rows[2] == rows[3] == rows[4] >= 0           # admitted on its third occurrence
    assert rows[5] == E.ROW_DEFAULT and rows[6] == rows[7] == E.ROW_DROPPED
    assert rows[8] >= 0 and rows[8] != rows[2]
    torch.cuda.synchronize()
    for k, r in ((9, rows[2]), (13, rows[8])):
        assert np.array_equal(to_np(T.rows[int(r)]), oracle.init_row(k, 32, 0.01))
    # the second step admits 7 (count 2 -> 3) and keeps 9's row
    rows2 = to_np(T.lookup_or_insert(torch.tensor([7, 9], dtype=torch.int64, device=DEV)))
    assert rows2[0] >= 0 and rows2[1] == rows[2]
    _, cnt = T.find(torch.tensor([7, 9, 11, 12], dtype=torch.int64, device=DEV))
    assert to_np(cnt).tolist() == [3, 4, 1, 0]


def test_table_full_refuses_without_hanging():
    cap = 64
    T = E.KeyedTable(cap, cap, 8, threshold=1, init_std=0.0, device=DEV)
    stats = torch.zeros(E.STAT_COUNT, dtype=torch.int64, device=DEV)
    keys = torch.arange(1, 201, dtype=torch.int64, device=DEV)
    rows = to_np(T.lookup_or_insert(keys, stats=stats))
    gk, gc, gr = (to_np(x) for x in T.export())
    assert gk.size == cap and set(gk.tolist()) <= set(range(1, 201))
    inserted = set(gk.tolist())
    for k, r in zip(range(1, 201), rows):
        assert (r >= 0) == (k in inserted)                  # refused keys read DEFAULT
    s = to_np(stats)
    assert s[E.STAT_NAMES.index("table_full")] == 200 - cap
    assert s[E.STAT_NAMES.index("table_inserted")] == cap
    assert np.all(to_np(T.rows[:cap]) == 0)                 # init_std = 0 -> zero rows


def test_table_high_load_probing():
    # 3900 distinct keys in 4096 slots (load 0.95): every probe sequence still
    # finds its key, distinct keys keep distinct rows, absent keys are not found
    cap = 1 << 12
    T = E.KeyedTable(cap, cap, 8, threshold=1, init_std=0.01, device=DEV)
    rng = np.random.default_rng(77)
    keys = np.unique(rng.integers(1, 1 << 62, size=4000, dtype=np.int64))[:3900]
    rng.shuffle(keys)
    kt = torch.from_numpy(keys).to(DEV)
    # inserted in two halves, the second probing past the first's keys
    r1 = to_np(T.lookup_or_insert(kt[:1950]))
    r2 = to_np(T.lookup_or_insert(kt[1950:]))
    rows = np.concatenate([r1, r2])
    assert np.all(rows >= 0) and np.unique(rows).size == keys.size
    fr, fc = T.find(kt)
    assert np.array_equal(to_np(fr), rows)
    assert np.all(to_np(fc) == 1)
    absent = np.setdiff1d(rng.integers(1, 1 << 62, size=500, dtype=np.int64), keys)
    ar, _ = T.find(torch.from_numpy(absent).to(DEV))
    assert np.all(to_np(ar) == E.ROW_DROPPED)
    gk, gc, gr = (to_np(x) for x in T.export())
    assert set(gk.tolist()) == set(keys.tolist())


def test_keyed_column_with_transform_variants():
    """A KEYED column with truncation, a mask, per-position weights and a default
    row: the rows come from the table, the rest as for hashed columns."""
    w = _keyed_workload(1 << 14, 500, 64, 3000)
    w.empty_frac = 0.3                       # empty bags read the default row
    w.cols[0].seq_max, w.cols[0].seq_keep_last = 40, 1
    w.cols[0].default_row = 5
    T, O, _ = _setup(w, seed=56)
    b = W.make_batch(w, seed=5600)
    mask = W.make_mask(b.n, 5600, 0.8)
    pw = W.make_position_weights(b.n, 5600)
    G = W.make_grad(w, seed=5600, device="cpu")
    rows = T.lookup_or_insert(torch.from_numpy(b.ids).to(DEV))
    torch.cuda.synchronize()
    before = to_np(T.rows).copy()
    cols = E.EmbeddingColumns(w.cols, [T.rows], batch=w.batch, max_ids=b.n, opt=W.OPT_SGD,
                              lr=w.lr, device=DEV)
    off = torch.from_numpy(b.offsets).to(DEV)
    Y = cols.forward(off, keyed_rows=rows, training=True,
                     weights=torch.from_numpy(pw).to(DEV), mask=torch.from_numpy(mask).to(DEV))
    cols.backward(G.to(DEV), want_count=False)
    torch.cuda.synchronize()
    # oracle on the GPU's own row indices (the table's placement is its choice)
    oc = oracle.Columns(w.cols, [before.copy()])
    g_rows = to_np(rows)
    Yr, Yb, _, _ = oracle.forward(oc, w.batch, b.offsets, keyed_rows=g_rows, mask=mask, pweights=pw)
    err = np.abs(to_np(Y).astype(np.float64) - Yr)
    assert np.all(err <= RTOL_F32 * Yb + 1e-12), "pooled outputs differ"
    ucol, urow, ug, ub = oracle.backward(oc, w.batch, b.offsets, G.numpy(), keyed_rows=g_rows,
                                         opt=W.OPT_SGD, lr=w.lr, mask=mask, pweights=pw)
    after = to_np(T.rows)
    d = np.abs(after[urow].astype(np.float64) - oc.weights[0][urow])
    tol = w.lr * RTOL_F32 * ub[:, :32] + 2.0 ** -22 * (np.abs(before[urow]) + np.abs(after[urow])) + 1e-30
    assert np.all(d <= tol), "updated rows differ"
    untouched = np.setdiff1d(np.arange(before.shape[0]), urow)
    # bitwise: pool rows no key owns are uninitialized memory (any bit pattern)
    assert np.array_equal(after[untouched].view(np.uint32), before[untouched].view(np.uint32))
    assert 5 in set(urow.tolist())           # the default row took the empty bags' gradient
