"""Keyed-table lifecycle on the GPU vs the oracle's table model: last-seen steps,
eviction with compaction and row reuse, checkpoint save / load (Monolith Sec. 2.1
expires inactive IDs).  As in the other table tests, slot placement and row
indices are the implementation's choice; the comparison covers the key set,
counts, last-seen steps, admission, per-occurrence outcomes and row values."""
import numpy as np
import pytest
import torch

import embedding_columns_amd as E
import oracle
import workloads as W
from gpu_harness import to_np
from oracle.table import OracleTable

pytestmark = pytest.mark.gpu
DEV = "cuda"
DIM = 16


def _batches(n_steps, seed, universe=3000, size=700):
    rng = np.random.default_rng(seed)
    z = W.ZipfSampler(universe, 1.05)
    out = []
    for _ in range(n_steps):
        k = z.sample(rng, size).astype(np.int64)
        k[rng.random(size) < 0.03] = 0                 # a few invalid keys
        out.append(k)
    return out


def _state(T):
    keys, counts, seen, adm, vals, step = T.save()
    keys, counts, seen, adm, vals = (to_np(x) for x in (keys, counts, seen, adm, vals))
    o = np.argsort(keys)
    return keys[o], counts[o], seen[o], adm[o].astype(bool), vals[o], step


def _check_against_model(T, O):
    keys, counts, seen, adm, vals, step = _state(T)
    assert np.array_equal(keys, O.keys), "key sets differ"
    assert np.array_equal(counts, O.count) and np.array_equal(seen, O.seen)
    assert np.array_equal(adm, O.admitted) and step == O.step_no
    if adm.any():
        assert np.array_equal(vals[adm], O.row_values(keys[adm])), "row values differ"


@pytest.mark.parametrize("threshold", [1, 2])
def test_eviction_steps_vs_model(threshold):
    steps = _batches(12, 31 + threshold)
    pre = np.arange(2001, 2101, dtype=np.int64)         # prepopulated, never seen again
    pre_rows = np.random.default_rng(5).normal(size=(pre.size, DIM)).astype(np.float32)
    evict_at = {2: 1, 5: 4, 8: 6, 11: 10}               # after step s: evict keys seen before m
    # rows needed at the peak: the model's largest admitted-key count at any time
    O = OracleTable(1 << 13, DIM, threshold, 0.01, pre, pre_rows)
    peak, admitted_total = int(O.admitted.sum()), 0
    for s, k in enumerate(steps):
        before = int(O.admitted.sum())
        O.step(k)
        peak = max(peak, int(O.admitted.sum()))
        admitted_total += int(O.admitted.sum()) - before
        if s in evict_at:
            O.evict(evict_at[s])
    assert admitted_total + pre.size > peak              # rows must be reused to finish

    T = E.KeyedTable(1 << 13, peak, DIM, threshold=threshold, init_std=0.01, device=DEV,
                     track_seen=True)
    stats = torch.zeros(E.STAT_COUNT, dtype=torch.int64, device=DEV)
    T.bulk_insert(torch.from_numpy(pre).to(DEV), torch.from_numpy(pre_rows).to(DEV), stats=stats)
    O = OracleTable(1 << 13, DIM, threshold, 0.01, pre, pre_rows)
    for s, k in enumerate(steps):
        rows = to_np(T.lookup_or_insert(torch.from_numpy(k).to(DEV), stats=stats))
        O.step(k)
        krows, pool_keys, pool = O.resolve(k)
        assert np.array_equal(rows == E.ROW_DEFAULT, krows == oracle.ROW_DEFAULT)
        assert np.array_equal(rows == E.ROW_DROPPED, krows == oracle.ROW_DROPPED)
        adm = rows >= 0
        # collisionless with reused rows: distinct admitted keys hold distinct rows
        pairs = np.unique(np.stack([k[adm], rows[adm]]), axis=1)
        assert np.unique(pairs[0]).size == pairs.shape[1] == np.unique(pairs[1]).size
        got = to_np(T.rows[torch.from_numpy(rows[adm]).long().to(DEV)])
        assert np.array_equal(got, pool[krows[adm]]), "row values read differ"
        if s in evict_at:
            n_live = T.evict(evict_at[s], stats=stats)
            n_ev = O.evict(evict_at[s])
            assert int(n_live.item()) == O.keys.size and n_ev > 0
        _check_against_model(T, O)
    st = to_np(stats)
    assert st[E.STAT_NAMES.index("table_full")] == 0
    assert st[E.STAT_NAMES.index("table_evicted")] > 0


def test_checkpoint_roundtrip():
    steps = _batches(6, 77)
    T = E.KeyedTable(1 << 12, 1 << 11, DIM, threshold=2, init_std=0.01, device=DEV,
                     track_seen=True)
    O = OracleTable(1 << 12, DIM, 2, 0.01)
    for s, k in enumerate(steps[:4]):
        T.lookup_or_insert(torch.from_numpy(k).to(DEV))
        O.step(k)
        if s == 2:
            T.evict(1)
            O.evict(1)
    # the saved rows carry changes a training step would make
    T.rows.mul_(1.5)
    O2 = OracleTable.restore(1 << 12, DIM, 2, 0.01, O.checkpoint())
    ck = O2.checkpoint()
    adm = ck[3]
    O2.store(ck[0][adm], ck[4][adm] * np.float32(1.5))
    R = E.KeyedTable(1 << 12, 1 << 11, DIM, threshold=2, init_std=0.01, device=DEV,
                     track_seen=True)
    R.load(T.save())
    _check_against_model(T, O2)
    _check_against_model(R, O2)
    for k in steps[4:]:
        kt = torch.from_numpy(k).to(DEV)
        a, b = to_np(T.lookup_or_insert(kt)), to_np(R.lookup_or_insert(kt))
        assert np.array_equal(a >= 0, b >= 0) and np.array_equal(a < 0, b < 0)
        assert np.array_equal(a[a < 0], b[a < 0])
        va = to_np(T.rows[torch.from_numpy(a[a >= 0]).long().to(DEV)])
        vb = to_np(R.rows[torch.from_numpy(b[b >= 0]).long().to(DEV)])
        assert np.array_equal(va, vb)
        O2.step(k)
    _check_against_model(R, O2)
    sa, sb = _state(T), _state(R)
    for x, y in zip(sa, sb):
        assert np.array_equal(x, y)


def test_evict_zeroes_freed_optimizer_state():
    T = E.KeyedTable(1 << 10, 256, DIM, threshold=1, init_std=0.01, device=DEV,
                     track_seen=True)
    state = torch.full((256, DIM), 7.0, dtype=torch.float32, device=DEV)
    old = to_np(T.lookup_or_insert(torch.arange(1, 41, dtype=torch.int64, device=DEV)))
    new = to_np(T.lookup_or_insert(torch.arange(31, 61, dtype=torch.int64, device=DEV)))
    T.evict(1, opt_state=state)                          # keys 1..30 were last seen at step 0
    st = to_np(state)
    assert np.all(st[old[:30]] == 0) and np.all(st[new] == 7.0)
    # the freed rows serve the next admissions
    again = to_np(T.lookup_or_insert(torch.arange(100, 130, dtype=torch.int64, device=DEV)))
    assert set(again.tolist()) == set(old[:30].tolist())


@pytest.mark.parametrize("depth,width", [(2, 64), (3, 1 << 20)])
def test_count_min_admission_vs_model(depth, width):
    """Count-min admission: absent keys live only in the sketch until their
    estimate reaches the threshold (a narrow sketch admits early through
    collisions, a wide one like exact counting); per step the key set, counts,
    admission, outcomes and row values match the model."""
    steps = _batches(8, 91 + depth, universe=2000, size=600)
    T = E.KeyedTable(1 << 12, 1 << 12, DIM, threshold=3, init_std=0.01, device=DEV,
                     track_seen=True)
    T.use_count_min(depth, width)
    O = OracleTable(1 << 12, DIM, 3, 0.01)
    O.use_count_min(depth, width)
    for s, k in enumerate(steps):
        rows = to_np(T.lookup_or_insert(torch.from_numpy(k).to(DEV)))
        O.step(k)
        krows, pool_keys, pool = O.resolve(k)
        assert np.array_equal(rows == E.ROW_DEFAULT, krows == oracle.ROW_DEFAULT)
        assert np.array_equal(rows == E.ROW_DROPPED, krows == oracle.ROW_DROPPED)
        adm = rows >= 0
        got = to_np(T.rows[torch.from_numpy(rows[adm]).long().to(DEV)])
        assert np.array_equal(got, pool[krows[adm]])
        _check_against_model(T, O)
        assert np.array_equal(to_np(T.sketch).astype(np.int64), O.sketch), "sketch counters differ"
        if s == 4:
            T.evict(3)
            O.evict(3)
            _check_against_model(T, O)
