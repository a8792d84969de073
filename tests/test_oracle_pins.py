"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each test ties one oracle function to a published value, a library routine that
computes the same special case, a closed form, an invariant, or a brute force on
tiny inputs, so that a dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.table import OracleTable

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GAMMA = 0x9E3779B97F4A7C15
M64 = (1 << 64) - 1


# ----------------------------------------------------------------- helpers

def _tiny_case(rng, kinds=(W.HASH, W.IDENTITY, W.BUCKET), C=4, B=6, max_len=5, rows_hi=7,
               dims=(4, 8), dtype=W.F32, pools=(W.SUM, W.MEAN), invalid=0.2):
    """A tiny batch with many collisions, duplicates, empty bags and invalid IDs."""
    cols = []
    bnd = np.sort(rng.normal(size=5).astype(np.float32))
    for c in range(C):
        kind = kinds[c % len(kinds)]
        rows = int(rng.integers(1, rows_hi + 1))
        if kind == W.BUCKET:
            rows = max(rows, bnd.size + 1)
        cols.append(W.Column(kind, pools[c % len(pools)], dtype, rows, int(rng.choice(dims)),
                             id_lo=-3, id_hi=50, boundaries=bnd if kind == W.BUCKET else None))
    lens = rng.integers(0, max_len + 1, size=C * B)
    offsets = np.zeros(C * B + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(lens)
    N = int(offsets[-1])
    ids = rng.integers(-5, 60, size=N).astype(np.int64)
    fv = rng.normal(size=N).astype(np.float32)
    fv[rng.random(N) < invalid] = np.nan
    fv[rng.random(N) < 0.1] = bnd[0]          # exact boundary hits
    weights = []
    for col in cols:
        w32 = rng.normal(0, 1, size=(col.rows, col.dim)).astype(np.float32)
        weights.append(w32 if dtype == W.F32 else
                       (torch.from_numpy(w32).to(torch.bfloat16).view(torch.int16).numpy()
                        .view(np.uint16)))
    return cols, B, offsets, ids, fv, weights


def _as_f64(col, w):
    if col.dtype == W.BF16:
        return (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return w.astype(np.float64)


def _torch_forward_and_grad(cols, weights, B, offsets, rows, G, pw=None):
    """embedding_bag per column on the oracle's row indices (a library routine),
    and autograd for the dense gradient of sum(Y * G).  With per-position
    weights pw, a sum bag is embedding_bag's per_sample_weights sum, and a mean
    bag the same sum divided by the bag's kept count."""
    Ys, grads = [], []
    off_c = 0
    for c, col in enumerate(cols):
        W64 = torch.tensor(np.vstack([_as_f64(col, weights[c]), np.zeros((1, col.dim))]),
                           dtype=torch.float64, requires_grad=True)
        a, e = offsets[c * B], offsets[(c + 1) * B]
        r = rows[a:e]
        keep = r != oracle.ROW_DROPPED
        idx = np.where(r == oracle.ROW_DEFAULT, col.rows, r)[keep]
        # offsets of the kept positions per bag
        starts = []
        kept_before = np.concatenate([[0], np.cumsum(keep)])
        for s in range(B):
            starts.append(kept_before[offsets[c * B + s] - a])
        mode = "mean" if col.pool == W.MEAN else "sum"
        if pw is None:
            y = torch.nn.functional.embedding_bag(torch.tensor(idx, dtype=torch.long), W64,
                                                  torch.tensor(starts, dtype=torch.long), mode=mode)
        else:
            psw = torch.tensor(pw[a:e][keep], dtype=torch.float64)
            y = torch.nn.functional.embedding_bag(torch.tensor(idx, dtype=torch.long), W64,
                                                  torch.tensor(starts, dtype=torch.long), mode="sum",
                                                  per_sample_weights=psw)
            if col.pool == W.MEAN:
                n = np.diff(np.concatenate([starts, [int(keep.sum())]]))
                y = y / torch.tensor(np.maximum(n, 1), dtype=torch.float64)[:, None]
        Gc = torch.tensor(G[:, off_c:off_c + col.dim], dtype=torch.float64)
        (y * Gc).sum().backward()
        Ys.append(y.detach().numpy())
        grads.append(W64.grad.numpy()[:col.rows])
        off_c += col.dim
    return np.hstack(Ys), grads


# ---------------------------------------------------------------- hashing

def test_splitmix64_published_vectors():
    with open(os.path.join(GOLDEN, "splitmix64_vectors.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) == 9
    for seed, i, out in rows:
        x = (int(seed) + int(i) * GAMMA) & M64
        assert int(oracle.splitmix64(np.array([x], dtype=np.uint64))[0]) == int(out)
        assert int(oracle.lib().oracle_splitmix64(x)) == int(out)


@pytest.mark.parametrize("rows", [1, 2, 3, 7, 1000, 1 << 20, (1 << 31) - 1, 10_000_000,
                                  (1 << 40) + 1, (1 << 62) + 12345])
def test_hash_mod_is_the_unsigned_remainder(rows):
    rng = np.random.default_rng(rows % 1000)
    ids = list(rng.integers(0, 1 << 62, size=200)) + [0, 1, (1 << 63) - 1, -1, -(1 << 63)]
    for i in ids:
        bits = int(i) & M64
        h = int(oracle.splitmix64(np.array([bits], dtype=np.uint64))[0])
        assert oracle.hash_mod(bits, rows) == h % rows


def test_hash_mod_large_hash_values():
    # IDs whose hash lies near 0 and near 2^64-1 would expose a signed or 32-bit remainder
    xs = np.arange(0, 200000, dtype=np.uint64)
    h = oracle.splitmix64(xs)
    for pick in (np.argmax(h), np.argmin(h)):
        for rows in (3, 1000, (1 << 31) - 1, (1 << 63) - 25):
            assert oracle.hash_mod(int(xs[pick]), rows) == int(h[pick]) % rows


# -------------------------------------------------------------- bucketize

def test_bucketize_matches_searchsorted_right():
    b = W.lognormal_boundaries(64)
    rng = np.random.default_rng(3)
    probes = np.concatenate([rng.lognormal(0, 1, 500).astype(np.float32), b,
                             np.nextafter(b, np.float32(-np.inf)), np.nextafter(b, np.float32(np.inf)),
                             np.array([0.0, -0.0, -1.0, np.inf, -np.inf, 1e-45, 3e38], np.float32)])
    for x in probes:
        k = oracle.bucketize(b, float(x))
        assert k == int(np.searchsorted(b, x, side="right"))
        assert k == int(torch.bucketize(torch.tensor([x]), torch.from_numpy(b), right=True)[0])
    assert oracle.bucketize(b, float("nan")) == oracle.ROW_DROPPED


def test_lognormal_boundaries_equal_mass():
    b = W.lognormal_boundaries(64)
    assert np.all(np.diff(b) > 0)
    x = np.random.default_rng(11).lognormal(0, 1, 650_000).astype(np.float32)
    k = np.searchsorted(b, x, side="right")
    frac = np.bincount(k, minlength=65) / x.size
    assert np.allclose(frac, 1 / 65, atol=0.0015)


# ------------------------------------------------------------- transforms

def test_transform_validity_brute_force():
    rng = np.random.default_rng(5)
    bnd = np.array([-1.0, 0.0, 0.0, 2.5], dtype=np.float32)
    cases = [
        (W.Column(W.HASH, 0, 0, 13, 4, id_lo=-4, id_hi=9), None),
        (W.Column(W.IDENTITY, 0, 0, 13, 4), None),
        (W.Column(W.BUCKET, 0, 0, 13, 4, boundaries=bnd), None),
        (W.Column(W.KEYED, 0, 0, 13, 4), None),
    ]
    for col, _ in cases:
        cs = oracle.Columns([col], [np.zeros((col.rows, col.dim), np.float32)])
        for _ in range(300):
            i = int(rng.integers(-20, 30))
            x = float(rng.choice([np.nan, -1.0, 0.0, -0.0, 1.0, 2.5, 3.0, -np.inf]))
            k = int(rng.integers(-3, 16))
            r = int(oracle.lib().oracle_row(cs.arr, i, x, k))
            if col.kind == W.HASH:
                exp = oracle.hash_mod(i & M64, col.rows) if -4 <= i < 9 else -1
            elif col.kind == W.IDENTITY:
                exp = i if 0 <= i < 13 else -1
            elif col.kind == W.BUCKET:
                exp = -1 if math.isnan(x) else sum(1 for v in bnd if v <= x)
            else:
                exp = -2 if k == -2 else (k if 0 <= k < 13 else -1)
            assert r == exp, (col.kind, i, x, k)


# ----------------------------------------------------------- forward pins

@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
def test_forward_matches_embedding_bag(seed, dtype):
    rng = np.random.default_rng(100 + seed)
    cols, B, off, ids, fv, weights = _tiny_case(rng, dtype=dtype)
    cs = oracle.Columns(cols, weights)
    Y, Yb, bag_n, rows = oracle.forward(cs, B, off, ids, fv)
    G = rng.normal(size=Y.shape).astype(np.float32)
    Yt, _ = _torch_forward_and_grad(cols, weights, B, off, rows, G)
    assert np.allclose(Y, Yt, rtol=0, atol=1e-6 * (1 + np.abs(Yt).max()))
    assert np.all(Y.astype(np.float64) - Yt <= 2 * np.spacing(np.abs(Yt).astype(np.float32)) + 1e-30)
    # bag counts: valid positions per bag, a brute-force recount
    for b in range(len(cols) * B):
        assert bag_n[b] == int(np.sum(rows[off[b]:off[b + 1]] != oracle.ROW_DROPPED))
    # the error scale is at least |Y|
    assert np.all(Yb + 1e-12 >= np.abs(Y) * (1 - 1e-6))


def test_forward_one_hot_and_empty_closed_forms():
    rng = np.random.default_rng(9)
    col = W.Column(W.IDENTITY, W.MEAN, W.F32, 10, 8)
    Wt = rng.normal(size=(10, 8)).astype(np.float32)
    cs = oracle.Columns([col], [Wt])
    off = np.array([0, 1, 1, 2, 3], dtype=np.int32)     # bags: {3}, {}, {7}, {42 (dropped)}
    ids = np.array([3, 7, 42], dtype=np.int64)
    Y, _, bag_n, rows = oracle.forward(cs, 4, off, ids)
    assert np.array_equal(Y[0], Wt[3]) and np.array_equal(Y[2], Wt[7])
    assert np.all(Y[1] == 0) and np.all(Y[3] == 0)
    assert list(bag_n) == [1, 0, 1, 0] and list(rows) == [3, 7, -1]


def test_forward_keyed_default_counts_in_mean():
    col = W.Column(W.KEYED, W.MEAN, W.F32, 4, 4)
    Wt = np.arange(16, dtype=np.float32).reshape(4, 4)
    cs = oracle.Columns([col], [Wt])
    off = np.array([0, 3], dtype=np.int32)
    Y, _, bag_n, _ = oracle.forward(cs, 1, off, keyed_rows=np.array([2, -2, -1], np.int32))
    assert bag_n[0] == 2
    assert np.array_equal(Y[0], Wt[2] / 2)


# ---------------------------------------------------------- backward pins

@pytest.mark.parametrize("seed", range(6))
def test_backward_matches_autograd_and_unique_set(seed):
    rng = np.random.default_rng(200 + seed)
    cols, B, off, ids, fv, weights = _tiny_case(rng)
    cs = oracle.Columns(cols, [w.copy() for w in weights])
    Y, _, bag_n, rows = oracle.forward(cs, B, off, ids, fv)
    G = rng.normal(size=Y.shape).astype(np.float32)
    ucol, urow, ug, ub = oracle.backward(cs, B, off, G, ids, fv, opt=W.OPT_EMIT)
    _, grads = _torch_forward_and_grad(cols, weights, B, off, rows, G)
    for c, col in enumerate(cols):
        a, e = off[c * B], off[(c + 1) * B]
        r = rows[a:e]
        touched = np.unique(r[r >= 0])
        sel = ucol == c
        assert np.array_equal(urow[sel], touched)            # distinct rows, ascending
        got = ug[sel][:, :col.dim]
        assert np.allclose(got, grads[c][touched], rtol=1e-12, atol=1e-12)
        # untouched rows have zero dense gradient
        mask = np.ones(col.rows, bool)
        mask[touched] = False
        assert np.all(grads[c][mask] == 0)
    # (column, row) ascending overall
    key = ucol.astype(np.int64) * (1 << 40) + urow
    assert np.all(np.diff(key) > 0)


@pytest.mark.parametrize("seed", range(4))
def test_backward_gradient_mass_invariant(seed):
    """sum over touched rows of dE = sum over bags of kappa_s * G[s], kappa_s = number of
    non-default contributors (sum), their share of the mean (mean), 0 if empty."""
    rng = np.random.default_rng(300 + seed)
    cols, B, off, ids, fv, weights = _tiny_case(rng, kinds=(W.HASH, W.KEYED, W.IDENTITY))
    keyed = rng.choice([-2, -1, 0, 1, 2, 3], size=int(off[-1])).astype(np.int32)
    cs = oracle.Columns(cols, weights)
    Y, _, bag_n, rows = oracle.forward(cs, B, off, ids, fv, keyed)
    G = rng.normal(size=Y.shape).astype(np.float32)
    ucol, urow, ug, _ = oracle.backward(cs, B, off, G, ids, fv, keyed)
    off_c = 0
    for c, col in enumerate(cols):
        lhs = ug[ucol == c][:, :col.dim].sum(axis=0)
        rhs = np.zeros(col.dim)
        for s in range(B):
            b = c * B + s
            r = rows[off[b]:off[b + 1]]
            k = np.sum(r >= 0)
            if bag_n[b] == 0:
                continue
            kappa = k / bag_n[b] if col.pool == W.MEAN else k
            rhs += kappa * G[s, off_c:off_c + col.dim].astype(np.float64)
        assert np.allclose(lhs, rhs, rtol=1e-10, atol=1e-10)
        off_c += col.dim


def test_reduce_id_worked_example():
    """RecIS Fig. 3: local Reduce-ID keeps each distinct ID once; the inverse map
    (here the per-row multiplicity carried by the gradient) restores the list."""
    lines = dict(l.split(":", 1) for l in open(os.path.join(GOLDEN, "recis_fig3_reduce_id.txt"))
                 if l.strip() and not l.startswith("#"))
    for g in ("gpu0", "gpu1"):
        ids = np.array(lines[f"{g}_ids"].split(), dtype=np.int64)
        reduced = np.array(lines[f"{g}_reduced"].split(), dtype=np.int64)
        col = W.Column(W.IDENTITY, W.SUM, W.F32, 10000, 4)
        cs = oracle.Columns([col], [np.zeros((10000, 4), np.float32)])
        off = np.array([0, ids.size], np.int32)
        G = np.ones((1, 4), np.float32)
        _, urow, ug, _ = oracle.backward(cs, 1, off, G, ids)
        assert set(urow.tolist()) == set(reduced.tolist()) and urow.size == reduced.size
        mult = dict(zip(urow.tolist(), ug[:, 0].tolist()))
        rebuilt = sorted(sum(([u] * int(m) for u, m in mult.items()), []))
        assert rebuilt == sorted(ids.tolist())


# ------------------------------------------------- truncation and masking

def _kept_positions(B, offsets, seq, mask):
    """Brute force: the raw positions that survive a per-column (seq_max, keep_last)
    truncation and a per-position mask, listed bag by bag."""
    keep = np.zeros(int(offsets[-1]), bool)
    for b in range(len(offsets) - 1):
        seq_max, last = seq[b // B]
        a, e = int(offsets[b]), int(offsets[b + 1])
        idx = list(range(a, e))
        if seq_max > 0:
            idx = idx[-seq_max:] if last else idx[:seq_max]
        for p in idx:
            keep[p] = mask is None or mask[p] != 0
    return keep


def _sliced(B, offsets, keep, *arrays):
    """The same batch with the non-surviving positions removed (new offsets)."""
    kept_before = np.concatenate([[0], np.cumsum(keep)]).astype(np.int32)
    return (kept_before[offsets],) + tuple(None if x is None else x[keep] for x in arrays)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("use_mask", [False, True])
def test_truncation_and_mask_equal_the_sliced_batch(seed, use_mask):
    """A truncated / masked batch pools and trains exactly like the batch with the
    dropped positions cut out; the kept set is listed by brute force."""
    rng = np.random.default_rng(700 + seed)
    cols, B, off, ids, fv, weights = _tiny_case(rng, kinds=(W.HASH, W.IDENTITY, W.BUCKET, W.KEYED),
                                                C=5, max_len=9)
    seq = [(0, 0), (3, 0), (3, 1), (1, 1), (2, 0)]
    for col, (m, last) in zip(cols, seq):
        col.seq_max, col.seq_keep_last = m, last
    N = int(off[-1])
    keyed = rng.choice([-2, -1, 0, 1, 2], size=N).astype(np.int32)
    mask = (rng.random(N) < 0.7).astype(np.uint8) if use_mask else None
    keep = _kept_positions(B, off, seq, mask)
    off2, ids2, fv2, keyed2 = _sliced(B, off, keep, ids, fv, keyed)
    plain = [W.Column(c.kind, c.pool, c.dtype, c.rows, c.dim, c.id_lo, c.id_hi, c.boundaries)
             for c in cols]

    Y, Yb, n, rows = oracle.forward(oracle.Columns(cols, weights), B, off, ids, fv, keyed, mask)
    Y2, Yb2, n2, rows2 = oracle.forward(oracle.Columns(plain, weights), B, off2, ids2, fv2, keyed2)
    assert np.array_equal(Y, Y2) and np.array_equal(Yb, Yb2) and np.array_equal(n, n2)
    assert np.all(rows[~keep] == oracle.ROW_DROPPED) and np.array_equal(rows[keep], rows2)

    G = rng.normal(size=Y.shape).astype(np.float32)
    wa, wb = [w.copy() for w in weights], [w.copy() for w in weights]
    ca, cb = oracle.Columns(cols, wa), oracle.Columns(plain, wb)
    ra = oracle.backward(ca, B, off, G, ids, fv, keyed, opt=W.OPT_SGD, lr=0.1, mask=mask)
    rb = oracle.backward(cb, B, off2, G, ids2, fv2, keyed2, opt=W.OPT_SGD, lr=0.1)
    for x, y in zip(ra, rb):
        assert np.array_equal(x, y)
    for x, y in zip(wa, wb):
        assert np.array_equal(x, y)


def test_truncation_keeps_first_or_last_closed_form():
    """Bag [0..9] of an IDENTITY sum column: keeping the first 3 sums rows 0..2, the
    last 3 sums rows 7..9, a limit above the length keeps all 10; a mask that zeroes
    the even positions halves what is left."""
    Wt = np.eye(10, 4, dtype=np.float32) + np.arange(10, dtype=np.float32)[:, None]
    off = np.array([0, 10], dtype=np.int32)
    ids = np.arange(10, dtype=np.int64)
    for m, last, want in [(3, 0, [0, 1, 2]), (3, 1, [7, 8, 9]), (12, 1, list(range(10))),
                          (0, 0, list(range(10)))]:
        col = W.Column(W.IDENTITY, W.SUM, W.F32, 10, 4, seq_max=m, seq_keep_last=last)
        Y, _, n, _ = oracle.forward(oracle.Columns([col], [Wt]), 1, off, ids)
        assert n[0] == len(want) and np.array_equal(Y[0], Wt[want].sum(axis=0))
        odd = (np.arange(10) % 2).astype(np.uint8)
        Y, _, n, _ = oracle.forward(oracle.Columns([col], [Wt]), 1, off, ids, mask=odd)
        got = [i for i in want if i % 2]
        assert n[0] == len(got) and np.array_equal(Y[0], Wt[got].sum(axis=0))


# ----------------------------------------------------- per-position weights

@pytest.mark.parametrize("seed", range(6))
def test_weighted_forward_and_backward_match_autograd(seed):
    """Per-position weights v (RecIS Sec. 3.2: Y_s = sum_r w_r E[i_r]; each
    contributor sends w_r G[s(r)] back): embedding_bag's per_sample_weights for
    sum bags, that sum over the kept count for mean bags, autograd for dE."""
    rng = np.random.default_rng(800 + seed)
    cols, B, off, ids, fv, weights = _tiny_case(rng, kinds=(W.HASH, W.IDENTITY, W.BUCKET))
    N = int(off[-1])
    pw = rng.normal(size=N).astype(np.float32)
    cs = oracle.Columns(cols, [w.copy() for w in weights])
    Y, Yb, bag_n, rows = oracle.forward(cs, B, off, ids, fv, pweights=pw)
    G = rng.normal(size=Y.shape).astype(np.float32)
    Yt, grads = _torch_forward_and_grad(cols, weights, B, off, rows, G, pw=pw)
    assert np.allclose(Y, Yt, rtol=0, atol=1e-6 * (1 + np.abs(Yt).max()))
    assert np.all(Yb + 1e-12 >= np.abs(Y) * (1 - 1e-6))
    ucol, urow, ug, ub = oracle.backward(cs, B, off, G, ids, fv, opt=W.OPT_EMIT, pweights=pw)
    for c, col in enumerate(cols):
        sel = ucol == c
        assert np.allclose(ug[sel][:, :col.dim], grads[c][urow[sel]], rtol=1e-12, atol=1e-12)
        assert np.all(ub[sel][:, :col.dim] + 1e-12 >= np.abs(ug[sel][:, :col.dim]))


def test_unit_and_power_of_two_weights():
    """All-one weights give the unweighted results bit for bit; weights of 2 give
    exactly twice the outputs and gradients."""
    rng = np.random.default_rng(850)
    cols, B, off, ids, fv, weights = _tiny_case(rng)
    N = int(off[-1])
    cs = oracle.Columns(cols, weights)
    G = rng.normal(size=(B, cs.sum_dim)).astype(np.float32)
    base = oracle.forward(cs, B, off, ids, fv)
    one = oracle.forward(cs, B, off, ids, fv, pweights=np.ones(N, np.float32))
    two = oracle.forward(cs, B, off, ids, fv, pweights=np.full(N, 2, np.float32))
    for x, y in zip(base, one):
        assert np.array_equal(x, y)
    assert np.array_equal(two[0], 2 * base[0])
    gb = oracle.backward(cs, B, off, G, ids, fv)
    g2 = oracle.backward(cs, B, off, G, ids, fv, pweights=np.full(N, 2, np.float32))
    assert np.array_equal(gb[1], g2[1]) and np.array_equal(2 * gb[2], g2[2])


# ------------------------------------------------------------- default row

@pytest.mark.parametrize("seed", range(4))
def test_default_row_equals_filling_empty_bags(seed):
    """A column with a default row d behaves like the same batch with the ID d
    inserted into every bag that has no valid ID (TF-style empty-row filling,
    which RECom merges into the lookup), forward and backward."""
    rng = np.random.default_rng(900 + seed)
    C, B = 3, 8
    cols, weights = [], []
    for c in range(C):
        rows, dim = int(rng.integers(5, 12)), int(rng.choice([4, 8]))
        cols.append(W.Column(W.IDENTITY, (W.SUM, W.MEAN)[c % 2], W.F32, rows, dim,
                             default_row=int(rng.integers(0, rows))))
        weights.append(rng.normal(size=(rows, dim)).astype(np.float32))
    lens = rng.integers(0, 4, size=C * B)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ids = rng.integers(-3, 14, size=int(off[-1])).astype(np.int64)
    # the filled batch, built by hand: bag b of column c gets d_c appended when none
    # of its IDs is in [0, rows_c)
    f_ids, f_lens = [], []
    for b in range(C * B):
        col = cols[b // B]
        seg = list(ids[off[b]:off[b + 1]])
        if not any(0 <= x < col.rows for x in seg):
            seg.append(col.default_row)
        f_ids += seg
        f_lens.append(len(seg))
    f_off = np.concatenate([[0], np.cumsum(f_lens)]).astype(np.int32)
    f_ids = np.array(f_ids, dtype=np.int64)
    plain = [W.Column(c.kind, c.pool, c.dtype, c.rows, c.dim) for c in cols]

    Y, Yb, _, _ = oracle.forward(oracle.Columns(cols, weights), B, off, ids)
    Y2, Yb2, _, _ = oracle.forward(oracle.Columns(plain, weights), B, f_off, f_ids)
    assert np.array_equal(Y, Y2) and np.array_equal(Yb, Yb2)
    G = rng.normal(size=Y.shape).astype(np.float32)
    wa, wb = [w.copy() for w in weights], [w.copy() for w in weights]
    ra = oracle.backward(oracle.Columns(cols, wa), B, off, G, ids, opt=W.OPT_SGD, lr=0.1)
    rb = oracle.backward(oracle.Columns(plain, wb), B, f_off, G, f_ids, opt=W.OPT_SGD, lr=0.1)
    assert np.array_equal(ra[0], rb[0]) and np.array_equal(ra[1], rb[1])
    assert np.allclose(ra[2], rb[2], rtol=1e-12, atol=1e-15)
    for x, y in zip(wa, wb):
        assert np.allclose(x, y, rtol=1e-6, atol=1e-7)


def test_default_row_closed_form():
    """Every bag empty: each output is row d, and d's gradient is the sum of all G rows."""
    rng = np.random.default_rng(950)
    Wt = rng.normal(size=(6, 4)).astype(np.float32)
    col = W.Column(W.HASH, W.MEAN, W.F32, 6, 4, id_lo=0, id_hi=10, default_row=4)
    off = np.array([0, 0, 2, 2, 3], dtype=np.int32)          # two empty, two all-invalid
    ids = np.array([-1, 10, 99], dtype=np.int64)
    Y, _, n, _ = oracle.forward(oracle.Columns([col], [Wt]), 4, off, ids)
    assert list(n) == [0, 0, 0, 0] and np.array_equal(Y, np.tile(Wt[4], (4, 1)))
    G = rng.normal(size=(4, 4)).astype(np.float32)
    ucol, urow, ug, _ = oracle.backward(oracle.Columns([col], [Wt]), 4, off, G, ids)
    assert list(urow) == [4] and np.allclose(ug[0], G.astype(np.float64).sum(axis=0), rtol=1e-15)


# ------------------------------------------------------------ optimizers

@pytest.mark.parametrize("opt,big_eps", [(W.OPT_SGD, False), (W.OPT_ADAGRAD, False),
                                         (W.OPT_ADAGRAD, True)])
@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
def test_row_update_matches_torch_optim(opt, big_eps, dtype):
    rng = np.random.default_rng(400 + opt + 10 * dtype)
    cols, B, off, ids, fv, weights = _tiny_case(rng, kinds=(W.HASH, W.IDENTITY), dtype=dtype,
                                                rows_hi=40, max_len=6)
    states = [rng.random(size=(c.rows, c.dim)).astype(np.float32) if opt == W.OPT_ADAGRAD
              else None for c in cols]
    before_w = [w.copy() for w in weights]
    before_s = [None if s is None else s.copy() for s in states]
    cs = oracle.Columns(cols, [w.copy() for w in weights], [None if s is None else s.copy()
                                                           for s in states])
    lr, eps = (0.05, 1e-8) if opt == W.OPT_ADAGRAD else (0.01, 0.0)
    if big_eps:        # a large eps separates eps outside the root from eps inside it
        eps = 0.3
        states = [np.where(rng.random(s.shape) < 0.5, 0, s).astype(np.float32) for s in states]
        before_s = [s.copy() for s in states]
        cs = oracle.Columns(cols, [w.copy() for w in weights], [s.copy() for s in states])
    Y, _, _, rows = oracle.forward(cs, B, off, ids, fv)
    G = rng.normal(size=Y.shape).astype(np.float32)
    ucol, urow, _, _ = oracle.backward(cs, B, off, G, ids, fv, opt=opt, lr=lr, eps=eps)
    _, grads = _torch_forward_and_grad(cols, before_w, B, off, rows, G)
    for c, col in enumerate(cols):
        p = torch.tensor(_as_f64(col, before_w[c]), requires_grad=True)
        p.grad = torch.tensor(grads[c])
        if opt == W.OPT_SGD:
            o = torch.optim.SGD([p], lr=lr)
        else:
            o = torch.optim.Adagrad([p], lr=lr, eps=eps, initial_accumulator_value=0.0)
            o.state[p]["sum"] = torch.tensor(before_s[c].astype(np.float64))
            o.state[p]["step"] = torch.tensor(0.0)
        # only rows with a gradient entry move: a dense step with g = 0 leaves
        # a row (and its accumulator) unchanged, which is the sparse update
        o.step()
        exp = p.detach()
        got = _as_f64(col, cs.weights[c])
        tol = (2.0 ** -7 if dtype == W.BF16 else 2.0 ** -23) * np.abs(exp.numpy()) + 1e-30
        assert np.all(np.abs(got - exp.numpy()) <= tol)
        touched = np.unique(urow[ucol == c])
        untouched = np.setdiff1d(np.arange(col.rows), touched)
        assert np.array_equal(cs.weights[c][untouched], before_w[c][untouched])
        if opt == W.OPT_ADAGRAD:
            s_exp = o.state[p]["sum"].numpy()
            assert np.allclose(cs.states[c], s_exp, rtol=2 ** -23, atol=0)
            assert np.array_equal(cs.states[c][untouched], before_s[c][untouched])


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(12)
    bits = rng.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    # add exact ties: bf16 value + half an ulp
    ties = ((bits[:2000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    f = np.concatenate([f, ties[np.isfinite(ties)], np.array([0.0, -0.0, 1e-40, -3e-39], np.float32)])
    exp = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.double_to_bf16(float(x)) for x in f], dtype=np.uint16)
    assert np.array_equal(got, exp)


# -------------------------------------------------------------- keyed rows

def test_init_row_is_uniform_with_requested_std():
    vals = np.concatenate([oracle.init_row(k, 32, 0.01) for k in range(1, 3001)])
    a = np.float32(0.01 * math.sqrt(3))
    assert np.all(np.abs(vals) <= a) and abs(vals.mean()) < 2e-4
    assert abs(vals.std() - 0.01) < 2e-4
    assert not np.array_equal(oracle.init_row(5, 32, 0.01), oracle.init_row(6, 32, 0.01))
    assert np.array_equal(oracle.init_row(5, 32, 0.01), oracle.init_row(5, 32, 0.01))


def test_table_model_vs_dict():
    """The numpy table model against a plain per-occurrence dict model."""
    rng = np.random.default_rng(21)
    pre = np.array([11, 12, 13], dtype=np.int64)
    pre_rows = rng.normal(size=(3, 4)).astype(np.float32)
    T = OracleTable(64, 4, 2, 0.01, pre, pre_rows)
    cnt = {11: 0, 12: 0, 13: 0}
    admitted = {11, 12, 13}
    for step in range(5):
        keys = rng.integers(-2, 25, size=30).astype(np.int64)
        uk, adm = T.step(keys)
        m = {}
        for k in keys.tolist():
            if k >= 1:
                m[k] = m.get(k, 0) + 1
        for k, v in m.items():
            cnt[k] = cnt.get(k, 0) + v
            if cnt[k] >= 2:
                admitted.add(k)
        assert sorted(uk.tolist()) == sorted(m)
        assert {int(k) for k, a in zip(uk, adm) if a} == {k for k in m if k in admitted}
        rows, pk, pool = T.resolve(keys)
        for k, r in zip(keys.tolist(), rows.tolist()):
            if k < 1:
                assert r == oracle.ROW_DROPPED
            elif k in admitted:
                assert pk[r] == k
                want = pre_rows[k - 11] if k in (11, 12, 13) else oracle.init_row(k, 4, 0.01)
                assert np.array_equal(pool[r], want)
            else:
                assert r == oracle.ROW_DEFAULT
        present, c2, _ = T.state(np.array(sorted(cnt), dtype=np.int64))
        assert present.all() and c2.tolist() == [cnt[k] for k in sorted(cnt)]
    with pytest.raises(Exception):
        OracleTable(2, 4, 2, 0.01).step(np.array([1, 2, 3], np.int64))


def test_table_lifecycle_vs_dict():
    """Last-seen steps, eviction and checkpoint/restore of the table model against a
    plain dict model: an evicted key loses count, admission and row, and starts
    anew; a restored model continues exactly like the original."""
    rng = np.random.default_rng(22)
    pre = np.array([5, 6], dtype=np.int64)
    pre_rows = rng.normal(size=(2, 4)).astype(np.float32)
    T = OracleTable(256, 4, 2, 0.01, pre, pre_rows)
    d = {5: dict(c=0, seen=0, row=pre_rows[0]), 6: dict(c=0, seen=0, row=pre_rows[1])}
    for step in range(12):
        keys = rng.integers(-1, 30, size=25).astype(np.int64)
        T.step(keys)
        for k in set(keys.tolist()):
            if k < 1:
                continue
            e = d.setdefault(k, dict(c=0, seen=0, row=None))
            e["c"] += int((keys == k).sum())
            e["seen"] = step
            if e["row"] is None and e["c"] >= 2:
                e["row"] = oracle.init_row(k, 4, 0.01)
        if step % 4 == 3:
            gone = [k for k, e in d.items() if e["seen"] < step - 2]
            for k in gone:
                del d[k]
            assert T.evict(step - 2) == len(gone)
        ks = np.array(sorted(d), dtype=np.int64)
        present, cnt, adm = T.state(ks)
        assert present.all() and cnt.tolist() == [d[k]["c"] for k in ks.tolist()]
        assert adm.tolist() == [d[k]["row"] is not None for k in ks.tolist()]
        assert T.keys.size == len(d)
        assert T.seen.tolist() == [d[k]["seen"] for k in ks.tolist()]
        for k, a in zip(ks.tolist(), adm.tolist()):
            if a:
                assert np.array_equal(T.row_values([k])[0], d[k]["row"])
    # restore from a checkpoint, then run both on the same steps
    R = OracleTable.restore(256, 4, 2, 0.01, T.checkpoint())
    for step in range(3):
        keys = rng.integers(-1, 40, size=25).astype(np.int64)
        a, b = T.step(keys), R.step(keys)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        assert T.evict(T.step_no - 2) == R.evict(R.step_no - 2)
        ca, cb = T.checkpoint(), R.checkpoint()
        for x, y in zip(ca[:5], cb[:5]):
            assert np.array_equal(x, y)
        assert ca[5] == cb[5]


def test_count_min_cells_are_splitmix64_outputs():
    """Cell j of key k is output j of a SplitMix64 generator seeded with k (the
    published vectors), reduced mod the width."""
    from oracle.table import count_min_cells
    with open(os.path.join(GOLDEN, "splitmix64_vectors.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    by_seed = {}
    for seed, i, out in rows:
        by_seed.setdefault(int(seed), {})[int(i)] = int(out)
    for seed, outs in by_seed.items():
        if seed >= 1 << 63:
            continue
        depth = max(outs) + 1
        for width in (1 << 62, 1000):
            cells = count_min_cells(np.array([seed], np.int64), depth, width)[:, 0]
            for j, out in outs.items():
                assert int(cells[j]) == out % width


def test_count_min_admission_vs_brute_force_and_exact():
    """The count-min model against a per-occurrence brute force with a narrow
    sketch (many collisions), and against exact counting with a wide one."""
    from oracle.table import count_min_cells
    rng = np.random.default_rng(23)
    steps = [rng.integers(-1, 400, size=120).astype(np.int64) for _ in range(8)]
    for width, depth in ((16, 3), (1 << 24, 3)):
        T = OracleTable(1024, 4, 3, 0.01)
        T.use_count_min(depth, width)
        E = OracleTable(1024, 4, 3, 0.01)                # exact counting in slots
        C = np.zeros((depth, width), dtype=np.int64)
        table = {}                                       # key -> count (keys in the table)
        for keys in steps:
            m = {}
            for k in keys.tolist():
                if k >= 1:
                    m[k] = m.get(k, 0) + 1
            absent = [k for k in m if k not in table]
            for k in absent:
                cells = count_min_cells(np.array([k], np.int64), depth, width)[:, 0]
                for j in range(depth):
                    C[j, cells[j]] += m[k]
            for k in m:
                if k in table:
                    table[k] += m[k]
            for k in absent:
                cells = count_min_cells(np.array([k], np.int64), depth, width)[:, 0]
                est = min(C[j, cells[j]] for j in range(depth))
                if est >= 3:
                    table[k] = int(est)
            T.step(keys)
            E.step(keys)
            assert T.keys.tolist() == sorted(table)
            assert T.count.tolist() == [table[k] for k in sorted(table)]
            assert T.admitted.all()                      # enter with count >= threshold
            rows, _, _ = T.resolve(keys)
            for k, r in zip(keys.tolist(), rows.tolist()):
                assert (r >= 0) == (k in table) and (r == oracle.ROW_DROPPED) == (k < 1)
            if width > 1 << 20:                          # no collisions: the exact outcome
                assert np.array_equal(rows, E.resolve(keys)[0])
                _, ec, ea = E.state(T.keys)
                assert np.array_equal(ec, T.count) and ea.all()


# --------------------------------------------------------------- generators

def test_generator_statistics_training_front_end():
    w = W.config(2, n_cols=40, batch=4096)
    b = W.make_batch(w, seed=2001)
    lens = np.diff(b.offsets)
    # Poisson(3) with 5% forced empty bags
    assert abs(lens.mean() - 0.95 * 3) < 0.05
    assert abs(np.mean(lens == 0) - (0.05 + 0.95 * math.exp(-3))) < 0.01
    assert abs(b.invalid_mask.mean() - 0.02) < 0.003
    bad = b.ids[b.invalid_mask]
    assert np.all((bad < 0) | (bad >= 1 << 40))
    good = b.ids[~b.invalid_mask]
    assert np.all((good >= 0) & (good < 1 << 40))


def _harmonic(n, s):
    if n <= 10**8:
        k = np.arange(1, n + 1, dtype=np.float64)
        return float(np.sum(k ** -s))
    from scipy.special import zeta
    # Euler-Maclaurin tail of zeta(s) beyond n
    return float(zeta(s) - n ** (1 - s) / (s - 1) + 0.5 * n ** -s - s * n ** (-s - 1) / 12)


def test_zipf_sampler_head_frequencies():
    rng = np.random.default_rng(7)
    for n, s in ((10_000_000, 1.05), (1 << 40, 1.1), (1000, 1.2)):
        z = W.ZipfSampler(n, s).sample(rng, 400_000)
        assert z.min() >= 1 and z.max() <= n
        H = _harmonic(n, s)
        for k in (1, 2, 5):
            p = k ** -s / H
            f = np.mean(z == k)
            assert abs(f - p) < 5 * math.sqrt(p / 400_000) + 1e-4, (n, s, k, f, p)


def test_keyed_workload_unseen_fraction():
    """Keys are pi(rank) with ranks Zipf(1.05) over 2^63-1 and the first 5e7 ranks
    prepopulated: P(unseen) = 1 - H(5e7, 1.05) / H(2^63-1, 1.05)."""
    z = W.ZipfSampler(W.KEY_SPACE_63, 1.05).sample(np.random.default_rng(8), 300_000)
    p_unseen = 1 - _harmonic(50_000_000, 1.05) / _harmonic(W.KEY_SPACE_63, 1.05)
    assert abs(p_unseen - 0.327) < 0.005
    assert abs(np.mean(z > 50_000_000) - p_unseen) < 0.005


def test_key_bijection():
    r = np.arange(0, 200_000, dtype=np.uint64)
    k = W.key_of_rank(r)
    assert k[0] == 0 and np.all(k[1:] >= 1)
    assert np.unique(k).size == r.size
    big = W.key_of_rank(np.array([W.KEY_SPACE_63, W.KEY_SPACE_63 - 1], dtype=np.uint64))
    assert np.all(big > 0) and big[0] != big[1]
