"""Seeded synthetic inputs for the fused multi-column embedding stage.

This module only draws inputs: column descriptions, jagged batches (CSR offsets,
raw int64 IDs, float feature values), embedding tables, upstream gradients and
the keys of a keyed table.  It holds none of the method's arithmetic (no ID hash,
no modulo, no bucketize, no pooling, no optimizer), so the CPU oracle and the HIP
path can both consume its output without sharing any computation.

The five workload shapes follow the workloads the pages describe:
  * tiny fused bag (8 hashed columns, B=256, D=16) -- a correctness case;
  * a training sparse front end (200 columns, Poisson bags, empty bags, invalid
    IDs, alternating sum/mean pooling, SGD) -- RecIS Table 1 sized feature sets;
  * many tiny inference columns (1000 columns, 30 % bucketized float columns)
    -- RECom's "thousands of embedding columns";
  * long behaviour sequences (bags of 200..2000 IDs, bf16 table, Adagrad)
    -- RecIS Sec. 3.1 "long behavior sequences";
  * a collisionless keyed table with a frequency filter (Monolith Sec. 2.1).
No public dataset is used; these draws stand in for the pages' workloads.
"""
from __future__ import annotations

import math
import statistics
from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np

# column kinds / pooling / dtypes / optimizers (plain integers, same values as include/emb.h)
HASH, IDENTITY, BUCKET, KEYED = 0, 1, 2, 3
SUM, MEAN = 0, 1
F32, BF16 = 0, 1
OPT_EMIT, OPT_SGD, OPT_ADAGRAD = 0, 1, 2

ID_SPACE_40 = 1 << 40
KEY_SPACE_63 = (1 << 63) - 1


@dataclass
class Column:
    kind: int
    pool: int
    dtype: int
    rows: int
    dim: int
    id_lo: int = 0
    id_hi: int = 0
    boundaries: Optional[np.ndarray] = None  # fp32, sorted, BUCKET only
    seq_max: int = 0                         # SeqTrunc: keep at most this many positions per bag
    seq_keep_last: int = 0                   # keep the last seq_max (1) or the first (0)
    default_row: int = -1                    # row filling an empty bag (-1: zero vector)


@dataclass
class Workload:
    name: str
    cols: List[Column]
    batch: int
    bag: str                      # "uniform" | "poisson" | "fixed" (per column overrides below)
    bag_lo: int = 1
    bag_hi: int = 1
    bag_mean: float = 3.0
    empty_frac: float = 0.0       # forced-empty bags
    invalid_frac: float = 0.0     # IDs replaced by out-of-range values
    id_dist: str = "uniform"      # "uniform" | "zipf"
    zipf_s: float = 1.0
    id_space: int = ID_SPACE_40   # ranks 1..id_space, raw id = rank - 1
    float_bag: int = 1            # bag length of BUCKET columns
    opt: int = OPT_EMIT
    lr: float = 0.0
    eps: float = 0.0
    init_std: float = 0.01
    training: bool = True
    # keyed table (KEYED columns)
    capacity: int = 0
    row_capacity: int = 0
    prepop: int = 0
    threshold: int = 2
    key_space: int = KEY_SPACE_63
    extra: dict = field(default_factory=dict)

    @property
    def sum_dim(self) -> int:
        return int(sum(c.dim for c in self.cols))


# ----------------------------------------------------------------------------
# bounded Zipf sampler: rejection-inversion (Hoermann & Derflinger, 1996)
# ----------------------------------------------------------------------------
def _helper1(y):
    # log1p(y)/y, -> 1 as y -> 0
    y = np.asarray(y, dtype=np.float64)
    out = np.ones_like(y)
    nz = np.abs(y) > 1e-8
    out[nz] = np.log1p(y[nz]) / y[nz]
    out[~nz] = 1.0 - y[~nz] * (0.5 - y[~nz] * (1.0 / 3.0))
    return out


def _helper2(y):
    # expm1(y)/y, -> 1 as y -> 0
    y = np.asarray(y, dtype=np.float64)
    out = np.ones_like(y)
    nz = np.abs(y) > 1e-8
    out[nz] = np.expm1(y[nz]) / y[nz]
    out[~nz] = 1.0 + y[~nz] * 0.5 * (1.0 + y[~nz] * (1.0 / 3.0))
    return out


class ZipfSampler:
    """P(k) proportional to k^-s on k = 1..n (n may be as large as 2^63-1)."""

    def __init__(self, n: int, s: float):
        assert n >= 1 and s > 0
        self.n, self.s = int(n), float(s)
        self.hx1 = float(self._H(np.array([1.5]))[0] - 1.0)
        self.hn = float(self._H(np.array([float(self.n) + 0.5]))[0])
        self.sc = 2.0 - float(self._Hinv(self._H(np.array([2.5])) - 2.0 ** (-self.s))[0])

    def _H(self, x):
        lx = np.log(x)
        return _helper2((1.0 - self.s) * lx) * lx

    def _Hinv(self, y):
        t = np.maximum(y * (1.0 - self.s), -1.0)
        return np.exp(_helper1(t) * y)

    def sample(self, rng: np.random.Generator, size: int) -> np.ndarray:
        """Ranks in [1, n] as uint64.  Ranks above 2^53 carry float64 spacing."""
        out = np.empty(size, dtype=np.uint64)
        todo = np.arange(size)
        while todo.size:
            u = self.hn + rng.random(todo.size) * (self.hx1 - self.hn)
            x = self._Hinv(u)
            kf = np.floor(x + 0.5)
            kf = np.clip(kf, 1.0, float(self.n))
            acc = (kf - x <= self.sc) | (u >= self._H(kf + 0.5) - kf ** (-self.s))
            k = kf[acc].astype(np.uint64)
            k = np.minimum(k, np.uint64(self.n))
            out[todo[acc]] = k
            todo = todo[~acc]
        return out


# ----------------------------------------------------------------------------
# keyed-table keys: a fixed bijection on [0, 2^63) with pi(0) = 0, so that
# ranks 1..2^63-1 map to distinct keys that look uniform on [1, 2^63).
# (xorshift / odd-multiply rounds; an input scrambler, unrelated to any hash the
# method uses.)
# ----------------------------------------------------------------------------
_M63 = np.uint64((1 << 63) - 1)
_K1 = np.uint64(0x2545F4914F6CDD1D)
_K2 = np.uint64(0x5851F42D4C957F2D)


def key_of_rank(ranks: np.ndarray) -> np.ndarray:
    x = np.asarray(ranks, dtype=np.uint64) & _M63
    with np.errstate(over="ignore"):
        x = x ^ (x >> np.uint64(31))
        x = (x * _K1) & _M63
        x = x ^ (x >> np.uint64(29))
        x = (x * _K2) & _M63
        x = x ^ (x >> np.uint64(32))
    return x.astype(np.int64)


def prepop_keys(n: int) -> np.ndarray:
    return key_of_rank(np.arange(1, n + 1, dtype=np.uint64))


# ----------------------------------------------------------------------------
# bucket boundaries: 64 boundaries at the j/65 quantiles of LogNormal(0, 1)
# ----------------------------------------------------------------------------
def lognormal_boundaries(n_b: int = 64) -> np.ndarray:
    nd = statistics.NormalDist()
    return np.array([math.exp(nd.inv_cdf(j / (n_b + 1))) for j in range(1, n_b + 1)],
                    dtype=np.float32)


# ----------------------------------------------------------------------------
# the five workloads (full size) and reduced variants for parity tests
# ----------------------------------------------------------------------------
def _log_uniform_rows(rng, n, lo, hi):
    return np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))).astype(np.int64)


def config(cfg: int, **ov) -> Workload:
    """Workload `cfg` (1..5) at full size; keyword overrides shrink it."""
    rng = np.random.default_rng(1000 * cfg + 999)
    if cfg == 1:
        C = ov.pop("n_cols", 8)
        rows = ov.pop("rows", 1000)
        cols = [Column(HASH, SUM, F32, rows, 16, 0, ID_SPACE_40) for _ in range(C)]
        w = Workload("tiny-fused-bag", cols, ov.pop("batch", 256), "uniform", 1, 4,
                     id_dist="uniform", opt=OPT_EMIT)
    elif cfg == 2:
        C = ov.pop("n_cols", 200)
        lo, hi = ov.pop("rows_range", (1e4, 1e6))
        rows = _log_uniform_rows(rng, C, lo, hi)
        dims = rng.choice([8, 16, 32, 64], size=C)
        cols = [Column(HASH, SUM if c % 2 == 0 else MEAN, F32, int(rows[c]), int(dims[c]),
                       0, ID_SPACE_40) for c in range(C)]
        w = Workload("training-front-end", cols, ov.pop("batch", 4096), "poisson", bag_mean=3.0,
                     empty_frac=0.05, invalid_frac=0.02, id_dist="zipf", zipf_s=1.1,
                     opt=OPT_SGD, lr=0.01)
    elif cfg == 3:
        C = ov.pop("n_cols", 1000)
        lo, hi = ov.pop("rows_range", (100, 1e5))
        rows = _log_uniform_rows(rng, C, lo, hi)
        dims = rng.choice([4, 8, 16], size=C)
        bnd = lognormal_boundaries(64)
        cols = []
        for c in range(C):
            if c % 10 >= 7:
                cols.append(Column(BUCKET, SUM, F32, max(int(rows[c]), 65), int(dims[c]),
                                   boundaries=bnd))
            else:
                cols.append(Column(HASH, SUM, F32, int(rows[c]), int(dims[c]), 0, ID_SPACE_40))
        w = Workload("many-tiny-columns-inference", cols, ov.pop("batch", 512), "uniform", 1, 8,
                     id_dist="zipf", zipf_s=1.2, float_bag=1, training=False)
    elif cfg == 4:
        C = ov.pop("n_cols", 4)
        rows = ov.pop("rows", 10_000_000)
        cols = [Column(IDENTITY, MEAN, BF16, rows, 64) for _ in range(C)]
        w = Workload("long-behavior-sequences", cols, ov.pop("batch", 2048), "uniform", 200, 2000,
                     id_dist="zipf", zipf_s=1.05, id_space=rows, opt=OPT_ADAGRAD, lr=0.05,
                     eps=1e-8)
    elif cfg == 5:
        cap = ov.pop("capacity", 1 << 26)
        rcap = ov.pop("row_capacity", cap)
        cols = [Column(KEYED, SUM, F32, rcap, 32)]
        w = Workload("collisionless-keyed-table", cols, ov.pop("batch", 8192), "fixed", 100, 100,
                     id_dist="keyed", zipf_s=1.05, opt=OPT_SGD, lr=0.01, capacity=cap,
                     row_capacity=rcap, prepop=ov.pop("prepop", 50_000_000), threshold=2)
    else:
        raise ValueError(cfg)
    for k in list(ov):
        if hasattr(w, k):
            setattr(w, k, ov.pop(k))
    if ov:
        raise TypeError(f"unknown overrides {sorted(ov)}")
    return w


@dataclass
class Batch:
    offsets: np.ndarray            # int32 [C*B+1], bag (c, s) at c*B+s
    ids: np.ndarray                # int64 [N]  (keys for KEYED columns)
    fvals: np.ndarray              # fp32  [N]  (values for BUCKET columns, 0 elsewhere)
    invalid_mask: np.ndarray       # bool [N]: IDs the generator pushed out of range
    forced_empty: np.ndarray       # bool [C*B]
    n: int = 0


def _bag_lengths(w: Workload, rng, col: Column) -> np.ndarray:
    B = w.batch
    if col.kind == BUCKET:
        return np.full(B, w.float_bag, dtype=np.int64)
    if w.bag == "uniform":
        return rng.integers(w.bag_lo, w.bag_hi + 1, size=B)
    if w.bag == "poisson":
        return rng.poisson(w.bag_mean, size=B)
    if w.bag == "fixed":
        return np.full(B, w.bag_lo, dtype=np.int64)
    raise ValueError(w.bag)


def make_batch(w: Workload, seed: int) -> Batch:
    """One jagged batch, column-major: all bags of column 0, then column 1, ..."""
    rng = np.random.default_rng(seed)
    C, B = len(w.cols), w.batch
    lens = np.empty(C * B, dtype=np.int64)
    forced = np.zeros(C * B, dtype=bool)
    for c, col in enumerate(w.cols):
        L = _bag_lengths(w, rng, col)
        if c in w.extra.get("lens", {}):          # per-column uniform lengths
            lo, hi = w.extra["lens"][c]
            L = rng.integers(lo, hi + 1, size=B)
        if w.empty_frac > 0 and col.kind != BUCKET:
            f = rng.random(B) < w.empty_frac
            L = np.where(f, 0, L)
            forced[c * B:(c + 1) * B] = f
        lens[c * B:(c + 1) * B] = L
    offsets = np.zeros(C * B + 1, dtype=np.int64)
    np.cumsum(lens, out=offsets[1:])
    N = int(offsets[-1])
    if N >= (1 << 31):
        raise ValueError("batch too large for int32 offsets")
    ids = np.zeros(N, dtype=np.int64)
    fvals = np.zeros(N, dtype=np.float32)
    invalid = np.zeros(N, dtype=bool)
    zipf = None
    if w.id_dist == "zipf":
        zipf = ZipfSampler(w.id_space, w.zipf_s)
    elif w.id_dist == "keyed":
        zipf = ZipfSampler(w.key_space, w.zipf_s)
    for c, col in enumerate(w.cols):
        a, e = int(offsets[c * B]), int(offsets[(c + 1) * B])
        n = e - a
        if n == 0:
            continue
        if col.kind == BUCKET:
            fvals[a:e] = rng.lognormal(0.0, 1.0, size=n).astype(np.float32)
            continue
        if w.id_dist == "uniform":
            ids[a:e] = rng.integers(0, w.id_space, size=n, dtype=np.int64)
        elif w.id_dist == "zipf":
            ids[a:e] = (zipf.sample(rng, n) - np.uint64(1)).astype(np.int64)
        elif w.id_dist == "keyed":
            ids[a:e] = key_of_rank(zipf.sample(rng, n))
        if w.invalid_frac > 0:
            bad = rng.random(n) < w.invalid_frac
            k = int(bad.sum())
            neg = rng.random(k) < 0.5
            mag = rng.integers(0, w.id_space, size=k, dtype=np.int64)
            vals = np.where(neg, -1 - mag, w.id_space + mag)
            seg = ids[a:e]
            seg[bad] = vals
            invalid[a:e] = bad
    return Batch(offsets.astype(np.int32), ids, fvals, invalid, forced, N)


def make_mask(n: int, seed: int, keep: float = 0.8) -> np.ndarray:
    """A per-position keep mask, uint8 [n]: 1 with probability `keep`, else 0."""
    rng = np.random.default_rng(seed + 7919)
    return (rng.random(n) < keep).astype(np.uint8)


def make_position_weights(n: int, seed: int) -> np.ndarray:
    """Per-position weights, fp32 [n]: uniform in [-1, 2) (signs of both kinds)."""
    rng = np.random.default_rng(seed + 104729)
    return rng.uniform(-1.0, 2.0, size=n).astype(np.float32)


def make_tables(w: Workload, seed: int, device="cpu"):
    """Per-column weight tensors ~ N(0, init_std) (bf16 columns rounded from fp32)
    and zeroed fp32 Adagrad accumulators.  Drawn with torch's generator on
    `device`; parity tests copy them to the other side."""
    import torch
    weights, states = [], []
    for c, col in enumerate(w.cols):
        if col.kind == KEYED:
            weights.append(None)
            states.append(None)
            continue
        g = torch.Generator(device=device)
        g.manual_seed(seed * 100003 + c)
        t = torch.randn(col.rows, col.dim, generator=g, device=device, dtype=torch.float32)
        t.mul_(w.init_std)
        if col.dtype == BF16:
            t = t.to(torch.bfloat16)
        weights.append(t)
        states.append(torch.zeros(col.rows, col.dim, device=device, dtype=torch.float32)
                      if w.opt == OPT_ADAGRAD else None)
    return weights, states


def make_grad(w: Workload, seed: int, device="cpu"):
    """Upstream gradient G ~ N(0, 1), fp32 [B, sum(D)]."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed * 7919 + 17)
    return torch.randn(w.batch, w.sum_dim, generator=g, device=device, dtype=torch.float32)


def make_prepop_rows(n: int, dim: int, std: float, seed: int, device="cpu"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed * 31 + 5)
    t = torch.randn(n, dim, generator=g, device=device, dtype=torch.float32)
    return t.mul_(std)
