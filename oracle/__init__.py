"""CPU oracle of the fused multi-column embedding stage -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, the smoke check and the benchmark's CPU-baseline leg may import this
package.  The product path (the HIP library and its binding) never touches it.

`oracle.c` holds the arithmetic (plain scalar loops, fp64 accumulation); this
module marshals numpy arrays into it with ctypes.  `table.py` holds the keyed
table model (frequency-filtered admission) in numpy.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

ROW_DROPPED = -1
ROW_DEFAULT = -2


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (plain C, no fused multiply-add contraction)."""
    if os.environ.get("ORACLE_LIB"):
        return _LIB                      # a prebuilt variant (mutation tests)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-std=c11", "-Wall",
                               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_SRC_OMP = os.path.join(_HERE, "oracle_omp.c")
_LIB_OMP = os.path.join(_HERE, "liboracle_omp.so")


def build_omp(force: bool = False) -> str:
    """Compile the timing mode (oracle_omp.c: the same oracle, columns over
    OpenMP threads)."""
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_SRC_OMP))
    if force or not os.path.exists(_LIB_OMP) or os.path.getmtime(_LIB_OMP) < newest:
        tmp = _LIB_OMP + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-std=c11", "-fopenmp", "-Wall",
                               "-shared", "-fPIC", _SRC_OMP, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_OMP)
    return _LIB_OMP


class _Col(C.Structure):
    _fields_ = [("kind", C.c_int32), ("pool", C.c_int32), ("dtype", C.c_int32),
                ("dim", C.c_int32), ("rows", C.c_int64), ("id_lo", C.c_int64),
                ("id_hi", C.c_int64), ("boundaries", C.c_void_p), ("n_boundaries", C.c_int64),
                ("weights", C.c_void_p), ("state", C.c_void_p), ("seq_max", C.c_int32),
                ("seq_keep_last", C.c_int32), ("default_row", C.c_int64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = C.CDLL(_LIB)
        L.oracle_splitmix64.restype = C.c_uint64
        L.oracle_splitmix64.argtypes = [C.c_uint64]
        L.oracle_splitmix64_array.argtypes = [C.c_void_p, C.c_void_p, C.c_int64]
        L.oracle_hash_mod.restype = C.c_int64
        L.oracle_hash_mod.argtypes = [C.c_uint64, C.c_int64]
        L.oracle_bucketize.restype = C.c_int64
        L.oracle_bucketize.argtypes = [C.c_void_p, C.c_int64, C.c_float]
        L.oracle_double_to_bf16.restype = C.c_uint16
        L.oracle_double_to_bf16.argtypes = [C.c_double]
        L.oracle_adagrad_elem.restype = C.c_double
        L.oracle_adagrad_elem.argtypes = [C.c_double] * 5 + [C.POINTER(C.c_double)]
        L.oracle_row.restype = C.c_int64
        L.oracle_row.argtypes = [C.POINTER(_Col), C.c_int64, C.c_float, C.c_int32]
        L.oracle_forward.restype = C.c_int64
        L.oracle_forward.argtypes = [C.POINTER(_Col), C.c_int32, C.c_int32] + [C.c_void_p] * 10
        L.oracle_backward.restype = C.c_int64
        L.oracle_backward.argtypes = ([C.POINTER(_Col), C.c_int32, C.c_int32] + [C.c_void_p] * 7
                                      + [C.c_int32, C.c_double, C.c_double]
                                      + [C.c_void_p] * 4 + [C.c_int64])
        L.oracle_init_row.argtypes = [C.c_int64, C.c_int32, C.c_double, C.c_void_p]
        L.oracle_adagrad_array.argtypes = [C.c_void_p] * 3 + [C.c_int64, C.c_double, C.c_double,
                                                                C.c_void_p, C.c_void_p]
        L.oracle_to_bf16_array.argtypes = [C.c_void_p, C.c_int64, C.c_void_p]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


# ------------------------------------------------------------------ scalars

def splitmix64(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x).astype(np.uint64))
    out = np.empty_like(x)
    lib().oracle_splitmix64_array(_p(x), _p(out), x.size)
    return out


def hash_mod(id_bits: int, rows: int) -> int:
    return int(lib().oracle_hash_mod(C.c_uint64(id_bits & (2**64 - 1)), rows))


def bucketize(boundaries: np.ndarray, x: float) -> int:
    b = np.ascontiguousarray(boundaries, dtype=np.float32)
    return int(lib().oracle_bucketize(_p(b), b.size, C.c_float(x)))


def double_to_bf16(v: float) -> int:
    return int(lib().oracle_double_to_bf16(float(v)))


def adagrad_elem(e, a, g, lr, eps):
    a_out = C.c_double()
    e2 = lib().oracle_adagrad_elem(e, a, g, lr, eps, C.byref(a_out))
    return e2, a_out.value


def adagrad_array(e, a, g, lr, eps):
    e = np.ascontiguousarray(e, dtype=np.float64)
    a = np.ascontiguousarray(a, dtype=np.float64)
    g = np.ascontiguousarray(g, dtype=np.float64)
    eo, ao = np.empty_like(e), np.empty_like(e)
    lib().oracle_adagrad_array(_p(e), _p(a), _p(g), e.size, lr, eps, _p(eo), _p(ao))
    return eo, ao


def to_bf16_array(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_to_bf16_array(_p(v), v.size, _p(out))
    return out


def init_row(key: int, dim: int, std: float) -> np.ndarray:
    out = np.empty(dim, dtype=np.float32)
    lib().oracle_init_row(int(key), dim, float(std), _p(out))
    return out


# ------------------------------------------------------------------ columns

class Columns:
    """Column descriptors + host tables (numpy) in the oracle's C layout.

    weights[c]: float32 [rows, dim] or uint16 (bf16 bits) [rows, dim]; states[c]:
    float32 [rows, dim] Adagrad accumulator or None.  Arrays are used in place."""

    def __init__(self, cols, weights, states=None):
        self.cols = cols
        self.weights = [None if w is None else np.ascontiguousarray(w) for w in weights]
        self.states = [None if (states is None or s is None) else np.ascontiguousarray(s)
                       for s in (states or [None] * len(cols))]
        self.bounds = [None if c.boundaries is None else
                       np.ascontiguousarray(c.boundaries, dtype=np.float32) for c in cols]
        arr = (_Col * len(cols))()
        for i, c in enumerate(cols):
            w = self.weights[i]
            if w is not None:
                assert w.shape == (c.rows, c.dim), (w.shape, c.rows, c.dim)
                assert w.dtype == (np.uint16 if c.dtype == 1 else np.float32)
            arr[i] = _Col(c.kind, c.pool, c.dtype, c.dim, c.rows, c.id_lo, c.id_hi,
                          _p(self.bounds[i]), 0 if self.bounds[i] is None else self.bounds[i].size,
                          _p(w), _p(self.states[i]), getattr(c, "seq_max", 0),
                          getattr(c, "seq_keep_last", 0), getattr(c, "default_row", -1))
        self.arr = arr
        self.sum_dim = int(sum(c.dim for c in cols))
        self.max_dim = int(max(c.dim for c in cols))


def _mask(mask):
    return None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)


def _pw(pweights):
    return None if pweights is None else np.ascontiguousarray(pweights, dtype=np.float32)


def forward(cols: Columns, B: int, offsets, ids=None, fvals=None, keyed_rows=None, mask=None,
            pweights=None):
    """Returns (Y fp32 [B, sumD], Ybound fp64 [B, sumD], bag_n int32 [C*B], rows int32 [N]).
    mask: uint8 [N] or None (positions with 0 are dropped); pweights: fp32 [N]
    per-position weights or None (all 1)."""
    mask, pweights = _mask(mask), _pw(pweights)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    n = int(offsets[-1])
    ids = None if ids is None else np.ascontiguousarray(ids, dtype=np.int64)
    fvals = None if fvals is None else np.ascontiguousarray(fvals, dtype=np.float32)
    keyed_rows = None if keyed_rows is None else np.ascontiguousarray(keyed_rows, dtype=np.int32)
    Y = np.zeros((B, cols.sum_dim), dtype=np.float32)
    Yb = np.zeros((B, cols.sum_dim), dtype=np.float64)
    bag_n = np.zeros(len(cols.cols) * B, dtype=np.int32)
    rows = np.zeros(max(n, 1), dtype=np.int32)
    lib().oracle_forward(cols.arr, len(cols.cols), B, _p(offsets), _p(ids), _p(fvals),
                         _p(keyed_rows), _p(mask), _p(pweights), _p(Y), _p(Yb), _p(bag_n),
                         _p(rows))
    return Y, Yb, bag_n, rows[:n]


def backward(cols: Columns, B: int, offsets, G, ids=None, fvals=None, keyed_rows=None,
             opt: int = 0, lr: float = 0.0, eps: float = 0.0, mask=None, pweights=None):
    """Gradient w.r.t. touched rows and the row update `opt` (applied in place to
    cols.weights / cols.states).  Returns (ucol int32 [U], urow int64 [U],
    ugrad fp64 [U, maxD], ubound fp64 [U, maxD])."""
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    n = int(offsets[-1])
    ids = None if ids is None else np.ascontiguousarray(ids, dtype=np.int64)
    fvals = None if fvals is None else np.ascontiguousarray(fvals, dtype=np.float32)
    keyed_rows = None if keyed_rows is None else np.ascontiguousarray(keyed_rows, dtype=np.int32)
    G = np.ascontiguousarray(G, dtype=np.float32)
    assert G.shape == (B, cols.sum_dim)
    mask, pweights = _mask(mask), _pw(pweights)
    cap = max(n + len(cols.cols), 1)          # + one default row per column at most
    ucol = np.zeros(cap, dtype=np.int32)
    urow = np.zeros(cap, dtype=np.int64)
    ug = np.zeros((cap, cols.max_dim), dtype=np.float64)
    ub = np.zeros((cap, cols.max_dim), dtype=np.float64)
    U = lib().oracle_backward(cols.arr, len(cols.cols), B, _p(offsets), _p(ids), _p(fvals),
                              _p(keyed_rows), _p(mask), _p(pweights), _p(G), opt, lr, eps,
                              _p(ucol), _p(urow), _p(ug),
                              _p(ub), cap)
    assert U >= 0
    return ucol[:U], urow[:U], ug[:U], ub[:U]


class ColumnSteps:
    """The timing mode: one forward (+ backward and update) of every column, the
    columns spread over `threads` OpenMP threads (oracle_omp.c).  G is split into
    per-column [B, dim] slices once, here; outputs go to per-column arrays."""

    def __init__(self, cols: Columns, B: int, G=None):
        L = C.CDLL(build_omp())
        L.oracle_step_columns.restype = C.c_int32
        L.oracle_step_columns.argtypes = ([C.POINTER(_Col), C.c_int32, C.c_int32] + [C.c_void_p] * 5
                                          + [C.c_int32, C.c_int32, C.c_double, C.c_double, C.c_int32])
        self.lib, self.cols, self.B = L, cols, B
        dims = [c.dim for c in cols.cols]
        offs = np.concatenate([[0], np.cumsum(dims)])
        self.Y = [np.zeros((B, d), dtype=np.float32) for d in dims]
        self.G = ([np.ascontiguousarray(G[:, offs[c]:offs[c + 1]], dtype=np.float32)
                   for c in range(len(dims))] if G is not None else None)
        self._yp = (C.c_void_p * len(dims))(*[y.ctypes.data for y in self.Y])
        self._gp = (C.c_void_p * len(dims))(*([g.ctypes.data for g in self.G] if self.G is not None
                                              else [None] * len(dims)))

    def run(self, offsets, ids=None, fvals=None, training=False, opt=0, lr=0.0, eps=0.0,
            threads=1) -> int:
        offsets = np.ascontiguousarray(offsets, dtype=np.int32)
        ids = None if ids is None else np.ascontiguousarray(ids, dtype=np.int64)
        fvals = None if fvals is None else np.ascontiguousarray(fvals, dtype=np.float32)
        return int(self.lib.oracle_step_columns(
            self.cols.arr, len(self.cols.cols), self.B, _p(offsets), _p(ids), _p(fvals),
            C.cast(self._yp, C.c_void_p), C.cast(self._gp, C.c_void_p), 1 if training else 0,
            opt, lr, eps, threads))
