"""Fused multi-column embedding stage for AMD MI355X (gfx950).

Thin ctypes binding over the C ABI in include/emb.h (libemb.so, built from
csrc/).  Every step of the forward and backward runs in the library's HIP
kernels; this module only marshals torch tensors (device memory) and the current
HIP stream into the C calls.  There is no CPU fallback: importing works without
a GPU, but every call needs the built library and a GPU tensor.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

__all__ = [
    "EmbError", "lib", "library_path", "ColumnDesc", "PlanOpts",
    "emb_plan_query", "emb_plan_create", "emb_plan_destroy", "emb_plan_forward_tile", "emb_forward", "emb_forward_ex", "emb_transform", "emb_forward_rows",
    "emb_forward_noalloc", "emb_stream_copy",
    "emb_backward",
    "emb_backward_dedup", "emb_backward_apply", "emb_backward_atomic",
    "emb_plan_workspace_view", "emb_table_query", "emb_table_create", "emb_table_destroy",
    "emb_table_rows", "emb_table_bulk_insert", "emb_table_lookup_or_insert", "emb_table_find",
    "emb_table_export", "emb_table_step", "emb_table_set_step", "emb_table_track_seen", "emb_table_use_count_min",
    "emb_table_evict",
    "emb_table_save", "emb_table_load", "emb_last_error", "EmbeddingColumns", "KeyedTable",
    "EmbeddingStage",
    "HASH", "IDENTITY", "BUCKET", "KEYED", "SUM", "MEAN", "F32", "BF16", "OPT_EMIT", "OPT_SGD",
    "OPT_ADAGRAD", "ROW_DROPPED", "ROW_DEFAULT", "STAT_COUNT",
]

HASH, IDENTITY, BUCKET, KEYED = 0, 1, 2, 3
SUM, MEAN = 0, 1
F32, BF16 = 0, 1
OPT_EMIT, OPT_SGD, OPT_ADAGRAD = 0, 1, 2
ROW_DROPPED, ROW_DEFAULT = -1, -2
STAT_COUNT = 16
STAT_NAMES = ["ids", "valid", "dropped", "default", "zero_bags", "unique", "table_inserted",
              "table_admitted", "table_full", "max_probe", "filtered", "table_evicted"]

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.environ.get("EMB_LIB") or os.path.join(_HERE, "libemb.so")


class EmbError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"emb status {status}: {msg}")
        self.status = status


class ColumnDesc(C.Structure):
    _fields_ = [("kind", C.c_int32), ("pool", C.c_int32), ("dtype", C.c_int32), ("dim", C.c_int32),
                ("rows", C.c_int64), ("id_lo", C.c_int64), ("id_hi", C.c_int64),
                ("boundaries", C.c_void_p), ("n_boundaries", C.c_int64),
                ("weights", C.c_void_p), ("opt_state", C.c_void_p), ("seq_max", C.c_int32),
                ("seq_keep_last", C.c_int32), ("default_row", C.c_int64)]


class PlanOpts(C.Structure):
    _fields_ = [("opt", C.c_int32), ("lr", C.c_float), ("eps", C.c_float), ("tile", C.c_int32),
                ("fwd_tile", C.c_int32)]


class WorkspaceView(C.Structure):
    _fields_ = [("keys", C.c_void_p), ("bags", C.c_void_p), ("bag_n", C.c_void_p)]


_lib = None
_VP, _I32, _I64, _F = C.c_void_p, C.c_int32, C.c_int64, C.c_float
_SIGS = {
    "emb_plan_query": [C.POINTER(ColumnDesc), _I32, _I32, _I64, C.POINTER(PlanOpts),
                       C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)],
    "emb_plan_create": [C.POINTER(ColumnDesc), _I32, _I32, _I64, C.POINTER(PlanOpts), _VP, _VP,
                        C.POINTER(_VP)],
    "emb_plan_destroy": [_VP],
    "emb_plan_forward_tile": [_VP, _I64, C.POINTER(_I32)],
    "emb_forward": [_VP, _VP, _VP, _VP, _VP, _I64, _VP, _VP, _I32, _VP, _VP],
    "emb_forward_ex": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I64, _VP, _VP, _I32, _VP, _VP],
    "emb_transform": [_VP, _VP, _VP, _VP, _VP, _VP, _I64, _VP, _VP, _VP],
    "emb_forward_rows": [_VP, _VP, _VP, _VP, _I64, _VP, _VP, _I32, _VP, _VP],
    "emb_forward_noalloc": [_VP, _VP, _VP, _VP, _VP, _I64, _VP, _VP, _VP],
    "emb_stream_copy": [_VP, _VP, _I64, _VP],
    "emb_backward": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "emb_backward_dedup": [_VP, _VP, _VP, _VP, _VP, _VP],
    "emb_backward_apply": [_VP, _VP, _VP, _VP, _VP],
    "emb_backward_atomic": [_VP, _VP, _VP, _VP],
    "emb_plan_workspace_view": [_VP, _VP, C.POINTER(WorkspaceView)],
    "emb_table_query": [_I64, _I64, _I32, C.POINTER(C.c_size_t)],
    "emb_table_create": [_I64, _I64, _I32, _I32, _F, _VP, _VP, C.POINTER(_VP)],
    "emb_table_destroy": [_VP],
    "emb_table_bulk_insert": [_VP, _VP, _VP, _I64, _VP, _VP],
    "emb_table_lookup_or_insert": [_VP, _VP, _I64, _VP, _VP, _VP],
    "emb_table_find": [_VP, _VP, _I64, _VP, _VP, _VP],
    "emb_table_export": [_VP, _VP, _VP, _VP, _VP, _VP],
    "emb_table_set_step": [_VP, _I64],
    "emb_table_track_seen": [_VP, _I32],
    "emb_table_use_count_min": [_VP, _I32, _I64, _VP],
    "emb_table_evict": [_VP, _I64, _VP, _VP, _VP, _VP],
    "emb_table_save": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "emb_table_load": [_VP, _VP, _VP, _VP, _VP, _VP, _I64, _VP, _VP],
}


def lib():
    """The loaded libemb.so; raises if it was not built (there is no fallback)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "or embedding_columns_amd/csrc/build.sh")
        L = C.CDLL(path)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = C.c_int
        L.emb_table_rows.argtypes = [_VP]
        L.emb_table_rows.restype = _VP
        L.emb_table_step.argtypes = [_VP]
        L.emb_table_step.restype = C.c_int64
        L.emb_last_error.argtypes = []
        L.emb_last_error.restype = C.c_char_p
        _lib = L
    return _lib


def emb_last_error() -> str:
    return lib().emb_last_error().decode()


def _check(status: int):
    if status != 0:
        raise EmbError(status, emb_last_error())


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("the embedding stage runs on the GPU: pass device tensors")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# --------------------------------------------------------------- C-ABI names

def emb_plan_query(descs, batch, max_ids, opts):
    pb, wb = C.c_size_t(), C.c_size_t()
    _check(lib().emb_plan_query(descs, len(descs), batch, max_ids, C.byref(opts), C.byref(pb),
                                C.byref(wb)))
    return pb.value, wb.value


def emb_plan_create(descs, batch, max_ids, opts, plan_mem, stream=None):
    out = _VP()
    _check(lib().emb_plan_create(descs, len(descs), batch, max_ids, C.byref(opts), _ptr(plan_mem),
                                 _stream(stream), C.byref(out)))
    return out.value


def emb_plan_destroy(plan):
    _check(lib().emb_plan_destroy(plan))


def emb_plan_forward_tile(plan, n_ids):
    t = _I32()
    _check(lib().emb_plan_forward_tile(plan, n_ids, C.byref(t)))
    return t.value


def emb_forward(plan, offsets, ids, fvals, keyed_rows, n_ids, out, workspace, training,
                stats=None, stream=None):
    _check(lib().emb_forward(plan, _ptr(offsets), _ptr(ids), _ptr(fvals), _ptr(keyed_rows), n_ids,
                             _ptr(out), _ptr(workspace), 1 if training else 0, _ptr(stats),
                             _stream(stream)))


def emb_forward_ex(plan, offsets, ids, fvals, keyed_rows, pweights, mask, n_ids, out, workspace,
                   training, stats=None, stream=None):
    _check(lib().emb_forward_ex(plan, _ptr(offsets), _ptr(ids), _ptr(fvals), _ptr(keyed_rows),
                                _ptr(pweights), _ptr(mask), n_ids, _ptr(out), _ptr(workspace),
                                1 if training else 0, _ptr(stats), _stream(stream)))


def emb_transform(plan, offsets, ids, fvals, keyed_rows, mask, n_ids, rows_out, stats=None,
                  stream=None):
    _check(lib().emb_transform(plan, _ptr(offsets), _ptr(ids), _ptr(fvals), _ptr(keyed_rows),
                               _ptr(mask), n_ids, _ptr(rows_out), _ptr(stats), _stream(stream)))


def emb_forward_rows(plan, offsets, rows, pweights, n_ids, out, workspace, training, stats=None,
                     stream=None):
    _check(lib().emb_forward_rows(plan, _ptr(offsets), _ptr(rows), _ptr(pweights), n_ids,
                                  _ptr(out), _ptr(workspace), 1 if training else 0, _ptr(stats),
                                  _stream(stream)))


def emb_forward_noalloc(plan, offsets, ids, fvals, keyed_rows, n_ids, out, stats=None,
                        stream=None):
    _check(lib().emb_forward_noalloc(plan, _ptr(offsets), _ptr(ids), _ptr(fvals),
                                     _ptr(keyed_rows), n_ids, _ptr(out), _ptr(stats),
                                     _stream(stream)))


def emb_backward(plan, grad_out, workspace, uniq_keys=None, uniq_grads=None, n_uniq=None,
                 stats=None, stream=None):
    _check(lib().emb_backward(plan, _ptr(grad_out), _ptr(workspace), _ptr(uniq_keys),
                              _ptr(uniq_grads), _ptr(n_uniq), _ptr(stats), _stream(stream)))


def emb_backward_dedup(plan, workspace, uniq_keys=None, n_uniq=None, stats=None, stream=None):
    _check(lib().emb_backward_dedup(plan, _ptr(workspace), _ptr(uniq_keys), _ptr(n_uniq),
                                    _ptr(stats), _stream(stream)))


def emb_backward_apply(plan, grad_out, workspace, uniq_grads=None, stream=None):
    _check(lib().emb_backward_apply(plan, _ptr(grad_out), _ptr(workspace), _ptr(uniq_grads),
                                    _stream(stream)))


def emb_backward_atomic(plan, grad_out, workspace, stream=None):
    _check(lib().emb_backward_atomic(plan, _ptr(grad_out), _ptr(workspace), _stream(stream)))


def emb_stream_copy(dst, src, nbytes, stream=None):
    _check(lib().emb_stream_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)))


def emb_plan_workspace_view(plan, workspace):
    v = WorkspaceView()
    _check(lib().emb_plan_workspace_view(plan, _ptr(workspace), C.byref(v)))
    return v


def emb_table_query(capacity, row_capacity, dim):
    b = C.c_size_t()
    _check(lib().emb_table_query(capacity, row_capacity, dim, C.byref(b)))
    return b.value


def emb_table_create(capacity, row_capacity, dim, threshold, init_std, table_mem, stream=None):
    out = _VP()
    _check(lib().emb_table_create(capacity, row_capacity, dim, threshold, init_std,
                                  _ptr(table_mem), _stream(stream), C.byref(out)))
    return out.value


def emb_table_destroy(table):
    _check(lib().emb_table_destroy(table))


def emb_table_rows(table):
    return lib().emb_table_rows(table)


def emb_table_bulk_insert(table, keys, rows, n, stats=None, stream=None):
    _check(lib().emb_table_bulk_insert(table, _ptr(keys), _ptr(rows), n, _ptr(stats),
                                       _stream(stream)))


def emb_table_lookup_or_insert(table, keys, n, rows_out, stats=None, stream=None):
    _check(lib().emb_table_lookup_or_insert(table, _ptr(keys), n, _ptr(rows_out), _ptr(stats),
                                            _stream(stream)))


def emb_table_find(table, keys, n, rows_out, counts_out=None, stream=None):
    _check(lib().emb_table_find(table, _ptr(keys), n, _ptr(rows_out), _ptr(counts_out),
                                _stream(stream)))


def emb_table_export(table, keys, counts, rows, n_out, stream=None):
    _check(lib().emb_table_export(table, _ptr(keys), _ptr(counts), _ptr(rows), _ptr(n_out),
                                  _stream(stream)))


def emb_table_step(table) -> int:
    return int(lib().emb_table_step(table))


def emb_table_set_step(table, step):
    _check(lib().emb_table_set_step(table, step))


def emb_table_use_count_min(table, depth, width, sketch):
    _check(lib().emb_table_use_count_min(table, depth, width, _ptr(sketch)))


def emb_table_track_seen(table, on):
    _check(lib().emb_table_track_seen(table, 1 if on else 0))


def emb_table_evict(table, min_seen, opt_state=None, n_live=None, stats=None, stream=None):
    _check(lib().emb_table_evict(table, min_seen, _ptr(opt_state), _ptr(n_live), _ptr(stats),
                                 _stream(stream)))


def emb_table_save(table, keys, counts, seen, admitted, values, n_out, stream=None):
    _check(lib().emb_table_save(table, _ptr(keys), _ptr(counts), _ptr(seen), _ptr(admitted),
                                _ptr(values), _ptr(n_out), _stream(stream)))


def emb_table_load(table, keys, counts, seen, admitted, values, n, stats=None, stream=None):
    _check(lib().emb_table_load(table, _ptr(keys), _ptr(counts), _ptr(seen), _ptr(admitted),
                                _ptr(values), n, _ptr(stats), _stream(stream)))


# ------------------------------------------------------------- convenience

def _u8(nbytes, device, zero=False):
    n = max(int(nbytes), 256)
    return (torch.zeros if zero else torch.empty)(n, dtype=torch.uint8, device=device)


class EmbeddingColumns:
    """A plan over columns with caller-owned tables (torch tensors on the GPU).

    cols: objects with kind, pool, dtype, rows, dim, id_lo, id_hi and optional
    boundaries (fp32 array-like), seq_max, seq_keep_last and default_row; weights[c]: [rows, dim] fp32/bf16 tensor (for a
    KEYED column, the table's row pool); states[c]: fp32 Adagrad accumulator."""

    def __init__(self, cols, weights, states=None, batch=1, max_ids=0, opt=OPT_EMIT, lr=0.0,
                 eps=0.0, tile=0, fwd_tile=0, device="cuda"):
        self.device = torch.device(device)
        self.batch, self.max_ids = int(batch), int(max_ids)
        self.cols = list(cols)
        self.weights = list(weights)
        self.states = list(states) if states is not None else [None] * len(self.cols)
        self.bounds = []
        descs = (ColumnDesc * len(self.cols))()
        for i, c in enumerate(self.cols):
            b = getattr(c, "boundaries", None)
            bt = None
            if c.kind == BUCKET and b is not None:
                bt = torch.as_tensor(b, dtype=torch.float32).to(self.device).contiguous()
            self.bounds.append(bt)
            w, s = self.weights[i], self.states[i]
            descs[i] = ColumnDesc(c.kind, c.pool, c.dtype, c.dim, c.rows, getattr(c, "id_lo", 0),
                                  getattr(c, "id_hi", 0), _ptr(bt) if bt is not None else None,
                                  0 if bt is None else bt.numel(), _ptr(w),
                                  _ptr(s) if s is not None else None, getattr(c, "seq_max", 0),
                                  getattr(c, "seq_keep_last", 0), getattr(c, "default_row", -1))
        self.descs = descs
        self.opts = PlanOpts(opt, lr, eps, tile, fwd_tile)
        self.sum_dim = sum(c.dim for c in self.cols)
        self.max_dim = max(c.dim for c in self.cols)
        pb, wb = emb_plan_query(descs, self.batch, self.max_ids, self.opts)
        self.plan_mem = _u8(pb, self.device)
        self.workspace = _u8(wb, self.device, zero=True)
        self.plan = emb_plan_create(descs, self.batch, self.max_ids, self.opts, self.plan_mem)
        self._destroy = lib().emb_plan_destroy   # still callable while the interpreter exits
        self.row_base = [0]
        for c in self.cols:
            self.row_base.append(self.row_base[-1] + c.rows)

    def __del__(self):
        p, destroy = getattr(self, "plan", None), getattr(self, "_destroy", None)
        if p and destroy:
            try:
                torch.cuda.synchronize(self.device)
            except Exception:
                pass
            destroy(p)
            self.plan = None

    def forward(self, offsets, ids=None, fvals=None, keyed_rows=None, training=True, stats=None,
                out=None, weights=None, mask=None):
        """weights: fp32 [n_ids] per-position weights or None; mask: uint8 [n_ids]
        (0 removes a position) or None.  Device tensors."""
        n = (ids if ids is not None else fvals if fvals is not None else keyed_rows)
        n_ids = 0 if n is None else n.numel()
        if out is None:
            out = torch.empty(self.batch, self.sum_dim, dtype=torch.float32, device=self.device)
        if mask is None and weights is None:
            emb_forward(self.plan, offsets, ids, fvals, keyed_rows, n_ids, out, self.workspace,
                        training, stats)
        else:
            assert mask is None or (mask.dtype == torch.uint8 and mask.numel() >= n_ids)
            assert weights is None or (weights.dtype == torch.float32 and weights.numel() >= n_ids)
            emb_forward_ex(self.plan, offsets, ids, fvals, keyed_rows, weights, mask, n_ids, out,
                           self.workspace, training, stats)
        self._n = n_ids
        return out

    def backward(self, grad_out, want_keys=False, want_grads=False, stats=None, want_count=True):
        """Returns (uniq_keys, uniq_grads, n_uniq) device tensors (None where not asked).
        With nothing asked (no keys, grads, count or stats) and SGD / Adagrad, the
        library skips building the unique-row list."""
        n_def = sum(1 for c in self.cols if getattr(c, "default_row", -1) >= 0)
        n = max(getattr(self, "_n", 0) + n_def, 1)
        keys = torch.empty(n, dtype=torch.int32, device=self.device) if want_keys else None
        grads = (torch.empty(n, self.max_dim, dtype=torch.float32, device=self.device)
                 if want_grads else None)
        nu = torch.zeros(1, dtype=torch.int64, device=self.device) if want_count else None
        emb_backward(self.plan, grad_out.contiguous(), self.workspace, keys, grads, nu, stats)
        return keys, grads, nu

    def __call__(self, offsets, ids=None, fvals=None, keyed_rows=None, weights=None, mask=None):
        """The pooled output [batch, sum(dim)]; under autograd (grad mode on) it is
        an EmbeddingStage node whose backward runs emb_backward."""
        if not torch.is_grad_enabled():
            return self.forward(offsets, ids, fvals, keyed_rows, training=False, weights=weights,
                                mask=mask)
        if getattr(self, "_anchor", None) is None:
            self._anchor = torch.zeros((), device=self.device, requires_grad=True)
        return EmbeddingStage.apply(self, self._anchor, offsets, ids, fvals, keyed_rows, weights,
                                    mask, *self.weights)

    def sparse_table_grads(self, keys, grads, n_uniq, want):
        """EMIT results as one sparse COO gradient [rows, dim] per table (None where
        want[c] is false): the distinct keys row_base_c + row are split by column."""
        n = int(n_uniq.item())
        k = keys[:n].to(torch.int64) & 0xFFFFFFFF
        base = torch.tensor(self.row_base, dtype=torch.int64, device=self.device)
        col = torch.searchsorted(base, k, right=True) - 1
        out = []
        for c, spec in enumerate(self.cols):
            if not want[c]:
                out.append(None)
                continue
            sel = col == c
            rows = (k[sel] - self.row_base[c]).unsqueeze(0)
            vals = grads[:n][sel][:, :spec.dim].to(self.weights[c].dtype)
            out.append(torch.sparse_coo_tensor(rows, vals, (spec.rows, spec.dim),
                                               is_coalesced=True))
        return out

    def backward_atomic(self, grad_out):
        """SGD by atomic scatter of every contribution (no sort; not bit-reproducible)."""
        emb_backward_atomic(self.plan, grad_out.contiguous(), self.workspace)

    def forward_tile(self, n_ids):
        """Positions per forward tile for a batch of n_ids positions."""
        return emb_plan_forward_tile(self.plan, n_ids)

    def workspace_view(self, n_ids):
        v = emb_plan_workspace_view(self.plan, self.workspace)
        base = self.workspace.data_ptr()
        nb = len(self.cols) * self.batch

        def view(ptr, count):
            off = ptr - base
            return self.workspace[off:off + 4 * count].view(torch.int32)
        return view(v.keys, n_ids), view(v.bags, n_ids), view(v.bag_n, nb)


class EmbeddingStage(torch.autograd.Function):
    """The fused stage as an autograd node: the forward is emb_forward (training),
    the backward emb_backward with the plan's optimizer.  Table lookup and update
    are framework operations, as Monolith Sec. 2.1 treats its hash-table lookups
    and updates like Variables.

    apply(cols, anchor, offsets, ids, fvals, keyed_rows, pweights, mask, *tables):
    `anchor` is a scalar that requires grad, so that autograd reaches this node even
    when no table does; `tables` are the plan's weight tensors.  With SGD or Adagrad
    the backward updates the touched rows in place and returns no table gradient.
    With EMIT it keeps the distinct touched keys, their gradients and their count
    on `cols.emitted`, and gives every table that requires grad a sparse COO
    gradient over its touched rows."""

    @staticmethod
    def forward(ctx, cols, anchor, offsets, ids, fvals, keyed_rows, pweights, mask, *tables):
        ctx.cols = cols
        ctx.want = [t is not None and t.requires_grad for t in tables]
        return cols.forward(offsets, ids, fvals, keyed_rows, training=True, weights=pweights,
                            mask=mask)

    @staticmethod
    def backward(ctx, grad_y):
        cols = ctx.cols
        g = grad_y.contiguous()
        if g.dtype != torch.float32:
            raise TypeError("the pooled output's gradient must be fp32")
        if cols.opts.opt != OPT_EMIT:
            cols.backward(g, want_count=False)
            return (None,) * (8 + len(ctx.want))
        keys, grads, nu = cols.backward(g, want_keys=True, want_grads=True)
        cols.emitted = (keys, grads, nu)
        return (None,) * 8 + tuple(cols.sparse_table_grads(keys, grads, nu, ctx.want))


class KeyedTable:
    """Collisionless keyed table (device memory owned by this object)."""

    def __init__(self, capacity, row_capacity, dim, threshold=2, init_std=0.01, device="cuda",
                 track_seen=False):
        self.device = torch.device(device)
        self.capacity, self.row_capacity, self.dim = int(capacity), int(row_capacity), int(dim)
        nbytes = emb_table_query(self.capacity, self.row_capacity, self.dim)
        self.mem = _u8(nbytes, self.device)
        self.table = emb_table_create(self.capacity, self.row_capacity, self.dim, threshold,
                                      init_std, self.mem)
        self._destroy = lib().emb_table_destroy
        if track_seen:
            emb_table_track_seen(self.table, True)
        ptr = emb_table_rows(self.table)
        off = ptr - self.mem.data_ptr()
        self.rows = self.mem[off:off + 4 * self.row_capacity * self.dim].view(torch.float32).view(
            self.row_capacity, self.dim)

    def __del__(self):
        t, destroy = getattr(self, "table", None), getattr(self, "_destroy", None)
        if t and destroy:
            destroy(t)
            self.table = None

    def bulk_insert(self, keys, rows=None, stats=None):
        emb_table_bulk_insert(self.table, keys, rows, keys.numel(), stats)

    def lookup_or_insert(self, keys, rows_out=None, stats=None):
        if rows_out is None:
            rows_out = torch.empty(keys.numel(), dtype=torch.int32, device=self.device)
        emb_table_lookup_or_insert(self.table, keys, keys.numel(), rows_out, stats)
        return rows_out

    def find(self, keys):
        rows = torch.empty(keys.numel(), dtype=torch.int32, device=self.device)
        counts = torch.empty(keys.numel(), dtype=torch.int32, device=self.device)
        emb_table_find(self.table, keys, keys.numel(), rows, counts)
        return rows, counts

    def use_count_min(self, depth, width):
        """Count-min admission with a fresh depth x width sketch (owned by this object)."""
        self.sketch = torch.zeros(depth, width, dtype=torch.int32, device=self.device)
        emb_table_use_count_min(self.table, depth, width, self.sketch)

    @property
    def step(self) -> int:
        """The table step the next lookup_or_insert records."""
        return emb_table_step(self.table)

    def set_step(self, step):
        emb_table_set_step(self.table, int(step))

    def evict(self, min_seen, opt_state=None, stats=None):
        """Removes keys last seen before step min_seen; returns the live-key count
        (a device tensor)."""
        n_live = torch.zeros(1, dtype=torch.int64, device=self.device)
        emb_table_evict(self.table, int(min_seen), opt_state, n_live, stats)
        return n_live

    def save(self):
        """A checkpoint: (keys, counts, last_seen, admitted, values, step)."""
        cap, dev = self.capacity, self.device
        keys = torch.empty(cap, dtype=torch.int64, device=dev)
        counts = torch.empty(cap, dtype=torch.int32, device=dev)
        seen = torch.empty(cap, dtype=torch.int32, device=dev)
        adm = torch.empty(cap, dtype=torch.uint8, device=dev)
        vals = torch.empty(cap, self.dim, dtype=torch.float32, device=dev)
        n = torch.zeros(1, dtype=torch.int64, device=dev)
        emb_table_save(self.table, keys, counts, seen, adm, vals, n)
        k = int(n.item())
        return keys[:k], counts[:k], seen[:k], adm[:k], vals[:k], self.step

    def load(self, ckpt, stats=None):
        keys, counts, seen, adm, vals, step = ckpt
        emb_table_load(self.table, keys, counts, seen, adm, vals.contiguous(), keys.numel(), stats)
        self.set_step(step)

    def export(self):
        keys = torch.empty(self.capacity, dtype=torch.int64, device=self.device)
        counts = torch.empty(self.capacity, dtype=torch.int32, device=self.device)
        rows = torch.empty(self.capacity, dtype=torch.int32, device=self.device)
        n = torch.zeros(1, dtype=torch.int64, device=self.device)
        emb_table_export(self.table, keys, counts, rows, n)
        k = int(n.item())
        return keys[:k], counts[:k], rows[:k]
