"""Runs one step of the HIP path and of the CPU oracle on the same seeded inputs
and compares them (used by the GPU parity tests and the smoke check)."""
from __future__ import annotations

import numpy as np
import torch

import embedding_columns_amd as E
import oracle
import workloads as W

RTOL_F32 = 1e-5      # relative to sum |term| (fp32 accumulation in a different order)


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def as_f64(col, w):
    if col.dtype == W.BF16:
        return (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return w.astype(np.float64)


def positions_columns(offsets, C, B):
    lens = np.diff(offsets.astype(np.int64))
    bag = np.repeat(np.arange(C * B), lens)
    return bag, bag // B


class Step:
    """One training (or inference) step of the HIP path."""

    def __init__(self, w: W.Workload, batch: W.Batch, weights, states, tile=0, device="cuda",
                 keyed_rows=None, keyed_pool=None, fwd_tile=0):
        self.dev = torch.device(device)
        self.w, self.b = w, batch
        self.gw = []
        for c, t in enumerate(weights):
            if w.cols[c].kind == W.KEYED:
                self.gw.append(keyed_pool)
            else:
                self.gw.append(t.to(self.dev).contiguous() if t is not None else None)
        self.gs = [None if s is None else s.to(self.dev).contiguous() for s in (states or [None] * len(w.cols))]
        self.cols = E.EmbeddingColumns(w.cols, self.gw, self.gs, batch=w.batch,
                                       max_ids=max(batch.n, 1), opt=w.opt, lr=w.lr, eps=w.eps,
                                       tile=tile, fwd_tile=fwd_tile, device=self.dev)
        self.off = torch.from_numpy(batch.offsets).to(self.dev)
        self.ids = torch.from_numpy(batch.ids).to(self.dev) if batch.n else torch.zeros(1, dtype=torch.int64, device=self.dev)
        self.fv = torch.from_numpy(batch.fvals).to(self.dev) if batch.n else torch.zeros(1, dtype=torch.float32, device=self.dev)
        self.kr = keyed_rows
        self.stats = torch.zeros(E.STAT_COUNT, dtype=torch.int64, device=self.dev)

    def forward(self, training=True, mask=None, pweights=None, split=False):
        """mask: uint8 numpy [N], pweights: fp32 numpy [N], or None (with both None
        the plain entry point runs).  split: emb_transform, then emb_forward_rows."""
        kinds = {c.kind for c in self.w.cols}
        n = self.b.n
        ids = self.ids[:n] if n else None
        fv = self.fv[:n] if n else None
        Y = torch.empty(self.w.batch, self.w.sum_dim, dtype=torch.float32, device=self.dev)
        args = (ids if (kinds & {W.HASH, W.IDENTITY}) and n else None,
                fv if W.BUCKET in kinds and n else None,
                self.kr if W.KEYED in kinds and n else None)
        if split:
            m = None if mask is None or not n else torch.from_numpy(
                np.ascontiguousarray(mask, dtype=np.uint8)).to(self.dev)
            v = None if pweights is None or not n else torch.from_numpy(
                np.ascontiguousarray(pweights, dtype=np.float32)).to(self.dev)
            self.rows = torch.full((max(n, 1),), -7, dtype=torch.int32, device=self.dev)
            E.emb_transform(self.cols.plan, self.off, *args, m, n, self.rows if n else None,
                            self.stats)
            E.emb_forward_rows(self.cols.plan, self.off, self.rows if n else None, v, n, Y,
                               self.cols.workspace, training, self.stats)
        elif mask is None and pweights is None:
            E.emb_forward(self.cols.plan, self.off, *args, n, Y, self.cols.workspace, training,
                          self.stats)
        else:
            m = None if mask is None or not n else torch.from_numpy(
                np.ascontiguousarray(mask, dtype=np.uint8)).to(self.dev)
            v = None if pweights is None or not n else torch.from_numpy(
                np.ascontiguousarray(pweights, dtype=np.float32)).to(self.dev)
            E.emb_forward_ex(self.cols.plan, self.off, *args, v, m, n, Y, self.cols.workspace,
                             training, self.stats)
        self.cols._n = n
        return Y

    def backward(self, G, want_grads=None, ask_unique=True):
        """ask_unique=False (SGD / Adagrad) asks for nothing back, so the library
        finds the segments from the sorted keys without the unique-row list."""
        if want_grads is None:
            want_grads = self.w.opt == W.OPT_EMIT
        if not ask_unique:
            return self.cols.backward(G.to(self.dev).contiguous(), want_count=False)
        return self.cols.backward(G.to(self.dev).contiguous(), want_keys=True,
                                  want_grads=want_grads, stats=self.stats)


def oracle_columns(w, weights_np, states_np=None):
    return oracle.Columns(w.cols, weights_np, states_np)


def check_forward(w, b, Y_gpu, ws_view, ref, training=True):
    """Bit-exact integer results, condition-aware float tolerance."""
    Y, Yb, bag_n, rows = ref
    C, B = len(w.cols), w.batch
    y = to_np(Y_gpu)
    err = np.abs(y.astype(np.float64) - Y.astype(np.float64))
    bad = err > RTOL_F32 * Yb
    assert not bad.any(), (f"forward mismatch at {np.argwhere(bad)[:5].tolist()}: "
                           f"gpu {y[bad][:5]} ref {Y[bad][:5]} bound {Yb[bad][:5]}")
    if not training or b.n == 0:
        return
    keys, bags, gbag_n = ws_view
    keys = to_np(keys).view(np.uint32).astype(np.int64)
    bags = to_np(bags)
    gbag_n = to_np(gbag_n)
    bag_idx, col_idx = positions_columns(b.offsets, C, B)
    row_base = np.concatenate([[0], np.cumsum([c.rows for c in w.cols])])
    total = row_base[-1]
    grows = np.where(keys == total, -1, np.where(keys == total + 1, -2, keys - row_base[col_idx]))
    assert np.array_equal(grows, rows.astype(np.int64)), "transformed rows differ"
    assert np.array_equal(bags, bag_idx), "bag index per position differs"
    assert np.array_equal(gbag_n, bag_n), "valid count per bag differs"


def check_unique(w, ukeys_gpu, nu_gpu, ucol, urow):
    nu = int(nu_gpu.item())
    row_base = np.concatenate([[0], np.cumsum([c.rows for c in w.cols])])
    ref_keys = row_base[ucol] + urow
    got = to_np(ukeys_gpu[:nu]).view(np.uint32).astype(np.int64) if nu else np.zeros(0, np.int64)
    assert nu == ref_keys.size, f"{nu} unique rows, oracle has {ref_keys.size}"
    assert np.array_equal(got, ref_keys), "unique row keys differ"


def check_emit(w, ugrads_gpu, nu, ucol, ug, ub):
    # lanes past a column's width are not written: convert only the written ones
    g = to_np(ugrads_gpu[:nu])
    for u in range(nu):
        D = w.cols[ucol[u]].dim
        err = np.abs(g[u, :D].astype(np.float64) - ug[u, :D])
        assert np.all(err <= RTOL_F32 * ub[u, :D]), f"gradient of unique row {u} differs"


def check_rows_sgd(col, before, after_gpu, after_ref, touched, gbound, lr):
    """Updated rows: E' = E - lr g with |g - g_ref| <= rtol sum|term|, plus rounding."""
    b64, g64, r64 = as_f64(col, before), as_f64(col, after_gpu), as_f64(col, after_ref)
    untouched = np.setdiff1d(np.arange(col.rows), touched)
    assert np.array_equal(after_gpu[untouched], before[untouched]), "untouched rows changed"
    d = np.abs(g64[touched] - r64[touched])
    ulp = 2.0 ** (-7 if col.dtype == W.BF16 else -22)
    tol = lr * RTOL_F32 * gbound + ulp * (np.abs(r64[touched]) + np.abs(b64[touched])) + 1e-30
    assert np.all(d <= tol), f"SGD rows differ: max {d.max()} tol {tol[d > tol][:3]}"


def check_rows_adagrad(col, before, st_before, after_gpu, st_gpu, g_ref, gbound, touched, lr, eps):
    """E'(g) = E - lr g / (sqrt(A + g^2) + eps) is monotone in g: the GPU result
    must lie between the oracle's E'(g_ref + delta) and E'(g_ref - delta),
    delta = rtol sum|term|, each rounded to the weight dtype, with fp32 slack."""
    untouched = np.setdiff1d(np.arange(col.rows), touched)
    assert np.array_equal(after_gpu[untouched], before[untouched]), "untouched rows changed"
    assert np.array_equal(st_gpu[untouched], st_before[untouched]), "untouched state changed"
    e0 = as_f64(col, before[touched]).ravel()
    a0 = st_before[touched].astype(np.float64).ravel()
    g = g_ref.ravel()
    dlt = RTOL_F32 * gbound.ravel() + 1e-30
    hi_e, _ = oracle.adagrad_array(e0, a0, g - dlt, lr, eps)
    lo_e, _ = oracle.adagrad_array(e0, a0, g + dlt, lr, eps)
    # fp32 evaluation of E - lr g / (sqrt(A) + eps) with the hardware square root and
    # reciprocal (about 1 ulp each), two rounded products, the rounded eps add and the
    # final subtraction: at most 4 ulp (2^-23 relative) of |E| + lr
    slack = 8 * 2.0 ** -24 * (np.abs(e0) + lr)
    lo_e, hi_e = lo_e - slack, hi_e + slack
    got = as_f64(col, after_gpu[touched]).ravel()
    if col.dtype == W.BF16:
        lo_e = as_f64(col, oracle.to_bf16_array(lo_e))
        hi_e = as_f64(col, oracle.to_bf16_array(hi_e))
    assert np.all((got >= lo_e) & (got <= hi_e)), "Adagrad rows outside the oracle's interval"
    # accumulator: A + g^2 over the same interval of g
    gmin = np.where((g - dlt <= 0) & (g + dlt >= 0), 0.0, np.minimum(np.abs(g - dlt), np.abs(g + dlt)))
    gmax = np.maximum(np.abs(g - dlt), np.abs(g + dlt))
    a_got = st_gpu[touched].astype(np.float64).ravel()
    lo_a = (a0 + gmin * gmin) * (1 - 2 ** -22)
    hi_a = (a0 + gmax * gmax) * (1 + 2 ** -22)
    assert np.all((a_got >= lo_a) & (a_got <= hi_a)), "Adagrad accumulators outside the interval"


def run_dense_case(w, seed, tile=0, training=True, device="cuda", check_bwd=True, ask_unique=True,
                   mask_keep=None, weighted=False, split=False, fwd_tile=0):
    """Full parity of one step for HASH / IDENTITY / BUCKET workloads.  With
    ask_unique=False the backward returns nothing (the benchmark's path) and only
    the updated rows are compared.  mask_keep: run the masked forward with a
    random mask that keeps each position with this probability.  weighted: pass
    random per-position weights.  split: the forward as emb_transform followed by
    emb_forward_rows, whose row codes must equal the oracle's bit for bit.  fwd_tile:
    the forward's own tile size (0: as the plan chooses)."""
    b = W.make_batch(w, seed=seed)
    mask = None if mask_keep is None else W.make_mask(b.n, seed, mask_keep)
    pw = W.make_position_weights(b.n, seed) if weighted else None
    wts, sts = W.make_tables(w, seed=seed, device="cpu")
    G = W.make_grad(w, seed=seed, device="cpu")
    st = Step(w, b, wts, sts, tile=tile, device=device, fwd_tile=fwd_tile)
    Y = st.forward(training=training, mask=mask, pweights=pw, split=split)
    ws = st.cols.workspace_view(max(b.n, 1)) if training else None
    ws = (ws[0][:b.n], ws[1][:b.n], ws[2]) if ws is not None else None
    host_w = [to_np(t) for t in wts]
    host_s = [None if s is None else to_np(s) for s in sts]
    oc = oracle_columns(w, [x.copy() for x in host_w], [None if s is None else s.copy() for s in host_s])
    ref = oracle.forward(oc, w.batch, b.offsets, b.ids, b.fvals, mask=mask, pweights=pw)
    torch.cuda.synchronize()
    if split and b.n:
        assert np.array_equal(to_np(st.rows)[:b.n], ref[3]), "emb_transform row codes differ"
    check_forward(w, b, Y, ws, ref, training)
    out = {"Y": Y, "step": st, "batch": b, "ref": ref, "mask": mask, "pweights": pw}
    if not (training and check_bwd):
        return out
    ukeys, ugrads, nu = st.backward(G, ask_unique=ask_unique)
    torch.cuda.synchronize()
    ucol, urow, ug, ub = oracle.backward(oc, w.batch, b.offsets, G.numpy(), b.ids, b.fvals,
                                         opt=w.opt, lr=w.lr, eps=w.eps, mask=mask, pweights=pw)
    if ask_unique:
        check_unique(w, ukeys, nu, ucol, urow)
    if w.opt == W.OPT_EMIT:
        check_emit(w, ugrads, int(nu.item()), ucol, ug, ub)
    for c, col in enumerate(w.cols):
        if w.opt == W.OPT_EMIT:
            assert np.array_equal(to_np(st.gw[c]), host_w[c]), "EMIT must not touch tables"
            continue
        sel = ucol == c
        touched = urow[sel]
        D = col.dim
        if w.opt == W.OPT_SGD:
            check_rows_sgd(col, host_w[c], to_np(st.gw[c]), oc.weights[c], touched,
                           ub[sel][:, :D], w.lr)
        else:
            check_rows_adagrad(col, host_w[c], host_s[c], to_np(st.gw[c]), to_np(st.gs[c]),
                               ug[sel][:, :D], ub[sel][:, :D], touched, w.lr, w.eps)
    out.update(ukeys=ukeys, ugrads=ugrads, nu=nu)
    return out
