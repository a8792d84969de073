"""The GPU's exact 64-bit remainder at its edges, bit for bit against the oracle.

RecIS Sec. 3.1 lists hashing and the modulo among the fused feature transforms;
the hashed row is the unsigned remainder of the SplitMix64 hash by the table
size.  The kernels compute it by a multiply-high with floor((2^64 - 1) / rows)
and one correction, which is exact by construction; these tests feed it what a
wrong remainder gets wrong: table sizes 1, 2, 2^10, 2^20, 10^7 and 2^31 - 1,
and raw IDs whose hash is exactly 0, 1, 2^64 - 1, 2^63, 2^32 +- 1, a multiple of
the table size or its neighbour (at the bottom, middle and top of the 64-bit
range), within 2^20 of 0 or of 2^64 - 1, plus random IDs over the whole int64
range.  The IDs are found by running SplitMix64 backwards on the host (a CPU
test checks each against the oracle's hash).  The row codes of emb_transform and
of the training forward must equal the oracle's bit for bit; the pooled outputs,
the distinct rows and the emitted gradients of one EMIT step through the same
columns are compared too (the 2^31 - 1 row table is 32 GiB of zeros on the GPU
with the touched rows filled, and a lazily allocated array on the host).
"""
import numpy as np
import pytest
import torch

import embedding_columns_amd as E
import oracle
import workloads as W
from gpu_harness import RTOL_F32, check_unique, to_np
from splitmix_inverse import M64, edge_hashes, id_for_hash

pytestmark = pytest.mark.gpu

ROWS = [1, 2, 1024, 1 << 20, 10_000_000, (1 << 31) - 1]
D = 4
B = 1024


def column_ids(rows, n_random, rng):
    hs = list(edge_hashes(rows))
    hs += [int(h) for h in rng.integers(0, 1 << 20, 2000, dtype=np.uint64)]
    hs += [M64 - int(h) for h in rng.integers(0, 1 << 20, 2000, dtype=np.uint64)]
    ids = [id_for_hash(h) for h in hs]
    ids += [int(x) for x in rng.integers(-(1 << 63), (1 << 63) - 1, n_random, dtype=np.int64)]
    ids = np.array(ids, dtype=np.int64)
    return ids[rng.permutation(ids.size)]


@pytest.mark.parametrize("n_random", [6_000, 100_000])
def test_hash_mod_edges(n_random):
    dev = torch.device("cuda")
    rng = np.random.default_rng(777 + n_random)
    cols, ids_all, offsets = [], [], [0]
    for c, rows in enumerate(ROWS):
        cols.append(W.Column(kind=W.HASH, pool=W.SUM if c % 2 == 0 else W.MEAN, dtype=W.F32,
                             rows=rows, dim=D, id_lo=-(1 << 63), id_hi=(1 << 63) - 1))
        ids = column_ids(rows, n_random, rng)
        cuts = np.sort(rng.integers(0, ids.size + 1, B - 1))
        lens = np.diff(np.concatenate([[0], cuts, [ids.size]]))
        offsets += list(offsets[-1] + np.cumsum(lens))
        ids_all.append(ids)
    ids = np.concatenate(ids_all)
    offsets = np.array(offsets, dtype=np.int32)
    n = ids.size
    # every ID here lies inside [id_lo, id_hi) except 2^63 - 1 itself
    host_w, gpu_w = [], []
    for c, col in enumerate(cols):
        a, e = int(offsets[c * B]), int(offsets[(c + 1) * B])
        h = oracle.splitmix64(ids[a:e].view(np.uint64))
        touched = np.unique([int(x) % col.rows for x in h])
        vals = rng.standard_normal((touched.size, D)).astype(np.float32) * np.float32(0.01)
        hw = np.zeros((col.rows, D), dtype=np.float32)      # lazily allocated pages
        hw[touched] = vals
        gw = torch.zeros((col.rows, D), dtype=torch.float32, device=dev)
        gw[torch.from_numpy(touched).to(dev)] = torch.from_numpy(vals).to(dev)
        host_w.append(hw)
        gpu_w.append(gw)
    G = rng.standard_normal((B, D * len(cols))).astype(np.float32)

    plan = E.EmbeddingColumns(cols, gpu_w, batch=B, max_ids=n, opt=E.OPT_EMIT, device=dev)
    off = torch.from_numpy(offsets).to(dev)
    gids = torch.from_numpy(ids).to(dev)
    rows_gpu = torch.full((n,), -7, dtype=torch.int32, device=dev)
    E.emb_transform(plan.plan, off, gids, None, None, None, n, rows_gpu)
    Y = plan.forward(off, ids=gids, training=True)
    # the forward's saved keys, before the backward's sort reuses their buffer
    wkeys, _, wbag_n = (t.clone() for t in plan.workspace_view(n))
    keys, grads, nu = plan.backward(torch.from_numpy(G).to(dev), want_keys=True, want_grads=True)
    torch.cuda.synchronize()

    oc = oracle.Columns(cols, host_w)
    Yr, Yb, bag_n, rows_ref = oracle.forward(oc, B, offsets, ids)
    # the transform's row codes, bit for bit (every position is valid except 2^63 - 1)
    got = to_np(rows_gpu)
    assert np.array_equal(got, rows_ref), (
        f"row codes differ at {np.flatnonzero(got != rows_ref)[:5].tolist()}")
    assert (rows_ref == -1).sum() == (ids == (1 << 63) - 1).sum()
    # the training forward's keys carry the same rows
    row_base = np.concatenate([[0], np.cumsum([c.rows for c in cols])]).astype(np.int64)
    col_of = np.repeat(np.arange(len(cols)), np.diff(offsets[::B].astype(np.int64)))
    k = to_np(wkeys).view(np.uint32).astype(np.int64)
    total = int(row_base[-1])
    grows = np.where(k == total, -1, k - row_base[col_of])
    assert np.array_equal(grows, rows_ref.astype(np.int64)), "forward keys differ"
    assert np.array_equal(to_np(wbag_n), bag_n)
    # pooled outputs
    err = np.abs(to_np(Y).astype(np.float64) - Yr.astype(np.float64))
    assert np.all(err <= RTOL_F32 * Yb), f"pooled outputs differ by {err.max()}"
    # distinct rows and emitted gradients
    ucol, urow, ug, ub = oracle.backward(oc, B, offsets, G, ids, opt=W.OPT_EMIT)
    w = W.Workload(name="modulo-edges", cols=cols, batch=B, bag="fixed")
    check_unique(w, keys, nu, ucol, urow)
    g = to_np(grads[:int(nu.item())])[:, :D].astype(np.float64)
    assert np.all(np.abs(g - ug[:, :D]) <= RTOL_F32 * ub[:, :D]), "emitted gradients differ"
