"""Forward parity for tables on both sides of the 4 GB line.

A table below 4 GB is read through a buffer descriptor whose record count is its
row count, so that dropped and default positions read zeros from the hardware's
range check; a table of 4 GB or more forms 64-bit row addresses.  Each case holds
one column just below the line and one just above it, for each load shape of the
walk (16-byte bf16 slices, 16-byte fp32 slices, 8-byte bf16 slices), with IDs
at the tables' last rows, at their first rows, at random and out of range, in
sum and mean bags.  The oracle runs on compact tables made of the touched rows
(the IDs renumbered into them), which pool to the same sums."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_harness import Step, check_forward, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
LINE = 0xFFFFFFFF          # the largest table, in bytes, read through the descriptor


def _ids(rng, rows, n):
    pool = np.concatenate([
        np.arange(rows - 2000, rows),                 # the last rows
        np.arange(0, 64),                             # the first rows
        rng.integers(0, rows, 500),                   # anywhere
        np.array([rows, rows + 7, -1, -5, 2 ** 40]),  # out of range: dropped
    ])
    return rng.choice(pool, n)


@pytest.mark.parametrize("dtype,dim", [(W.BF16, 64), (W.F32, 256), (W.BF16, 12)],
                         ids=["bf16-16B", "f32-16B", "bf16-8B"])
def test_forward_on_both_sides_of_4gb(dtype, dim):
    esz = 2 if dtype == W.BF16 else 4
    below = LINE // (dim * esz)
    cols = [W.Column(W.IDENTITY, W.SUM, dtype, below, dim),
            W.Column(W.IDENTITY, W.MEAN, dtype, below + 1, dim)]
    assert cols[0].rows * dim * esz <= LINE < cols[1].rows * dim * esz
    B = 64
    rng = np.random.default_rng(910 + dim)
    lens = rng.integers(0, 40, 2 * B)
    lens[[3, B + 5]] = 0                                # empty bags
    offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n = int(offsets[-1])
    ids = np.concatenate([_ids(rng, c.rows, int(lens[i * B:(i + 1) * B].sum()))
                          for i, c in enumerate(cols)]).astype(np.int64)
    b = W.Batch(offsets, ids, np.zeros(n, np.float32), np.zeros(n, bool), lens == 0, n)
    w = W.Workload("4gb-line", cols, B, "fixed", training=False)

    tdt = torch.bfloat16 if dtype == W.BF16 else torch.float32
    tabs, compact, remapped = [], [], ids.copy()
    for i, c in enumerate(cols):
        t = torch.zeros((c.rows, dim), dtype=tdt, device=DEV)
        sel = slice(int(offsets[i * B]), int(offsets[(i + 1) * B]))
        cid = ids[sel]
        valid = (cid >= 0) & (cid < c.rows)
        touched = np.unique(cid[valid])
        vals = torch.randn((touched.size, dim), generator=torch.Generator().manual_seed(i + dim))
        t[torch.from_numpy(touched).to(DEV)] = vals.to(DEV, tdt)
        tabs.append(t)
        compact.append(to_np(t[torch.from_numpy(touched).to(DEV)]))
        # the same IDs in the compact table; dropped ones stay out of its range
        remapped[sel] = np.where(valid, np.searchsorted(touched, cid), -1)
    torch.cuda.synchronize()

    st = Step(w, b, tabs, None, tile=128)
    Y = st.forward(training=False)
    cw = W.Workload("compact", [W.Column(W.IDENTITY, c.pool, dtype, m.shape[0], dim)
                                for c, m in zip(cols, compact)], B, "fixed", training=False)
    ref = oracle.forward(oracle.Columns(cw.cols, compact), B, offsets, remapped, b.fvals)
    torch.cuda.synchronize()
    check_forward(cw, b, Y, None, ref, training=False)
    assert np.count_nonzero(to_np(Y)) > 0
