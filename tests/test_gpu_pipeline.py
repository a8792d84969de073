"""The forward in two launches (emb_transform, then emb_forward_rows) vs the oracle,
and the transform of the next batch on a second stream during the backward.

emb_transform must produce the oracle's row code of every position bit for bit
(hash + mod, identity, bucketize, keyed rows, truncation, the mask); the forward
from those rows must then meet the same bar as the fused forward, backward
included.  The pipelined test runs RecIS Sec. 3.3's overlap: batch t+1's
transform on its own stream while step t's sort and update run, and compares
the tables with a sequential run."""
import numpy as np
import pytest
import torch

import embedding_columns_amd as E
import workloads as W
from gpu_harness import run_dense_case, Step, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("tile", [64, 256])
def test_split_front_end_sgd(tile):
    w = W.config(2, n_cols=24, batch=512, rows_range=(1e2, 1e4))
    run_dense_case(w, seed=9100 + tile, tile=tile, split=True)


def test_split_many_tiny_columns_emit():
    w = W.config(3, n_cols=60, batch=128, rows_range=(100, 3000), opt=W.OPT_EMIT, training=True)
    run_dense_case(w, seed=9200, tile=64, split=True)


def test_split_long_bags_adagrad_truncation_mask_weights():
    w = W.config(4, n_cols=4, batch=24, rows=50_000)
    for c, col in enumerate(w.cols):
        if c % 2:
            col.seq_max, col.seq_keep_last = 300, c % 4 == 1
    run_dense_case(w, seed=9300, tile=128, split=True, mask_keep=0.8, weighted=True)


def test_split_default_rows_and_empty_batch():
    w = W.config(2, n_cols=10, batch=64, rows_range=(50, 500), empty_frac=0.5)
    for c, col in enumerate(w.cols):
        col.default_row = c
    run_dense_case(w, seed=9400, tile=64, split=True)
    w = W.config(2, n_cols=10, batch=64, rows_range=(50, 500), empty_frac=1.0)
    run_dense_case(w, seed=9401, tile=64, split=True)


def test_transform_counts_equal_fused_counts():
    w = W.config(2, n_cols=10, batch=200, rows_range=(100, 1000), opt=W.OPT_EMIT)
    for c, col in enumerate(w.cols):
        if c % 3 == 0:
            col.seq_max = 2
    b = W.make_batch(w, seed=9500)
    mask = W.make_mask(b.n, 9500, 0.8)
    got = []
    for split in (False, True):
        wts, sts = W.make_tables(w, seed=9500, device="cpu")
        st = Step(w, b, wts, sts, tile=128)
        st.forward(training=True, mask=mask, split=split)
        torch.cuda.synchronize()
        got.append(to_np(st.stats))
    assert np.array_equal(got[0], got[1])


def test_pipelined_transform_on_second_stream():
    """Three SGD steps: the transform of batch t+1 runs on another stream (default
    priority) while step t's backward runs; the tables end bit-identical to three
    sequential fused steps."""
    w = W.config(2, n_cols=16, batch=512, rows_range=(1e2, 1e4))
    batches = [W.make_batch(w, seed=9600 + i) for i in range(3)]
    grads = [W.make_grad(w, seed=9600 + i, device="cpu") for i in range(3)]
    n_max = max(b.n for b in batches)
    dev = torch.device("cuda")
    finals = []
    for pipelined in (False, True):
        wts, _ = W.make_tables(w, seed=9600, device="cpu")
        gw = [t.to(dev).contiguous() for t in wts]
        cols = E.EmbeddingColumns(w.cols, gw, batch=w.batch, max_ids=n_max, opt=W.OPT_SGD,
                                  lr=w.lr, tile=256, device=dev)
        offs = [torch.from_numpy(b.offsets).to(dev) for b in batches]
        ids = [torch.from_numpy(b.ids).to(dev) for b in batches]
        G = [g.to(dev) for g in grads]
        Y = torch.empty(w.batch, w.sum_dim, dtype=torch.float32, device=dev)
        if not pipelined:
            for t in range(3):
                E.emb_forward(cols.plan, offs[t], ids[t], None, None, batches[t].n, Y,
                              cols.workspace, 1)
                cols._n = batches[t].n
                cols.backward(G[t], want_count=False)
        else:
            side = torch.cuda.Stream(device=dev)
            main = torch.cuda.current_stream(dev)
            rows = [torch.empty(n_max, dtype=torch.int32, device=dev) for _ in range(2)]
            ready = [torch.cuda.Event() for _ in range(3)]
            E.emb_transform(cols.plan, offs[0], ids[0], None, None, None, batches[0].n, rows[0])
            ready[0].record(main)
            for t in range(3):
                main.wait_event(ready[t])
                E.emb_forward_rows(cols.plan, offs[t], rows[t % 2], None, batches[t].n, Y,
                                   cols.workspace, 1)
                if t + 1 < 3:
                    # the next transform starts once this forward has read rows[t % 2]'s
                    # sibling buffer for the last time (two steps ago)
                    fwd_done = torch.cuda.Event()
                    fwd_done.record(main)
                    side.wait_event(fwd_done)
                    E.emb_transform(cols.plan, offs[t + 1], ids[t + 1], None, None, None,
                                    batches[t + 1].n, rows[(t + 1) % 2], stream=side)
                    ready[t + 1].record(side)
                cols._n = batches[t].n
                cols.backward(G[t], want_count=False)
        torch.cuda.synchronize()
        finals.append([to_np(x) for x in gw])
    for a, b in zip(*finals):
        assert np.array_equal(a, b)
