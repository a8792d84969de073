"""The forward's two tile capacities vs the oracle.

The forward kernel exists for tiles of up to 256 positions and, with more inputs
per lane and fewer waves per SIMD, of up to 512.  A plan without a fixed size
takes 512-position tiles for a batch whose mean bag has 64 positions or more
(long sequences: fewer bags cut into pieces) and that makes at least 6144 such
tiles, else 256; fwd_tile fixes the size.  These cases run the long instance on
long bags, forced onto short bags (many bags and columns per tile, bags never
cut), with the extended forward's parts (truncation, the mask, weights, default
rows), the split transform, and sizes between the two capacities; the backward
behind it runs on its own tile size.  The full-size long-sequence case (its
own test module) takes the long tiles by the plan's choice."""
import pytest

import embedding_columns_amd as E
import workloads as W
from gpu_harness import run_dense_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("tile,fwd_tile", [(0, 0), (128, 512), (64, 320), (256, 448)])
def test_long_sequences_bf16_adagrad_forward_tiles(tile, fwd_tile):
    # bags of 200..2000 IDs: every tile boundary cuts a bag; (0, 0): the plan's choice (256 here)
    w = W.config(4, n_cols=4, batch=40, rows=100_000)
    run_dense_case(w, seed=4100 + fwd_tile + tile, tile=tile, fwd_tile=fwd_tile)


def test_long_sequences_hot_rows_forward_tiles():
    # 5,000-row tables: hot rows, and the backward's segments from the sorted keys
    w = W.config(4, n_cols=4, batch=40, rows=5_000)
    run_dense_case(w, seed=4114, fwd_tile=512, tile=64, ask_unique=False)


@pytest.mark.parametrize("tile", [64, 256])
def test_short_bags_in_long_tiles(tile):
    # Poisson(3) bags, empty bags, invalid IDs, sum/mean, dims 8..64, SGD; ~170 bags a tile
    w = W.config(2, n_cols=24, batch=512, rows_range=(1e2, 1e4))
    run_dense_case(w, seed=4200 + tile, tile=tile, fwd_tile=512)


@pytest.mark.parametrize("training", [False, True])
def test_many_tiny_columns_in_long_tiles(training):
    # hashed and bucketized columns; a tile spans tens of columns
    w = W.config(3, n_cols=100, batch=128, rows_range=(100, 1e4))
    run_dense_case(w, seed=4300, tile=256, fwd_tile=512, training=training, check_bwd=False)


@pytest.mark.parametrize("split", [False, True])
def test_long_tiles_truncation_mask_weights(split):
    w = W.config(4, n_cols=4, batch=24, rows=50_000)
    for c, col in enumerate(w.cols):
        if c % 2:
            col.seq_max, col.seq_keep_last = 300, c % 4 == 1
    run_dense_case(w, seed=4400 + split, split=split, mask_keep=0.8, weighted=True, fwd_tile=512)


def test_long_tiles_default_rows_masked_out():
    # a mask keeping 0.1 % of positions leaves most long bags empty: default rows
    w = W.config(4, n_cols=4, batch=24, rows=50_000)
    for c, col in enumerate(w.cols):
        col.default_row = (7 * c + 3) % col.rows
    run_dense_case(w, seed=4500, mask_keep=0.001, fwd_tile=512)


def test_long_tiles_emit():
    w = W.config(4, n_cols=4, batch=32, rows=20_000, opt=W.OPT_EMIT)
    run_dense_case(w, seed=4600, fwd_tile=512)


def test_forward_tile_choice():
    many = 512 * 6144                  # positions of the fewest long tiles worth taking
    top = 3_200_000

    def plan(batch, **kw):
        w = W.config(4, n_cols=4, batch=batch, rows=1000)
        wts, sts = W.make_tables(w, seed=1, device="cuda")
        return E.EmbeddingColumns(w.cols, wts, sts, batch=batch, max_ids=top, opt=w.opt, lr=w.lr,
                                  eps=w.eps, device="cuda", **kw)
    # 160 bags: the batch's size decides
    p = plan(40)
    assert [p.forward_tile(n) for n in (0, 1, many - 1, many, top)] == [256, 256, 256, 512, 512]
    with pytest.raises(E.EmbError):
        p.forward_tile(top + 1)
    # 50,000 bags: the mean bag decides (64 positions)
    p = plan(12_500)
    assert [p.forward_tile(n) for n in (many, 64 * 50_000 - 1, 64 * 50_000)] == [256, 256, 512]
    assert {plan(40, tile=128).forward_tile(n) for n in (0, top)} == {128}
    assert {plan(40, tile=128, fwd_tile=320).forward_tile(n) for n in (0, top)} == {320}
    assert {plan(40, fwd_tile=64).forward_tile(n) for n in (0, top)} == {64}
