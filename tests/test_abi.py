"""The C-ABI library loads without a GPU, exports every entry point that
include/emb.h declares, and rejects bad arguments on the host before any launch."""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "emb.h")


@pytest.fixture(scope="module")
def L():
    import embedding_columns_amd as E
    if not os.path.exists(E.library_path()):
        subprocess.check_call(["bash", os.path.join(ROOT, "embedding_columns_amd", "csrc", "build.sh")])
    return E


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(emb_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared()
    for must in ("emb_plan_create", "emb_forward", "emb_backward", "emb_table_lookup_or_insert"):
        assert must in names


def test_library_exports_every_declared_symbol(L):
    lib = C.CDLL(L.library_path())
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_symbols_are_plain_c(L):
    out = subprocess.run(["nm", "-D", "--defined-only", L.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (emb_[a-z0-9_]+)$", out, flags=re.M))
    assert set(declared()) <= exported


def _col(L, **kw):
    d = dict(kind=L.HASH, pool=L.SUM, dtype=L.F32, dim=16, rows=1000, id_lo=0, id_hi=1 << 40,
             boundaries=None, n_boundaries=0, weights=4096, opt_state=None, default_row=-1)
    d.update(kw)
    return L.ColumnDesc(**d)


def _query(L, cols, batch=8, max_ids=100, opt=0, lr=0.0, eps=0.0, tile=0, fwd_tile=0):
    arr = (L.ColumnDesc * max(len(cols), 1))(*cols)
    pb, wb = C.c_size_t(), C.c_size_t()
    s = L.lib().emb_plan_query(arr, len(cols), batch, max_ids, C.byref(L.PlanOpts(opt, lr, eps, tile, fwd_tile)),
                               C.byref(pb), C.byref(wb))
    return s, pb.value, wb.value, L.emb_last_error()


def test_plan_query_accepts_a_valid_plan(L):
    s, pb, wb, _ = _query(L, [_col(L), _col(L, kind=L.BUCKET, boundaries=8192, n_boundaries=64,
                                          rows=65, dim=4)])
    assert s == 0 and pb >= 2 * 112 and wb > 0


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dim=6), 2, "multiple of 4"),
    (dict(dim=260), 2, "<= 256"),
    (dict(dtype=1, dim=14), 2, "multiple of 4"),
    (dict(dtype=1, dim=264), 2, "<= 256"),
    (dict(rows=0), 1, "rows"),
    (dict(rows=1 << 31), 1, "rows"),
    (dict(kind=7), 1, "kind"),
    (dict(pool=3), 1, "pooling"),
    (dict(id_lo=5, id_hi=5), 1, "id_lo"),
    (dict(weights=None), 1, "weights"),
    (dict(weights=4100), 1, "aligned"),
    (dict(kind=2, boundaries=8192, n_boundaries=64, rows=64), 1, "n_boundaries + 1"),
    (dict(kind=2, boundaries=None, n_boundaries=3, rows=64), 1, "boundaries"),
    (dict(kind=3, dtype=1, dim=16), 2, "fp32"),
    (dict(seq_max=-1), 1, "seq_max"),
    (dict(seq_max=4, seq_keep_last=2), 1, "seq_keep_last"),
    (dict(default_row=1000), 1, "default_row"),
    (dict(default_row=-2), 1, "default_row"),
])
def test_plan_query_rejects_bad_columns(L, kw, status, msg):
    s, _, _, err = _query(L, [_col(L), _col(L, **kw)])
    assert s == status and msg in err


def test_plan_query_rejects_bad_plans(L):
    assert _query(L, [])[0] == 1
    assert _query(L, [_col(L)], batch=0)[0] == 1
    assert _query(L, [_col(L)], max_ids=-1)[0] == 2
    assert _query(L, [_col(L)], tile=100)[0] == 1
    assert _query(L, [_col(L)], tile=512)[0] == 1                        # the backward's tiles <= 256
    for ft in (32, 100, 576, -64):
        s, _, _, err = _query(L, [_col(L)], fwd_tile=ft)
        assert s == 1 and "fwd_tile" in err, ft
    assert _query(L, [_col(L)], fwd_tile=512)[0] == 0
    assert _query(L, [_col(L)], tile=64, fwd_tile=448)[0] == 0
    assert _query(L, [_col(L)], opt=2, lr=0.05, eps=1e-8)[0] == 1          # Adagrad without state
    assert _query(L, [_col(L, opt_state=8192)], opt=2, lr=0.05, eps=1e-8)[0] == 0
    big = [_col(L, rows=(1 << 31) - 1) for _ in range(3)]
    s, _, _, err = _query(L, big)
    assert s == 2 and "2^32" in err


def test_workspace_grows_with_batch(L):
    _, _, w1, _ = _query(L, [_col(L)], batch=8, max_ids=1000)
    _, _, w2, _ = _query(L, [_col(L)], batch=8, max_ids=100000)
    assert w2 > w1


def test_workspace_holds_the_shorter_tiles(L):
    # per-tile partials and tickets are sized for the shorter of the two tile sizes
    _, _, w256, _ = _query(L, [_col(L)], batch=8, max_ids=100000)
    _, _, w64, _ = _query(L, [_col(L)], batch=8, max_ids=100000, fwd_tile=64)
    _, _, w512, _ = _query(L, [_col(L)], batch=8, max_ids=100000, fwd_tile=512)
    assert w64 > w256 and w512 == w256


def test_table_query_validation(L):
    b = C.c_size_t()
    assert L.lib().emb_table_query(1 << 10, 1000, 32, C.byref(b)) == 0 and b.value >= (1 << 10) * 16 + 1000 * 128
    assert L.lib().emb_table_query(1000, 1000, 32, C.byref(b)) == 1
    assert L.lib().emb_table_query(1 << 10, 0, 32, C.byref(b)) == 1
    assert L.lib().emb_table_query(1 << 10, 10, 30, C.byref(b)) == 2


def test_calls_fail_loudly_on_null_plan(L):
    assert L.lib().emb_forward(None, None, None, None, None, 0, None, None, 0, None, None) == 1
    assert L.lib().emb_backward(None, None, None, None, None, None, None, None) == 1
    assert "plan" in L.emb_last_error()
    assert L.lib().emb_backward_dedup(None, None, None, None, None, None) == 1
    assert L.lib().emb_backward_apply(None, None, None, None, None) == 1
    assert L.lib().emb_backward_atomic(None, None, None, None) == 1
    assert L.lib().emb_forward_ex(None, None, None, None, None, None, None, 0, None, None, 0, None,
                                  None) == 1
    assert L.lib().emb_transform(None, None, None, None, None, None, 0, None, None, None) == 1
    assert L.lib().emb_table_evict(None, 0, None, None, None, None) == 1
    assert L.lib().emb_table_save(None, None, None, None, None, None, None, None) == 1
    assert L.lib().emb_table_load(None, None, None, None, None, None, 0, None, None) == 1
    assert L.lib().emb_table_set_step(None, 0) == 1 and L.lib().emb_table_step(None) == -1
    assert L.lib().emb_table_track_seen(None, 1) == 1
    assert L.lib().emb_table_use_count_min(None, 2, 16, None) == 1
    assert L.lib().emb_forward_rows(None, None, None, None, 0, None, None, 0, None, None) == 1
