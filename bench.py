"""Throughput of the fused multi-column embedding stage on one MI355X.

Default workload: long behaviour sequences, the largest workload that runs on one
GPU -- 4 identity columns, batch 2048, bags of 200..2000 IDs (9.0 M positions per
step), Zipf(1.05) item IDs over 1e7-row bf16 tables of dim 64 (fp32 accumulation),
mean pooling, one Adagrad step (lr 0.05, eps 1e-8, fp32 state).  A step is one
forward launch plus the backward (sort of the touched row keys, then a
segment-sum and the Adagrad update of each distinct row) over one batch already
resident in HBM; steps cycle a pool of pre-generated batches.  Other workloads:
--workload tiny | front-end | inference | keyed.

Prints one JSON line: lookups/s (valid (column, sample, ID) positions per second
over the timed steps, host clock), every library call of the step timed with HIP
events on its stream, the roofline of the call with the largest time per step
(algorithmic bytes / its average time, against the 8 TB/s peak and against the
bandwidth of a plain streaming copy measured in the same run), the HBM traffic of
that kernel from the committed counter summary, and the CPU oracle timed on the
host, single-threaded and with its columns over OpenMP threads.

  python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--workload NAME]

(the keyed-table workload defaults to 20 steps after 5)
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "embedding_columns_amd", "csrc")


def source_hash() -> str:
    """sha256 over the HIP/C++ sources: a counter summary applies only to the
    kernels it was measured on."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h"))
                    + glob.glob(os.path.join(CSRC, "*.cpp"))):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when the kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"source_sha256:\s*([0-9a-f]{64})", txt)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", txt)
    if not m or not t or m.group(1) != source_hash():
        return None
    return int(t.group(1))
WORKLOADS = {"tiny": 1, "front-end": 2, "inference": 3, "long-seq": 4, "keyed": 5}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def elem_size(col):
    return 2 if col.dtype == 1 else 4


def fwd_bytes(w, b, valid_per_col, gathers_per_col, training):
    """Algorithmic bytes of one forward: raw inputs, CSR offsets, one row read
    per valid non-default position, the pooled output, and (training) one 4-byte
    row index per valid position kept for the backward."""
    C, B = len(w.cols), w.batch
    n_int = sum(int(b.offsets[(c + 1) * B] - b.offsets[c * B]) for c, col in enumerate(w.cols)
                if col.kind != 2)
    n_flt = b.n - n_int
    byts = 8 * n_int + 4 * n_flt + 4 * (C * B + 1)
    byts += sum(gathers_per_col[c] * col.dim * elem_size(col) for c, col in enumerate(w.cols))
    byts += 4 * B * w.sum_dim
    if training:
        byts += 4 * sum(valid_per_col)
    return byts


def bwd_bytes(w, valid_total, uniq_per_col):
    """Saved row indices + upstream gradient read once + the row update of each
    distinct touched row (EMIT: key + gradient; SGD: row read + write; Adagrad:
    row read + write and the fp32 accumulator read + write)."""
    byts = 4 * valid_total + 4 * w.batch * w.sum_dim
    for c, col in enumerate(w.cols):
        u, d, e = uniq_per_col[c], col.dim, elem_size(col)
        if w.opt == 0:
            byts += u * (4 + 4 * d)
        elif w.opt == 1:
            byts += u * 2 * d * e
        else:
            byts += u * (2 * d * e + 8 * d)
    return byts


def per_col_counts(w, b):
    C, B = len(w.cols), w.batch
    valid, gathers = [], []
    for c, col in enumerate(w.cols):
        a, e = int(b.offsets[c * B]), int(b.offsets[(c + 1) * B])
        v = (e - a) - int(b.invalid_mask[a:e].sum())
        if col.kind == 2:
            v = (e - a) - int(np.isnan(b.fvals[a:e]).sum())
        valid.append(v)
        gathers.append(v)
    return valid, gathers


def run(args):
    import torch

    import embedding_columns_amd as E
    import workloads as W

    dev = torch.device("cuda:0")
    cfg = WORKLOADS[args.workload]
    w = W.config(cfg)
    keyed = cfg == 5
    training = w.training and not args.inference
    t0 = time.time()
    n_pool = args.batches if not keyed else args.warmup + args.steps
    batches = [W.make_batch(w, seed=1000 * cfg + i) for i in range(n_pool)]
    log(f"[bench] {w.name}: {n_pool} batches generated in {time.time() - t0:.1f}s, "
        f"positions/batch {np.mean([b.n for b in batches]):.0f}")
    dbat = []
    for j, b in enumerate(batches):
        dbat.append(dict(off=torch.from_numpy(b.offsets).to(dev), ids=torch.from_numpy(b.ids).to(dev),
                         fv=torch.from_numpy(b.fvals).to(dev), n=b.n,
                         pw=(torch.from_numpy(W.make_position_weights(b.n, 1000 * cfg + j)).to(dev)
                             if args.weights else None)))
    max_ids = max(b.n for b in batches)

    table = None
    if keyed:
        table = E.KeyedTable(w.capacity, w.row_capacity, 32, threshold=w.threshold,
                             init_std=w.init_std, device=dev)
        t0 = time.time()
        chunk = 10_000_000
        for s in range(0, w.prepop, chunk):
            k = torch.from_numpy(W.key_of_rank(np.arange(s + 1, min(s + chunk, w.prepop) + 1,
                                                         dtype=np.uint64))).to(dev)
            rows = W.make_prepop_rows(k.numel(), 32, w.init_std, seed=s, device=dev)
            table.bulk_insert(k, rows)
            del rows
        torch.cuda.synchronize()
        log(f"[bench] prepopulated {w.prepop} keys in {time.time() - t0:.1f}s")
        weights, states = [table.rows], [None]
    else:
        weights, states = W.make_tables(w, seed=cfg, device=dev)
    plan = E.EmbeddingColumns(w.cols, weights, states, batch=w.batch, max_ids=max_ids, opt=w.opt,
                              lr=w.lr, eps=w.eps, tile=args.tile, fwd_tile=args.fwd_tile, device=dev)
    G = W.make_grad(w, seed=cfg, device=dev)
    stats = torch.zeros(E.STAT_COUNT, dtype=torch.int64, device=dev)
    Y = torch.empty(w.batch, w.sum_dim, dtype=torch.float32, device=dev)
    # keyed: one rows buffer per step, read after the timed region for the counts
    krows = torch.empty(n_pool, max_ids, dtype=torch.int32, device=dev) if keyed else None
    kinds = {c.kind for c in w.cols}
    # EMIT: the backward's output, the distinct rows' keys and gradients
    emit = training and w.opt == 0
    ukeys = torch.empty(max(max_ids, 1), dtype=torch.int32, device=dev) if emit else None
    nuniq = torch.zeros(1, dtype=torch.int64, device=dev) if emit else None
    ugrads = (torch.empty(max(max_ids, 1), max(c.dim for c in w.cols), dtype=torch.float32, device=dev)
              if emit else None)

    # device counters only with --stats (their atomics cost time); they are then
    # reported summed over the timed steps
    tstats = stats if args.stats else None
    kstats = stats if args.stats else None

    # --pipeline: batch i+1's transform (emb_transform) runs on a second stream at
    # default priority while step i's backward runs; step i's forward gathers from
    # the row codes (emb_forward_rows).  Row-code buffers alternate between steps.
    pipe = args.pipeline and not keyed
    if pipe:
        main_s = torch.cuda.current_stream(dev)
        side_s = torch.cuda.Stream(device=dev)
        prow = [torch.empty(max(max_ids, 1), dtype=torch.int32, device=dev) for _ in range(2)]
        ready = {}
        tev = []

    def transform(i, stream):
        d = dbat[i % len(dbat)]
        E.emb_transform(plan.plan, d["off"], d["ids"] if kinds & {0, 1} else None,
                        d["fv"] if 2 in kinds else None, None, None, d["n"], prow[i % 2], tstats,
                        stream=stream)
        ready[i] = torch.cuda.Event()
        ready[i].record(stream)

    # events of one timed step: named points on the launch stream; each library
    # call of the step lies between two of them
    def mark(ev, name):
        if ev is not None:
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            ev[name] = e

    def step(i, ev=None):
        d = dbat[i % len(dbat)]
        n = d["n"]
        mark(ev, "start")
        if keyed:
            table.lookup_or_insert(d["ids"], rows_out=krows[i][:n], stats=kstats)
            mark(ev, "table")
        if pipe:
            if i not in ready:
                transform(i, main_s)
            main_s.wait_event(ready.pop(i))
            mark(ev, "fwd0")
        if pipe:
            E.emb_forward_rows(plan.plan, d["off"], prow[i % 2], None, n, Y, plan.workspace,
                               training, tstats)
            mark(ev, "fwd")
            # the next transform may overwrite prow[(i + 1) % 2] once this forward is
            # queued: that buffer's last reader was the previous step's forward
            done = torch.cuda.Event()
            done.record(main_s)
            side_s.wait_event(done)
            if ev is not None:
                t0e, t1e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                t0e.record(side_s)
            transform(i + 1, side_s)
            if ev is not None:
                t1e.record(side_s)
                tev.append((t0e, t1e))
        elif args.weights:
            E.emb_forward_ex(plan.plan, d["off"], d["ids"] if kinds & {0, 1} else None,
                             d["fv"] if 2 in kinds else None, krows[i][:n] if keyed else None,
                             d["pw"], None, n, Y, plan.workspace, training, tstats)
            mark(ev, "fwd")
        else:
            E.emb_forward(plan.plan, d["off"], d["ids"] if kinds & {0, 1} else None,
                          d["fv"] if 2 in kinds else None, krows[i][:n] if keyed else None, n, Y,
                          plan.workspace, training, tstats)
            mark(ev, "fwd")
        if training and args.atomic_backward:
            # the pages' backward (atomic adds, no sort), for comparison
            E.emb_backward_atomic(plan.plan, G, plan.workspace)
            mark(ev, "apply")
        elif training:
            E.emb_backward_dedup(plan.plan, plan.workspace, ukeys, nuniq, tstats)
            mark(ev, "dedup")
            E.emb_backward_apply(plan.plan, G, plan.workspace, ugrads)
            mark(ev, "apply")

    # --graph: each batch's forward, dedup and apply captured once as three HIP
    # graphs (the library's calls are plain kernel launches on the caller's
    # stream, with no allocation, copy or memset), then replayed: one host call
    # per stage instead of one per kernel.  Events between the replays time the
    # stages as in the eager loop.
    graphs = []

    def capture():
        torch.cuda.synchronize()
        for j, d in enumerate(dbat):
            n = d["n"]
            ids = d["ids"] if kinds & {0, 1} else None
            fv = d["fv"] if 2 in kinds else None
            gs = [torch.cuda.CUDAGraph() for _ in range(3 if training else 1)]
            with torch.cuda.graph(gs[0]):
                E.emb_forward(plan.plan, d["off"], ids, fv, None, n, Y, plan.workspace, training, tstats)
            if training:
                with torch.cuda.graph(gs[1]):
                    E.emb_backward_dedup(plan.plan, plan.workspace, ukeys, nuniq, tstats)
                with torch.cuda.graph(gs[2]):
                    E.emb_backward_apply(plan.plan, G, plan.workspace, ugrads)
            graphs.append(gs)
        torch.cuda.synchronize()

    def replay(i, ev=None):
        gs = graphs[i % len(graphs)]
        mark(ev, "start")
        gs[0].replay()
        mark(ev, "fwd")
        if training:
            gs[1].replay()
            mark(ev, "dedup")
            gs[2].replay()
            mark(ev, "apply")

    # per-batch algorithmic bytes (dense workloads: valid counts from the generator's
    # masks, distinct rows from one untimed backward per batch)
    counts = [per_col_counts(w, b) for b in batches]
    uniq = []
    if training and not keyed:
        for i, b in enumerate(batches):
            E.emb_forward(plan.plan, dbat[i]["off"], dbat[i]["ids"] if kinds & {0, 1} else None,
                          dbat[i]["fv"] if 2 in kinds else None, None, b.n, Y, plan.workspace,
                          True, None)
            keys = torch.empty(max(b.n, 1), dtype=torch.int32, device=dev)
            nu = torch.zeros(1, dtype=torch.int64, device=dev)
            E.emb_backward(plan.plan, G, plan.workspace, keys, None, nu, None)
            k = keys[:int(nu.item())].cpu().numpy().view(np.uint32).astype(np.int64)
            rb = np.array(plan.row_base)
            uniq.append(np.bincount(np.searchsorted(rb, k, side="right") - 1, minlength=len(w.cols)))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.graph:
        capture()
        run_step = replay
    else:
        run_step = step
    stats.zero_()
    evs = [dict() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"[bench] {args.steps} timed steps in {wall * 1e3:.1f} ms")
    st = stats.cpu().numpy()

    def span(a, b):
        return np.array([e[a].elapsed_time(e[b]) for e in evs])

    # the calls of a step and the events around each
    calls = {}
    if keyed:
        calls["table_lookup"] = ("start", "table")
    calls["fwd_kernel"] = ("fwd0" if pipe else ("table" if keyed else "start"), "fwd")
    if training and args.atomic_backward:
        calls["atomic_apply"] = ("fwd", "apply")
    elif training:
        calls["dedup"] = ("fwd", "dedup")
        calls["seg_apply"] = ("dedup", "apply")
    ms = {k: span(*v) for k, v in calls.items()}
    step_ms = span("start", "apply" if training else "fwd")

    idx = [(args.warmup + i) % len(dbat) for i in range(args.steps)]
    if keyed:
        # per timed step: positions reading a row, reading DEFAULT, distinct rows
        rows_read, defaults, distinct = [], [], []
        for i in range(args.steps):
            r = krows[args.warmup + i][:batches[args.warmup + i].n]
            rows_read.append(int((r >= 0).sum().item()))
            defaults.append(int((r == -2).sum().item()))
            distinct.append(int(torch.unique(r[r >= 0]).numel()))
        lookups = sum(rows_read) + sum(defaults)         # admitted rows + DEFAULT reads
        n_steps = args.steps
        fb = np.mean([fwd_bytes(w, batches[j], [counts[j][0][0]], [rows_read[k]], True)
                      for k, j in enumerate(idx)])
        ub = np.mean([bwd_bytes(w, rows_read[k], [distinct[k]]) for k in range(n_steps)])
        # per key: the key, one 16-byte slot, its row code out
        tb = float(np.mean([28 * batches[j].n for j in idx]))
        step_bytes = fb + ub + tb
    else:
        lookups = sum(sum(counts[j][0]) for j in idx)
        fb = np.mean([fwd_bytes(w, batches[j], counts[j][0], counts[j][1], training) for j in idx])
        ub = (np.mean([bwd_bytes(w, sum(counts[j][0]), uniq[j]) for j in idx]) if training else 0.0)
        tb = 0.0
        step_bytes = fb + ub
    algo = {"table_lookup": tb, "fwd_kernel": fb, "dedup": 0.0, "seg_apply": ub, "atomic_apply": ub}
    launches = {"table_lookup": "ht_count, ht_admit, ht_resolve", "fwd_kernel": "fwd_kernel",
                "dedup": "the sort of the touched keys (overhead: no algorithmic bytes)",
                "seg_apply": "seg_apply", "atomic_apply": "atomic_apply"}

    # a plain streaming copy of 1 GiB (read + write), the library's own kernel
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    E.emb_stream_copy(dst, src, src.numel() * 4)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    reps = 10
    for _ in range(reps):
        E.emb_stream_copy(dst, src, src.numel() * 4)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) * reps / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    value = lookups / wall
    ms_step = 1000.0 * wall / args.steps
    kernels = {}
    for k, v in ms.items():
        avg = float(np.mean(v))
        kernels[k] = {"us": round(1000 * avg, 2), "median_us": round(1000 * float(np.median(v)), 2),
                      "launches": launches[k], "algorithmic_bytes": int(algo[k]),
                      "gbs": round(algo[k] / (avg * 1e-3) / 1e9, 1)}
    if pipe:
        kernels["transform_side_stream"] = {
            "us": round(1000 * float(np.mean([a.elapsed_time(b) for a, b in tev])), 2)}
    # the dominant call: the largest time per step
    dom = max(ms, key=lambda k: float(np.mean(ms[k])))
    dk = kernels[dom]
    achieved = dk["gbs"]
    traffic = measured_traffic(dom, w.name)
    out = {
        "metric": "pooled embedding lookups/sec (fwd+bwd) at 1 GPU; achieved HBM GB/s vs peak",
        "value": round(value, 1),
        "unit": "lookups/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if any(c.dtype == 1 for c in w.cols) else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "columns": len(w.cols), "batch": w.batch,
                   "positions_per_step": int(np.mean([batches[j].n for j in idx])),
                   "valid_lookups_per_step": int(lookups / args.steps),
                   "optimizer": ["emit", "sgd", "adagrad"][w.opt] if training else "none",
                   "backward": ("atomic" if args.atomic_backward else "sorted") if training else "none",
                   "tile": plan.opts.tile or 256, "fwd_tile": plan.forward_tile(batches[idx[0]].n),
                   "fwd_launches_per_step": 2 if pipe else 1,
                   "pipelined_transform": bool(pipe),
                   "position_weights": bool(args.weights),
                   "hip_graph": bool(args.graph)},
        "step_gbs": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_median_ms": round(float(np.median(step_ms)), 4),
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes": dk["algorithmic_bytes"], "launch_us": dk["us"],
                     "copy_gbs": round(copy_gbs, 1), "frac_of_copy": round(achieved / copy_gbs, 4)},
        "kernels": kernels,
    }
    if args.stats:
        out["counters"] = {n: int(v) for n, v in zip(E.STAT_NAMES, st)}
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = {"read": 1 << 30, "write": 1 << 30}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, batches, plan, G, weights, states)
    print(json.dumps(out), flush=True)


def host_cpu():
    """(logical CPUs this process may use, the CPU model name)"""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return n, model


def cpu_baseline(w, batches, plan, G, weights, states, min_seconds=8.0):
    """The oracle (C, fp64) on this machine's host cores, forward + backward + the
    row update over batches of the same workload, each mode cycled for at least
    min_seconds (a bounded sample of the timed run): single-threaded (the
    reference mode), and with the columns spread over OpenMP threads (as many as
    OMP_NUM_THREADS, else the CPUs this process may use).  The reported value is
    the faster of the two."""
    import torch

    import oracle
    import workloads as W
    if any(c.kind == W.KEYED for c in w.cols):
        return None
    t0 = time.time()
    host_w = []
    for t in weights:
        h = t.cpu()
        host_w.append(h.view(torch.int16).numpy().view(np.uint16) if h.dtype == torch.bfloat16
                      else h.numpy())
    host_s = [None if s is None else s.cpu().numpy() for s in states]
    Gh = G.cpu().numpy()
    log(f"[bench] oracle inputs copied to host in {time.time() - t0:.1f}s")
    ncpu, model = host_cpu()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or ncpu
    step = "forward + backward + update" if w.training else "forward"

    def timed(run_one):
        dt, valid, runs, i = 0.0, 0, 0, 0
        while dt < min_seconds:
            b = batches[i % len(batches)]
            t0 = time.perf_counter()
            run_one(b)
            dt += time.perf_counter() - t0
            valid += sum(per_col_counts(w, b)[0])
            runs += 1
            i += 1
        return valid / dt, runs, valid, dt

    # single-threaded reference mode
    oc = oracle.Columns(w.cols, host_w, host_s)

    def one_ref(b):
        oracle.forward(oc, w.batch, b.offsets, b.ids, b.fvals)
        if w.training:
            oracle.backward(oc, w.batch, b.offsets, Gh, b.ids, b.fvals, opt=w.opt, lr=w.lr,
                            eps=w.eps)
    v1, r1, n1, t1 = timed(one_ref)
    # columns over threads (the same oracle, one column per call)
    cs = oracle.ColumnSteps(oracle.Columns(w.cols, host_w, host_s), w.batch, Gh)
    used = [1]

    def one_par(b):
        used[0] = cs.run(b.offsets, b.ids, b.fvals, training=w.training, opt=w.opt, lr=w.lr,
                         eps=w.eps, threads=threads)
    vp, rp, np_, tp = timed(one_par)
    busy = min(used[0], len(w.cols))          # a column is one thread's work
    modes = [
        {"value": round(v1, 1), "cores": 1,
         "sample": f"{r1} steps over {min(r1, len(batches))} batches ({n1} valid lookups), "
                   f"{step}, fp64 C, 1 thread: {t1:.1f}s"},
        {"value": round(vp, 1), "cores": busy,
         "sample": f"{rp} steps ({np_} valid lookups), {step}, fp64 C, the {len(w.cols)} "
                   f"columns over {used[0]} OpenMP threads: {tp:.1f}s"},
    ]
    best = max(modes, key=lambda m: m["value"])
    return {"value": best["value"], "unit": "lookups/s", "cores": best["cores"], "kind": "oracle",
            "sample": best["sample"] + f"; host: {ncpu} CPUs, {model}", "modes": modes,
            "host_cpus": ncpu, "cpu_model": model}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 100; 20 for the keyed workload, whose steps each "
                         "need a batch of their own)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 10; 5 keyed)")
    ap.add_argument("--workload", default="long-seq", choices=sorted(WORKLOADS))
    ap.add_argument("--batches", type=int, default=4)
    ap.add_argument("--tile", type=int, default=0, help="positions per tile (0: 256)")
    ap.add_argument("--fwd-tile", type=int, default=0,
                    help="positions per forward tile (0: --tile if given, else chosen per batch)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stats", action="store_true", help="collect the device counters while timing")
    ap.add_argument("--atomic-backward", action="store_true",
                    help="SGD by atomic scatter (no sort) instead of the sorted segment apply")
    ap.add_argument("--inference", action="store_true", help="forward only (no backward)")
    ap.add_argument("--weights", action="store_true",
                    help="per-position weights (the extended forward, emb_forward_ex)")
    ap.add_argument("--pipeline", action="store_true",
                    help="transform the next batch on a second stream during the backward")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (known bytes) to scale HBM counters")
    ap.add_argument("--graph", action="store_true",
                    help="replay each batch's forward, dedup and apply as captured HIP graphs")
    args = ap.parse_args()
    if args.graph and (WORKLOADS[args.workload] == 5 or args.pipeline or args.weights
                       or args.atomic_backward):
        print("--graph covers the plain forward and the sorted backward of the dense workloads",
              file=sys.stderr)
        sys.exit(2)
    keyed = WORKLOADS[args.workload] == 5
    if args.steps is None:
        args.steps = 20 if keyed else 100
    if args.warmup is None:
        args.warmup = 5 if keyed else 10
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(column-wise sharding with one all-to-all is designed, not built).", file=sys.stderr)
        sys.exit(2)
    run(args)


if __name__ == "__main__":
    main()
