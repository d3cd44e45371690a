#!/usr/bin/env python3
"""Benchmark of one context-parallel rank's blockwise (zigzag ring) attention
hot path on one MI355X.

A step is one pass of the whole path over one synthetic packed batch that is
already resident in HBM:
    zigzag partition of Q, dO (this rank) and K, V (every source rank)
    for each ring step: tile scheduler + forward step, then LSE merge
    backward preprocess (delta), then for each ring step: backward step
Workload (default): the long-tail packed microbatch -- 65536 tokens, one
49152-token sequence plus 15 short ones, causal, zigzag cp=4, rank 0,
Hq=32 / Hkv=8, d=128, bf16.

FLOPs are causal-adjusted: counted from the exact number of allowed
(query, key) pairs (cpattn_count_pairs), forward 4*d*Hq per pair and
backward 10*d*Hq per pair, never from max_seqlen.

Timing: the step (ring.rank_step) is captured once as a HIP graph and each
timed step is one replay (K replays after W untimed ones, bracketed by
synchronizations).  In it the gathers of the later K/V shares and of dO, the
gradient fills and the merges run on a second stream beside the forward
steps, as the ring overlaps its transfers with compute; the results are the
same bit for bit.  The same calls issued eagerly on one stream, one host call
per kernel with events around each call, give the per-kernel figures and are
reported beside it.

Prints one JSON line.  Only N=1 is measured: the library runs one rank's share on one GPU.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E


def note(msg):
    """One progress line on stderr per finished phase (the JSON line stays alone on stdout)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default="long_tail")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true")
    p.add_argument("--no-graph", action="store_true",
                   help="skip the graph-replay figure (counter runs: only the timed steps dispatch)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a device copy of a known size (reference for HBM byte counters)")
    p.add_argument("--gemm-ceiling", action="store_true",
                   help="run only the library bf16 GEMM ceiling (torch.matmul) and print it")
    p.add_argument("--write-traffic", nargs=4, metavar=("CAL_FETCH", "CAL_WRITE", "RUN_FETCH", "RUN_WRITE"),
                   help="CPU only: turn four rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE of "
                        "--copy-calibration, then of a --steps 2 --warmup 0 --no-extras run) into "
                        "profiles/traffic.json for the current kernel sources")
    return p.parse_args()


class Timer:
    """Per-call durations with events on the launch stream."""

    def __init__(self, torch):
        self.torch = torch
        self.events = {}

    def __call__(self, name, fn):
        t = self.torch
        a = t.cuda.Event(enable_timing=True)
        b = t.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.events.setdefault(name, []).append((a, b))

    def stats(self):
        out = {}
        for k, evs in self.events.items():
            ms = [a.elapsed_time(b) for a, b in evs]
            out[k] = {"calls": len(ms), "total_ms": sum(ms), "avg_ms": sum(ms) / len(ms), "ms": ms}
        return out


# host-only sources: they launch nothing, so they cannot change a kernel's traffic
HOST_ONLY_SOURCES = ("dcp_plan.hip",)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "context_attention_varlen_amd", "csrc"))):
        if f not in HOST_ONLY_SOURCES:
            h.update(open(os.path.join(ROOT, "context_attention_varlen_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel):
    """HBM bytes per launch from the committed counter summary, only if it was
    taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except ValueError:
        return None
    ent = rec.get(kernel)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def _counter_rows(folder, counter):
    """(kernel name, KiB) per dispatch, in dispatch order, from a rocprofv3
    --pmc csv folder."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                name = r["Kernel_Name"]
                name = name[5:] if name.startswith("void ") else name
                rows.append((int(r["Dispatch_Id"]), name.rsplit("(", 1)[0], float(r["Counter_Value"])))
    rows.sort()
    return [(n, v) for _, n, v in rows]


def write_traffic(cal_fetch, cal_write, run_fetch, run_write):
    """HBM bytes per launch of the attention kernels: FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch) of one bench step, each scaled by what the same counter
    reads for the 1 GiB device copy of --copy-calibration."""
    import statistics
    scales = []
    for folder, counter in ((cal_fetch, "FETCH_SIZE"), (cal_write, "WRITE_SIZE")):
        vals = [v for n, v in _counter_rows(folder, counter) if "copyBuffer" in n]
        if not vals:
            raise SystemExit(f"no device-copy dispatch with {counter} in {folder}")
        scales.append((1 << 30) / (statistics.median(vals) * 1024))
    rec = {"_comment": "HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch), "
                       f"scaled by what each counter reads for a 1 GiB device copy (bench.py --copy-calibration): "
                       f"FETCH_SIZE x {scales[0]:.3f}, WRITE_SIZE x {scales[1]:.3f}. Workload: bench.py "
                       "--no-cpu-baseline --no-extras --no-graph --steps 2 --warmup 0 (long_tail, 4 ring steps); "
                       "the first step's launches are listed.",
           "read_scale": round(scales[0], 4), "write_scale": round(scales[1], 4)}
    fetch = _counter_rows(run_fetch, "FETCH_SIZE")
    write = _counter_rows(run_write, "WRITE_SIZE")
    src = kernel_source_hash()
    for name in sorted({n for n, _ in fetch if n.startswith("cpattn::")}):
        fb = [v * 1024 * scales[0] for n, v in fetch if n == name]
        wb = [v * 1024 * scales[1] for n, v in write if n == name]
        per_step = max(1, len(fb) // 2)
        fb, wb = fb[:per_step], wb[:per_step]
        rec[name] = {"source_hash": src, "launches": per_step,
                     "fetch_bytes_per_launch": [int(x) for x in fb],
                     "write_bytes_per_launch": [int(x) for x in wb],
                     "bytes_per_launch": int((sum(fb) + sum(wb)) / per_step)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(path)


def run_hot_path(c, torch, w, steps, warmup, graph=True):
    import numpy as np

    import workloads
    from context_attention_varlen_amd.ring import ForwardBuffers, RankPlan, StepBuffers, rank_step

    x = workloads.draw(w)
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    g = {k: torch.from_numpy(v).to(td).cuda() for k, v in x.items()}
    plan = RankPlan.make(w.cu_seqlens, w.cp, w.rank)
    tl = plan.tokens_local
    q = torch.empty((tl, w.heads_q, w.head_dim), dtype=td, device="cuda")
    do = torch.empty_like(q) if w.backward else None
    ks = [torch.empty((tl, w.heads_kv, w.head_dim), dtype=td, device="cuda") for _ in range(w.cp)]
    vs = [torch.empty_like(ks[0]) for _ in range(w.cp)]
    bufs = ForwardBuffers.make(q, tl, plan.num_seqs)
    if w.backward:
        dq = torch.zeros((tl, w.heads_q, w.head_dim), dtype=torch.float32, device="cuda")
        dk = [torch.zeros(ks[0].shape, dtype=torch.float32, device="cuda") for _ in range(w.cp)]
        dv = [torch.zeros(ks[0].shape, dtype=torch.float32, device="cuda") for _ in range(w.cp)]
        delta = torch.empty((w.heads_q, tl), dtype=torch.float32, device="cuda")
    tf = (w.tf_chunk, w.tf_num)
    steps_ = [c.make_step(w.cp, w.rank, s, *tf) for s in range(w.cp)]
    r = w.rank
    cu_g, nseq = plan.cu_global_dev, plan.num_seqs

    def step(tm):
        tm("partition", lambda: c.cpattn_partition(g["q"], q, cu_g, nseq, w.cp, r))
        if w.backward:
            tm("partition", lambda: c.cpattn_partition(g["dout"], do, cu_g, nseq, w.cp, r))
        for j in range(w.cp):
            tm("partition", lambda j=j: c.cpattn_partition(g["k"], ks[j], cu_g, nseq, w.cp, j))
            tm("partition", lambda j=j: c.cpattn_partition(g["v"], vs[j], cu_g, nseq, w.cp, j))
        bufs.reset()
        for s in range(w.cp):
            j = c.cpattn_step_source(steps_[s])
            tm("fwd_step", lambda s=s, j=j: c.cpattn_fwd_step(
                q, ks[j], vs[j], plan.cu_local_dev, plan.cu_local_dev, nseq, w.mask, steps_[s], 0.0,
                bufs.out_partial, bufs.lse_partial, bufs.workspace))
            tm("merge", lambda: c.cpattn_merge(bufs.out, bufs.lse, bufs.out_partial, bufs.lse_partial))
        if w.backward:
            for t_ in [dq] + dk + dv:
                c.cpattn_fill_f32(t_, 0.0)
            tm("bwd_preprocess", lambda: c.cpattn_bwd_preprocess(bufs.out, do, delta))
            for s in range(w.cp):
                j = c.cpattn_step_source(steps_[s])
                tm("bwd_step", lambda s=s, j=j: c.cpattn_bwd_step(
                    q, ks[j], vs[j], do, bufs.lse, delta, plan.cu_local_dev, plan.cu_local_dev, nseq, w.mask,
                    steps_[s], 0.0, dq, dk[j], dv[j], bufs.workspace))

    null = lambda name, fn: fn()  # noqa: E731
    for _ in range(warmup):
        step(null)
    torch.cuda.synchronize()
    tm = Timer(torch)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    marks[0].record()
    for i in range(steps):
        step(tm)
        marks[i + 1].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    # a schedule the device rejected (bad cu_seqlens) would time empty kernels
    ws_status = c.cpattn_workspace_status(bufs.workspace)
    if ws_status != c.OK:
        raise SystemExit(f"bench: the tile scheduler rejected the batch: {c.status_string(ws_status)}")
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    spread = {"median": round(step_ms[steps // 2] if steps % 2 else (step_ms[steps // 2 - 1] + step_ms[steps // 2]) / 2, 4),
              "min": round(step_ms[0], 4), "max": round(step_ms[-1], 4)}
    ok = bool(torch.isfinite(bufs.out).all().item()) and (not w.backward or bool(torch.isfinite(dq).all().item()))
    pairs = [c.cpattn_count_pairs(w.cu_seqlens, w.mask, st) for st in steps_]
    # the graph holds the same calls through ring.rank_step with its second
    # stream: the later K/V gathers, the dO gather, the gradient fills and
    # the merges (double-buffered partials) run beside the forward steps, as
    # the ring overlaps its transfers with compute; results are identical
    sb = StepBuffers(q, do, ks, vs, bufs, (torch.empty_like(bufs.out_partial), torch.empty_like(bufs.lse_partial)),
                     dq if w.backward else None, dk if w.backward else None, dv if w.backward else None,
                     delta if w.backward else None)
    side = torch.cuda.Stream()
    step_graph = lambda _tm: rank_step(g["q"], g["k"], g["v"], g["dout"] if w.backward else None,  # noqa: E731
                                       plan, w.mask, sb, side=side)
    gr = graph_steps(torch, step_graph, null, steps, warmup) if graph else None
    if gr is not None and c.cpattn_workspace_status(bufs.workspace) != c.OK:
        raise SystemExit("bench: the tile scheduler rejected the batch during the graph replays")
    return wall_ms, tm.stats(), pairs, ok, x, gr, spread


def graph_steps(torch, step, null, steps, warmup, extra=True):
    """A step captured once as a HIP graph (every call only enqueues kernels,
    on the capture stream or on a stream forked from it and joined back, so
    it captures as is): `warmup` untimed replays, then exactly `steps` timed
    replays bracketed by synchronizations (the step rate the headline
    reports), then (extra) replays up to 100 in all so that a sampler of GPU
    activity sees the step running.  None if this torch build cannot capture."""
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(null)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(null)
    except RuntimeError as e:
        print(f"graph capture unavailable: {e}", file=sys.stderr, flush=True)
        return None
    for _ in range(max(warmup, 1)):
        graph.replay()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    marks[0].record()
    for i in range(steps):
        graph.replay()
        marks[i + 1].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    spread = {"median": round(step_ms[steps // 2] if steps % 2 else (step_ms[steps // 2 - 1] + step_ms[steps // 2]) / 2, 4),
              "min": round(step_ms[0], 4), "max": round(step_ms[-1], 4)}
    # more replays, at least 100 in all (about 2 s of the long-tail step)
    reps = max(100 - steps, 0) if extra else 0
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea.record()
    for _ in range(reps):
        graph.replay()
    eb.record()
    torch.cuda.synchronize()
    return {"wall_ms": wall_ms, "spread": spread, "extra_replays": reps,
            "extra_ms_per_step": ea.elapsed_time(eb) / reps if reps else None}


def cpu_baseline(w, x, rows=512):
    """The oracle, as it stands, on a bounded sample of the same workload:
    `rows` seeded query rows of the rank (all q-heads), forward and backward
    against every key they may attend."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                   default=1)
    except Exception:  # pragma: no cover
        blas = 1
    cu = w.cu_seqlens
    _, l2g, qpos, qseq = oracle.local_rows(cu, w.cp, w.rank)
    rng = np.random.default_rng(1005)
    sel = np.sort(rng.choice(len(l2g), size=min(rows, len(l2g)), replace=False))
    T = int(cu[-1])
    seq = np.repeat(np.arange(len(cu) - 1), np.diff(cu))
    pos = np.arange(T) - cu[seq]
    keep = np.isin(seq, np.unique(qseq[sel]))
    t0 = time.perf_counter()
    o, lse = oracle.attention(x["q"][l2g[sel]], x["k"][keep], x["v"][keep], qseq[sel], qpos[sel], seq[keep],
                              pos[keep], w.mask, tf_chunk=w.tf_chunk, tf_num=w.tf_num)
    if w.backward:
        delta = oracle.bwd_delta(o, x["dout"][l2g[sel]])
        oracle.attention_backward(x["q"][l2g[sel]], x["k"][keep], x["v"][keep], x["dout"][l2g[sel]], lse, delta,
                                  qseq[sel], qpos[sel], seq[keep], pos[keep], w.mask,
                                  tf_chunk=w.tf_chunk, tf_num=w.tf_num)
    dt = time.perf_counter() - t0
    pairs = int(sum(oracle.allowed(w.mask, qpos[i], pos[(seq == qseq[i])], w.tf_chunk, w.tf_num).sum()
                    for i in sel))
    per_pair = (4 + (10 if w.backward else 0)) * w.head_dim * w.heads_q
    return {"value": round(pairs * per_pair / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{len(sel)} seeded query rows of rank {w.rank} ({w.heads_q} q-heads), "
                      f"{'forward+backward' if w.backward else 'forward'} against all {pairs} allowed "
                      f"(query, key) pairs per head, fp64 NumPy"}


def _static_cp_plan(lens, gpus, max_cp, mem):
    """Packing-only baseline with a static cp: samples in batch order are
    packed into microbatches of at most max_cp*mem tokens, every microbatch
    split max_cp ways, and dealt round-robin to the gpus/max_cp groups."""
    mbs, cur, tok = [], [], 0
    for L in lens:
        if cur and tok + L > max_cp * mem:
            mbs.append(cur)
            cur, tok = [], 0
        cur.append(L)
        tok += L
    if cur:
        mbs.append(cur)
    groups = gpus // max_cp
    return [(mb, max_cp, j % groups) for j, mb in enumerate(mbs)]


def _time_rank_share(c, torch, pool, lens, cp, reps=2):
    """ms of rank 0's attention for one microbatch (every sequence
    zigzag-split over cp ranks): cp forward steps with merges, the backward
    preprocess and cp backward steps.  Inputs are random; only time counts."""
    import numpy as np
    from context_attention_varlen_amd.ring import ForwardBuffers
    loc = [L // cp for L in lens]
    T = sum(loc)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(loc)]).astype(np.int32), device="cuda")
    q, k, v, do = (pool[n][:T] for n in ("q", "k", "v", "do"))
    # delta is [Hq, T] contiguous: a view of the front of a flat buffer
    dq, dk, dv = pool["dq"][:T], pool["dk"][:T], pool["dv"][:T]
    delta = pool["delta"][:pool["q"].shape[1] * T].view(pool["q"].shape[1], T)
    bufs = ForwardBuffers.make(q, T, len(lens))
    steps = [c.make_step(cp, 0, s) for s in range(cp)]

    def run():
        bufs.reset()
        for s in range(cp):
            c.cpattn_fwd_step(q, k, v, cu, cu, len(lens), c.CAUSAL, steps[s], 0.0, bufs.out_partial,
                              bufs.lse_partial, bufs.workspace)
            c.cpattn_merge(bufs.out, bufs.lse, bufs.out_partial, bufs.lse_partial)
        c.cpattn_bwd_preprocess(bufs.out, do, delta)
        for s in range(cp):
            c.cpattn_bwd_step(q, k, v, do, bufs.lse, delta, cu, cu, len(lens), c.CAUSAL, steps[s], 0.0,
                              dq, dk, dv, bufs.workspace)
    run()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def dynamic_cp_extra(c, torch, gen):
    """Dynamic-CP plan of a long-tail global batch (host planner), scored by
    the planner's model and by timing every microbatch's rank share on the
    attention path, against a packing-only plan with a static cp."""
    import time

    import numpy as np

    import workloads
    lens = workloads.global_batch_lengths()
    G, MAXCP, MEM, Hq, Hkv, d = 16, 8, 32768, 32, 8, 128
    cfg = (G, MAXCP, 1, 1, MEM, 1, 0, 1, 8, -1)
    reps = 20
    t0 = time.perf_counter()
    for _ in range(reps):
        plan = c.cpattn_dcp_plan_batch(lens, *cfg)
    plan_ms = (time.perf_counter() - t0) / reps * 1e3
    sb = plan["sample_bucket"]
    dyn = [([lens[i] for i in np.flatnonzero(sb == j)], int(plan["cp"][j]), int(plan["rank"][j]))
           for j in range(plan["num_buckets"])]
    static = _static_cp_plan(lens, G, MAXCP, MEM)
    pool = {n: torch.randn((MEM, Hq if n in ("q", "do") else Hkv, d), device="cuda", generator=gen).bfloat16()
            for n in ("q", "k", "v", "do")}
    pool.update({"dq": torch.zeros((MEM, Hq, d), device="cuda"), "dk": torch.zeros((MEM, Hkv, d), device="cuda"),
                 "dv": torch.zeros((MEM, Hkv, d), device="cuda"), "delta": torch.zeros(Hq * MEM, device="cuda")})

    samples = []     # (sum S^2 / cp, sum S / cp, ms) per timed microbatch share

    def score(mbs, group_of):
        rank_ms, rank_model = np.zeros(G), np.zeros(G)
        meas, model = [], []
        for lens_b, cp, first in mbs:
            if not lens_b:
                continue
            ms = _time_rank_share(c, torch, pool, lens_b, cp)
            w = sum(L * L for L in lens_b) / cp
            for r in group_of(first, cp):
                rank_ms[r] += ms
                rank_model[r] += w
            meas.append(ms)
            model.append(w)
            samples.append((w, sum(lens_b) / cp, ms))
        fit = np.polyfit(model, meas, 1)
        r2 = 1 - np.sum((np.polyval(fit, model) - meas) ** 2) / np.sum((np.asarray(meas) - np.mean(meas)) ** 2)
        return rank_ms, rank_model, r2

    d_ms, d_model, d_r2 = score(dyn, lambda first, cp: range(first, first + cp))
    s_ms, s_model, s_r2 = score(static, lambda g, cp: range(g * cp, (g + 1) * cp))
    # calibration of w(S) = a S^2 + b S for this library on this shape:
    # least squares of the measured share times on (sum S^2 / cp, sum S / cp)
    A = np.asarray([[x[0], x[1]] for x in samples])
    coef, *_ = np.linalg.lstsq(A, np.asarray([x[2] for x in samples]), rcond=None)
    del pool
    torch.cuda.empty_cache()
    return {"samples": len(lens), "tokens": int(sum(lens)), "longest": int(max(lens)), "gpus": G, "max_cp": MAXCP,
            "mem_tokens": MEM, "heads": [Hq, Hkv], "head_dim": d, "workload_model": "S^2",
            "planner_ms": round(plan_ms, 3), "m": plan["m"], "knee": plan["knee"],
            "microbatches": plan["num_buckets"],
            "cp_sizes": {str(k): int(v) for k, v in zip(*np.unique(plan["cp"], return_counts=True))},
            "model_step": float(d_model.max()), "model_static_step": float(s_model.max()),
            "model_speedup": round(float(s_model.max() / d_model.max()), 3),
            "measured_step_ms": round(float(d_ms.max()), 2), "measured_mean_rank_ms": round(float(d_ms.mean()), 2),
            "measured_static_step_ms": round(float(s_ms.max()), 2),
            "measured_static_mean_rank_ms": round(float(s_ms.mean()), 2),
            "measured_speedup": round(float(s_ms.max() / d_ms.max()), 3),
            "model_fit_r2": [round(float(d_r2), 4), round(float(s_r2), 4)],
            "calibrated_ns_per_S2": round(float(coef[0]) * 1e6, 6), "calibrated_ns_per_token": round(float(coef[1]) * 1e6, 3)}


def long_video_step(c, torch, steps=5, warmup=1):
    """The long-video rank's whole step as its own measurement: zigzag
    partition of Q (rank 0) and of K/V for all 8 source ranks, then 8 x
    (tile scheduler + forward step + LSE merge), 262144 tokens at cp = 8,
    28/4 heads, d = 128, bf16.  Inputs are device-random (only time counts;
    the parity tests check this shape against the oracle).  Per-call times
    are HIP events on the launch stream; the forward kernel and the merge
    get their roofline objects (merge: algorithmic bytes of the rows that are
    live in each step)."""
    import workloads
    from context_attention_varlen_amd.ring import ForwardBuffers, RankPlan, StepBuffers, rank_step
    w = workloads.WORKLOADS["long_video"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    plan = RankPlan.make(w.cu_seqlens, w.cp, w.rank)
    mk = lambda h: (torch.randn((w.tokens, h, w.head_dim), device="cuda", generator=gen)  # noqa: E731
                    * w.value_scale).bfloat16()
    qg, kg, vg = mk(w.heads_q), mk(w.heads_kv), mk(w.heads_kv)
    tl = plan.tokens_local
    q = torch.empty((tl, w.heads_q, w.head_dim), dtype=torch.bfloat16, device="cuda")
    ks = [torch.empty((tl, w.heads_kv, w.head_dim), dtype=torch.bfloat16, device="cuda") for _ in range(w.cp)]
    vs = [torch.empty_like(ks[0]) for _ in range(w.cp)]
    bufs = ForwardBuffers.make(q, tl, plan.num_seqs)
    sts = [c.make_step(w.cp, w.rank, s) for s in range(w.cp)]
    cu_g, cu_l, nseq = plan.cu_global_dev, plan.cu_local_dev, plan.num_seqs

    def step(tm):
        tm("partition", lambda: c.cpattn_partition(qg, q, cu_g, nseq, w.cp, w.rank))
        for j in range(w.cp):
            tm("partition", lambda j=j: c.cpattn_partition(kg, ks[j], cu_g, nseq, w.cp, j))
            tm("partition", lambda j=j: c.cpattn_partition(vg, vs[j], cu_g, nseq, w.cp, j))
        bufs.reset()
        for s in range(w.cp):
            j = c.cpattn_step_source(sts[s])
            tm("fwd_step", lambda s=s, j=j: c.cpattn_fwd_step(q, ks[j], vs[j], cu_l, cu_l, nseq, w.mask, sts[s], 0.0,
                                                             bufs.out_partial, bufs.lse_partial, bufs.workspace))
            tm("merge", lambda: c.cpattn_merge(bufs.out, bufs.lse, bufs.out_partial, bufs.lse_partial))

    null = lambda name, fn: fn()  # noqa: E731
    for _ in range(warmup):
        step(null)
    torch.cuda.synchronize()
    tm = Timer(torch)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        step(tm)
    b.record()
    torch.cuda.synchronize()
    ws_status = c.cpattn_workspace_status(bufs.workspace)
    if ws_status != c.OK:
        raise SystemExit(f"bench: the tile scheduler rejected the long-video batch: {c.status_string(ws_status)}")
    ms = a.elapsed_time(b) / steps
    st = tm.stats()
    # the same step as a graph through ring.rank_step, its K/V gathers after
    # the first source's and its merges on a second stream
    sb = StepBuffers(q, None, ks, vs, bufs, (torch.empty_like(bufs.out_partial), torch.empty_like(bufs.lse_partial)),
                     None, None, None, None)
    side = torch.cuda.Stream()
    gr = graph_steps(torch, lambda _tm: rank_step(qg, kg, vg, None, plan, w.mask, sb, side=side), null, steps,
                     warmup, extra=False)
    pairs = [c.cpattn_count_pairs(w.cu_seqlens, w.mask, x) for x in sts]
    flops = 4 * w.head_dim * w.heads_q * sum(pairs)
    fwd = st["fwd_step"]
    f_avg = fwd["avg_ms"]
    f_ach = flops / w.cp / (f_avg * 1e-3) / 1e12
    # merge bytes: 8d + 2d + 12 per live (token, head) row, 4 per skipped row;
    # on rank 0 every row is live at step 0 and only the second chunk after
    live0 = tl * w.heads_q
    live_s = (tl // 2) * w.heads_q
    m_bytes = [live0 * (10 * w.head_dim + 12)] + [live_s * (10 * w.head_dim + 12) + (tl * w.heads_q - live_s) * 4
                                                   for _ in range(w.cp - 1)]
    mg = st["merge"]
    m_ach = sum(m_bytes) / (mg["total_ms"] / steps * 1e-3) / 1e9
    del qg, kg, vg, q, ks, vs, bufs, sb
    torch.cuda.empty_cache()
    gms = gr["wall_ms"] if gr is not None else None
    return {
        "workload": "long_video: 262144 tokens, causal zigzag cp=8 rank 0, Hq=28/Hkv=4, d=128, bf16; "
                    "partition + 8 x (scheduler + forward step + merge)",
        "steps": steps, "ms_per_step": round(ms, 4), "pairs_per_head": sum(pairs), "flops_per_step": flops,
        "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
        "pct_of_bf16_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        # the step as one graph replay, gathers and merges beside the forward steps
        "graph_overlapped": None if gms is None else {
            "ms_per_step": round(gms, 4), "tflops": round(flops / (gms * 1e-3) / 1e12, 1),
            "pct_of_bf16_peak": round(100 * flops / (gms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)},
        "per_call_ms_per_step": {k: round(v["total_ms"] / steps, 4) for k, v in st.items()},
        "roofline": {"bound": "mfma", "kernel": "cpattn::fwd_bf16_kernel<128, 4>", "achieved": round(f_ach, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(f_ach / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "avg_launch_ms": round(f_avg, 4),
                     "algorithmic_flops_per_launch": int(flops / w.cp)},
        "merge_roofline": {"bound": "hbm", "kernel": "cpattn::merge_kernel<128, true>", "achieved": round(m_ach, 1),
                           "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(m_ach / PEAK_HBM_GBPS, 4),
                           "traffic": None, "avg_launch_ms": round(mg["avg_ms"], 4),
                           "algorithmic_bytes_per_step": int(sum(m_bytes))},
    }


def extras(c, torch):
    """Forward and merge figures of the other workloads (not part of `value`)."""
    import workloads
    from context_attention_varlen_amd.ring import ForwardBuffers, RankPlan, partition
    out = {}
    gen = torch.Generator(device="cuda")
    for name in ("packed_varlen", "long_video", "tf_dit", "tf_dit_split"):
        w = workloads.WORKLOADS[name]
        gen.manual_seed(0)
        plan = RankPlan.make(w.cu_seqlens, w.cp, w.rank, tf=(w.tf_chunk, w.tf_num) if w.tf_chunk else None)
        mk = lambda h: (torch.randn((w.tokens, h, w.head_dim), device="cuda", generator=gen)  # noqa: E731
                        * w.value_scale).bfloat16()
        qg, kg, vg = mk(w.heads_q), mk(w.heads_kv), mk(w.heads_kv)
        q = partition(qg, plan)
        ks = [partition(kg, plan, j) for j in range(w.cp)]
        vs = [partition(vg, plan, j) for j in range(w.cp)]
        del qg, kg, vg
        bufs = ForwardBuffers.make(q, ks[0].shape[0], plan.num_seqs)
        tf = (w.tf_chunk, w.tf_num)
        sts = [c.make_step(w.cp, w.rank, s, *tf) for s in range(w.cp)]
        pairs = sum(c.cpattn_count_pairs(w.cu_seqlens, w.mask, st) for st in sts)
        tm = Timer(torch)
        for it in range(4):
            bufs.reset()
            for s in range(w.cp):
                j = c.cpattn_step_source(sts[s])
                f = lambda s=s, j=j: c.cpattn_fwd_step(q, ks[j], vs[j], plan.cu_local_dev, plan.cu_local_dev,  # noqa
                                                       plan.num_seqs, w.mask, sts[s], 0.0, bufs.out_partial,
                                                       bufs.lse_partial, bufs.workspace)
                (tm if it else (lambda n, fn: fn()))("fwd", f)
                c.cpattn_merge(bufs.out, bufs.lse, bufs.out_partial, bufs.lse_partial)
        torch.cuda.synchronize()
        st = tm.stats()["fwd"]
        ms = st["total_ms"] / 3
        tfl = 4 * w.head_dim * w.heads_q * pairs / (ms * 1e-3) / 1e12
        per_step = [sum(st["ms"][s::w.cp]) / 3 for s in range(w.cp)]
        out[name] = {"fwd_ms": round(ms, 3), "fwd_tflops": round(tfl, 1),
                     "pct_peak": round(100 * tfl / PEAK_BF16_TFLOPS, 1), "pairs_per_head": pairs,
                     "fwd_ms_per_ring_step": [round(x, 3) for x in per_step],
                     "fwd_tflops_per_ring_step": [
                         round(4 * w.head_dim * w.heads_q * c.cpattn_count_pairs(w.cu_seqlens, w.mask, sts[s])
                               / (per_step[s] * 1e-3) / 1e12, 1) for s in range(w.cp)]}
        note(f"extra {name} forward done")
        if w.backward:
            do = partition(mk(w.heads_q), plan)
            dq = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
            dk = torch.zeros(ks[0].shape, dtype=torch.float32, device="cuda")
            dv = torch.zeros_like(dk)
            delta = torch.empty((w.heads_q, q.shape[0]), dtype=torch.float32, device="cuda")
            tb = Timer(torch)
            for it in range(4):
                c.cpattn_bwd_preprocess(bufs.out, do, delta)
                for s in range(w.cp):
                    j = c.cpattn_step_source(sts[s])
                    f = lambda s=s, j=j: c.cpattn_bwd_step(q, ks[j], vs[j], do, bufs.lse, delta,  # noqa: E731
                                                           plan.cu_local_dev, plan.cu_local_dev, plan.num_seqs,
                                                           w.mask, sts[s], 0.0, dq, dk, dv, bufs.workspace)
                    (tb if it else (lambda n, fn: fn()))("bwd", f)
            torch.cuda.synchronize()
            bms = tb.stats()["bwd"]["total_ms"] / 3
            btf = 10 * w.head_dim * w.heads_q * pairs / (bms * 1e-3) / 1e12
            out[name].update({"bwd_ms": round(bms, 3), "bwd_tflops": round(btf, 1),
                              "bwd_pct_peak": round(100 * btf / PEAK_BF16_TFLOPS, 1)})
            del do, dq, dk, dv, delta
        if name == "long_video":
            # merge with every partial row live (finite lse_partial)
            bufs.lse_partial.normal_()
            tm2 = Timer(torch)
            for it in range(6):
                (tm2 if it else (lambda n, fn: fn()))("merge", lambda: c.cpattn_merge(
                    bufs.out, bufs.lse, bufs.out_partial, bufs.lse_partial))
            torch.cuda.synchronize()
            mst = tm2.stats()["merge"]
            rows = q.shape[0] * w.heads_q
            nbytes = rows * (8 * w.head_dim + 2 * w.head_dim + 12)
            out["merge_long_video_all_live"] = {
                "avg_ms": round(mst["avg_ms"], 4), "bytes": nbytes,
                "gbps": round(nbytes / (mst["avg_ms"] * 1e-3) / 1e9, 1),
                "pct_peak_hbm": round(100 * nbytes / (mst["avg_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 1)}
        del q, ks, vs, bufs
        torch.cuda.empty_cache()
    # Ulysses sequence->head exchange on one device: 4-way group over the
    # long-video sequence (262144 tokens, 28 q-heads -> 7 per member), the
    # shards in HBM, one member's gather of its head group
    n, T, H, d = 4, 262144, 28, 128
    shards = [torch.randn((T // n, H, d), device="cuda", generator=gen).bfloat16() for _ in range(n)]
    dst = torch.empty((T, H // n, d), dtype=torch.bfloat16, device="cuda")
    tm = Timer(torch)
    for it in range(6):
        (tm if it else (lambda nm, fn: fn()))("gather", lambda: c.cpattn_seq_to_head(shards, 1, dst))
    torch.cuda.synchronize()
    gms = tm.stats()["gather"]["avg_ms"]
    nbytes = 2 * T * (H // n) * d * 2
    out["ulysses_seq_to_head_long_video"] = {
        "avg_ms": round(gms, 4), "bytes": nbytes, "gbps": round(nbytes / (gms * 1e-3) / 1e9, 1),
        "pct_peak_hbm": round(100 * nbytes / (gms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 1)}
    del shards, dst
    # height/width split of a video latent (31 frames x 30 x 52 tokens,
    # 24 heads): one rank's gather at cp = 8 (2 x 4 grid)
    frames, Hh, Ww, cp = 31, 30, 52, 8
    split = c.cpattn_split_hw(Hh, Ww, cp)
    Tv = frames * Hh * Ww
    src = torch.randn((Tv, 24, d), device="cuda", generator=gen).bfloat16()
    loc = torch.empty((Tv // cp, 24, d), dtype=torch.bfloat16, device="cuda")
    cu_dev = torch.tensor([0, Tv], dtype=torch.int32, device="cuda")
    tm = Timer(torch)
    for it in range(6):
        (tm if it else (lambda nm, fn: fn()))("hw", lambda: c.cpattn_partition_hw(src, loc, cu_dev, 1, frames, Hh, Ww,
                                                                                   split, 3))
    torch.cuda.synchronize()
    hms = tm.stats()["hw"]["avg_ms"]
    nbytes = 2 * (Tv // cp) * 24 * d * 2
    out["hw_split_partition_video_latent"] = {
        "split": list(split), "avg_ms": round(hms, 4), "bytes": nbytes, "gbps": round(nbytes / (hms * 1e-3) / 1e9, 1),
        "pct_peak_hbm": round(100 * nbytes / (hms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 1)}
    del src, loc
    torch.cuda.empty_cache()
    note("exchange extras done")
    out["dynamic_cp_global_batch"] = dynamic_cp_extra(c, torch, gen)
    note("dynamic-cp extra done")
    return out


def gemm_ceiling(torch):
    """The vendor library's dense bf16 GEMM rate on this GPU (torch.matmul,
    which dispatches to hipBLASLt), timed with events: the practical ceiling
    a matrix-core kernel meets under the chip's power limit, beside the
    nominal 2.5 PFLOP/s."""
    out = {"kernel": "torch.matmul bf16 (hipBLASLt)"}
    for n, reps in ((8192, 20), (16384, 6)):
        a = torch.randn((n, n), device="cuda", dtype=torch.bfloat16)
        b = torch.randn((n, n), device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            a @ b
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            a @ b
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[f"gemm_{n}_cubed"] = {"ms": round(ms, 4), "tflops": round(2 * n ** 3 / (ms * 1e-3) / 1e12, 1)}
        del a, b
    torch.cuda.empty_cache()
    out["tflops"] = max(v["tflops"] for k, v in out.items() if k.startswith("gemm_"))
    out["pct_of_bf16_peak"] = round(100 * out["tflops"] / PEAK_BF16_TFLOPS, 1)
    return out


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library runs one rank's share "
              "on one MI355X and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        # 1 GiB read + 1 GiB written per copy: the reference that scales the
        # FETCH_SIZE / WRITE_SIZE counters of the attention kernels
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read_per_copy": 4 * n, "bytes_written_per_copy": 4 * n,
                                               "copies": 4}}), flush=True)
        return
    if args.gemm_ceiling:
        print(json.dumps({"gemm_ceiling": gemm_ceiling(torch)}), flush=True)
        return
    import context_attention_varlen_amd as c
    import workloads

    w = workloads.WORKLOADS[args.workload]
    eager_ms, st, pairs, finite, x, gr, eager_spread = run_hot_path(c, torch, w, args.steps, args.warmup,
                                                                    graph=not args.no_graph)
    # the headline times the step as one captured HIP graph per step; the
    # eager loop (one host call per kernel, per-call events) gives the
    # per-kernel figures and is reported beside it
    wall_ms, spread = (gr["wall_ms"], gr["spread"]) if gr is not None else (eager_ms, eager_spread)
    note(f"timed region done ({args.steps} steps)")
    P = sum(pairs)
    fwd_flops = 4 * w.head_dim * w.heads_q * P
    bwd_flops = 10 * w.head_dim * w.heads_q * P if w.backward else 0
    tflops = (fwd_flops + bwd_flops) / (wall_ms * 1e-3) / 1e12

    # dominant kernel and its roofline
    kern = {"fwd_step": ("cpattn::fwd_bf16_kernel<128, 4>", fwd_flops / w.cp),
            "bwd_step": ("cpattn::(anonymous namespace)::bwd_bf16_kernel<128>", bwd_flops / w.cp)}
    dom = max((k for k in kern if k in st), key=lambda k: st[k]["total_ms"])
    kname, flops_per_launch = kern[dom]
    avg_ms = st[dom]["avg_ms"]
    achieved = flops_per_launch / (avg_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": kname, "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_for(kname), "avg_launch_ms": round(avg_ms, 4),
                "algorithmic_flops_per_launch": int(flops_per_launch)}

    # the other attention kernel of the step, on the same footing (not the dominant one)
    other = [k for k in kern if k in st and k != dom]
    roofline_other = None
    if other:
        k2 = other[0]
        n2, f2 = kern[k2]
        a2 = f2 / (st[k2]["avg_ms"] * 1e-3) / 1e12
        roofline_other = {"bound": "mfma", "kernel": n2, "achieved": round(a2, 1), "peak": PEAK_BF16_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(a2 / PEAK_BF16_TFLOPS, 4), "traffic": traffic_for(n2),
                          "avg_launch_ms": round(st[k2]["avg_ms"], 4), "algorithmic_flops_per_launch": int(f2)}

    per_call = {k: {"calls_per_step": v["calls"] // args.steps, "avg_ms": round(v["avg_ms"], 4),
                    "ms_per_step": round(v["total_ms"] / args.steps, 4)} for k, v in st.items()}
    # ring step s of every timed step (step 0 holds the rank's own K/V share)
    for k in ("fwd_step", "merge", "bwd_step"):
        if k in st and per_call[k]["calls_per_step"] == w.cp:
            ms = st[k]["ms"]
            per_call[k]["per_ring_step_ms"] = [round(sum(ms[s::w.cp]) / len(ms[s::w.cp]), 4) for s in range(w.cp)]
    fwd_ms = st["fwd_step"]["total_ms"] / args.steps
    per_call["fwd_step"]["tflops"] = round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 1)
    if "bwd_step" in st:
        bwd_ms = st["bwd_step"]["total_ms"] / args.steps
        per_call["bwd_step"]["tflops"] = round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 1)

    rec = {
        "metric": "blockwise attn TFLOP/s (causal-adjusted) + % of bf16 MFMA peak, 1 MI355X",
        "value": round(tflops, 2), "unit": "TFLOP/s", "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 4),
        "step_ms_events": spread,
        "timing": ("each timed step is one replay of the whole step captured as a HIP graph "
                   "(warmup replays untimed); in it the later K/V gathers, the dO gather, the gradient fills "
                   "and the merges run on a second stream beside the forward steps") if gr is not None else
                  "each timed step is the eager sequence of library calls",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16; long-tail lengths drawn as in workloads/)",
        "config": {"workload": f"{w.name}: {w.tokens} tokens ({len(w.seqlens)} sequences, longest "
                               f"{max(w.seqlens)}), causal zigzag cp={w.cp} rank {w.rank}, "
                               f"Hq={w.heads_q}/Hkv={w.heads_kv}, d={w.head_dim}, "
                               f"{'forward+backward' if w.backward else 'forward'}",
                   "global_batch": 1, "seq_len": w.tokens, "tokens_local": w.tokens // w.cp,
                   "parallelism": f"cp{w.cp} (one rank's share on one GPU)"},
        "pairs_per_head": P, "flops_per_step": fwd_flops + bwd_flops, "outputs_finite": finite,
        "per_call": per_call, "roofline": roofline, "roofline_other_attention_kernel": roofline_other,
        # not `value`: the same steps issued eagerly, one host call per kernel
        # with events around each call (the per_call and roofline figures)
        "eager": {"ms_per_step": round(eager_ms, 4), "step_ms_events": eager_spread,
                  "tflops": round((fwd_flops + bwd_flops) / (eager_ms * 1e-3) / 1e12, 2)},
        # the graph replayed further (100 replays in all, for GPU-activity sampling)
        "graph_replay": None if gr is None or not gr["extra_replays"] else {
            "replays": gr["extra_replays"], "ms_per_step": round(gr["extra_ms_per_step"], 4),
            "tflops": round((fwd_flops + bwd_flops) / (gr["extra_ms_per_step"] * 1e-3) / 1e12, 2)},
    }
    # the device's own figures: CU count and peak shader clock, and the dense
    # bf16 matrix-core peak they give (4096 FLOP per clock per CU on gfx950)
    cus, khz = c.cpattn_device_info(torch.cuda.current_device())
    rec["device"] = {"name": torch.cuda.get_device_properties(0).name,
                     "arch": torch.cuda.get_device_properties(0).gcnArchName, "cus": cus,
                     "peak_clock_mhz": khz / 1000,
                     "bf16_peak_at_peak_clock_tflops": round(cus * 4096 * khz * 1e3 / 1e12, 1)}
    # GPU phases first, the host-only oracle baseline last
    if not args.no_extras:
        rec["long_video_step"] = long_video_step(c, torch)
        note("long-video step done")
        rec["extras"] = extras(c, torch)
        # the library GEMM on the same device, and the attention kernels' matrix
        # work against it (the backward executes 7 products per pair, 5 credited)
        ceil = gemm_ceiling(torch)
        ceil["fwd_over_gemm"] = round(per_call["fwd_step"]["tflops"] / ceil["tflops"], 3)
        if "bwd_step" in st:
            ceil["bwd_executed_over_gemm"] = round(per_call["bwd_step"]["tflops"] * 7 / 5 / ceil["tflops"], 3)
        rec["practical_ceiling"] = ceil
        note("gemm ceiling done")
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, x)
        note("cpu baseline done")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
