#!/usr/bin/env python3
"""Benchmark of the sparse latent attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input: the new
KV rows rounded through fp8 and written into the window ring, the window slot
lists built, compressed positions appended (when the workload has them) and
the sparse attention itself -- all through the C ABI on one stream.  Decode
workloads run the step as one launch (sa_sparse_attn_decode_step, the lists
built inside the attention kernel); prefill workloads as two (the chunk's fp8
round trip, then sa_sparse_attn_prefill_step with the lists built inside the
attention kernel); ``--unfused`` times the separate calls.
``--kv8`` holds the decode cache fp8-resident (e4m3fn codes + E8M0 block
scales) and runs the one-launch step on it: the same results, bit for bit,
from about half the gathered bytes.  ``--rope`` fuses the output's inverse
rotary embedding into the epilogue.  ``--select`` measures the indexer's
selection tail on its own workload instead (one JSON line of its own).

Default workload: the long prefill with compressed positions -- 8192 queries,
64 heads, head dim 512, each query's list a causal 128-wide window plus up to
2048 compressed positions (1.24 TFLOP of attention per step, MFMA bound): the
largest configuration, and the one whose whole work a step covers on one GPU.
``--workload N`` measures the other configurations the same way: 2 = decode over
the window ring (batch 64 at position 5000, HBM bound), 3 = window-only prefill
(4096 queries), 4 = decode with compressed positions (batch 128, 128 heads);
1 = the tiny ring run is correctness-only and not benchmarked.

Inputs are resident in HBM before the timed region.  Small workloads rotate
through enough independently generated input sets (more than twice the 256 MiB
MALL) that every step reads its inputs from HBM, not from cache.

The steps are captured as a chain in a HIP graph -- at least 32 steps, cycling
through the input sets -- and replayed, so the host's launch cost stays out of
the measurement (``--no-graphs`` launches eagerly).  The attention kernel's
duration is taken with HIP events on the launch stream around a graph of the
same number of back-to-back attention launches alone.  ``--sets 1`` keeps one
input set resident instead, to measure the same step with its inputs warm in
the caches.

Prints one JSON line: throughput (query-heads/s), the roofline position of the
attention kernel, and the CPU oracle timed on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
MALL_BYTES = 256 << 20
CHAIN_MIN = 32                 # steps per captured graph, at least


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5],
                    help="1 (the tiny ring run) only with --cpu-only")
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets (0 = automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    ap.add_argument("--cpu-only", action="store_true",
                    help="time only the CPU oracle on the workload (threads from OMP_NUM_THREADS, else all "
                         "cores) and print its JSON object; no GPU is used")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration under rocprofv3)")
    ap.add_argument("--unfused", action="store_true",
                    help="run the step as separate calls (ring update, lists, attention) instead of "
                         "building the lists inside the attention kernel")
    ap.add_argument("--kv8", action="store_true",
                    help="decode: the cache held fp8-resident (e4m3fn codes + E8M0 block scales) and read "
                         "and written in that form by the one-launch step (bitwise the same results)")
    ap.add_argument("--rope", action="store_true",
                    help="fuse the output's inverse rotary embedding (last 64 values) into the attention epilogue")
    ap.add_argument("--select", action="store_true",
                    help="measure the indexer selection tail (sa_indexer_topk) on its workload instead")
    ap.add_argument("--select-start-pos", type=int, default=None,
                    help="with --select: decode position instead of the workload's (rows of more than "
                         "16384 positions take the streaming form)")
    ap.add_argument("--no-graphs", dest="graphs", action="store_false",
                    help="launch every step eagerly from Python instead of replaying HIP graphs")
    return ap.parse_args()


def algorithmic_work(w, idx_sets, fused=False, kv8=False):
    """Algorithmic bytes and flops of one attention launch (valid entries only).
    Decode: every valid gathered row is HBM traffic (rows differ per sequence).
    Prefill: the unique KV rows referenced are read once; repeats come from cache.
    Fused prefill: the list is built in the kernel, only the compressed entries
    are read.  Fused decode step: the list is written instead of read (compressed entries
    still read), and the new row is read once and written once into the ring
    (it enters the attention from registers instead of the ring).  kv8: a row is
    d code bytes plus its 16-byte scale record; the new row is read as bf16 and
    written as codes + record."""
    import torch
    idx = idx_sets[0]
    valid = int((idx >= 0).sum().item())
    flops = 4.0 * w.h * w.d * valid
    q_bytes = w.b * w.s * w.h * w.d * 2
    o_bytes = q_bytes
    idx_bytes = idx.numel() * 4
    sink_bytes = w.h * 4
    row_bytes = w.d + 16 if kv8 else 2 * w.d
    if w.start_pos > 0:
        kv_bytes = valid * row_bytes
    else:
        uniq = 0
        for bi in range(w.b):
            u = idx[bi].flatten()
            uniq += int(torch.unique(u[u >= 0]).numel())
        kv_bytes = uniq * w.d * 2
    if fused and w.start_pos == 0:
        idx_bytes = w.b * w.s * w.n_comp * 4   # the compressed positions; the list stays in the kernel
    elif fused:
        idx_bytes += w.b * w.s * w.n_comp * 4
        kv_bytes += w.b * w.d * 2     # new row: read raw + written, minus the gathered copy the count holds
    total = q_bytes + o_bytes + idx_bytes + sink_bytes + kv_bytes
    return dict(bytes=total, flops=flops, valid=valid, kv_bytes=kv_bytes)


def source_sha():
    """Hash of every kernel source: a counter summary taken on other sources is stale."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "sparse_latent_attention_02_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_tag(wid, fused, kv8, rope_dim=0):
    return f"w{wid}{'_kv8' if kv8 else ''}{'_rope' if rope_dim else ''}{'' if fused else '_unfused'}"


def measured_traffic(tag):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(HERE, "profiles", f"attn_{tag}_hbm_traffic.json")
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != source_sha():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(wid, target_s):
    """The oracle (plain C, OpenMP over queries) on a bounded sample of the same
    workload: the same step (fp8 round trip of the new rows and ring write,
    window lists, compressed append, attention) for n queries of input set 0
    (the first n sequences of a decode batch, n positions spread evenly over a
    prefill chunk), repeated when the whole batch takes well under the target time.  The
    cache contents before the step (rows already rounded through fp8) are
    prepared outside the timed region, as they are for the GPU."""
    import numpy as np
    import oracle
    from sparse_latent_attention_02_amd import workloads as wl
    w = wl.WORKLOADS[wid]
    raw = wl.generate(wid)
    bits = wl.bf16_bits
    # the oracle's OpenMP loops get this many threads, set explicitly (another
    # OpenMP runtime in the process, torch's, may have fixed its own count)
    threads = oracle.set_threads(int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0)))
    if wid == 1:
        return ring_run_baseline(w, raw, threads, target_s)
    sink = raw["sink"].numpy()
    comp = np.ascontiguousarray(raw["comp"].numpy()) if raw["comp"] is not None else None

    def prepare(nq):
        # a query sample: decode -> the first nq sequences; prefill -> nq queries
        # evenly spread over the chunk (their lists grow with the position)
        if w.start_pos > 0:
            kv = bits(raw["kv"][:nq]).copy()
            oracle.act_quant_fp8_inplace(kv)
            slot = w.start_pos % w.window
            return dict(kv=kv, new=bits(raw["kv"][:nq, slot:slot + 1]).copy(), q=bits(raw["q"][:nq]),
                        comp=comp[:nq] if comp is not None else None, nb=nq)
        comp_rows = None
        if w.n_comp:
            comp_rows = bits(raw["kv"][:, w.win_rows:]).copy()
            oracle.act_quant_fp8_inplace(comp_rows)
        sel = np.unique(np.linspace(0, w.s - 1, nq).round().astype(np.int64))   # spread over the chunk
        return dict(chunk=bits(raw["kv"][:, : w.win_rows]).copy(), comp_rows=comp_rows,
                    q=np.ascontiguousarray(bits(raw["q"])[:, sel]), sel=sel)

    def step(p):
        if w.start_pos > 0:
            nb, kv = p["nb"], p["kv"]
            new = p["new"].copy()
            oracle.act_quant_fp8_inplace(new)
            ring = np.ascontiguousarray(kv[:, : w.window])
            oracle.ring_write(ring, new, w.start_pos)
            kv[:, : w.window] = ring
            idx = np.empty((nb, 1, w.topk), dtype=np.int32)
            oracle.window_topk_idxs_into(idx, w.window, nb, 1, w.start_pos)
            if p["comp"] is not None:
                oracle.append_compressed_idxs(idx, w.win_cols, p["comp"], w.win_rows)
            oracle.sparse_attn(p["q"], kv, sink, idx, w.scale)
        else:
            chunk = p["chunk"].copy()
            oracle.act_quant_fp8_inplace(chunk)
            kv = chunk if p["comp_rows"] is None else np.concatenate([chunk, p["comp_rows"]], axis=1)
            full = np.empty((1, w.s, w.topk), dtype=np.int32)
            oracle.window_topk_idxs_into(full, w.window, 1, w.s, 0)
            if comp is not None:
                oracle.append_compressed_idxs(full, w.win_cols, comp, w.win_rows)
            oracle.sparse_attn(p["q"], kv, sink, np.ascontiguousarray(full[:, p["sel"]]), w.scale)

    def timed(p, reps=1):
        t0 = time.perf_counter()
        for _ in range(reps):
            step(p)
        return time.perf_counter() - t0

    nq_total = w.b if w.start_pos > 0 else w.s
    unit = min(nq_total, max(1, threads))          # one query per thread in the probe
    # two probes separate the per-query cost from the per-step fixed cost
    t1 = timed(prepare(unit))
    u4 = min(nq_total, 4 * unit)
    t4 = timed(prepare(u4)) if u4 > unit else t1
    per_q = max((t4 - t1) / (u4 - unit) if u4 > unit else t1 / unit, 1e-6)
    fixed = max(0.0, t1 - unit * per_q)
    nq = int(min(nq_total, max(unit, (target_s - fixed) / per_q)))
    if w.start_pos == 0:
        nq = max(unit, nq // unit * unit)
    p = prepare(nq)
    t = timed(p)
    reps = 1
    if nq == nq_total and t < target_s / 2:
        reps = int(min(1000, max(1, target_s / max(t, 1e-6))))
        t = timed(p, reps)
    return {"value": reps * nq * w.h / t, "unit": "query-heads/s", "cores": threads, "kind": "oracle",
            "sample": f"{nq} of {nq_total} queries (all {w.h} heads) of input set 0"
                      f"{' spread evenly over the chunk' if w.start_pos == 0 else ''}"
                      f"{f', {reps} passes' if reps > 1 else ''}, full step (fp8 round trip of the new rows "
                      f"and ring write, window lists{', compressed append' if comp is not None else ''}, "
                      f"attention); {t:.2f} s"}


def ring_run_baseline(w, raw, threads, target_s):
    """The oracle over the tiny ring run: a 12-token prefill written into an
    8-slot ring, then decode steps at positions 12 and 13 (fp8 round trip of the
    new rows, ring write, window lists, attention), repeated to the target time."""
    import numpy as np
    import oracle
    from sparse_latent_attention_02_amd import workloads as wl
    bits = wl.bf16_bits
    sink = raw["sink"].numpy()
    q_pre, kv_pre = bits(raw["q_prefill"]), bits(raw["kv_prefill"])
    q_dec = [bits(raw["q_dec"][i]) for i in range(2)]
    kv_dec = [bits(raw["kv_dec"][i]) for i in range(2)]

    def run():
        chunk = kv_pre.copy()
        oracle.act_quant_fp8_inplace(chunk)
        ring = np.zeros((1, w.window, w.d), dtype=np.uint16)
        oracle.ring_write(ring, chunk, 0)
        oracle.sparse_attn(q_pre, chunk, sink, oracle.window_topk_idxs(w.window, 1, 12, 0), w.scale)
        for i, pos in enumerate((12, 13)):
            row = kv_dec[i].copy()
            oracle.act_quant_fp8_inplace(row)
            oracle.ring_write(ring, row, pos)
            oracle.sparse_attn(q_dec[i], ring, sink, oracle.window_topk_idxs(w.window, 1, 1, pos), w.scale)

    run()
    passes, t0 = 0, time.perf_counter()
    while True:
        run()
        passes += 1
        el = time.perf_counter() - t0
        if el > target_s or passes >= 100000:
            break
    qh = (12 + 2) * w.h
    return {"value": passes * qh / el, "unit": "query-heads/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole ring run (prefill 12, decode 12 and 13; {qh} query-heads), {passes} passes; "
                      f"{el:.2f} s"}


def copy_calibration():
    """A plain streaming copy of known size (1 GiB read, 1 GiB written) with the
    same 16-byte-per-lane access width as the kernels, for scaling the HBM byte
    counters of a rocprofv3 run."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def bench_select(args):
    """The indexer selection tail on its workload (decode, 128 queries x 16384
    scored compressed positions, top 2048): HBM bound -- the scores are read and
    the selected columns written once (the radix passes work on keys held in
    registers).  --select-start-pos moves the decode position; rows of more than
    16384 positions are re-read from memory in each pass, and the algorithmic
    bytes still count one read."""
    import torch
    import numpy as np
    import sparse_latent_attention_02_amd as sa
    from sparse_latent_attention_02_amd import workloads as wl
    cfg = wl.SELECT_WORKLOAD
    b, s, start_pos, ratio = cfg["b"], cfg["s"], cfg["start_pos"], cfg["ratio"]
    if args.select_start_pos is not None:
        start_pos = args.select_start_pos
    T = (start_pos + s) // ratio
    topk = min(cfg["index_topk"], T)
    win = cfg["offset"]
    bytes_per = b * s * T * 4 + b * s * topk * 4
    n_sets = args.sets or max(1, min(96, math.ceil(2 * MALL_BYTES / bytes_per)))
    scores = [wl.indexer_scores(3000 + k, b, s, T).cuda() for k in range(n_sets)]
    outs = [torch.empty((b, s, win + topk), dtype=torch.int32, device="cuda") for _ in range(n_sets)]
    call = lambda i: sa.indexer_topk(scores[i], start_pos, ratio, cfg["index_topk"], win, out=outs[i], col0=win)
    if args.copy_calibration:
        copy_calibration()
    for i in range(args.warmup):
        call(i % n_sets)
    torch.cuda.synchronize()
    def capture(ids):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in ids:
                call(i)
        return g
    # exactly `steps` calls: whole chains over the input sets, then a shorter tail
    full = capture(range(n_sets))
    rem = args.steps % n_sets
    tail = capture(range(rem)) if rem else None

    def run(k):
        for _ in range(k // n_sets):
            full.replay()
        if k % n_sets:
            tail.replay()
    run(args.steps)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record(stream)
    run(args.steps)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    n = args.steps
    ms = e0.elapsed_time(e1) / n
    achieved = bytes_per / (ms / 1e3) / 1e9
    line = {
        "metric": "indexer_topk query rows/s", "value": round(b * s / (ms / 1e3), 1), "unit": "rows/s",
        "n_gpus": 1, "steps": n, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"indexer selection tail: b={b} decode at position {start_pos}, ratio {ratio}, "
                               f"{T} scored positions, top {topk}, offset {win}",
                   "input_sets": n_sets, "launch": f"hip graphs of {n_sets} calls (and the tail)", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("select") if start_pos == cfg["start_pos"] else None,
                     "algorithmic_bytes": bytes_per, "kernel_ms_mean": round(ms, 5), "kernel_launches_timed": n},
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle.set_threads(int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0)))
        sc = wl.indexer_scores(3000, b, s, T).numpy()
        t0 = time.perf_counter()
        passes = 0
        while True:
            oracle.indexer_topk(sc, start_pos, ratio, cfg["index_topk"], win)
            passes += 1
            el = time.perf_counter() - t0
            if el > args.cpu_seconds or passes >= 1000:
                break
        line["cpu_baseline"] = {"value": round(passes * b * s / el, 1), "unit": "rows/s", "cores": threads,
                                "kind": "oracle", "sample": f"input set 0 ({b} rows), {passes} passes; {el:.2f} s"}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU; runs over several GPUs are not part of it "
              "(sparse_attn shards over batch/queries or heads with no exchange step).", file=sys.stderr)
        sys.exit(2)

    if args.cpu_only:
        line = {"workload": args.workload, "cpu_baseline": cpu_baseline(args.workload, args.cpu_seconds)}
        print(json.dumps(line), flush=True)
        return
    if args.workload == 1:
        print("bench.py: workload 1 is timed with --cpu-only only (it is a correctness case)", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_latent_attention_02_amd as sa
    from sparse_latent_attention_02_amd import pipeline
    from sparse_latent_attention_02_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    sa.lib()
    if args.select:
        bench_select(args)
        return
    w = wl.WORKLOADS[args.workload]

    # ---- inputs resident in HBM, rotating sets for small workloads ----
    raw0 = wl.generate(args.workload)
    if args.kv8 and (w.start_pos == 0 or args.unfused):
        print("bench.py: --kv8 applies to the one-launch decode step (workloads 2 and 4)", file=sys.stderr)
        sys.exit(2)
    rope_dim = pipeline.ROPE_DIM if args.rope else 0
    if args.rope and args.kv8:
        print("bench.py: --rope and --kv8 are not combined", file=sys.stderr)
        sys.exit(2)
    sets = [pipeline.prepare(args.workload, raw0, kv8=args.kv8, rope_dim=rope_dim)]
    pipeline.build_index(sets[0])
    torch.cuda.synchronize()
    # the lists built in the attention kernel unless --unfused
    fused = not args.unfused
    if args.kv8:
        step_fn = kern_fn = pipeline.step_fused_kv8
    elif w.start_pos > 0:
        step_fn = pipeline.step_fused if fused else pipeline.step
        kern_fn = pipeline.step_fused if fused else pipeline.attend    # the dominant kernel's launch
    else:
        step_fn = pipeline.step_fused_prefill if fused else pipeline.step
        kern_fn = pipeline.attend_fused_prefill if fused else pipeline.attend
    work = algorithmic_work(w, [sets[0].idx], fused, args.kv8)
    if rope_dim:
        work["bytes"] += w.b * w.s * rope_dim * 4       # each query's table row
    n_sets = args.sets or max(1, min(48, math.ceil(2 * MALL_BYTES / work["bytes"])))
    for k in range(1, n_sets):
        sets.append(pipeline.prepare(args.workload, wl.generate(args.workload, seed_offset=97 * k), kv8=args.kv8,
                                     rope_dim=rope_dim))
    del raw0
    torch.cuda.synchronize()

    if args.copy_calibration:
        copy_calibration()

    # ---- warmup (eager), then one HIP graph per input set for the step and for
    #      the attention launch alone: replays keep the host out of the timing ----
    for i in range(args.warmup):
        step_fn(sets[i % n_sets])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    if args.graphs:
        # one graph holds a chain of steps over consecutive input sets (as a
        # decode loop over layers would), so graph launch cost is paid once per
        # chain; a second graph holds the attention launches alone, back to back
        def capture(fn, ids):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in ids:
                    fn(sets[i])
            return g
        # (a chain of at least CHAIN_MIN steps, cycling through the sets, so that
        # a single resident set is not timed one graph launch per step)
        chain = n_sets * max(1, math.ceil(CHAIN_MIN / n_sets))
        ids = [i % n_sets for i in range(chain)]
        full = capture(step_fn, ids)
        rem = args.steps % chain
        tail = capture(step_fn, ids[:rem]) if rem else None

        def run_steps(k):
            for _ in range(k // chain):
                full.replay()
            if k % chain:
                assert k % chain == rem
                tail.replay()
        attn_graph = capture(kern_fn, ids)
        n_attn_reps = max(1, math.ceil(args.steps / chain))
        run_attn = lambda: [attn_graph.replay() for _ in range(n_attn_reps)]
        n_attn = n_attn_reps * chain
        launch_desc = f"hip graph of {chain} steps over the {n_sets} input set{'s' if n_sets > 1 else ''}"
    else:
        def run_steps(k):
            for i in range(k):
                step_fn(sets[i % n_sets])
        n_attn = max(args.steps, n_sets)
        run_attn = lambda: [kern_fn(sets[i % n_sets]) for i in range(n_attn)]
        launch_desc = "eager"
    run_steps(args.steps)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps ----
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    run_steps(args.steps)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps

    # ---- attention kernel duration: HIP events around back-to-back launches ----
    a_start = torch.cuda.Event(enable_timing=True)
    a_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a_start.record(stream)
    run_attn()
    a_end.record(stream)
    torch.cuda.synchronize()
    attn_mean = a_start.elapsed_time(a_end) / n_attn

    qh = w.b * w.s * w.h
    value = qh / (ms_step / 1e3)
    hbm_s = work["bytes"] / PEAK_HBM_GBS / 1e9
    mfma_s = work["flops"] / PEAK_BF16_TFLOPS / 1e12
    if hbm_s >= mfma_s:
        achieved = work["bytes"] / (attn_mean / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = work["flops"] / (attn_mean / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    roof["traffic"] = measured_traffic(traffic_tag(args.workload, fused, args.kv8, rope_dim))
    roof["algorithmic_bytes"] = work["bytes"]
    roof["algorithmic_flops"] = work["flops"]
    roof["kernel_ms_mean"] = round(attn_mean, 5)
    roof["kernel_launches_timed"] = n_attn

    line = {
        "metric": "sparse_attn query-heads/s",
        "value": round(value, 1),
        "unit": "query-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.b, "queries_per_seq": w.s, "heads": w.h, "head_dim": w.d,
                   "topk": w.topk, "kv_rows_per_seq": w.rows, "valid_entries": work["valid"],
                   "input_sets": n_sets, "launch": launch_desc,
                   "step": ("separate calls" if not fused else "one-launch decode step" if w.start_pos > 0
                            else "chunk fp8 round trip, then attention with the list built in the kernel"),
                   "kv_cache": "fp8 e4m3fn codes + E8M0 block scales" if args.kv8 else "bf16",
                   "output_rotation": f"inverse rotary embedding of the last {rope_dim} values, fused"
                   if rope_dim else "none",
                   "parallelism": "single GPU"},
        "roofline": roof,
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
