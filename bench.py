"""Decode-step benchmark: KV-read GB/s, fraction of the HBM roofline, steps/s.

One step is the whole hot path on one batch: append one token of K/V per
sequence, then attention of every query head over its cache, the new token
included. By default the step is one gqa_decode_step launch (append and
attention fused); --unfused runs gqa_kv_append then gqa_decode_attention. Inputs are seeded synthetic caches of the named
workload (default: one Llama-3-70B-shaped GQA layer, b=16, h=64, g=8, d=128,
bf16, lengths uniform on [1024, 8192]), resident in HBM before timing starts.

So that every step reads its K/V from HBM rather than from the 256 MB
last-level cache, the benchmark keeps several independent cache sets (same
drawn lengths, contents from their own seeds) and cycles through them, one
set per step; each set's lengths grow by one per step it takes, as in a real
decode loop.

value = algorithmic KV bytes of all timed steps / wall time of those steps,
where the bytes of one step are sum_b g * L_b * (d_k + d_v) * elem_bytes at
the attended lengths L_b. roofline.achieved uses the same bytes per decode
launch over the decode kernel's average launch duration, from HIP events on
the launch stream: for the fused step (one launch per step) the timed
region's time over the step count; with --unfused, a pair of events around
each decode launch. The roofline's peak is the nominal 8 TB/s; the line also
states the rate against the read bandwidth this part sustains, measured in
the same run by a plain streaming read of 2 GiB (gqa_read_bandwidth: one
workgroup per compute unit, the decode kernels' non-temporal 16-byte loads;
20 launches back to back): roofline.measured_read_gbs, frac_of_measured_read;
and the time of the same read of exactly one step's KV bytes in one launch
(roofline.read_of_step_bytes_us), the floor of a step's time on this part.

With --layer the step is one gqa_decode_layer call instead: the query, key
and value projections of the new token (one launch), the fused append +
attention, and the output projection, with d_model = h * d_k and bf16
weights in the packed layout. Each layer set holds its own cache and its own
device copy of the four weight matrices, and consecutive steps go to
consecutive sets, as a decode step walks the layers of a model. Its value is
(weight bytes + KV bytes) per step over the step time, and its roofline is
that of the whole layer (three launches).

With --fold the step is the mean-fold of a multi-head cache to fewer KV
heads (gqa_fold_kv_heads on K, then on V; default: the long MHA workload,
g = 32 -> 8): value = bytes read and written per step over the step time.
The line also carries the lesson's comparison at the same cache and queries:
the relative change of the attention output against MHA for each folded g,
and the decode time over each folded cache.

With --paged B the caches live in pools of B-position blocks behind shuffled
block tables (gqa_decode_step_paged); bytes and timing as for the step.

With --tokens N (N > 1) each step appends N new tokens per sequence and runs
their causal attention (gqa_decode_step_multi: two launches; with --paged B
too, gqa_decode_step_multi_paged); bytes are those the last token attends,
read once for all N tokens.

With --graph the timed steps are captured in one HIP graph and replayed, which
removes the host's per-call cost (it matters for the small, launch-bound
workloads).

After the timed region the same number of steps runs again with an event
between consecutive steps: their p10 / p50 / p90 go into the line
("per_step_us"). roofline.traffic is the HBM traffic over algorithmic bytes
measured by the committed counter summary (both on one set of lengths, and
only while the decode sources match its stamp) times this line's bytes.

With --gscale the line is the long-context comparison across KV-head counts
(g = 32 / 8 / 1 on one seed): bytes and time per step, and the time ratio.

With --flushed R, R more steps are timed one at a time after the timed region,
each after a 1 GiB fill that evicts every cache level: the line gains their
p10 / p50 / p90 latency ("flushed"). The CPU baseline times the fp64 oracle on
every host core the process may use and on one core (--cpu-threads T: T threads).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--paged B] [--tokens N]
                       [--graph] [--layer | --fold G | --gscale] [--flushed R] [--cpu-threads T]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "KV-read GB/s and % of HBM roofline; decode-attention steps/sec"
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def traffic_from_profile(workload: str):
    """HBM traffic over algorithmic bytes of the decode launch, from the committed counter summary.

    The ratio (both measured in one counter run, on one set of lengths) if the
    summary's source stamp matches the current decode sources, else None.
    """
    from gqa_kv_cache_decode_amd import rocprof_summary

    path = os.path.join(PROFILE_DIR, f"decode_traffic_{workload}.txt")
    rec = rocprof_summary.read_traffic(path)
    if not rec or rec.get("kernel_source_hash") != rocprof_summary.kernel_source_hash():
        return None
    return float(rec["hbm_bytes_per_launch"]) / float(rec["algorithmic_bytes_per_launch"]), os.path.relpath(path, ROOT)


def cpu_baseline(wl, batch_host, budget_s: float, threads: int = 0):
    """Time the fp64 oracle (as it stands) on full decode steps of one cache set.

    Half the budget with every host core this process may run on (or the
    given thread count), half on one core; the same algorithmic bytes as the
    GPU line.
    """
    import oracle

    threads = threads or len(os.sched_getaffinity(0))
    kc = batch_host.k_cache.copy()
    vc = batch_host.v_cache.copy()
    lens = batch_host.lens.copy()
    q = batch_host.q(0)
    kn, vn = batch_host.new_kv(0)
    oracle.kv_append(kc, vc, kn, vn, lens)
    kv_bytes = int(lens.sum()) * wl.g * 2 * wl.d * wl.elem_bytes

    def timed(nthreads, seconds):
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.decode_attention(q, kc, vc, lens, wl.scale, threads=nthreads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds or reps >= 1000:
                return reps, el

    reps, el = timed(threads, budget_s / 2)
    reps1, el1 = timed(1, budget_s / 2)
    return {"value": round(kv_bytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} repetition(s) of one full decode step (b={wl.b}, all sequences, "
                      f"sum L={int(lens.sum())}) of cache set 0, fp64 oracle on {threads} OpenMP threads "
                      f"(all host cores available to the process); then {reps1} on one thread",
            "seconds": round(el, 3),
            "one_core": {"value": round(kv_bytes * reps1 / el1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                         "seconds": round(el1, 3)}}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--sets", type=int, default=0, help="cache sets to cycle (0: enough for >= 1.5 GB)")
    ap.add_argument("--path", type=int, default=0, help="0 auto, 1 vector, 2 matrix")
    ap.add_argument("--workgroups", type=int, default=0, help="persistent grid size (0: automatic)")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="oracle time budget, half on all cores, half on one (0: skip)")
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (0: every core the process may use)")
    ap.add_argument("--gscale", action="store_true",
                    help="the long-context MHA comparison: g = 32, 8, 1 KV heads on the same seed (h = 32, "
                         "b = 4, L = 32769), bytes and time per step and the time ratio")
    ap.add_argument("--flushed", type=int, default=0, metavar="R",
                    help="after the timed steps, time R more steps one at a time, each after a 1 GiB fill "
                         "(outside the events) that evicts the caches; adds p10/p50/p90 to the line")
    ap.add_argument("--unfused", action="store_true",
                    help="run the step as gqa_kv_append + gqa_decode_attention instead of gqa_decode_step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a 1 GiB device copy first (reference for HBM byte counters)")
    ap.add_argument("--layer", action="store_true",
                    help="time the whole decode layer (projections + step) instead of the step alone")
    ap.add_argument("--graph", action="store_true",
                    help="capture the timed steps in one HIP graph and time its replay (no host launch cost)")
    ap.add_argument("--tokens", type=int, default=1, metavar="N",
                    help="new tokens per sequence and step (N > 1: gqa_decode_step_multi[_paged], causal)")
    ap.add_argument("--paged", type=int, default=0, metavar="B",
                    help="keep the caches in pools of B-position blocks behind shuffled block tables")
    ap.add_argument("--fold", type=int, default=0, metavar="G",
                    help="time the mean-fold of the workload's cache to G KV heads instead of the step")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported. Across GPUs the step would be "
              "sharded by sequence (or by KV head) with no exchange, so its per-GPU work is the one-GPU "
              "step on that GPU's share.", file=sys.stderr)
        sys.exit(2)

    import torch

    from gqa_kv_cache_decode_amd import api, inputs
    from gqa_kv_cache_decode_amd.workloads import HEADLINE, WORKLOADS, kv_bytes_attended

    wl = WORKLOADS[args.workload or HEADLINE]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    total_steps = args.warmup + 2 * args.steps + args.flushed
    if args.layer:
        if wl.dtype != "bf16" or args.unfused:
            print("--layer runs bf16 workloads with the fused step only", file=sys.stderr)
            sys.exit(2)
        return bench_layer(args, wl, dev)
    if args.fold:
        return bench_fold(args, WORKLOADS[args.workload or "mha_long_bf16_g32"], dev)
    if args.gscale:
        return bench_gscale(args, dev)

    # cache sets
    set_bytes = wl.b * wl.g * wl.cap * wl.d * 2 * wl.elem_bytes
    n_sets = args.sets or max(2, math.ceil(1.5e9 / set_bytes))
    n_sets = min(n_sets, total_steps) if total_steps > 0 else 1
    ntok = args.tokens
    grow = math.ceil(total_steps / n_sets) * ntok + 1
    log(f"workload {wl.name}: {n_sets} cache sets of {set_bytes / 1e6:.1f} MB")

    def to_dev(a):
        t = torch.from_numpy(a)
        return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).to(dev)

    def to_pool(cache, bs, seed):
        # every block of every sequence to a random place in one pool (block table [b, max_blocks])
        b, g, cap, d = cache.shape
        mb = (cap + bs - 1) // bs
        gen = torch.Generator(device="cpu").manual_seed(seed)
        perm = torch.randperm(b * mb, generator=gen).to(torch.int32)
        pool = torch.empty(b * mb, g, bs, d, dtype=cache.dtype, device=dev)
        padded = torch.zeros(b, g, mb * bs, d, dtype=cache.dtype, device=dev)
        padded[:, :, :cap] = cache
        pool[perm.long().to(dev)] = padded.view(b, g, mb, bs, d).permute(0, 2, 1, 3, 4).reshape(b * mb, g, bs, d)
        del padded, cache
        return pool, perm.view(b, mb).to(dev)

    if args.paged and (args.unfused or args.paged < 32 or args.paged & (args.paged - 1)):
        print("--paged B: B a power of two >= 32, fused step only", file=sys.stderr)
        sys.exit(2)
    if args.graph and args.unfused:
        print("--graph times the fused step only", file=sys.stderr)
        sys.exit(2)
    if ntok < 1 or (ntok > 1 and args.unfused):
        print("--tokens N: N >= 1; N > 1 times the multi-token step (append + attention), not --unfused",
              file=sys.stderr)
        sys.exit(2)
    sets = []
    host0 = None
    for r in range(n_sets):
        # every set shares set 0's drawn lengths (identical bytes per step); contents differ
        batch = inputs.Batch(seed=wl.seed + 1000 * r, b=wl.b, h=wl.h, g=wl.g, d=wl.d, cap=wl.cap + grow,
                             lens=wl.lens if r == 0 else host0.lens.tolist(), dtype=wl.dtype, poison=False)
        if r == 0:
            host0 = batch
        sets.append({
            "kc": to_dev(batch.k_cache), "vc": to_dev(batch.v_cache),
            "lens": torch.from_numpy(batch.lens.copy()).to(dev), "lens_h": batch.lens.copy(),
            "cap": wl.cap + grow,
        })
        if r != 0:
            del batch
        if args.paged:
            st = sets[-1]
            st["kc"], st["table"] = to_pool(st["kc"], args.paged, wl.seed + r)
            st["vc"], _ = to_pool(st["vc"], args.paged, wl.seed + r)
    log("caches resident" + (f" as pools of {args.paged}-position blocks" if args.paged else ""))
    cap = wl.cap + grow
    max_len_bound = int(max(s["lens_h"].max() for s in sets)) + grow
    ws = api.make_workspace(wl.b, wl.h, wl.g, wl.d, wl.d, max_len_bound, dt, dev)
    out = torch.empty(wl.b, wl.h, wl.d, dtype=dt, device=dev)
    qs = [to_dev(inputs.draw_q(wl.seed, s, wl.b, wl.h, wl.d, wl.dtype)) for s in range(min(total_steps, 64))]
    news = []
    for s in range(min(total_steps, 64)):
        kn, vn = inputs.draw_new_kv(wl.seed, s, wl.b, wl.g, wl.d, wl.d, wl.dtype)
        news.append((to_dev(kn), to_dev(vn)))
    if ntok > 1:
        # token r of step s uses the one-token draws of index s * N + r, stacked token-major
        ws = api.make_multi_workspace(wl.b, ntok, wl.h, wl.g, wl.d, wl.d, dt, dev)
        out = torch.empty(wl.b, ntok, wl.h, wl.d, dtype=dt, device=dev)
        nq = min(total_steps, 16)
        qs = [torch.stack([to_dev(inputs.draw_q(wl.seed, s * ntok + r, wl.b, wl.h, wl.d, wl.dtype))
                           for r in range(ntok)], dim=1).contiguous() for s in range(nq)]
        news = []
        for s in range(nq):
            rows = [inputs.draw_new_kv(wl.seed, s * ntok + r, wl.b, wl.g, wl.d, wl.d, wl.dtype) for r in range(ntok)]
            news.append((torch.stack([to_dev(k) for k, _ in rows], dim=1).contiguous(),
                         torch.stack([to_dev(v) for _, v in rows], dim=1).contiguous()))

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream()

    # Every set starts from set 0's lengths and grows by ntok per step it
    # takes, so a step's host-side bound and byte count follow from how many
    # steps its set has taken (tables, so the timed loop issues launches and
    # little else: steps of ~20 us are otherwise bound by the host).
    lens0 = sets[0]["lens_h"].copy()
    max0 = int(lens0.max())
    taken = [0] * n_sets
    bytes_after = []  # bytes_after[c]: attended bytes of a set's step number c (0-based)

    def step_bytes(c):
        while len(bytes_after) <= c:
            bytes_after.append(kv_bytes_attended(wl.g, wl.d, wl.d, wl.elem_bytes, lens0 + ntok * (len(bytes_after) + 1)))
        return bytes_after[c]

    launched = []  # attended bytes of every decode launch of the run, in order

    def step(i, ev_pair=None):
        si = i % n_sets
        st = sets[si]
        kn, vn = news[i % len(news)]
        c = taken[si]
        max_len = max0 + ntok * c
        if args.unfused:
            api.kv_append(st["kc"], st["vc"], kn, vn, st["lens"], max_len)
        if ev_pair is not None:
            ev_pair[0].record(stream)
        if args.unfused:
            api.decode_attention(out, qs[i % len(qs)], st["kc"], st["vc"], st["lens"], max_len + 1, wl.scale, ws,
                                 path=args.path, workgroups=args.workgroups)
        elif args.paged and ntok > 1:
            api.decode_step_multi_paged(out, qs[i % len(qs)], kn, vn, st["kc"], st["vc"], st["lens"], st["table"],
                                        max_len, wl.scale, ws)
        elif args.paged:
            api.decode_step_paged(out, qs[i % len(qs)], kn, vn, st["kc"], st["vc"], st["lens"], st["table"], max_len,
                                  wl.scale, ws)
        elif ntok > 1:
            api.decode_step_multi(out, qs[i % len(qs)], kn, vn, st["kc"], st["vc"], st["lens"], max_len, wl.scale, ws)
        else:
            api.decode_step(out, qs[i % len(qs)], kn, vn, st["kc"], st["vc"], st["lens"], max_len, wl.scale, ws,
                            path=args.path, workgroups=args.workgroups)
        if ev_pair is not None:
            ev_pair[1].record(stream)
        taken[si] = c + 1
        launched.append(step_bytes(c))
        return step_bytes(c)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("warmup done")

    # The fused step is one launch of the decode kernel, so the timed region is
    # exactly `steps` back-to-back launches of it and its average launch
    # duration is the region's time over `steps` (launch gaps included). The
    # two-call form brackets each decode launch with its own pair of events.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)] if args.unfused else [None] * args.steps
    total_bytes = 0
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    if args.graph:
        # The library only enqueues kernels on the given stream, so the whole
        # timed loop is captured once (host mirrors of the lengths advance as
        # the launches are recorded; the device state is untouched until the
        # replay) and replayed once inside the timed region.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for k in range(args.steps):
                total_bytes += step(args.warmup + k, None)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
    wall0 = time.perf_counter()
    t_start.record(stream)
    if args.graph:
        graph.replay()
    else:
        for k in range(args.steps):
            total_bytes += step(args.warmup + k, evs[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    elapsed_ms = t_start.elapsed_time(t_end)
    if args.unfused:
        kern_ms = [a.elapsed_time(b) for a, b in evs]
    else:
        kern_ms = [elapsed_ms / args.steps]
    kern_avg_ms = float(np.mean(kern_ms))
    bytes_per_launch = total_bytes / args.steps
    log(f"timed {args.steps} steps: {elapsed_ms:.3f} ms (host wall {wall * 1e3:.1f} ms); "
        f"decode kernel avg {kern_avg_ms * 1e3:.2f} us, median {np.median(kern_ms) * 1e3:.2f} us")

    value = total_bytes / (elapsed_ms / 1e3) / 1e9
    achieved = bytes_per_launch / (kern_avg_ms / 1e3) / 1e9
    # The same number of steps again, with an event between consecutive steps
    # (outside the timed region above): the spread of single steps.
    per_step = None
    if not args.graph and args.steps >= 5:
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        marks[0].record(stream)
        for k in range(args.steps):
            step(args.warmup + args.steps + k, None)
            marks[k + 1].record(stream)
        torch.cuda.synchronize()
        d = np.array([marks[k].elapsed_time(marks[k + 1]) * 1e3 for k in range(args.steps)])
        per_step = {"p10_us": round(float(np.percentile(d, 10)), 2), "p50_us": round(float(np.median(d)), 2),
                    "p90_us": round(float(np.percentile(d, 90)), 2), "steps": args.steps,
                    "what": "a second pass of as many steps, one event between consecutive steps"}
        log(f"per step: p10 / p50 / p90 {per_step['p10_us']} / {per_step['p50_us']} / {per_step['p90_us']} us")
    flushed = None
    if args.flushed > 0 and not args.graph:
        # one step at a time, each after a 1 GiB fill outside its events (every
        # cache level evicted): the latency of a cold step, not a throughput
        fill = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        lat = []
        for k in range(args.flushed):
            fill.fill_(k & 255)
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            step(args.warmup + 2 * args.steps + k, ev)
            ev[1].synchronize()
            lat.append(ev[0].elapsed_time(ev[1]) * 1e3)
        del fill
        flushed = {"reps": args.flushed, "p10_us": round(float(np.percentile(lat, 10)), 2),
                   "p50_us": round(float(np.median(lat)), 2), "p90_us": round(float(np.percentile(lat, 90)), 2),
                   "what": "per-step events around the " + ("decode launch" if args.unfused else "step's launches")
                           + ", each step after a 1 GiB fill"}
        log(f"flushed steps: p10 / p50 / p90 {flushed['p10_us']} / {flushed['p50_us']} / {flushed['p90_us']} us")
    # a multi-token call is planned as a one-token call with N * h heads
    plan_path, plan_wgs, plan_merge, plan_stream = api.plan(wl.b, wl.h * ntok, wl.g, wl.d, wl.d, cap, max_len_bound,
                                                            dt, api.PATH_AUTO if ntok > 1 else args.path,
                                                            args.workgroups, stream_flag=True)
    plan_stream = plan_stream and ntok == 1
    traffic = None if (args.paged or ntok > 1 or args.unfused) else traffic_from_profile(wl.name)

    read_gbs, read_step_us = measured_read_bandwidth(dev, step_bytes=bytes_per_launch)
    log(f"measured streaming read: {read_gbs:.1f} GB/s; of one step's KV bytes: {read_step_us:.2f} us")

    cpu = None
    if args.cpu_seconds > 0 and ntok == 1:
        log("timing the CPU oracle ...")
        cpu = cpu_baseline(wl, host0, args.cpu_seconds, args.cpu_threads)

    lens0 = host0.lens
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed_ms / args.steps, 5),
        "steps_per_s": round(args.steps / (elapsed_ms / 1e3), 1),
        "hbm_roofline_frac_of_step": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.name + (f"_paged_blocks{args.paged}" if args.paged else "")
                        + (f"_{ntok}_tokens" if ntok > 1 else ""),
            "b": wl.b, "h": wl.h, "g": wl.g, "d_k": wl.d, "d_v": wl.d,
            "lens": list(wl.lens) if isinstance(wl.lens, (list, tuple)) else wl.lens,
            "lens_drawn_mean": float(lens0.mean()), "lens_drawn_min": int(lens0.min()),
            "lens_drawn_max": int(lens0.max()), "cache_sets": n_sets, "seed": wl.seed,
            "path": {1: "vector", 2: "matrix"}[plan_path], "workgroups": plan_wgs,
            "split_merge": "second launch" if plan_merge == api.MERGE_KERNEL else "in the decode kernel",
            "step_api": ("gqa_kv_append + gqa_decode_attention" if args.unfused else
                         f"gqa_decode_step_multi_paged ({ntok} tokens, blocks of {args.paged})"
                         if args.paged and ntok > 1 else
                         f"gqa_decode_step_paged (blocks of {args.paged})" if args.paged else
                         f"gqa_decode_step_multi ({ntok} tokens: append + causal attention)" if ntok > 1 else
                         "gqa_decode_step"),
            "new_tokens_per_step": ntok, "tokens_per_s": round(wl.b * ntok * args.steps / (elapsed_ms / 1e3), 1),
            "launch": "one HIP graph of all timed steps" if args.graph else "eager, one call per step",
            "kv_bytes_per_step": int(bytes_per_launch),
            # every decode launch of this run (warm-up, timed, percentile pass):
            # the denominator of a counter run's traffic ratio
            "kv_bytes_per_launch_all": int(round(float(np.mean(launched)))),
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else int(round(traffic[0] * bytes_per_launch)),
            "traffic_ratio": None if traffic is None else round(traffic[0], 4),
            "traffic_source": None if traffic is None else traffic[1],
            "kernel": ("decode_stream_kernel" if plan_stream else
                       "decode_matrix_kernel" if plan_path == 2 else "decode_vector_kernel")
                      + (" + merge_partials_kernel" if plan_merge == api.MERGE_KERNEL else "")
                      + ("" if args.unfused else " (fused step)" if ntok == 1 else
                         f" (causal, {ntok} tokens) + kv_append_kernel") + (", paged" if args.paged else ""),
            "kernel_avg_us": round(kern_avg_ms * 1e3, 3),
            # the same rate against what a plain streaming read sustains on this part
            "measured_read_gbs": round(read_gbs, 1),
            "frac_of_measured_read": round(achieved / read_gbs, 4),
            # the same read of exactly one step's KV bytes, one launch: the floor of a step's time
            "read_of_step_bytes_us": round(read_step_us, 2),
        },
        "cpu_baseline": cpu,
    }
    if per_step is not None:
        rec["per_step_us"] = per_step
    if flushed is not None:
        rec["flushed"] = flushed
    print(json.dumps(rec), flush=True)


def measured_read_bandwidth(dev, step_bytes: float, nbytes: int = 2 << 30, reps: int = 20):
    """gqa_read_bandwidth with one 512-thread workgroup per compute unit, timed back to back
    like the decode steps: the GB/s of reading a buffer of nbytes (far beyond the last-level
    cache), the rate the decode kernels' roofline is also stated against; and the time of
    reading one step's KV bytes in one launch, from windows of that buffer taken in rotation
    (as the cache sets are), so that no window is still in the last-level cache when it is
    read again."""
    import torch

    from gqa_kv_cache_decode_amd import api

    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(torch.cuda.get_device_properties(dev).multi_processor_count, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def timed(views):
        # back to back, as the decode steps are timed: the region's time over the launches
        for v in views[:3]:
            api.read_bandwidth(v, sink)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for k in range(reps):
            api.read_bandwidth(views[k % len(views)], sink)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    ms = timed([buf])
    if int((sink.to(torch.int64) % (1 << 32)).sum().item()) % (1 << 32) != (nbytes // 4) % (1 << 32):
        raise RuntimeError("streaming read: the checksum of the read buffer is wrong")
    words = max(4, int(step_bytes) // 16 * 4)
    windows = [buf[k * words:(k + 1) * words] for k in range(max(1, min(8, buf.numel() // words)))]
    step_ms = timed(windows)
    del buf, windows
    return nbytes / (ms / 1e3) / 1e9, step_ms * 1e3


def bench_layer(args, wl, dev):
    """Whole-layer decode steps (gqa_decode_layer), cycling through layer sets."""
    import torch

    from gqa_kv_cache_decode_amd import api, inputs
    from gqa_kv_cache_decode_amd.workloads import kv_bytes_attended

    dt = torch.bfloat16
    h, g, d = wl.h, wl.g, wl.d
    d_model = h * d
    total_steps = args.warmup + args.steps
    w_shapes = [(h * d, d_model), (g * d, d_model), (g * d, d_model), (d_model, h * d)]
    w_bytes = sum(2 * o * i for o, i in w_shapes)
    cache_bytes = wl.b * g * wl.cap * d * 2 * wl.elem_bytes
    n_sets = args.sets or max(2, math.ceil(1.5e9 / (w_bytes + cache_bytes)))
    n_sets = min(n_sets, total_steps) if total_steps > 0 else 1
    grow = math.ceil(total_steps / n_sets) + 1
    cap = wl.cap + grow
    log(f"layer {wl.name}, d_model={d_model}: {n_sets} layer sets of {(w_bytes + cache_bytes) / 1e6:.1f} MB")

    def to_dev(a):
        return torch.from_numpy(a).view(torch.bfloat16).to(dev)

    # one draw of each matrix; every layer set packs its own device copy
    w_host = [inputs.draw_weight(wl.seed, k, o, i, "bf16") for k, (o, i) in enumerate(w_shapes)]
    sets, host0 = [], None
    for r in range(n_sets):
        batch = inputs.Batch(seed=wl.seed + 1000 * r, b=wl.b, h=h, g=g, d=d, cap=cap,
                             lens=wl.lens if r == 0 else host0.lens.tolist(), dtype="bf16", poison=False)
        if r == 0:
            host0 = batch
        ws_dev = []
        for w in w_host:
            t = to_dev(w)
            ws_dev.append(api.PackedWeight(t))
            del t
        sets.append({"w": ws_dev, "kc": to_dev(batch.k_cache), "vc": to_dev(batch.v_cache),
                     "lens": torch.from_numpy(batch.lens.copy()).to(dev), "lens_h": batch.lens.copy()})
        if r != 0:
            del batch
    torch.cuda.synchronize()
    log("layer sets resident")
    max_len_bound = int(max(st["lens_h"].max() for st in sets)) + grow
    ws = api.make_workspace(wl.b, h, g, d, d, max_len_bound, dt, dev)
    scratch = api.LayerScratch(wl.b, h, g, d, d, dt, dev)
    xs = [to_dev(inputs.draw_x(wl.seed, s, wl.b, d_model, "bf16")) for s in range(min(total_steps, 64))]
    y = torch.empty(wl.b, d_model, dtype=dt, device=dev)
    io_bytes = 2 * wl.b * (2 * d_model + 2 * h * d + 2 * g * d)  # x, y, q, attn, k_new, v_new

    def step(i):
        st = sets[i % n_sets]
        api.decode_layer(y, xs[i % len(xs)], *st["w"], st["kc"], st["vc"], st["lens"], int(st["lens_h"].max()),
                         wl.scale, ws, scratch)
        st["lens_h"] += 1
        return kv_bytes_attended(g, d, d, wl.elem_bytes, st["lens_h"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("warmup done")
    stream = torch.cuda.current_stream()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    kv_total = 0
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(args.steps):
        kv_total += step(args.warmup + k)
    t_end.record(stream)
    torch.cuda.synchronize()
    elapsed_ms = t_start.elapsed_time(t_end)
    step_ms = elapsed_ms / args.steps
    bytes_per_step = w_bytes + kv_total / args.steps + io_bytes
    value = bytes_per_step / (step_ms / 1e3) / 1e9
    log(f"timed {args.steps} layer steps: {elapsed_ms:.3f} ms, {step_ms * 1e3:.2f} us per step")
    lens0 = host0.lens
    rec = {
        "metric": METRIC + " (whole decode layer: weight + KV bytes)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "steps_per_s": round(args.steps / (elapsed_ms / 1e3), 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name + "_layer", "b": wl.b, "h": h, "g": g, "d_k": d, "d_v": d, "d_model": d_model,
            "lens": list(wl.lens) if isinstance(wl.lens, (list, tuple)) else wl.lens,
            "lens_drawn_mean": float(lens0.mean()), "layer_sets": n_sets, "seed": wl.seed,
            "step_api": "gqa_decode_layer", "weight_bytes_per_step": w_bytes,
            "kv_bytes_per_step": int(kv_total / args.steps), "io_bytes_per_step": io_bytes,
        },
        "roofline": {
            "bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "gqa_decode_layer (linear_bf16_kernel, fused decode step, linear_bf16_kernel)",
            "kernel_avg_us": round(step_ms * 1e3, 3),
        },
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def bench_gscale(args, dev):
    """The long-context comparison across KV-head counts: g = 32 (MHA), 8 and 1 (MQA) on one seed.

    h = 32 query heads, b = 4, 32,768 cached positions plus the appended one,
    bf16. Each g runs the fused step on two cache sets in rotation (each set
    larger than the last-level cache): bytes read per step scale with g (the
    TF2 GQA lesson's cache-size rule), and the time ratio g = 32 : g = 1 is
    reported beside the review's "about 12x faster decoding" for MQA, which
    is a whole-decoder figure on unstated hardware (context, not a target).
    """
    import torch

    from gqa_kv_cache_decode_amd import api, inputs
    from gqa_kv_cache_decode_amd.workloads import WORKLOADS, kv_bytes_attended

    steps, warmup = max(args.steps, 5), args.warmup
    res = {}
    for g in (32, 8, 1):
        wl = WORKLOADS[f"mha_long_bf16_g{g}"]
        grow = warmup + steps + 2
        cap = wl.cap + grow
        sets = []
        for r in range(2):
            bt = inputs.Batch(seed=wl.seed + 1000 * r, b=wl.b, h=wl.h, g=wl.g, d=wl.d, cap=cap, lens=wl.lens,
                              dtype=wl.dtype, poison=False)
            to = lambda a: torch.from_numpy(a).view(torch.bfloat16).to(dev)
            sets.append({"kc": to(bt.k_cache), "vc": to(bt.v_cache), "lens": torch.from_numpy(bt.lens.copy()).to(dev),
                         "lens_h": bt.lens.copy()})
            del bt
        q = torch.from_numpy(inputs.draw_q(wl.seed, 0, wl.b, wl.h, wl.d, wl.dtype)).view(torch.bfloat16).to(dev)
        kn, vn = [torch.from_numpy(a).view(torch.bfloat16).to(dev)
                  for a in inputs.draw_new_kv(wl.seed, 0, wl.b, wl.g, wl.d, wl.d, wl.dtype)]
        out = torch.empty(wl.b, wl.h, wl.d, dtype=torch.bfloat16, device=dev)
        ws = api.make_workspace(wl.b, wl.h, wl.g, wl.d, wl.d, cap, torch.bfloat16, dev)
        stream = torch.cuda.current_stream()

        def step(i):
            st = sets[i % 2]
            api.decode_step(out, q, kn, vn, st["kc"], st["vc"], st["lens"], int(st["lens_h"].max()), wl.scale, ws)
            st["lens_h"] += 1
            return kv_bytes_attended(wl.g, wl.d, wl.d, wl.elem_bytes, st["lens_h"])

        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        total = 0
        e0.record(stream)
        for k in range(steps):
            total += step(warmup + k)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        plan_path, wgs, merge = api.plan(wl.b, wl.h, wl.g, wl.d, wl.d, cap, int(sets[0]["lens_h"].max()),
                                         torch.bfloat16)
        res[g] = {"kv_bytes_per_step": int(total / steps), "us_per_step": round(us, 2),
                  "tb_per_s": round(total / steps / (us * 1e-6) / 1e12, 3),
                  "path": {1: "vector", 2: "matrix"}[plan_path], "workgroups": wgs,
                  "split_merge": "second launch" if merge == api.MERGE_KERNEL else "in the decode kernel"}
        log(f"g={g}: {us:.1f} us per step, {res[g]['tb_per_s']} TB/s")
        del sets, ws
        torch.cuda.empty_cache()
    ratio = res[32]["us_per_step"] / res[1]["us_per_step"]
    rec = {
        "metric": "decode-step time across KV-head counts at the same shape (g = 32 / 8 / 1)",
        "value": round(ratio, 2), "unit": "x (time g=32 / time g=1)", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mha_long_bf16_g32_g8_g1", "b": 4, "h": 32, "d_k": 128, "d_v": 128,
                   "attended_len": 32769, "seed": 1005, "step_api": "gqa_decode_step"},
        "per_g": {str(g): r for g, r in res.items()},
        "bytes_ratio_g32_over_g1": round(res[32]["kv_bytes_per_step"] / res[1]["kv_bytes_per_step"], 2),
        "pages_claim": "about 12x faster decoding with multi-query attention than multi-head (Fast Transformer "
                       "Decoding review, 4.2 Speed): a whole decoder on hardware the pages do not state; context only",
    }
    print(json.dumps(rec), flush=True)


def bench_fold(args, wl, dev):
    """Mean-fold of a multi-head cache to fewer KV heads, and the output change it brings."""
    import torch

    from gqa_kv_cache_decode_amd import api, inputs
    from gqa_kv_cache_decode_amd.workloads import kv_bytes_attended

    g_dst = args.fold
    if wl.g % g_dst != 0:
        print(f"--fold {g_dst}: {wl.name} has g={wl.g}, not a multiple", file=sys.stderr)
        sys.exit(2)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    batch = inputs.Batch(seed=wl.seed, b=wl.b, h=wl.h, g=wl.g, d=wl.d, cap=wl.cap, lens=wl.lens, dtype=wl.dtype,
                         poison=False)
    L = batch.lens.copy()  # attended lengths: the drawn cache as it is

    def to_dev(a):
        t = torch.from_numpy(a)
        return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).to(dev)

    kc, vc = to_dev(batch.k_cache), to_dev(batch.v_cache)
    lens = torch.from_numpy(L.astype(np.int32)).to(dev)
    rows = int(L.max())
    q = to_dev(batch.q(0))
    del batch
    kf = torch.empty(wl.b, g_dst, wl.cap, wl.d, dtype=dt, device=dev)
    vf = torch.empty_like(kf)
    stream = torch.cuda.current_stream()

    def fold(k_dst, v_dst):
        api.fold_kv_heads(k_dst, kc, lens, rows)
        api.fold_kv_heads(v_dst, vc, lens, rows)

    for _ in range(args.warmup):
        fold(kf, vf)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        fold(kf, vf)
    t1.record(stream)
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / args.steps
    e = wl.elem_bytes
    bytes_step = 2 * (wl.g + g_dst) * int(L.sum()) * wl.d * e  # K and V: g_src rows read, g_dst written
    value = bytes_step / (step_ms / 1e3) / 1e9
    log(f"fold {wl.g} -> {g_dst}: {step_ms * 1e3:.1f} us per step (two launches)")

    # the lesson's comparison at the same cache and queries
    def attend(k, v, g):
        out = torch.empty(wl.b, wl.h, wl.d, dtype=dt, device=dev)
        ws = api.make_workspace(wl.b, wl.h, g, wl.d, wl.d, rows, dt, dev)
        api.decode_attention(out, q, k, v, lens, rows, wl.scale, ws)
        torch.cuda.synchronize()
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(10):
            api.decode_attention(out, q, k, v, lens, rows, wl.scale, ws)
        b_.record(stream)
        torch.cuda.synchronize()
        return out.float(), a.elapsed_time(b_) / 10 * 1e3

    ref, ref_us = attend(kc, vc, wl.g)
    report = {str(wl.g): {"rel_l2_change": 0.0, "decode_us": round(ref_us, 2),
                          "kv_bytes": kv_bytes_attended(wl.g, wl.d, wl.d, e, L)}}
    for g in sorted({g_dst, 1} | {x for x in (8, 4) if wl.g % x == 0 and x < wl.g}, reverse=True):
        k2 = torch.empty(wl.b, g, wl.cap, wl.d, dtype=dt, device=dev)
        v2 = torch.empty_like(k2)
        fold(k2, v2)
        out, us = attend(k2, v2, g)
        report[str(g)] = {"rel_l2_change": round(float((out - ref).norm() / ref.norm()), 4),
                          "decode_us": round(us, 2), "kv_bytes": kv_bytes_attended(g, wl.d, wl.d, e, L)}
        del k2, v2
    rec = {
        "metric": "KV-head mean-fold GB/s (bytes read + written); output change vs MHA at the same cache",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}_fold_to_g{g_dst}", "b": wl.b, "h": wl.h, "g_src": wl.g, "g_dst": g_dst,
                   "d": wl.d, "attended_len": int(L.max()), "step_api": "gqa_fold_kv_heads (K, then V)",
                   "bytes_per_step": bytes_step},
        "roofline": {"bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "fold_heads_kernel",
                     "kernel_avg_us": round(step_ms * 1e3 / 2, 3)},
        "fold_report": report,
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
