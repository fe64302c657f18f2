#!/usr/bin/env python3
"""Decode-step benchmark of the persistent megakernel on one MI355X.

    python bench.py [--gpus 1] [--steps 32] [--warmup 2] [--workload qwen3-8b]

One step is one full decode step of the workload (embedding, every layer's
RMSNorm/QKV/QK-norm+RoPE+KV-append/attention/merge/O/SwiGLU MLP or routed
experts, final norm and lm_head) on synthetic inputs already resident in HBM.
Prints one JSON line: ms/token (median over the timed steps, mean beside it;
per-step HIP events on the stream the worker kernel is launched on) and the
algorithmic HBM bandwidth of the step (weights read -- for routed experts the
distinct experts the GPU chose, read back per step -- plus KV read, KV
written and logits, over the step time) against MI355X's 8 TB/s peak and the
box's measured streaming-read rate; the same step in launch-per-task mode,
eager and replayed as a HIP graph; greedy steps in one launch; the paged KV
layout; and the oracle's ms/token on the host cores over a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "mk_worker_qwen3-8b_b1_traffic.txt")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kv_bytes(shape, batch: int, positions: np.ndarray) -> float:
    """KV read (positions 0..p of each sequence and layer) plus KV written."""
    s = shape
    kv_row = 2 * s.n_kv_heads * s.head_dim * 2  # K and V of one position, one layer
    return float(sum(int(p) + 1 for p in positions) * kv_row * s.n_layers + batch * kv_row * s.n_layers)


def algorithmic_bytes(shape, batch: int, positions: np.ndarray, weight_bytes: float) -> float:
    """Bytes one step must move: weights read, embedding rows, norm gains, KV
    read and written, logits."""
    s = shape
    gains = s.n_layers * (2 * s.hidden + 2 * s.head_dim) * 4 + s.hidden * 4
    embed = batch * s.hidden * 2
    logits = batch * s.vocab * 4
    return float(weight_bytes + embed + gains + kv_bytes(s, batch, positions) + logits)


def expert_bytes(shape, experts: np.ndarray) -> float:
    """Weight bytes of the distinct routed experts chosen in each layer
    (experts [L][B][top_k] from the GPU's routing record)."""
    per_expert = 3 * shape.expert_intermediate * shape.hidden * 2
    return float(sum(len(np.unique(experts[l])) for l in range(experts.shape[0])) * per_expert)


def time_steps(sess, tok_dev, pos0: np.ndarray, warmup: int, steps: int, routed: bool = False, noalloc=False):
    """Per-step HIP events on the stream the step is launched on (the
    session's stream is torch's current stream), bracketing exactly the
    decode_step enqueue; token/position copies sit outside.  Routed models
    synchronise after each step to read the GPU's expert choice (the events
    still time only the launch)."""
    import torch
    import decode_megakernel_persistent_amd as mk
    st = torch.cuda.current_stream()
    pos = torch.as_tensor(pos0.astype(np.int32), device=sess.device)
    pos_list, experts = [], []
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]

    def enqueue():
        if noalloc:
            mk.mk_decode_step_noalloc(sess.g, sess.tokens.data_ptr(), sess.positions.data_ptr(), sess.kv,
                                      sess.logits.data_ptr(), sess.stream)
        else:
            sess.enqueue()
    torch.cuda.synchronize()
    for i in range(warmup):
        sess.tokens.copy_(tok_dev[i % tok_dev.shape[0]])
        sess.positions.copy_(pos + i)
        enqueue()
    torch.cuda.synchronize()
    sess.check()
    t0 = time.perf_counter()
    for i in range(steps):
        k = warmup + i
        sess.tokens.copy_(tok_dev[k % tok_dev.shape[0]])
        sess.positions.copy_(pos + k)
        pos_list.append(pos0 + k)
        ev[i][0].record(st)
        enqueue()
        ev[i][1].record(st)
        if routed:
            torch.cuda.synchronize()
            experts.append(sess.read_routing(0, with_logits=False)[0])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sess.check()
    times = [a.elapsed_time(b) for a, b in ev]
    return times, pos_list, experts, wall


def stream_probe(gib: float = 4.0, reps: int = 5) -> float:
    """The box's streaming-read rate (GB/s): a plain 16-byte-load read of a
    buffer far larger than the caches, median of `reps` timed reads."""
    import torch
    import decode_megakernel_persistent_amd as mk
    n = int(gib * (1 << 30))
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    blocks = 256 * 8
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    times = []
    for r in range(reps + 1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        mk.mk_stream_read(buf.data_ptr(), n, sink.data_ptr(), blocks, st.cuda_stream)
        b.record(st)
        torch.cuda.synchronize()
        if r:
            times.append(a.elapsed_time(b))
    del buf
    torch.cuda.empty_cache()
    return n / (statistics.median(times) * 1e-3) / 1e9


def calibrate_copy(mib: int, reps: int = 3) -> None:
    """Plain device-to-device copies of a known size (each reads and writes
    `mib` MiB once) for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration copies: {reps} x {mib} MiB read + {mib} MiB written")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, weights, kv_k, kv_v, tokens0, pos0, budget_s: float):
    """The oracle (as it stands) on the host cores: whole decode steps of the
    same workload until about `budget_s` seconds of CPU work have run."""
    import oracle
    orc = oracle.Oracle(w.shape, w.batch, w.capacity, threads=0)
    orc.set_weights(weights)
    orc.K[...] = kv_k
    orc.V[...] = kv_v
    n, t0 = 0, time.perf_counter()
    while True:
        orc.decode(tokens0, pos0 + n)
        n += 1
        if time.perf_counter() - t0 >= budget_s or n >= 32:
            break
    el = time.perf_counter() - t0
    threads = orc.threads
    orc.close()
    return el * 1000.0 / (n * w.batch), n, threads


def activation_bytes(sess) -> float:
    """Bytes of inter-task activations one step writes and reads back (the
    scratch past the event state, written once and read once at least)."""
    return 2.0 * float(sess.stats.scratch_bytes)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="qwen3-8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-lpt", action="store_true")
    ap.add_argument("--multi-steps", type=int, default=16,
                    help="also time mk_decode_steps with this many greedy steps per launch (0 = skip)")
    ap.add_argument("--paged", type=int, default=16, metavar="PAGE",
                    help="also time the step on a paged KV cache with this page size (0 = skip)")
    ap.add_argument("--no-stream-probe", action="store_true")
    ap.add_argument("--attribution", action="store_true",
                    help="also run one step with the timing trace: per-layer split and the five-bucket attribution")
    ap.add_argument("--timeline-json", default="", help="with --attribution: write the Perfetto timeline here")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--profile-only", action="store_true", help="one mode's steps only (for profilers)")
    ap.add_argument("--profile-mode", choices=["persistent", "lpt"], default="persistent")
    ap.add_argument("--lds-ring", action="store_true",
                    help="batch-1 GEMV tiles fed through the LDS weight ring instead of registers")
    ap.add_argument("--no-watchdog", action="store_true",
                    help="launch no dispatch wavefront (for counter runs, which serialise dispatches)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after the steps, run plain copies of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the decoder runs on one GPU only (no sharding or collectives); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import dataclasses
    import synth
    import decode_megakernel_persistent_amd as mk
    from decode_megakernel_persistent_amd import timeline

    base = synth.WORKLOADS[args.workload]
    # capacity for every position the run writes
    w = dataclasses.replace(base, steps=args.warmup + args.steps + max(args.multi_steps, 0))
    s = w.shape
    routed = s.n_experts > 0
    t_setup = time.perf_counter()
    weights = synth.weights(s)
    lens = synth.lengths(w)
    L, B, Hkv, cap, D = s.n_layers, w.batch, s.n_kv_heads, w.capacity, s.head_dim
    kv_k = np.zeros((L, B, Hkv, cap, D), dtype=np.uint16)
    kv_v = np.zeros_like(kv_k)
    # random cache entries stand in for the tiny workload's oracle-prefilled prompt
    synth.fill_kv(s, B, cap, lens, kv_k, kv_v)
    ntok = args.warmup + args.steps
    toks = synth.tokens(w, ntok)  # [B, ntok]
    log(f"inputs ready in {time.perf_counter() - t_setup:.1f}s")

    mode = mk.MK_LAUNCH_PER_TASK if args.profile_only and args.profile_mode == "lpt" else mk.MK_PERSISTENT
    sess = mk.Session(s, B, cap, mk.make_opts(mode=mode, no_watchdog=int(args.no_watchdog), lds_ring=int(args.lds_ring)))
    sess.load(weights)
    sess.set_kv(kv_k, kv_v)
    tok_dev = torch.as_tensor(toks.T.copy(), device=sess.device)  # [ntok, B]
    pos0 = lens.astype(np.int64)
    log(f"graph: {sess.stats.tasks} tasks, {sess.stats.events} events, {sess.stats.workers} workers; "
        f"loaded in {time.perf_counter() - t_setup:.1f}s")

    times, pos_list, experts, wall = time_steps(sess, tok_dev, pos0, args.warmup, args.steps, routed)
    med = statistics.median(times)
    mean = statistics.fmean(times)
    wbytes = [float(sess.stats.weight_bytes) + (expert_bytes(s, e) if routed else 0.0)
              for e in (experts if routed else [None] * len(pos_list))]
    bytes_steps = [algorithmic_bytes(s, B, p, wb) for p, wb in zip(pos_list, wbytes)]
    bytes_mean = statistics.fmean(bytes_steps)
    # algorithmic bytes per launch / the average launch duration (the rocprofv3 figure)
    achieved = bytes_mean / (mean * 1e-3) / 1e9
    achieved_med = bytes_mean / (med * 1e-3) / 1e9
    log(f"{'launch-per-task' if mode else 'persistent'}: median {med:.4f} ms/step, mean {mean:.4f}, "
        f"{achieved:.0f} GB/s ({bytes_mean / 1e9:.3f} GB/step), wall {wall:.3f}s for {args.steps} steps")
    if args.profile_only:
        sess.close()
        if args.calibrate_copy:
            calibrate_copy(args.calibrate_copy)
        log("profile run done")
        return

    stream_gbs = None
    if not args.no_stream_probe:
        stream_gbs = stream_probe()
        log(f"streaming read probe: {stream_gbs:.0f} GB/s")

    noalloc = None
    if sess.stats.scratch_bytes <= 64 << 20:
        sess.set_kv(kv_k, kv_v)
        t_n, _, _, _ = time_steps(sess, tok_dev, pos0, args.warmup, args.steps, False, noalloc=True)
        noalloc = {"median_ms_per_step": round(statistics.median(t_n), 4), "ms_per_step": round(statistics.fmean(t_n), 4)}
        log(f"static-scratch step (mk_decode_step_noalloc): median {noalloc['median_ms_per_step']:.4f} ms")

    lpt = None
    if not args.no_lpt:
        sess.set_kv(kv_k, kv_v)
        sess.set_mode(mk.MK_LAUNCH_PER_TASK)
        t_l, _, _, _ = time_steps(sess, tok_dev, pos0, args.warmup, args.steps, False)
        med_l, mean_l = statistics.median(t_l), statistics.fmean(t_l)
        lpt = {"median_ms_per_step": round(med_l, 4), "ms_per_step": round(mean_l, 4),
               "launches_per_step": int(sess.stats.launches_per_step),
               "persistent_speedup": round(med_l / med, 3),
               "overhead_share": round(1.0 - med / med_l, 4)}
        log(f"launch-per-task: median {med_l:.4f} ms/step")
        # the same launches captured once into a HIP graph and replayed: what
        # remains of the gap to the persistent kernel is not host launch cost
        h = sess.capture_lpt_graph()
        st = torch.cuda.current_stream()
        pos_t = torch.as_tensor(pos0.astype(np.int32), device=sess.device)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.warmup + args.steps)]
        for i in range(args.warmup + args.steps):
            sess.tokens.copy_(tok_dev[i % tok_dev.shape[0]])
            sess.positions.copy_(pos_t + i)
            ev[i][0].record(st)
            sess.replay_lpt_graph(h)
            ev[i][1].record(st)
        torch.cuda.synchronize()
        sess.check()
        t_g = [a.elapsed_time(b) for a, b in ev[args.warmup:]]
        lpt["graph_median_ms_per_step"] = round(statistics.median(t_g), 4)
        lpt["graph_persistent_speedup"] = round(statistics.median(t_g) / med, 3)
        log(f"launch-per-task as a HIP graph: median {statistics.median(t_g):.4f} ms/step")
        sess.set_mode(mk.MK_PERSISTENT)

    multi = None
    n_multi = min(args.multi_steps, cap - int(pos0.max()))
    if n_multi > 1:
        # the whole greedy loop on the device: n_multi steps per launch, tokens
        # fed back from the lm_head argmax; events bracket only the launch
        sess.set_kv(kv_k, kv_v)
        sess.tokens.copy_(tok_dev[0])
        sess.positions.copy_(torch.as_tensor(pos0.astype(np.int32), device=sess.device))
        out_tok = torch.empty((n_multi, B), dtype=torch.int32, device=sess.device)
        st = torch.cuda.current_stream()
        reps = 4
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps + 1)]
        for r in range(reps + 1):  # the first launch is a warmup
            ev[r][0].record(st)
            mk.mk_decode_steps(sess.g, sess.tokens.data_ptr(), sess.positions.data_ptr(), sess.kv,
                               sess.logits.data_ptr(), out_tok.data_ptr(), n_multi, sess.stream)
            ev[r][1].record(st)
        torch.cuda.synchronize()
        sess.check()
        t_m = [a.elapsed_time(b) for a, b in ev[1:]]
        per = statistics.median(t_m) / n_multi
        multi = {"steps_per_launch": n_multi, "launches": reps, "median_ms_per_step": round(per, 4),
                 "ms_per_token": round(per / B, 4), "tokens_per_s": round(B * 1000.0 / per, 2),
                 "speedup_vs_one_step_launches": round(med / per, 4)}
        log(f"multi-step: {n_multi} steps per launch, {per:.4f} ms/step")

    attribution = None
    if args.attribution:
        # one step with the timing trace (clocks only, one record per task)
        tr = mk.Session(s, B, cap, mk.make_opts(trace=2, lds_ring=int(args.lds_ring)))
        tr.load(weights)
        tr.set_kv(kv_k, kv_v)
        for i in range(2):
            tr.step(toks[:, i], pos0 + i)
            torch.cuda.synchronize()
            tr.check()
        recs = tr.read_trace()
        tasks = mk.mk_get_tasks(tr.g)
        if args.timeline_json:
            timeline.to_perfetto(recs, tasks, args.timeline_json)
        split = timeline.layer_split(recs, tasks)
        per_op = timeline.attribute(recs, tasks)
        phases = timeline.task_phases(recs, tasks)
        crit = timeline.op_phases(recs, tasks)
        tr.close()
        attribution = {
            "layer_split": split,
            "per_operator": {k: v for k, v in per_op.items()},
            "task_phases": {k: {kk: (int(vv) if kk == "tasks" else float(vv)) for kk, vv in v.items()}
                            for k, v in phases.items()},
            "layer_critical_path_us": crit,
            "buckets": timeline.buckets(med, lpt["median_ms_per_step"] if lpt else med,
                                        lpt["graph_median_ms_per_step"] if lpt else None,
                                        bytes_mean, activation_bytes(sess), stream_gbs, HBM_PEAK_GBS, split)}
        log("attribution: " + json.dumps(attribution["buckets"]))

    paged = None
    if args.paged:
        ps = mk.Session(s, B, cap, mk.make_opts(lds_ring=int(args.lds_ring)), page_size=args.paged, spare_pages=B, page_seed=1)
        ps.load(weights)
        ps.set_kv(kv_k, kv_v)
        t_p, _, _, _ = time_steps(ps, tok_dev, pos0, args.warmup, args.steps, False)
        paged = {"page_size": args.paged, "median_ms_per_step": round(statistics.median(t_p), 4),
                 "contiguous_median_ms_per_step": round(med, 4),
                 "paged_over_contiguous": round(statistics.median(t_p) / med, 4)}
        log(f"paged KV ({args.paged}-row pages): median {statistics.median(t_p):.4f} ms/step")
        ps.close()
        del ps

    traffic = None
    if os.path.exists(PROFILE_TRAFFIC) and args.workload == "qwen3-8b" and B == 1:
        from decode_megakernel_persistent_amd import profsum
        prof = profsum.read_kv(PROFILE_TRAFFIC)
        # counters taken on the kernels as they are now, else null
        if prof.get("source_hash") == mk.source_hash():
            traffic = int(float(prof["traffic_bytes_per_launch"]))

    stats = sess.stats
    sess.close()
    cpu = None
    if not args.no_cpu_baseline:
        del tok_dev
        torch.cuda.empty_cache()
        ms_cpu, n_cpu, threads = cpu_baseline(w, weights, kv_k, kv_v, toks[:, 0], pos0, args.cpu_budget)
        cpu = {"value": round(ms_cpu, 2), "unit": "ms/token", "cores": int(threads), "kind": "oracle",
               "cpu_model": cpu_model(),
               "sample": f"{n_cpu} whole decode steps of the same workload (batch {B}) on the host, fp64 oracle"}

    ctx = int(lens.max())
    out = {
        "metric": "decode ms/token and weight-stream HBM GB/s vs peak, batch 1 (1 GPU)",
        "value": round(med / B, 4),
        "unit": "ms/token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med, 4),
        "mean_ms_per_step": round(mean, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}-shaped decoder, batch {B}, KV context {ctx}"
                               + (" (ragged)" if w.ragged else ""),
                   "batch": B, "context": ctx, "layers": s.n_layers, "hidden": s.hidden,
                   "mode": "persistent", "workers": int(stats.workers)},
        "hbm_gbps": round(achieved, 1),
        "hbm_frac_of_peak": round(achieved / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": round(bytes_mean), "kernel": "mk_worker",
                     "launch_ms_mean": round(mean, 4), "achieved_at_median": round(achieved_med, 1),
                     "stream_probe_gbs": round(stream_gbs, 1) if stream_gbs else None,
                     "frac_of_stream_probe": round(achieved / stream_gbs, 4) if stream_gbs else None},
        "launch_per_task": lpt,
        "multi_step": multi,
        "static_scratch_step": noalloc,
        "paged_kv": paged,
        "attribution": attribution,
        "cpu_baseline": cpu,
        "tokens_per_s": round(B * 1000.0 / med, 2),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
