#!/usr/bin/env python3
"""Decode-step benchmark of the persistent megakernel on one MI355X.

    python bench.py [--gpus 1] [--steps 32] [--warmup 2] [--workload qwen3-8b]

One step is one full decode step of the workload (embedding, every layer's
RMSNorm/QKV/QK-norm+RoPE+KV-append/attention/merge/O/SwiGLU MLP, final norm
and lm_head) on synthetic inputs already resident in HBM.  Prints one JSON
line: ms/token (mean over the timed steps, per-step HIP events on the
launching stream) and the algorithmic HBM bandwidth of the step (weights read
+ KV read + KV written + logits, divided by the step time) against MI355X's
8 TB/s peak, the same step in launch-per-task mode, and the oracle's ms/token
on the host cores over a bounded sample.
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




def algorithmic_bytes(shape, batch: int, positions: np.ndarray, weight_bytes: int) -> float:
    """Bytes one step must move: weights read, embedding rows, norm gains,
    KV read (positions 0..p for each sequence and layer), KV written, logits."""
    s = shape
    kv_row = 2 * s.n_kv_heads * s.head_dim * 2  # K and V of one position, one layer
    kv_read = sum(int(p) + 1 for p in positions) * kv_row * s.n_layers
    kv_write = batch * kv_row * s.n_layers
    gains = s.n_layers * (2 * s.hidden + 2 * s.head_dim) * 4 + s.hidden * 4
    embed = batch * s.hidden * 2
    logits = batch * s.vocab * 4
    return float(weight_bytes + embed + gains + kv_read + kv_write + logits)


def time_steps(sess, tok_dev, pos0: np.ndarray, warmup: int, steps: int):
    """Per-step HIP events on the stream the step is launched on (the
    session's stream is torch's current stream), bracketing exactly the
    decode_step enqueue; the next step's token/position copies sit outside."""
    import torch
    st = torch.cuda.current_stream()
    pos = torch.as_tensor(pos0.astype(np.int32), device=sess.device)
    pos_list = []
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(warmup):
        sess.tokens.copy_(tok_dev[i % tok_dev.shape[0]])
        sess.positions.copy_(pos + i)
        sess.enqueue()
    torch.cuda.synchronize()
    sess.check()
    t0 = time.perf_counter()
    for i in range(steps):
        k = warmup + i
        sess.tokens.copy_(tok_dev[k % tok_dev.shape[0]])
        sess.positions.copy_(pos + k)
        pos_list.append(pos0 + k)
        ev[i][0].record(st)
        sess.enqueue()
        ev[i][1].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sess.check()
    times = [a.elapsed_time(b) for a, b in ev]
    return times, pos_list, wall


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
    print(f"[bench] calibration copies: {reps} x {mib} MiB read + {mib} MiB written", file=sys.stderr, flush=True)


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
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--profile-only", action="store_true", help="persistent steps only (for profilers)")
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

    base = synth.WORKLOADS[args.workload]
    # capacity for every position the run writes
    w = dataclasses.replace(base, steps=args.warmup + args.steps)
    s = w.shape
    t_setup = time.perf_counter()
    weights = synth.weights(s)
    lens = synth.lengths(w)
    L, B, Hkv, cap, D = s.n_layers, w.batch, s.n_kv_heads, w.capacity, s.head_dim
    kv_k = np.zeros((L, B, Hkv, cap, D), dtype=np.uint16)
    kv_v = np.zeros_like(kv_k)
    if w.prompt:
        # the tiny workload's prompt is prefilled by the oracle in the parity
        # tests; for timing, random cache entries of the same length stand in
        synth.fill_kv(s, B, cap, lens, kv_k, kv_v)
    else:
        synth.fill_kv(s, B, cap, lens, kv_k, kv_v)
    ntok = args.warmup + args.steps
    toks = synth.tokens(w, ntok)  # [B, ntok]
    print(f"[bench] inputs ready in {time.perf_counter() - t_setup:.1f}s", file=sys.stderr, flush=True)

    sess = mk.Session(s, B, cap, mk.make_opts(mode=mk.MK_PERSISTENT, no_watchdog=int(args.no_watchdog)))
    sess.load(weights)
    sess.set_kv(kv_k, kv_v)
    tok_dev = torch.as_tensor(toks.T.copy(), device=sess.device)  # [ntok, B]
    pos0 = lens.astype(np.int64)
    print(f"[bench] graph: {sess.stats.tasks} tasks, {sess.stats.events} events, "
          f"{sess.stats.workers} workers; loaded in {time.perf_counter() - t_setup:.1f}s", file=sys.stderr, flush=True)

    times, pos_list, wall = time_steps(sess, tok_dev, pos0, args.warmup, args.steps)
    med = statistics.median(times)
    mean = statistics.fmean(times)
    bytes_steps = [algorithmic_bytes(s, B, p, sess.stats.weight_bytes) for p in pos_list]
    bytes_mean = statistics.fmean(bytes_steps)
    # algorithmic bytes per launch / the average launch duration
    achieved = bytes_mean / (mean * 1e-3) / 1e9
    print(f"[bench] persistent: mean {mean:.4f} ms/step, median {med:.4f}, {achieved:.0f} GB/s "
          f"({bytes_mean / 1e9:.3f} GB/step), wall {wall:.3f}s for {args.steps} steps", file=sys.stderr, flush=True)
    if args.profile_only:
        sess.close()
        if args.calibrate_copy:
            calibrate_copy(args.calibrate_copy)
        print("[bench] profile run done", file=sys.stderr, flush=True)
        return

    lpt = None
    if not args.no_lpt:
        sess.set_kv(kv_k, kv_v)
        sess.set_mode(mk.MK_LAUNCH_PER_TASK)
        t_l, _, _ = time_steps(sess, tok_dev, pos0, args.warmup, args.steps)
        mean_l = statistics.fmean(t_l)
        lpt = {"ms_per_step": round(mean_l, 4), "median_ms": round(statistics.median(t_l), 4),
               "launches_per_step": int(sess.stats.launches_per_step),
               "persistent_speedup": round(mean_l / mean, 3),
               "overhead_share": round(1.0 - mean / mean_l, 4)}
        print(f"[bench] launch-per-task: mean {mean_l:.4f} ms/step", file=sys.stderr, flush=True)
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
        mean_g = statistics.fmean(t_g)
        lpt["graph_ms_per_step"] = round(mean_g, 4)
        lpt["graph_persistent_speedup"] = round(mean_g / mean, 3)
        print(f"[bench] launch-per-task as a HIP graph: mean {mean_g:.4f} ms/step", file=sys.stderr, flush=True)
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
        per = statistics.fmean(t_m) / n_multi
        multi = {"steps_per_launch": n_multi, "launches": reps, "ms_per_step": round(per, 4),
                 "ms_per_token": round(per / B, 4), "tokens_per_s": round(B * 1000.0 / per, 2),
                 "speedup_vs_one_step_launches": round(mean / per, 4)}
        print(f"[bench] multi-step: {n_multi} steps per launch, {per:.4f} ms/step", file=sys.stderr, flush=True)

    traffic = None
    if os.path.exists(PROFILE_TRAFFIC) and args.workload == "qwen3-8b" and B == 1:
        from decode_megakernel_persistent_amd import profsum
        prof = profsum.read_kv(PROFILE_TRAFFIC)
        # counters taken on the kernels as they are now, else null
        if prof.get("source_hash") == mk.source_hash():
            traffic = int(float(prof["traffic_bytes_per_launch"]))

    cpu = None
    if not args.no_cpu_baseline:
        sess.close()
        del tok_dev
        torch.cuda.empty_cache()
        ms_cpu, n_cpu, threads = cpu_baseline(w, weights, kv_k, kv_v, toks[:, 0], pos0, args.cpu_budget)
        cpu = {"value": round(ms_cpu, 2), "unit": "ms/token", "cores": int(threads), "kind": "oracle",
               "sample": f"{n_cpu} whole decode steps of the same workload (batch {B}) on the host, fp64 oracle"}
    else:
        sess.close()

    out = {
        "metric": "decode ms/token and weight-stream HBM GB/s vs peak, batch 1 (1 GPU)",
        "value": round(mean / B, 4),
        "unit": "ms/token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean, 4),
        "median_ms_per_step": round(med, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}-shaped decoder, batch {B}, KV context {int(lens.max())}",
                   "batch": B, "context": int(lens.max()), "layers": s.n_layers, "hidden": s.hidden,
                   "mode": "persistent", "workers": int(sess.stats.workers)},
        "hbm_gbps": round(achieved, 1),
        "hbm_frac_of_peak": round(achieved / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": round(bytes_mean), "kernel": "mk_worker",
                     "launch_ms": round(mean, 4)},
        "launch_per_task": lpt,
        "multi_step": multi,
        "cpu_baseline": cpu,
        "tokens_per_s": round(B * 1000.0 / mean, 2),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
