"""Timeline export and time attribution from the per-task trace.

Each trace record carries the task id, the worker it ran on, its XCC, and two
timestamps of the 100 MHz device wall clock: after its dependency wait ended
and before its trigger.  From these:

* ``to_perfetto`` writes a Chrome/Perfetto JSON timeline (one track per
  worker, one slice per task, named by operator and layer), the counterpart
  of the profiling trace the MPK demo writes (page "Mirage Persistent Kernel
  (MPK)", section 7.2, the profiling flag);
* ``attribute`` splits each worker's step into "run" (dependency met ->
  trigger: staging, compute, epilogue) and "wait" (the previous task's
  trigger -> this task's dependency met: weight prefetch issue, the event hop
  and the wait for the slowest producer), summed per operator kind;
* ``layer_split`` gives, per decoder layer, the span of the layer and the
  median task run time of each operator, i.e. how much of a layer is weight
  streaming and how much is hops and tails;
* ``buckets`` splits the gap between the launch-per-task step and the
  persistent step, and between the persistent step and the weight roofline,
  into the five buckets of the same page's attribution plan (section 8:
  launch/dispatch elimination, on-chip staging, prefetch and latency hiding,
  the weight-traffic roofline, inter-kernel L2 activation reuse), each from a
  measurement or a byte count stated with it.
"""

from __future__ import annotations

import json
from collections import defaultdict
from typing import Dict, List, Optional

import numpy as np

TICK_US = 0.01  # 100 MHz wall clock


def _kinds(tasks: np.ndarray) -> List[str]:
    from . import OP_KINDS
    return [OP_KINDS[k] for k in tasks[:, 0]]


def unwrap(clk: np.ndarray) -> np.ndarray:
    """32-bit clock samples of one step (spanning far less than 2^31 ticks)
    -> int64 ticks relative to the earliest, across a wrap of the counter."""
    c = clk.astype(np.int64)
    lo = c.min()
    c = np.where(c - lo > (1 << 31), c - (1 << 32), c)
    return c - c.min()


def _times_us(recs: np.ndarray):
    both = unwrap(np.concatenate([recs["clk_start"], recs["clk_end"]]))
    n = len(recs)
    return both[:n].astype(np.float64) * TICK_US, both[n:].astype(np.float64) * TICK_US


def to_perfetto(recs: np.ndarray, tasks: np.ndarray, path: str) -> int:
    """Write the timeline; returns the number of slices (one per record)."""
    kinds = _kinds(tasks)
    t0, t1 = _times_us(recs)
    ev = []
    for i, r in enumerate(recs):
        t = int(r["task"])
        ev.append({"name": f"{kinds[t]} L{tasks[t, 1]}", "cat": kinds[t], "ph": "X", "pid": 0,
                   "tid": int(r["worker"]), "ts": float(t0[i]), "dur": max(float(t1[i] - t0[i]), 0.01),
                   "args": {"task": t, "xcc": int(r["xcc"]), "dep_seen": int(r["dep_seen"])}})
    meta = [{"name": "thread_name", "ph": "M", "pid": 0, "tid": w, "args": {"name": f"worker {w}"}}
            for w in sorted({int(r["worker"]) for r in recs})]
    with open(path, "w") as f:
        json.dump({"traceEvents": meta + ev, "displayTimeUnit": "ns"}, f)
    return len(ev)


def attribute(recs: np.ndarray, tasks: np.ndarray) -> Dict[str, dict]:
    """Per operator kind: tasks, mean run (us), total run and wait across
    workers (us).  For every worker, run + wait over its tasks equals the time
    from the step's first start to that worker's last trigger."""
    kinds = _kinds(tasks)
    t0, t1 = _times_us(recs)
    out: Dict[str, dict] = defaultdict(lambda: {"tasks": 0, "run_us": 0.0, "wait_us": 0.0})
    by_worker = defaultdict(list)
    for i, r in enumerate(recs):
        by_worker[int(r["worker"])].append(i)
    step_begin = t0.min()
    for w, idx in by_worker.items():
        idx.sort(key=lambda i: t0[i])
        prev_end = step_begin
        for i in idx:
            k = kinds[int(recs[i]["task"])]
            d = out[k]
            d["tasks"] += 1
            d["run_us"] += t1[i] - t0[i]
            d["wait_us"] += max(t0[i] - prev_end, 0.0)
            prev_end = max(prev_end, t1[i])
    res = {}
    span = float(t1.max() - t0.min())
    for k, d in out.items():
        res[k] = {"tasks": d["tasks"], "mean_run_us": round(d["run_us"] / max(d["tasks"], 1), 3),
                  "run_us_total": round(d["run_us"], 1), "wait_us_total": round(d["wait_us"], 1)}
    res["_span_us"] = {"tasks": len(recs), "mean_run_us": 0.0, "run_us_total": round(span, 1), "wait_us_total": 0.0}
    return res


def layer_split(recs: np.ndarray, tasks: np.ndarray) -> Dict[str, float]:
    """Median over layers of: the layer's span (first start to last trigger of
    its tasks) and the sum over its operators of the median task run time."""
    kinds = _kinds(tasks)
    t0, t1 = _times_us(recs)
    per_layer = defaultdict(lambda: defaultdict(list))
    first, last = defaultdict(lambda: np.inf), defaultdict(lambda: -np.inf)
    for i, r in enumerate(recs):
        t = int(r["task"])
        l = int(tasks[t, 1])
        if l < 0:
            continue
        per_layer[l][kinds[t]].append(t1[i] - t0[i])
        first[l] = min(first[l], t0[i])
        last[l] = max(last[l], t1[i])
    spans = [last[l] - first[l] for l in per_layer]
    runs = [sum(float(np.median(v)) for v in per_layer[l].values()) for l in per_layer]
    return {"layers": len(per_layer), "layer_span_us": round(float(np.median(spans)), 2) if spans else 0.0,
            "layer_median_run_us": round(float(np.median(runs)), 2) if runs else 0.0}


def task_phases(recs: np.ndarray, tasks: np.ndarray) -> Dict[str, dict]:
    """Timing-trace records only (trace = 2, whose ticket fields hold the
    clocks of task entry and of the start of the dependency wait).  Per
    operator kind, the mean per task of four consecutive intervals on its
    worker: ``post`` (the worker's previous trigger -> this task's entry: the
    rest of the previous task after its trigger, its epilogue, and the next
    descriptor), ``issue`` (entry -> wait begins: pre-wait loads issued),
    ``wait`` (-> dependency met) and ``run`` (-> trigger).  ``_per_worker``
    holds each interval summed over a worker's tasks, averaged over workers;
    their sum is the mean over workers of the first entry -> last trigger."""
    kinds = _kinds(tasks)
    n = len(recs)
    allc = unwrap(np.concatenate([recs["t_start"], recs["t_end"], recs["clk_start"], recs["clk_end"]]))
    ent, wb, dm, tr = (allc[i * n:(i + 1) * n].astype(np.float64) * TICK_US for i in range(4))
    sums: Dict[str, np.ndarray] = defaultdict(lambda: np.zeros(5))
    by_worker = defaultdict(list)
    for i, r in enumerate(recs):
        by_worker[int(r["worker"])].append(i)
    for idx in by_worker.values():
        idx.sort(key=lambda i: ent[i])
        prev = ent[idx[0]]
        for i in idx:
            a = sums[kinds[int(recs[i]["task"])]]
            a += (1.0, ent[i] - prev, wb[i] - ent[i], dm[i] - wb[i], tr[i] - dm[i])
            prev = tr[i]
    out: Dict[str, dict] = {}
    tot = np.zeros(4)
    for k, a in sums.items():
        out[k] = {"tasks": int(a[0]), "post_us": round(a[1] / a[0], 3), "issue_us": round(a[2] / a[0], 3),
                  "wait_us": round(a[3] / a[0], 3), "run_us": round(a[4] / a[0], 3)}
        tot += a[1:]
    nw = max(len(by_worker), 1)
    out["_per_worker"] = {"tasks": n // nw, "post_us": round(tot[0] / nw, 3), "issue_us": round(tot[1] / nw, 3),
                          "wait_us": round(tot[2] / nw, 3), "run_us": round(tot[3] / nw, 3)}
    return out


def op_phases(recs: np.ndarray, tasks: np.ndarray) -> Dict[str, float]:
    """Critical path of a layer, per operator kind: the median over layers of
    the time from the previous operator's last trigger to this operator's last
    trigger, the operators of a layer taken in the order of their first
    trigger (the first operator of a layer counts from the previous layer's
    last trigger; the first layer is skipped)."""
    kinds = _kinds(tasks)
    _, t1 = _times_us(recs)
    last = defaultdict(lambda: -np.inf)
    first = defaultdict(lambda: np.inf)
    for i, r in enumerate(recs):
        t = int(r["task"])
        key = (int(tasks[t, 1]), kinds[t])
        if key[0] < 0:
            continue
        last[key] = max(last[key], t1[i])
        first[key] = min(first[key], t1[i])
    layers = sorted({l for l, _ in last})
    ph: Dict[str, list] = defaultdict(list)
    prev_end = None
    for l in layers:
        ops = sorted([k for (ll, k) in last if ll == l], key=lambda k: first[(l, k)])
        for k in ops:
            if prev_end is not None:
                ph[k].append(last[(l, k)] - prev_end)
            prev_end = last[(l, k)]
    return {k: round(float(np.median(v)), 2) for k, v in ph.items()}


def buckets(t_persistent_ms: float, t_lpt_ms: float, t_graph_ms: Optional[float], alg_bytes: float,
            act_bytes: float, stream_gbs: Optional[float], peak_gbs: float = 8000.0,
            split: Optional[Dict[str, float]] = None) -> Dict[str, dict]:
    """The five-bucket attribution, from measured step times and byte counts.

    (i)   launch/dispatch elimination: launch-per-task minus persistent, split
          into host launch cost (eager launch-per-task minus the same launches
          replayed as a HIP graph) and GPU-side kernel boundaries (graph replay
          minus persistent: dispatch and drain per kernel, activations through
          HBM between kernels, no prefetch across operators);
    (ii)  on-chip staging: not separable from these measurements (inputs are
          staged in LDS inside the task run time); reported as None;
    (iii) prefetch / latency hiding: the persistent step's time above its
          weight-roofline time, split with the layer timeline (when given)
          into weight streaming inside tasks and hops / tails between them;
    (iv)  the weight-traffic roofline: algorithmic bytes at the nominal peak
          and at the measured streaming-read rate (the floor no schedule can
          beat);
    (v)   inter-kernel L2 activation reuse: bounded by the activation bytes a
          step moves over its algorithmic bytes, i.e. the most any cache
          could save.
    """
    roof_peak = alg_bytes / (peak_gbs * 1e9) * 1e3
    roof_stream = alg_bytes / (stream_gbs * 1e9) * 1e3 if stream_gbs else None
    out = {
        "i_launch_elimination": {
            "ms": round(t_lpt_ms - t_persistent_ms, 4),
            "host_launch_ms": round(t_lpt_ms - t_graph_ms, 4) if t_graph_ms is not None else None,
            "gpu_kernel_boundaries_ms": round(t_graph_ms - t_persistent_ms, 4) if t_graph_ms is not None else None,
            "share_of_launch_per_task": round(1.0 - t_persistent_ms / t_lpt_ms, 4)},
        "ii_onchip_staging": {"ms": None, "note": "inside task run time; not separable without counters"},
        "iii_prefetch_latency": {"ms_above_stream_roofline": round(t_persistent_ms - roof_stream, 4)
                                 if roof_stream else None,
                                 "ms_above_peak_roofline": round(t_persistent_ms - roof_peak, 4)},
        "iv_weight_roofline": {"ms_at_peak": round(roof_peak, 4),
                               "ms_at_stream_rate": round(roof_stream, 4) if roof_stream else None,
                               "persistent_over_peak": round(t_persistent_ms / roof_peak, 3)},
        "v_l2_activation_reuse": {"activation_bytes": int(act_bytes),
                                  "bound_share_of_step": round(act_bytes / alg_bytes, 5)},
    }
    if split:
        span, run = split["layer_span_us"], split["layer_median_run_us"]
        out["iii_prefetch_latency"]["layer_span_us"] = span
        out["iii_prefetch_latency"]["layer_run_us"] = run
        out["iii_prefetch_latency"]["layer_hops_and_tails_us"] = round(span - run, 2)
    return out
