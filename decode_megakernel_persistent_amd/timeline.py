"""Timeline export and time attribution from the per-task trace.

Each trace record carries the task id, the worker it ran on, its XCC, and two
timestamps of the 100 MHz device wall clock: after its dependency wait ended
and before its trigger.  From these:

* ``to_perfetto`` writes a Chrome/Perfetto JSON timeline (one track per
  worker, one slice per task, coloured by operator), the counterpart of the
  profiling trace the MPK demo writes (page "Mirage Persistent Kernel (MPK)",
  section 7.2, the --profiling flag);
* ``attribute`` splits each worker's step time into "run" (dependency met ->
  trigger: staging, compute, epilogue) and "wait" (previous trigger -> this
  task's dependency met: weight prefetch issue plus waiting on the event),
  summed per operator kind.
"""

from __future__ import annotations

import json
from collections import defaultdict
from typing import Dict

import numpy as np

TICK_US = 0.01  # 100 MHz wall clock


def _kinds(tasks: np.ndarray):
    from . import OP_KINDS
    return [OP_KINDS[k] for k in tasks[:, 0]]


def _unwrap(clk: np.ndarray) -> np.ndarray:
    """32-bit clock samples of one step -> int64 ticks relative to the earliest."""
    c = clk.astype(np.int64)
    lo = c.min()
    c = np.where(c - lo > (1 << 31), c - (1 << 32), c)
    return c - c.min()


def to_perfetto(recs: np.ndarray, tasks: np.ndarray, path: str) -> None:
    kinds = _kinds(tasks)
    both = _unwrap(np.concatenate([recs["clk_start"], recs["clk_end"]]))
    n = len(recs)
    t0, t1 = both[:n], both[n:]
    ev = []
    for i, r in enumerate(recs):
        t = int(r["task"])
        ev.append({"name": f"{kinds[t]} L{tasks[t, 1]}", "cat": kinds[t], "ph": "X", "pid": 0,
                   "tid": int(r["worker"]), "ts": float(t0[i]) * TICK_US,
                   "dur": max(float(t1[i] - t0[i]) * TICK_US, 0.01),
                   "args": {"task": t, "xcc": int(r["xcc"]), "dep_seen": int(r["dep_seen"])}})
    with open(path, "w") as f:
        json.dump({"traceEvents": ev, "displayTimeUnit": "us"}, f)


def attribute(recs: np.ndarray, tasks: np.ndarray) -> Dict[str, dict]:
    """Per operator kind: tasks, mean run (us), total run and wait across workers (us)."""
    kinds = _kinds(tasks)
    both = _unwrap(np.concatenate([recs["clk_start"], recs["clk_end"]]))
    n = len(recs)
    t0, t1 = both[:n].astype(np.float64) * TICK_US, both[n:].astype(np.float64) * TICK_US
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
            prev_end = t1[i]
    res = {}
    span = float(t1.max() - t0.min())
    for k, d in out.items():
        res[k] = {"tasks": d["tasks"], "mean_run_us": round(d["run_us"] / max(d["tasks"], 1), 3),
                  "run_us_total": round(d["run_us"], 1), "wait_us_total": round(d["wait_us"], 1)}
    res["_span_us"] = {"tasks": n, "mean_run_us": 0.0, "run_us_total": round(span, 1), "wait_us_total": 0.0}
    return res
