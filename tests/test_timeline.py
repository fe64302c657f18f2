"""Timeline export and attribution (decode_megakernel_persistent_amd.timeline)
on synthetic trace records, on the CPU: one Perfetto slice per task at the
right place across a wrap of the 32-bit device clock, per-worker run + wait
equal to that worker's span, the per-layer split, and the bucket arithmetic."""

import json

import numpy as np
import pytest

import decode_megakernel_persistent_amd as mk
from decode_megakernel_persistent_amd import timeline

K = {k: i for i, k in enumerate(mk.OP_KINDS)}


def _records(rows):
    """rows: (task, worker, clk_start, clk_end) in ticks."""
    recs = np.zeros(len(rows), dtype=mk.TRACE_DTYPE)
    for i, (t, w, a, b) in enumerate(rows):
        recs[i]["task"], recs[i]["worker"] = t, w
        recs[i]["clk_start"], recs[i]["clk_end"] = a % (1 << 32), b % (1 << 32)
    return recs


# task table rows: {op_kind, layer, dep, trig, a0..a3}
TASKS = np.array([[K["qkv"], 0, -1, 0, 0, 0, 0, 0],
                  [K["qkv"], 0, -1, 0, 1, 0, 0, 0],
                  [K["attn"], 0, 0, 1, 0, 0, 0, 0],
                  [K["oproj"], 0, 1, 2, 0, 0, 0, 0],
                  [K["qkv"], 1, 2, 3, 0, 0, 0, 0],
                  [K["oproj"], 1, 3, -1, 0, 0, 0, 0]], dtype=np.int32)
BASE = (1 << 32) - 250  # the device clock wraps inside the step
ROWS = [(0, 0, BASE + 0, BASE + 100), (1, 1, BASE + 10, BASE + 90),
        (2, 1, BASE + 150, BASE + 300), (3, 0, BASE + 320, BASE + 400),
        (4, 1, BASE + 450, BASE + 600), (5, 0, BASE + 650, BASE + 700)]


def test_unwrap_keeps_order_across_the_clock_wrap():
    recs = _records(ROWS)
    t0, t1 = timeline._times_us(recs)
    np.testing.assert_allclose(t0, np.array([0, 10, 150, 320, 450, 650]) * timeline.TICK_US)
    np.testing.assert_allclose(t1, np.array([100, 90, 300, 400, 600, 700]) * timeline.TICK_US)


def test_perfetto_has_one_slice_per_task_on_its_worker(tmp_path):
    recs = _records(ROWS)
    p = str(tmp_path / "t.json")
    assert timeline.to_perfetto(recs, TASKS, p) == len(ROWS)
    d = json.load(open(p))
    sl = [e for e in d["traceEvents"] if e["ph"] == "X"]
    assert sorted(e["args"]["task"] for e in sl) == list(range(len(ROWS)))
    by_task = {e["args"]["task"]: e for e in sl}
    assert by_task[2]["tid"] == 1 and by_task[2]["name"] == "attn L0"
    assert by_task[2]["ts"] == pytest.approx(1.5) and by_task[2]["dur"] == pytest.approx(1.5)
    # slices of one worker do not overlap
    for w in (0, 1):
        mine = sorted((e["ts"], e["ts"] + e["dur"]) for e in sl if e["tid"] == w)
        assert all(a[1] <= b[0] for a, b in zip(mine, mine[1:]))


def test_run_plus_wait_is_each_workers_span():
    recs = _records(ROWS)
    att = timeline.attribute(recs, TASKS)
    run = sum(v["run_us_total"] for k, v in att.items() if k != "_span_us")
    wait = sum(v["wait_us_total"] for k, v in att.items() if k != "_span_us")
    # worker 0 ends at 700, worker 1 at 600 (ticks from the step's first start)
    assert run + wait == pytest.approx((700 + 600) * timeline.TICK_US)
    assert att["qkv"]["tasks"] == 3 and att["oproj"]["tasks"] == 2
    assert att["qkv"]["run_us_total"] == pytest.approx((100 + 80 + 150) * timeline.TICK_US)
    assert att["_span_us"]["run_us_total"] == pytest.approx(7.0)


def test_layer_split():
    recs = _records(ROWS)
    sp = timeline.layer_split(recs, TASKS)
    assert sp["layers"] == 2
    # layer 0 spans 0..400 ticks, layer 1 450..700: median 325 ticks
    assert sp["layer_span_us"] == pytest.approx(3.25)
    # layer 0 run: qkv median 90, attn 150, oproj 80 -> 320; layer 1: 150 + 50 -> 200
    assert sp["layer_median_run_us"] == pytest.approx(2.6)


def test_bucket_arithmetic():
    b = timeline.buckets(t_persistent_ms=3.0, t_lpt_ms=7.5, t_graph_ms=7.4, alg_bytes=16e9, act_bytes=48e6,
                         stream_gbs=6400.0, split={"layer_span_us": 89.0, "layer_median_run_us": 55.0})
    assert b["i_launch_elimination"]["ms"] == pytest.approx(4.5)
    assert b["i_launch_elimination"]["host_launch_ms"] == pytest.approx(0.1)
    assert b["i_launch_elimination"]["gpu_kernel_boundaries_ms"] == pytest.approx(4.4)
    assert b["i_launch_elimination"]["share_of_launch_per_task"] == pytest.approx(0.6)
    assert b["iv_weight_roofline"]["ms_at_peak"] == pytest.approx(2.0)
    assert b["iv_weight_roofline"]["ms_at_stream_rate"] == pytest.approx(2.5)
    assert b["iii_prefetch_latency"]["ms_above_stream_roofline"] == pytest.approx(0.5)
    assert b["iii_prefetch_latency"]["layer_hops_and_tails_us"] == pytest.approx(34.0)
    assert b["v_l2_activation_reuse"]["bound_share_of_step"] == pytest.approx(0.003)
    assert b["ii_onchip_staging"]["ms"] is None


def _timing_records(rows):
    """rows: (task, worker, entry, wait_begin, dep_met, trigger) in ticks."""
    recs = np.zeros(len(rows), dtype=mk.TRACE_DTYPE)
    for i, (t, w, e, wb, d, tr) in enumerate(rows):
        recs[i]["task"], recs[i]["worker"] = t, w
        recs[i]["t_start"], recs[i]["t_end"] = e % (1 << 32), wb % (1 << 32)
        recs[i]["clk_start"], recs[i]["clk_end"] = d % (1 << 32), tr % (1 << 32)
    return recs


# the same six tasks with entry and wait-begin clocks (timing trace)
TROWS = [(0, 0, BASE - 20, BASE - 10, BASE + 0, BASE + 100), (1, 1, BASE - 20, BASE + 5, BASE + 10, BASE + 90),
         (2, 1, BASE + 110, BASE + 120, BASE + 150, BASE + 300), (3, 0, BASE + 120, BASE + 200, BASE + 320, BASE + 400),
         (4, 1, BASE + 310, BASE + 330, BASE + 450, BASE + 600), (5, 0, BASE + 420, BASE + 430, BASE + 650, BASE + 700)]


def test_task_phases_partition_each_workers_time():
    recs = _timing_records(TROWS)
    ph = timeline.task_phases(recs, TASKS)
    # worker 0: tasks 0, 3, 5 -> post 0 + 20 + 20, issue 10 + 80 + 10, wait 10 + 120 + 220, run 100 + 80 + 50
    # worker 1: tasks 1, 2, 4 -> post 0 + 20 + 10, issue 25 + 10 + 20, wait 5 + 30 + 120, run 80 + 150 + 150
    pw = ph["_per_worker"]
    assert pw["post_us"] == pytest.approx((40 + 30) / 2 * timeline.TICK_US)
    assert pw["issue_us"] == pytest.approx((100 + 55) / 2 * timeline.TICK_US)
    assert pw["wait_us"] == pytest.approx((350 + 155) / 2 * timeline.TICK_US)
    assert pw["run_us"] == pytest.approx((230 + 380) / 2 * timeline.TICK_US)
    # the four intervals add up to first entry -> last trigger per worker (720 and 620 ticks)
    assert sum(pw[k] for k in ("post_us", "issue_us", "wait_us", "run_us")) == pytest.approx(670 * timeline.TICK_US)
    assert ph["oproj"]["tasks"] == 2
    assert ph["oproj"]["run_us"] == pytest.approx((80 + 50) / 2 * timeline.TICK_US)
    assert ph["attn"]["wait_us"] == pytest.approx(30 * timeline.TICK_US)


def test_op_phases_follow_the_last_triggers():
    recs = _timing_records(TROWS)
    ph = timeline.op_phases(recs, TASKS)
    # layer 0: qkv ends 100, attn 300, oproj 400; layer 1: qkv ends 600, oproj 700
    assert ph["attn"] == pytest.approx(2.0)
    assert ph["oproj"] == pytest.approx(np.median([1.0, 1.0]))
    assert ph["qkv"] == pytest.approx(2.0)  # 400 -> 600 (layer 0's qkv has no predecessor)
