"""End-to-end parity of the HIP decoder against the oracle, through the C ABI.

Every step compares logits (relative L2 <= 1e-2) and greedy tokens (equal when
the oracle's top-2 margin > 0.05) under teacher forcing, and the bf16 key and
value rows the step appended (every layer, sequence and kv head) against the
oracle's.  Routed-expert steps also compare the router logits and check the
GPU's expert choice (harness.oracle_reference); nothing is exempted.  In trace
mode the integer task trace of every step is checked against the graph: each
task exactly once, no task started before the triggers of its dependency
event ended, observed counters at their targets, final counters = need x
steps.
"""

import dataclasses

import numpy as np
import pytest
import torch

import decode_megakernel_persistent_amd as mk
import synth
from tests import harness

pytestmark = pytest.mark.gpu


def run_steps(w, prep, mode, steps, trace=True, workers=0, gemv=mk.MK_GEMV_AUTO, attn_chunks=0, merge_tasks=0,
              no_fusion=0, per_task_launch=0, page_size=0, lds_ring=0):
    opts = mk.make_opts(mode=mode, trace=int(trace), num_workers=workers, gemv=gemv, attn_chunks=attn_chunks,
                        merge_tasks=merge_tasks, no_fusion=no_fusion, per_task_launch=per_task_launch,
                        lds_ring=lds_ring)
    sess = mk.Session(w.shape, w.batch, w.capacity, opts, page_size=page_size, spare_pages=3 if page_size else 0)
    try:
        sess.load(prep.weights)
        sess.set_kv(prep.k0, prep.v0)
        orc = harness.oracle.Oracle(w.shape, w.batch, w.capacity)
        orc.set_weights(prep.weights)
        orc.K[...] = prep.k0
        orc.V[...] = prep.v0
        tok, pos = prep.tokens.copy(), prep.positions.copy()
        reports, info = [], {}
        kv_worst = [0.0, 0.0, 0.0]
        routed = w.shape.n_experts > 0
        for s in range(steps):
            harness.log(f"[step] {w.name} mode={mode} step={s} pos={pos.tolist()[:4]}")
            lg_g = sess.step(tok, pos)
            torch.cuda.synchronize()
            sess.check()
            lg_g = lg_g.cpu().numpy()
            routing = sess.read_routing(0, with_logits=True) if routed else None
            lg_o = harness.oracle_reference(orc, tok, pos, routing, info)
            reports.append(harness.compare(lg_g, lg_o))
            # the key / value rows this step appended, against the oracle's
            kd, vd = sess.kv_rows(pos)
            bi = np.arange(w.batch)
            for dev, ref in ((kd, orc.K[:, bi, :, pos, :].transpose(1, 0, 2, 3)),
                             (vd, orc.V[:, bi, :, pos, :].transpose(1, 0, 2, 3))):
                err = harness.kv_row_errors(dev, ref)
                kv_worst = [max(x, y) for x, y in zip(kv_worst, err)]
                assert err[1] <= harness.KV_EXCESS_TOL and err[2] <= harness.KV_MISMATCH_TOL, (s, err)
            if trace == 2:
                # timing trace: record i is task i, stamped by a worker, clocks ordered
                recs = sess.read_trace()
                np.testing.assert_array_equal(recs["task"], np.arange(len(recs)))
                assert recs["worker"].min() >= 0 and recs["worker"].max() < sess.stats.workers
                assert np.all(recs["step"] == recs["step"][0])
                dt = (recs["clk_end"].astype(np.int64) - recs["clk_start"].astype(np.int64)) % (1 << 32)
                assert np.all(dt < 10_000_000)  # < 0.1 s at 100 MHz
            elif trace:
                recs = sess.read_trace()
                cnt = sess.read_counters()
                sess.check_trace(recs, s, cnt)
            tok = harness.oracle.greedy(lg_o)
            pos = pos + 1
        harness.log(f"[kv] {w.name}: appended rows within {kv_worst[0]:.2f} bf16 ulp of the oracle's "
                    f"(beyond one ulp: {kv_worst[1]:.1e} of the row RMS; elements differing: "
                    f"{100 * kv_worst[2]:.2f}% at most)")
        if routed:
            harness.log(f"[route] {w.name}: {info.get('routing_diffs', 0)} (layer, sequence) choices differed from "
                        f"the oracle's top-k; smallest gap {info.get('min_route_gap', np.inf):.2e}; "
                        f"router logits within {info.get('router_err', 0.0):.2e} "
                        f"(relative L2 {info.get('router_rel', 0.0):.2e})")
        return reports, sess.stats
    finally:
        sess.close()


def assert_reports(reports):
    worst = max(r["rel_l2"] for rep in reports for r in rep)
    bad = [(s, b, r) for s, rep in enumerate(reports) for b, r in enumerate(rep) if not r["ok"]]
    total = sum(len(rep) for rep in reports)
    harness.log(f"[parity] steps={len(reports)} comparisons={total} worst rel_l2={worst:.3e} failures={len(bad)}")
    assert not bad, f"parity failures (step, seq, report): {bad[:5]}"


@pytest.fixture(scope="module")
def tiny():
    w = synth.WORKLOADS["tiny"]
    return w, harness.prepare(w)


@pytest.mark.parametrize("mode", [mk.MK_PERSISTENT, mk.MK_LAUNCH_PER_TASK])
def test_tiny_16_steps(tiny, mode):
    w, prep = tiny
    reports, _ = run_steps(w, prep, mode, steps=w.steps)
    assert_reports(reports)


def test_tiny_small_worker_count(tiny):
    # fewer workers than tasks per op: several tasks of one op per worker
    w, prep = tiny
    reports, st = run_steps(w, prep, mk.MK_PERSISTENT, steps=3, workers=8)
    assert st.workers == 8
    assert_reports(reports)


@pytest.mark.parametrize("merge_tasks", [1, 2])
def test_tiny_merge_variants(tiny, merge_tasks):
    # 1: one merge task per (sequence, kv head); 2: the last chunk merges
    w, prep = tiny
    for mode in (mk.MK_PERSISTENT, mk.MK_LAUNCH_PER_TASK):
        reports, st = run_steps(w, prep, mode, steps=3, merge_tasks=merge_tasks)
        assert_reports(reports)


def test_tiny_timing_trace(tiny):
    w, prep = tiny
    reports, _ = run_steps(w, prep, mk.MK_PERSISTENT, steps=2, trace=2)
    assert_reports(reports)


def test_timeline_export_from_a_timing_trace(tiny, tmp_path):
    # the Perfetto timeline of one persistent step: one slice per task on its
    # worker's track, slices of a worker disjoint, and per-worker run + wait
    # equal to the worker's span
    import json
    from decode_megakernel_persistent_amd import timeline
    w, prep = tiny
    sess = mk.Session(w.shape, w.batch, w.capacity, mk.make_opts(trace=2))
    try:
        sess.load(prep.weights)
        sess.set_kv(prep.k0, prep.v0)
        sess.step(prep.tokens, prep.positions)
        torch.cuda.synchronize()
        sess.check()
        recs = sess.read_trace()
        tasks = mk.mk_get_tasks(sess.g)
        p = str(tmp_path / "timeline.json")
        assert timeline.to_perfetto(recs, tasks, p) == sess.stats.tasks
        sl = [e for e in json.load(open(p))["traceEvents"] if e["ph"] == "X"]
        assert sorted(e["args"]["task"] for e in sl) == list(range(sess.stats.tasks))
        for wk in {e["tid"] for e in sl}:
            mine = sorted((e["ts"], e["ts"] + e["dur"]) for e in sl if e["tid"] == wk)
            assert all(a[1] <= b[0] + 0.011 for a, b in zip(mine, mine[1:]))
        att = timeline.attribute(recs, tasks)
        t0, t1 = timeline._times_us(recs)
        ends = {}
        for i, r in enumerate(recs):
            ends[int(r["worker"])] = max(ends.get(int(r["worker"]), 0.0), t1[i] - t0.min())
        total = sum(v["run_us_total"] + v["wait_us_total"] for k, v in att.items() if k != "_span_us")
        assert abs(total - sum(ends.values())) <= 1e-3 * sum(ends.values()) + 1.0
        sp = timeline.layer_split(recs, tasks)
        assert sp["layers"] == w.shape.n_layers and 0 < sp["layer_median_run_us"] <= sp["layer_span_us"]
        harness.log(f"[timeline] tiny: {len(sl)} slices, layer span {sp['layer_span_us']} us, "
                    f"median task run per layer {sp['layer_median_run_us']} us")
    finally:
        sess.close()


def test_tiny_one_chunk_and_many_chunks(tiny):
    w, prep = tiny
    for C in (1, 7):
        reports, st = run_steps(w, prep, mk.MK_PERSISTENT, steps=2, attn_chunks=C)
        assert st.attn_chunks == C
        assert_reports(reports)


@pytest.mark.parametrize("lens", [[0, 1, 2, 33], [0, 1, 2, 33, 5, 9, 17, 40]])
@pytest.mark.parametrize("mode", [mk.MK_PERSISTENT, mk.MK_LAUNCH_PER_TASK])
def test_tiny_ragged_edge_positions(lens, mode):
    # sequences at positions 0 and 1 (a cache holding only the new row, or one
    # more) beside longer ones, with 7 chunks per (sequence, kv head): most
    # chunks of the short sequences cover no cached row.  4 sequences run on
    # the VALU tiles, 8 on the MFMA tiles.
    w = dataclasses.replace(synth.WORKLOADS["tiny"], name=f"tiny-ragged-b{len(lens)}", batch=len(lens))
    prep = harness.prepare(w, lens=lens)
    reports, st = run_steps(w, prep, mode, steps=3, attn_chunks=7)
    assert st.attn_chunks == 7
    assert_reports(reports)


@pytest.mark.parametrize("mode", [mk.MK_PERSISTENT, mk.MK_LAUNCH_PER_TASK])
def test_tiny_normalised_graph_with_empty_tasks(tiny, mode):
    # one event per dependency edge: normalisation inserts empty tasks (a task
    # with several dependency events gets one empty task per event feeding a
    # fresh event), which run and trigger like any task
    w, prep = tiny
    reports, st = run_steps(w, prep, mode, steps=3, workers=16, no_fusion=1)
    assert st.empty_tasks > 0
    harness.log(f"[normalise] {st.tasks} tasks of which {st.empty_tasks} empty, {st.events} events")
    assert_reports(reports)


def test_tiny_one_launch_per_task(tiny):
    # launch-per-task stress mode: literally one kernel launch per task
    w, prep = tiny
    reports, st = run_steps(w, prep, mk.MK_LAUNCH_PER_TASK, steps=2, per_task_launch=1)
    assert_reports(reports)


@pytest.mark.parametrize("batch,gemv", [(1, mk.MK_GEMV_MFMA), (3, mk.MK_GEMV_AUTO), (8, mk.MK_GEMV_AUTO),
                                        (16, mk.MK_GEMV_AUTO)])
def test_tiny_batches(batch, gemv):
    # batch 3: VALU dot products; batch 8 / 16 (and batch 1 when forced): the
    # MFMA skinny-GEMM tiles, with zero-padded sequences past the batch
    w = dataclasses.replace(synth.WORKLOADS["tiny"], name=f"tiny-b{batch}", batch=batch)
    prep = harness.prepare(w)
    reports, st = run_steps(w, prep, mk.MK_PERSISTENT, steps=3, gemv=gemv)
    assert_reports(reports)
    reports, _ = run_steps(w, prep, mk.MK_LAUNCH_PER_TASK, steps=1, trace=False, gemv=gemv)
    assert_reports(reports)


@pytest.fixture(scope="module", params=["qwen3-0.6b", "qwen3-1.7b", "qwen3-8b"])
def dense(request):
    w = synth.WORKLOADS[request.param]
    return w, harness.prepare(w)


def test_dense_parity_persistent(dense):
    # the configured 32 decode steps, trace on
    w, prep = dense
    reports, st = run_steps(w, prep, mk.MK_PERSISTENT, steps=w.steps)
    assert st.empty_tasks == 0
    assert_reports(reports)


def test_dense_parity_launch_per_task(dense):
    w, prep = dense
    reports, _ = run_steps(w, prep, mk.MK_LAUNCH_PER_TASK, steps=2, trace=False)
    assert_reports(reports)


def test_dense_lds_ring_parity(dense):
    # batch-1 tiles fed through the LDS weight ring (loader wavefronts, LDS-DMA
    # loads, run-ahead into the next tile): the configured steps with the
    # ticketed trace, and launch-per-task steps (no run-ahead)
    w, prep = dense
    reports, st = run_steps(w, prep, mk.MK_PERSISTENT, steps=w.steps, lds_ring=1)
    assert st.ring_ops > 0 and st.ring_kb in (2, 4)
    assert_reports(reports)
    reports, _ = run_steps(w, prep, mk.MK_LAUNCH_PER_TASK, steps=2, trace=False, lds_ring=1)
    assert_reports(reports)


@pytest.fixture(scope="module")
def b16():
    w = synth.WORKLOADS["qwen3-8b-b16"]
    return w, harness.prepare(w)


def test_8b_batch16_ragged_parity(b16):
    # 16 sequences with independent positions U{1..2048}; MFMA GEMV tiles
    w, prep = b16
    assert len(set(prep.positions.tolist())) > 8
    reports, st = run_steps(w, prep, mk.MK_PERSISTENT, steps=8)
    assert_reports(reports)
    reports, _ = run_steps(w, prep, mk.MK_LAUNCH_PER_TASK, steps=1, trace=False)
    assert_reports(reports)


MOE_SMALL = synth.ModelShape(n_layers=2, hidden=256, n_q_heads=8, n_kv_heads=1, head_dim=64, intermediate=0,
                             vocab=1024, tied_embeddings=False, n_experts=16, top_k=4, expert_intermediate=128)


@pytest.mark.parametrize("batch", [2, 8])
def test_small_moe_parity(batch):
    # router GEMV, routing on the dispatch wavefront, expert gate-up / down
    # slots over gathered tokens, combine; batch 2 VALU, batch 8 MFMA router
    w = synth.Workload(name=f"moe-small-b{batch}", shape=MOE_SMALL, batch=batch, context=96, steps=4, ragged=True)
    prep = harness.prepare(w)
    reports, st = run_steps(w, prep, mk.MK_PERSISTENT, steps=4)
    assert_reports(reports)
    reports, _ = run_steps(w, prep, mk.MK_LAUNCH_PER_TASK, steps=2, trace=False)
    assert_reports(reports)


@pytest.mark.slow
def test_30b_a3b_batch8_parity():
    # 48 layers, 128 experts, top-8, batch 8 at context 1024 (61 GB of
    # weights); the configured 16 decode steps
    w = synth.WORKLOADS["qwen3-30b-a3b"]
    prep = harness.prepare(w)
    reports, st = run_steps(w, prep, mk.MK_PERSISTENT, steps=w.steps)
    assert_reports(reports)
    reports, _ = run_steps(w, prep, mk.MK_LAUNCH_PER_TASK, steps=1, trace=False)
    assert_reports(reports)
