"""The host task-graph compiler and the event protocol, on the CPU.

Invariants of the compiled tables (MPK review page 2512.22219, section 2.4):
every task has at most one dependency event and one trigger event, each
event's dependents are one contiguous id range, ids are topological, each
event's target equals its number of triggering tasks.  Edge preservation is
checked by brute force: every read/write conflict edge derived from the
tasks' footprints is implied by a path in the final event graph.  The
protocol itself runs on host threads (the same tables, no-op bodies) and the
trace checker must accept clean runs and flag planted faults.
"""

import os
import subprocess

import numpy as np
import pytest

import decode_megakernel_persistent_amd as mk
import synth

TINY = synth.WORKLOADS["tiny"]
SMALL = synth.ModelShape(n_layers=3, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, intermediate=1024,
                         vocab=2048, tied_embeddings=True)
MOE = synth.ModelShape(n_layers=2, hidden=256, n_q_heads=8, n_kv_heads=1, head_dim=64, intermediate=0, vocab=1024,
                       tied_embeddings=False, n_experts=16, top_k=4, expert_intermediate=128)


def build(shape, batch=1, cap=64, **kw):
    kw.setdefault("num_workers", 16)
    return mk.mk_build_graph(shape, batch, cap, mk.make_opts(**kw))


def check_invariants(g):
    tasks = mk.mk_get_tasks(g)
    ev = mk.mk_get_events(g)
    off, ids = mk.mk_get_worker_lists(g)
    n, ne = len(tasks), len(ev)
    dep, trig = tasks[:, 2], tasks[:, 3]
    assert dep.min() >= -1 and dep.max() < ne and trig.min() >= -1 and trig.max() < ne
    counts = np.bincount(trig[trig >= 0], minlength=ne)
    np.testing.assert_array_equal(ev[:, 0], counts)            # need == number of triggers
    for e, (need, first, last, prod) in enumerate(ev):
        assert need >= 1
        members = np.nonzero(dep == e)[0]
        if last >= first:
            np.testing.assert_array_equal(members, np.arange(first, last + 1))  # contiguous range
            assert np.nonzero(trig == e)[0].max() < first                      # topological
        else:
            assert members.size == 0
    # worker lists: a partition of the ids, each increasing
    assert sorted(ids.tolist()) == list(range(n))
    for w in range(len(off) - 1):
        lst = ids[off[w]:off[w + 1]]
        assert np.all(np.diff(lst) > 0)
    return tasks, ev


def ancestors_matrix(tasks, ev):
    n = len(tasks)
    anc = np.zeros((n, n), dtype=bool)
    prods = [[] for _ in range(len(ev))]
    for t in range(n):
        if tasks[t, 3] >= 0:
            prods[tasks[t, 3]].append(t)
    for t in range(n):  # ids are topological
        e = tasks[t, 2]
        for p in prods[e] if e >= 0 else []:
            anc[t, p] = True
            anc[t] |= anc[p]
    return anc


@pytest.mark.parametrize("shape,batch,kw", [
    (TINY.shape, 1, {}),
    (TINY.shape, 1, {"merge_tasks": 1}),
    (TINY.shape, 1, {"merge_tasks": 2}),
    (SMALL, 1, {"num_workers": 64}),
    (TINY.shape, 3, {"attn_chunks": 3}),
    (SMALL, 2, {"num_workers": 7}),
    (MOE, 2, {"num_workers": 8}),
])
def test_invariants_and_edge_preservation(shape, batch, kw):
    g = build(shape, batch, **kw)
    try:
        tasks, ev = check_invariants(g)
        raw = mk.mk_get_raw_edges(g)
        assert len(raw) > 0
        anc = ancestors_matrix(tasks, ev)
        implied = anc[raw[:, 1], raw[:, 0]]
        assert implied.all(), f"{(~implied).sum()} footprint edges not implied by the event graph"
    finally:
        mk.mk_destroy_graph(g)


def test_decoder_graphs_need_no_empty_tasks_and_fusion_shrinks_events():
    g = build(TINY.shape)
    try:
        st = mk.mk_graph_stats(g)
        assert st.empty_tasks == 0                      # deep, not wide
        assert st.events < 10 * TINY.shape.n_layers
    finally:
        mk.mk_destroy_graph(g)
    g = build(TINY.shape, no_fusion=1, num_workers=4)
    try:
        st2 = mk.mk_graph_stats(g)
        assert st2.empty_tasks > 0 and st2.events > 10 * st.events
        tasks, ev = check_invariants(g)                 # normalisation restores <=1 dep / <=1 trigger
        raw = mk.mk_get_raw_edges(g)
        anc = ancestors_matrix(tasks, ev)
        assert anc[raw[:, 1], raw[:, 0]].all()
    finally:
        mk.mk_destroy_graph(g)


def test_head_group_aligned_qkv_tiles():
    # each attention task depends on exactly the QKV tiles of its own kv head
    g = build(SMALL, 1, num_workers=16)
    try:
        tasks, ev = check_invariants(g)
        kinds = [mk.OP_KINDS[k] for k in tasks[:, 0]]
        G = SMALL.n_q_heads // SMALL.n_kv_heads
        rows_per_group = (G + 2) * SMALL.head_dim
        for t in np.nonzero(np.array(kinds) == "attn")[0][:8]:
            e = tasks[t, 2]
            prods = np.nonzero(tasks[:, 3] == e)[0]
            groups = {tasks[p, 5] // rows_per_group for p in prods}
            assert groups == {tasks[t, 5]}
    finally:
        mk.mk_destroy_graph(g)


@pytest.mark.parametrize("merge_tasks,merges,merge_events", [(0, 256, 8), (1, 8, 8), (2, 0, 0)])
def test_8b_graph_shape_counts(merge_tasks, merges, merge_events):
    s = synth.WORKLOADS["qwen3-8b"]
    g = mk.mk_build_graph(s.shape, 1, s.capacity, mk.make_opts(num_workers=256, merge_tasks=merge_tasks))
    try:
        st = mk.mk_graph_stats(g)
        assert st.attn_chunks == 32
        # per layer: 256 QKV + 256 attention chunks + merges + 256 O + 256 gate-up + 256 down
        assert st.tasks == 1 + 36 * (256 * 5 + merges) + 256
        assert st.empty_tasks == 0
        # per layer: 8 QKV head groups, (8 chunk groups), attention/merge -> O, O, gate-up, down
        # plus the embedding event and the terminal event of the lm_head tiles
        assert st.events == 36 * (12 + merge_events) + 2
        # one launch per consumer range (the lm_head event has none) plus the roots
        assert st.launches_per_step == (st.events - 1) + 1
        assert st.max_tasks_per_worker <= 36 * (5 + (merges + 255) // 256) + 2
        assert abs(st.weight_bytes / 1e9 - 15.137) < 0.01
    finally:
        mk.mk_destroy_graph(g)


@pytest.mark.parametrize("shape,batch", [(TINY.shape, 1), (MOE, 2)])
def test_simulated_protocol_traces_pass(shape, batch):
    g = build(shape, batch, num_workers=8)
    try:
        recs, cnt = mk.mk_simulate(g, steps=3)
        mk.mk_check_trace(g, recs, 2, cnt)
    finally:
        mk.mk_destroy_graph(g)


@pytest.mark.parametrize("fault,status", [(1, mk.MK_ERR_TIMEOUT), (2, mk.MK_ERR_TRACE), (3, mk.MK_ERR_TRACE)])
def test_checker_catches_planted_faults(fault, status):
    g = build(TINY.shape, num_workers=8)
    try:
        with pytest.raises(mk.MkError) as e:
            recs, cnt = mk.mk_simulate(g, steps=1, fault=fault, timeout_ms=300)
            mk.mk_check_trace(g, recs, 0, cnt)
        assert e.value.status == status
    finally:
        mk.mk_destroy_graph(g)


def test_checker_rejects_tampered_traces():
    g = build(TINY.shape, num_workers=8)
    try:
        recs, cnt = mk.mk_simulate(g, steps=1)
        mk.mk_check_trace(g, recs, 0, cnt)
        dup = recs.copy()
        dup[1] = dup[0]
        with pytest.raises(mk.MkError, match="more than once"):
            mk.mk_check_trace(g, dup, 0, cnt)
        with pytest.raises(mk.MkError, match="records"):
            mk.mk_check_trace(g, recs[:-1], 0, cnt)
        low = recs.copy()
        k = int(np.nonzero(mk.mk_get_tasks(g)[low["task"], 2] >= 0)[0][0])
        low["dep_seen"][k] = 0
        with pytest.raises(mk.MkError, match="below target"):
            mk.mk_check_trace(g, low, 0, cnt)
    finally:
        mk.mk_destroy_graph(g)


def test_timing_trace_is_not_checkable():
    g = build(TINY.shape, num_workers=8, trace=2)
    try:
        recs, cnt = mk.mk_simulate(g, steps=1)
        with pytest.raises(mk.MkError) as e:
            mk.mk_check_trace(g, recs, 0, cnt)
        assert e.value.status == mk.MK_ERR_ARG
    finally:
        mk.mk_destroy_graph(g)
    with pytest.raises(mk.MkError):
        build(TINY.shape, trace=3)


def test_protocol_under_thread_sanitizer(tmp_path):
    from decode_megakernel_persistent_amd import build as b
    exe = b.build_tsan()
    r = subprocess.run([exe, "8", "3"], capture_output=True, text=True, timeout=600,
                       env={**os.environ, "TSAN_OPTIONS": "halt_on_error=1"})
    assert r.returncode == 0, r.stdout + r.stderr
    assert "WARNING: ThreadSanitizer" not in r.stderr
    assert r.stdout.count("ok") == 2


def test_dump_graph_json(tmp_path):
    import json
    g = build(TINY.shape)
    try:
        p = str(tmp_path / "g.json")
        mk.mk_dump_graph(g, p)
        d = json.load(open(p))
        assert len(d["tasks"]) == mk.mk_graph_stats(g).tasks
        assert d["gemv"] == "valu"
    finally:
        mk.mk_destroy_graph(g)


@pytest.mark.parametrize("wname,gemv", [("tiny", mk.MK_GEMV_AUTO), ("qwen3-8b", mk.MK_GEMV_AUTO),
                                        ("qwen3-8b-b16", mk.MK_GEMV_AUTO)])
def test_lm_head_terminal_event(wname, gemv):
    # the lm_head tiles trigger one event that no task of the step waits on;
    # a multi-step launch waits on it before the next step's embedding
    w = synth.WORKLOADS[wname]
    g = mk.mk_build_graph(w.shape, w.batch, w.capacity, mk.make_opts(gemv=gemv))
    try:
        tasks, ev = mk.mk_get_tasks(g), mk.mk_get_events(g)
        lm = np.nonzero(tasks[:, 0] == mk.OP_KINDS.index("lmhead"))[0]
        trig = set(tasks[lm, 3].tolist())
        assert len(trig) == 1
        e = trig.pop()
        assert e >= 0
        need, first, last, producers = ev[e]
        assert need == len(lm) == producers
        assert last < first  # no consumers
        assert not np.any(tasks[:, 2] == e)  # nobody depends on it
        # tiles are numbered 0..n-1 (the candidate buffer's index)
        assert sorted(tasks[lm, 4].tolist()) == list(range(len(lm)))
    finally:
        mk.mk_destroy_graph(g)


def _upstream_tasks(tasks, event):
    """Every task the given event depends on, transitively (reverse walk over triggers)."""
    prod = {}
    for t, e in enumerate(tasks[:, 3]):
        if e >= 0:
            prod.setdefault(int(e), []).append(t)
    seen, stack, evs = set(), [int(event)], set()
    while stack:
        e = stack.pop()
        if e in evs:
            continue
        evs.add(e)
        for t in prod.get(e, []):
            if t not in seen:
                seen.add(t)
                if tasks[t, 2] >= 0:
                    stack.append(int(tasks[t, 2]))
    return seen


@pytest.mark.parametrize("wname,steps", [("qwen3-0.6b", 32), ("tiny-40", 40)])
def test_multistep_kv_rows_cross_xcds_only_after_an_ordering_event(wname, steps):
    # In a launch of n steps, the row appended at step s by the last chunk
    # task of (layer, sequence, kv head) is read at later steps by whichever
    # chunk covers it as the positions grow.  List those reads: some are by a
    # worker on another XCD (worker index mod 8 on gfx950).  The append is an
    # agent-scope store completed before its task triggers; the reader is
    # ordered after that trigger because (1) every worker's list of a step
    # ends with an lm_head tile and (2) the lm_head tiles depend transitively
    # on every attention chunk of the step, so a worker starts the next step's
    # tasks only after every append of the step has become visible.
    import dataclasses
    w = (dataclasses.replace(synth.WORKLOADS["tiny"], name="tiny-40", steps=40) if wname == "tiny-40"
         else synth.WORKLOADS[wname])
    g = mk.mk_build_graph(w.shape, w.batch, w.capacity, mk.make_opts(num_workers=256))
    try:
        tasks = mk.mk_get_tasks(g)
        off, ids = mk.mk_get_worker_lists(g)
        st = mk.mk_graph_stats(g)
        C, W = st.attn_chunks, st.workers
        worker = np.empty(len(tasks), dtype=np.int64)
        for wk in range(W):
            worker[ids[off[wk]:off[wk + 1]]] = wk
        attn = np.nonzero(tasks[:, 0] == mk.OP_KINDS.index("attn"))[0]
        where = {(int(tasks[t, 1]), int(tasks[t, 4]), int(tasks[t, 5]), int(tasks[t, 6])): int(worker[t]) for t in attn}
        # the in-launch rows and their readers
        p0 = int(synth.lengths(w)[0]) if not w.prompt else w.prompt
        cross = reads = 0
        for (l, b, gi, ch), wk in where.items():
            if ch != C - 1:
                continue
            for s in range(steps):
                r = p0 + s                      # row appended at step s
                for s2 in range(s + 1, steps):
                    ln = p0 + s2 + 1
                    c = next(c for c in range(C) if c * ln // C <= r < (c + 1) * ln // C)
                    if c != C - 1:
                        reads += 1
                        if where[(l, b, gi, c)] % 8 != wk % 8:
                            cross += 1
        assert cross > 0, "the configuration never moves a row across XCDs: the test would not cover the hazard"
        # (1) the last task of every worker's list is an lm_head tile
        lm = mk.OP_KINDS.index("lmhead")
        for wk in range(W):
            assert tasks[ids[off[wk + 1] - 1], 0] == lm
        # (2) the lm_head tiles wait on one event upstream of every attention chunk
        lm_tasks = np.nonzero(tasks[:, 0] == lm)[0]
        deps = set(tasks[lm_tasks, 2].tolist())
        assert len(deps) == 1
        up = _upstream_tasks(tasks, deps.pop())
        assert set(attn.tolist()) <= up
        print(f"{wname}: {reads} in-launch row reads by other chunks, {cross} of them on another XCD")
    finally:
        mk.mk_destroy_graph(g)


@pytest.mark.parametrize("wname,batch,kw,ring_kb,ring_ops", [
    # 8B: rows of 8 KB (K = 4096) and 24 KB (down, K = 12288): 4 KB segments; every GEMV op per layer + lm_head
    ("qwen3-8b", 1, {"lds_ring": 1}, 4, 36 * 4 + 1),
    # 0.6B: rows of 2 KB (K = 1024) and 6 KB (down, K = 3072): 2 KB segments
    ("qwen3-0.6b", 1, {"lds_ring": 1}, 2, 28 * 4 + 1),
    ("qwen3-1.7b", 1, {"lds_ring": 1}, 4, 28 * 4 + 1),
    # tiny: 512-byte rows (K = 256) are not whole kilobytes
    ("tiny", 1, {"lds_ring": 1}, 0, 0),
    # batch above 1, the MFMA path, and the default (option off): no ring
    ("qwen3-8b", 2, {"lds_ring": 1}, 0, 0),
    ("qwen3-8b", 1, {"gemv": mk.MK_GEMV_MFMA, "lds_ring": 1}, 0, 0),
    ("qwen3-8b", 1, {}, 0, 0),
])
def test_lds_ring_assignment(wname, batch, kw, ring_kb, ring_ops):
    """With lds_ring, batch-1 GEMV tiles with whole-KB rows are fed through
    the LDS weight ring; one segment size per graph divides every such row."""
    s = synth.WORKLOADS[wname]
    g = mk.mk_build_graph(s.shape, batch, s.capacity, mk.make_opts(num_workers=256, **kw))
    try:
        st = mk.mk_graph_stats(g)
        assert (st.ring_kb, st.ring_ops) == (ring_kb, ring_ops)
    finally:
        mk.mk_destroy_graph(g)


def test_lds_ring_option_is_validated():
    with pytest.raises(mk.MkError):
        build(TINY.shape, lds_ring=2)


@pytest.mark.parametrize("pct", [100, 85, 120])
def test_xcd_weighted_row_split(pct):
    """xcd_rows_pct: the O, gate-up, down and lm_head tiles of a VALU graph
    still cover their operator's rows exactly once, contiguously in tile
    order, and a tile whose worker sits on an odd XCD (worker mod 8 odd) gets
    about pct percent of the rows of an even-XCD tile; weight offsets follow
    the rows (gate-up tiles hold gate and up rows, two per output row)."""
    s = synth.WORKLOADS["qwen3-8b"]
    g = mk.mk_build_graph(s.shape, 1, s.capacity, mk.make_opts(num_workers=256, xcd_rows_pct=pct))
    try:
        t = mk.mk_get_tasks(g)
        off, ids = mk.mk_get_worker_lists(g)
        worker = np.empty(len(t), np.int64)
        for w in range(len(off) - 1):
            worker[ids[off[w]:off[w + 1]]] = w
        H, I, V = s.shape.hidden, s.shape.intermediate, s.shape.vocab
        Hq, D = s.shape.n_q_heads, s.shape.head_dim
        checked = 0
        for kind, N, K in (("oproj", H, Hq * D), ("gateup", I, H), ("down", H, I), ("lmhead", V, H)):
            k = mk.OP_KINDS.index(kind)
            layers = sorted(set(t[t[:, 0] == k][:, 1].tolist()))
            for layer in layers[:3]:
                sel = np.nonzero((t[:, 0] == k) & (t[:, 1] == layer))[0]
                rows = t[sel]
                order = np.argsort(rows[:, 4])                     # tile order
                a1, a2, a3 = rows[order, 5], rows[order, 6], rows[order, 7]
                assert a1[0] == 0 and np.all(a1[1:] == a1[:-1] + a2[:-1]) and a1[-1] + a2[-1] == N
                assert np.all(a2 >= 1)
                np.testing.assert_array_equal(a3, a1 * K * (2 if kind == "gateup" else 1))
                odd = (worker[sel[order]] % 8) % 2 == 1
                ratio = a2[odd].mean() / a2[~odd].mean()
                # whole rows: a tile of ~16 rows moves in steps of one row
                assert abs(ratio - pct / 100.0) < 0.02 + 1.5 / a2.mean(), (kind, layer, ratio)
                checked += 1
        assert checked >= 10
        st = mk.mk_graph_stats(g)
        assert abs(st.weight_bytes / 1e9 - 15.137) < 0.01
    finally:
        mk.mk_destroy_graph(g)


def test_xcd_rows_option_is_validated():
    with pytest.raises(mk.MkError):
        build(TINY.shape, xcd_rows_pct=20)
