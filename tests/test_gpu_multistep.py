"""On-device multi-step greedy decode (mk_decode_steps) through the C ABI.

One launch of N steps must reproduce, bit for bit, N single-step launches of
the same kernels whose greedy token is taken on the host (argmax of the
returned fp32 logits, ties to the lowest id): the same tokens, the same last
logits and the same KV cache.  The device tokens and last logits are also
checked against the oracle under teacher forcing with the device's tokens
(tokens equal wherever the oracle's top-2 margin exceeds 0.05, logits within
relative L2 1e-2).
"""

import dataclasses

import numpy as np
import pytest
import torch

import decode_megakernel_persistent_amd as mk
import synth
from tests import harness

pytestmark = pytest.mark.gpu

MOE_SMALL = synth.ModelShape(n_layers=2, hidden=256, n_q_heads=8, n_kv_heads=1, head_dim=64, intermediate=0,
                             vocab=1024, tied_embeddings=False, n_experts=16, top_k=4, expert_intermediate=128)


def host_greedy(lg: np.ndarray) -> np.ndarray:
    return np.argmax(lg, axis=-1).astype(np.int32)  # first maximum = lowest id


def new_session(w, prep, **kw):
    sess = mk.Session(w.shape, w.batch, w.capacity, mk.make_opts(**kw))
    sess.load(prep.weights)
    sess.set_kv(prep.k0, prep.v0)
    return sess


def check_multistep(w, prep, n, oracle_check=True, **kw):
    a = new_session(w, prep, **kw)
    b = new_session(w, prep, **kw)
    try:
        harness.log(f"[multi] {w.name} n={n} one launch")
        out = a.decode(prep.tokens, prep.positions, n)
        torch.cuda.synchronize()
        a.check()
        dev_tok = out.cpu().numpy()
        dev_lg = a.logits.cpu().numpy()
        a_routing = ([a.read_routing(s, with_logits=(s == n - 1)) for s in range(n)]
                     if w.shape.n_experts else None)
        harness.log(f"[multi] {w.name} n={n} host loop")
        tok, host_tok = prep.tokens.copy(), []
        for s in range(n):
            lg = b.step(tok, prep.positions + s)
            torch.cuda.synchronize()
            b.check()
            lg = lg.cpu().numpy()
            tok = host_greedy(lg)
            host_tok.append(tok)
        np.testing.assert_array_equal(dev_tok, np.stack(host_tok))
        np.testing.assert_array_equal(dev_lg, lg)
        assert torch.equal(a.k_cache, b.k_cache) and torch.equal(a.v_cache, b.v_cache)
    finally:
        a.close()
        b.close()
    if oracle_check:
        # teacher forcing with the device's tokens; routed steps are checked on
        # the device's recorded expert choice of each step (router logits are
        # kept for the launch's last step only)
        routings = [a_routing[s] for s in range(n)] if w.shape.n_experts else [None] * n
        orc = harness.oracle.Oracle(w.shape, w.batch, w.capacity)
        orc.set_weights(prep.weights)
        orc.K[...] = prep.k0
        orc.V[...] = prep.v0
        tok = prep.tokens.copy()
        for s in range(n):
            lg_o = harness.oracle_reference(orc, tok, prep.positions + s, routings[s])
            margin = harness.oracle.top2_margin(lg_o)
            want = harness.oracle.greedy(lg_o)
            sure = margin > 0.05
            assert np.all(dev_tok[s][sure] == want[sure]), (s, dev_tok[s], want, margin)
            tok = dev_tok[s]
        rep = harness.compare(dev_lg, lg_o)
        harness.log(f"[multi] {w.name} last-step rel_l2 {max(r['rel_l2'] for r in rep):.3e}")
        assert all(r["ok"] for r in rep), rep
    return dev_tok


def test_tiny_multistep_matches_single_steps():
    w = synth.WORKLOADS["tiny"]
    check_multistep(w, harness.prepare(w), 8)


@pytest.mark.parametrize("batch", [3, 8])
def test_tiny_batches_multistep(batch):
    # batch 3: VALU lm_head candidates; batch 8: MFMA tiles, ragged positions
    w = dataclasses.replace(synth.WORKLOADS["tiny"], name=f"tiny-b{batch}", batch=batch)
    check_multistep(w, harness.prepare(w), 5)


def test_moe_multistep_routes_every_step():
    # routing runs on the dispatch wavefront once per step of the launch; the
    # device's choice of every step is read back and checked against the oracle
    w = synth.Workload(name="moe-small-b2", shape=MOE_SMALL, batch=2, context=96, steps=8, ragged=True)
    check_multistep(w, harness.prepare(w), 8)


def test_8b_multistep_matches_single_steps():
    w = synth.WORKLOADS["qwen3-8b"]
    check_multistep(w, harness.prepare(w), 8)


@pytest.mark.parametrize("wname", ["qwen3-0.6b", "qwen3-8b"])
def test_lds_ring_multistep_matches_single_steps(wname):
    # the LDS weight ring's loaders run ahead from tile to tile across a whole
    # multi-step launch: bit-exact against one-step launches, tokens and last
    # logits against the oracle
    w = synth.WORKLOADS[wname]
    check_multistep(w, harness.prepare(w), 8, lds_ring=1)


def test_tied_embedding_multistep_crosses_chunk_boundaries():
    # 0.6B (tied lm_head, VALU tiles) for its configured 32 steps in one launch:
    # with 18 chunks over 513..544 positions, rows appended early in the launch
    # fall into other chunks (other workers, other XCDs) later in it
    w = synth.WORKLOADS["qwen3-0.6b"]
    check_multistep(w, harness.prepare(w), w.steps)


def test_tiny_multistep_crosses_chunk_boundaries():
    # 40 steps in one launch from position 32: with 3 chunks, the row written at
    # step 0 moves from the last chunk into chunk 1 at step 16
    w = dataclasses.replace(synth.WORKLOADS["tiny"], name="tiny-40", steps=40)
    check_multistep(w, harness.prepare(w), 40)


def test_8b_batch16_multistep():
    # 16 ragged sequences on the MFMA tiles: every candidate column in use
    w = synth.WORKLOADS["qwen3-8b-b16"]
    check_multistep(w, harness.prepare(w), 4)


def test_multistep_argument_errors():
    w = synth.WORKLOADS["tiny"]
    prep = harness.prepare(w)
    sess = new_session(w, prep)
    try:
        with pytest.raises(mk.MkError) as e:
            sess.decode(prep.tokens, prep.positions, 0)
        assert e.value.status == mk.MK_ERR_ARG
        sess.set_mode(mk.MK_LAUNCH_PER_TASK)
        with pytest.raises(mk.MkError) as e:
            sess.decode(prep.tokens, prep.positions, 2)
        assert e.value.status == mk.MK_ERR_ARG
    finally:
        sess.close()
    traced = new_session(w, prep, trace=1)
    try:
        with pytest.raises(mk.MkError) as e:
            traced.decode(prep.tokens, prep.positions, 2)
        assert e.value.status == mk.MK_ERR_ARG
    finally:
        traced.close()


def test_multistep_past_capacity_is_reported():
    # positions + n - 1 reach the cache capacity: the attention bounds check
    # clamps the position and reports bad input, read back by mk_check
    w = synth.WORKLOADS["tiny"]
    prep = harness.prepare(w)
    sess = new_session(w, prep)
    try:
        pos = np.full(w.batch, w.capacity - 2, dtype=np.int32)
        sess.decode(prep.tokens, pos, 4)
        torch.cuda.synchronize()
        with pytest.raises(mk.MkError) as e:
            sess.check()
        assert e.value.status == mk.MK_ERR_ARG
        # the state is reset: a valid launch runs again
        sess.decode(prep.tokens, prep.positions, 2)
        torch.cuda.synchronize()
        sess.check()
    finally:
        sess.close()


def test_persistent_after_launch_per_task_steps():
    # launch-per-task steps advance the event epoch but not the workers'
    # arrival / completion counts: a later persistent launch (one step or
    # several) must still pass the dispatch wavefront's residency handshake
    w = synth.WORKLOADS["tiny"]
    prep = harness.prepare(w)
    sess = new_session(w, prep)
    try:
        tok, pos = prep.tokens.copy(), prep.positions.copy()
        for mode, n in ((mk.MK_PERSISTENT, 2), (mk.MK_LAUNCH_PER_TASK, 2), (mk.MK_PERSISTENT, 1)):
            sess.set_mode(mode)
            for _ in range(n):
                harness.log(f"[mode] {mode} pos {pos.tolist()}")
                lg = sess.step(tok, pos)
                torch.cuda.synchronize()
                sess.check()
                tok, pos = host_greedy(lg.cpu().numpy()), pos + 1
        out = sess.decode(tok, pos, 3)
        torch.cuda.synchronize()
        sess.check()
        t = out.cpu().numpy()
        assert t.min() >= 0 and t.max() < w.shape.vocab
    finally:
        sess.close()
