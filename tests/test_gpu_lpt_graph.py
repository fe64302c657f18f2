"""Launch-per-task mode captured into a HIP graph (mk_capture_lpt_graph).

Every replay must equal, bit for bit, an eager launch-per-task step of the
same kernels on the same inputs, and match the oracle (logits relative L2 <=
1e-2, tokens where the top-2 margin exceeds 0.05); replays alternate with the
program's own eager work and synchronisations, and each one is checked.  A persistent step
after the replays must still match (the replays count as steps for the event
epochs), and the KV caches must agree at the end.
"""

import numpy as np
import pytest
import torch

import decode_megakernel_persistent_amd as mk
import synth
from tests import harness

pytestmark = pytest.mark.gpu


def new_session(w, prep, **kw):
    sess = mk.Session(w.shape, w.batch, w.capacity, mk.make_opts(**kw))
    sess.load(prep.weights)
    sess.set_kv(prep.k0, prep.v0)
    return sess


@pytest.mark.parametrize("wname,per_task,merge_tasks", [("tiny", 0, 0), ("tiny", 1, 0), ("tiny", 0, 2),
                                                        ("qwen3-0.6b", 0, 0), ("qwen3-0.6b", 0, 2)])
def test_lpt_graph_replays_match_eager_steps(wname, per_task, merge_tasks):
    # merge_tasks = 2: the last-arriving attention chunk merges, found from an
    # arrival counter that every replay advances
    w = synth.WORKLOADS[wname]
    prep = harness.prepare(w)
    gs = new_session(w, prep, merge_tasks=merge_tasks)
    es = new_session(w, prep, merge_tasks=merge_tasks)
    orc = harness.oracle.Oracle(w.shape, w.batch, w.capacity)
    orc.set_weights(prep.weights)
    orc.K[...] = prep.k0
    orc.V[...] = prep.v0
    try:
        gs.set_mode(mk.MK_LAUNCH_PER_TASK, per_task)
        es.set_mode(mk.MK_LAUNCH_PER_TASK, per_task)
        h = gs.capture_lpt_graph()
        tok, pos = prep.tokens.copy(), prep.positions.copy()
        for s in range(4):
            harness.log(f"[graph] {wname} per_task={per_task} replay {s} pos {pos.tolist()[:4]}")
            gs.tokens.copy_(torch.as_tensor(tok.astype(np.int32)))
            gs.positions.copy_(torch.as_tensor(pos.astype(np.int32)))
            gs.replay_lpt_graph(h)
            torch.cuda.synchronize()
            gs.check()
            lg_g = gs.logits.cpu().numpy()
            # eager work between replays: the reference step and an unrelated reduction
            lg_e = es.step(tok, pos)
            torch.cuda.synchronize()
            es.check()
            lg_e = lg_e.cpu().numpy()
            assert float(torch.ones(1 << 16, device=gs.device).sum().item()) == float(1 << 16)
            np.testing.assert_array_equal(lg_g, lg_e)
            # and the replay against the oracle (teacher forcing with its tokens)
            lg_o = orc.decode(tok, pos)
            rep = harness.compare(lg_g, lg_o)
            harness.log(f"[graph] replay {s}: rel_l2 {max(r['rel_l2'] for r in rep):.2e}")
            assert all(r["ok"] for r in rep), rep
            tok, pos = harness.oracle.greedy(lg_o), pos + 1
        # a persistent step after the replays
        gs.set_mode(mk.MK_PERSISTENT)
        es.set_mode(mk.MK_PERSISTENT)
        lg_g = gs.step(tok, pos)
        lg_e = es.step(tok, pos)
        torch.cuda.synchronize()
        gs.check()
        es.check()
        np.testing.assert_array_equal(lg_g.cpu().numpy(), lg_e.cpu().numpy())
        assert torch.equal(gs.k_cache, es.k_cache) and torch.equal(gs.v_cache, es.v_cache)
    finally:
        gs.close()
        es.close()


def test_lpt_graph_capture_refuses_trace():
    w = synth.WORKLOADS["tiny"]
    prep = harness.prepare(w)
    sess = new_session(w, prep, trace=1)
    try:
        with pytest.raises(mk.MkError) as e:
            sess.capture_lpt_graph()
        assert e.value.status == mk.MK_ERR_ARG
    finally:
        sess.close()
