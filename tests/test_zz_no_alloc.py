"""mk_decode_step_noalloc: the step on the library's static scratch must give
exactly what mk_decode_step gives on the caller's scratch (the same kernels on
the same inputs: logits and the appended cache rows bit for bit), on two
calls in a row, the second with a smaller graph whose state starts where the
first left the shared array; in both execution modes; and a graph whose
scratch exceeds the static array is refused with a clear error.
"""

import dataclasses

import numpy as np
import pytest
import torch

import decode_megakernel_persistent_amd as mk
import synth
from tests import harness

pytestmark = pytest.mark.gpu


def _pair(w, prep, mode):
    sessions = []
    for _ in range(2):
        s = mk.Session(w.shape, w.batch, w.capacity, mk.make_opts(mode=mode))
        s.load(prep.weights)
        s.set_kv(prep.k0, prep.v0)
        sessions.append(s)
    return sessions


def _step_both(ref, st, tok, pos):
    lg_r = ref.step(tok, pos)
    st.tokens.copy_(torch.as_tensor(np.asarray(tok, dtype=np.int32)))
    st.positions.copy_(torch.as_tensor(np.asarray(pos, dtype=np.int32)))
    mk.mk_decode_step_noalloc(st.g, st.tokens.data_ptr(), st.positions.data_ptr(), st.kv, st.logits.data_ptr(),
                              st.stream)
    torch.cuda.synchronize()
    ref.check()
    st.check()
    return lg_r.cpu().numpy(), st.logits.cpu().numpy()


@pytest.mark.parametrize("mode", [mk.MK_PERSISTENT, mk.MK_LAUNCH_PER_TASK])
def test_noalloc_matches_decode_step_on_two_calls(mode):
    # first: 0.6B (11 MiB of scratch), then the tiny decoder (64 KiB): the
    # second call's state must not depend on what the first left behind
    big = synth.WORKLOADS["qwen3-0.6b"]
    small = dataclasses.replace(synth.WORKLOADS["tiny"], name="tiny-b3", batch=3)
    for w in (big, small):
        prep = harness.prepare(w)
        ref, st = _pair(w, prep, mode)
        try:
            tok, pos = prep.tokens.copy(), prep.positions.copy()
            for step in range(2):
                harness.log(f"[noalloc] {w.name} mode {mode} step {step}")
                a, b = _step_both(ref, st, tok, pos)
                np.testing.assert_array_equal(a, b)
                tok, pos = harness.oracle.greedy(a), pos + 1
            assert torch.equal(ref.k_cache, st.k_cache) and torch.equal(ref.v_cache, st.v_cache)
            # the graph's own scratch still works after calls on the static one
            a = ref.step(tok, pos)
            b = st.step(tok, pos)
            torch.cuda.synchronize()
            ref.check()
            st.check()
            np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())
        finally:
            ref.close()
            st.close()


def test_noalloc_refuses_a_graph_larger_than_the_static_scratch():
    w = synth.WORKLOADS["qwen3-8b-b16"]
    g = mk.mk_build_graph(w.shape, w.batch, w.capacity, mk.make_opts())
    try:
        kv = mk.mk_kv_cache(1, 1, w.capacity, 0, None, 0, 0)
        with pytest.raises(mk.MkError) as e:
            mk.mk_decode_step_noalloc(g, 1, 1, kv, 1, 0)
        assert e.value.status == mk.MK_ERR_ARG and "static scratch" in str(e.value)
    finally:
        mk.mk_destroy_graph(g)
