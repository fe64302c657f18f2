"""Paged KV cache: the attention chunks and the KV append address cache rows
through a page table (pools [L][n_pages][Hkv][page][D]), the layout a
serving pipeline keeps inside the megakernel (review page of arXiv
2512.22219, adoption paragraph: paged attention inside the mega-kernel).

The oracle keeps its contiguous caches; the session scatters the same
initial entries into pages spread over the pool by a seeded random
permutation (with spare pages left unused).  Checks: parity with the oracle
(logits, tokens, the appended rows read back through the page table, the task
trace), bit-exact equality with the contiguous layout on the same inputs (the
same arithmetic, other addresses), and a bad page number reported without a
write.
"""

import dataclasses

import numpy as np
import pytest
import torch

import decode_megakernel_persistent_amd as mk
import synth
from tests import harness
from tests.test_gpu_parity import assert_reports, run_steps

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lens", [[0, 1, 2, 33], [0, 1, 2, 33, 5, 9, 17, 40]])
@pytest.mark.parametrize("mode", [mk.MK_PERSISTENT, mk.MK_LAUNCH_PER_TASK])
def test_paged_tiny_ragged(lens, mode):
    # pages of 16 rows; 7 chunks per (sequence, kv head), so chunks start and
    # end inside pages and some span two
    w = dataclasses.replace(synth.WORKLOADS["tiny"], name=f"tiny-paged-b{len(lens)}", batch=len(lens))
    prep = harness.prepare(w, lens=lens)
    reports, st = run_steps(w, prep, mode, steps=3, attn_chunks=7, page_size=16)
    assert_reports(reports)


def test_paged_8b_batch16_ragged():
    # 16 sequences at positions U{1..2048} in 16-row pages, MFMA tiles
    w = synth.WORKLOADS["qwen3-8b-b16"]
    prep = harness.prepare(w)
    reports, _ = run_steps(w, prep, mk.MK_PERSISTENT, steps=2, page_size=16)
    assert_reports(reports)
    reports, _ = run_steps(w, prep, mk.MK_LAUNCH_PER_TASK, steps=1, trace=False, page_size=16)
    assert_reports(reports)


@pytest.mark.parametrize("wname,page", [("qwen3-8b", 16), ("qwen3-8b", 64), ("tiny", 32)])
def test_paged_equals_contiguous_bit_for_bit(wname, page):
    w = synth.WORKLOADS[wname]
    prep = harness.prepare(w)
    ref = mk.Session(w.shape, w.batch, w.capacity)
    pg = mk.Session(w.shape, w.batch, w.capacity, page_size=page, spare_pages=5, page_seed=11)
    try:
        for s in (ref, pg):
            s.load(prep.weights)
            s.set_kv(prep.k0, prep.v0)
        tok, pos = prep.tokens.copy(), prep.positions.copy()
        for step in range(3):
            harness.log(f"[paged] {wname} page {page} step {step}")
            a = ref.step(tok, pos)
            b = pg.step(tok, pos)
            torch.cuda.synchronize()
            ref.check()
            pg.check()
            a, b = a.cpu().numpy(), b.cpu().numpy()
            np.testing.assert_array_equal(a, b)
            tok, pos = harness.oracle.greedy(a), pos + 1
        kc, vc = pg.kv_contiguous()
        assert torch.equal(kc, ref.k_cache) and torch.equal(vc, ref.v_cache)
    finally:
        ref.close()
        pg.close()


def test_paged_multistep_matches_contiguous():
    # 40 greedy steps in one launch over pages: the same tokens, last logits
    # and cache as the contiguous layout
    w = dataclasses.replace(synth.WORKLOADS["tiny"], name="tiny-40", steps=40)
    prep = harness.prepare(w)
    ref = mk.Session(w.shape, w.batch, w.capacity)
    pg = mk.Session(w.shape, w.batch, w.capacity, page_size=16, spare_pages=2, page_seed=3)
    try:
        outs = []
        for s in (ref, pg):
            s.load(prep.weights)
            s.set_kv(prep.k0, prep.v0)
            outs.append(s.decode(prep.tokens, prep.positions, 40))
        torch.cuda.synchronize()
        ref.check()
        pg.check()
        assert torch.equal(outs[0], outs[1])
        assert torch.equal(ref.logits, pg.logits)
        kc, vc = pg.kv_contiguous()
        assert torch.equal(kc, ref.k_cache) and torch.equal(vc, ref.v_cache)
    finally:
        ref.close()
        pg.close()


def test_paged_bad_page_number_is_reported():
    # a page table entry outside the pool, met by the step's appending chunk:
    # reported through mk_check, no row written anywhere
    w = synth.WORKLOADS["tiny"]
    prep = harness.prepare(w)
    sess = mk.Session(w.shape, w.batch, w.capacity, page_size=16, spare_pages=0)
    try:
        sess.load(prep.weights)
        sess.set_kv(prep.k0, prep.v0)
        before_k, before_v = sess.k_cache.clone(), sess.v_cache.clone()
        pos = int(prep.positions[0])
        sess.page_table[0, pos // 16] = sess.n_pages  # one past the pool
        sess.step(prep.tokens, prep.positions)
        torch.cuda.synchronize()
        with pytest.raises(mk.MkError) as e:
            sess.check()
        assert e.value.status == mk.MK_ERR_ARG
        assert torch.equal(sess.k_cache, before_k) and torch.equal(sess.v_cache, before_v)
    finally:
        sess.close()


def test_paged_argument_errors():
    w = synth.WORKLOADS["tiny"]
    prep = harness.prepare(w)
    sess = mk.Session(w.shape, w.batch, w.capacity, page_size=16)
    try:
        sess.load(prep.weights)
        good = sess.kv
        for field, value in (("page_size", 24), ("page_size", 8), ("n_pages", 0), ("page_table", None),
                             ("reserved", 1)):
            bad = mk.mk_kv_cache(good.k, good.v, good.capacity, good.page_size, good.page_table, good.n_pages, 0)
            setattr(bad, field, value)
            with pytest.raises(mk.MkError) as e:
                mk.mk_decode_step(sess.g, sess.tokens.data_ptr(), sess.positions.data_ptr(), bad,
                                  sess.logits.data_ptr(), sess.stream)
            assert e.value.status == mk.MK_ERR_ARG, field
    finally:
        sess.close()
