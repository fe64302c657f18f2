"""Pins of the oracle against values fixed by mathematics or by independent
library routines (never against the oracle itself).

Each test names the oracle function it pins.  A plausible mistake in any of
them (a dropped term, a wrong sign or index, a transposed operand, a wrong
RoPE pairing, a missing bf16 rounding, a cache indexing error) fails at least
one test here.
"""

import dataclasses
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from tests import torch_ref

RNG = np.random.default_rng(12345)


def bf16(a):
    return synth.f32_to_bf16(np.asarray(a, dtype=np.float32))


def widen(b):
    return synth.bf16_to_f32(b).astype(np.float64)


# ----------------------------------------------------------------- RoPE
def test_rope_identity_at_position_zero():
    v = RNG.standard_normal(128)
    assert np.array_equal(oracle.rope(v, 0), v)  # bit-exact: cos 0 = 1, sin 0 = 0


@pytest.mark.parametrize("pos", [1, 7, 513, 2047])
def test_rope_matches_complex_rotation(pos):
    # rotate-half RoPE == multiplying z_i = v_i + j v_{i+D/2} by e^{j pos theta^(-2i/D)}
    D, theta = 128, 1e6
    v = RNG.standard_normal(D)
    z = (v[:D // 2] + 1j * v[D // 2:]) * np.exp(1j * pos * theta ** (-2.0 * np.arange(D // 2) / D))
    want = np.concatenate([z.real, z.imag])
    np.testing.assert_allclose(oracle.rope(v, pos, theta), want, rtol=0, atol=1e-12)


def test_rope_unit_vector_closed_form():
    # pair 0 has frequency 1: e_0 at position p becomes (cos p) e_0 + (sin p) e_{D/2}
    D = 8
    for p in (1, 2, 3, 100):
        v = np.zeros(D)
        v[0] = 1.0
        out = oracle.rope(v, p)
        assert abs(out[0] - math.cos(p)) < 1e-15 and abs(out[D // 2] - math.sin(p)) < 1e-15
        assert np.all(out[[1, 2, 3, 5, 6, 7]] == 0.0)


def test_rope_preserves_pair_norms():
    D = 64
    v = RNG.standard_normal(D)
    out = oracle.rope(v, 1234)
    n_in = np.hypot(v[:D // 2], v[D // 2:])
    n_out = np.hypot(out[:D // 2], out[D // 2:])
    np.testing.assert_allclose(n_out, n_in, rtol=1e-6, atol=0)


def test_rope_relative_position():
    D = 128
    q, k = RNG.standard_normal(D), RNG.standard_normal(D)
    base = oracle.rope(q, 40) @ oracle.rope(k, 13)
    for shift in (1, 100, 1000):
        assert abs(oracle.rope(q, 40 + shift) @ oracle.rope(k, 13 + shift) - base) < 1e-5 * max(1.0, abs(base))


# ----------------------------------------------------------------- RMSNorm
def test_rmsnorm_constant_input_closed_form():
    eps = 1e-6
    for c in (0.5, -3.0, 1e-3):
        y = oracle.rmsnorm(np.full(256, c), None, eps)
        np.testing.assert_allclose(y, c / math.sqrt(c * c + eps), rtol=1e-15)


def test_rmsnorm_output_rms_and_gain():
    eps = 1e-6
    x = RNG.standard_normal(4096) * 3.0
    y = oracle.rmsnorm(x, None, eps)
    ms = np.mean(x * x)
    assert abs(math.sqrt(np.mean(y * y)) - math.sqrt(ms / (ms + eps))) < 1e-12
    g = RNG.standard_normal(4096)
    np.testing.assert_allclose(oracle.rmsnorm(x, g, eps), y * g, rtol=1e-14)
    # library routine
    want = F.rms_norm(torch.from_numpy(x), (4096,), weight=torch.from_numpy(g), eps=eps).numpy()
    np.testing.assert_allclose(oracle.rmsnorm(x, g, eps), want, rtol=1e-12)


# ----------------------------------------------------------------- matvec
def test_matvec_one_hot_and_numpy():
    W = bf16(RNG.standard_normal((37, 300)))
    x = np.zeros(300)
    x[123] = 1.0
    np.testing.assert_array_equal(oracle.matvec(W, x), widen(W)[:, 123])
    x = RNG.standard_normal(300)
    np.testing.assert_allclose(oracle.matvec(W, x), widen(W) @ x, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------- attention
def test_attention_single_position_is_v0():
    D = 64
    q = RNG.standard_normal(D)
    K, V = bf16(RNG.standard_normal((1, D))), bf16(RNG.standard_normal((1, D)))
    o, w = oracle.attention(q, K, V)
    assert w[0] == 1.0
    np.testing.assert_array_equal(o, widen(V)[0])


def test_attention_equal_keys_give_mean_of_values():
    D, T = 64, 37
    q = RNG.standard_normal(D)
    K = np.repeat(bf16(RNG.standard_normal((1, D))), T, axis=0)
    V = bf16(RNG.standard_normal((T, D)))
    o, w = oracle.attention(q, K, V)
    np.testing.assert_allclose(w, 1.0 / T, rtol=1e-14)
    np.testing.assert_allclose(o, widen(V).mean(axis=0), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("T", [2, 33, 2049])
def test_attention_softmax_rows_sum_to_one_and_match_sdpa(T):
    D = 128
    q = RNG.standard_normal(D) * 3.0
    K, V = bf16(RNG.standard_normal((T, D))), bf16(RNG.standard_normal((T, D)))
    o, w = oracle.attention(q, K, V)
    assert abs(w.sum() - 1.0) < 1e-6
    assert np.all(w >= 0)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None, None, None, :],
                                         torch.from_numpy(widen(K))[None, None], torch.from_numpy(widen(V))[None, None])
    np.testing.assert_allclose(o, ref.reshape(D).numpy(), rtol=1e-10, atol=1e-12)


def test_attention_brute_force_tiny():
    # brute force with plain Python loops on a 3-position, 4-dim head
    D, T = 4, 3
    q = RNG.standard_normal(D)
    K, V = bf16(RNG.standard_normal((T, D))), bf16(RNG.standard_normal((T, D)))
    Kd, Vd = widen(K), widen(V)
    s = [sum(q[d] * Kd[t, d] for d in range(D)) / 2.0 for t in range(T)]
    e = [math.exp(v) for v in s]
    want = [sum(e[t] * Vd[t, d] for t in range(T)) / sum(e) for d in range(D)]
    o, _ = oracle.attention(q, K, V)
    np.testing.assert_allclose(o, want, rtol=1e-12)


# ----------------------------------------------------------------- SwiGLU
def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12
    assert abs(oracle.silu(-40.0)) < 1e-12
    for z in (-3.0, -0.5, 0.25, 2.0):
        assert abs(oracle.silu(-z) - (oracle.silu(z) - z)) < 1e-14   # silu(-z) = silu(z) - z
        assert abs(oracle.silu(z) - F.silu(torch.tensor(z, dtype=torch.float64)).item()) < 1e-15


# ----------------------------------------------------------------- routing
def test_route_matches_full_sort_and_renormalises():
    for trial in range(20):
        lg = RNG.standard_normal(128) * 2
        e, w = oracle.route(lg, 8)
        p = np.exp(lg - lg.max())
        p /= p.sum()
        order = np.argsort(-p, kind="stable")[:8]
        np.testing.assert_array_equal(e, order)
        np.testing.assert_allclose(w, p[order] / p[order].sum(), rtol=1e-12)
        assert abs(w.sum() - 1.0) < 1e-12


def test_route_ties_go_to_lower_index():
    lg = np.zeros(16)
    lg[[3, 9, 12]] = 1.0
    e, w = oracle.route(lg, 4)
    np.testing.assert_array_equal(e, [3, 9, 12, 0])


def test_route_gap_hand_written():
    # smallest chosen logit minus largest unchosen logit
    assert oracle.route_gap([3.0, 1.0, 2.0, 0.0], [0, 2]) == 1.0
    assert oracle.route_gap([-5.0, -1.0, -3.0, -2.0], [1, 3]) == 1.0
    assert oracle.route_gap([0.5, 0.25, 4.0], [2]) == 3.5
    # exact ties across the boundary: gap 0, whichever tied expert is chosen
    assert oracle.route_gap([1.0, 1.0, 0.0], [0]) == 0.0
    assert oracle.route_gap([1.0, 1.0, 0.0], [1]) == 0.0
    # a choice that is not a top-k has a negative gap
    assert oracle.route_gap([3.0, 1.0, 2.0, 0.0], [0, 1]) == -1.0
    # every expert chosen: nothing to compare against
    assert oracle.route_gap([1.0, 2.0], [0, 1]) == math.inf


def test_route_weights_closed_form():
    lg = np.array([0.3, -1.2, 2.0, 0.7])
    w = oracle.route_weights(lg, [0, 2])
    ea, ec = math.exp(0.3), math.exp(2.0)
    np.testing.assert_allclose(w, [ea / (ea + ec), ec / (ea + ec)], rtol=1e-14)
    # the weights follow the listed order
    np.testing.assert_allclose(oracle.route_weights(lg, [2, 0]), w[::-1], rtol=1e-15)
    # one expert carries the whole weight
    assert oracle.route_weights(lg, [3])[0] == 1.0
    # the top-k choice gets exactly route()'s weights
    for trial in range(5):
        lg = RNG.standard_normal(64) * 2
        e, want = oracle.route(lg, 6)
        np.testing.assert_array_equal(oracle.route_weights(lg, e), want)


def test_top2_margin_hand_written():
    # top-1 minus top-2 logit, per row; 0 when the two largest tie
    assert oracle.top2_margin(np.array([3.0, 1.0, 2.0])) == 1.0
    assert oracle.top2_margin(np.array([5.0, 5.0, 1.0])) == 0.0
    assert oracle.top2_margin(np.array([-1.0, -3.0, -2.0])) == 1.0
    assert oracle.top2_margin(np.array([0.0, -7.5])) == 7.5
    rows = np.array([[0.0, 0.5, 0.25, 0.125], [2.0, -1.0, 2.0, 1.5], [-4.0, -6.0, -4.5, -9.0]])
    np.testing.assert_array_equal(oracle.top2_margin(rows), [0.25, 0.0, 0.5])


# ----------------------------------------------------------------- whole decoder
MICRO = synth.ModelShape(n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, intermediate=96,
                         vocab=97, tied_embeddings=False)


def _micro_weights(shape, seed=7):
    return synth.weights(shape, seed=seed, threads=1)


def test_incremental_decode_equals_full_recompute():
    ws = _micro_weights(MICRO)
    toks = synth.uniform_i32("pin.tokens", 12, 99, 0, MICRO.vocab - 1)
    o = oracle.Oracle(MICRO, batch=1, cap=16, threads=2)
    o.set_weights(ws)
    for p, t in enumerate(toks):
        lg = o.decode([t], [p])[0]
    full = o.full_forward(toks)
    assert np.linalg.norm(lg - full) <= 1e-9 * np.linalg.norm(full)


@pytest.mark.parametrize("tied", [False, True])
def test_decoder_matches_independent_torch_model(tied):
    shape = dataclasses.replace(MICRO, tied_embeddings=tied)
    ws = _micro_weights(shape)
    toks = synth.uniform_i32("pin.tokens2", 9, 5, 0, shape.vocab - 1)
    o = oracle.Oracle(shape, batch=1, cap=16, threads=1)
    o.set_weights(ws)
    for p, t in enumerate(toks):
        lg = o.decode([t], [p])[0]
    ref = torch_ref.forward_last_logits(shape, ws, toks)
    assert np.linalg.norm(lg - ref) <= 1e-6 * np.linalg.norm(ref)


def test_moe_decoder_matches_independent_torch_model():
    shape = synth.ModelShape(n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=1, head_dim=16, intermediate=0,
                             vocab=61, tied_embeddings=False, n_experts=6, top_k=2, expert_intermediate=32)
    ws = _micro_weights(shape, seed=3)
    toks = synth.uniform_i32("pin.tokens3", 7, 5, 0, shape.vocab - 1)
    o = oracle.Oracle(shape, batch=1, cap=8, threads=1)
    o.set_weights(ws)
    for p, t in enumerate(toks):
        lg = o.decode([t], [p])[0]
    ref = torch_ref.forward_last_logits(shape, ws, toks)
    assert np.linalg.norm(lg - ref) <= 1e-6 * np.linalg.norm(ref)


MOE_MICRO = synth.ModelShape(n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=1, head_dim=16, intermediate=0,
                             vocab=61, tied_embeddings=False, n_experts=6, top_k=2, expert_intermediate=32)


def _moe_run(forced=None):
    ws = _micro_weights(MOE_MICRO, seed=3)
    toks = synth.uniform_i32("pin.tokens3", 7, 5, 0, MOE_MICRO.vocab - 1)
    o = oracle.Oracle(MOE_MICRO, batch=1, cap=8, threads=1)
    o.set_weights(ws)
    for p, t in enumerate(toks[:-1]):
        o.decode([t], [p])
    if forced is not None:
        o.force_routing(np.asarray(forced, dtype=np.int32).reshape(MOE_MICRO.n_layers, 1, MOE_MICRO.top_k))
    lg = o.decode([toks[-1]], [len(toks) - 1])[0]
    return o, ws, toks, lg


def test_router_logits_and_routing_gap_match_torch():
    # the recorded router logits of the last step and the smallest routing gap
    # over the layers, against router logits from the independent torch model
    o, ws, toks, _ = _moe_run()
    rl = []
    torch_ref.forward_last_logits(MOE_MICRO, ws, toks, router_out=rl)
    gaps = []
    for l in range(MOE_MICRO.n_layers):
        np.testing.assert_allclose(o.last_router_logits(l, 0), rl[l], rtol=1e-9, atol=1e-12)
        r = torch.from_numpy(rl[l])
        top = torch.topk(r, MOE_MICRO.top_k).indices
        rest = torch.ones(MOE_MICRO.n_experts, dtype=torch.bool)
        rest[top] = False
        gaps.append(float(r[top].min() - r[rest].max()))
        assert set(o.last_routing(l, 0)[0].tolist()) == set(top.tolist())
    assert abs(o.last_routing_gap(0) - min(gaps)) < 1e-9


def test_forced_routing_matches_torch_with_the_same_choice():
    # the last step evaluated on a choice that is not the top-k: in every layer
    # the second chosen expert is replaced by the best unchosen one
    o, ws, toks, natural = _moe_run()
    forced = []
    for l in range(MOE_MICRO.n_layers):
        e, _ = o.last_routing(l, 0)
        r = o.last_router_logits(l, 0)
        order = np.argsort(-r, kind="stable")
        forced.append([int(e[0]), int(order[MOE_MICRO.top_k])])
    o2, _, _, lg = _moe_run(forced)
    ref = torch_ref.forward_last_logits(MOE_MICRO, ws, toks, forced_last=forced)
    assert np.linalg.norm(lg - ref) <= 1e-6 * np.linalg.norm(ref)
    assert np.linalg.norm(lg - natural) > 1e-3 * np.linalg.norm(natural)  # the choice mattered
    for l in range(MOE_MICRO.n_layers):
        e, w = o2.last_routing(l, 0)
        assert e.tolist() == forced[l]
        assert abs(w.sum() - 1.0) < 1e-12
    # forcing the oracle's own choice changes nothing, bit for bit
    own = [o.last_routing(l, 0)[0].tolist() for l in range(MOE_MICRO.n_layers)]
    _, _, _, same = _moe_run(own)
    np.testing.assert_array_equal(same, natural)


def test_forced_routing_rejects_bad_choices():
    o = oracle.Oracle(MOE_MICRO, batch=1, cap=8, threads=1)
    with pytest.raises(RuntimeError):
        o.force_routing(np.array([[[0, 0]], [[1, 2]]], dtype=np.int32))   # repeated expert
    with pytest.raises(RuntimeError):
        o.force_routing(np.array([[[0, 6]], [[1, 2]]], dtype=np.int32))   # id out of range
    o.force_routing(None)


def test_moe_with_one_expert_reduces_to_dense_mlp():
    dense = dataclasses.replace(MICRO, intermediate=40)
    moe = dataclasses.replace(MICRO, intermediate=0, n_experts=1, top_k=1, expert_intermediate=40)
    wd = _micro_weights(dense)
    wm = {}
    for k, v in wd.items():
        for part in ("w_gate", "w_up", "w_down"):
            if k.endswith("." + part):
                k = k.replace(part, "experts.0." + part)
        wm[k] = v
    for l in range(MICRO.n_layers):
        wm[f"layers.{l}.router"] = synth.normal_bf16(f"r{l}", 64, 1, 0.02).reshape(1, 64)
    a = oracle.Oracle(dense, 1, 8, threads=1)
    a.set_weights(wd)
    b = oracle.Oracle(moe, 1, 8, threads=1)
    b.set_weights(wm)
    for p, t in enumerate([5, 17, 3, 60]):
        la, lb = a.decode([t], [p])[0], b.decode([t], [p])[0]
        np.testing.assert_array_equal(la, lb)
        e, w = b.last_routing(0, 0)
        assert e[0] == 0 and w[0] == 1.0


def test_batch_invariance():
    ws = _micro_weights(MICRO)
    B = 3
    lens = [5, 1, 9]
    many = oracle.Oracle(MICRO, batch=B, cap=16, threads=2)
    many.set_weights(ws)
    kv = [RNG.integers(0, 1 << 16, size=many.K.shape, dtype=np.uint16) for _ in range(2)]
    # keep the random bit patterns finite: clear the exponent's top bit
    kv = [np.where((a & 0x7f80) == 0x7f80, a & 0xbfff, a) for a in kv]
    many.K[...] = kv[0]
    many.V[...] = kv[1]
    toks = np.array([4, 50, 96], dtype=np.int32)
    got = many.decode(toks, lens)
    for b in range(B):
        one = oracle.Oracle(MICRO, batch=1, cap=16, threads=1)
        one.set_weights(ws)
        one.K[...] = many.K[:, b:b + 1]
        one.V[...] = many.V[:, b:b + 1]
        np.testing.assert_array_equal(one.decode([toks[b]], [lens[b]])[0], got[b])


def test_decode_writes_new_kv_rounded_at_position():
    ws = _micro_weights(MICRO)
    o = oracle.Oracle(MICRO, batch=1, cap=16, threads=1)
    o.set_weights(ws)
    before = o.K.copy()
    o.decode([11], [6])
    changed = np.argwhere(np.any(o.K != before, axis=-1))
    assert set(map(tuple, changed[:, [0, 3]])) <= {(l, 6) for l in range(MICRO.n_layers)}
    assert np.all(o.K[:, 0, :, 6] != 0)


def test_greedy_ties_lowest_id():
    lg = np.array([[0.0, 2.0, 2.0, 1.0]])
    assert oracle.greedy(lg)[0] == 1
