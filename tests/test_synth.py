"""The seeded generator: its stated definition, re-implemented here in numpy,
and determinism across thread counts."""

import math

import numpy as np

import synth

M = (1 << 64) - 1


def mix64(z):
    z = (z + 0x9E3779B97F4A7C15) & M
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & M
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & M
    z ^= z >> 31
    return z


def fnv1a(s):
    h = 0xcbf29ce484222325
    for ch in s.encode():
        h ^= ch
        h = (h * 0x100000001b3) & M
    return h


def draw(seed, key, i):
    return mix64(mix64(mix64(seed) ^ key) ^ i)


def test_key_and_draw_definition():
    lib = synth._load()
    for name in ("embed", "layers.3.wq", "k.0.0.1"):
        assert lib.synth_key(name.encode()) == fnv1a(name)
    for i in (0, 1, 2, 12345, 2 ** 40 + 7):
        assert lib.synth_draw(5, fnv1a("x"), i) == draw(5, fnv1a("x"), i)


def test_normal_definition_box_muller():
    name, seed, sigma = "layers.0.wk", 0, 0.02
    got = synth.normal_bf16(name, 64, seed, sigma, start=10, threads=1)
    key = fnv1a(name)
    want = []
    for idx in range(10, 74):
        j = idx >> 1
        u1 = 1.0 - (draw(seed, key, 2 * j) >> 11) * 2.0 ** -53
        u2 = (draw(seed, key, 2 * j + 1) >> 11) * 2.0 ** -53
        r = math.sqrt(-2.0 * math.log(u1))
        z = r * (math.sin(2 * math.pi * u2) if idx & 1 else math.cos(2 * math.pi * u2))
        want.append(sigma * z)
    np.testing.assert_array_equal(got, synth.f32_to_bf16(np.array(want, dtype=np.float32)))


def test_deterministic_across_threads_and_slices():
    a = synth.normal_bf16("t", 300001, 3, 1.0, threads=1)
    b = synth.normal_bf16("t", 300001, 3, 1.0, threads=7)
    np.testing.assert_array_equal(a, b)
    c = synth.normal_bf16("t", 1001, 3, 1.0, start=1000, threads=1)
    np.testing.assert_array_equal(a[1000:2001], c)


def test_uniform_ints_in_range_and_moments():
    v = synth.uniform_i32("tokens", 100000, 2, 0, 151935)
    assert v.min() >= 0 and v.max() <= 151935
    assert abs(v.mean() / 151935 - 0.5) < 0.01


def test_normal_moments():
    v = synth.bf16_to_f32(synth.normal_bf16("m", 200000, 0, 1.0)).astype(np.float64)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.01


def test_workload_presets_match_stated_shapes():
    w = synth.WORKLOADS
    s8 = w["qwen3-8b"].shape
    assert (s8.n_layers, s8.hidden, s8.n_q_heads, s8.n_kv_heads, s8.head_dim, s8.intermediate, s8.vocab) == \
        (36, 4096, 32, 8, 128, 12288, 151936)
    # weight bytes of the 8B shape (untied): about 16.4 GB
    assert abs(synth.weight_bytes(s8) / 1e9 - 16.38) < 0.01
    assert w["qwen3-8b-b16"].batch == 16 and w["qwen3-30b-a3b"].batch == 8
    assert w["tiny"].capacity >= 32 + 16
