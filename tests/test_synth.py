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
    # the stated single-precision Box-Muller, re-implemented with numpy float32;
    # libm and numpy may differ by an ulp in logf/cosf, which can move a value
    # across a bf16 rounding boundary, so a few one-ulp differences are allowed
    name, seed, sigma = "layers.0.wk", 0, 0.02
    n, start = 4096, 10
    got = synth.normal_bf16(name, n, seed, sigma, start=start, threads=1)
    key = fnv1a(name)
    idx = np.arange(start, start + n)
    pairs = idx >> 1
    d1 = np.array([draw(seed, key, int(2 * j)) for j in pairs], dtype=np.uint64)
    d2 = np.array([draw(seed, key, int(2 * j + 1)) for j in pairs], dtype=np.uint64)
    u1 = np.float32(1.0) - (d1 >> np.uint64(40)).astype(np.float32) * np.float32(2.0 ** -24)
    u2 = (d2 >> np.uint64(40)).astype(np.float32) * np.float32(2.0 ** -24)
    r = np.sqrt(np.float32(-2.0) * np.log(u1))
    a = np.float32(6.28318530717958647692) * u2
    z = np.where(idx & 1, r * np.sin(a), r * np.cos(a)).astype(np.float32)
    want = synth.f32_to_bf16(np.float32(sigma) * z)
    diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
    assert diff.max() <= 1 and np.count_nonzero(diff) <= n // 100


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
