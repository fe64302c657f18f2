"""Seeded synthetic inputs for the decode workloads.

This module is shared by the oracle side and the HIP side.  It holds none of
the decoder's arithmetic: it only defines the workload shapes and turns
(seed, tensor name, element index) into bf16 weights, bf16 KV-cache entries,
token ids and sequence lengths (generator definition in ``synth.c``).

Input recipe (the pages measure on Qwen3 checkpoints and a fixed prompt; none
is available here, so random tensors of the same shapes stand in for them):

* every weight matrix (embeddings, projections, router, lm_head): N(0, 0.02),
  rounded to bf16; norm gains: 1.0
* pre-filled KV-cache entries: N(0, 1) bf16, taken as already normalised and
  rotated keys
* token ids: uniform over the vocabulary; batch-16 lengths: uniform in [1, 2048]
* seeds: weights 0, KV 1, tokens 2, lengths 3
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Dict, Iterator, List, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmksynth.so")
_lib = None

SEED_WEIGHTS = 0
SEED_KV = 1
SEED_TOKENS = 2
SEED_LENGTHS = 3
WEIGHT_SIGMA = 0.02


def build(verbose: bool = False) -> str:
    """Compile synth.c into libmksynth.so next to it."""
    import subprocess

    src = os.path.join(_HERE, "synth.c")
    cmd = ["gcc", "-O3", "-shared", "-fPIC", "-pthread", "-o", _LIB_PATH, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.synth_key.argtypes = [ctypes.c_char_p]
    lib.synth_key.restype = ctypes.c_uint64
    lib.synth_draw.argtypes = [ctypes.c_uint64] * 3
    lib.synth_draw.restype = ctypes.c_uint64
    lib.synth_normal.argtypes = [ctypes.c_uint64] * 3
    lib.synth_normal.restype = ctypes.c_double
    lib.synth_fill_normal_bf16.argtypes = [u16p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                           ctypes.c_double, ctypes.c_int]
    lib.synth_fill_normal_bf16.restype = ctypes.c_int
    lib.synth_fill_uniform_i32.argtypes = [i32p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                           ctypes.c_int32, ctypes.c_int32]
    lib.synth_fill_uniform_i32.restype = ctypes.c_int
    lib.synth_fill_const_bf16.argtypes = [u16p, ctypes.c_int64, ctypes.c_float]
    lib.synth_fill_const_bf16.restype = ctypes.c_int
    _lib = lib
    return lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, 64))


# ----------------------------------------------------------------- shapes
@dataclasses.dataclass(frozen=True)
class ModelShape:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    tied_embeddings: bool
    n_experts: int = 0
    top_k: int = 0
    expert_intermediate: int = 0
    rms_eps: float = 1e-6
    rope_theta: float = 1e6

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    batch: int
    context: int          # pre-filled KV length (per sequence unless ragged)
    steps: int            # decode steps
    ragged: bool = False  # lengths ~ U{1..context} per sequence
    prompt: int = 0       # >0: prompt tokens prefilled by the oracle (tiny config)

    @property
    def capacity(self) -> int:
        """KV-cache slots per sequence: every position a run can write, rounded up to 32."""
        need = max(self.context, self.prompt) + self.steps + 1
        return (need + 31) // 32 * 32


TINY = ModelShape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=768, vocab=4096,
                  tied_embeddings=False)
QWEN3_06B = ModelShape(n_layers=28, hidden=1024, n_q_heads=16, n_kv_heads=8, head_dim=128, intermediate=3072,
                       vocab=151936, tied_embeddings=True)
QWEN3_17B = ModelShape(n_layers=28, hidden=2048, n_q_heads=16, n_kv_heads=8, head_dim=128, intermediate=6144,
                       vocab=151936, tied_embeddings=True)
QWEN3_8B = ModelShape(n_layers=36, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, intermediate=12288,
                      vocab=151936, tied_embeddings=False)
QWEN3_30B_A3B = ModelShape(n_layers=48, hidden=2048, n_q_heads=32, n_kv_heads=4, head_dim=128, intermediate=0,
                           vocab=151936, tied_embeddings=False, n_experts=128, top_k=8, expert_intermediate=768)

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", TINY, batch=1, context=0, steps=16, prompt=32),
    "qwen3-0.6b": Workload("qwen3-0.6b", QWEN3_06B, batch=1, context=512, steps=32),
    "qwen3-1.7b": Workload("qwen3-1.7b", QWEN3_17B, batch=1, context=1024, steps=32),
    "qwen3-8b": Workload("qwen3-8b", QWEN3_8B, batch=1, context=2048, steps=32),
    "qwen3-8b-b16": Workload("qwen3-8b-b16", QWEN3_8B, batch=16, context=2048, steps=32, ragged=True),
    "qwen3-30b-a3b": Workload("qwen3-30b-a3b", QWEN3_30B_A3B, batch=8, context=1024, steps=16),
}


def tensor_specs(s: ModelShape) -> List[Tuple[str, int, int, str]]:
    """(name, rows, cols, kind) for every logical tensor; kind is 'w' (N(0,0.02)) or 'g' (gain 1.0).

    Matrices are row-major [out, in] as in nn.Linear; vectors use cols = 1.
    """
    H, D, Hq, Hkv = s.hidden, s.head_dim, s.n_q_heads, s.n_kv_heads
    out = [("embed", s.vocab, H, "w")]
    for l in range(s.n_layers):
        p = f"layers.{l}."
        out += [(p + "in_norm", H, 1, "g"), (p + "wq", Hq * D, H, "w"), (p + "wk", Hkv * D, H, "w"),
                (p + "wv", Hkv * D, H, "w"), (p + "q_norm", D, 1, "g"), (p + "k_norm", D, 1, "g"),
                (p + "wo", H, Hq * D, "w"), (p + "post_norm", H, 1, "g")]
        if s.n_experts == 0:
            I = s.intermediate
            out += [(p + "w_gate", I, H, "w"), (p + "w_up", I, H, "w"), (p + "w_down", H, I, "w")]
        else:
            Ie = s.expert_intermediate
            out.append((p + "router", s.n_experts, H, "w"))
            for e in range(s.n_experts):
                q = p + f"experts.{e}."
                out += [(q + "w_gate", Ie, H, "w"), (q + "w_up", Ie, H, "w"), (q + "w_down", H, Ie, "w")]
    out.append(("final_norm", H, 1, "g"))
    if not s.tied_embeddings:
        out.append(("lm_head", s.vocab, H, "w"))
    return out


def weight_bytes(s: ModelShape) -> int:
    return sum(r * c * 2 for _, r, c, _ in tensor_specs(s))


def normal_bf16(name: str, n: int, seed: int, sigma: float, start: int = 0,
                threads: Optional[int] = None, out: Optional[np.ndarray] = None) -> np.ndarray:
    """n bf16 values (as uint16) of tensor `name`, elements start..start+n-1."""
    lib = _load()
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == n
    if n:
        lib.synth_fill_normal_bf16(out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), n, seed,
                                   lib.synth_key(name.encode()), start, sigma, threads or default_threads())
    return out


def const_bf16(n: int, value: float) -> np.ndarray:
    lib = _load()
    out = np.empty(n, dtype=np.uint16)
    if n:
        lib.synth_fill_const_bf16(out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), n, value)
    return out


def uniform_i32(name: str, n: int, seed: int, lo: int, hi: int, start: int = 0) -> np.ndarray:
    lib = _load()
    out = np.empty(n, dtype=np.int32)
    if n:
        rc = lib.synth_fill_uniform_i32(out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n, seed,
                                        lib.synth_key(name.encode()), start, lo, hi)
        assert rc == 0
    return out


def tensor(s: ModelShape, name: str, rows: int, cols: int, kind: str, seed: int = SEED_WEIGHTS,
           threads: Optional[int] = None) -> np.ndarray:
    if kind == "g":
        return const_bf16(rows * cols, 1.0).reshape(rows, cols) if cols > 1 else const_bf16(rows, 1.0)
    a = normal_bf16(name, rows * cols, seed, WEIGHT_SIGMA, threads=threads)
    return a.reshape(rows, cols) if cols > 1 else a


def iter_weights(s: ModelShape, seed: int = SEED_WEIGHTS, threads: Optional[int] = None
                 ) -> Iterator[Tuple[str, np.ndarray]]:
    for name, rows, cols, kind in tensor_specs(s):
        yield name, tensor(s, name, rows, cols, kind, seed, threads)


def weights(s: ModelShape, seed: int = SEED_WEIGHTS, threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    return dict(iter_weights(s, seed, threads))


def lengths(w: Workload) -> np.ndarray:
    """Pre-filled KV length of each sequence."""
    if w.prompt:
        return np.full(w.batch, w.prompt, dtype=np.int32)
    if w.ragged:
        return uniform_i32("lengths", w.batch, SEED_LENGTHS, 1, w.context)
    return np.full(w.batch, w.context, dtype=np.int32)


def tokens(w: Workload, count: Optional[int] = None, name: str = "tokens") -> np.ndarray:
    """`count` token ids per sequence, shape [batch, count] (default: the prompt, or one start token)."""
    n = count if count is not None else max(w.prompt, 1)
    return uniform_i32(name, w.batch * n, SEED_TOKENS, 0, w.shape.vocab - 1).reshape(w.batch, n)


def kv_entries(s: ModelShape, layer: int, b: int, g: int, which: str, n: int, seed: int = SEED_KV) -> np.ndarray:
    """n pre-filled positions of K (which='k') or V of (layer, sequence b, kv head g): [n, head_dim] bf16."""
    name = f"{which}.{layer}.{b}.{g}"
    return normal_bf16(name, n * s.head_dim, seed, 1.0, threads=1 if n * s.head_dim < 65536 else None
                       ).reshape(n, s.head_dim)


def fill_kv(s: ModelShape, batch: int, cap: int, lens: np.ndarray, k_out: np.ndarray, v_out: np.ndarray,
            seed: int = SEED_KV) -> None:
    """Fill contiguous caches [L][B][Hkv][cap][D] (uint16) with N(0,1) bf16 for positions < lens[b]; zeros after."""
    assert k_out.shape == (s.n_layers, batch, s.n_kv_heads, cap, s.head_dim)
    k_out[...] = 0
    v_out[...] = 0
    for l in range(s.n_layers):
        for b in range(batch):
            n = int(lens[b])
            for g in range(s.n_kv_heads):
                k_out[l, b, g, :n] = kv_entries(s, l, b, g, "k", n, seed)
                v_out[l, b, g, :n] = kv_entries(s, l, b, g, "v", n, seed)


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 bits (finite inputs)."""
    x = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    x = x + 0x7FFF + ((x >> 16) & 1)
    return (x >> 16).astype(np.uint16)
