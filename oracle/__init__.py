"""Oracle: a plain CPU reference decoder (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package.  It shares no code with the HIP decoder in
``decode_megakernel_persistent_amd``; both only consume the bf16 bytes made by
``synth``.  The arithmetic lives in ``oracle.cpp`` (IEEE double throughout).

Every function here is pinned by ``tests/test_oracle_pins.py`` against values
fixed by mathematics, not by itself (see the header of ``oracle.cpp``).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "oracle.cpp")
    cmd = ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", "-o", _LIB_PATH, src]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


class _Shape(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("expert_intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("tied_embeddings", ctypes.c_int32),
                ("rms_eps", ctypes.c_double), ("rope_theta", ctypes.c_double)]


_dp = ctypes.POINTER(ctypes.c_double)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_last_error.restype = ctypes.c_char_p
    lib.orc_rmsnorm.argtypes = [_dp, _dp, ctypes.c_int64, ctypes.c_double, _dp]
    lib.orc_matvec.argtypes = [_u16p, _dp, ctypes.c_int64, ctypes.c_int64, _dp]
    lib.orc_rope.argtypes = [_dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_double]
    lib.orc_attention.argtypes = [_dp, _u16p, _u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _dp, _dp]
    lib.orc_silu.argtypes = [ctypes.c_double]
    lib.orc_silu.restype = ctypes.c_double
    lib.orc_route.argtypes = [_dp, ctypes.c_int32, ctypes.c_int32, _i32p, _dp]
    lib.orc_create.argtypes = [ctypes.POINTER(_Shape), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    lib.orc_create.restype = ctypes.c_void_p
    lib.orc_destroy.argtypes = [ctypes.c_void_p]
    lib.orc_threads.argtypes = [ctypes.c_void_p]
    lib.orc_threads.restype = ctypes.c_int32
    lib.orc_set_weight.argtypes = [ctypes.c_void_p, ctypes.c_char_p, _u16p, ctypes.c_int64, ctypes.c_int64]
    lib.orc_set_weight.restype = ctypes.c_int32
    lib.orc_kv.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    lib.orc_kv.restype = _u16p
    lib.orc_kv_elems.argtypes = [ctypes.c_void_p]
    lib.orc_kv_elems.restype = ctypes.c_int64
    lib.orc_decode.argtypes = [ctypes.c_void_p, _i32p, _i32p, _dp, _dp]
    lib.orc_decode.restype = ctypes.c_int32
    lib.orc_full_forward.argtypes = [ctypes.c_void_p, _i32p, ctypes.c_int32, _dp]
    lib.orc_full_forward.restype = ctypes.c_int32
    lib.orc_last_routing.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, _i32p, _dp]
    lib.orc_last_routing.restype = ctypes.c_int32
    lib.orc_last_routing_gap.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    lib.orc_last_routing_gap.restype = ctypes.c_double
    lib.orc_route_weights.argtypes = [_dp, ctypes.c_int32, ctypes.c_int32, _i32p, _dp]
    lib.orc_route_gap.argtypes = [_dp, ctypes.c_int32, ctypes.c_int32, _i32p]
    lib.orc_route_gap.restype = ctypes.c_double
    lib.orc_last_router_logits.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, _dp]
    lib.orc_last_router_logits.restype = ctypes.c_int32
    lib.orc_force_routing.argtypes = [ctypes.c_void_p, _i32p]
    lib.orc_force_routing.restype = ctypes.c_int32
    _lib = lib
    return lib


def _d(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


# ----------------------------------------------------------------- primitives
def rmsnorm(x, g=None, eps: float = 1e-6) -> np.ndarray:
    x = _f64(x)
    y = np.empty_like(x)
    gp = _d(_f64(g)) if g is not None else None
    _load().orc_rmsnorm(_d(x), gp, x.size, eps, _d(y))
    return y


def matvec(W_bf16: np.ndarray, x) -> np.ndarray:
    W = np.ascontiguousarray(W_bf16, dtype=np.uint16)
    x = _f64(x)
    y = np.empty(W.shape[0], dtype=np.float64)
    _load().orc_matvec(W.ctypes.data_as(_u16p), _d(x), W.shape[0], W.shape[1], _d(y))
    return y


def rope(v, pos: int, theta: float = 1e6) -> np.ndarray:
    v = _f64(v).copy()
    _load().orc_rope(_d(v), v.size, pos, theta)
    return v


def attention(q, K_bf16: np.ndarray, V_bf16: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(output [D], softmax weights [T]) of one head over T cached bf16 rows."""
    q = _f64(q)
    K = np.ascontiguousarray(K_bf16, dtype=np.uint16)
    V = np.ascontiguousarray(V_bf16, dtype=np.uint16)
    T, D = K.shape
    o = np.empty(D, dtype=np.float64)
    w = np.empty(max(T, 1), dtype=np.float64)
    _load().orc_attention(_d(q), K.ctypes.data_as(_u16p), V.ctypes.data_as(_u16p), T, D, D, _d(o), _d(w))
    return o, w[:T]


def silu(z: float) -> float:
    return _load().orc_silu(float(z))


def route(logits, k: int) -> Tuple[np.ndarray, np.ndarray]:
    lg = _f64(logits)
    e = np.empty(k, dtype=np.int32)
    w = np.empty(k, dtype=np.float64)
    _load().orc_route(_d(lg), lg.size, k, e.ctypes.data_as(_i32p), _d(w))
    return e, w


def route_weights(logits, experts) -> np.ndarray:
    """Weights of a given expert choice: softmax over all logits, renormalised over the choice."""
    lg = _f64(logits)
    e = np.ascontiguousarray(experts, dtype=np.int32)
    w = np.empty(e.size, dtype=np.float64)
    _load().orc_route_weights(_d(lg), lg.size, e.size, e.ctypes.data_as(_i32p), _d(w))
    return w


def route_gap(logits, experts) -> float:
    """Smallest chosen logit minus the largest unchosen one (0 at an exact tie)."""
    lg = _f64(logits)
    e = np.ascontiguousarray(experts, dtype=np.int32)
    return float(_load().orc_route_gap(_d(lg), lg.size, e.size, e.ctypes.data_as(_i32p)))


# ----------------------------------------------------------------- model
class Oracle:
    """The reference decoder for one model shape, batch and cache capacity.

    Weights are borrowed (the caller keeps the numpy arrays alive); the oracle
    owns its own bf16 KV cache [L][B][Hkv][cap][D].
    """

    def __init__(self, shape, batch: int, cap: int, threads: int = 0):
        lib = _load()
        s = _Shape(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                   shape.intermediate, shape.n_experts, shape.top_k, shape.expert_intermediate, shape.vocab,
                   int(shape.tied_embeddings), shape.rms_eps, shape.rope_theta)
        self._h = lib.orc_create(ctypes.byref(s), batch, cap, threads)
        if not self._h:
            raise RuntimeError(lib.orc_last_error().decode())
        self.shape, self.batch, self.cap = shape, batch, cap
        self._keep: Dict[str, np.ndarray] = {}
        n = lib.orc_kv_elems(self._h)
        dims = (shape.n_layers, batch, shape.n_kv_heads, cap, shape.head_dim)
        self.K = np.ctypeslib.as_array(lib.orc_kv(self._h, 0), shape=(n,)).reshape(dims)
        self.V = np.ctypeslib.as_array(lib.orc_kv(self._h, 1), shape=(n,)).reshape(dims)

    @property
    def threads(self) -> int:
        return _load().orc_threads(self._h)

    def close(self):
        if self._h:
            _load().orc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_weight(self, name: str, a: np.ndarray):
        a = np.ascontiguousarray(a, dtype=np.uint16)
        rows = a.shape[0]
        cols = a.shape[1] if a.ndim == 2 else 1
        self._keep[name] = a
        rc = _load().orc_set_weight(self._h, name.encode(), a.ctypes.data_as(_u16p), rows, cols)
        if rc:
            raise RuntimeError(_load().orc_last_error().decode())

    def set_weights(self, ws: Dict[str, np.ndarray]):
        for k, v in ws.items():
            self.set_weight(k, v)

    def decode(self, tokens, positions, want_resid: bool = False):
        """Logits [B, V] (float64) of one decode step; optionally also the final residual [B, H]."""
        t = np.ascontiguousarray(tokens, dtype=np.int32).reshape(self.batch)
        p = np.ascontiguousarray(positions, dtype=np.int32).reshape(self.batch)
        lg = np.empty((self.batch, self.shape.vocab), dtype=np.float64)
        rs = np.empty((self.batch, self.shape.hidden), dtype=np.float64) if want_resid else None
        rc = _load().orc_decode(self._h, t.ctypes.data_as(_i32p), p.ctypes.data_as(_i32p), _d(lg),
                                _d(rs) if rs is not None else None)
        if rc:
            raise RuntimeError(_load().orc_last_error().decode())
        return (lg, rs) if want_resid else lg

    def full_forward(self, tokens) -> np.ndarray:
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        lg = np.empty(self.shape.vocab, dtype=np.float64)
        rc = _load().orc_full_forward(self._h, t.ctypes.data_as(_i32p), t.size, _d(lg))
        if rc:
            raise RuntimeError(_load().orc_last_error().decode())
        return lg

    def last_routing_gap(self, b: int) -> float:
        """Smallest router-logit gap between a chosen and an unchosen expert of
        sequence b over the layers of the last decode (inf for dense models)."""
        return float(_load().orc_last_routing_gap(self._h, b))

    def last_router_logits(self, layer: int, b: int) -> np.ndarray:
        """Router logits [E] of (layer, sequence b) in the last decode step."""
        out = np.empty(self.shape.n_experts, dtype=np.float64)
        if _load().orc_last_router_logits(self._h, layer, b, _d(out)):
            raise RuntimeError("no router logits (dense model or bad index)")
        return out

    def force_routing(self, experts: Optional[np.ndarray]):
        """Evaluate the following decode steps on a given expert choice
        [L][B][top_k] (None: the oracle's own top-k)."""
        if experts is None:
            rc = _load().orc_force_routing(self._h, None)
        else:
            e = np.ascontiguousarray(experts, dtype=np.int32)
            s = self.shape
            assert e.shape == (s.n_layers, self.batch, s.top_k), e.shape
            rc = _load().orc_force_routing(self._h, e.ctypes.data_as(_i32p))
        if rc:
            raise RuntimeError(_load().orc_last_error().decode())

    def last_routing(self, layer: int, b: int) -> Tuple[np.ndarray, np.ndarray]:
        k = self.shape.top_k
        e = np.empty(k, dtype=np.int32)
        w = np.empty(k, dtype=np.float64)
        if _load().orc_last_routing(self._h, layer, b, e.ctypes.data_as(_i32p), _d(w)):
            raise RuntimeError("no routing (dense model)")
        return e, w


def greedy(logits: np.ndarray) -> np.ndarray:
    """argmax over the last axis, ties to the lowest id."""
    return np.argmax(logits, axis=-1).astype(np.int32)


def top2_margin(logits: np.ndarray) -> np.ndarray:
    part = np.partition(logits, -2, axis=-1)
    return part[..., -1] - part[..., -2]
