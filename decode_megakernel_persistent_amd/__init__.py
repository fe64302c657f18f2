"""Persistent decode megakernel for MI355X (gfx950): Python binding of libmk.so.

The functions here carry the C ABI's names (include/mk.h) and only marshal
arguments; every step of the decode runs in the library's HIP kernels.  PyTorch
provides device memory and streams.  ``Session`` bundles the buffers one graph
needs (weight arena, scratch, trace, KV cache, token/position/logit tensors).

The library is loaded after torch so that both use the same HIP runtime; a
missing or unloadable library raises immediately (there is no fallback).
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np
import torch  # noqa: F401  (loads the HIP runtime libmk.so must share)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmk.so")


def source_hash(csrc: Optional[str] = None) -> str:
    """Hash of the sources the device kernels and their task tables are built
    from (ties profiler counters to the kernels they were taken on).  Of
    runtime.hip only the kernel part counts: its host section (the C ABI, from
    the line that opens it) launches the kernels but does not change what they
    read or write."""
    import hashlib
    h = hashlib.sha256()
    for f in ("device.h", "runtime.hip", "graph.cpp", "graph.h", "tables.h"):
        with open(os.path.join(csrc or os.path.join(_PKG, "csrc"), f), "rb") as fh:
            data = fh.read()
        if f == "runtime.hip":
            cut = data.find(HOST_SECTION_MARKER)
            if cut < 0:
                raise RuntimeError("runtime.hip: host section marker not found")
            data = data[:cut]
        h.update(data)
    return h.hexdigest()[:16]


HOST_SECTION_MARKER = b"// ==================================================================== host"

MK_OK = 0
MK_ERR_ARG = -1
MK_ERR_SHAPE = -2
MK_ERR_HIP = -3
MK_ERR_NOT_RESIDENT = -4
MK_ERR_TIMEOUT = -5
MK_ERR_TRACE = -6
MK_ERR_STATE = -7
MK_PERSISTENT = 0
MK_LAUNCH_PER_TASK = 1
MK_GEMV_AUTO, MK_GEMV_VALU, MK_GEMV_MFMA = 0, 1, 2

OP_KINDS = ["empty", "embed", "qkv", "attn", "merge", "oproj", "gateup", "down", "lmhead", "router", "route",
            "moe_gu", "moe_down", "combine"]


class MkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


class mk_model_shape(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("expert_intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("tied_embeddings", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_double)]


class mk_build_opts(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("per_task_launch", ctypes.c_int32), ("num_workers", ctypes.c_int32),
                ("trace", ctypes.c_int32), ("attn_chunks", ctypes.c_int32), ("gemv", ctypes.c_int32),
                ("spin_timeout_us", ctypes.c_int32), ("no_fusion", ctypes.c_int32), ("merge_tasks", ctypes.c_int32),
                ("no_watchdog", ctypes.c_int32), ("prefetch_loads", ctypes.c_int32),
                ("late_trigger", ctypes.c_int32), ("lds_ring", ctypes.c_int32),
                ("xcd_rows_pct", ctypes.c_int32), ("reserved", ctypes.c_int32 * 2)]


class mk_tensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("data", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("on_device", ctypes.c_int32)]


class mk_kv_cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("capacity", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("page_table", ctypes.c_void_p), ("n_pages", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class mk_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "tasks", "empty_tasks", "events", "ops", "workers", "launches_per_step", "raw_edges", "reduced_edges",
        "max_tasks_per_worker", "weight_bytes", "arena_bytes", "scratch_bytes", "trace_bytes")] + \
        [(n, ctypes.c_int32) for n in ("batch", "max_ctx", "attn_chunks", "gemv", "ring_kb", "ring_ops")]


TRACE_DTYPE = np.dtype([("task", np.int32), ("worker", np.int16), ("xcc", np.int16), ("t_start", np.uint32),
                        ("t_end", np.uint32), ("dep_seen", np.uint32), ("step", np.uint32),
                        ("clk_start", np.uint32), ("clk_end", np.uint32)])
assert TRACE_DTYPE.itemsize == 32

_lib = None
_vp = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_i64p = ctypes.POINTER(ctypes.c_int64)


def lib():
    """Load libmk.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: run `python -m decode_megakernel_persistent_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "mk_build_graph": [ctypes.POINTER(mk_model_shape), ctypes.c_int32, ctypes.c_int32,
                           ctypes.POINTER(mk_build_opts), ctypes.POINTER(_vp)],
        "mk_workspace_size": [_vp, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t),
                              ctypes.POINTER(ctypes.c_size_t)],
        "mk_load_weights": [_vp, ctypes.POINTER(mk_tensor), ctypes.c_int32, _vp, _vp, _vp, _vp],
        "mk_decode_step": [_vp, _vp, _vp, ctypes.POINTER(mk_kv_cache), _vp, _vp],
        "mk_decode_steps": [_vp, _vp, _vp, ctypes.POINTER(mk_kv_cache), _vp, _vp, ctypes.c_int32, _vp],
        "mk_decode_step_noalloc": [_vp, _vp, _vp, ctypes.POINTER(mk_kv_cache), _vp, _vp],
        "mk_capture_lpt_graph": [_vp, _vp, _vp, ctypes.POINTER(mk_kv_cache), _vp, ctypes.POINTER(_vp)],
        "mk_lpt_graph_launch": [_vp, _vp],
        "mk_set_mode": [_vp, ctypes.c_int32, ctypes.c_int32],
        "mk_check": [_vp],
        "mk_read_trace": [_vp, _vp, ctypes.c_int64, _i64p],
        "mk_check_trace": [_vp, _vp, ctypes.c_int64, ctypes.c_uint32, _u32p],
        "mk_read_counters": [_vp, _u32p, ctypes.c_int64],
        "mk_read_routing": [_vp, ctypes.c_int32, _i32p, _vp, _vp, ctypes.c_int64],
        "mk_stream_read": [_vp, ctypes.c_uint64, _vp, ctypes.c_int32, _vp],
        "mk_simulate": [_vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int64,
                        _i64p, _u32p],
        "mk_graph_stats": [_vp, ctypes.POINTER(mk_stats)],
        "mk_dump_graph": [_vp, ctypes.c_char_p],
        "mk_get_tasks": [_vp, _i32p, ctypes.c_int64],
        "mk_get_events": [_vp, _i32p, ctypes.c_int64],
        "mk_get_worker_lists": [_vp, _i32p, _i32p, ctypes.c_int64],
        "mk_get_raw_edges": [_vp, _i32p, ctypes.c_int64, _i64p],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int32
    L.mk_destroy_graph.argtypes = [_vp]
    L.mk_destroy_graph.restype = None
    L.mk_lpt_graph_destroy.argtypes = [_vp]
    L.mk_lpt_graph_destroy.restype = None
    L.mk_last_error.restype = ctypes.c_char_p
    L.mk_last_error.argtypes = []
    L.mk_hip_runtime_path.restype = ctypes.c_char_p
    L.mk_hip_runtime_path.argtypes = []
    _lib = L
    return L


EXPORTED = ["mk_build_graph", "mk_workspace_size", "mk_load_weights", "mk_decode_step", "mk_decode_steps",
            "mk_decode_step_noalloc",
            "mk_capture_lpt_graph", "mk_lpt_graph_launch", "mk_lpt_graph_destroy", "mk_set_mode", "mk_check",
            "mk_read_trace", "mk_check_trace", "mk_read_counters", "mk_read_routing", "mk_simulate", "mk_graph_stats", "mk_dump_graph",
            "mk_get_tasks", "mk_get_events", "mk_get_worker_lists", "mk_get_raw_edges", "mk_destroy_graph",
            "mk_last_error", "mk_hip_runtime_path", "mk_stream_read"]


def _chk(rc: int, what: str):
    if rc != MK_OK:
        raise MkError(rc, f"{what}: {lib().mk_last_error().decode()}")


def mk_last_error() -> str:
    return lib().mk_last_error().decode()


def mk_hip_runtime_path() -> str:
    return lib().mk_hip_runtime_path().decode()


def make_shape(s) -> mk_model_shape:
    """mk_model_shape from any object with the synth.ModelShape fields."""
    return mk_model_shape(s.n_layers, s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.intermediate, s.n_experts,
                          s.top_k, s.expert_intermediate, s.vocab, int(s.tied_embeddings), s.rms_eps, s.rope_theta)


def make_opts(mode=MK_PERSISTENT, per_task_launch=0, num_workers=0, trace=0, attn_chunks=0, gemv=MK_GEMV_AUTO,
              spin_timeout_us=0, no_fusion=0, merge_tasks=0, no_watchdog=0,
              prefetch_loads=0, late_trigger=0, lds_ring=0, xcd_rows_pct=0) -> mk_build_opts:
    o = mk_build_opts()
    o.mode, o.per_task_launch, o.num_workers, o.trace = mode, per_task_launch, num_workers, trace
    o.attn_chunks, o.gemv, o.spin_timeout_us, o.no_fusion = attn_chunks, gemv, spin_timeout_us, no_fusion
    o.merge_tasks, o.no_watchdog, o.prefetch_loads = merge_tasks, no_watchdog, prefetch_loads
    o.late_trigger, o.lds_ring, o.xcd_rows_pct = late_trigger, lds_ring, xcd_rows_pct
    return o


def mk_build_graph(shape, batch: int, max_ctx: int, opts: Optional[mk_build_opts] = None) -> int:
    sh = shape if isinstance(shape, mk_model_shape) else make_shape(shape)
    out = _vp()
    _chk(lib().mk_build_graph(ctypes.byref(sh), batch, max_ctx, ctypes.byref(opts or make_opts()), ctypes.byref(out)),
         "mk_build_graph")
    return out.value


def mk_destroy_graph(g: int):
    lib().mk_destroy_graph(g)


def mk_workspace_size(g: int) -> Tuple[int, int, int]:
    a, s, t = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _chk(lib().mk_workspace_size(g, ctypes.byref(a), ctypes.byref(s), ctypes.byref(t)), "mk_workspace_size")
    return a.value, s.value, t.value


def _ptr(x) -> Tuple[int, int]:
    """(address, on_device) of a torch tensor or numpy array."""
    if isinstance(x, torch.Tensor):
        return x.data_ptr(), int(x.is_cuda)
    if isinstance(x, np.ndarray):
        assert x.flags.c_contiguous
        return x.ctypes.data, 0
    raise TypeError(type(x))


def mk_load_weights(g: int, tensors: Sequence[Tuple[str, object]], d_arena: int, d_scratch: int, d_trace: int,
                    stream: int = 0):
    """tensors: (name, bf16 data as uint16/int16 numpy array or torch tensor) pairs."""
    arr = (mk_tensor * len(tensors))()
    names = []
    for i, (name, t) in enumerate(tensors):
        addr, dev = _ptr(t)
        shp = tuple(t.shape)
        rows, cols = (shp[0], shp[1]) if len(shp) == 2 else (shp[0], 1)
        names.append(name.encode())
        arr[i] = mk_tensor(names[-1], addr, rows, cols, dev)
    _chk(lib().mk_load_weights(g, arr, len(tensors), d_arena, d_scratch, d_trace or None, stream or None),
         "mk_load_weights")


def mk_decode_step(g: int, d_tokens: int, d_positions: int, kv: mk_kv_cache, d_logits: int, stream: int = 0):
    _chk(lib().mk_decode_step(g, d_tokens, d_positions, ctypes.byref(kv), d_logits, stream or None), "mk_decode_step")


def mk_decode_step_noalloc(g: int, d_tokens: int, d_positions: int, kv: mk_kv_cache, d_logits: int,
                           stream: int = 0):
    _chk(lib().mk_decode_step_noalloc(g, d_tokens, d_positions, ctypes.byref(kv), d_logits, stream or None),
         "mk_decode_step_noalloc")


def mk_stream_read(d_buf: int, nbytes: int, d_sink: int, blocks: int, stream: int = 0):
    _chk(lib().mk_stream_read(d_buf, nbytes, d_sink, blocks, stream or None), "mk_stream_read")


def mk_capture_lpt_graph(g: int, d_tokens: int, d_positions: int, kv: mk_kv_cache, d_logits: int) -> int:
    out = _vp()
    _chk(lib().mk_capture_lpt_graph(g, d_tokens, d_positions, ctypes.byref(kv), d_logits, ctypes.byref(out)),
         "mk_capture_lpt_graph")
    return out.value


def mk_lpt_graph_launch(lg: int, stream: int = 0):
    _chk(lib().mk_lpt_graph_launch(lg, stream or None), "mk_lpt_graph_launch")


def mk_lpt_graph_destroy(lg: int):
    lib().mk_lpt_graph_destroy(lg)


def mk_decode_steps(g: int, d_tokens: int, d_positions: int, kv: mk_kv_cache, d_logits: int, d_tokens_out: int,
                    n_steps: int, stream: int = 0):
    _chk(lib().mk_decode_steps(g, d_tokens, d_positions, ctypes.byref(kv), d_logits, d_tokens_out or None, n_steps,
                               stream or None), "mk_decode_steps")


def mk_set_mode(g: int, mode: int, per_task_launch: int = 0):
    _chk(lib().mk_set_mode(g, mode, per_task_launch), "mk_set_mode")


def mk_check(g: int):
    _chk(lib().mk_check(g), "mk_check")


def mk_read_trace(g: int, cap: int) -> np.ndarray:
    buf = np.zeros(cap, dtype=TRACE_DTYPE)
    n = ctypes.c_int64()
    _chk(lib().mk_read_trace(g, buf.ctypes.data, cap, ctypes.byref(n)), "mk_read_trace")
    return buf[:min(n.value, cap)]


def mk_check_trace(g: int, recs: np.ndarray, step: int, counters: Optional[np.ndarray] = None):
    recs = np.ascontiguousarray(recs, dtype=TRACE_DTYPE)
    cp = counters.ctypes.data_as(_u32p) if counters is not None else None
    _chk(lib().mk_check_trace(g, recs.ctypes.data, len(recs), step, cp), "mk_check_trace")


def mk_read_counters(g: int, n_events: int) -> np.ndarray:
    out = np.zeros(n_events, dtype=np.uint32)
    _chk(lib().mk_read_counters(g, out.ctypes.data_as(_u32p), n_events), "mk_read_counters")
    return out


def mk_read_routing(g: int, shape, batch: int, step: int, with_logits: bool = False):
    """(experts [L,B,K] int32, weights [L,B,K] float32, router logits [L,B,E] float32 or None)
    of step `step` of the last launch of a routed-expert graph (after sync)."""
    L, K, E = shape.n_layers, shape.top_k, shape.n_experts
    e = np.zeros((L, batch, K), dtype=np.int32)
    w = np.zeros((L, batch, K), dtype=np.float32)
    rl = np.zeros((L, batch, E), dtype=np.float32) if with_logits else None
    cap = max(e.size, rl.size if rl is not None else 0)
    _chk(lib().mk_read_routing(g, step, e.ctypes.data_as(_i32p), w.ctypes.data,
                               rl.ctypes.data if rl is not None else None, cap), "mk_read_routing")
    return e, w, rl


def mk_simulate(g: int, steps: int = 1, fault: int = 0, timeout_ms: int = 2000, threads: int = 0):
    """(trace records of the last step, final counters) from the host-thread protocol simulator."""
    st = mk_graph_stats(g)
    recs = np.zeros(st.tasks, dtype=TRACE_DTYPE)
    cnt = np.zeros(max(st.events, 1), dtype=np.uint32)
    n = ctypes.c_int64()
    _chk(lib().mk_simulate(g, threads, steps, fault, timeout_ms, recs.ctypes.data, st.tasks, ctypes.byref(n),
                           cnt.ctypes.data_as(_u32p)), "mk_simulate")
    return recs[:n.value], cnt[:st.events]


def mk_graph_stats(g: int) -> mk_stats:
    s = mk_stats()
    _chk(lib().mk_graph_stats(g, ctypes.byref(s)), "mk_graph_stats")
    return s


def mk_dump_graph(g: int, path: str):
    _chk(lib().mk_dump_graph(g, path.encode()), "mk_dump_graph")


def mk_get_tasks(g: int) -> np.ndarray:
    n = mk_graph_stats(g).tasks
    rows = np.zeros((n, 8), dtype=np.int32)
    _chk(lib().mk_get_tasks(g, rows.ctypes.data_as(_i32p), n), "mk_get_tasks")
    return rows


def mk_get_events(g: int) -> np.ndarray:
    n = mk_graph_stats(g).events
    rows = np.zeros((max(n, 1), 4), dtype=np.int32)
    _chk(lib().mk_get_events(g, rows.ctypes.data_as(_i32p), n), "mk_get_events")
    return rows[:n]


def mk_get_worker_lists(g: int) -> Tuple[np.ndarray, np.ndarray]:
    st = mk_graph_stats(g)
    off = np.zeros(st.workers + 2, dtype=np.int32)
    ids = np.zeros(st.tasks, dtype=np.int32)
    _chk(lib().mk_get_worker_lists(g, off.ctypes.data_as(_i32p), ids.ctypes.data_as(_i32p), st.tasks),
         "mk_get_worker_lists")
    return off, ids


def mk_get_raw_edges(g: int) -> np.ndarray:
    n = ctypes.c_int64()
    _chk(lib().mk_get_raw_edges(g, None, 0, ctypes.byref(n)), "mk_get_raw_edges")
    rows = np.zeros((max(n.value, 1), 2), dtype=np.int32)
    _chk(lib().mk_get_raw_edges(g, rows.ctypes.data_as(_i32p), n.value, ctypes.byref(n)), "mk_get_raw_edges")
    return rows[:n.value]


# ----------------------------------------------------------------- session
class Session:
    """One compiled graph plus the caller-owned device buffers it runs on."""

    def __init__(self, shape, batch: int, max_ctx: int, opts: Optional[mk_build_opts] = None,
                 device: str = "cuda:0", page_size: int = 0, spare_pages: int = 0, page_seed: int = 0):
        """page_size > 0: a paged KV cache (pools [L][n_pages][Hkv][page_size][D]
        and a page table [B][max_ctx / page_size]); every sequence's logical
        pages are spread over the pool by a seeded random permutation, with
        `spare_pages` pages left unused."""
        self.shape, self.batch, self.max_ctx = shape, batch, max_ctx
        self.device = torch.device(device)
        self.opts = opts or make_opts()
        self.g = mk_build_graph(shape, batch, max_ctx, self.opts)
        self.stats = mk_graph_stats(self.g)
        arena, scratch, trace = mk_workspace_size(self.g)
        self.arena = torch.empty(arena, dtype=torch.uint8, device=self.device)
        self.scratch = torch.empty(scratch, dtype=torch.uint8, device=self.device)
        self.trace_buf = torch.empty(max(trace, 1), dtype=torch.uint8, device=self.device) if trace else None
        L, Hkv, D = shape.n_layers, shape.n_kv_heads, shape.head_dim
        self.page_size = page_size
        if page_size:
            if max_ctx % page_size:
                raise ValueError("max_ctx must be a multiple of page_size")
            pps = max_ctx // page_size
            self.n_pages = batch * pps + spare_pages
            perm = np.random.default_rng(page_seed).permutation(self.n_pages)[:batch * pps]
            self.page_table_host = perm.reshape(batch, pps).astype(np.int32)
            self.page_table = torch.as_tensor(self.page_table_host, device=self.device)
            # k_cache / v_cache hold the pools in this mode
            self.k_cache = torch.zeros((L, self.n_pages, Hkv, page_size, D), dtype=torch.int16, device=self.device)
            self.v_cache = torch.zeros_like(self.k_cache)
            self.kv = mk_kv_cache(self.k_cache.data_ptr(), self.v_cache.data_ptr(), max_ctx, page_size,
                                  self.page_table.data_ptr(), self.n_pages, 0)
        else:
            self.n_pages = 0
            self.k_cache = torch.zeros((L, batch, Hkv, max_ctx, D), dtype=torch.int16, device=self.device)
            self.v_cache = torch.zeros_like(self.k_cache)
            self.kv = mk_kv_cache(self.k_cache.data_ptr(), self.v_cache.data_ptr(), max_ctx, 0, None, 0, 0)
        self.tokens = torch.zeros(batch, dtype=torch.int32, device=self.device)
        self.positions = torch.zeros(batch, dtype=torch.int32, device=self.device)
        self.logits = torch.zeros((batch, shape.vocab), dtype=torch.float32, device=self.device)
        self.steps = 0

    def close(self):
        for h in getattr(self, "_lpt_graphs", []):
            mk_lpt_graph_destroy(h)
        self._lpt_graphs = []
        if getattr(self, "g", None):
            mk_destroy_graph(self.g)
            self.g = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def stream(self) -> int:
        return torch.cuda.current_stream(self.device).cuda_stream

    def load(self, weights: Dict[str, np.ndarray], upload: bool = True):
        """Repack bf16 weights (numpy uint16 arrays) into the arena.  With upload=True
        each tensor is first copied to the device, so the library repacks device to device."""
        items: List[Tuple[str, object]] = []
        for name, a in weights.items():
            if upload:
                t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(self.device)
            else:
                t = np.ascontiguousarray(a)
            items.append((name, t))
        mk_load_weights(self.g, items, self.arena.data_ptr(), self.scratch.data_ptr(),
                        self.trace_buf.data_ptr() if self.trace_buf is not None else 0, self.stream)
        torch.cuda.synchronize(self.device)
        del items

    def set_kv(self, k: np.ndarray, v: np.ndarray):
        """Copy host bf16 caches [L][B][Hkv][cap][D] into the device caches
        (scattered into their pages when the cache is paged)."""
        for dst, src in ((self.k_cache, k), (self.v_cache, v)):
            t = torch.from_numpy(np.ascontiguousarray(src).view(np.int16))
            if not self.page_size:
                dst.copy_(t)
                continue
            L, B, Hkv, cap, D = t.shape
            P = self.page_size
            pages = t.reshape(L, B, Hkv, cap // P, P, D).permute(0, 1, 3, 2, 4, 5).reshape(L, B * (cap // P), Hkv, P, D)
            dst[:, torch.as_tensor(self.page_table_host.reshape(-1), dtype=torch.long, device=self.device)] = \
                pages.to(self.device)

    def kv_contiguous(self) -> Tuple[torch.Tensor, torch.Tensor]:
        """The caches as device tensors [L][B][Hkv][cap][D] (gathered from their pages when paged)."""
        if not self.page_size:
            return self.k_cache, self.v_cache
        L, B, P = self.shape.n_layers, self.batch, self.page_size
        idx = torch.as_tensor(self.page_table_host.reshape(-1), dtype=torch.long, device=self.device)
        out = []
        for pool in (self.k_cache, self.v_cache):
            g = pool[:, idx]  # [L][B*pps][Hkv][P][D]
            Hkv, D = g.shape[2], g.shape[4]
            out.append(g.reshape(L, B, self.max_ctx // P, Hkv, P, D).permute(0, 1, 3, 2, 4, 5)
                       .reshape(L, B, Hkv, self.max_ctx, D))
        return out[0], out[1]

    def step(self, tokens, positions):
        """Enqueue one decode step; returns the device logits tensor [B, V] (valid after sync)."""
        self.tokens.copy_(torch.as_tensor(np.asarray(tokens, dtype=np.int32).reshape(self.batch)))
        self.positions.copy_(torch.as_tensor(np.asarray(positions, dtype=np.int32).reshape(self.batch)))
        self.enqueue()
        return self.logits

    def enqueue(self):
        """One decode step on the current tokens/positions tensors (no host copies)."""
        mk_decode_step(self.g, self.tokens.data_ptr(), self.positions.data_ptr(), self.kv, self.logits.data_ptr(),
                       self.stream)
        self.steps += 1

    def decode(self, tokens, positions, n_steps: int):
        """Enqueue n_steps greedy steps in one persistent launch, starting from
        tokens at positions; returns the device tensor [n_steps, B] of greedy
        tokens (valid after sync).  self.logits holds the last step's logits."""
        self.tokens.copy_(torch.as_tensor(np.asarray(tokens, dtype=np.int32).reshape(self.batch)))
        self.positions.copy_(torch.as_tensor(np.asarray(positions, dtype=np.int32).reshape(self.batch)))
        out = torch.full((n_steps, self.batch), -1, dtype=torch.int32, device=self.device)
        mk_decode_steps(self.g, self.tokens.data_ptr(), self.positions.data_ptr(), self.kv, self.logits.data_ptr(),
                        out.data_ptr(), n_steps, self.stream)
        self.steps += n_steps
        return out

    def capture_lpt_graph(self) -> int:
        """Capture one launch-per-task step on this session's buffers into a HIP
        graph; replay with replay_lpt_graph after writing tokens/positions."""
        torch.cuda.synchronize(self.device)
        h = mk_capture_lpt_graph(self.g, self.tokens.data_ptr(), self.positions.data_ptr(), self.kv,
                                 self.logits.data_ptr())
        self._lpt_graphs = getattr(self, "_lpt_graphs", []) + [h]
        return h

    def replay_lpt_graph(self, h: int):
        mk_lpt_graph_launch(h, self.stream)
        self.steps += 1

    def set_mode(self, mode: int, per_task_launch: int = 0):
        mk_set_mode(self.g, mode, per_task_launch)

    def check(self):
        torch.cuda.synchronize(self.device)
        mk_check(self.g)

    def read_trace(self) -> np.ndarray:
        torch.cuda.synchronize(self.device)
        return mk_read_trace(self.g, self.stats.tasks)

    def read_counters(self) -> np.ndarray:
        torch.cuda.synchronize(self.device)
        return mk_read_counters(self.g, self.stats.events)

    def read_routing(self, step: int = 0, with_logits: bool = True):
        """Expert choice (and, for the launch's last step, router logits) of step
        `step` of the last launch: see mk_read_routing."""
        torch.cuda.synchronize(self.device)
        return mk_read_routing(self.g, self.shape, self.batch, step, with_logits)

    def kv_rows(self, positions) -> Tuple[np.ndarray, np.ndarray]:
        """Host copies of the K and V cache rows at positions[b] of every
        layer, sequence and kv head: two bf16 arrays [L][B][Hkv][D] (uint16)."""
        torch.cuda.synchronize(self.device)
        p = np.asarray(positions, dtype=np.int64).reshape(self.batch)
        if self.page_size:
            P = self.page_size
            bi = torch.as_tensor(self.page_table_host[np.arange(self.batch), p // P].astype(np.int64), device=self.device)
            pos = torch.as_tensor(p % P, device=self.device)
        else:
            bi = torch.arange(self.batch, device=self.device)
            pos = torch.as_tensor(p, device=self.device)
        # advanced indices split by a slice: the (sequence, row) axis comes first, [B][L][Hkv][D]
        k = self.k_cache[:, bi, :, pos, :].permute(1, 0, 2, 3)
        v = self.v_cache[:, bi, :, pos, :].permute(1, 0, 2, 3)
        return (k.contiguous().cpu().numpy().view(np.uint16), v.contiguous().cpu().numpy().view(np.uint16))

    def check_trace(self, recs: np.ndarray, step: int, counters: Optional[np.ndarray] = None):
        mk_check_trace(self.g, recs, step, counters)
