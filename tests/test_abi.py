"""The C-ABI library: it loads, exports every entry point include/mk.h
declares, shares the caller's HIP runtime, and reports argument errors
synchronously (no device work in this file)."""

import os
import re

import pytest
import torch

import decode_megakernel_persistent_amd as mk
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "mk.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = mk.lib()
    names = declared_functions()
    assert len(names) >= 19
    for n in names:
        assert hasattr(L, n), f"libmk.so does not export {n}"
    assert set(names) == set(mk.EXPORTED)


def test_same_hip_runtime_as_torch():
    path = mk.mk_hip_runtime_path()
    assert path.endswith("libamdhip64.so") or "libamdhip64.so" in path
    torch_lib = os.path.join(os.path.dirname(torch.__file__), "lib")
    assert os.path.realpath(path).startswith(os.path.realpath(torch_lib)), path


def test_struct_sizes_match_header():
    import ctypes
    assert ctypes.sizeof(mk.mk_build_opts) == 16 * 4
    assert ctypes.sizeof(mk.mk_tensor) == 40
    assert mk.TRACE_DTYPE.itemsize == 32


def test_argument_errors_are_synchronous():
    s = synth.WORKLOADS["tiny"].shape
    with pytest.raises(mk.MkError) as e:
        mk.mk_build_graph(s, 0, 64)
    assert e.value.status == mk.MK_ERR_SHAPE and "batch" in str(e.value)
    bad = mk.make_shape(s)
    bad.n_q_heads = 3
    with pytest.raises(mk.MkError) as e:
        mk.mk_build_graph(bad, 1, 64)
    assert e.value.status == mk.MK_ERR_SHAPE
    o = mk.make_opts(num_workers=8)
    o.reserved[0] = 1
    with pytest.raises(mk.MkError):
        mk.mk_build_graph(s, 1, 64, o)
    with pytest.raises(mk.MkError) as e:
        mk.mk_build_graph(s, 8, 64, mk.make_opts(num_workers=8, gemv=mk.MK_GEMV_VALU))
    assert "VALU" in str(e.value)


def test_decode_before_load_is_a_state_error():
    s = synth.WORKLOADS["tiny"].shape
    g = mk.mk_build_graph(s, 1, 64, mk.make_opts(num_workers=8))
    try:
        kv = mk.mk_kv_cache(1, 1, 64)
        with pytest.raises(mk.MkError) as e:
            mk.mk_decode_step(g, 1, 1, kv, 1, 0)
        assert e.value.status == mk.MK_ERR_STATE
        assert "not loaded" in mk.mk_last_error()
    finally:
        mk.mk_destroy_graph(g)


def test_workspace_sizes_and_stats():
    w = synth.WORKLOADS["tiny"]
    g = mk.mk_build_graph(w.shape, 1, w.capacity, mk.make_opts(num_workers=16, trace=1))
    try:
        a, sc, tr = mk.mk_workspace_size(g)
        st = mk.mk_graph_stats(g)
        assert a >= synth.weight_bytes(w.shape) and a % 256 == 0
        assert tr == st.tasks * 32
        assert st.workers == 16 and st.batch == 1 and st.max_ctx == w.capacity
        assert st.gemv == mk.MK_GEMV_VALU
    finally:
        mk.mk_destroy_graph(g)


def test_source_hash_tracks_kernels_not_host_code(tmp_path):
    # profiler counters are tied to the kernels through this hash: an edit of
    # the C-ABI host section keeps it, an edit of device code changes it
    import shutil
    src = os.path.join(ROOT, "decode_megakernel_persistent_amd", "csrc")
    d = tmp_path / "csrc"
    shutil.copytree(src, d)
    h0 = mk.source_hash(str(d))
    assert h0 == mk.source_hash()
    rt = (d / "runtime.hip").read_text()
    assert mk.HOST_SECTION_MARKER.decode() in rt
    (d / "runtime.hip").write_text(rt + "\n// host-side comment\n")
    assert mk.source_hash(str(d)) == h0
    dev = (d / "device.h").read_text()
    (d / "device.h").write_text(dev + "\n// device-side comment\n")
    assert mk.source_hash(str(d)) != h0
