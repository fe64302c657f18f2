"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* the graph compiler, the protocol simulator and the trace checker
  (``csrc/graph.cpp``, ``csrc/sim.cpp``) through the ``sim_main`` driver, over
  dense and routed-expert graphs, both merge modes, normalised graphs with
  empty tasks and an odd worker count;
* the oracle (``oracle/oracle.cpp``) through ``tests/sanitize/oracle_main.cpp``:
  its primitives at their edge cases, and dense (tied and untied) and
  routed-expert decoders over ragged positions including position 0, forced
  routing and the full causal recompute.

Any report aborts the program (``-fno-sanitize-recover=all``), so a zero exit
status with the driver's last line means no finding.
"""

import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN_ENV = {**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def test_compiler_and_simulator_under_asan_ubsan():
    from decode_megakernel_persistent_amd import build as b
    exe = b.build_asan()
    r = subprocess.run([exe, "8", "3", "all"], capture_output=True, text=True, timeout=600, env=SAN_ENV)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    assert r.stdout.count("steps ok") == 7


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-pthread", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "oracle", "oracle.cpp"), os.path.join(HERE, "sanitize", "oracle_main.cpp"),
                    "-o", exe], check=True, timeout=600)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=SAN_ENV)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    assert r.stdout.strip().endswith("oracle ok")
