"""Shared run protocol of the parity tests.

Teacher forcing: every step feeds both the oracle and the GPU decoder the
oracle's greedy token, each keeping its own KV cache, so one near-tie flip on
the GPU cannot cascade into later steps.

Comparison per sequence and step: logits relative L2 error <= 1e-2, and the
greedy token must match whenever the oracle's top-1 minus top-2 logit exceeds
0.05 (the stated tolerances of the workload).
"""

from __future__ import annotations

import dataclasses
import sys
import time
from typing import Dict, List, Optional

import numpy as np

import oracle
import synth

REL_L2_TOL = 1e-2
MARGIN = 0.05
# Routed experts: the expert choice is an integer decided by floating point.
# The GPU decides it in fp32 from its own router logits, the oracle in fp64; a
# (step, sequence) whose oracle routing gap (smallest chosen minus largest
# unchosen router logit, over all layers) is below this may legitimately
# route differently, so it is not compared (both results are correct).  The
# GPU's hidden state is within ~1e-5 relative of the oracle's, so its router
# logits (|r| ~ 1) are within ~1e-5..1e-4 absolute; 3e-4 leaves a margin.
ROUTE_GAP_TOL = 3e-4


@dataclasses.dataclass
class Prepared:
    workload: synth.Workload
    weights: Dict[str, np.ndarray]
    orc: oracle.Oracle
    k0: np.ndarray          # initial caches (copy of the oracle's)
    v0: np.ndarray
    tokens: np.ndarray      # first step's tokens [B]
    positions: np.ndarray   # first step's positions [B]


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def prepare(w: synth.Workload, threads: int = 0, weights: Optional[Dict[str, np.ndarray]] = None) -> Prepared:
    s = w.shape
    t0 = time.time()
    ws = weights if weights is not None else synth.weights(s, threads=threads or None)
    orc = oracle.Oracle(s, w.batch, w.capacity, threads=threads)
    orc.set_weights(ws)
    lens = synth.lengths(w)
    if w.prompt:
        # the oracle prefills the prompt one position at a time
        prompt = synth.tokens(w, w.prompt)
        for p in range(w.prompt):
            lg = orc.decode(prompt[:, p], np.full(w.batch, p, dtype=np.int32))
        tokens = oracle.greedy(lg)
        positions = np.full(w.batch, w.prompt, dtype=np.int32)
    else:
        synth.fill_kv(s, w.batch, w.capacity, lens, orc.K, orc.V)
        tokens = synth.tokens(w, 1)[:, 0].copy()
        positions = lens.astype(np.int32).copy()
    log(f"[prepare] {w.name}: weights+cache ready in {time.time() - t0:.1f}s")
    return Prepared(w, ws, orc, orc.K.copy(), orc.V.copy(), tokens, positions)


def compare(lg_gpu: np.ndarray, lg_orc: np.ndarray, gaps: Optional[List[float]] = None) -> List[dict]:
    out = []
    for b in range(lg_orc.shape[0]):
        if gaps is not None and gaps[b] < ROUTE_GAP_TOL:
            out.append(dict(rel_l2=0.0, margin=0.0, tok_oracle=int(np.argmax(lg_orc[b])),
                            tok_gpu=int(np.argmax(lg_gpu[b])), ok=True, exempt=True, route_gap=gaps[b]))
            continue
        ref = lg_orc[b]
        err = float(np.linalg.norm(lg_gpu[b].astype(np.float64) - ref) / np.linalg.norm(ref))
        margin = float(oracle.top2_margin(ref))
        tok_o = int(np.argmax(ref))
        tok_g = int(np.argmax(lg_gpu[b]))
        out.append(dict(rel_l2=err, margin=margin, tok_oracle=tok_o, tok_gpu=tok_g,
                        ok=(err <= REL_L2_TOL) and (tok_o == tok_g or margin <= MARGIN)))
    return out
