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
# Routed experts: the expert choice is an integer decided by floating point,
# in fp32 on the GPU (from its own router logits) and in fp64 in the oracle,
# so the two may choose differently where two router logits are within
# rounding of each other.  The GPU's choice is never exempted:
#  - its router logits are logits too: relative L2 error <= REL_L2_TOL against
#    the oracle's (evaluated on the same choice of the earlier layers);
#  - its choice must be the exact top-k of its own router logits;
#  - its choice must be a top-k of the oracle's router logits up to twice the
#    GPU's measured router-logit error on that row (what two valid decisions
#    within that error can differ by), or up to ROUTE_GAP_REL of the row's RMS
#    for steps whose GPU router logits are not kept (earlier steps of a
#    multi-step launch);
#  - where it differs from the oracle's own top-k, the oracle is re-run on the
#    GPU's choice (the same definition, the other valid decision) and the
#    logits are compared with that.
ROUTE_GAP_REL = 2e-3


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


def prepare(w: synth.Workload, threads: int = 0, weights: Optional[Dict[str, np.ndarray]] = None,
            lens: Optional[np.ndarray] = None) -> Prepared:
    """Weights, the oracle and the initial caches of a workload.  ``lens``
    (optional) overrides the pre-filled length of each sequence: N(0,1)
    entries at positions < lens[b], and the first step at position lens[b]."""
    s = w.shape
    t0 = time.time()
    ws = weights if weights is not None else synth.weights(s, threads=threads or None)
    orc = oracle.Oracle(s, w.batch, w.capacity, threads=threads)
    orc.set_weights(ws)
    if lens is not None:
        lens = np.asarray(lens, dtype=np.int32)
        synth.fill_kv(s, w.batch, w.capacity, lens, orc.K, orc.V)
        tokens = synth.tokens(w, 1)[:, 0].copy()
        log(f"[prepare] {w.name}: weights+cache ready in {time.time() - t0:.1f}s (lengths {lens.tolist()})")
        return Prepared(w, ws, orc, orc.K.copy(), orc.V.copy(), tokens, lens.copy())
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


def compare(lg_gpu: np.ndarray, lg_orc: np.ndarray) -> List[dict]:
    out = []
    for b in range(lg_orc.shape[0]):
        ref = lg_orc[b]
        err = float(np.linalg.norm(lg_gpu[b].astype(np.float64) - ref) / np.linalg.norm(ref))
        margin = float(oracle.top2_margin(ref))
        tok_o = int(np.argmax(ref))
        tok_g = int(np.argmax(lg_gpu[b]))
        out.append(dict(rel_l2=err, margin=margin, tok_oracle=tok_o, tok_gpu=tok_g,
                        ok=(err <= REL_L2_TOL) and (tok_o == tok_g or margin <= MARGIN)))
    return out


def is_topk(r: np.ndarray, chosen, tol: float) -> bool:
    """`chosen` is a top-k of r up to tol: its smallest value is at least the largest other value minus tol."""
    return oracle.route_gap(r, np.asarray(chosen)) >= -tol


def oracle_reference(orc, tok, pos, routing=None, info: Optional[dict] = None) -> np.ndarray:
    """The oracle's logits for one step, for comparison with the GPU's.

    Dense models: the oracle's decode.  Routed models (``routing`` = the GPU's
    (experts [L,B,K], weights [L,B,K], router logits [L,B,E] or None) for
    this step): the oracle decodes with its own top-k; if the GPU chose a
    different set anywhere, the oracle re-decodes the step on the GPU's
    choice.  The GPU's choice is then checked layer by layer as described
    above (router logits, exact top-k of its own, top-k of the oracle's within
    the measured error) and its weights against the definition.  The oracle's
    cache afterwards holds the keys/values of the run returned."""
    lg = orc.decode(tok, pos)
    if orc.shape.n_experts == 0:
        return lg
    e_g, w_g, rl_g = routing
    L, B, K = e_g.shape
    diff = [(l, b) for l in range(L) for b in range(B)
            if set(e_g[l, b].tolist()) != set(orc.last_routing(l, b)[0].tolist())]
    if diff:
        orc.force_routing(e_g)
        try:
            lg = orc.decode(tok, pos)
        finally:
            orc.force_routing(None)
    min_gap = np.inf
    for l in range(L):
        for b in range(B):
            r_o = orc.last_router_logits(l, b)
            rms = float(np.sqrt(np.mean(r_o * r_o)))
            tol = ROUTE_GAP_REL * rms
            if rl_g is not None:
                r_g = rl_g[l, b].astype(np.float64)
                err = float(np.abs(r_g - r_o).max())
                rel = float(np.linalg.norm(r_g - r_o) / np.linalg.norm(r_o))
                assert rel <= REL_L2_TOL, f"layer {l} seq {b}: router logits relative L2 error {rel}"
                assert is_topk(r_g, e_g[l, b], 1e-6 * rms), \
                    f"layer {l} seq {b}: GPU experts {e_g[l, b]} are not the top-{K} of its router logits"
                tol = 2.0 * err + 1e-6 * rms
                if info is not None:
                    info["router_err"] = max(info.get("router_err", 0.0), err)
                    info["router_rel"] = max(info.get("router_rel", 0.0), rel)
            gap = oracle.route_gap(r_o, e_g[l, b])
            min_gap = min(min_gap, gap)
            assert gap >= -tol, f"layer {l} seq {b}: GPU experts {e_g[l, b]} are not a top-{K} (gap {gap}, tol {tol})"
            np.testing.assert_allclose(w_g[l, b], oracle.route_weights(r_o, e_g[l, b]), rtol=0, atol=1e-3)
    if info is not None:
        info["routing_diffs"] = info.get("routing_diffs", 0) + len(diff)
        info["min_route_gap"] = min(info.get("min_route_gap", np.inf), min_gap)
    return lg


def kv_row_errors(dev: np.ndarray, orc: np.ndarray):
    """Differences between bf16 cache rows [..., D] appended by the GPU and by
    the oracle: (largest difference in units of one bf16 ulp at each
    element's magnitude, floored at a quarter of its row's RMS; largest
    difference beyond that one ulp, relative to the row's RMS; fraction of
    elements that differ at all)."""
    d = synth.bf16_to_f32(dev.astype(np.uint16)).astype(np.float64)
    o = synth.bf16_to_f32(orc.astype(np.uint16)).astype(np.float64)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True)) + 1e-300
    scale = np.maximum(np.abs(o), rms / 4) + 1e-300
    ulp = np.exp2(np.floor(np.log2(scale)) - 7)  # bf16: 8 significant bits
    diff = np.abs(d - o)
    return (float((diff / ulp).max()), float((np.maximum(diff - ulp, 0.0) / rms).max()),
            float(np.mean(dev != orc)))


# Both sides round the same new key/value to bf16 (round to nearest even).
# Rounding alone makes them differ by at most one ulp where their unrounded
# values straddle a rounding boundary; the unrounded values differ by the
# decoder's own fp32 error, for which the stated bound on logits (1e-2
# relative) is taken: every element must lie within one ulp plus 1e-2 of its
# row's RMS.  Measured beyond the ulp: 0 on the VALU tiles (batch <= 4) and up
# to ~1.5e-3 of the RMS on the MFMA tiles (batch 16, bf16 hi/lo inputs: ~3e-5
# logits error, ~3e-4 for a sequence attending over few positions).  At most
# a quarter of the elements may differ at all: a wrong rounding mode
# (truncation) changes about half of them.
KV_EXCESS_TOL = 1e-2
KV_MISMATCH_TOL = 0.25
