"""Comparison helpers for the GPU parity tests (library vs the CPU oracle)."""
from __future__ import annotations

import sys
from typing import Dict, List, Optional

import numpy as np
import torch

import oracle

# Floating-point bar: max |gpu - oracle| <= FP_TOL * max |oracle|, each stage against its own maximum.
FP_TOL = 2e-2
# Expert choices may differ only where two oracle router logits lie within this distance.
ROUTER_TIE = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.float().numpy().astype(np.float64)
    return t.numpy()


def host_out(y: np.ndarray) -> np.ndarray:
    """Oracle output (bf16 bit patterns or fp32) as fp64."""
    if y.dtype == np.uint16:
        return (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return y.astype(np.float64)


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    d = float(np.max(np.abs(gpu - ref))) if ref.size else 0.0
    if m == 0.0:
        return 0.0 if d == 0.0 else float("inf")
    return d / m


def assert_close(name: str, gpu, ref, tol: float = FP_TOL):
    e = rel_err(gpu, ref)
    assert e <= tol, f"{name}: max|err| / max|oracle| = {e:.3e} > {tol}"
    return e


def expert_mismatch(gpu_ex: np.ndarray, orc_ex: np.ndarray, logits: np.ndarray) -> Optional[str]:
    """None if the sets agree, else 'near-tie' (allowed) or a description (a failure)."""
    if list(gpu_ex) == list(orc_ex):
        return None
    # allowed only if every swapped expert sits within ROUTER_TIE of the oracle's k-th logit boundary
    kth = logits[orc_ex[-1]]
    for e in set(gpu_ex) ^ set(orc_ex):
        if abs(logits[e] - kth) > ROUTER_TIE:
            return f"experts {list(gpu_ex)} vs oracle {list(orc_ex)} (gap {abs(logits[e] - kth):.3e})"
    # same set but a different order is only allowed for near-equal logits too
    for a, b in zip(gpu_ex, orc_ex):
        if a != b and abs(logits[a] - logits[b]) > ROUTER_TIE:
            return f"order {list(gpu_ex)} vs {list(orc_ex)}"
    return "near-tie"


def check_rows(spec, t: Dict[str, torch.Tensor], dbg: Dict[str, torch.Tensor], y: torch.Tensor, rows: List[int],
               stages=("sel", "o", "h", "route", "y")) -> Dict[str, float]:
    """Stage-wise parity of the fused step's outputs on `rows` against the oracle. Returns the worst errors.
    Every stage in `stages` is compared for every row (a near-tie expert swap skips only that row's FFN)."""
    orc = oracle.LayerOracle(spec, t)
    x = host(t["x"]).astype(np.float64)
    worst = {"o": 0.0, "h-x": 0.0, "y-h": 0.0, "y": 0.0, "gates": 0.0, "near_ties": 0, "logit_abs": 0.0,
             "gap_min": float("inf"), "gaps_below_1e-5": 0}
    n_cmp = {"sel": 0, "o": 0, "h": 0, "route": 0, "y": 0}
    sel_g = host(dbg["sel"]) if "sel" in dbg else None
    for b in rows:
        r = orc.row(b, stages)
        if sel_g is not None:
            assert np.array_equal(sel_g[b], r["sel"]), f"row {b}: sel differs at " \
                f"{np.nonzero(sel_g[b] != r['sel'])[0][:8]}"
            n_cmp["sel"] += 1
        if "o" not in r:
            continue
        if "o" in dbg:
            worst["o"] = max(worst["o"], assert_close(f"row {b} o", host(dbg["o"])[b], r["o"]))
            n_cmp["o"] += 1
        if "h" not in r:
            continue
        hg = host(dbg["h"])[b]
        worst["h-x"] = max(worst["h-x"], assert_close(f"row {b} h-x", hg - x[b], r["h"] - x[b]))
        n_cmp["h"] += 1
        if "experts" not in r:
            continue
        if "logits" in dbg:
            # how far the GPU's router logits sit from the oracle's fp64 ones, against the margin that decides
            # the expert choice: the gap between the k_e-th and the next oracle logit of the token
            worst["logit_abs"] = max(worst["logit_abs"], float(np.max(np.abs(host(dbg["logits"])[b] - r["logits"]))))
            srt = np.sort(r["logits"])[::-1]
            if len(srt) > spec.ke:
                gap = float(srt[spec.ke - 1] - srt[spec.ke])
                worst["gap_min"] = min(worst["gap_min"], gap)
                worst["gaps_below_1e-5"] += gap < 1e-5
        mm = expert_mismatch(host(dbg["experts"])[b], r["experts"], r["logits"])
        if mm is not None and mm != "near-tie":
            raise AssertionError(f"row {b}: {mm}")
        n_cmp["route"] += 1
        if mm == "near-tie":
            worst["near_ties"] += 1
            say(f"row {b}: expert choice differs at a near-tie (<= {ROUTER_TIE}); FFN output not compared")
            continue
        worst["gates"] = max(worst["gates"], assert_close(f"row {b} gates", host(dbg["gates"])[b], r["gates"]))
        if "y64" not in r:
            continue
        yg = host(y)[b]
        y32 = host(dbg["y32"])[b]
        worst["y-h"] = max(worst["y-h"], assert_close(f"row {b} y-h", y32 - hg, r["y64"] - r["h"]))
        worst["y"] = max(worst["y"], assert_close(f"row {b} y", yg, host_out(r["y"])))
        n_cmp["y"] += 1
    want = {"sel": "sel" in stages, "o": "o" in stages, "h": "h" in stages, "route": "route" in stages,
            "y": "y" in stages}
    for k, on in want.items():
        if on:
            need = len(rows) - (worst["near_ties"] if k == "y" else 0)
            assert n_cmp[k] == need, f"stage {k} compared on {n_cmp[k]} of {need} rows"
    worst["rows"] = len(rows)
    return worst
