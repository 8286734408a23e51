"""The parity checker: how GPU results are compared with the fp64 oracle.

Bars (the decode-attention contract): routed block indices identical except for
swaps inside the near-tie band; max |d out| <= 1e-2 on fp16 outputs of O(1)
magnitude; |d lse| <= 1e-3.  Per-part partials (one block's low-rank part, its
residual rows, one window chunk) are held to |d lse| <= 1e-3 and
||d o|| / ||o|| <= 1e-3.

Near-tie band (the reading of "exact where the fp32 score gap exceeds 1e-4
relative"): with s_(K) the K-th largest fp64 score and s_(K+1) the next,
tau = max(1e-4 * max(|s_(K)|, |s_(K+1)|), 1e-7 * |q_bar| * max_j |c_j|).
A GPU set is accepted iff every GPU-chosen block has s >= s_(K) - tau and
every oracle-chosen block the GPU dropped has s <= s_(K) + tau.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

TOL_OUT = 1e-2
TOL_LSE = 1e-3
TOL_PART_REL = 1e-3
NEAR_TIE_REL = 1e-4


@dataclasses.dataclass
class RouteCheck:
    ok: bool
    near_ties: int
    message: str = ""


def check_route_set(gpu_sel: np.ndarray, scores: np.ndarray, top_k: int, qbar_norm: float,
                    key_norm_max: float) -> RouteCheck:
    """gpu_sel: the GPU's indices for one (sequence, KV head), -1 padded to top_k."""
    n = scores.size
    k_eff = min(top_k, n)
    sel = np.asarray(gpu_sel, dtype=np.int64)
    valid = sel[:k_eff]
    if np.any(sel[k_eff:] != -1):
        return RouteCheck(False, 0, f"padding beyond K_eff={k_eff} is not -1: {sel}")
    if k_eff == 0:
        return RouteCheck(True, 0)
    if np.any(valid < 0) or np.any(valid >= n):
        return RouteCheck(False, 0, f"index out of range: {valid}")
    if np.any(np.diff(valid) <= 0):
        return RouteCheck(False, 0, f"indices not strictly ascending: {valid}")
    order = np.lexsort((np.arange(n), -scores))
    ref = set(order[:k_eff].tolist())
    got = set(valid.tolist())
    if got == ref:
        return RouteCheck(True, 0)
    sK = scores[order[k_eff - 1]]
    sK1 = scores[order[k_eff]] if k_eff < n else sK
    tau = max(NEAR_TIE_REL * max(abs(sK), abs(sK1)), 1e-7 * qbar_norm * key_norm_max)
    extra = got - ref
    missing = ref - got
    bad = [j for j in extra if scores[j] < sK - tau] + [j for j in missing if scores[j] > sK + tau]
    if bad:
        return RouteCheck(False, len(extra), f"routing differs outside the near-tie band "
                          f"(tau={tau:.3g}, s_K={sK:.6g}): blocks {sorted(bad)}")
    return RouteCheck(True, len(extra))


def check_routing(gpu_idx: np.ndarray, scores: Dict[Tuple[int, int], np.ndarray],
                  keys: Dict[Tuple[int, int], np.ndarray], q: np.ndarray, n_kv_heads: int,
                  top_k: int) -> RouteCheck:
    """All (sequence, KV head) pairs.  gpu_idx [B][Hkv][top_k]."""
    B, Hq, _ = q.shape
    G = Hq // n_kv_heads
    ties = 0
    for b in range(B):
        for h in range(n_kv_heads):
            qbar = q[b, h * G:(h + 1) * G].astype(np.float64).mean(axis=0)
            kn = keys[(b, h)]
            kmax = float(np.linalg.norm(kn, axis=1).max()) if kn.size else 0.0
            r = check_route_set(gpu_idx[b, h], scores[(b, h)], top_k,
                                float(np.linalg.norm(qbar)), kmax)
            if not r.ok:
                return RouteCheck(False, ties, f"(b={b}, h={h}) {r.message}")
            ties += r.near_ties
    return RouteCheck(True, ties)


@dataclasses.dataclass
class OutCheck:
    ok: bool
    max_out: float
    max_lse: float
    rel_l2: float
    message: str = ""


def check_outputs(out, lse, ref_out, ref_lse, tol_out: float = TOL_OUT,
                  tol_lse: float = TOL_LSE) -> OutCheck:
    o = np.asarray(out, dtype=np.float64)
    r = np.asarray(ref_out, dtype=np.float64)
    l = np.asarray(lse, dtype=np.float64)
    rl = np.asarray(ref_lse, dtype=np.float64)
    if o.shape != r.shape or l.shape != rl.shape:
        return OutCheck(False, np.inf, np.inf, np.inf, f"shape {o.shape}/{l.shape} vs {r.shape}/{rl.shape}")
    if not np.all(np.isfinite(o)):
        return OutCheck(False, np.inf, np.inf, np.inf, "non-finite output")
    same_inf = (l == rl) & ~np.isfinite(rl)
    with np.errstate(invalid="ignore"):        # -inf - -inf is masked by same_inf
        dl = np.where(same_inf, 0.0, np.abs(l - rl))
    dl = np.where(np.isnan(dl), np.inf, dl)
    mo = float(np.abs(o - r).max()) if o.size else 0.0
    ml = float(dl.max()) if dl.size else 0.0
    rel = float(np.linalg.norm(o - r) / max(np.linalg.norm(r), 1e-30)) if o.size else 0.0
    ok = mo <= tol_out and ml <= tol_lse
    msg = "" if ok else f"max|d out|={mo:.3g} (tol {tol_out}), max|d lse|={ml:.3g} (tol {tol_lse})"
    return OutCheck(ok, mo, ml, rel, msg)


def check_partials(o, lse, ref_o, ref_lse, tol_rel: float = TOL_PART_REL,
                   tol_lse: float = TOL_LSE) -> OutCheck:
    """Per-part partials: |d lse| <= tol_lse and ||d o|| / ||o|| <= tol_rel per part."""
    o = np.asarray(o, dtype=np.float64)
    r = np.asarray(ref_o, dtype=np.float64)
    l = np.asarray(lse, dtype=np.float64)
    rl = np.asarray(ref_lse, dtype=np.float64)
    same_inf = (l == rl) & ~np.isfinite(rl)
    with np.errstate(invalid="ignore"):        # -inf - -inf is masked by same_inf
        dl = np.where(same_inf, 0.0, np.abs(l - rl))
    dl = np.where(np.isnan(dl), np.inf, dl)
    num = np.linalg.norm(o - r, axis=-1)
    den = np.maximum(np.linalg.norm(r, axis=-1), 1e-30)
    rel = np.where(np.isfinite(rl), num / den, num)
    ml = float(dl.max()) if dl.size else 0.0
    mr = float(rel.max()) if rel.size else 0.0
    ok = ml <= tol_lse and mr <= tol_rel and bool(np.all(np.isfinite(o)))
    msg = "" if ok else f"partials: max rel|d o|={mr:.3g} (tol {tol_rel}), max|d lse|={ml:.3g}"
    return OutCheck(ok, float(np.abs(o - r).max()) if o.size else 0.0, ml, mr, msg)


def describe(results: List[OutCheck]) -> str:
    return "; ".join(f"out {r.max_out:.2e} lse {r.max_lse:.2e} rel {r.rel_l2:.2e}" for r in results)
