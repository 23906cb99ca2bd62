"""Comparison rules for the GPU-vs-oracle parity tests.

Allocation rule (near ties): S_o and S_g are the (item, level) refinements
selected by the oracle and the GPU for one stage of one (request, KV head)
unit; tau_o is the smallest gain the oracle selected.  A refinement in the
symmetric difference is a near tie iff |g_o - tau_o| <= 1e-6 * tau_o, with g_o
the oracle's gain for it; near ties are counted and reported, any other
difference fails, and the total number of refinements must match exactly.
Outputs: relative L2 error per (request, query head) <= 2e-3.
"""
import numpy as np

NEAR_TIE_REL = 1e-6
OUT_REL_L2 = 2e-3


def alloc_mismatch(t_gpu, t_or, w_or, W, rel=NEAR_TIE_REL):
    """Returns (n_near_ties, n_bad, detail)."""
    t_gpu = np.asarray(t_gpu, dtype=np.int64)
    t_or = np.asarray(t_or, dtype=np.int64)
    if t_gpu.sum() != t_or.sum():
        return 0, 1, f"total refinements differ: gpu {t_gpu.sum()} oracle {t_or.sum()}"
    diff = np.nonzero(t_gpu != t_or)[0]
    if len(diff) == 0:
        return 0, 0, ""
    w = np.asarray(w_or, dtype=np.float64)
    sel_items = np.nonzero(t_or > 0)[0]
    tau = np.min(w[sel_items] * 4.0 ** (-t_or[sel_items].astype(np.float64)))
    near = bad = 0
    worst = 0.0
    for i in diff:
        lo, hi = sorted((int(t_gpu[i]), int(t_or[i])))
        for lvl in range(lo + 1, hi + 1):
            g = w[i] * 4.0 ** (-lvl)
            r = abs(g - tau) / tau
            worst = max(worst, r)
            if r <= rel:
                near += 1
            else:
                bad += 1
    return near, bad, f"{len(diff)} items differ, worst |g-tau|/tau = {worst:.3e}"


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b, axis=-1) / np.maximum(np.linalg.norm(b, axis=-1), 1e-300)
