"""Comparison rules for the GPU-vs-oracle parity tests.

Allocation rule.  S_o and S_g are the (item, level) refinements selected by
the oracle and the GPU for one stage of one selection domain (a (request,
KV head) unit, or a request under pooled budgets); g_o is the oracle's gain
of a refinement and tau_o the smallest gain the oracle selected.

* The total number of refinements must match exactly.
* Every refinement in the symmetric difference must be a near tie:
  |g_o - tau_o| <= 1e-6 * tau_o.
* Exact ties are decided by the lowest-index rule of ChooseDepths, so the GPU
  may not swap a refinement the oracle chose for one it did not choose when
  the two have bitwise-equal oracle gains: any such pair fails, however close
  to tau_o it lies.  (A swap between two refinements whose oracle gains
  differ, both within the window, is a near tie: the two sides rounded the
  weights differently.)

Near ties are counted and reported per case.  Outputs: relative L2 error per
(request, query head) <= 2e-3.
"""
import numpy as np

NEAR_TIE_REL = 1e-6
OUT_REL_L2 = 2e-3

# one line per parity case (near-tie counts, worst output error), printed in
# the test session's terminal summary
REPORT = []


def _gain(w, lvl, gains):
    return float(w) * (4.0 ** (-lvl) if gains is None else float(gains[lvl]))


def _levels(t_from, t_to, w, gains=None):
    """(item, level, gain) of the levels item i holds in t_to but not in
    t_from."""
    out = []
    for i in np.nonzero(t_to > t_from)[0]:
        for lvl in range(int(t_from[i]) + 1, int(t_to[i]) + 1):
            out.append((int(i), lvl, _gain(w[i], lvl, gains)))
    return out


def alloc_mismatch(t_gpu, t_or, w_or, W, rel=NEAR_TIE_REL, start=0, gains=None):
    """Returns (n_near_ties, n_bad, detail) for one selection domain.

    t_gpu, t_or: depth per item (GPU, oracle); w_or: the oracle's item
    weights (gain of level t = w * 4^-t, or w * gains[t] with a gain table);
    start: the mandatory minimum depth (levels up to it are not chosen, so
    they do not define tau_o)."""
    t_gpu = np.asarray(t_gpu, dtype=np.int64)
    t_or = np.asarray(t_or, dtype=np.int64)
    if t_gpu.sum() != t_or.sum():
        return 0, 1, f"total refinements differ: gpu {t_gpu.sum()} oracle {t_or.sum()}"
    if np.array_equal(t_gpu, t_or):
        return 0, 0, ""
    w = np.asarray(w_or, dtype=np.float64)
    if np.any(t_gpu < start):
        return 0, 1, f"a depth below the minimum {start}"
    sel = np.nonzero(t_or > start)[0]
    if len(sel) == 0:
        return 0, 1, "the oracle chose no level, the GPU did"
    tau = min(_gain(w[i], int(t_or[i]), gains) for i in sel)
    extra = _levels(t_or, t_gpu, w, gains)     # chosen by the GPU only
    missing = _levels(t_gpu, t_or, w, gains)   # chosen by the oracle only
    near = bad = 0
    worst = 0.0
    for (_, _, g) in extra + missing:
        r = abs(g - tau) / tau
        worst = max(worst, r)
        if r <= rel:
            near += 1
        else:
            bad += 1
    # exact-tie swaps: a GPU-only and an oracle-only refinement with
    # bitwise-equal oracle gains
    miss_gains = {}
    for (i, lvl, g) in missing:
        miss_gains.setdefault(g, []).append((i, lvl))
    swaps = []
    for (i, lvl, g) in extra:
        if g in miss_gains:
            swaps.append(((i, lvl), miss_gains[g][0]))
    bad += len(swaps)
    det = (f"{int(np.count_nonzero(t_gpu != t_or))} items differ, worst |g-tau|/tau = "
           f"{worst:.3e}, exact-tie swaps {len(swaps)}")
    if swaps:
        det += f" (gpu-only, oracle-only) e.g. {swaps[:3]}"
    return near, bad, det


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b, axis=-1) / np.maximum(np.linalg.norm(b, axis=-1), 1e-300)
