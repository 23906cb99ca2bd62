"""Pins of the float64 oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  None of them compares the oracle with
itself: each checks a closed form, a brute-force optimum, a value printed on
the pages (tests/golden/pages_values.json), an invariant, or a textbook
routine that the method reduces to in a special case.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))


def _rand_bf16(rng, shape, scale=1.0):
    from query_adaptive_decode_amd.synth import round_to_bf16
    return round_to_bf16(rng.standard_normal(shape) * scale)


# ---------------------------------------------------------------- P1 encoder
def test_bf16_directed_rounding_matches_torch_grid():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000),
                        [0.0, 0.1, -0.1, 1.0, -1.0, 3.0e38, 1e-40, -1e-40]])
    dn, up = O.bf16_down(v), O.bf16_up(v)
    t_dn = torch.tensor(dn, dtype=torch.float64).to(torch.bfloat16).to(torch.float64).numpy()
    t_up = torch.tensor(up, dtype=torch.float64).to(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(dn) & np.isfinite(up)
    assert np.array_equal(t_dn[fin], dn[fin]) and np.array_equal(t_up[fin], up[fin])
    assert np.all(dn <= v) and np.all(up[fin] >= v[fin])
    # adjacent grid points: no bf16 value strictly between dn and up
    bits = torch.tensor(dn[fin], dtype=torch.float64).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int32)
    nxt = np.where(dn[fin] >= 0, bits + 1, bits - 1)
    nxt_val = torch.tensor(nxt.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    exact = dn[fin] == up[fin]
    assert np.all(exact | (up[fin] == nxt_val) | ((dn[fin] == 0) & (up[fin] > 0)))
    # two printed-by-construction cases: 0.1 lies between 0x3DCC and 0x3DCD
    assert O.bf16_down(0.1) == 0.099609375 and O.bf16_up(0.1) == 0.10009765625


def test_codes_at_cell_boundaries_are_floor():
    # group min -1, max 1 -> lo = -1, rng = 2; a value exactly on the
    # boundary lo + k*rng/256 must get code k (floor), the top gets 255 (clamp)
    W = 8
    k = np.arange(0, 257)
    col = -1.0 + k * 2.0 / 256.0
    X = np.zeros((len(k) // 32 * 32, 2))
    X[:, 0] = col[: X.shape[0]]
    X[:, 1] = 0.5
    X[0, 0], X[1, 0] = -1.0, 1.0
    enc = O.encode_stream(X, W, 32)
    for g in range(enc.n_groups):
        lo, r = enc.lo[g, 0], enc.rng[g, 0]
        xs = X[g * 32:(g + 1) * 32, 0]
        want = [min(math.floor((Fraction(x) - Fraction(lo)) * 256 / Fraction(r)), 255) for x in xs]
        assert list(enc.codes[g * 32:(g + 1) * 32, 0]) == want
    assert enc.lo[0, 0] == -1.0 and enc.rng[0, 0] == 2.0
    assert list(enc.codes[2:8, 0]) == [2, 3, 4, 5, 6, 7]
    assert enc.codes[1, 0] == 255
    # a constant channel has rng 0 and code 0
    assert np.all(enc.rng[:, 1] == 0.0) and np.all(enc.codes[:, 1] == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefix_cells_contain_value_and_nest(dtype):
    from query_adaptive_decode_amd.synth import round_to_bf16, round_to_f32
    rng = np.random.default_rng(7)
    X = rng.standard_normal((32 * 6, 16)) * np.exp(rng.uniform(-3, 3, 16))
    X = round_to_bf16(X) if dtype == "bf16" else round_to_f32(X)
    W = 8
    enc = O.encode_stream(X, W, 32)
    gi = np.arange(enc.t_packed) // 32
    lo, r = enc.lo[gi], enc.rng[gi]
    # exact floor definition, checked with rationals on every scalar
    for j in range(0, enc.t_packed, 7):
        for c in range(16):
            want = min(math.floor((Fraction(float(X[j, c])) - Fraction(float(lo[j, c])))
                                  * 256 / Fraction(float(r[j, c]))), 255)
            assert enc.codes[j, c] == want
    assert np.all(lo <= X[:enc.t_packed]) and np.all(X[:enc.t_packed] <= lo + r)
    prev_lo, prev_hi = lo, lo + r
    for t in range(0, W + 1):
        P = O.prefix(enc.codes, t, W)
        xh = O.reconstruct(lo, r, P, t)
        # |x - x_hat_t| <= rng / 2^(t+1)
        assert np.all(np.abs(X[:enc.t_packed] - xh) <= r / 2.0 ** (t + 1) * (1 + 1e-15))
        cell_lo = lo + r * P / 2.0 ** t
        cell_hi = lo + r * (P + 1) / 2.0 ** t
        assert np.all(cell_lo >= prev_lo - 1e-12 * r) and np.all(cell_hi <= prev_hi + 1e-12 * r)
        prev_lo, prev_hi = cell_lo, cell_hi
    # full depth equals the W-bit midpoint quantiser
    full = O.reconstruct(lo, r, O.prefix(enc.codes, W, W), W)
    assert np.array_equal(full, lo + r * (2 * enc.codes + 1) / 2.0 ** (W + 1))


def test_nonfinite_group_is_flagged_and_not_coded():
    X = np.ones((64, 4))
    X[3, 2] = np.nan
    enc = O.encode_stream(X, 8, 32)
    assert enc.bad.tolist() == [True, False]
    assert np.all(enc.codes[:32] == 0) and np.all(enc.rng[0] == 0)


def test_plane_packing_round_trip():
    rng = np.random.default_rng(3)
    cap = 96
    K = _rand_bf16(rng, (70, 64))
    V = _rand_bf16(rng, (70, 64))
    ek, ev = O.encode_stream(K), O.encode_stream(V)
    p = O.pack_unit(ek, ev, cap, "bf16")
    # decode the planes back to codes by hand from the layout description
    kc = np.zeros((64, 64), dtype=np.int64)
    for c in range(64):
        for pl in range(8):
            for gam in range(2):
                w = int(p["Kplanes"][gam // 16, c, pl, gam % 16])
                for i in range(32):
                    kc[gam * 32 + i, c] |= ((w >> i) & 1) << (7 - pl)
    assert np.array_equal(kc, ek.codes)
    vc = np.zeros((64, 64), dtype=np.int64)
    for j in range(64):
        for pl in range(8):
            for wd in range(2):
                w = int(p["Vplanes"][j, pl, wd])
                for i in range(32):
                    vc[j, wd * 32 + i] |= ((w >> i) & 1) << (7 - pl)
    assert np.array_equal(vc, ev.codes)
    assert p["Kplanes"][0, :, :, 2:].sum() == 0 and p["Vplanes"][64:].sum() == 0
    lo = torch.tensor((p["Kmeta"][:2] & 0xFFFF).astype(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(lo, ek.lo)


# -------------------------------------------------------- P2/P3 brute force

def test_key_planes_span_tiles():
    # 34 closed groups: three 16-group tiles, the last one partly filled
    rng = np.random.default_rng(5)
    cap = 1120
    K = _rand_bf16(rng, (1090, 32))
    ek = O.encode_stream(K)
    p = O.pack_unit(ek, O.encode_stream(K), cap, "bf16")
    kp = p["Kplanes"]
    assert kp.shape == (3, 32, 8, 16)
    kc = np.zeros((34 * 32, 32), dtype=np.int64)
    for gam in range(34):
        w = kp[gam // 16, :, :, gam % 16].astype(np.int64)        # [c][plane]
        bits = (w[None, :, :] >> np.arange(32)[:, None, None]) & 1  # [i][c][plane]
        kc[gam * 32:(gam + 1) * 32] = (bits << (7 - np.arange(8))[None, None, :]).sum(axis=2)
    assert np.array_equal(kc, ek.codes)
    assert kp[2, :, :, 2:].sum() == 0

def _brute_best(a, W, B):
    """Exact minimum of sum_i a_i 4^-t_i over t in {0..W}^N, sum t <= B.
    Canonical optimum: fewest increments, then lexicographically largest."""
    af = [Fraction(float(x)) for x in a]
    best = None
    for t in itertools.product(range(W + 1), repeat=len(a)):
        if sum(t) > B:
            continue
        obj = sum(ai * Fraction(1, 4 ** ti) for ai, ti in zip(af, t))
        key = (obj, sum(t), tuple(-x for x in t))
        if best is None or key < best[0]:
            best = (key, t)
    return best[1], best[0][0]


@pytest.mark.parametrize("seed", range(12))
def test_greedy_equals_brute_force_optimum(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(2, 5))
    W = int(rng.integers(2, 5)) if seed % 3 else 8
    Bmax = min(N * W, 6) if W == 8 else N * W
    a = rng.exponential(1.0, N) * 10.0 ** rng.integers(-2, 3, N)
    if seed % 4 == 0:
        a[1] = a[0]                     # exact tie between items 0 and 1
    if seed % 5 == 0:
        a[-1] = 0.0                     # zero-weight item: never refined
    for B in range(0, Bmax + 1):
        t = O.choose_depths(a, O.gain_table(W), W, B)
        tb, obj = _brute_best(a, W, B)
        assert tuple(t) == tuple(tb), (a, W, B, t, tb)
        af = [Fraction(float(x)) for x in a]
        assert sum(af[i] * Fraction(1, 4 ** int(t[i])) for i in range(N)) == obj


def test_pooled_layer_budgets_equal_brute_force():
    # per-layer budgets ([ReadKV] Sec. 3.3): the key schedule of a request is
    # the optimum over all G * d key items under one budget, and the value
    # schedule the optimum over all G * T_packed value items; checked by
    # exhaustive search on a tiny layer (G = 2 KV heads, d = 2, 4 packed
    # tokens each in groups of 2, W = 2), with the second head's keys and
    # values 8x larger so that per-head budgets would choose differently
    from query_adaptive_decode_amd.synth import round_to_bf16
    rng = np.random.default_rng(53)
    W, G, d, T = 2, 2, 2, 5
    Ks = [round_to_bf16(rng.standard_normal((T, d)) * (1.0 + 7.0 * g)) for g in range(G)]
    Vs = [round_to_bf16(rng.standard_normal((T, d)) * (1.0 + 7.0 * g)) for g in range(G)]
    q = round_to_bf16(rng.standard_normal((G, d)))
    differs = False
    for rk, rv in [(0.25, 0.25), (0.5, 0.75), (0.75, 1.0), (1.25, 0.5), (2.0, 1.75)]:
        res = O.decode_request(q, Ks, Vs, W=W, R_K=rk, R_V=rv, group_tokens=2)
        assert res["BK"] == math.floor(rk * G * d) and res["BV"] == math.floor(rv * G * 4)
        tb, _ = _brute_best(res["wk"], W, res["BK"])
        assert tuple(res["tK"].reshape(-1)) == tuple(tb), (rk, res["tK"], tb)
        tb, _ = _brute_best(res["wv"], W, res["BV"])
        assert tuple(res["tV"].reshape(-1)) == tuple(tb), (rv, res["tV"], tb)
        per_head = [O.decode_unit(q[g:g + 1], Ks[g], Vs[g], W=W, R_K=rk, R_V=rv, group_tokens=2)
                    for g in range(G)]
        differs |= not np.array_equal(np.stack([r["tK"] for r in per_head]), res["tK"])
    assert differs
    # a KV head with a non-finite query reads nothing; the others keep the
    # whole layer budget
    qb = q.copy()
    qb[0, 1] = np.nan
    res = O.decode_request(qb, Ks, Vs, W=W, R_K=0.75, R_V=1.0, group_tokens=2)
    assert res["tK"][0].sum() == 0 and res["tV"][0].sum() == 0 and np.isnan(res["out"][0]).all()
    assert res["tK"][1].sum() == min(res["BK"], W * int((res["wk"][2:] > 0).sum()))
    assert np.isfinite(res["out"][1]).all()


def _brute_best_from(a, W, B, lo):
    """Exact minimum of sum_i a_i 4^-t_i over t in {lo..W}^N whose increments
    beyond lo total at most max(0, B - lo N); canonical optimum as in
    _brute_best."""
    af = [Fraction(float(x)) for x in a]
    rem = max(0, B - lo * len(a))
    best = None
    for t in itertools.product(range(lo, W + 1), repeat=len(a)):
        if sum(t) - lo * len(a) > rem:
            continue
        obj = sum(ai * Fraction(1, 4 ** ti) for ai, ti in zip(af, t))
        key = (obj, sum(t), tuple(-x for x in t))
        if best is None or key < best[0]:
            best = (key, t)
    return best[1]


@pytest.mark.parametrize("seed", range(6))
def test_min_depth_one_equals_brute_force(seed):
    # the restricted reader's mandatory minimum depth ([ReadKV] App. F.8),
    # with its levels counted against the budget (App. F.6)
    rng = np.random.default_rng(100 + seed)
    N, W = 4, 3
    a = rng.exponential(1.0, N) * 10.0 ** rng.integers(-2, 3, N)
    if seed % 2 == 0:
        a[2] = a[1]                     # an exact tie
    if seed % 3 == 0:
        a[0] = 0.0                      # zero weight: stays at depth 1
    for B in range(0, N * W + 2):
        t = O.choose_depths(a, O.gain_table(W), W, B, start=1)
        assert tuple(t) == tuple(_brute_best_from(a, W, B, 1)), (a, B, t)
        assert t.min() >= 1


@pytest.mark.parametrize("seed", range(4))
def test_value_packets_equal_brute_force(seed):
    # two-token value packets: tokens 2m and 2m+1 share a depth and a packet
    # level costs two token levels; the packet schedule minimises
    # sum_j a_j 4^-t_j over schedules with shared depths
    rng = np.random.default_rng(200 + seed)
    W = 3
    a = rng.exponential(1.0, 6) * 10.0 ** rng.integers(-2, 3, 6)
    af = [Fraction(float(x)) for x in a]
    for start in (0, 1):
        for B in range(0, 6 * W + 2):
            t, wp = O.pair_depths(a, O.gain_table(W), W, B, start)
            assert np.array_equal(t[0::2], t[1::2])
            best = None
            rem = max(0, B // 2 - start * 3)
            for tp in itertools.product(range(start, W + 1), repeat=3):
                if sum(tp) - 3 * start > rem:
                    continue
                obj = sum(af[j] * Fraction(1, 4 ** tp[j // 2]) for j in range(6))
                key = (obj, sum(tp), tuple(-x for x in tp))
                if best is None or key < best[0]:
                    best = (key, tp)
            assert tuple(t[0::2]) == best[1], (a, B, start, t)


def test_min_depth_one_forces_uniform_values_at_rate_one():
    # [ReadKV] App. F.8: a mandatory minimum depth of one forces uniform
    # value reading when the value budget is R_V = 1 (with and without
    # packets; keys likewise at R_K = 1)
    from query_adaptive_decode_amd.synth import round_to_bf16
    rng = np.random.default_rng(59)
    K = round_to_bf16(rng.standard_normal((300, 128)) * rng.uniform(0.1, 5, 128))
    V = round_to_bf16(rng.standard_normal((300, 128)))
    q = round_to_bf16(rng.standard_t(3, (4, 128)))
    for pairs in (False, True):
        res = O.decode_unit(q, K, V, R_K=1.0, R_V=1.0, min_depth=1, value_pairs=pairs)
        assert np.all(res["tV"] == 1) and np.all(res["tK"] == 1)
        res0 = O.decode_unit(q, K, V, R_K=1.0, R_V=1.0, value_pairs=pairs)
        assert not np.all(res0["tV"] == 1)   # without the floor the schedule is not uniform


def test_objective_identity_exact():
    rng = np.random.default_rng(11)
    a = rng.exponential(1.0, 6)
    W = 8
    for B in (0, 3, 10, 25, 48):
        t = [int(x) for x in O.choose_depths(a, O.gain_table(W), W, B)]
        af = [Fraction(float(x)) for x in a]
        D = lambda s: Fraction(1, 4 ** s)  # noqa: E731
        gains = sum(af[i] * (D(s - 1) - D(s)) for i in range(6) for s in range(1, t[i] + 1))
        assert sum(af[i] * D(t[i]) for i in range(6)) == sum(af) - gains
        assert sum(t) == min(B, W * int((a > 0).sum()))


def test_prop8_counterexample_harness():
    g = GOLD["prop8_counterexample"]
    lists, B = g["gain_lists"], g["budget"]
    # naive current-gain rule on arbitrary gain lists
    t = [0, 0]
    tot = 0
    for _ in range(B):
        cand = [(lists[i][t[i]], -i) for i in range(2) if t[i] < len(lists[i])]
        gbest, negi = max(cand)
        t[-negi] += 1
        tot += gbest
    # brute force over prefix-closed selections
    best = max(sum(lists[0][:x]) + sum(lists[1][:y])
               for x in range(3) for y in range(3) if x + y <= B)
    assert tot == g["current_gain_greedy_total"] and best == g["optimum_total"]


# ------------------------------------------------------- P4 closed forms
def _water_level_cost(a, W, B):
    a = np.asarray(a, dtype=np.float64)
    pos = a[a > 0]
    if B >= W * len(pos):
        return float(np.sum(pos * 4.0 ** -W))
    lo, hi = 1e-300, float(pos.max())
    for _ in range(400):
        tau = math.sqrt(lo * hi)
        tt = np.minimum(W, np.maximum(0.0, np.log(pos / tau) / np.log(4.0)))
        if tt.sum() > B:
            lo = tau
        else:
            hi = tau
    tt = np.minimum(W, np.maximum(0.0, np.log(pos / hi) / np.log(4.0)))
    return float(np.sum(pos * 4.0 ** -tt))


@pytest.mark.parametrize("seed", range(6))
def test_threshold_form_rounding_bound_and_nesting(seed):
    rng = np.random.default_rng(100 + seed)
    N, W = 200, 8
    a = np.exp(rng.normal(0, 4, N))
    a[:5] = 0.0
    gains = O.gain_table(W)
    prev = np.zeros(N, dtype=np.int64)
    for B in [0, 1, 7, 50, 333, 800, 1000, 1559, 1560, 2000]:
        t = O.choose_depths(a, gains, W, B)
        # threshold form from a library sort of every candidate gain
        cand = np.array([a[i] * 4.0 ** -s for i in range(N) for s in range(1, W + 1)])
        cand = cand[cand > 0]
        if B == 0:
            assert t.sum() == 0
        elif B >= len(cand):
            assert np.all(t[a > 0] == W) and np.all(t[a == 0] == 0)
        else:
            tau = np.sort(cand)[::-1][B - 1]
            above = np.array([sum(a[i] * 4.0 ** -s > tau for s in range(1, W + 1)) for i in range(N)])
            at = np.array([any(a[i] * 4.0 ** -s == tau for s in range(1, W + 1)) for i in range(N)])
            need = B - above.sum()
            extra = np.zeros(N, dtype=np.int64)
            extra[np.nonzero(at)[0][:need]] = 1
            assert np.array_equal(t, above + extra)
            # continuous relaxation and integer-rounding factor
            I = float(np.sum(a * 4.0 ** -t))
            C = _water_level_cost(a, W, B)
            assert C <= I * (1 + 1e-9) and I <= GOLD["kappa_int"]["value"] * C * (1 + 1e-9)
        assert np.all(t >= prev)            # schedules nest as B grows
        prev = t


def test_kappa_int_value():
    f = np.linspace(0, 1, 2_000_001)
    k = np.max((1 - 0.75 * f) * 4.0 ** f)
    fstar = 4.0 / 3.0 - 1.0 / math.log(4.0)
    assert abs((1 - 0.75 * fstar) * 4 ** fstar - GOLD["kappa_int"]["value"]) < 5e-10
    assert abs(k - GOLD["kappa_int"]["value"]) < 1e-9


# ----------------------------------------------- P5 R = W is plain attention
@pytest.mark.parametrize("gt,dtype", [(32, "f32"), (32, "bf16"), (8, "bf16")])
def test_full_read_equals_quantised_sdpa(gt, dtype):
    from query_adaptive_decode_amd.synth import round_to_bf16, round_to_f32
    cast = round_to_bf16 if dtype == "bf16" else round_to_f32
    rng = np.random.default_rng(5)
    d, T, gqa = 64, 32 * 5 + 13, 4
    K = cast(rng.standard_normal((T, d)) * np.exp(rng.uniform(-1, 1, d)))
    V = cast(rng.standard_normal((T, d)))
    q = cast(rng.standard_normal((gqa, d)))
    res = O.decode_unit(q, K, V, W=8, R_K=8.0, R_V=8.0, group_tokens=gt, diagnostics=True)
    assert np.all(res["tK"] == 8) and np.all(res["tV"] == 8)
    ek, ev = res["enc_k"], res["enc_v"]
    tp = ek.t_packed
    gi = np.arange(tp) // gt
    Kq = np.concatenate([ek.lo[gi] + ek.rng[gi] * (2 * ek.codes + 1) / 512.0, K[tp:]])
    Vq = np.concatenate([ev.lo[gi] + ev.rng[gi] * (2 * ev.codes + 1) / 512.0, V[tp:]])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, :, None, :], torch.tensor(Kq)[None, None].expand(1, gqa, T, d),
        torch.tensor(Vq)[None, None].expand(1, gqa, T, d))[0, :, 0, :].numpy()
    assert np.allclose(res["out"], ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------- P6 Theorem 1 allocation pattern
def test_theorem1_support_read_to_full_depth():
    rng = np.random.default_rng(9)
    d, L, k = 128, 8, 24
    K = rng.uniform(-1, 1, (64, d)).astype(np.float32).astype(np.float64)
    V = rng.uniform(-1, 1, (64, d)).astype(np.float32).astype(np.float64)
    q = np.zeros((1, d))
    supp = rng.choice(d, k, replace=False)
    q[0, supp] = rng.standard_normal(k).astype(np.float32)
    res = O.decode_unit(q, K, V, W=L, R_K=L * k / d, R_V=2.0)
    assert res["BK"] == L * k
    want = np.zeros(d, dtype=np.int64)
    want[supp] = L
    assert np.array_equal(res["tK"], want)


# -------------------------------------- P7 two-token worked example (adapted)
@pytest.mark.parametrize("b,eta", [(1, 1), (1, -1), (-1, 1), (-1, -1)])
def test_two_token_example(b, eta):
    m, a = 8, 1.5
    rng = np.random.default_rng(21)
    K = np.zeros((2, m))
    K[0, 0], K[1, 0] = b * a, -b * a
    V = rng.integers(-64, 65, (2, m)) / 64.0
    V[0, 0], V[1, 0] = 0.25, -0.75
    q = np.zeros((1, m))
    q[0, 0] = eta * 10.0 * math.sqrt(m) / a
    res = O.decode_unit(q, K, V, W=8, R_K=1.0 / m, R_V=4.0, group_tokens=2)
    assert res["BK"] == 1 and res["tK"][0] == 1 and res["tK"][1:].sum() == 0
    assert np.allclose(res["zhat"][0], [5 * eta * b, -5 * eta * b], rtol=0, atol=1e-13)
    p = 1.0 / (1.0 + math.exp(-10.0))
    jstar = 0 if eta * b == 1 else 1
    assert res["BV"] == 8
    want_t = [0, 0]
    want_t[jstar] = 8
    assert list(res["tV"]) == want_t
    lo, hi = V.min(axis=0), V.max(axis=0)
    rng_ = hi - lo                               # exact bf16 on this grid
    vstar = np.where(V[jstar] == hi, hi - rng_ / 512, lo + rng_ / 512)
    vstar = np.where(rng_ == 0, lo, vstar)
    other = lo + rng_ / 2
    want = p * vstar + (1 - p) * other
    assert np.allclose(res["out"][0], want, rtol=0, atol=1e-15)


# ---------------------------------------------------- P8 invariants
def test_error_decomposition_and_softmax_lipschitz():
    from query_adaptive_decode_amd.synth import round_to_bf16
    rng = np.random.default_rng(31)
    d, T, gqa = 128, 32 * 8 + 5, 4
    K = round_to_bf16(rng.standard_normal((T, d)) * np.exp(rng.uniform(-2, 2, d)))
    V = round_to_bf16(rng.standard_normal((T, d)))
    q = round_to_bf16(rng.standard_t(3, (gqa, d)))
    res = O.decode_unit(q, K, V, W=8, R_K=2.0, R_V=2.0, diagnostics=True)
    z = q @ K.T / math.sqrt(d)
    alpha = O.softmax(z)
    o = alpha @ V
    EV = V - res["Vhat"]
    lhs = o - res["out"]
    rhs = (alpha - res["ahat"]) @ V + res["ahat"] @ EV
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-12)
    for h in range(gqa):
        assert np.linalg.norm(alpha[h] - res["ahat"][h]) <= np.linalg.norm(z[h] - res["zhat"][h]) / 2 + 1e-15


def test_budget_accounting_and_write_once():
    from query_adaptive_decode_amd.synth import round_to_bf16
    rng = np.random.default_rng(41)
    d, T = 128, 32 * 10 + 7
    K = round_to_bf16(rng.standard_normal((T, d)))
    V = round_to_bf16(rng.standard_normal((T, d)))
    q = round_to_bf16(rng.standard_normal((4, d)))
    for RK, RV in [(3.3, 2.7), (0.0, 8.0), (1.0, 0.5)]:
        res = O.decode_unit(q, K, V, R_K=RK, R_V=RV)
        assert res["BK"] == math.floor(float(np.float32(RK)) * d)
        assert res["BV"] == math.floor(float(np.float32(RV)) * res["tp"])
        assert res["tK"].sum() == min(res["BK"], 8 * int((res["wk"] > 0).sum()))
        assert res["tV"].sum() == min(res["BV"], 8 * int((res["wv"] > 0).sum()))
        bits = res["tp"] * res["tK"].sum() + d * res["tV"].sum()
        assert bits <= (res["BK"] * res["tp"] + d * res["BV"])
    # closed groups never change when more tokens arrive
    e1 = O.encode_stream(K[:200])
    e2 = O.encode_stream(K)
    assert np.array_equal(e1.codes, e2.codes[:e1.t_packed])
    assert np.array_equal(e1.lo, e2.lo[:e1.n_groups])


def test_logical_reads_at_full_depth_equal_the_stored_record():
    # reading every plane of every closed group (R = W, the full-read limit of
    # [ReadKV] App. C.3) asks for exactly the bits the store holds for them:
    # the plane arrays, the metadata arrays and energies, and the open group
    # slots in use -- sizes from the store's format description
    from oracle import store_format as F
    from query_adaptive_decode_amd.synth import round_to_bf16
    rng = np.random.default_rng(43)
    d, W = 128, 8
    for tp, r, dt in [(1024, 0, 0), (1024, 5, 0), (512, 31, 1)]:
        n = tp + r
        K = round_to_bf16(rng.standard_normal((n, d)))
        V = round_to_bf16(rng.standard_normal((n, d)))
        q = round_to_bf16(rng.standard_normal((2, d)))
        res = O.decode_unit(q, K, V, R_K=8.0, R_V=8.0)
        assert res["tK"].min() == W and res["tV"].min() == W
        esize = 2 if dt == 0 else 4
        lr = O.logical_reads(res["tK"], res["tV"], n, d, elem_bits=8 * esize)
        lay = F.region_layout(1, d, W, tp, esize)   # one KV head, capacity tp
        size = {k: lay[k][1] for k in ("Kplanes", "Vplanes", "Kmeta", "Vmeta", "EK", "EV",
                                       "Ktail", "Vtail")}
        assert lr["key_payload"] == 8 * size["Kplanes"]
        assert lr["value_payload"] == 8 * size["Vplanes"]
        assert lr["metadata"] == 8 * (size["Kmeta"] + size["Vmeta"] + size["EK"] + size["EV"])
        assert lr["open_group"] == 8 * (size["Ktail"] + size["Vtail"]) * r // 32


def test_nonfinite_query_reads_nothing():
    from query_adaptive_decode_amd.synth import round_to_bf16
    rng = np.random.default_rng(47)
    K = round_to_bf16(rng.standard_normal((100, 128)))
    V = round_to_bf16(rng.standard_normal((100, 128)))
    for bad in (np.nan, np.inf, -np.inf):
        q = round_to_bf16(rng.standard_normal((4, 128)))
        q[2, 17] = bad
        res = O.decode_unit(q, K, V, R_K=4.0, R_V=4.0)
        assert np.isnan(res["out"]).all() and res["out"].shape == (4, 128)
        assert res["tK"].sum() == 0 and res["tV"].sum() == 0 and len(res["tV"]) == 96


def test_empty_context_reads_nothing():
    # Reading (the pages read a non-empty context): no tokens -> no key
    # energy, so only the minimum key depth; no value items; the output is
    # the empty sum, zero, whatever the query.  The counters charge only E^K.
    rng = np.random.default_rng(53)
    q = rng.standard_normal((4, 128))
    empty = np.zeros((0, 128))
    for md in (0, 1):
        for qq in (q, np.where(np.arange(128) == 5, np.nan, q)):
            r = O.decode_unit(qq, empty, empty, R_K=4.0, R_V=4.0, min_depth=md)
            assert np.array_equal(r["out"], np.zeros((4, 128)))
            assert np.all(r["tK"] == md) and r["tV"].size == 0
        r = O.decode_request(np.vstack([q, q]), [empty, empty], [empty, empty], R_K=3.0, R_V=2.0,
                             min_depth=md)
        assert np.array_equal(r["out"], np.zeros((2, 4, 128)))
        assert np.all(r["tK"] == md) and r["tV"].shape == (2, 0)
    lr = O.logical_reads(np.zeros(128, dtype=np.int64), np.zeros(0, dtype=np.int64), 0)
    assert lr == dict(key_payload=0, value_payload=0, metadata=128 * 64, open_group=0)
    # one open token: the softmax over it is 1, so the output is its value
    # exactly (the open-group path next to the empty case)
    K1, V1 = rng.standard_normal((1, 128)), rng.standard_normal((1, 128))
    r = O.decode_unit(q, K1, V1, R_K=4.0, R_V=4.0)
    assert np.array_equal(r["out"], np.repeat(V1, 4, axis=0))


# ---------------------------------------------------- P9 reuse model
def test_reuse_model_printed_values():
    g = GOLD["reuse_overhead_N8192_L128_W8_W0_4"]
    eta = O.reuse_overhead(8192, 128, 8, 4) * 100
    assert abs(eta - g["value_percent"]) <= g["printed_precision"]
    assert O.reuse_reads(8192, 128) == 128 * 8192 + 128 * 127 // 2
    assert Fraction(4 * (0 + 201), 4 * O.reuse_reads(0, 201)) == Fraction(1, 100)
    assert abs(O.reuse_overhead(0, 201, 8, 4) * 100 - GOLD["reuse_overhead_N0_L201_W8_W0_4"]["value_percent"]) < 1e-12
    # the fraction is largest at N = 0 for fixed L
    assert all(O.reuse_overhead(N, 201, 8, 4) <= 0.01 + 1e-15 for N in (0, 1, 10, 1000, 10 ** 6))


# ------------------------------------- item weights minimise realised error
# The key and value weights are the diagonal surrogate of the expected squared
# logit / output error ([ReadKV] App. D.2, E.3.2: for independent zero-mean
# residuals E[(q.e)^2] = sum_c q_c^2 E[e_c^2]; a residual uniform in a cell of
# width w has E[e^2] = w^2/12).  On data where that model holds, the schedule
# the oracle picks must beat schedules picked from other plausible weights on
# the realised error.
def _realised_logit_err(q, K, enc, t):
    tp = enc.t_packed
    gi = np.arange(tp) // 32
    Kh = O.reconstruct(enc.lo[gi], enc.rng[gi], O.prefix(enc.codes, t[None, :], 8), t[None, :])
    return float(np.sum((q @ (K[:tp] - Kh).T) ** 2))


def test_key_weights_minimise_realised_logit_error():
    rng = np.random.default_rng(77)
    d, T, gqa = 64, 32 * 64, 4
    scale = np.exp(rng.uniform(-2, 2, d))
    K = rng.uniform(-1, 1, (T, d)) * scale
    q = rng.standard_t(2.0, (gqa, d))
    enc = O.encode_stream(K)
    gains = O.gain_table(8)
    E = np.sum(enc.rng ** 2, axis=0)
    BK = 96
    ours = O.choose_depths(O.key_weights(q, enc), gains, 8, BK)
    base = _realised_logit_err(q, K, enc, ours)
    alts = [np.sum(q ** 2, axis=0) * E, np.sum(np.abs(q), axis=0) * E, np.sum(q ** 2, axis=0),
            np.sum(q ** 2, axis=0) * np.sqrt(E), np.sum(np.abs(q), axis=0) * np.sqrt(E)]
    n_diff = 0
    for w in alts:
        t = O.choose_depths(w, gains, 8, BK)
        if not np.array_equal(t, ours):
            n_diff += 1
            assert base < _realised_logit_err(q, K, enc, t)
    assert n_diff >= 3


def test_value_weights_minimise_realised_output_error():
    rng = np.random.default_rng(78)
    d, ng, gqa = 32, 48, 4
    T = 32 * ng
    gscale = np.exp(rng.uniform(-2.5, 2.5, ng))
    V = rng.uniform(-1, 1, (T, d)) * np.repeat(gscale, 32)[:, None]
    enc = O.encode_stream(V)
    logits = rng.normal(0, 2.0, (gqa, T))
    alpha = O.softmax(logits)
    gains = O.gain_table(8)
    BV = 2 * T
    gi = np.arange(T) // 32

    def err(t):
        Vh = O.reconstruct(enc.lo[gi], enc.rng[gi], O.prefix(enc.codes, t[:, None], 8), t[:, None])
        return float(np.sum((alpha @ (V - Vh)) ** 2))

    ours = O.choose_depths(O.value_weights(alpha, enc, "physical"), gains, 8, BV)
    base = err(ours)
    s = np.repeat(np.sum(enc.rng ** 2, axis=1), 32)
    alts = [np.sum(alpha ** 2, axis=0) * s, np.sum(alpha ** 2, axis=0),
            np.sum(np.abs(alpha), axis=0) * s, np.sum(alpha, axis=0) ** 2 * np.sqrt(s)]
    n_diff = 0
    for w in alts:
        t = O.choose_depths(w, gains, 8, BV)
        if not np.array_equal(t, ours):
            n_diff += 1
            assert base < err(t)
    assert n_diff >= 3
