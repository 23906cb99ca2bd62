"""Pins of the oracle's Lloyd-tree codec (oracle/lloyd.py) against what the
pages print and what the mathematics fixes.  CPU only.

Printed values: [ReadKV] App. D.1 (the D(t) table, Lemma 7's gain
intervals), App. E.1.1-E.1.3 (eps_8, Q_2(1), the two-token construction).
Independent checks: conditional means and distortions by numerical
integration, Lloyd stationarity, the 4-level Lloyd-Max quantiser of a
Gaussian, orthogonality of the Hadamard-sign transform, brute-force cells,
brute-force optimal allocations with the tree's gains, and attention with no
quantisation when every token is in the open group.
"""
import itertools
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
from scipy import integrate
from scipy.stats import norm

from oracle import lloyd as L
from oracle.readkv import choose_depths, softmax

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))


@pytest.fixture(scope="module")
def tree():
    return L.lloyd_tree()


def _sig_round(x, text):
    """x rounded to the significant digits printed in ``text`` (".03484" has
    four, "1" one)."""
    digits = len(text.replace(".", "").lstrip("0"))
    return float(f"{x:.{digits}g}")


# ----------------------------------------------------------- printed tables
def test_distortion_table_matches_printed_digits(tree):
    printed = GOLD["lloyd_distortion_table"]["D"]
    for t, txt in enumerate(printed):
        assert _sig_round(tree.D[t], txt) == float(txt), (t, tree.D[t], txt)


def test_float32_gains_lie_in_printed_intervals(tree):
    g = GOLD["lloyd_gain_intervals"]
    for t in range(1, 9):
        v = Fraction(float(np.float32(tree.gains[t])))  # the float32 entry, exactly
        assert Fraction(g["lower"][t - 1]) < v < Fraction(g["upper"][t - 1]), (t, float(v))
        assert tree.gains32[t] == float(v)
    # the intervals are disjoint and ordered: Delta_1 > ... > Delta_8 > 0
    assert all(tree.gains32[t] > tree.gains32[t + 1] > 0 for t in range(1, 8))


def test_gains_are_differences_of_the_distortion_curve(tree):
    for t in range(1, 9):
        assert abs(tree.gains[t] - (tree.D[t - 1] - tree.D[t])) <= 1e-13


def test_depth_two_reconstruction_of_one(tree):
    g = GOLD["lloyd_Q2_of_1"]
    q2 = L.lloyd_reconstruct(L.tree_codes(np.array([1.0, -1.0]), tree, 8), 2, 0.0, 1.0, tree, 8)
    assert Fraction(g["lower"]) < Fraction(float(q2[0])) < Fraction(g["upper"])
    assert q2[1] == -q2[0]
    assert (q2[0] - 1.0) ** 2 > 0.26052610


def test_eps8_below_printed_bound_and_attained_at_cell_endpoints(tree):
    edges, cent = tree.edges[8], tree.cent32[8]
    eps = 0.0
    for j in range(256):
        lo, hi = max(edges[j], -1.0), min(edges[j + 1], 1.0)
        if lo < hi:
            eps = max(eps, abs(lo - cent[j]), abs(hi - cent[j]))
    assert eps < GOLD["lloyd_eps8"]["upper"]
    # brute force over a fine grid of [-1, 1] reaches the endpoint maximum
    z = np.linspace(-1.0, 1.0, 400001)
    err = np.abs(z - L.lloyd_reconstruct(L.tree_codes(z, tree, 8), 8, 0.0, 1.0, tree, 8))
    assert err.max() <= eps + 1e-12 and err.max() > eps - 1e-4
    rho = 1.0 / (1.0 + math.exp(10.0))
    p = 1.0 - rho
    assert (p * eps + rho) ** 2 < 9.50e-5


# --------------------------------------------- the tree from the mathematics
def test_depth_one_centroid_is_the_half_normal_mean(tree):
    assert tree.cent32[1][1] == float(np.float32(math.sqrt(2.0 / math.pi)))
    assert tree.bounds[0][0] == 0.0


def test_four_level_lloyd_max_gaussian_quantiser(tree):
    # the 4-level Lloyd-Max quantiser of N(0,1): thresholds 0, +-0.9816,
    # levels +-0.4528, +-1.510 (Max, 1960)
    assert abs(tree.edges[2][3] - 0.9816) < 5e-5
    assert abs(tree.cent[2][2] - 0.4528) < 5e-5 and abs(tree.cent[2][3] - 1.5104) < 5e-5


def test_centroids_are_conditional_means_by_integration(tree):
    rng = np.random.default_rng(3)
    for t in (1, 3, 8):
        for P in rng.choice(2 ** t, size=min(6, 2 ** t), replace=False):
            a, b = tree.edges[t][P], tree.edges[t][P + 1]
            mass = integrate.quad(norm.pdf, a, b, epsabs=0, epsrel=1e-13)[0]
            mom = integrate.quad(lambda z: z * norm.pdf(z), a, b, epsabs=0, epsrel=1e-13)[0]
            assert abs(mom / mass - tree.cent[t][P]) < 1e-9 * max(1.0, abs(tree.cent[t][P]))


def test_splits_are_lloyd_stationary_and_nested(tree):
    for t in range(1, 9):
        e, c = tree.edges[t], tree.cent[t]
        # every inner edge is the midpoint of its two neighbouring centroids
        # (edges of depth t-1 are midpoints at depth t too: Lloyd stationarity
        # holds for the split that made them)
        for i in range(1, 2 ** t):
            if i % 2 == 1:  # made by splitting depth-(t-1) cell i // 2
                assert abs(e[i] - 0.5 * (c[i - 1] + c[i])) < 1e-12
        # depth-(t-1) edges are kept
        assert set(tree.edges[t - 1]).issubset(set(e))
    # the encoder's boundaries are midpoints of the float32 child centroids
    for t in range(8):
        for P in range(2 ** t):
            assert tree.bounds[t][P] == (tree.cent32[t + 1][2 * P] + tree.cent32[t + 1][2 * P + 1]) / 2


def test_distortion_by_integration(tree):
    for t in (1, 2, 5, 8):
        e, c = tree.edges[t], tree.cent[t]
        D = sum(integrate.quad(lambda z, cc=c[i]: (z - cc) ** 2 * norm.pdf(z), e[i], e[i + 1],
                               epsabs=1e-16, epsrel=1e-12)[0] for i in range(2 ** t))
        assert abs(D - tree.D[t]) < 1e-10


def test_tree_codes_name_the_cell_that_holds_z(tree):
    rng = np.random.default_rng(5)
    b8 = np.sort(np.concatenate([tree.bounds[t] for t in range(8)]))
    z = np.concatenate([rng.standard_normal(20000) * 1.5, b8, np.nextafter(b8, -np.inf),
                        [-np.inf, np.inf, 0.0, -0.0, 50.0, -50.0]])
    leaf = L.tree_codes(z, tree, 8)
    assert np.array_equal(leaf, np.searchsorted(b8, z, side="right"))
    for W in (1, 2, 4, 7):
        assert np.array_equal(L.tree_codes(z, tree, W), leaf >> (8 - W))
    assert L.tree_codes(np.array([np.nan]), tree, 8)[0] == 0


# ------------------------------------------------ Hadamard-sign transforms
def test_inv_sqrt_d_is_correctly_rounded():
    getcontext().prec = 60
    for d in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        k = L.inv_sqrt_d(d)
        exact = Decimal(1) / Decimal(d).sqrt()
        up, dn = np.nextafter(k, np.inf), np.nextafter(k, -np.inf)
        assert abs(Decimal(k) - exact) <= abs(Decimal(float(up)) - exact)
        assert abs(Decimal(k) - exact) <= abs(Decimal(float(dn)) - exact)


def test_hadamard_sign_transform_is_orthogonal():
    rng = np.random.default_rng(7)
    s = 1 - 2 * rng.integers(0, 2, 128)
    U = L.hs_transform(np.eye(128), s)            # row i = U e_i = column i of U
    assert np.allclose(U @ U.T, np.eye(128), atol=1e-14)
    x = rng.standard_normal((5, 128))
    y = rng.standard_normal((5, 128))
    assert np.allclose(L.hs_inverse(L.hs_transform(x, s), s), x, atol=1e-13)
    assert np.allclose(np.sum(L.hs_transform(x, s) * L.hs_transform(y, s), 1), np.sum(x * y, 1))
    # App. E.1.3: U e_j has every entry +-1/sqrt(d)
    assert np.all(np.abs(np.abs(U) - 1 / math.sqrt(128)) < 1e-16)


# ---------------------------------------------------------------- calibration
def test_calibration_recovers_channel_mean_and_rms():
    rng = np.random.default_rng(9)
    s = 1 - 2 * rng.integers(0, 2, 128)
    mu = rng.standard_normal(128)
    sig = np.exp(rng.uniform(-1, 1, 128))
    pm = 1 - 2 * (np.arange(64)[:, None] % 2)    # +-1 in alternate tokens
    Y = mu[None, :] + sig[None, :] * pm            # mean mu, rms deviation sig
    m, sg = L.calibrate(L.hs_inverse(Y, s), s)
    assert np.allclose(m, mu, rtol=1e-6, atol=1e-7) and np.allclose(sg, sig, rtol=1e-6)
    assert np.array_equal(m, m.astype(np.float32).astype(np.float64))
    # a constant channel has scale 1
    m2, s2 = L.calibrate(np.zeros((8, 128)), None)
    assert np.all(s2 == 1.0) and np.all(m2 == 0.0)


# ---------------------------------------------------------------- allocation
def test_choose_depths_with_tree_gains_is_optimal_by_brute_force(tree):
    """Prop. 8 with Lemma 7's decreasing gains: the marginal-gain rule
    minimises sum_i a_i D(t_i) over every legal schedule; exact rationals."""
    rng = np.random.default_rng(11)
    g = tree.gains32
    D = [Fraction(1)]
    for t in range(1, 9):
        D.append(D[-1] - Fraction(float(g[t])))
    for trial in range(40):
        n, W = int(rng.integers(2, 4)), int(rng.integers(2, 5))
        a = rng.choice([0.0, 0.5, 1.0, 3.0, 7.25, 0.125], size=n)
        B = int(rng.integers(0, n * W + 2))
        t = choose_depths(a, g, W, B)
        obj = sum(Fraction(float(a[i])) * D[t[i]] for i in range(n))
        best = min(sum(Fraction(float(a[i])) * D[s[i]] for i in range(n))
                   for s in itertools.product(range(W + 1), repeat=n) if sum(s) <= B)
        assert obj == best and t.sum() <= B


# ------------------------------------------------------- worked examples
def test_two_token_attention_construction(tree):
    """App. E.1.2: identity transforms, zero means, unit scales; keys
    +-b c_1 e_1, query eta (5 sqrt(m)/c_1) e_1, B_K = 1, B_V = 8: both keys
    are read exactly, and all eight value levels go to the high-attention
    token, so the output is p Q_8(v_jstar)."""
    m, d = 128, 128
    c1 = tree.cent32[1][1]
    assert (math.exp(20) * tree.gains32[8] / tree.gains32[1]) > GOLD["lloyd_two_token_ratio"]["lower"]
    rng = np.random.default_rng(13)
    codec = L.Codec(tree=tree, sK=None, sV=None, muK=np.zeros((1, d)), sigK=np.ones((1, d)),
                    muV=np.zeros((1, d)), sigV=np.ones((1, d)))
    for b, eta in itertools.product((-1, 1), (-1, 1)):
        K = np.zeros((2, d))
        K[0, 0], K[1, 0] = b * c1, -b * c1
        V = rng.uniform(-1, 1, (2, d))
        q = np.zeros((1, d))
        q[0, 0] = eta * 5.0 * math.sqrt(m) / c1
        sk = L.lloyd_encode_stream(K, tree, None, 0.0, 1.0, 8, group_tokens=2)
        sv = L.lloyd_encode_stream(V, tree, None, 0.0, 1.0, 8, group_tokens=2)
        r = L.lloyd_decode_unit(q, sk, sv, codec, W=8, R_K=1.0 / m, R_V=4.0, vscale="unit")
        jstar = 0 if eta * b == 1 else 1
        assert r["tK"][0] == 1 and r["tK"][1:].sum() == 0
        assert np.allclose(r["zhat"][0], [5 * eta * b, -5 * eta * b], atol=1e-12)
        assert list(r["tV"]) == ([8, 0] if jstar == 0 else [0, 8])
        p = 1.0 / (1.0 + math.exp(-10.0))
        b8 = np.sort(np.concatenate([tree.bounds[t] for t in range(8)]))
        q8 = tree.cent32[8][np.searchsorted(b8, V[jstar], side="right")]
        assert np.allclose(r["out"][0], p * q8, rtol=1e-12, atol=1e-15)
        eps8 = 0.0097
        rho = 1 - p
        assert np.all(np.abs(p * V[jstar] + rho * V[1 - jstar] - r["out"][0]) <= p * eps8 + rho)


def test_full_unit_ball_obstruction(tree):
    """App. E.1.3: x = y = e_j, normalized Hadamard-sign transform, shared
    scale 1/sqrt(d): every key weight is 1/d^2, a budget of 2d gives every
    channel depth 2, and the inner-product estimate is Q_2(1)."""
    d = 128
    rng = np.random.default_rng(17)
    s = (1 - 2 * rng.integers(0, 2, d)).astype(np.float64)
    sc = 1.0 / math.sqrt(d)
    codec = L.Codec(tree=tree, sK=s, sV=s, muK=np.zeros((1, d)), sigK=np.full((1, d), sc),
                    muV=np.zeros((1, d)), sigV=np.full((1, d), sc))
    j = 5
    x = np.zeros((32, d))
    x[:, j] = 1.0       # one closed group of copies of e_j
    y = np.zeros((1, d))
    y[0, j] = 1.0
    sk = L.lloyd_encode_stream(x, tree, s, 0.0, sc, 8)
    sv = L.lloyd_encode_stream(x, tree, s, 0.0, sc, 8)
    assert np.allclose(L.lloyd_key_weights(L.hs_transform(y, s), codec.sigK[0]), 1.0 / d ** 2,
                       rtol=1e-12)
    r = L.lloyd_decode_unit(y, sk, sv, codec, W=8, R_K=2.0, R_V=0.0)
    assert np.all(r["tK"] == 2)
    q2 = float(tree.cent32[2][3])
    assert np.allclose(r["zhat"][0] * math.sqrt(d), q2, rtol=1e-12)


# -------------------------------------------------- decode: special cases
def test_open_group_only_is_plain_attention(tree):
    """Fewer than 32 tokens: nothing is packed, so the output is textbook
    softmax attention over the exact keys and values."""
    rng = np.random.default_rng(19)
    d, T = 128, 20
    s = (1 - 2 * rng.integers(0, 2, d)).astype(np.float64)
    codec = L.make_codec(tree, s, s, [rng.standard_normal((64, d))], [rng.standard_normal((64, d))])
    K, V, q = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((3, d))
    sk = L.lloyd_encode_stream(K, tree, s, codec.muK[0], codec.sigK[0], 8)
    sv = L.lloyd_encode_stream(V, tree, s, codec.muV[0], codec.sigV[0], 8)
    r = L.lloyd_decode_unit(q, sk, sv, codec, W=8, R_K=4, R_V=4)
    ref = softmax(q @ K.T / math.sqrt(d)) @ V
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


def test_empty_request_output_is_zero(tree):
    """Reading: a request with no tokens outputs the empty sum (zero) and
    allocates its key depths as any request does (these key weights hold no
    context term); a non-finite query gets the minimum depths."""
    rng = np.random.default_rng(29)
    d = 128
    s = (1 - 2 * rng.integers(0, 2, d)).astype(np.float64)
    codec = L.make_codec(tree, s, s, [rng.standard_normal((64, d))], [rng.standard_normal((64, d))])
    empty = np.zeros((0, d))
    sk = L.lloyd_encode_stream(empty, tree, s, codec.muK[0], codec.sigK[0], 8)
    sv = L.lloyd_encode_stream(empty, tree, s, codec.muV[0], codec.sigV[0], 8)
    q = rng.standard_normal((3, d))
    r = L.lloyd_decode_unit(q, sk, sv, codec, W=8, R_K=4, R_V=4)
    assert np.array_equal(r["out"], np.zeros((3, d))) and r["tV"].size == 0
    # the same key depths as a request with tokens (the weights are equal)
    K = rng.standard_normal((40, d))
    sk2 = L.lloyd_encode_stream(K, tree, s, codec.muK[0], codec.sigK[0], 8)
    sv2 = L.lloyd_encode_stream(K, tree, s, codec.muV[0], codec.sigV[0], 8)
    r2 = L.lloyd_decode_unit(q, sk2, sv2, codec, W=8, R_K=4, R_V=4)
    assert np.array_equal(r["tK"], r2["tK"]) and r["tK"].sum() == 4 * d
    q[1, 3] = np.nan
    r = L.lloyd_decode_unit(q, sk, sv, codec, W=8, R_K=4, R_V=4, min_depth=1)
    assert np.array_equal(r["out"], np.zeros((3, d))) and np.all(r["tK"] == 1)


def test_full_read_is_attention_over_depth_w_cells(tree):
    """R = W: every key channel and value token is read to depth W, so the
    output is attention over the depth-W reconstructions, built here from
    the sorted cell boundaries (searchsorted) and the transforms' matrices."""
    rng = np.random.default_rng(23)
    d, T, W = 128, 96 + 7, 6
    sK = (1 - 2 * rng.integers(0, 2, d)).astype(np.float64)
    sV = (1 - 2 * rng.integers(0, 2, d)).astype(np.float64)
    codec = L.make_codec(tree, sK, sV, [rng.standard_normal((128, d))], [rng.standard_normal((128, d))])
    K, V, q = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((2, d))
    sk = L.lloyd_encode_stream(K, tree, sK, codec.muK[0], codec.sigK[0], W)
    sv = L.lloyd_encode_stream(V, tree, sV, codec.muV[0], codec.sigV[0], W)
    r = L.lloyd_decode_unit(q, sk, sv, codec, W=W, R_K=W, R_V=W)
    assert np.all(r["tK"] == W) and np.all(r["tV"] == W)
    from scipy.linalg import hadamard
    UK = hadamard(d) * sK[None, :] / math.sqrt(d)
    UV = hadamard(d) * sV[None, :] / math.sqrt(d)
    bw = np.sort(np.concatenate([tree.bounds[t] for t in range(W)]))

    def q_w(X, U, mu, sig):
        z = (X @ U.T - mu) / sig
        return mu + sig * tree.cent32[W][np.searchsorted(bw, z, side="right")]
    Kh = q_w(K[:96], UK, codec.muK[0], codec.sigK[0])
    Vh = q_w(V[:96], UV, codec.muV[0], codec.sigV[0])
    qp = q @ UK.T
    logits = np.concatenate([qp @ Kh.T, q @ K[96:].T], axis=1) / math.sqrt(d)
    a = softmax(logits)
    ref = (a[:, :96] @ Vh) @ UV + a[:, 96:] @ V[96:]
    assert np.allclose(r["out"], ref, rtol=1e-9, atol=1e-9)


def test_nonfinite_group_and_query(tree):
    rng = np.random.default_rng(29)
    d = 128
    K = rng.standard_normal((64, d))
    K[40, 3] = np.inf
    sk = L.lloyd_encode_stream(K, tree, None, 0.0, 1.0, 8)
    assert list(sk.bad) == [False, True] and np.all(sk.codes[32:] == 0)
    codec = L.Codec(tree=tree, sK=None, sV=None, muK=np.zeros((1, d)), sigK=np.ones((1, d)),
                    muV=np.zeros((1, d)), sigV=np.ones((1, d)))
    q = rng.standard_normal((2, d))
    q[1, 0] = np.nan
    r = L.lloyd_decode_unit(q, sk, sk, codec, W=8, R_K=4, R_V=4)
    assert np.all(np.isnan(r["out"])) and np.all(r["tK"] == 0) and np.all(r["tV"] == 0)


def test_per_layer_budget_with_one_head_equals_per_head(tree):
    rng = np.random.default_rng(31)
    d = 128
    codec = L.make_codec(tree, None, None, [rng.standard_normal((64, d))], [rng.standard_normal((64, d))])
    K, V, q = rng.standard_normal((70, d)), rng.standard_normal((70, d)), rng.standard_normal((4, d))
    sk = L.lloyd_encode_stream(K, tree, None, codec.muK[0], codec.sigK[0], 8)
    sv = L.lloyd_encode_stream(V, tree, None, codec.muV[0], codec.sigV[0], 8)
    a = L.lloyd_decode_request(q, [(sk, sv)], codec, R_K=2.5, R_V=3.0, scope="layer")
    b = L.lloyd_decode_request(q, [(sk, sv)], codec, R_K=2.5, R_V=3.0, scope="kv_head")
    assert np.array_equal(a["tK"], b["tK"]) and np.array_equal(a["tV"], b["tV"])
    assert np.array_equal(a["out"], b["out"])


def test_metadata_bits():
    assert L.TABLE_ENTRIES == 518
    assert L.lloyd_metadata_bits(8) == 8 * 4 * 128 * 32 + 518 * 32
