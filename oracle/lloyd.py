"""ReadKV's own progressive codec, written out plainly in float64 (CPU, numpy).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Each function names
the passage of [ReadKV] ("Read What Matters: Query-Adaptive Quantization for
KV Caches", arXiv 2610.11245) it follows.

The codec of Sec. 3.1 and App. D.1: every transformed scalar x' of a key or
value is standardised with a calibrated channel mean and scale,
z = (x' - mu) / sigma, and stored as its path in a binary tree fitted to
Z ~ N(0, 1): a node's interval is cut in two where the expected squared
error under N(0, 1) is lowest, a child reconstructs to E[Z | child], and at
that cut the boundary equals the average of the two children's
reconstructions (the Lloyd condition).  A depth-t prefix of the path
reconstructs to mu + sigma * (centroid of its depth-t cell); depth 0 gives mu.

Readings taken where the pages leave a step open (each is listed in the
design notes of the repository):

* The deployed table holds float32 entries (App. D.1, Lemma 7): the tree is
  built in float64 and its centroids and the eight refinement gains
  Delta_t = D(t-1) - D(t) are rounded to float32.  The encoder's boundaries
  are the midpoints of the float32 child centroids, taken exactly in float64.
  The tree is built on the positive half line and mirrored (the density is
  even), so the table is exactly symmetric.
* A scalar goes to the upper child when z >= boundary.  A store with W < 8
  planes keeps the first W levels of the same depth-8 tree.
* Hadamard-sign transform U x = H (s . x) / sqrt(d) with the Sylvester
  Hadamard matrix H and a sign vector s drawn once per layer, one for keys
  and queries, one for values (Sec. 3.1); the output is mapped back with
  U^T y = s . (H y) / sqrt(d).
* Calibration (App. D.1): per KV head and transformed channel, mu is the mean
  and sigma the root-mean-square deviation of a calibration split, summed
  left to right in token order in float64, then rounded to float32; a zero
  or non-finite sigma is replaced by 1.
* A closed group holding a non-finite value on one side (keys or values)
  stores code 0 for all of that side's scalars and raises the store's flag.
* Key weight a_c = sum_h (q'_{h,c} sigma^K_c)^2 (Eq. (2)); value weight
  a_j = s_g sum_h alpha_hat_{h,j}^2 with s_g = sum_c (sigma^V_c)^2 or 1
  (Eq. (3), App. D.2).  Tokens of the open group are read exactly: their
  logits are q . k / sqrt(d) and their values are added after the inverse
  value transform.
* A request with no tokens: output zero (the empty sum) whatever the query;
  its key depths are allocated as for any request (these key weights hold no
  context term).
* Logical reads (App. A.1): each decode call is charged one load of the
  layer's calibration arrays (mu, sigma of keys and values, float32) and of
  the decoder table (510 centroids of depths 1..8 and 8 gains, float32).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
from scipy.linalg import hadamard
from scipy.special import ndtr

from .readkv import budget, choose_depths, softmax

__all__ = [
    "TREE_DEPTH", "LloydTree", "lloyd_tree", "inv_sqrt_d", "hs_transform", "hs_inverse",
    "calibrate", "Codec", "make_codec", "tree_codes", "LloydStream", "lloyd_encode_stream",
    "lloyd_reconstruct", "lloyd_key_weights", "lloyd_value_weights", "lloyd_decode_request",
    "lloyd_decode_unit", "lloyd_metadata_bits", "TABLE_ENTRIES",
]

TREE_DEPTH = 8
TABLE_ENTRIES = (2 ** (TREE_DEPTH + 1) - 2) + TREE_DEPTH  # centroids of depths 1..8, gains


# ----------------------------------------------------------------------------
# The Gaussian Lloyd tree ([ReadKV] App. D.1)
# ----------------------------------------------------------------------------
def _pdf(x: float) -> float:
    return 0.0 if math.isinf(x) else math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _mass(a: float, b: float) -> float:
    """P(a < Z < b) for 0 <= a < b (upper-tail form keeps tail cells exact)."""
    return float(ndtr(-a) - ndtr(-b))


def _cmean(a: float, b: float) -> float:
    """E[Z | a < Z < b], 0 <= a < b <= inf."""
    return (_pdf(a) - _pdf(b)) / _mass(a, b)


def _split(a: float, b: float) -> float:
    """The Lloyd-stationary split of (a, b): the point x with
    x = (E[Z | a<Z<x] + E[Z | x<Z<b]) / 2, by bisection (x minus that
    midpoint is negative near a and positive near b)."""
    lo = a
    hi = b if not math.isinf(b) else _cmean(a, b) + 40.0
    for _ in range(400):
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        f = mid - 0.5 * (_cmean(a, mid) + _cmean(mid, b))
        if f < 0.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


@dataclass
class LloydTree:
    """edges[t]: the 2^t + 1 cell edges at depth t (float64, -inf .. inf);
    cent[t]: the 2^t centroids (float64); D[t]: distortion after t bits;
    gains[t] = Delta_t = D(t-1) - D(t) (index 0 unused); the float32 table:
    cent32[t], gains32[t]; bounds[t][P]: the boundary that splits depth-t
    cell P, the midpoint of its float32 children (float64, exact)."""
    edges: list
    cent: list
    D: np.ndarray
    gains: np.ndarray
    cent32: list
    gains32: np.ndarray
    bounds: list

    def flat_centroids32(self) -> np.ndarray:
        """float32 centroids in one array, index (2^t - 1) + P (depth 0 at 0)."""
        return np.concatenate([self.cent32[t] for t in range(TREE_DEPTH + 1)])


def lloyd_tree(depth: int = TREE_DEPTH) -> LloydTree:
    """Build the depth-``depth`` tree for N(0, 1) ([ReadKV] App. D.1)."""
    # positive half: cells of (0, inf), refined level by level
    half_edges = [[0.0, math.inf]]
    for t in range(1, depth):
        e = half_edges[-1]
        nxt = [e[0]]
        for i in range(len(e) - 1):
            nxt += [_split(e[i], e[i + 1]), e[i + 1]]
        half_edges.append(nxt)
    edges, cent, D = [], [], []
    for t in range(depth + 1):
        if t == 0:
            ed = [-math.inf, math.inf]
            cs = [0.0]
            d_t = 1.0
        else:
            he = half_edges[t - 1]
            pos = [_cmean(he[i], he[i + 1]) for i in range(len(he) - 1)]
            ed = [-x for x in reversed(he[1:])] + he
            cs = [-c for c in reversed(pos)] + pos
            # D(t) = E[Z^2] - E[Q_t(Z)^2] = 1 - sum_cells P(cell) c^2
            d_t = 1.0 - 2.0 * sum(_mass(he[i], he[i + 1]) * pos[i] ** 2 for i in range(len(pos)))
        edges.append(np.array(ed))
        cent.append(np.array(cs))
        D.append(d_t)
    D = np.array(D)
    # Delta_t from the cell sums directly (no cancellation against 1)
    gains = np.zeros(depth + 1)
    for t in range(1, depth + 1):
        he_t = half_edges[t - 1]
        s_t = sum(_mass(he_t[i], he_t[i + 1]) * _cmean(he_t[i], he_t[i + 1]) ** 2
                  for i in range(len(he_t) - 1))
        if t == 1:
            s_prev = 0.0
        else:
            he_p = half_edges[t - 2]
            s_prev = sum(_mass(he_p[i], he_p[i + 1]) * _cmean(he_p[i], he_p[i + 1]) ** 2
                         for i in range(len(he_p) - 1))
        gains[t] = 2.0 * (s_t - s_prev)
    cent32 = [c.astype(np.float32).astype(np.float64) for c in cent]
    gains32 = gains.astype(np.float32).astype(np.float64)
    bounds = [np.array([(cent32[t + 1][2 * P] + cent32[t + 1][2 * P + 1]) / 2.0
                        for P in range(2 ** t)]) for t in range(depth)]
    return LloydTree(edges=edges, cent=cent, D=D, gains=gains, cent32=cent32,
                     gains32=gains32, bounds=bounds)


def tree_codes(z: np.ndarray, tree: LloydTree, W: int) -> np.ndarray:
    """The W-bit path of every standardised scalar z: walk down from the
    root, taking the upper child when z >= the node's boundary; the path of
    the depth-8 walk truncated to its first W bits.  (NaN goes to code 0.)"""
    z = np.asarray(z, dtype=np.float64)
    P = np.zeros(z.shape, dtype=np.int64)
    for t in range(TREE_DEPTH):
        beta = tree.bounds[t][P]
        P = 2 * P + (z >= beta).astype(np.int64)
    return P >> (TREE_DEPTH - W)


# ----------------------------------------------------------------------------
# Hadamard-sign transforms ([ReadKV] Sec. 3.1)
# ----------------------------------------------------------------------------
def inv_sqrt_d(d: int) -> float:
    """1/sqrt(d) correctly rounded, for d a power of two: 2^(-k/2) is a power
    of two for even k and sqrt(1/2) 2^(-(k-1)/2) for odd k."""
    k = int(d).bit_length() - 1
    assert d == 1 << k
    return math.ldexp(1.0, -k // 2) if k % 2 == 0 else math.ldexp(math.sqrt(0.5), -(k - 1) // 2)


def hs_transform(X: np.ndarray, signs) -> np.ndarray:
    """U x = H (s . x) / sqrt(d) for each row x of X (float64).  signs=None:
    the identity transform (used by the worked examples of App. E.1.2)."""
    X = np.asarray(X, dtype=np.float64)
    if signs is None:
        return X.copy()
    d = X.shape[-1]
    H = hadamard(d).astype(np.float64)
    return ((X * signs) @ H) * inv_sqrt_d(d)


def hs_inverse(Y: np.ndarray, signs) -> np.ndarray:
    """U^T y = s . (H y) / sqrt(d) for each row y of Y (signs=None: identity)."""
    Y = np.asarray(Y, dtype=np.float64)
    if signs is None:
        return Y.copy()
    d = Y.shape[-1]
    H = hadamard(d).astype(np.float64)
    return ((Y @ H) * inv_sqrt_d(d)) * signs


# ----------------------------------------------------------------------------
# Calibration ([ReadKV] App. D.1) and the codec state of one layer
# ----------------------------------------------------------------------------
def calibrate(Xcal: np.ndarray, signs: np.ndarray):
    """Per transformed channel of one KV head: mean and root-mean-square
    deviation of the calibration tokens Xcal [N][d], sums left to right in
    token order, rounded to float32 (returned as float64 arrays)."""
    Xp = hs_transform(Xcal, signs)
    n = Xp.shape[0]
    s = np.zeros(Xp.shape[1])
    for j in range(n):
        s = s + Xp[j]
    mu = s / n
    s2 = np.zeros(Xp.shape[1])
    for j in range(n):
        dv = Xp[j] - mu
        s2 = s2 + dv * dv
    sigma = np.sqrt(s2 / n)
    sigma = np.where(np.isfinite(sigma) & (sigma > 0.0), sigma, 1.0)
    f32 = lambda v: v.astype(np.float32).astype(np.float64)  # noqa: E731
    return f32(mu), f32(sigma)


@dataclass
class Codec:
    """One layer's codec state: the tree, the sign vectors of U_K and U_V,
    and per KV head g the float32 calibration arrays muK[g], sigK[g], muV[g],
    sigV[g] (each [d])."""
    tree: LloydTree
    sK: np.ndarray
    sV: np.ndarray
    muK: np.ndarray
    sigK: np.ndarray
    muV: np.ndarray
    sigV: np.ndarray

    def s_phys(self, g: int) -> float:
        """s_g = sum_c (sigma^V_{g,c})^2, left to right (App. D.2)."""
        s = 0.0
        for v in self.sigV[g]:
            s = s + v * v
        return s


def make_codec(tree: LloydTree, sK, sV, Kcal: list, Vcal: list) -> Codec:
    """Calibrate every KV head g from its calibration tokens Kcal[g], Vcal[g]."""
    muK, sigK, muV, sigV = [], [], [], []
    for g in range(len(Kcal)):
        m, s = calibrate(Kcal[g], sK)
        muK.append(m)
        sigK.append(s)
        m, s = calibrate(Vcal[g], sV)
        muV.append(m)
        sigV.append(s)
    f64 = lambda v: None if v is None else np.asarray(v, dtype=np.float64)  # noqa: E731
    return Codec(tree=tree, sK=f64(sK), sV=f64(sV), muK=np.array(muK), sigK=np.array(sigK), muV=np.array(muV), sigV=np.array(sigV))


# ----------------------------------------------------------------------------
# Encoder ([ReadKV] Sec. 3.1, Algorithm 1 encoder)
# ----------------------------------------------------------------------------
@dataclass
class LloydStream:
    """One KV stream after encoding: codes [T_packed][d] (W-bit paths),
    tail [r][d] (exact values of the open group), bad [n_groups]."""
    W: int
    group_tokens: int
    codes: np.ndarray
    tail: np.ndarray
    bad: np.ndarray

    @property
    def t_packed(self) -> int:
        return self.codes.shape[0]

    @property
    def n_groups(self) -> int:
        return self.codes.shape[0] // self.group_tokens

    # the store keeps no group metadata for this code: zero lo / rng
    @property
    def lo(self) -> np.ndarray:
        return np.zeros((self.n_groups, self.codes.shape[1]))

    @property
    def rng(self) -> np.ndarray:
        return np.zeros((self.n_groups, self.codes.shape[1]))


def lloyd_encode_stream(X: np.ndarray, tree: LloydTree, signs, mu, sigma, W: int = 8,
                        group_tokens: int = 32) -> LloydStream:
    """Encode the closed groups of one stream X [T][d]: transform, standardise
    z = (x' - mu) / sigma, store the tree path of every scalar."""
    X = np.asarray(X, dtype=np.float64)
    T, d = X.shape
    ng = T // group_tokens
    tp = ng * group_tokens
    codes = np.zeros((tp, d), dtype=np.int64)
    bad = np.zeros(ng, dtype=bool)
    for gam in range(ng):
        rows = X[gam * group_tokens:(gam + 1) * group_tokens]
        if not np.isfinite(rows).all():
            bad[gam] = True
            continue
        z = (hs_transform(rows, signs) - mu) / sigma
        codes[gam * group_tokens:(gam + 1) * group_tokens] = tree_codes(z, tree, W)
    return LloydStream(W=W, group_tokens=group_tokens, codes=codes, tail=X[tp:].copy(), bad=bad)


def lloyd_reconstruct(codes: np.ndarray, t, mu, sigma, tree: LloydTree, W: int) -> np.ndarray:
    """mu + sigma * (float32 centroid of the depth-t cell named by the first
    t bits of the path); depth 0 gives mu."""
    t = np.asarray(t, dtype=np.int64)
    P = np.right_shift(codes, W - t)
    table = tree.flat_centroids32()
    return mu + sigma * table[(np.left_shift(1, t) - 1) + P]


# ----------------------------------------------------------------------------
# Weights and one decode step ([ReadKV] Sec. 3.2-3.3, Algorithm 1)
# ----------------------------------------------------------------------------
def lloyd_key_weights(qp_heads: np.ndarray, sig: np.ndarray) -> np.ndarray:
    """a_c = sum_{h in S(g)} (q'_{h,c} sigma^K_c)^2, heads left to right
    (Eq. (2))."""
    a = np.zeros(qp_heads.shape[1])
    for h in range(qp_heads.shape[0]):
        x = qp_heads[h] * sig
        a = a + x * x
    return a


def lloyd_value_weights(alpha_packed: np.ndarray, s: float) -> np.ndarray:
    """a_j = s_g sum_{h in S(g)} alpha_hat_{h,j}^2, heads left to right
    (Eq. (3))."""
    asq = np.zeros(alpha_packed.shape[1])
    for h in range(alpha_packed.shape[0]):
        asq = asq + alpha_packed[h] * alpha_packed[h]
    return asq * s


def _pairs(wv, gains, W, BV, start):
    wp = wv[0::2] + wv[1::2]
    return np.repeat(choose_depths(wp, gains, W, BV // 2, start), 2), wp


def lloyd_decode_request(q_all, streams, codec: Codec, W=8, R_K=4.0, R_V=4.0,
                         vscale="physical", scope="kv_head", min_depth=0, value_pairs=False):
    """One decode step of one request over its G KV streams (staged(2)).

    q_all   : [H][d] query heads of the request (H = G * gqa), exact values
    streams : G pairs (LloydStream of keys, LloydStream of values)
    scope   : "kv_head" -- one key and one value budget per KV head;
              "layer"   -- one pooled budget over all KV heads (Sec. 3.3),
              items ordered by KV head, then channel / token
    Returns out [G][gqa][d], tK [G][d], tV [G][T_packed], the weights and
    budgets, and the reconstructed logits zhat [G][gqa][T].

    Stage 1: q' = U_K q; key weights (Eq. (2)) -> ChooseDepths with the
      tree's gains.  Intermediate decoder: logits q' . k_hat' / sqrt(d) for
      packed tokens (k_hat' = mu + sigma * centroid), q . k / sqrt(d) for the
      open group, softmax over all tokens.  Stage 2: value weights (Eq. (3))
      -> ChooseDepths.  Final decoder: o = U_V^T (sum_packed alpha v_hat')
      + sum_open alpha v.
    """
    q_all = np.asarray(q_all, dtype=np.float64)
    G = len(streams)
    d = q_all.shape[1]
    gqa = q_all.shape[0] // G
    tree = codec.tree
    gains = tree.gains32
    tp = streams[0][0].t_packed
    qs = [q_all[g * gqa:(g + 1) * gqa] for g in range(G)]
    good = [bool(np.isfinite(qs[g]).all()) for g in range(G)]
    qp = [hs_transform(qs[g], codec.sK) for g in range(G)]
    wk = [lloyd_key_weights(qp[g], codec.sigK[g]) if good[g] else np.zeros(d) for g in range(G)]
    nv = tp // 2 if value_pairs else tp

    def keys(ws, BK):
        return choose_depths(ws, gains, W, BK, min_depth)

    if scope == "layer":
        BK = budget(R_K, G * d)
        tK = keys(np.concatenate(wk), BK).reshape(G, d)
    else:
        BK = budget(R_K, d)
        tK = np.stack([keys(wk[g], BK) for g in range(G)])

    if tp == 0 and all(streams[g][0].tail.shape[0] == 0 for g in range(G)):
        # No tokens in the request: the output is the empty sum, zero, whatever
        # the query; the key depths are allocated as for any request (these key
        # weights do not depend on the context), the minimum for a non-finite
        # query.
        for g in range(G):
            if not good[g]:
                tK[g] = min_depth
        return dict(out=np.zeros((G, gqa, d)), tK=tK, tV=np.zeros((G, 0), dtype=np.int64),
                    wk=np.concatenate(wk) if G else np.zeros(0), wv=np.zeros(0), BK=BK, BV=0,
                    zhat=[np.zeros((gqa, 0))] * G, ahat=[np.zeros((gqa, 0))] * G, tp=0, nv=0)

    zhat, ahat = [], []
    for g in range(G):
        sk = streams[g][0]
        Khat = lloyd_reconstruct(sk.codes, tK[g][None, :], codec.muK[g], codec.sigK[g], tree, W)
        z = np.concatenate([qp[g] @ Khat.T, qs[g] @ sk.tail.T], axis=1) * inv_sqrt_d(d)
        zhat.append(z)
        ahat.append(softmax(z) if good[g] else np.full(z.shape, np.nan))

    sv = [codec.s_phys(g) if vscale == "physical" else 1.0 for g in range(G)]
    wv = [lloyd_value_weights(ahat[g][:, :tp], sv[g]) if good[g] else np.zeros(tp) for g in range(G)]

    def values(ws, BV):
        if value_pairs:
            return _pairs(ws, gains, W, BV, min_depth)
        return choose_depths(ws, gains, W, BV, min_depth), ws

    if scope == "layer":
        BV = budget(R_V, G * tp)
        tV, wvp = values(np.concatenate(wv), BV)
        tV = tV.reshape(G, tp)
    else:
        BV = budget(R_V, tp)
        res = [values(wv[g], BV) for g in range(G)]
        tV = np.stack([r[0] for r in res]) if G else np.zeros((0, tp), dtype=np.int64)
        wvp = np.concatenate([r[1] for r in res]) if G else np.zeros(0)
    for g in range(G):
        if not good[g]:
            tK[g] = min_depth
            tV[g] = min_depth

    out = np.zeros((G, gqa, d))
    for g in range(G):
        sv_ = streams[g][1]
        Vhat = lloyd_reconstruct(sv_.codes, tV[g][:, None], codec.muV[g], codec.sigV[g], tree, W)
        o_t = ahat[g][:, :tp] @ Vhat
        out[g] = hs_inverse(o_t, codec.sV) + ahat[g][:, tp:] @ sv_.tail
    return dict(out=out, tK=tK, tV=tV, wk=np.concatenate(wk) if G else np.zeros(0), wv=wvp,
                BK=BK, BV=BV, zhat=zhat, ahat=ahat, tp=tp, nv=nv)


def lloyd_decode_unit(q_heads, sk: LloydStream, sv: LloydStream, codec: Codec, g: int = 0, **kw):
    """lloyd_decode_request for one (request, KV head) unit with per-KV-head
    budgets: the codec's head g supplies the calibration arrays."""
    sub = Codec(tree=codec.tree, sK=codec.sK, sV=codec.sV, muK=codec.muK[g:g + 1],
                sigK=codec.sigK[g:g + 1], muV=codec.muV[g:g + 1], sigV=codec.sigV[g:g + 1])
    r = lloyd_decode_request(q_heads, [(sk, sv)], sub, scope="kv_head", **kw)
    return dict(out=r["out"][0], tK=r["tK"][0], tV=r["tV"][0], wk=r["wk"], wv=r["wv"], BK=r["BK"],
                BV=r["BV"], zhat=r["zhat"][0], ahat=r["ahat"][0], tp=r["tp"])


def lloyd_metadata_bits(G: int, d: int = 128) -> int:
    """Shared decoder data one decode call is charged for ([ReadKV] App.
    A.1): the layer's calibration arrays (mu and sigma of keys and values,
    float32, per KV head and channel) and the decoder table (float32)."""
    return G * 4 * d * 32 + TABLE_ENTRIES * 32
