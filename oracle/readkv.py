"""ReadKV decode step, written out plainly in float64 (CPU, numpy).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Each function names
the passage it follows.  Pages cited:

* [ReadKV] "Read What Matters: Query-Adaptive Quantization for KV Caches"
  (Bhandari, Gretta, Balasubramanian, Kasiviswanathan), arXiv 2610.11245.
* [AATC] "KV Cache Compression Through the Lens of Transform Coding",
  arXiv 2608.14191.

Readings taken where the pages leave a step open (each is listed with its
reason in the design notes of the repository):

* Codec: a per-(channel, 32-token group) uniform min/max quantiser stored as
  W MSB-first bit-planes instead of the pages' calibrated Gaussian Lloyd tree.
  The depth-t prefix P = code >> (W - t) names a dyadic cell of the group's
  range and reconstructs to its midpoint, which is the conditional mean of a
  uniform source on that cell ([ReadKV] App. D.1: every child of the tree
  stores its conditional mean).
* Distortion curve: D(t) proportional to 4^-t, the uniform-quantiser MSE
  range^2 / (12 * 4^t) ([AATC] App. B, Eq. (28)); the refinement gain of
  level t is therefore proportional to 4^-t.  A common positive factor (3/4,
  1/12, T/d_h) multiplies every gain of a stage and changes no choice, so the
  gain table used is exactly 4^-t (t = 1..W).
* Key item weight ([ReadKV] Sec. 3.2, Eq. (2), with sigma^2 read as the
  channel's summed squared group range) and value item weight (Eq. (3), with
  the physical-scale choice s_g of App. D.2 read per group, or s = 1).
* Budgets per (request, KV head): B_K = floor(R_K * d_h),
  B_V = floor(R_V * T_packed), R given as float32 ([ReadKV] Sec. 2 uses
  floor(R d); App. F.1 converts rates to integer increment budgets); or per
  request over all its KV heads (decode_request), items ordered by KV head.
* Tokens of the not-yet-full group are kept exactly and enter the softmax and
  the output, but not the allocation.
* A query with a non-finite value reads nothing: depths 0, outputs NaN.
* A unit with no tokens at all (the pages' read is over a non-empty context)
  reads nothing: its key weights are zero (no key energy), so its key depths
  are the minimum, and its output is the empty sum, zero, whatever the query.
* Restricted reader (min_depth=1, value_pairs): the minimum depth applies to
  both stages and its levels count against the budget; a value packet's
  weight is the sum of its two tokens' weights.
"""
from __future__ import annotations

import heapq
import math
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

__all__ = [
    "bf16_down", "bf16_up", "encode_stream", "EncodedStream", "prefix",
    "reconstruct", "gain_table", "choose_depths", "key_weights",
    "value_weights", "budget", "decode_unit", "softmax",
    "reuse_overhead", "reuse_reads", "logical_reads", "decode_request", "pair_depths",
]


# ----------------------------------------------------------------------------
# bfloat16 directed rounding (metadata precision reading)
# ----------------------------------------------------------------------------
_BF16_MIN_QUANTUM_EXP = -133   # bf16 subnormal spacing 2^-133
_BF16_MAX = float(np.array([0x7F7F0000], dtype=np.uint32).view(np.float32)[0])


def _bf16_directed(v: np.ndarray, up: bool) -> np.ndarray:
    """Round float64 values to bfloat16 (8 significant bits) toward +inf
    (``up``) or -inf.  v = m * 2^e with 0.5 <= |m| < 1; the bf16 grid near v
    has spacing 2^(e-8) (never finer than 2^-133)."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    qe = np.maximum(e.astype(np.int64) - 8, _BF16_MIN_QUANTUM_EXP)
    scaled = np.ldexp(v, (-qe).astype(np.int32))      # exact power-of-2 scale
    k = np.ceil(scaled) if up else np.floor(scaled)
    out = np.ldexp(k, qe.astype(np.int32))
    out = np.where(np.abs(out) > _BF16_MAX, np.copysign(np.inf, out), out)
    return out


def bf16_down(v):
    """Largest bfloat16 value <= v."""
    return _bf16_directed(v, up=False)


def bf16_up(v):
    """Smallest bfloat16 value >= v."""
    return _bf16_directed(v, up=True)


# ----------------------------------------------------------------------------
# Encoder: progressive uniform code per (channel, token group)
# ----------------------------------------------------------------------------
@dataclass
class EncodedStream:
    """One KV stream (one request, one KV head) after encoding.

    lo, rng : [n_groups][d] float64 -- bf16 group minimum (rounded down) and
              range (rounded up)
    codes   : [T_packed][d] int64 -- W-bit cell index of every packed scalar
    tail    : [r][d] float64 -- exact values of the open (not full) group
    bad     : [n_groups] bool -- group held a non-finite value (not coded)
    """
    W: int
    group_tokens: int
    lo: np.ndarray
    rng: np.ndarray
    codes: np.ndarray
    tail: np.ndarray
    bad: np.ndarray

    @property
    def n_groups(self) -> int:
        return self.lo.shape[0]

    @property
    def t_packed(self) -> int:
        return self.n_groups * self.group_tokens


def _exact_floor_ratio(num: np.ndarray, den: np.ndarray) -> np.ndarray:
    """floor(num / den) for float64 num >= 0, den > 0, evaluated exactly.
    The float quotient is used unless it lies within 1e-9 of an integer, in
    which case the exact rational quotient decides."""
    ratio = num / den
    out = np.floor(ratio)
    near = np.abs(ratio - np.rint(ratio)) <= 1e-9 * np.maximum(1.0, ratio)
    for idx in zip(*np.nonzero(near)):
        out[idx] = math.floor(Fraction(float(num[idx])) / Fraction(float(den[idx])))
    return out


def encode_stream(X: np.ndarray, W: int = 8, group_tokens: int = 32) -> EncodedStream:
    """Encode one stream's tokens X [T][d] (float64 holding the exact input
    values) group by group.

    Per channel c of a closed group (tokens 32*gamma .. 32*gamma+31):
      lo   = largest bf16 <= min_j x_j
      rng  = smallest bf16 >= fl64(max_j x_j - lo)
      code = min(floor(fl64(x - lo) * 2^W / rng), 2^W - 1)   (0 if rng = 0)
    This is the uniform scalar quantiser of [AATC] Sec. III-C, Definition 2
    (per-group zero point and scale) in its mid-rise cell form, so that every
    MSB-first prefix of the code is itself a uniform cell index ([ReadKV]
    Sec. 3.1: a stored W-bit path whose every prefix is decodable).
    """
    X = np.asarray(X, dtype=np.float64)
    T, d = X.shape
    gt = int(group_tokens)
    ng = T // gt
    tp = ng * gt
    G = X[:tp].reshape(ng, gt, d)
    finite = np.isfinite(G).all(axis=1)                    # [ng][d]
    bad = ~finite.all(axis=1)                              # [ng]
    Gs = np.where(bad[:, None, None], 0.0, G)
    lo = bf16_down(Gs.min(axis=1))
    rng = bf16_up(Gs.max(axis=1) - lo)
    # a range beyond the bf16 limit cannot be stored either: treat as bad
    bad = bad | ~(np.isfinite(lo) & np.isfinite(rng)).all(axis=1)
    lo = np.where(bad[:, None], 0.0, lo)
    rng = np.where(bad[:, None], 0.0, rng)
    lo = np.where(lo == 0.0, 0.0, lo)   # a zero minimum is stored as +0
    diff = Gs - lo[:, None, :]                             # fl64(x - lo) >= 0
    num = np.ldexp(diff, W)
    den = np.broadcast_to(rng[:, None, :], num.shape)
    codes = np.zeros(num.shape, dtype=np.int64)
    pos = den > 0
    if pos.any():
        q = _exact_floor_ratio(num[pos], den[pos])
        codes[pos] = np.minimum(q, 2 ** W - 1).astype(np.int64)
    lo = np.where(bad[:, None], 0.0, lo)
    rng = np.where(bad[:, None], 0.0, rng)
    codes[bad] = 0
    return EncodedStream(W=W, group_tokens=gt, lo=lo, rng=rng,
                         codes=codes.reshape(tp, d), tail=X[tp:].copy(), bad=bad)


def prefix(codes: np.ndarray, t: np.ndarray, W: int) -> np.ndarray:
    """Depth-t prefix P = code >> (W - t) (the first t MSB-first planes)."""
    return np.right_shift(codes, (W - np.asarray(t, dtype=np.int64)))


def reconstruct(lo, rng, P, t):
    """Midpoint of the depth-t dyadic cell named by prefix P:
    x_hat = lo + rng * (2P + 1) / 2^(t+1).  Depth 0 gives the group midpoint
    lo + rng/2.  (Reading of [ReadKV] Sec. 3.1 / App. D.1 for a uniform cell.)"""
    t = np.asarray(t, dtype=np.int64)
    return lo + rng * (2.0 * P + 1.0) / np.ldexp(1.0, t + 1)


# ----------------------------------------------------------------------------
# Allocation: ChooseDepths ([ReadKV] Sec. 3.3; exactness App. E.2.1 Prop. 8)
# ----------------------------------------------------------------------------
def gain_table(W: int) -> np.ndarray:
    """Refinement gain of level t = 1..W for D(t) ~ 4^-t, up to the common
    factor 3/4 (index 0 unused)."""
    return np.array([0.0] + [math.ldexp(1.0, -2 * t) for t in range(1, W + 1)])


def choose_depths(a: np.ndarray, gains: np.ndarray, W: int, B: int, start: int = 0) -> np.ndarray:
    """ChooseDepths(a, D, W, B): start from depth 0 everywhere and repeatedly
    deepen, by one level, the eligible item (depth < W) whose next refinement
    has the largest positive weighted gain a_i * gain[t_i + 1]; stop after B
    increments or when no positive gain remains.  Ties go to the lowest item
    index.  Max-heap form, O(N + B log N) ([ReadKV] Sec. 3.3).

    start = 1: the mandatory minimum depth of the restricted reader ([ReadKV]
    Sec. 5.1, App. F.8): every item starts at depth 1, and those N levels
    count against the budget (App. F.6 counts l*N + k(W - l) increments for a
    lower depth l), so max(0, B - N) increments remain."""
    a = np.asarray(a, dtype=np.float64)
    n = a.shape[0]
    t = np.full(n, start, dtype=np.int64)
    heap = []
    for i in range(n):
        if start >= W:
            break
        g = float(a[i]) * float(gains[start + 1])
        if g > 0.0:
            heap.append((-g, i))
    heapq.heapify(heap)
    B = max(0, B - start * n)
    taken = 0
    while taken < B and heap:
        negg, i = heapq.heappop(heap)
        t[i] += 1
        taken += 1
        if t[i] < W:
            g = float(a[i]) * float(gains[t[i] + 1])
            if g > 0.0:
                heapq.heappush(heap, (-g, i))
    return t


def budget(R: float, n_items: int) -> int:
    """Integer increment budget floor(R * N) with R taken as float32."""
    return int(math.floor(float(np.float32(R)) * n_items))


def key_weights(q_heads: np.ndarray, enc_k: EncodedStream) -> np.ndarray:
    """Key channel weight for one KV head ([ReadKV] Sec. 3.2, Eq. (2)):
    a_c = sum_{h in S(g)} q_{h,c}^2 * E_c, with E_c = sum over closed groups of
    rng_c^2 (the channel's scale, summed left to right in group order), and
    the head sum also taken left to right."""
    qsq = np.zeros(q_heads.shape[1])
    for h in range(q_heads.shape[0]):
        qsq = qsq + q_heads[h] * q_heads[h]
    E = np.zeros(q_heads.shape[1])
    for gam in range(enc_k.n_groups):
        E = E + enc_k.rng[gam] * enc_k.rng[gam]
    return qsq * E


def group_energy_v(enc_v: EncodedStream) -> np.ndarray:
    """s for each value group: sum over channels of rng^2, left to right."""
    E = np.zeros(enc_v.n_groups)
    for c in range(enc_v.rng.shape[1]):
        E = E + enc_v.rng[:, c] * enc_v.rng[:, c]
    return E


def value_weights(alpha_packed: np.ndarray, enc_v: EncodedStream,
                  vscale: str = "physical") -> np.ndarray:
    """Value token weight ([ReadKV] Sec. 3.2, Eq. (3)):
    a_j = s * sum_{h in S(g)} alpha_hat_{h,j}^2, where s is the summed squared
    channel range of token j's group (physical scale, App. D.2) or 1 (unit)."""
    asq = np.zeros(alpha_packed.shape[1])
    for h in range(alpha_packed.shape[0]):
        asq = asq + alpha_packed[h] * alpha_packed[h]
    if vscale == "unit":
        return asq
    s = np.repeat(group_energy_v(enc_v), enc_v.group_tokens)
    return asq * s


def softmax(z: np.ndarray) -> np.ndarray:
    m = z.max(axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=-1, keepdims=True)


# ----------------------------------------------------------------------------
# One decode step for one (request, KV head) unit ([ReadKV] Sec. 3, Alg. 1)
# ----------------------------------------------------------------------------
def pair_depths(wv, gains, W, BV, start):
    """Two-token value packets ([ReadKV] Sec. 5.1, App. F.8): tokens 2m and
    2m + 1 share one depth, so a packet is one item whose weight is the sum
    of its tokens' weights (the objective sum_j a_j D(t_j) with t shared),
    and one packet level costs two token levels: floor(B_V / 2) packet
    levels.  Returns the per-token depths."""
    wp = wv[0::2] + wv[1::2]
    tp2 = choose_depths(wp, gains, W, BV // 2, start)
    return np.repeat(tp2, 2), wp


def _empty_unit(gq, d, R_K, min_depth):
    """A unit with no tokens: zero key weights, key depths at the minimum,
    no value items, output the empty sum (zero)."""
    return dict(out=np.zeros((gq, d)), tK=np.full(d, min_depth, dtype=np.int64),
                tV=np.zeros(0, dtype=np.int64), wk=np.zeros(d), wv=np.zeros(0),
                BK=budget(R_K, d), BV=0, zhat=None, ahat=None, tp=0)


def decode_unit(q_heads, K, V, W=8, R_K=4.0, R_V=4.0, group_tokens=32,
                vscale="physical", enc_k=None, enc_v=None, diagnostics=False,
                min_depth=0, value_pairs=False):
    """Two-stage (staged(2)) read for the query heads S(g) sharing one KV
    stream.

    q_heads : [gqa][d] float64 (exact query values)
    K, V    : [T][d] float64 (exact cached values, append order)
    Returns a dict with ``out`` [gqa][d], key depths ``tK`` [d], value depths
    ``tV`` [T_packed], reconstructed logits, probabilities and weights.

    Stage 1: key weights (Eq. (2)) -> ChooseDepths with B_K.
    Intermediate decoder: logits q . k_hat / sqrt(d_h) from the reconstructed
      keys (exact keys for open-group tokens), softmax over all tokens.
    Stage 2: value weights (Eq. (3)) from those probabilities -> ChooseDepths
      with B_V over the packed tokens.
    Final decoder: o_h = sum_j alpha_hat_{h,j} v_hat_j.
    min_depth = 1 and value_pairs: the restricted GPU reader of [ReadKV]
    Sec. 5.1 / App. F.8 (mandatory minimum depth one in both stages;
    adjacent value tokens share a depth); ``wv`` then holds the packet
    weights.
    """
    q_heads = np.asarray(q_heads, dtype=np.float64)
    d = q_heads.shape[1]
    if np.asarray(K).shape[0] == 0:
        return _empty_unit(q_heads.shape[0], d, R_K, min_depth)
    if enc_k is None:
        enc_k = encode_stream(K, W, group_tokens)
    if enc_v is None:
        enc_v = encode_stream(V, W, group_tokens)
    tp = enc_k.t_packed
    gains = gain_table(W)
    gidx = np.arange(tp) // group_tokens

    if not np.isfinite(q_heads).all():
        # The pages define no read for a query that is not a real vector.
        # Reading: the unit reads nothing beyond the mandatory minimum depth
        # and every output of its query heads is NaN.
        gq = q_heads.shape[0]
        nv = tp // 2 if value_pairs else tp
        return dict(out=np.full((gq, d), np.nan), tK=np.full(d, min_depth, dtype=np.int64),
                    tV=np.full(tp, min_depth, dtype=np.int64), wk=np.zeros(d), wv=np.zeros(nv),
                    BK=budget(R_K, d), BV=budget(R_V, tp), zhat=None, ahat=None, tp=tp)

    # stage 1: key prefix depths
    wk = key_weights(q_heads, enc_k)
    BK = budget(R_K, d)
    tK = choose_depths(wk, gains, W, BK, min_depth)

    # intermediate decoder
    Khat = reconstruct(enc_k.lo[gidx], enc_k.rng[gidx],
                       prefix(enc_k.codes, tK[None, :], W), tK[None, :])
    Kfull_hat = np.concatenate([Khat, enc_k.tail], axis=0)
    zhat = (q_heads @ Kfull_hat.T) / math.sqrt(d)
    ahat = softmax(zhat)

    # stage 2: value prefix depths
    wv = value_weights(ahat[:, :tp], enc_v, vscale)
    BV = budget(R_V, tp)
    if value_pairs:
        tV, wv = pair_depths(wv, gains, W, BV, min_depth)
    else:
        tV = choose_depths(wv, gains, W, BV, min_depth)

    Vhat = reconstruct(enc_v.lo[gidx], enc_v.rng[gidx],
                       prefix(enc_v.codes, tV[:, None], W), tV[:, None])
    Vfull_hat = np.concatenate([Vhat, enc_v.tail], axis=0)
    out = ahat @ Vfull_hat

    res = dict(out=out, tK=tK, tV=tV, wk=wk, wv=wv, BK=BK, BV=BV,
               zhat=zhat, ahat=ahat, tp=tp)
    if diagnostics:
        res.update(Khat=Kfull_hat, Vhat=Vfull_hat, enc_k=enc_k, enc_v=enc_v)
    return res


# ----------------------------------------------------------------------------
# One decode step for one request with per-layer budgets ([ReadKV] Sec. 3.3)
# ----------------------------------------------------------------------------
def decode_request(q_all, Ks, Vs, W=8, R_K=4.0, R_V=4.0, group_tokens=32,
                   vscale="physical", encs=None, min_depth=0, value_pairs=False):
    """The flexible reader of [ReadKV] Sec. 3.3: one key budget and one
    value budget for the whole layer of a request instead of one per KV head
    (the per-head budgets are the GPU reader's restriction of Sec. 5.1 /
    App. F.8).  Stage 1 runs ChooseDepths over the G * d_h key channels
    with B_K = floor(R_K * G * d_h); stage 2 over the G * T_packed packed
    tokens with B_V = floor(R_V * G * T_packed).  Items are ordered by KV
    head, then channel / token; ties go to the lowest in that order.

    q_all : [H][d] (query heads of the request, H = G * gqa)
    Ks, Vs: G arrays [T][d] (the request's KV streams)
    encs  : optional list of (enc_k, enc_v) per KV head
    Returns out [G][gqa][d], tK [G][d], tV [G][T_packed], the pooled weight
    vectors wk [G*d], wv [G*T_packed] and budgets BK, BV.  A KV head with a
    non-finite query value reads nothing (zero weights, NaN outputs).
    """
    q_all = np.asarray(q_all, dtype=np.float64)
    G = len(Ks)
    d = q_all.shape[1]
    gqa = q_all.shape[0] // G
    if np.asarray(Ks[0]).shape[0] == 0:
        # no tokens in the request (every KV head empty): see _empty_unit
        return dict(out=np.zeros((G, gqa, d)), tK=np.full((G, d), min_depth, dtype=np.int64),
                    tV=np.zeros((G, 0), dtype=np.int64), wk=np.zeros(G * d), wv=np.zeros(0),
                    BK=budget(R_K, G * d), BV=0, tp=0)
    if encs is None:
        encs = [(encode_stream(Ks[g], W, group_tokens), encode_stream(Vs[g], W, group_tokens))
                for g in range(G)]
    tp = encs[0][0].t_packed
    gains = gain_table(W)
    gidx = np.arange(tp) // group_tokens
    qs = [q_all[g * gqa:(g + 1) * gqa] for g in range(G)]
    good = [bool(np.isfinite(qs[g]).all()) for g in range(G)]

    # stage 1: pooled key items
    wk = np.concatenate([key_weights(qs[g], encs[g][0]) if good[g] else np.zeros(d)
                         for g in range(G)])
    BK = budget(R_K, G * d)
    tK = choose_depths(wk, gains, W, BK, min_depth).reshape(G, d)

    # intermediate decoder, per KV head
    ahat = []
    for g in range(G):
        ek = encs[g][0]
        Khat = reconstruct(ek.lo[gidx], ek.rng[gidx], prefix(ek.codes, tK[g][None, :], W),
                           tK[g][None, :])
        z = (qs[g] @ np.concatenate([Khat, ek.tail], axis=0).T) / math.sqrt(d)
        ahat.append(softmax(z) if good[g] else np.full(z.shape, np.nan))

    # stage 2: pooled value items
    wv = np.concatenate([value_weights(ahat[g][:, :tp], encs[g][1], vscale) if good[g]
                         else np.zeros(tp) for g in range(G)])
    BV = budget(R_V, G * tp)
    if value_pairs:
        tV, wv = pair_depths(wv, gains, W, BV, min_depth)
        tV = tV.reshape(G, tp)
    else:
        tV = choose_depths(wv, gains, W, BV, min_depth).reshape(G, tp)

    out = np.zeros((G, gqa, d))
    for g in range(G):
        ev = encs[g][1]
        Vhat = reconstruct(ev.lo[gidx], ev.rng[gidx], prefix(ev.codes, tV[g][:, None], W),
                           tV[g][:, None])
        out[g] = ahat[g] @ np.concatenate([Vhat, ev.tail], axis=0)
    return dict(out=out, tK=tK, tV=tV, wk=wk, wv=wv, BK=BK, BV=BV, tp=tp)


# ----------------------------------------------------------------------------
# Logical-read accounting of one decode unit ([ReadKV] App. A.1)
# ----------------------------------------------------------------------------
def logical_reads(tK, tV, n_tokens, d=128, group_tokens=32, elem_bits=16):
    """Bits one decode of a (request, KV head) unit asks for ([ReadKV] App.
    A.1 counts payload and metadata the reader requests, not workspace):

    key payload   = T_packed * sum_c t^K_c   (t bits of every packed token)
    value payload = d * sum_j t^V_j          (t bits of every channel)
    metadata      = lo and rng (16 bits each) of every closed group and
                    channel of keys and of values, plus the channel energies
                    E^K (d x 64 bits) and the group energies E^V (64 bits each)
    open group    = keys and values of the not-yet-closed group, exact.
    """
    tp = (n_tokens // group_tokens) * group_tokens
    ng = tp // group_tokens
    return dict(key_payload=int(tp * int(np.sum(tK))),
                value_payload=int(d * int(np.sum(tV))),
                metadata=int(2 * ng * d * 32 + d * 64 + ng * 64),
                open_group=int(2 * (n_tokens - tp) * d * elem_bits))


# ----------------------------------------------------------------------------
# Payload-only reuse model ([ReadKV] App. A.2-A.3)
# ----------------------------------------------------------------------------
def reuse_reads(N: int, L: int) -> int:
    """Historical-cache reads over L decode steps after an N-token prompt:
    sum_{t=0}^{L-1} (N + t)."""
    return sum(N + t for t in range(L))


def reuse_overhead(N: int, L: int, W: int, W0: int) -> float:
    """Extra insertion traffic of storing W instead of W0 bits, as a fraction
    of the W0-bit cumulative reads: (W - W0) * inserted / (W0 * reads), with
    one insertion per prompt and per generated token."""
    return (W - W0) * (N + L) / (W0 * reuse_reads(N, L))
