"""Seeded synthetic inputs for ReadKV decode workloads.

This module only draws numbers: it holds none of the method's arithmetic (no
quantiser, no allocation, no attention).  Both the HIP path's tests/benchmark
and the float64 oracle take their inputs from here, so they see identical
values.

Every draw comes from numpy's PCG64 seeded with
``SeedSequence([workload_id, stream, b, g, step])``, so any single
(request, KV head) unit or decode step can be regenerated on its own.

Workloads (shapes and value distributions follow the decode workloads used to
study the method; the pages measure quality on public suites and a model's
layer activations, which are replaced here by these synthetic caches):

1. tiny: 1 query head / 1 KV head, d=128, T0=1024, batch 1, fp32 K/V with
   per-channel scale sigma_c ~ LogUniform[0.1, 10], q ~ N(0,1), 16 steps.
2. llama3-8b layer: 32 q / 8 KV heads (GQA 4), d=128, batch 16, T0=8192,
   bf16 K/V = sigma (.) z + A_g u_j (rank-8 shared part), q bf16 with
   Student-t(3) channel magnitudes, 128 steps appending one token each.
3. long context: as 2 with batch 4, T0=131072, 64 planted needle keys per
   (request, KV head) aligned (cos ~0.9) with the query heads, 8 steps.
4. large batch: 28 q / 4 KV heads (GQA 7), batch 64, per-request T0 drawn
   uniformly from [2048, 32768], 16 steps.
5. encode+decode mix: 32/8 heads, batch 32, T0=16384, 256 steps, R=3 budgets.

Options a test may add to a workload (``workload(id, **overrides)``):

* ``key_ties``: key channel 2k+1 repeats channel 2k in every token, and so
  does the query, so key weights come in bitwise-equal pairs;
* ``gap=(Q, D, period)``: the heads of KV group g share a direction u (per
  request and KV group); their queries are Q u + N(0, 1) noise, and every
  ``period``-th token (seeded phase) gets D u added to its key, which puts
  the other tokens a few hundred nats below those peaks;
* ``q_scale``: the query is multiplied by this factor (near-uniform
  attention when small);
* ``q_log2_spread``: query channel c scaled by an exact power of two.

For the pages' own codec (Gaussian Lloyd tree with Hadamard-sign transforms)
two more draws: ``codec_signs`` (the two sign vectors, drawn once per layer)
and ``calibration_split`` (held-out tokens of every KV head, from the same
distribution as the cache but from draws of their own).
"""
from __future__ import annotations

import numpy as np

# stream ids for SeedSequence
(_S_K, _S_V, _S_Q, _S_SIGMA, _S_A, _S_NEEDLE, _S_LEN, _S_QBASE, _S_GAP, _S_CAL,
 _S_SIGN) = range(11)

WORKLOADS = {
    1: dict(name="tiny-1q1kv-d128-T1024", B=1, H=1, G=1, d=128, T0=1024,
            steps=16, dtype="f32", W=8, R=[(4.0, 4.0)], structure="iid"),
    2: dict(name="llama3-8b-layer-B16-T8192", B=16, H=32, G=8, d=128, T0=8192,
            steps=128, dtype="bf16", W=8, R=[(4.0, 4.0), (2.0, 2.0)],
            structure="lowrank"),
    3: dict(name="long-context-B4-T131072", B=4, H=32, G=8, d=128, T0=131072,
            steps=8, dtype="bf16", W=8, R=[(4.0, 4.0), (2.0, 2.0)],
            structure="needles"),
    4: dict(name="large-batch-B64-T2k-32k-gqa7", B=64, H=28, G=4, d=128,
            T0=(2048, 32768), steps=16, dtype="bf16", W=8,
            R=[(6.0, 6.0), (4.0, 4.0), (2.0, 2.0)], structure="lowrank"),
    5: dict(name="encode-decode-B32-T16384", B=32, H=32, G=8, d=128, T0=16384,
            steps=256, dtype="bf16", W=8,
            R=[(3.0, 3.0), (3.5, 2.5), (3.3, 2.7)], structure="lowrank"),
}


def workload(wid: int, **overrides) -> dict:
    """Return a copy of workload ``wid`` with optional field overrides
    (e.g. smaller B/T0 for parity tests that keep the same distributions)."""
    cfg = dict(WORKLOADS[wid])
    cfg["id"] = wid
    cfg.update(overrides)
    return cfg


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [int(k) for k in key])))


def round_to_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Cast to float32 (round-to-nearest-even), then to bfloat16
    (round-to-nearest-even on the upper 16 bits); returned as float64."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def cast(cfg: dict, x: np.ndarray) -> np.ndarray:
    return round_to_bf16(x) if cfg["dtype"] == "bf16" else round_to_f32(x)


def to_device_bits(cfg: dict, x: np.ndarray) -> np.ndarray:
    """Exact dtype values (float64) -> raw element array for upload:
    uint16 bf16 bit patterns or float32."""
    f = np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)
    if cfg["dtype"] == "bf16":
        return (f.view(np.uint32) >> 16).astype(np.uint16)
    return f


def context_lengths(cfg: dict) -> np.ndarray:
    """Prefill length T0 per request (ragged for workload 4)."""
    T0 = cfg["T0"]
    if isinstance(T0, tuple):
        r = _rng(cfg["id"], _S_LEN, 0, 0, 0)
        return r.integers(T0[0], T0[1] + 1, size=cfg["B"]).astype(np.int64)
    return np.full(cfg["B"], int(T0), dtype=np.int64)


def total_tokens(cfg: dict) -> np.ndarray:
    return context_lengths(cfg) + int(cfg["steps"])


def codec_signs(cfg: dict):
    """The sign vectors of the key and the value Hadamard-sign transforms:
    two int8 arrays [d] of +-1."""
    r = _rng(cfg["id"], _S_SIGN, 0, 0, 0)
    s = r.integers(0, 2, size=(2, cfg["d"]))
    s = (1 - 2 * s).astype(np.int8)
    return s[0].copy(), s[1].copy()


def _sigma(cfg, stream, g):
    r = _rng(cfg["id"], _S_SIGMA, stream, g, 0)
    return np.exp(r.uniform(np.log(0.1), np.log(10.0), size=cfg["d"]))


def _q_base(cfg, b):
    r = _rng(cfg["id"], _S_QBASE, b, 0, 0)
    return r.standard_t(3.0, size=(cfg["H"], cfg["d"]))


def kv_unit(cfg: dict, b: int, g: int, n_tokens: int | None = None):
    """Keys and values of one (request b, KV head g) stream, tokens
    [0, n_tokens) in append order; float64 arrays [n][d] holding values that
    are exact in the workload's dtype."""
    d = cfg["d"]
    n_all = int(total_tokens(cfg)[b])
    n = n_all if n_tokens is None else int(n_tokens)
    assert n <= n_all
    out = []
    for stream in (_S_K, _S_V):
        sig = _sigma(cfg, stream, g)
        r = _rng(cfg["id"], stream, b, g, 0)
        z = r.standard_normal((n_all, d))
        x = z * sig[None, :]
        if cfg["structure"] in ("lowrank", "needles"):
            ra = _rng(cfg["id"], _S_A, stream, g, 0)
            A = ra.normal(0.0, np.sqrt(1.0 / 8.0), size=(d, 8))
            u = r.standard_normal((n_all, 8))
            x = x + u @ A.T
        if cfg["structure"] == "needles" and stream == _S_K:
            x = _plant_needles(cfg, b, g, x)
        if stream == _S_K and cfg.get("gap"):
            Q, D, period = cfg["gap"]
            phase = int(_rng(cfg["id"], _S_GAP, b, g, 1).integers(0, period))
            x = x.copy()
            x[phase::period] += D * _gap_dir(cfg, b, g)[None, :]
        if stream == _S_K and cfg.get("key_ties"):
            x = x.copy()
            x[:, 1::2] = x[:, 0::2]
        out.append(cast(cfg, x[:n]))
    return out[0], out[1]


def calibration_split(cfg: dict, g: int, n: int):
    """n held-out keys and values of KV head g ([n][d] float64, exact in the
    workload's dtype): the cache's per-channel scales and shared low-rank
    part, with token draws of their own (no needles, ties or gaps)."""
    d = cfg["d"]
    out = []
    for stream in (_S_K, _S_V):
        sig = _sigma(cfg, stream, g)
        r = _rng(cfg["id"], _S_CAL, stream, g, 0)
        x = r.standard_normal((n, d)) * sig[None, :]
        if cfg["structure"] in ("lowrank", "needles"):
            ra = _rng(cfg["id"], _S_A, stream, g, 0)
            A = ra.normal(0.0, np.sqrt(1.0 / 8.0), size=(d, 8))
            x = x + r.standard_normal((n, 8)) @ A.T
        out.append(cast(cfg, x))
    return out[0], out[1]


def _gap_dir(cfg, b, g):
    u = _rng(cfg["id"], _S_GAP, b, g, 0).standard_normal(cfg["d"])
    return u / np.linalg.norm(u)


def needle_positions(cfg: dict, b: int, g: int) -> np.ndarray:
    """64 needle positions per (b, g) among the prefill tokens; needle i is
    aligned with query head g*gqa + (i % gqa)."""
    r = _rng(cfg["id"], _S_NEEDLE, b, g, 0)
    T0 = int(context_lengths(cfg)[b])
    return np.sort(r.choice(T0, size=64, replace=False))


def _plant_needles(cfg, b, g, x):
    gqa = cfg["H"] // cfg["G"]
    qb = _q_base(cfg, b)
    r = _rng(cfg["id"], _S_NEEDLE, b, g, 1)
    pos = needle_positions(cfg, b, g)
    x = x.copy()
    for i, j in enumerate(pos):
        h = g * gqa + (i % gqa)
        qh = qb[h] / np.linalg.norm(qb[h])
        xi = r.standard_normal(cfg["d"])
        xi -= (xi @ qh) * qh
        xi /= np.linalg.norm(xi)
        x[j] = np.linalg.norm(x[j]) * (0.9 * qh + np.sqrt(0.19) * xi)
    return x


def q_step(cfg: dict, b: int, step: int) -> np.ndarray:
    """Query of request b at decode step ``step``: float64 [H][d], exact in
    the workload's dtype."""
    r = _rng(cfg["id"], _S_Q, b, 0, step)
    shape = (cfg["H"], cfg["d"])
    if cfg["structure"] == "iid":
        q = r.standard_normal(shape)
    elif cfg["structure"] == "needles":
        q = _q_base(cfg, b) + 0.1 * r.standard_normal(shape)
    else:
        q = r.standard_t(3.0, size=shape)
    if cfg.get("gap"):
        Q = cfg["gap"][0]
        gqa = cfg["H"] // cfg["G"]
        u = np.stack([_gap_dir(cfg, b, h // gqa) for h in range(cfg["H"])])
        q = Q * u + r.standard_normal(shape)
    if cfg.get("q_scale"):
        q = q * float(cfg["q_scale"])
    if cfg.get("key_ties"):
        q = q.copy()
        q[:, 1::2] = q[:, 0::2]
    spread = cfg.get("q_log2_spread", 0)
    if spread:
        # channel c scaled by an exact power of two from 2^-spread up to 1:
        # key weights then span about 2 * spread binary orders of magnitude
        q = q * np.exp2(np.round(np.linspace(-float(spread), 0.0, shape[1])))
    return cast(cfg, q)


def new_token(cfg: dict, b: int, g: int, step: int):
    """The key/value appended to unit (b, g) at decode step ``step``."""
    T0 = int(context_lengths(cfg)[b])
    K, V = kv_unit(cfg, b, g, T0 + step + 1)
    return K[T0 + step], V[T0 + step]
