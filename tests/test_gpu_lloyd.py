"""GPU parity of the pages' own code (Lloyd tree, Hadamard-sign transforms,
calibration): the HIP library through its C ABI against oracle/lloyd.py on
the same seeded inputs.

* calibration arrays, signs and tables in the store's codec block equal the
  oracle's, byte for byte;
* the device encoder's key and value planes and open-group buffers equal the
  oracle's encoding packed by the format description (bit-exact);
* key depths equal the oracle's, value depths equal up to near ties
  (parity_util; exact-tie swaps fail), outputs within 2e-3 relative L2 per
  (request, query head), read counters equal the schedules' accounting.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import lloyd as L
from oracle import store_format as F
from query_adaptive_decode_amd import binding, synth, workload
from query_adaptive_decode_amd.binding import (NUM_COUNTERS, RESTRICT_MIN_DEPTH1,
                                               RESTRICT_VALUE_PAIRS, SCOPE_KV_HEAD, SCOPE_LAYER,
                                               ReadKVCache, VSCALE_PHYSICAL, VSCALE_UNIT)
from tests import parity_util as PU
from tests.parity_util import OUT_REL_L2, alloc_mismatch, rel_l2

pytestmark = pytest.mark.gpu

NCAL = 512
TREE = L.lloyd_tree()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    binding.lib()   # raises if the library was not built


def oracle_codec(cfg):
    sk, sv = synth.codec_signs(cfg)
    cal = [synth.calibration_split(cfg, g, NCAL) for g in range(cfg["G"])]
    return L.make_codec(TREE, sk, sv, [k for k, _ in cal], [v for _, v in cal])


class LloydRun:
    """Calibrate, prefill, then `steps` rounds of (append one token, decode
    at every rate) on the GPU; the decodes are kept on the host."""

    def __init__(self, cfg, steps, rates=(), vscale=VSCALE_PHYSICAL, policy=SCOPE_KV_HEAD,
                 keep_steps=None, qmod=None, empty=()):
        # empty: requests that are given no token at all (prefill or steps)
        cfg = dict(cfg, codec="lloyd")
        self.empty = set(empty)
        self.cfg, self.steps, self.rates, self.vscale, self.policy = cfg, steps, rates, vscale, policy
        self.min1 = 1 if policy & RESTRICT_MIN_DEPTH1 else 0
        self.pairs = bool(policy & RESTRICT_VALUE_PAIRS)
        self.scope = "layer" if policy & SCOPE_LAYER else "kv_head"
        B, H, G = cfg["B"], cfg["H"], cfg["G"]
        self.T0 = synth.context_lengths(cfg)
        for b in self.empty:
            self.T0[b] = 0
        say(f"[case] lloyd {cfg['name']} B={B} H={H} G={G} W={cfg['W']} T0={self.T0.tolist()[:4]} "
            f"steps={steps} rates={list(rates)} vscale={vscale} policy={policy}")
        h = workload.host_inputs(cfg, steps)
        self.qf = {}
        for s in range(steps):
            qf = np.stack([synth.q_step(cfg, b, s) for b in range(B)])
            if qmod is not None:
                qf = qmod(qf, s)
                h["q"][s] = synth.to_device_bits(cfg, qf)
            self.qf[s] = qf
        dv = workload.to_device(h)
        del h
        ci = workload.calibration_inputs(cfg, NCAL)
        cd = workload.to_device(dict(kcal=ci["kcal"], vcal=ci["vcal"]))
        self.lcfg = workload.config_for(cfg, steps)
        cap = self.lcfg.capacity_tokens
        self.cache = cache = ReadKVCache(self.lcfg)
        binding.codec_init(self.lcfg, cache.store, ci["sk"].tolist(), ci["sv"].tolist(),
                           cd["kcal"], cd["vcal"])
        live = torch.tensor([0 if b in self.empty else 1 for b in range(B)], dtype=torch.int32,
                            device="cuda")
        cache.append(dv["kpre"], dv["vpre"], n_new=dv["npre"].to(torch.int32) * live,
                     n_max=dv["kpre"].shape[2])
        self.rec = []
        keep = set(range(steps)) if keep_steps is None else set(keep_steps)
        for s in range(steps):
            cache.append(dv["kstep"][s], dv["vstep"][s], n_new=live if self.empty else None)
            if s not in keep:
                continue
            for (rk, rv) in rates:
                tk = torch.zeros(B * G * 128, dtype=torch.uint8, device="cuda")
                tv = torch.zeros(B * G * ((cap + 31) // 32 * 32), dtype=torch.uint8, device="cuda")
                ctr = torch.full((NUM_COUNTERS,), -1, dtype=torch.int64, device="cuda")
                out = cache.decode(dv["q"][s], rk, rv, vscale=vscale, key_depths=tk,
                                   value_depths=tv, counters=ctr, policy=policy)
                self.rec.append(dict(step=s, rk=rk, rv=rv, out=out.cpu().numpy(),
                                     tk=tk.cpu().numpy().reshape(B, G, 128),
                                     tv=tv.cpu().numpy().reshape(B, G, -1), ctr=ctr.cpu().numpy()))
        torch.cuda.synchronize()
        self.store = cache.store.cpu().numpy()
        self.flags, self.lens = cache.status()
        say(f"[gpu done] flags={self.flags} lens={self.lens[:4]}")
        self.codec = oracle_codec(cfg)
        self._units, self._enc = {}, {}

    def n_of(self, b, step):
        """Tokens of request b at the decode of `step`."""
        return 0 if b in self.empty else int(self.T0[b]) + step + 1

    def unit(self, b, g):
        if (b, g) not in self._units:
            self._units[(b, g)] = synth.kv_unit(self.cfg, b, g, int(self.T0[b]) + self.steps)
        return self._units[(b, g)]

    def enc(self, b, g, n):
        key = (b, g, n)
        if key not in self._enc:
            K, V = self.unit(b, g)
            c, W = self.codec, self.cfg["W"]
            self._enc = {k: v for k, v in self._enc.items() if k[:2] != (b, g)}
            self._enc[key] = (L.lloyd_encode_stream(K[:n], TREE, c.sK, c.muK[g], c.sigK[g], W),
                              L.lloyd_encode_stream(V[:n], TREE, c.sV, c.muV[g], c.sigV[g], W))
        return self._enc[key]

    def check_store(self, units=None):
        cfg = self.cfg
        hdr = F.read_header(self.store)
        assert hdr["codec"] == 1
        hb = F.header_bytes(cfg["B"])
        want = F.codec_block(self.codec, cfg["G"], cfg["d"])
        got = self.store[hb:hb + want.size]
        assert np.array_equal(got, want), "codec block differs"
        units = units or [(b, g) for b in range(cfg["B"]) for g in range(cfg["G"])]
        for (b, g) in units:
            n = int(self.T0[b]) + self.steps
            sk, sv = self.enc(b, g, n)
            exp = F.pack_unit(sk, sv, hdr["requests"][b]["cap"], cfg["dtype"])
            dev = F.unpack_unit(self.store, hdr, b, g)
            for k in ("Kplanes", "Vplanes", "Kmeta", "Vmeta", "EK", "EV"):
                assert np.array_equal(dev[k], exp[k]), f"{k} differs in unit ({b},{g})"
            r = n % 32   # tail slots past the open group's tokens are not defined
            for k in ("Ktail", "Vtail"):
                assert np.array_equal(dev[k][:r], exp[k][:r]), f"{k} differs in unit ({b},{g})"


def test_lloyd_codec_block_and_encoder_bf16():
    cfg = synth.workload(2, B=2, T0=1000)
    r = LloydRun(cfg, steps=40)
    r.check_store()


def test_lloyd_encoder_gqa7_w6_ragged():
    cfg = synth.workload(4, B=3, T0=(40, 700), W=6)
    r = LloydRun(cfg, steps=9)
    r.check_store()


def test_lloyd_encoder_nonfinite_group_sets_flag():
    cfg = dict(synth.workload(1, T0=70), codec="lloyd")
    # a NaN in the prefill's second group of keys: that group is coded 0
    orig = synth.kv_unit

    def patched(c, b, g, n_tokens=None):
        K, V = orig(c, b, g, n_tokens)
        K = K.copy()
        if K.shape[0] > 40:
            K[40, 7] = np.nan
        return K, V
    synth.kv_unit = patched
    try:
        r = LloydRun(cfg, steps=3)
        assert r.flags & 1
        r.check_store()
    finally:
        synth.kv_unit = orig


def _check_decode(r, record_property, name, units=None, bound=None):
    """Every kept decode of the run against the oracle (per-KV-head or
    per-layer budgets), near ties counted and bounded."""
    cfg = r.cfg
    G, H, W = cfg["G"], cfg["H"], cfg["W"]
    gqa = H // G
    ebits = 16 if cfg["dtype"] == "bf16" else 32
    vs = "unit" if r.vscale == VSCALE_UNIT else "physical"
    st = dict(near=0, checks=0, worst=0.0)
    reqs = sorted({b for b, _ in units}) if units else list(range(cfg["B"]))
    for it in r.rec:
        tag0 = f"step={it['step']} R=({it['rk']},{it['rv']}) {r.scope}"
        # read counters: payloads and open group from the GPU's own schedules,
        # metadata one load of the calibration arrays and the table per call
        tot = [0, 0, 0, 0]
        for b in range(cfg["B"]):
            n = r.n_of(b, it["step"])
            tp = n // 32 * 32
            for g in range(G):
                tot[0] += tp * int(it["tk"][b, g].sum())
                tot[1] += 128 * int(it["tv"][b, g, :tp].sum())
                tot[3] += 2 * (n - tp) * 128 * ebits
        tot[2] = L.lloyd_metadata_bits(G)
        assert it["ctr"].tolist() == tot, f"read counters {tag0}"
        for b in reqs:
            n = r.n_of(b, it["step"])
            gs = [g for (bb, g) in units if bb == b] if units else list(range(G))
            streams = [r.enc(b, g, n) for g in range(G)]
            res = L.lloyd_decode_request(r.qf[it["step"]][b], streams, r.codec, W=W, R_K=it["rk"],
                                         R_V=it["rv"], vscale=vs, scope=r.scope,
                                         min_depth=r.min1, value_pairs=r.pairs)
            tag = f"{tag0} request={b} n={n}"
            tp = res["tp"]
            if r.scope == "layer":
                assert np.array_equal(it["tk"][b], res["tK"]), f"key depths differ {tag}"
                tvg, tvo = it["tv"][b, :, :tp].reshape(-1), res["tV"].reshape(-1)
                if r.pairs:
                    assert np.array_equal(tvg[0::2], tvg[1::2]), f"packet depths {tag}"
                    tvg, tvo = tvg[0::2], tvo[0::2]
                near, bad, det = alloc_mismatch(tvg, tvo, res["wv"], W, start=r.min1,
                                                gains=TREE.gains32)
                assert bad == 0, f"value depths differ {tag}: {det}"
                st["near"] += near
                st["checks"] += 1
            else:
                nv = tp // 2 if r.pairs else tp
                for g in gs:
                    assert np.array_equal(it["tk"][b, g], res["tK"][g]), f"key depths differ {tag} g={g}"
                    tvg, tvo = it["tv"][b, g, :tp], res["tV"][g]
                    if r.pairs:
                        assert np.array_equal(tvg[0::2], tvg[1::2]), f"packet depths {tag} g={g}"
                        tvg, tvo = tvg[0::2], tvo[0::2]
                    near, bad, det = alloc_mismatch(tvg, tvo, res["wv"][g * nv:(g + 1) * nv], W,
                                                    start=r.min1, gains=TREE.gains32)
                    assert bad == 0, f"value depths differ {tag} g={g}: {det}"
                    st["near"] += near
                    st["checks"] += 1
            for g in gs:
                got = it["out"][b, g * gqa:(g + 1) * gqa]
                want = res["out"][g]
                if np.isnan(want).all():
                    assert np.isnan(got).all(), f"outputs of a non-finite query {tag} g={g}"
                    continue
                err = rel_l2(got, want)
                st["worst"] = max(st["worst"], float(err.max()))
                assert np.all(err <= OUT_REL_L2), f"output rel L2 {err.max():.3e} {tag} g={g}"
    if bound is None:
        bound = 2 + st["checks"] // 50
    line = (f"lloyd {name}: {st['near']} near-tie refinements over {st['checks']} checks "
            f"(bound {bound}); worst output rel L2 {st['worst']:.2e}")
    PU.REPORT.append(line)
    record_property("near_ties", st["near"])
    record_property("worst_rel_l2", st["worst"])
    say("[report] " + line)
    assert st["near"] <= bound, line
    return st


def test_lloyd_decode_bf16_gqa4(record_property):
    cfg = synth.workload(2, B=2, T0=1000)
    r = LloydRun(cfg, steps=3, rates=[(4.0, 4.0), (2.0, 2.0), (8.0, 1.5), (0.5, 6.0)])
    _check_decode(r, record_property, "bf16 gqa4 B=2 T0=1000")


def test_lloyd_decode_fp32_tiny_unit_scale(record_property):
    cfg = synth.workload(1, T0=1024)
    r = LloydRun(cfg, steps=3, rates=[(4.0, 4.0), (1.0, 7.0)], vscale=VSCALE_UNIT)
    _check_decode(r, record_property, "fp32 tiny unit scale")


@pytest.mark.parametrize("T0", [5, 31, 32, 33, 511, 513, 2047])
def test_lloyd_decode_ragged_tails(T0, record_property):
    cfg = synth.workload(2, B=1, H=8, G=2, T0=T0)
    r = LloydRun(cfg, steps=2, rates=[(4.0, 4.0), (2.0, 2.0)])
    _check_decode(r, record_property, f"tails T0={T0}")


def test_lloyd_decode_layer_budgets(record_property):
    cfg = synth.workload(2, B=2, H=16, G=4, T0=700)
    r = LloydRun(cfg, steps=2, rates=[(4.0, 4.0), (2.0, 3.0)], policy=SCOPE_LAYER)
    _check_decode(r, record_property, "layer budgets")


def test_lloyd_decode_restricted_gqa7_ragged(record_property):
    cfg = synth.workload(4, B=3, T0=(300, 1500))
    pol = SCOPE_KV_HEAD | RESTRICT_MIN_DEPTH1 | RESTRICT_VALUE_PAIRS
    r = LloydRun(cfg, steps=2, rates=[(4.0, 4.0), (2.0, 2.0)], policy=pol)
    _check_decode(r, record_property, "restricted gqa7 ragged")


def test_lloyd_decode_exact_ties_partial_budgets(record_property):
    """R_K = 0: every key reads depth 0, so every packed token of a unit has
    the same logit and the value weights tie exactly; a partial value budget
    must go to the lowest token indices.  Key ties: duplicated key and query
    channels give bitwise-equal key weights in pairs."""
    cfg = synth.workload(2, B=1, H=8, G=2, T0=300)
    r = LloydRun(cfg, steps=1, rates=[(0.0, 1.3), (0.0, 2.7)])
    _check_decode(r, record_property, "exact value ties", bound=0)
    cfg = synth.workload(2, B=1, H=8, G=2, T0=300, key_ties=True)
    r = LloydRun(cfg, steps=1, rates=[(1.5, 2.0), (3.25, 2.0)])
    _check_decode(r, record_property, "key ties")


def test_lloyd_decode_nonfinite_query(record_property):
    def qmod(q, s):
        q = q.copy()
        q[0, 5, 17] = np.inf   # request 0, query head 5 (KV head 1)
        return q
    cfg = synth.workload(2, B=2, H=8, G=2, T0=400)
    r = LloydRun(cfg, steps=1, rates=[(4.0, 4.0)], qmod=qmod)
    _check_decode(r, record_property, "non-finite query")


def test_lloyd_decode_layer_budgets_many_block_selection(record_property):
    # 8 KV heads x 2,560 tokens per request: the value selection over many
    # blocks per request
    cfg = synth.workload(2, B=2, T0=2500)
    r = LloydRun(cfg, steps=1, rates=[(4.0, 4.0), (2.0, 1.0)], policy=SCOPE_LAYER)
    _check_decode(r, record_property, "layer budgets, many-block selection")


@pytest.mark.parametrize("H,G", [(4, 2), (10, 2), (16, 2)], ids=["gqa2", "gqa5", "gqa8"])
def test_lloyd_decode_other_head_ratios(H, G, record_property):
    cfg = synth.workload(2, B=2, H=H, G=G, T0=700)
    r = LloydRun(cfg, steps=1, rates=[(4.0, 4.0), (2.5, 1.5)])
    _check_decode(r, record_property, f"gqa{H // G}")


@pytest.mark.parametrize("policy", [SCOPE_KV_HEAD, SCOPE_LAYER], ids=["kv_head", "layer"])
def test_lloyd_decode_empty_request(policy, record_property):
    # request 2 holds no token: outputs exactly zero, key depths allocated as
    # for the others
    cfg = synth.workload(4, B=3, T0=(40, 900))
    r = LloydRun(cfg, steps=1, rates=[(4.0, 4.0), (2.0, 1.0)], policy=policy, empty=[2])
    _check_decode(r, record_property, f"empty request {r.scope}")


def test_lloyd_decode_full_shape_sampled(record_property):
    """The Llama-3-8B-shaped layer at full size (B=16, T0=8192) in the
    launch configuration of the benchmark, 4 units checked on one step at
    both rates."""
    cfg = synth.workload(2)
    r = LloydRun(cfg, steps=1, rates=[(4.0, 4.0), (2.0, 2.0)])
    _check_decode(r, record_property, "full shape sampled", units=[(0, 0), (5, 3), (11, 6), (15, 7)])


@pytest.mark.parametrize("wid,rates,units", [
    # long context, 131k tokens: the split value path (weights on all compute
    # units, then one selection block per unit reading them from memory)
    (3, [(4.0, 4.0), (2.0, 2.0)], [(0, 0), (3, 7)]),
    # large batch, GQA 7, ragged 2k..32k prompts
    (4, [(6.0, 6.0), (2.0, 2.0)], [(0, 0), (17, 2), (63, 3)]),
    # encode + decode mix at its own shape and rates
    (5, [(3.0, 3.0), (3.5, 2.5)], [(0, 0), (31, 7)]),
])
def test_lloyd_decode_other_workloads_sampled(wid, rates, units, record_property):
    cfg = synth.workload(wid)
    r = LloydRun(cfg, steps=1, rates=rates)
    _check_decode(r, record_property, f"workload {wid} sampled", units=units)
