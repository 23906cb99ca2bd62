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
                 keep_steps=None, qmod=None):
        cfg = dict(cfg, codec="lloyd")
        self.cfg, self.steps, self.rates, self.vscale, self.policy = cfg, steps, rates, vscale, policy
        self.min1 = 1 if policy & RESTRICT_MIN_DEPTH1 else 0
        self.pairs = bool(policy & RESTRICT_VALUE_PAIRS)
        self.scope = "layer" if policy & SCOPE_LAYER else "kv_head"
        B, H, G = cfg["B"], cfg["H"], cfg["G"]
        self.T0 = synth.context_lengths(cfg)
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
        cache.append(dv["kpre"], dv["vpre"], n_new=dv["npre"].to(torch.int32),
                     n_max=dv["kpre"].shape[2])
        self.rec = []
        keep = set(range(steps)) if keep_steps is None else set(keep_steps)
        for s in range(steps):
            cache.append(dv["kstep"][s], dv["vstep"][s])
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
