"""readkv_decode_attn_noalloc (the entry point for callers that cannot
allocate) against readkv_decode_attn with a caller workspace, through the C
ABI: two cases in a row, the second with a smaller input (fewer requests,
shorter contexts, another head geometry), so that the second call runs on
scratch still holding the first call's contents.  Depth schedules and read
counters must be equal, outputs bitwise equal (the same kernels on the same
inputs); the call must leave the device's free memory unchanged."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from query_adaptive_decode_amd import binding as Bd
from query_adaptive_decode_amd import synth, workload

pytestmark = pytest.mark.gpu


def _free_bytes():
    h = ctypes.CDLL("libamdhip64.so")
    free, total = ctypes.c_size_t(), ctypes.c_size_t()
    assert h.hipMemGetInfo(ctypes.byref(free), ctypes.byref(total)) == 0
    return free.value


def _prepared(cfg):
    h = workload.host_inputs(cfg, 1)
    dv = workload.to_device(h)
    lcfg = workload.config_for(cfg, 1)
    cache = Bd.ReadKVCache(lcfg)
    if cfg.get("codec") == "lloyd":
        ci = workload.calibration_inputs(cfg, 128)
        cd = workload.to_device(dict(kcal=ci["kcal"], vcal=ci["vcal"]))
        Bd.codec_init(lcfg, cache.store, ci["sk"].tolist(), ci["sv"].tolist(), cd["kcal"], cd["vcal"])
    cache.append(dv["kpre"], dv["vpre"], n_new=dv["npre"].to(torch.int32),
                 n_max=dv["kpre"].shape[2])
    cache.append(dv["kstep"][0], dv["vstep"][0])
    return lcfg, cache, dv["q"][0]


@pytest.mark.parametrize("codec", ["uniform", "lloyd"])
def test_noalloc_matches_workspace_entry_point_on_two_calls(codec):
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    cases = [synth.workload(2, B=4, T0=6000, codec=codec),                # larger input first
             synth.workload(4, B=2, T0=(100, 900), codec=codec)]          # then a smaller one
    for ci, cfg in enumerate(cases):
        print(f"[case] noalloc {cfg['name']} B={cfg['B']} T0={synth.context_lengths(cfg).tolist()}",
              flush=True)
        lcfg, cache, q = _prepared(cfg)
        assert Bd.workspace_bytes(lcfg) <= Bd.NOALLOC_SCRATCH_BYTES
        B, H, G = cfg["B"], cfg["H"], cfg["G"]
        cap = (lcfg.capacity_tokens + 31) // 32 * 32
        lens = synth.context_lengths(cfg) + 1
        for (rk, rv) in [(4.0, 4.0), (3.3, 2.7)]:
            bufs = []
            for _ in range(2):
                bufs.append(dict(
                    out=torch.full((B, H, 128), float("nan"), dtype=torch.float32, device="cuda"),
                    tk=torch.zeros(B * G * 128, dtype=torch.uint8, device="cuda"),
                    tv=torch.zeros(B * G * cap, dtype=torch.uint8, device="cuda"),
                    ctr=torch.zeros(Bd.NUM_COUNTERS, dtype=torch.int64, device="cuda")))
            ref, got = bufs
            cache.decode(q, rk, rv, out=ref["out"], key_depths=ref["tk"], value_depths=ref["tv"],
                         counters=ref["ctr"])
            torch.cuda.synchronize()
            free0 = _free_bytes()
            Bd.decode_attn_noalloc(lcfg, cache.store, q, rk, rv, got["out"], key_depths=got["tk"],
                                   value_depths=got["tv"], counters=got["ctr"])
            torch.cuda.synchronize()
            free1 = _free_bytes()
            if ci > 0:
                assert free1 == free0, (free0, free1)
            assert torch.equal(ref["tk"], got["tk"])
            tv_r = ref["tv"].view(B, G, cap).cpu().numpy()
            tv_g = got["tv"].view(B, G, cap).cpu().numpy()
            for b in range(B):
                tp = int(lens[b]) // 32 * 32
                assert np.array_equal(tv_r[b, :, :tp], tv_g[b, :, :tp]), (ci, rk, rv, b)
            assert torch.equal(ref["ctr"], got["ctr"])
            assert torch.equal(ref["out"], got["out"]), (ci, rk, rv)
            print(f"[ok] case {ci} R=({rk},{rv}) free bytes {free0} -> {free1}", flush=True)
            sys.stdout.flush()
