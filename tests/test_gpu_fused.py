"""GPU: the single-launch reader (policy flag SINGLE_LAUNCH: the whole decode
step as one cooperative launch with grid-wide barriers between its stages)
against the float64 oracle, and against the split launches on the same cache.

* against the oracle: the parity rules of the split path (key depths equal,
  value depths up to counted near ties, outputs within 2e-3 relative L2,
  read counters equal to the oracle's accounting);
* against the split launches: key and value depths and read counters
  bitwise equal (the same selection code on the same weights); outputs
  within 1e-5 relative L2 (only the split of each unit's chunks into gather
  runs, and so the order of their partial sums, differs);
* unsupported requests (more units than blocks that fit at once) fail with
  READKV_EUNSUPPORTED and launch nothing.
"""
import numpy as np
import pytest
import torch

from query_adaptive_decode_amd import synth, workload
from query_adaptive_decode_amd.binding import (NUM_COUNTERS, RESTRICT_MIN_DEPTH1,
                                               RESTRICT_VALUE_PAIRS, SCOPE_KV_HEAD, SINGLE_LAUNCH,
                                               ReadKVCache, ReadKVError, VSCALE_UNIT)
from tests.parity_util import rel_l2
from tests.test_gpu_parity import Run, report, say

pytestmark = pytest.mark.gpu

SPLIT_REL_L2 = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from query_adaptive_decode_amd import binding
    binding.lib()


# ------------------------------------------------------------ against the oracle
def test_fused_tiny_fp32(record_property):
    # fp32 keys, values and query; one query head on one KV head
    cfg = synth.workload(1)
    run = Run(cfg, steps=8, rates=[(4.0, 4.0), (2.0, 2.0), (8.0, 1.0)], scope=SINGLE_LAUNCH,
              repeat=True)
    report(record_property, "single launch tiny fp32", run.check())


def test_fused_llama_shape_small_context(record_property):
    cfg = synth.workload(2, B=2, T0=2000)
    run = Run(cfg, steps=2, rates=[(4.0, 4.0), (2.0, 2.0), (3.3, 2.7)], scope=SINGLE_LAUNCH,
              repeat=True)
    report(record_property, "single launch llama shape T0=2000", run.check())


def test_fused_gqa7_ragged_batch(record_property):
    cfg = synth.workload(4, B=3, T0=(40, 1500))
    run = Run(cfg, steps=2, rates=[(6.0, 6.0), (2.0, 2.0), (3.5, 2.5)], scope=SINGLE_LAUNCH)
    report(record_property, "single launch gqa7 ragged", run.check())


@pytest.mark.parametrize("T0", [5, 33, 1025])
def test_fused_ragged_tails(T0, record_property):
    cfg = synth.workload(2, B=1, H=8, G=2, T0=T0)
    run = Run(cfg, steps=2, rates=[(4.0, 4.0), (0.0, 0.0), (8.0, 8.0)], scope=SINGLE_LAUNCH)
    report(record_property, f"single launch tails T0={T0}", run.check())


@pytest.mark.parametrize("H,G", [(4, 2), (6, 2), (10, 2), (12, 2), (16, 2)],
                         ids=["gqa2", "gqa3", "gqa5", "gqa6", "gqa8"])
def test_fused_other_head_ratios(H, G, record_property):
    # the other query-per-KV-head ratios (two blocks per compute unit above 4)
    cfg = synth.workload(2, B=2, H=H, G=G, T0=700)
    run = Run(cfg, steps=1, rates=[(4.0, 4.0), (2.5, 1.5)], scope=SINGLE_LAUNCH)
    report(record_property, f"single launch gqa{H // G}", run.check())


def test_fused_fewer_planes(record_property):
    cfg = synth.workload(2, B=2, H=8, G=2, T0=900, W=5)
    run = Run(cfg, steps=1, rates=[(2.5, 2.5), (5.0, 5.0), (6.0, 1.0)], scope=SINGLE_LAUNCH)
    report(record_property, "single launch W=5", run.check())


def test_fused_empty_request(record_property):
    # request 0 holds no token: zero outputs, minimum key depths
    cfg = synth.workload(2, B=3, H=8, G=2, T0=600)
    run = Run(cfg, steps=1, rates=[(4.0, 4.0), (2.0, 3.0)], scope=SINGLE_LAUNCH, empty=[0])
    report(record_property, "single launch, empty request", run.check())


def test_fused_restricted_reader_unit_scale(record_property):
    cfg = synth.workload(2, B=2, T0=1500)
    flags = SINGLE_LAUNCH | RESTRICT_MIN_DEPTH1 | RESTRICT_VALUE_PAIRS
    run = Run(cfg, steps=1, rates=[(4.0, 4.0), (1.0, 1.0), (3.3, 2.7)], scope=flags)
    st = run.check()
    cfg = synth.workload(3, B=1, H=8, G=2, T0=3000)
    run = Run(cfg, steps=1, rates=[(4.0, 4.0), (2.0, 2.0)], vscale=VSCALE_UNIT, scope=SINGLE_LAUNCH)
    st2 = run.check()
    report(record_property, "single launch restricted + unit scale",
           dict(near=st["near"] + st2["near"], checks=st["checks"] + st2["checks"],
                worst=max(st["worst"], st2["worst"])))


def test_fused_exact_ties(record_property):
    # R_K = 0: the 32 tokens of a closed group have equal logits and value
    # weights; duplicated key channels: key weights in bitwise-equal pairs
    cfg = synth.workload(2, B=2, T0=2000)
    run = Run(cfg, steps=1, rates=[(0.0, 1.3), (0.0, 2.7)], scope=SINGLE_LAUNCH)
    st = run.check()
    cfg = synth.workload(2, B=2, T0=700, key_ties=True)
    run = Run(cfg, steps=1, rates=[(2.5078125, 4.0), (1.0078125, 1.0)], scope=SINGLE_LAUNCH)
    st2 = run.check()
    report(record_property, "single launch exact ties",
           dict(near=st["near"] + st2["near"], checks=st["checks"] + st2["checks"],
                worst=max(st["worst"], st2["worst"])))


# ------------------------------------------------------------ against the split launches
def _both_ways(cfg, steps, rates, policy=SCOPE_KV_HEAD):
    """One cache; every decode run split and single-launch.  Returns the
    largest output difference (rel L2)."""
    B, G = cfg["B"], cfg["G"]
    say(f"[case] split vs single launch {cfg['name']} B={B} H={cfg['H']} G={G} steps={steps} "
        f"rates={rates} policy={policy:#x}")
    h = workload.host_inputs(cfg, steps)
    dv = workload.to_device(h)
    del h
    lcfg = workload.config_for(cfg, steps)
    cap = lcfg.capacity_tokens
    cache = ReadKVCache(lcfg)
    cache.append(dv["kpre"], dv["vpre"], n_new=dv["npre"].to(torch.int32), n_max=dv["kpre"].shape[2])
    worst = 0.0
    for s in range(steps):
        cache.append(dv["kstep"][s], dv["vstep"][s])
        for (rk, rv) in rates:
            res = []
            for pol in (policy, policy | SINGLE_LAUNCH):
                tk = torch.zeros(B * G * 128, dtype=torch.uint8, device="cuda")
                tv = torch.zeros(B * G * ((cap + 31) // 32 * 32), dtype=torch.uint8, device="cuda")
                ctr = torch.full((NUM_COUNTERS,), -1, dtype=torch.int64, device="cuda")
                out = cache.decode(dv["q"][s], rk, rv, key_depths=tk, value_depths=tv, counters=ctr,
                                   policy=pol)
                res.append((out.cpu().numpy(), tk.cpu().numpy(), tv.cpu().numpy(),
                            ctr.cpu().numpy()))
            (o0, k0, v0, c0), (o1, k1, v1, c1) = res
            tag = f"step={s} R=({rk},{rv})"
            assert np.array_equal(k0, k1), f"key depths differ {tag}"
            assert np.array_equal(v0, v1), f"value depths differ {tag}"
            assert np.array_equal(c0, c1), f"read counters differ {tag}"
            err = rel_l2(o1, o0)
            worst = max(worst, float(err.max()))
            assert np.all(err <= SPLIT_REL_L2), f"outputs differ {err.max():.3e} {tag}"
    torch.cuda.synchronize()
    say(f"[split vs single launch] {cfg['name']}: worst rel L2 {worst:.2e}")
    return worst


@pytest.mark.timeout(600)
def test_fused_equals_split_full_size_llama_layer(record_property):
    # the benchmark's configuration (B=16, 32/8 heads, T0=8192)
    cfg = synth.workload(2)
    w = _both_ways(cfg, steps=1, rates=[(4.0, 4.0), (2.0, 2.0), (3.3, 2.7)])
    record_property("worst_rel_l2_vs_split", w)


@pytest.mark.timeout(600)
def test_fused_equals_split_gqa7_and_restricted(record_property):
    cfg = synth.workload(4, B=12, T0=(2000, 9000))
    w = _both_ways(cfg, steps=1, rates=[(6.0, 6.0), (2.0, 2.0)])
    cfg = synth.workload(2, B=4, T0=3000)
    w2 = _both_ways(cfg, steps=2, rates=[(4.0, 4.0), (1.0, 1.0)],
                    policy=RESTRICT_MIN_DEPTH1 | RESTRICT_VALUE_PAIRS)
    record_property("worst_rel_l2_vs_split", max(w, w2))


@pytest.mark.timeout(900)
def test_fused_equals_split_large_batch_and_long_prompt_full_shapes(record_property):
    # B=64, 28 query / 4 KV heads, ragged 2k-32k prompts (256 units, two
    # blocks per unit at GQA 7); B=32 with 16,384-token prompts (256 units)
    w = _both_ways(synth.workload(4), steps=1, rates=[(6.0, 6.0), (2.0, 2.0)])
    w2 = _both_ways(synth.workload(5), steps=1, rates=[(3.3, 2.7)])
    record_property("worst_rel_l2_vs_split", max(w, w2))


def test_fused_rejects_more_units_than_blocks():
    # 260 requests x 8 KV heads: 2080 units, more than the blocks of 256
    # threads that fit on the chip at once (at most 8 per compute unit); the
    # split launches take it
    cfg = synth.workload(2, B=260, H=8, G=8, T0=40)
    say("[case] single launch, 2080 units")
    h = workload.host_inputs(cfg, 1)
    dv = workload.to_device(h)
    cache = ReadKVCache(workload.config_for(cfg, 1))
    cache.append(dv["kpre"], dv["vpre"], n_new=dv["npre"].to(torch.int32), n_max=dv["kpre"].shape[2])
    cache.append(dv["kstep"][0], dv["vstep"][0])
    out = cache.decode(dv["q"][0], 4.0, 4.0)
    torch.cuda.synchronize()
    assert np.isfinite(out.cpu().numpy()).all()
    with pytest.raises(ReadKVError) as e:
        cache.decode(dv["q"][0], 4.0, 4.0, policy=SINGLE_LAUNCH)
    assert e.value.code == -5
