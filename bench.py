#!/usr/bin/env python3
"""ReadKV decode-step benchmark on one MI355X.

Workload: the Llama-3-8B-shaped attention layer (32 query / 8 KV heads,
head_dim 128, batch 16, 8192-token prompt, W = 8 stored bits), synthetic
seeded K/V/q.  One step = append one token per request through the encoder
+ one ReadKV decode (key allocation, score, value allocation, value gather,
output reduction), for read rates R = 4 and R = 2 (R_K = R_V = R).

Prints one JSON line.  `value` is query-heads x context-tokens per second at
(W, R) = (8, 4) with the step's inputs resident in HBM and the caches
flushed before every step (reading a 512 MiB buffer pushes the store out of
L2 and the Infinity Cache and leaves only clean lines behind); the warm
figure (steps replayed back to back)
sits beside it.  Both are graph replays timed with HIP events.  Also
reported: per-kernel HIP-event durations (warm and flushed), the roofline
of the dominant kernel, bytes moved per step from the committed rocprofv3
request counters (when they were taken on these sources), a measured
device-copy bandwidth, and the float64 oracle's CPU throughput on this
host (all cores, and one core).

The same step over the pages' own code (Gaussian Lloyd tree with
Hadamard-sign transforms, calibrated on a held-out synthetic split) is
timed the same way at `--lloyd-rates` and reported under "lloyd_codec".
The single-launch reader (one cooperative launch per decode) is timed as
eager steps beside the split launches at `--single-launch-rates`
("single_launch").

`--counters-run` runs the fixed sequence the counter profiles are taken on
(see query_adaptive_decode_amd/profile_summary.py) and prints nothing else
(`--lloyd` there: the same sequence over the Lloyd code).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
KERNELS = ["score", "value_alloc", "value_gather"]
METRIC = "decode attn query-heads·ctx-tokens/s + achieved HBM GB/s vs peak, (W,R)=(8,4),(8,2)"
FLUSH_BYTES = 512 << 20


def _hip():
    h = ctypes.CDLL("libamdhip64.so")
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    return h


def _events(h, n):
    evs = []
    for _ in range(n):
        e = ctypes.c_void_p()
        assert h.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    return evs


def _elapsed(h, a, b):
    ms = ctypes.c_float()
    assert h.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
    return ms.value


class Stepper:
    """Device state of one rate: the store (prefilled), fixed input buffers
    that one step's graph reads, and the decode outputs."""

    def __init__(self, cfg, dev, lcfg, R, torch, codec=None, policy=None):
        from query_adaptive_decode_amd import binding as Bd
        self.Bd, self.torch, self.cfg, self.dev, self.lcfg, self.R = Bd, torch, cfg, dev, lcfg, R
        self.policy = Bd.SCOPE_KV_HEAD if policy is None else policy
        B, H, G, d = cfg["B"], cfg["H"], cfg["G"], cfg["d"]
        self.cache = Bd.ReadKVCache(lcfg)
        if codec is not None:   # Lloyd code: signs and calibration before the prompt
            Bd.codec_init(lcfg, self.cache.store, codec["sk"], codec["sv"], codec["kcal"],
                          codec["vcal"])
        self.cache.append(dev["kpre"], dev["vpre"])
        self.out = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
        self.kbuf = torch.empty_like(dev["kstep"][0])
        self.vbuf = torch.empty_like(dev["vstep"][0])
        self.qbuf = torch.empty_like(dev["q"][0])
        capmax = (lcfg.capacity_tokens + 31) // 32 * 32
        self.tk = torch.zeros(B * G * d, dtype=torch.uint8, device="cuda")
        self.tv = torch.zeros((B, G, capmax), dtype=torch.uint8, device="cuda")
        self.s = 0          # next decode step (index into the step inputs)
        self.graph = None

    def load(self):
        """Copy step s's inputs into the fixed buffers (outside any timing)."""
        self.kbuf.copy_(self.dev["kstep"][self.s])
        self.vbuf.copy_(self.dev["vstep"][self.s])
        self.qbuf.copy_(self.dev["q"][self.s])

    def step_eager(self):
        self.load()
        self.cache.append(self.kbuf, self.vbuf)
        self.cache.decode(self.qbuf, self.R, self.R, out=self.out, policy=self.policy)
        self.s += 1

    def capture(self):
        torch = self.torch
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.cache.append(self.kbuf, self.vbuf)
            self.cache.decode(self.qbuf, self.R, self.R, out=self.out, policy=self.policy)
        torch.cuda.synchronize()


def flush_buffer(torch):
    """A 512 MiB device buffer, written once (its lines are clean by the
    time it is read again)."""
    return torch.empty(FLUSH_BYTES // 8, dtype=torch.int64, device="cuda").fill_(1)


def flush(scratch):
    """Evict the store from the L2s and the 256 MB Infinity Cache by reading
    512 MiB.  A read leaves clean lines behind; a write would leave about
    256 MB of dirty lines whose write-back to HBM lands in the timed step."""
    scratch.sum()


def run_rate(cfg, dev, lcfg, R, warmup, steps, torch, h, codec=None, policy=None):
    """Warm and flushed step times (graph replays) and per-kernel durations
    (HIP events on the launch stream around each stage).  policy: the decode
    policy (default per-KV-head budgets)."""
    B, H, G, d = cfg["B"], cfg["H"], cfg["G"], cfg["d"]
    T0 = int(cfg["T0"])
    st = Stepper(cfg, dev, lcfg, R, torch, codec, policy)
    for _ in range(warmup):
        st.step_eager()
    st.capture()
    stream = torch.cuda.current_stream().cuda_stream
    scratch = flush_buffer(torch)
    e0, e1 = _events(h, 2)

    def timed_replay(evict):
        st.load()
        if evict:
            flush(scratch)
        h.hipEventRecord(ctypes.c_void_p(e0), ctypes.c_void_p(stream))
        st.graph.replay()
        h.hipEventRecord(ctypes.c_void_p(e1), ctypes.c_void_p(stream))
        h.hipEventSynchronize(ctypes.c_void_p(e1))
        n = T0 + st.s + 1
        st.s += 1
        return _elapsed(h, e0, e1), n

    res = {}
    for mode in ("warm", "evicted"):
        tot, qh_tok = 0.0, 0
        for _ in range(steps):
            ms, n = timed_replay(mode == "evicted")
            tot += ms
            qh_tok += B * H * n
        res[mode] = dict(ms_per_step=tot / steps, qh_tok_per_s=qh_tok / (tot * 1e-3))
    # per-kernel durations: the timed entry point records events between
    # its stages; the append is bracketed separately
    ksum = torch.zeros((), dtype=torch.int64, device="cuda")
    vsum = torch.zeros((), dtype=torch.int64, device="cuda")
    kern = {}
    tp_list = []
    for mode in ("warm", "evicted"):
        evs = [_events(h, len(KERNELS) + 1) for _ in range(steps)]
        eenc = [_events(h, 2) for _ in range(steps)]
        for i in range(steps):
            st.load()
            if mode == "evicted":
                flush(scratch)
            h.hipEventRecord(ctypes.c_void_p(eenc[i][0]), ctypes.c_void_p(stream))
            st.cache.append(st.kbuf, st.vbuf)
            h.hipEventRecord(ctypes.c_void_p(eenc[i][1]), ctypes.c_void_p(stream))
            st.Bd.decode_attn_timed(lcfg, st.cache.store, st.qbuf, R, R, st.cache.workspace, evs[i],
                                    out=st.out, key_depths=st.tk, value_depths=st.tv.view(-1),
                                    policy=st.policy)
            n = T0 + st.s + 1
            tp = n // 32 * 32
            if mode == "warm":
                tp_list.append(tp)
                ksum += st.tk.sum(dtype=torch.int64)
                vsum += st.tv[:, :, :tp].sum(dtype=torch.int64)
            st.s += 1
        torch.cuda.synchronize()
        km = {k: 0.0 for k in KERNELS}
        enc = 0.0
        for i in range(steps):
            for k in range(len(KERNELS)):
                km[KERNELS[k]] += _elapsed(h, evs[i][k], evs[i][k + 1])
            enc += _elapsed(h, eenc[i][0], eenc[i][1])
        kern[mode] = {k: v / steps for k, v in km.items()}
        kern[mode]["append"] = enc / steps
    del scratch
    tpm = sum(tp_list) / steps
    ng = tpm / 32
    kpay = float(ksum.item()) / steps * tpm / 8            # bytes per launch, all (b,g)
    vpay = float(vsum.item()) / steps * d / 8
    if codec is None:
        meta = B * G * ng * d * 4                          # one of K or V metadata
        # the score launch also reads q and E^K for the key allocation in its prologue
        alg = {"score": kpay + meta + B * G * d * 8 + B * H * d * 2, "value_gather": vpay + meta,
               "value_alloc": B * G * ng * 8}
        step_bytes = kpay + vpay + 2 * meta
    else:
        # Lloyd code: no per-group metadata; the calibration arrays (4 x G x d
        # float32) and the decoder table (518 float32) once per call; the
        # score stage (key allocation + score) reads q
        shared = G * d * 16 + 518 * 4
        alg = {"score": kpay + B * H * d * 2 + G * d * 8, "value_gather": vpay + G * d * 8,
               "value_alloc": 0.0}
        step_bytes = kpay + vpay + shared
    return dict(R=R, time=res, kernel_ms=kern, alg_bytes=alg, step_alg_bytes=step_bytes,
                key_bits=float(ksum.item()) / steps / (B * G * d),
                value_bits=float(vsum.item()) / steps / (B * G * tpm), steps_used=st.s)


def run_single_launch(cfg, dev, lcfg, R, warmup, steps, torch, h):
    """The single-launch reader beside the split launches, both as eager
    steps (a cooperative launch is not captured in a graph), alternating step
    by step on one cache: HIP events before the append, and from the timed
    decode entry point around the decode; warm, and with the caches flushed
    before each step."""
    from query_adaptive_decode_amd.binding import SCOPE_KV_HEAD, SINGLE_LAUNCH
    B, H = cfg["B"], cfg["H"]
    T0 = int(cfg["T0"])
    st = Stepper(cfg, dev, lcfg, R, torch)
    stream = torch.cuda.current_stream().cuda_stream
    scratch = flush_buffer(torch)
    paths = (("split", SCOPE_KV_HEAD), ("single_launch", SINGLE_LAUNCH))

    def one(policy, evict):
        ev = _events(h, 5)
        st.load()
        if evict:
            flush(scratch)
        h.hipEventRecord(ctypes.c_void_p(ev[0]), ctypes.c_void_p(stream))
        st.cache.append(st.kbuf, st.vbuf)
        st.Bd.decode_attn_timed(lcfg, st.cache.store, st.qbuf, R, R, st.cache.workspace, ev[1:],
                                out=st.out, policy=policy)
        h.hipEventSynchronize(ctypes.c_void_p(ev[4]))
        n = T0 + st.s + 1
        st.s += 1
        return _elapsed(h, ev[0], ev[4]), _elapsed(h, ev[1], ev[4]), n

    for i in range(warmup):
        one(paths[i % 2][1], False)
    res = {name: {} for name, _ in paths}
    for mode in ("warm", "evicted"):
        acc = {name: [0.0, 0.0, 0] for name, _ in paths}
        for _ in range(steps):
            for name, pol in paths:
                step_ms, dec_ms, n = one(pol, mode == "evicted")
                acc[name][0] += step_ms
                acc[name][1] += dec_ms
                acc[name][2] += B * H * n
        for name, (tot, dec, qh) in acc.items():
            res[name][mode] = dict(ms_per_step=tot / steps, decode_ms=dec / steps,
                                   qh_tok_per_s=qh / (tot * 1e-3))
    del scratch
    return res


def copy_bandwidth(torch, h, mib=1024, reps=5):
    """A plain device-to-device copy of `mib` MiB timed with events: bytes
    moved (read + write) per second."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = _events(h, 2)
    best = None
    for _ in range(reps):
        h.hipEventRecord(ctypes.c_void_p(e0), ctypes.c_void_p(stream))
        dst.copy_(src)
        h.hipEventRecord(ctypes.c_void_p(e1), ctypes.c_void_p(stream))
        h.hipEventSynchronize(ctypes.c_void_p(e1))
        ms = _elapsed(h, e0, e1)
        best = ms if best is None else min(best, ms)
    del src, dst
    return 2.0 * (mib << 20) / (best * 1e-3) / 1e9


def _oracle_unit(args):
    """One decode step of one (request, KV head) unit by the oracle, on one
    thread; returns (query-heads x context-tokens, seconds)."""
    wid, b, g = args
    try:
        from threadpoolctl import threadpool_limits
        lim = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        lim = None
    import oracle as O
    from query_adaptive_decode_amd import synth
    cfg = synth.workload(wid)
    gqa = cfg["H"] // cfg["G"]
    n = int(cfg["T0"]) + 1
    K, V = synth.kv_unit(cfg, b, g, n)
    q = synth.q_step(cfg, b, 0)[g * gqa:(g + 1) * gqa]
    t = time.perf_counter()
    O.decode_unit(q, K, V, W=cfg["W"], R_K=4.0, R_V=4.0)
    dt = time.perf_counter() - t
    del lim
    return gqa * n, dt


def cpu_baseline(cfg, budget_s=20.0):
    """The float64 oracle, untuned, on this host's cores: a process pool
    over (request, KV head) units (one thread each) for one decode step,
    and the same work on one core."""
    import multiprocessing as mp
    # worker processes are spawned (fresh interpreters that never open the
    # GPU), at most 16: the host's CPU share of one GPU
    cores = min(len(os.sched_getaffinity(0)), 16)
    units = [(cfg["id"], b, g) for b in range(cfg["B"]) for g in range(cfg["G"])]
    one = [_oracle_unit(units[0]) for _ in range(2)][-1]
    per_unit = one[1]
    # as many units as the pool finishes in about budget_s (all of one step
    # when that fits)
    n_units = max(cores, min(len(units), int(budget_s * cores / max(per_unit, 1e-3))))
    n_units = min(n_units, len(units))
    ctx = mp.get_context("spawn")
    t = time.perf_counter()
    with ctx.Pool(processes=cores) as pool:
        res = pool.map(_oracle_unit, units[:n_units], chunksize=1)
    wall = time.perf_counter() - t
    qh_tok = sum(r[0] for r in res)
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return dict(value=qh_tok / wall, unit="query-heads*ctx-tokens/s", cores=cores, kind="oracle",
                sample=f"{n_units} of {len(units)} (request, KV head) units of one decode step at "
                       f"T={int(cfg['T0']) + 1}, (W,R)=(8,4): float64 numpy, a pool of {cores} "
                       f"processes (one thread each; inputs drawn inside the timed tasks), "
                       f"{wall:.1f} s; CPU {model}",
                single_core=dict(value=one[0] / one[1], seconds_per_unit=per_unit))


def counters_run(cfg, dev, lcfg, rates, warmup, steps, torch, codec=None):
    """The fixed launch sequence the rocprofv3 request-counter passes are
    taken on: a 512 MiB device copy (calibration), then per rate `warmup`
    steps, `steps` warm steps and `steps` steps each after a 512 MiB flush,
    all eager."""
    src = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    scratch = flush_buffer(torch)
    for R in rates:
        st = Stepper(cfg, dev, lcfg, R, torch, codec)
        for _ in range(warmup + steps):
            st.step_eager()
        for _ in range(steps):
            st.load()
            flush(scratch)
            st.cache.append(st.kbuf, st.vbuf)
            st.cache.decode(st.qbuf, st.R, st.R, out=st.out)
            st.s += 1
        torch.cuda.synchronize()
        del st
    print(f"# counters run: rates {rates}, warmup {warmup}, {steps} warm + {steps} flushed steps",
          file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rates", default="4,2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--lloyd-rates", default="4,2",
                    help="rates timed over the Lloyd-tree code ('' for none)")
    ap.add_argument("--single-launch-rates", default="4,2",
                    help="rates at which the single-launch reader is timed beside the split "
                         "launches, as eager steps ('' for none)")
    ap.add_argument("--policy-rates", default="4,2",
                    help="rates at which per-layer budgets and the restricted reader are timed "
                         "('' for none)")
    ap.add_argument("--counters-run", action="store_true",
                    help="run the fixed sequence the counter profiles are taken on, print no line")
    ap.add_argument("--lloyd", action="store_true",
                    help="with --counters-run: over the Lloyd-tree code")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: the decode path has no multi-GPU mode "
                                   "(requests and KV heads are independent; see the sharding "
                                   "notes); run with --gpus 1"}))
        sys.exit(2)
    from query_adaptive_decode_amd import synth, workload
    cfg = synth.workload(2)
    rates = [float(r) for r in args.rates.split(",")]
    per_rate = args.warmup + (2 if args.counters_run else 4) * args.steps
    if per_rate > int(cfg["steps"]):
        print(json.dumps({"error": f"warmup + {2 if args.counters_run else 4} x steps = {per_rate} "
                                   f"exceeds the workload's {cfg['steps']} decode steps"}))
        sys.exit(2)
    import torch
    t = time.perf_counter()
    hin = workload.host_inputs(cfg, per_rate)
    dev = workload.to_device(hin)
    del hin
    lcfg = workload.config_for(cfg, per_rate)
    lrates = [float(r) for r in args.lloyd_rates.split(",") if r.strip()]
    codec, lcfg_ll = None, None
    if lrates or args.lloyd:
        ci = workload.calibration_inputs(cfg, 512)
        cd = workload.to_device(dict(kcal=ci["kcal"], vcal=ci["vcal"]))
        codec = dict(sk=ci["sk"].tolist(), sv=ci["sv"].tolist(), kcal=cd["kcal"], vcal=cd["vcal"])
        lcfg_ll = workload.config_for(dict(cfg, codec="lloyd"), per_rate)
    print(f"# inputs ready in {time.perf_counter() - t:.1f} s", file=sys.stderr, flush=True)
    if args.counters_run:
        if args.lloyd:
            counters_run(cfg, dev, lcfg_ll, rates, args.warmup, args.steps, torch, codec)
        else:
            counters_run(cfg, dev, lcfg, rates, args.warmup, args.steps, torch)
        return
    from query_adaptive_decode_amd import profile_summary as PS
    h = _hip()
    copy_gbps = copy_bandwidth(torch, h)
    print(f"# device copy: {copy_gbps:.0f} GB/s moved", file=sys.stderr, flush=True)
    moved = PS.committed_bytes()   # per-kernel bytes from the counters, or None
    res = {}
    for R in rates:
        r = run_rate(cfg, dev, lcfg, R, args.warmup, args.steps, torch, h)
        res[R] = r
        tm, km = r["time"], r["kernel_ms"]
        print(f"# R={R:g}: evicted {tm['evicted']['ms_per_step']:.3f} ms/step "
              f"({tm['evicted']['qh_tok_per_s'] / 1e9:.2f} G qh*tok/s), warm "
              f"{tm['warm']['ms_per_step']:.3f} ms/step ({tm['warm']['qh_tok_per_s'] / 1e9:.2f} G); "
              f"kernels evicted {json.dumps({k: round(v * 1e3, 1) for k, v in km['evicted'].items()})} us, "
              f"warm {json.dumps({k: round(v * 1e3, 1) for k, v in km['warm'].items()})} us",
              file=sys.stderr, flush=True)
    head = res[rates[0]]
    kev = head["kernel_ms"]["evicted"]
    dom = max(["score", "value_gather"], key=lambda k: kev[k])
    ach = head["alg_bytes"][dom] / (kev[dom] * 1e-3) / 1e9

    def rate_key(R):
        return f"8,{R:g}"

    def moved_of(R, mode):
        if not moved:
            return None
        m = moved.get(rate_key(R), {}).get(mode)
        if not m:
            return None
        return m

    traffic = None
    m_dom = moved_of(rates[0], "evicted")
    if m_dom and dom in m_dom["kernels"]:
        traffic = m_dom["kernels"][dom]["read_bytes"] + m_dom["kernels"][dom]["write_bytes"]
    line = {
        "metric": METRIC,
        "value": head["time"]["evicted"]["qh_tok_per_s"],
        "unit": "query-heads*ctx-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["time"]["evicted"]["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8 codes; i8 MFMA + f64 logits; f16 MFMA + f32 values",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "batch": cfg["B"], "q_heads": cfg["H"],
                   "kv_heads": cfg["G"], "head_dim": cfg["d"], "prompt_tokens": cfg["T0"],
                   "W": cfg["W"], "R": rates, "budget_scope": "kv_head",
                   "step": "append 1 token/request + decode, caches flushed before each step"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS, "traffic": traffic,
                     "alg_bytes_per_launch": head["alg_bytes"][dom], "kernel_us": kev[dom] * 1e3,
                     "timing": "HIP events, caches flushed before each step"},
        "copy_peak_GBps": copy_gbps,
        "rates": {},
    }
    for R, r in res.items():
        tm, km = r["time"], r["kernel_ms"]
        ent = {
            "evicted_ms_per_step": tm["evicted"]["ms_per_step"],
            "evicted_qh_tok_per_s": tm["evicted"]["qh_tok_per_s"],
            "warm_ms_per_step": tm["warm"]["ms_per_step"],
            "warm_qh_tok_per_s": tm["warm"]["qh_tok_per_s"],
            "kernel_us": {mode: {k: v * 1e3 for k, v in km[mode].items()} for mode in km},
            "logical_bytes_per_step": r["step_alg_bytes"],
            "logical_GBps": {mode: r["step_alg_bytes"] / (tm[mode]["ms_per_step"] * 1e-3) / 1e9
                             for mode in tm},
            "key_bits_per_scalar": r["key_bits"],
            "value_bits_per_scalar": r["value_bits"],
            "kernel_alg_GBps_evicted": {k: r["alg_bytes"][k] / (km["evicted"][k] * 1e-3) / 1e9
                                        for k in ("score", "value_gather")},
        }
        ent["logical_frac_of_peak"] = {m: v / HBM_PEAK_GBPS for m, v in ent["logical_GBps"].items()}
        for mode in ("evicted", "warm"):
            m = moved_of(R, mode)
            if m:
                step_b = m["step_read_bytes"] + m["step_write_bytes"]
                gbps = step_b / (tm[mode]["ms_per_step"] * 1e-3) / 1e9
                ent[f"moved_{mode}"] = {
                    "bytes_per_step": step_b, "read_bytes": m["step_read_bytes"],
                    "write_bytes": m["step_write_bytes"], "GBps": gbps,
                    "frac_of_peak": gbps / HBM_PEAK_GBPS, "frac_of_copy": gbps / copy_gbps,
                    "per_kernel_bytes": {k: v["read_bytes"] + v["write_bytes"]
                                         for k, v in m["kernels"].items()}}
        m_pre, m_ev = moved_of(R, "prefill"), moved_of(R, "evicted")
        if m_pre and m_ev and "append" in m_ev["kernels"]:
            # encoder writes (the prompt's encoding, then one append per step)
            # against the decode steps' reads, over the prompt plus L steps
            L = 128
            enc_w = m_pre["step_write_bytes"] + L * m_ev["kernels"]["append"]["write_bytes"]
            dec_r = L * m_ev["step_read_bytes"]
            ent["encode_traffic"] = {
                "steps": L, "prompt_tokens": int(cfg["T0"]), "prefill_write_bytes": m_pre["step_write_bytes"],
                "append_write_bytes_per_step": m_ev["kernels"]["append"]["write_bytes"],
                "decode_read_bytes_per_step": m_ev["step_read_bytes"],
                "encode_write_over_decode_read": enc_w / dec_r}
        line["rates"][rate_key(R)] = ent
    if moved is None:
        line["moved_bytes_note"] = ("no counter summary for these kernel sources "
                                    "(profiles/ was taken on other sources)")
    if lrates:
        ll = {"code": "Gaussian Lloyd tree (depth 8, float32 table) + Hadamard-sign transforms, "
                      "calibrated on 512 held-out synthetic tokens per KV head",
              "dtype": "u8 tree paths; f64 logits over centroids; f16 MFMA + f32 values",
              "rates": {}}
        moved_ll = PS.committed_bytes(PS.SUMMARY_LLOYD)
        for R in lrates:
            r = run_rate(cfg, dev, lcfg_ll, R, args.warmup, args.steps, torch, h, codec)
            tm, km = r["time"], r["kernel_ms"]
            print(f"# Lloyd R={R:g}: evicted {tm['evicted']['ms_per_step']:.3f} ms/step "
                  f"({tm['evicted']['qh_tok_per_s'] / 1e9:.2f} G qh*tok/s), warm "
                  f"{tm['warm']['ms_per_step']:.3f} ms/step; kernels evicted "
                  f"{json.dumps({k: round(v * 1e3, 1) for k, v in km['evicted'].items()})} us",
                  file=sys.stderr, flush=True)
            ent = {
                "evicted_ms_per_step": tm["evicted"]["ms_per_step"],
                "evicted_qh_tok_per_s": tm["evicted"]["qh_tok_per_s"],
                "warm_ms_per_step": tm["warm"]["ms_per_step"],
                "warm_qh_tok_per_s": tm["warm"]["qh_tok_per_s"],
                "kernel_us": {mode: {k: v * 1e3 for k, v in km[mode].items()} for mode in km},
                "logical_bytes_per_step": r["step_alg_bytes"],
                "logical_GBps": {mode: r["step_alg_bytes"] / (tm[mode]["ms_per_step"] * 1e-3) / 1e9
                                 for mode in tm},
                "key_bits_per_scalar": r["key_bits"],
                "value_bits_per_scalar": r["value_bits"],
                "kernel_alg_GBps_evicted": {k: r["alg_bytes"][k] / (km["evicted"][k] * 1e-3) / 1e9
                                            for k in ("score", "value_gather")},
            }
            m = moved_ll.get(rate_key(R), {}).get("evicted") if moved_ll else None
            if m:
                step_b = m["step_read_bytes"] + m["step_write_bytes"]
                gbps = step_b / (tm["evicted"]["ms_per_step"] * 1e-3) / 1e9
                ent["moved_evicted"] = {"bytes_per_step": step_b, "GBps": gbps,
                                        "frac_of_peak": gbps / HBM_PEAK_GBPS,
                                        "per_kernel_bytes": {k: v["read_bytes"] + v["write_bytes"]
                                                             for k, v in m["kernels"].items()}}
            ll["rates"][rate_key(R)] = ent
        line["lloyd_codec"] = ll
    prates = [float(r) for r in args.policy_rates.split(",") if r.strip()]
    if prates:
        from query_adaptive_decode_amd import binding as Bd
        pols = {
            "layer": ("one key and one value budget per request over all its KV heads "
                      "(READKV_SCOPE_LAYER)", Bd.SCOPE_LAYER),
            "restricted": ("per-KV-head budgets, minimum depth one and two-token value packets "
                           "(READKV_RESTRICT_MIN_DEPTH1 | READKV_RESTRICT_VALUE_PAIRS)",
                           Bd.RESTRICT_MIN_DEPTH1 | Bd.RESTRICT_VALUE_PAIRS),
        }
        out_p = {}
        for name, (what, pol) in pols.items():
            ent_p = {"what": what, "rates": {}}
            for R in prates:
                r = run_rate(cfg, dev, lcfg, R, args.warmup, args.steps, torch, h, policy=pol)
                tm, km = r["time"], r["kernel_ms"]
                print(f"# {name} R={R:g}: evicted {tm['evicted']['ms_per_step']:.3f} ms/step "
                      f"({tm['evicted']['qh_tok_per_s'] / 1e9:.2f} G qh*tok/s), warm "
                      f"{tm['warm']['ms_per_step']:.3f} ms/step; kernels evicted "
                      f"{json.dumps({k: round(v * 1e3, 1) for k, v in km['evicted'].items()})} us",
                      file=sys.stderr, flush=True)
                ent_p["rates"][rate_key(R)] = {
                    "evicted_ms_per_step": tm["evicted"]["ms_per_step"],
                    "evicted_qh_tok_per_s": tm["evicted"]["qh_tok_per_s"],
                    "warm_ms_per_step": tm["warm"]["ms_per_step"],
                    "warm_qh_tok_per_s": tm["warm"]["qh_tok_per_s"],
                    "kernel_us": {mode: {k: v * 1e3 for k, v in km[mode].items()} for mode in km},
                    "logical_bytes_per_step": r["step_alg_bytes"],
                    "key_bits_per_scalar": r["key_bits"],
                    "value_bits_per_scalar": r["value_bits"],
                    "kernel_alg_GBps_evicted": {k: r["alg_bytes"][k] / (km["evicted"][k] * 1e-3) / 1e9
                                                for k in ("score", "value_gather")},
                }
            out_p[name] = ent_p
        line["policies"] = out_p
    srates = [float(r) for r in args.single_launch_rates.split(",") if r.strip()]
    if srates:
        sl = {"what": "one cooperative launch per decode (grid-wide barriers between the "
                      "stages) against the split launches, eager steps alternating on one "
                      "cache; step = append + decode",
              "rates": {}}
        from query_adaptive_decode_amd.binding import ReadKVError
        for R in srates:
            try:
                r = run_single_launch(cfg, dev, lcfg, R, args.warmup, args.steps, torch, h)
            except ReadKVError as e:
                # e.g. a device without cooperative launch: the headline line
                # still prints, with the reason here
                sl["rates"][rate_key(R)] = {"error": str(e)}
                print(f"# single launch R={R:g}: {e}", file=sys.stderr, flush=True)
                continue
            print(f"# single launch R={R:g}: evicted step {r['single_launch']['evicted']['ms_per_step']:.3f} "
                  f"ms (decode {r['single_launch']['evicted']['decode_ms']:.3f}), split eager "
                  f"{r['split']['evicted']['ms_per_step']:.3f} ms (decode "
                  f"{r['split']['evicted']['decode_ms']:.3f})", file=sys.stderr, flush=True)
            sl["rates"][rate_key(R)] = {
                name: {f"{mode}_{k}": v for mode, d in r[name].items() for k, v in d.items()}
                for name in r}
        line["single_launch"] = sl
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
