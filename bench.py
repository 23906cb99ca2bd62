#!/usr/bin/env python3
"""ReadKV decode-step benchmark on one MI355X.

Workload: the Llama-3-8B-shaped attention layer (32 query / 8 KV heads,
head_dim 128, batch 16, 8192-token prompt, W = 8 stored bits), synthetic
seeded K/V/q.  One step = append one token per request through the encoder
+ one ReadKV decode (key allocation, score, value allocation, value gather,
output reduction), for read rates R = 4 and R = 2 (R_K = R_V = R).

Prints one JSON line.  `value` is query-heads x context-tokens per second
at (W, R) = (8, 4) with inputs resident in HBM; per-rate figures, the
per-kernel roofline of the dominant kernel (live HIP-event timing) and the
float64 oracle's CPU throughput on a bounded sample are included.
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
METRIC = "decode attn query-heads\u00b7ctx-tokens/s + achieved HBM GB/s vs peak, (W,R)=(8,4),(8,2)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_decode_step_llama3-8b-B16-T8192.txt")


def source_hash():
    """sha256 over the HIP sources and headers the library is built from."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "query_adaptive_decode_amd", "csrc")
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None when it was taken on other sources (or is missing)."""
    try:
        rows = [l.strip() for l in open(TRAFFIC_FILE) if "=" in l and not l.startswith("#")]
    except OSError:
        return None
    kv = dict(l.split("=", 1) for l in rows)
    if kv.get("source_sha256") != source_hash():
        return None
    try:
        return float(kv[f"{kernel}.fetch_bytes"]) + float(kv[f"{kernel}.write_bytes"])
    except (KeyError, ValueError):
        return None


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


def run_rate(cfg, dev, lcfg, R, warmup, steps, torch, evict=True):
    from query_adaptive_decode_amd import binding as Bd
    B, H, G, d = cfg["B"], cfg["H"], cfg["G"], cfg["d"]
    T0 = int(cfg["T0"])
    cache = Bd.ReadKVCache(lcfg)
    cache.append(dev["kpre"], dev["vpre"])
    out = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
    capmax = (lcfg.capacity_tokens + 31) // 32 * 32
    tk = torch.zeros(B * G * d, dtype=torch.uint8, device="cuda")
    tv = torch.zeros((B, G, capmax), dtype=torch.uint8, device="cuda")
    s = 0
    for _ in range(warmup):
        cache.append(dev["kstep"][s], dev["vstep"][s])
        cache.decode(dev["q"][s], R, R, out=out)
        s += 1
    torch.cuda.synchronize()
    # ---- timed region: whole steps (append + decode), recorded once into a
    # HIP graph and replayed, so host launch overhead is not timed ----
    s0 = s
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            cache.append(dev["kstep"][s0 + i], dev["vstep"][s0 + i])
            cache.decode(dev["q"][s0 + i], R, R, out=out)
    torch.cuda.synchronize()
    t_begin = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_begin
    s = s0 + steps
    ctx = [T0 + i + 1 for i in range(s0, s0 + steps)]
    qh_tok = B * H * sum(ctx)
    # ---- per-kernel timing with HIP events on the launch stream ----
    h = _hip()
    stream = torch.cuda.current_stream().cuda_stream
    ev = [_events(h, len(KERNELS) + 1) for _ in range(steps)]
    eenc = [_events(h, 2) for _ in range(steps)]
    ksum = torch.zeros((), dtype=torch.int64, device="cuda")
    vsum = torch.zeros((), dtype=torch.int64, device="cuda")
    tp_list = []
    for i in range(steps):
        h.hipEventRecord(ctypes.c_void_p(eenc[i][0]), ctypes.c_void_p(stream))
        cache.append(dev["kstep"][s], dev["vstep"][s])
        h.hipEventRecord(ctypes.c_void_p(eenc[i][1]), ctypes.c_void_p(stream))
        Bd.decode_attn_timed(lcfg, cache.store, dev["q"][s], R, R, cache.workspace, ev[i], out=out,
                             key_depths=tk, value_depths=tv.view(-1))
        n = T0 + s + 1
        tp = n // 32 * 32
        tp_list.append(tp)
        ksum += tk.sum(dtype=torch.int64)
        vsum += tv[:, :, :tp].sum(dtype=torch.int64)
        s += 1
    torch.cuda.synchronize()
    # ---- cache-evicted steps: a 512 MiB write before each step pushes the
    # store out of L2 and the Infinity Cache; the step is timed with events ----
    evict_ms = None
    if evict:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        tot = 0.0
        for i in range(steps):
            scratch.fill_(i & 0xFF)
            ev0.record()
            cache.append(dev["kstep"][s], dev["vstep"][s])
            cache.decode(dev["q"][s], R, R, out=out)
            ev1.record()
            ev1.synchronize()
            tot += ev0.elapsed_time(ev1)
            s += 1
        evict_ms = tot / steps
        del scratch
    kern_ms = {k: 0.0 for k in KERNELS}
    enc_ms = 0.0
    for i in range(steps):
        for k in range(len(KERNELS)):
            kern_ms[KERNELS[k]] += _elapsed(h, ev[i][k], ev[i][k + 1])
        enc_ms += _elapsed(h, eenc[i][0], eenc[i][1])
    kern_ms = {k: v / steps for k, v in kern_ms.items()}
    enc_ms /= steps
    tpm = sum(tp_list) / steps
    ng = tpm / 32
    kpay = float(ksum.item()) / steps * tpm / 8            # bytes per launch, all (b,g)
    vpay = float(vsum.item()) / steps * d / 8
    meta = B * G * ng * d * 4                              # one of K or V metadata
    # the score launch also reads q and E^K for the key allocation in its prologue
    alg = {"score": kpay + meta + B * G * d * 8 + B * H * d * 2, "value_gather": vpay + meta,
           "value_alloc": B * G * ng * 8}
    step_bytes = kpay + vpay + 2 * meta
    return dict(R=R, ms_per_step=wall / steps * 1e3, qh_tok_per_s=qh_tok / wall,
                evicted_ms_per_step=evict_ms,
                kernel_ms=kern_ms, encode_ms=enc_ms, alg_bytes=alg, step_alg_bytes=step_bytes,
                logical_GBps_step=step_bytes / (wall / steps) / 1e9,
                mean_key_bits_per_scalar=float(ksum.item()) / steps / (B * G * d),
                mean_value_bits_per_scalar=float(vsum.item()) / steps / (B * G * tpm))


def cpu_baseline(cfg, budget_s=12.0):
    """The float64 oracle, untuned, on this host: one decode step of a
    sample of (request, KV head) units, single-threaded."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    import oracle as O
    from query_adaptive_decode_amd import synth
    gqa = cfg["H"] // cfg["G"]
    T0 = int(cfg["T0"])
    units = [(b, g) for b in range(cfg["B"]) for g in range(cfg["G"])]
    ctx = None
    done = 0
    qh_tok = 0
    t_all = 0.0
    import contextlib
    lim = threadpool_limits(limits=1) if threadpool_limits else contextlib.nullcontext()
    with lim:
        for (b, g) in units:
            K, V = synth.kv_unit(cfg, b, g, T0 + 1)
            q = synth.q_step(cfg, b, 0)[g * gqa:(g + 1) * gqa]
            t = time.perf_counter()
            O.decode_unit(q, K, V, W=cfg["W"], R_K=4.0, R_V=4.0)
            t_all += time.perf_counter() - t
            done += 1
            qh_tok += gqa * (T0 + 1)
            ctx = T0 + 1
            if t_all >= budget_s and done >= 2:
                break
    _ = np
    return dict(value=qh_tok / t_all, unit="query-heads*ctx-tokens/s", cores=1, kind="oracle",
                sample=f"{done} of {len(units)} (request, KV head) units, one decode step at "
                       f"T={ctx}, (W,R)=(8,4), float64 numpy single thread, {t_all:.1f} s")


def copy_probe(torch, mib=512, reps=3):
    """A plain device-to-device copy of a known size: its FETCH_SIZE /
    WRITE_SIZE counter readings give the scale from counter units to bytes."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"# copy probe: {reps} copies of {mib} MiB", file=sys.stderr, flush=True)
    del src, dst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rates", default="4,2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-evict", action="store_true",
                    help="skip the cache-evicted per-step timing")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 512 MiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: the decode path has no multi-GPU mode "
                                   "(requests and KV heads are independent; see the sharding "
                                   "notes); run with --gpus 1"}))
        sys.exit(2)
    import torch
    from query_adaptive_decode_amd import synth, workload

    cfg = synth.workload(2)
    rates = [float(r) for r in args.rates.split(",")]
    if args.copy_probe:
        copy_probe(torch)
    total_steps = args.warmup + (3 if not args.no_evict else 2) * args.steps
    if total_steps > int(cfg["steps"]):
        print(json.dumps({"error": f"warmup + {'3' if not args.no_evict else '2'} x steps = {total_steps} "
                                   f"exceeds the workload's {cfg['steps']} decode steps"}))
        sys.exit(2)
    t = time.perf_counter()
    hin = workload.host_inputs(cfg, total_steps)
    dev = workload.to_device(hin)
    del hin
    lcfg = workload.config_for(cfg, total_steps)
    print(f"# inputs ready in {time.perf_counter() - t:.1f} s", file=sys.stderr, flush=True)
    res = {}
    for R in rates:
        res[R] = run_rate(cfg, dev, lcfg, R, args.warmup, args.steps, torch, evict=not args.no_evict)
        r = res[R]
        print(f"# R={R}: {r['ms_per_step']:.3f} ms/step, {r['qh_tok_per_s'] / 1e9:.2f} G qh*tok/s, "
              f"kernels {json.dumps({k: round(v * 1e3, 1) for k, v in r['kernel_ms'].items()})} us, "
              f"encode {r['encode_ms'] * 1e3:.1f} us, evicted "
              f"{(r['evicted_ms_per_step'] or 0.0):.3f} ms/step", file=sys.stderr, flush=True)
    head = res[rates[0]]
    dom = max(["score", "value_gather"], key=lambda k: head["kernel_ms"][k])
    ach = head["alg_bytes"][dom] / (head["kernel_ms"][dom] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": head["qh_tok_per_s"],
        "unit": "query-heads*ctx-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8 codes; i8 MFMA + f64 logits; f16 MFMA + f32 values",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "batch": cfg["B"], "q_heads": cfg["H"],
                   "kv_heads": cfg["G"], "head_dim": cfg["d"], "prompt_tokens": cfg["T0"],
                   "W": cfg["W"], "R": rates, "step": "append 1 token/request + decode"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(dom),
                     "alg_bytes_per_launch": head["alg_bytes"][dom],
                     "kernel_us": head["kernel_ms"][dom] * 1e3},
        "rates": {f"8,{R:g}": {
            "qh_tok_per_s": r["qh_tok_per_s"], "ms_per_step": r["ms_per_step"],
            "evicted_ms_per_step": r["evicted_ms_per_step"],
            "kernel_us": {k: v * 1e3 for k, v in r["kernel_ms"].items()},
            "encode_us": r["encode_ms"] * 1e3,
            "logical_bytes_per_step": r["step_alg_bytes"],
            "logical_GBps_step": r["logical_GBps_step"],
            "key_bits_per_scalar": r["mean_key_bits_per_scalar"],
            "value_bits_per_scalar": r["mean_value_bits_per_scalar"],
            "kernel_alg_GBps": {k: r["alg_bytes"][k] / (r["kernel_ms"][k] * 1e-3) / 1e9
                                for k in ("score", "value_gather")}}
            for R, r in res.items()},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
