"""Bytes moved per kernel launch from rocprofv3 request counters.

The committed summary ``profiles/hbm_bytes_decode_step_llama3-8b-B16-T8192.txt``
is written by this module from two ``rocprofv3 --pmc`` passes over
``bench.py --counters-run`` (a 512 MiB device copy, then per rate: warm-up
steps, warm steps, and steps each after a 512 MiB cache flush) and read by
``bench.py``, which reports the bytes only when the summary was taken on the
kernel sources it runs (sha256 over query_adaptive_decode_amd/csrc).

Counters (summed over the L2 channels):
  read  = 32 TCC_EA0_RDREQ_32B + 64 TCC_EA0_RDREQ_64B + 128 TCC_EA0_RDREQ_128B
  write = 32 (TCC_EA0_WRREQ - TCC_EA0_WRREQ_64B) + 64 TCC_EA0_WRREQ_64B
  dram  = 32 TCC_EA0_RDREQ_DRAM_32B (reads sent to the memory controllers)
Each is divided by what it gives for the copy (512 MiB read and written),
so the bytes are in units the copy fixes.  Usage:

  python -m query_adaptive_decode_amd.profile_summary --p1 DIR --p2 DIR \\
      --warmup W --steps N --rates 4,2 --command "..." --out FILE
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SUMMARY = os.path.join(ROOT, "profiles", "hbm_bytes_decode_step_llama3-8b-B16-T8192.txt")
# the same step over the Lloyd-tree code (bench.py --counters-run --lloyd)
SUMMARY_LLOYD = os.path.join(ROOT, "profiles", "hbm_bytes_decode_step_lloyd_llama3-8b-B16-T8192.txt")
COPY_BYTES = 512 << 20

# kernel name prefix -> short name (bench.py's stage names where they exist)
NAMES = [("k_append_small", "append"), ("k_key_alloc", "key_alloc"), ("k_score", "score"),
         ("k_key_alloc_lloyd", "key_alloc"), ("k_score_lloyd", "score"),
         ("k_out_reduce_lloyd", "out_reduce"),
         ("k_value_alloc_unit", "value_alloc"), ("k_value_weights", "value_weights"),
         ("k_value_select", "value_select"), ("k_gather", "value_gather"),
         ("k_out_reduce", "out_reduce")]
STEP_KERNELS = list(dict.fromkeys(n for _, n in NAMES))
# the prompt's encoding (one launch each per rate, when its store is filled)
PREFILL = [("k_encode_tiles", "encode_tiles"), ("k_ek_update", "encode_ek"),
           ("k_tail_update", "encode_tail")]
PREFILL_KERNELS = [n for _, n in PREFILL]


def source_hash() -> str:
    """sha256 over the HIP sources and headers the library is built from."""
    h = hashlib.sha256()
    d = os.path.join(HERE, "csrc")
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def _short(kname: str):
    base = kname.split("(")[0].replace("void ", "").replace("readkv::", "").split("<")[0].strip()
    for pre, short in NAMES + PREFILL:
        if base == pre:
            return short
    if "copyBuffer" in kname:
        return "copy"
    return None


def _dispatches(pdir: str):
    """{short name: [(dispatch id, {counter: value})] in dispatch order}"""
    rows = {}
    for f in glob.glob(os.path.join(pdir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            n = _short(r["Kernel_Name"])
            if n is None:
                continue
            rows.setdefault(n, {}).setdefault(int(r["Dispatch_Id"]), {})[r["Counter_Name"]] = \
                float(r["Counter_Value"])
    return {n: sorted(v.items()) for n, v in rows.items()}


def summarize(p1: str, p2: str, warmup: int, steps: int, rates):
    """Per rate and mode (warm / evicted): median counter values per launch
    of each step kernel, turned into bytes with the copy's scale."""
    d1, d2 = _dispatches(p1), _dispatches(p2)

    def merged(n):
        a, b = d1.get(n, []), d2.get(n, [])
        if len(a) != len(b):
            raise ValueError(f"{n}: {len(a)} vs {len(b)} dispatches in the two passes")
        return [{**x[1], **y[1]} for x, y in zip(a, b)]

    def raw_bytes(c):
        rd = 32 * c["TCC_EA0_RDREQ_32B_sum"] + 64 * c["TCC_EA0_RDREQ_64B_sum"] + \
            128 * c["TCC_EA0_RDREQ_128B_sum"]
        wr = 32 * (c["TCC_EA0_WRREQ_sum"] - c["TCC_EA0_WRREQ_64B_sum"]) + 64 * c["TCC_EA0_WRREQ_64B_sum"]
        dram = 32 * c["TCC_EA0_RDREQ_DRAM_32B_sum"]
        return rd, wr, dram

    copies = merged("copy")
    big = max(copies, key=lambda c: raw_bytes(c)[0])
    crd, cwr, cdram = raw_bytes(big)
    scale = dict(read=COPY_BYTES / crd, write=COPY_BYTES / cwr, dram=COPY_BYTES / cdram)
    out = dict(copy=dict(raw_read=crd, raw_write=cwr, raw_dram=cdram, counters=big), scale=scale,
               rates={})
    per_rate = warmup + 2 * steps
    for ri, R in enumerate(rates):
        ent = {}
        for mode, lo in (("warm", warmup), ("evicted", warmup + steps)):
            ks = {}
            for n in STEP_KERNELS:
                launches = merged(n) if n in d1 else []
                if not launches:
                    continue
                if len(launches) % per_rate:
                    raise ValueError(f"{n}: {len(launches)} launches, not a multiple of {per_rate}")
                sel = launches[ri * per_rate + lo: ri * per_rate + lo + steps]
                rd = statistics.median(raw_bytes(c)[0] for c in sel) * scale["read"]
                wr = statistics.median(raw_bytes(c)[1] for c in sel) * scale["write"]
                dr = statistics.median(raw_bytes(c)[2] for c in sel) * scale["dram"]
                ks[n] = dict(read_bytes=rd, write_bytes=wr, dram_read_bytes=dr, launches=len(sel))
            ent[mode] = dict(kernels=ks, step_read_bytes=sum(k["read_bytes"] for k in ks.values()),
                             step_write_bytes=sum(k["write_bytes"] for k in ks.values()))
        # the prompt's encoding: launch ri of each prefill kernel
        pk = {}
        for n in PREFILL_KERNELS:
            launches = merged(n) if n in d1 else []
            if len(launches) > ri:
                c = launches[ri]
                rd, wr, dr = raw_bytes(c)
                pk[n] = dict(read_bytes=rd * scale["read"], write_bytes=wr * scale["write"],
                             dram_read_bytes=dr * scale["dram"], launches=1)
        if pk:
            ent["prefill"] = dict(kernels=pk, step_read_bytes=sum(k["read_bytes"] for k in pk.values()),
                                  step_write_bytes=sum(k["write_bytes"] for k in pk.values()))
        out["rates"][f"8,{R:g}"] = ent
    return out


def write_summary(s, path, command, warmup, steps, rates):
    lines = [
        "# Bytes moved per launch (rocprofv3 request counters) of the ReadKV decode step,",
        "# Llama-3-8B-shaped layer B=16 H=32 G=8 d=128 T=8192 W=8; valid only for the kernel",
        "# sources with the hash below.  Written by query_adaptive_decode_amd/profile_summary.py.",
        f"# command (two passes, counters below): {command}",
        "#   pass 1: TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum",
        "#   pass 2: TCC_BUBBLE_sum TCC_EA0_RDREQ_DRAM_32B_sum TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_64B_sum",
        f"# launch sequence: 512 MiB copy; per rate {rates}: the prompt's encoding (prefill), "
        f"{warmup} warm-up, {steps} warm, {steps} flushed steps; medians over the {steps} launches "
        f"of each mode",
        f"source_sha256={source_hash()}",
        f"copy.raw_read_bytes={s['copy']['raw_read']:.0f}",
        f"copy.raw_write_bytes={s['copy']['raw_write']:.0f}",
        f"copy.raw_dram_read_bytes={s['copy']['raw_dram']:.0f}",
        f"copy.counters={' '.join(f'{k}:{v:.0f}' for k, v in sorted(s['copy']['counters'].items()))}",
        f"scale.read={s['scale']['read']:.6f}",
        f"scale.write={s['scale']['write']:.6f}",
        f"scale.dram={s['scale']['dram']:.6f}",
    ]
    for rk, ent in s["rates"].items():
        for mode, m in ent.items():
            for n, k in m["kernels"].items():
                for f in ("read_bytes", "write_bytes", "dram_read_bytes"):
                    lines.append(f"{rk}.{mode}.{n}.{f}={k[f]:.0f}")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def committed_bytes(path: str = SUMMARY):
    """{"8,R": {mode: {"kernels": {name: {...}}, "step_read_bytes", ...}}}
    from the committed summary, or None when it is missing or was taken on
    other kernel sources."""
    try:
        kv = dict(l.strip().split("=", 1) for l in open(path) if "=" in l and not l.startswith("#"))
    except OSError:
        return None
    if kv.get("source_sha256") != source_hash():
        return None
    out = {}
    for k, v in kv.items():
        parts = k.split(".")
        if len(parts) != 4 or not parts[0].startswith("8,"):
            continue
        rk, mode, n, f = parts
        out.setdefault(rk, {}).setdefault(mode, {"kernels": {}}).setdefault("kernels", {}) \
            .setdefault(n, {})[f] = float(v)
    for rk in out:
        for mode, m in out[rk].items():
            m["step_read_bytes"] = sum(k.get("read_bytes", 0.0) for k in m["kernels"].values())
            m["step_write_bytes"] = sum(k.get("write_bytes", 0.0) for k in m["kernels"].values())
    return out or None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--p1", required=True)
    ap.add_argument("--p2", required=True)
    ap.add_argument("--warmup", type=int, required=True)
    ap.add_argument("--steps", type=int, required=True)
    ap.add_argument("--rates", default="4,2")
    ap.add_argument("--command", default="")
    ap.add_argument("--out", default=SUMMARY)
    a = ap.parse_args()
    rates = [float(r) for r in a.rates.split(",")]
    s = summarize(a.p1, a.p2, a.warmup, a.steps, rates)
    write_summary(s, a.out, a.command, a.warmup, a.steps, rates)
    print(f"copy: raw read {s['copy']['raw_read'] / 2**20:.1f} MiB, write "
          f"{s['copy']['raw_write'] / 2**20:.1f} MiB, dram {s['copy']['raw_dram'] / 2**20:.1f} MiB "
          f"(512 MiB each)")
    for rk, ent in s["rates"].items():
        for mode, m in ent.items():
            print(f"{rk} {mode}: step read {m['step_read_bytes'] / 1e6:.1f} MB write "
                  f"{m['step_write_bytes'] / 1e6:.1f} MB; " +
                  ", ".join(f"{n} {k['read_bytes'] / 1e6:.1f}/{k['write_bytes'] / 1e6:.1f}"
                            for n, k in m["kernels"].items()))


if __name__ == "__main__":
    main()
