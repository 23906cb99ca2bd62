"""Build the HIP library libreadkv.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libreadkv.so")
SOURCES = ["abi.hip", "codec.hip", "encode.hip", "alloc.hip", "decode.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source to an object (in parallel) and link the shared
    library.  Always recompiles."""
    os.makedirs(LIBDIR, exist_ok=True)
    cc = hipcc()
    objs, procs = [], []
    for s in SOURCES:
        obj = os.path.join(LIBDIR, s.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, s), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    errs = []
    for s, p in procs:
        out, _ = p.communicate()
        txt = out.decode(errors="replace")
        # hipcc's host pass does not know the gfx feature flag; that warning is harmless
        txt = "\n".join(ln for ln in txt.splitlines() if "packed-fp32-ops" not in ln
                        and "not a recognized feature" not in ln)
        if p.returncode != 0:
            errs.append(f"--- {s} ---\n{txt}")
        elif verbose and txt.strip():
            print(txt)
    if errs:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
