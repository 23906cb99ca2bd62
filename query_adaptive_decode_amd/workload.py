"""Device-resident inputs for a decode workload: prefill keys/values, the
token appended at every step, and every step's queries, drawn by
``synth`` and uploaded once.  Data movement only."""
from __future__ import annotations

import numpy as np
import torch

from . import synth
from .binding import BF16, CODEC_LLOYD, CODEC_UNIFORM, F32, make_config


def config_for(cfg: dict, steps: int | None = None):
    """Library config for a workload: capacity = longest prefill + steps.
    ``cfg["codec"] == "lloyd"`` selects the Lloyd-tree code."""
    steps = cfg["steps"] if steps is None else steps
    cap = int(synth.context_lengths(cfg).max()) + int(steps)
    return make_config(W=cfg["W"], head_dim=cfg["d"], num_q_heads=cfg["H"],
                       num_kv_heads=cfg["G"], batch=cfg["B"], capacity_tokens=cap,
                       kv_dtype=BF16 if cfg["dtype"] == "bf16" else F32,
                       codec=CODEC_LLOYD if cfg.get("codec") == "lloyd" else CODEC_UNIFORM)


def calibration_inputs(cfg: dict, n: int):
    """The Lloyd code's inputs in upload form: (signs_k, signs_v) int8 [d]
    and the calibration split kcal, vcal [n][G][d]."""
    sk, sv = synth.codec_signs(cfg)
    edt = np.uint16 if cfg["dtype"] == "bf16" else np.float32
    kc = np.zeros((n, cfg["G"], cfg["d"]), dtype=edt)
    vc = np.zeros((n, cfg["G"], cfg["d"]), dtype=edt)
    for g in range(cfg["G"]):
        K, V = synth.calibration_split(cfg, g, n)
        kc[:, g] = synth.to_device_bits(cfg, K)
        vc[:, g] = synth.to_device_bits(cfg, V)
    return dict(sk=sk, sv=sv, kcal=kc, vcal=vc)


def host_inputs(cfg: dict, steps: int | None = None) -> dict:
    """numpy arrays in upload form (uint16 bf16 bits or float32):
    kpre/vpre [B][G][T0max][d], npre [B], kstep/vstep [steps][B][G][1][d],
    q [steps][B][H][d]."""
    steps = cfg["steps"] if steps is None else steps
    B, H, G, d = cfg["B"], cfg["H"], cfg["G"], cfg["d"]
    T0 = synth.context_lengths(cfg)
    T0max = int(T0.max())
    edt = np.uint16 if cfg["dtype"] == "bf16" else np.float32
    kpre = np.zeros((B, G, T0max, d), dtype=edt)
    vpre = np.zeros((B, G, T0max, d), dtype=edt)
    kst = np.zeros((steps, B, G, 1, d), dtype=edt)
    vst = np.zeros((steps, B, G, 1, d), dtype=edt)
    for b in range(B):
        n0 = int(T0[b])
        for g in range(G):
            K, V = synth.kv_unit(cfg, b, g, n0 + steps)
            kpre[b, g, :n0] = synth.to_device_bits(cfg, K[:n0])
            vpre[b, g, :n0] = synth.to_device_bits(cfg, V[:n0])
            kst[:, b, g, 0] = synth.to_device_bits(cfg, K[n0:n0 + steps])
            vst[:, b, g, 0] = synth.to_device_bits(cfg, V[n0:n0 + steps])
    q = np.zeros((steps, B, H, d), dtype=edt)
    for s in range(steps):
        for b in range(B):
            q[s, b] = synth.to_device_bits(cfg, synth.q_step(cfg, b, s))
    return dict(kpre=kpre, vpre=vpre, npre=T0.astype(np.int32), kstep=kst, vstep=vst, q=q)


def to_device(h: dict, device="cuda") -> dict:
    out = {}
    for k, v in h.items():
        t = torch.from_numpy(np.ascontiguousarray(v))
        if v.dtype == np.uint16:
            t = t.view(torch.int16).view(torch.bfloat16)
        out[k] = t.to(device)
    return out
