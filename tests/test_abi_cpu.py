"""CPU-side checks of the C-ABI library: it loads, exports every declared
symbol, and its host-only entry points validate arguments and size buffers
as the header documents.  No GPU work is launched here."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "readkv.h")


def _lib_or_skip():
    from query_adaptive_decode_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libreadkv.so not built (run __graft_entry__.build())")
    return binding


def declared_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(readkv_\w+)\(", txt, re.M)))


def test_header_compiles_as_c():
    src = '#include "readkv.h"\nint main(void){readkv_config c; (void)c; return 0;}\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                        "-x", "c", "-", "-fsyntax-only"], input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_library_exports_every_declared_symbol():
    b = _lib_or_skip()
    decl = declared_functions()
    assert set(decl) == set(b.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", b.LIB_PATH], capture_output=True,
                         text=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in decl:
        assert name in syms, name
        getattr(b.lib(), name)


def test_config_validation_codes():
    b = _lib_or_skip()
    ok = b.make_config(num_q_heads=32, num_kv_heads=8, batch=4, capacity_tokens=8192)
    assert b.validate_config(ok) == 0
    cases = {
        -1: [dict(W=0), dict(W=9), dict(num_q_heads=30, num_kv_heads=8), dict(batch=0),
             dict(capacity_tokens=0), dict(num_kv_heads=0), dict(capacity_tokens=(1 << 26) + 1),
             dict(codec=2), dict(codec=-1)],
        -4: [dict(kv_dtype=7)],
        -5: [dict(head_dim=64), dict(group_tokens=16), dict(num_q_heads=80, num_kv_heads=8)],
    }
    for code, variants in cases.items():
        for v in variants:
            kw = dict(num_q_heads=32, num_kv_heads=8, batch=4, capacity_tokens=8192)
            kw.update(v)
            assert b.validate_config(b.make_config(**kw)) == code, v
    assert b.lib().readkv_validate_config(None) == -1
    assert b.lib().readkv_strerror(-2).decode() == "append larger than the store capacity"


def test_store_size_matches_format_description():
    b = _lib_or_skip()
    from oracle import store_format as F
    for (B, H, G, cap, dt) in [(1, 1, 1, 1024, 1), (16, 32, 8, 8320, 0), (3, 28, 4, 100, 0)]:
        cfg = b.make_config(num_q_heads=H, num_kv_heads=G, batch=B, capacity_tokens=cap, kv_dtype=dt)
        caps = [cap - 7 * i for i in range(B)]
        for rc in (None, caps):
            want = F.header_bytes(B)
            for i in range(B):
                c = cap if rc is None else rc[i]
                c = (c + 31) // 32 * 32
                want += F.region_layout(G, 128, 8, c, 2 if dt == 0 else 4)["_size"]
            assert b.store_bytes(cfg, rc) == want
    cfg = b.make_config(batch=2, capacity_tokens=64)
    with pytest.raises(b.ReadKVError):
        b.store_bytes(cfg, [64, 65])           # above capacity_tokens
    assert b.workspace_bytes(cfg) > 0
    # the Lloyd code: a codec block between the header and the regions
    for (B, G, cap) in [(1, 1, 1024), (16, 8, 8320)]:
        c0 = b.make_config(num_q_heads=4 * G, num_kv_heads=G, batch=B, capacity_tokens=cap)
        c1 = b.make_config(num_q_heads=4 * G, num_kv_heads=G, batch=B, capacity_tokens=cap,
                           codec=b.CODEC_LLOYD)
        assert b.store_bytes(c1) == b.store_bytes(c0) + F.codec_block_bytes(G, 128)
        # logits (8 bytes per token and query head) in place of exponentials (4)
        assert b.workspace_bytes(c1) >= b.workspace_bytes(c0) + B * 4 * G * cap * 4


def test_lloyd_tree_table_equals_the_oracles():
    """The library builds the tree on the host in its own code; its float32
    centroids, boundaries and gains equal the oracle's bit for bit."""
    b = _lib_or_skip()
    import numpy as np
    from oracle import lloyd as L
    cent, bnd, gains = b.codec_tables()
    T = L.lloyd_tree()
    assert np.array_equal(np.array(cent, dtype=np.float64), T.flat_centroids32())
    assert np.array_equal(np.array(bnd), np.concatenate([T.bounds[t] for t in range(8)]))
    assert np.array_equal(np.array(gains), T.gains32)


def test_codec_init_rejects_bad_arguments():
    b = _lib_or_skip()
    cfg = b.make_config(num_q_heads=8, num_kv_heads=2, batch=1, capacity_tokens=64)
    P = ctypes.c_void_p
    fake = P(0x1000)
    # a uniform-code store, then a Lloyd store with bad signs / sizes: all
    # rejected on the host before any device access
    assert b.lib().readkv_codec_init(ctypes.byref(cfg), fake, None, None, fake, fake, 8, None) == -1
    cl = b.make_config(num_q_heads=8, num_kv_heads=2, batch=1, capacity_tokens=64,
                       codec=b.CODEC_LLOYD)
    bad = (ctypes.c_int8 * 128)(*([1] * 127 + [0]))
    assert b.lib().readkv_codec_init(ctypes.byref(cl), fake, ctypes.cast(bad, P), None, fake, fake,
                                     8, None) == -1
    assert b.lib().readkv_codec_init(ctypes.byref(cl), fake, None, None, fake, fake, 0, None) == -1
    assert b.lib().readkv_codec_init(ctypes.byref(cl), fake, None, None, None, fake, 8, None) == -1


def test_entry_points_reject_bad_arguments_before_launch():
    b = _lib_or_skip()
    L = b.lib()
    cfg = b.make_config(batch=2, capacity_tokens=256)
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: every call below fails its host checks
    by = ctypes.byref(cfg)
    assert L.readkv_encode_append(by, None, fake, fake, None, 4, None) == -1
    assert L.readkv_encode_append(by, fake, fake, fake, None, -1, None) == -1
    assert L.readkv_encode_append(by, fake, fake, fake, None, 257, None) == -2
    assert L.readkv_encode_append(by, fake, None, fake, None, 4, None) == -1
    ws = b.workspace_bytes(cfg)
    dec = L.readkv_decode_attn

    def call(cfgp=by, store=fake, rk=1.0, rv=1.0, scope=0, vscale=0, wsb=ws):
        return dec(cfgp, store, fake, rk, rv, scope, vscale, fake, fake, wsb, None, None, None, None)

    assert call(scope=0x2) == -1 and call(scope=0x80) == -1   # unknown policy bits
    # the single-launch reader: per-KV-head budgets and the uniform code only
    assert call(scope=b.SCOPE_LAYER | b.SINGLE_LAUNCH) == -5
    lloyd = b.make_config(batch=2, capacity_tokens=256, codec=b.CODEC_LLOYD)
    assert call(cfgp=ctypes.byref(lloyd), scope=b.SINGLE_LAUNCH, wsb=b.workspace_bytes(lloyd)) == -5
    assert call(scope=b.SINGLE_LAUNCH | b.RESTRICT_MIN_DEPTH1, rk=float("nan")) == -1

    for rk, rv in [(float("nan"), 1.0), (1.0, float("inf")), (-0.5, 1.0), (1.0, -1.0)]:
        assert call(rk=rk, rv=rv) == -1
    assert call(vscale=5) == -1
    assert call(scope=2) == -1 and call(scope=-1) == -1
    many = b.make_config(num_q_heads=66, num_kv_heads=33, batch=2, capacity_tokens=256)
    assert call(cfgp=ctypes.byref(many), scope=1, wsb=b.workspace_bytes(many)) == -5   # pooling over > 32 KV heads
    assert call(wsb=ws - 1) == -3
    assert call(store=None) == -1
    assert L.readkv_store_init(by, fake, 16, None, None) == -3
    bad = b.make_config(batch=2, capacity_tokens=256, head_dim=64)
    assert call(cfgp=ctypes.byref(bad)) == -5
    # the allocation-free entry point refuses a workspace need above its
    # fixed scratch before touching a device
    big = b.make_config(num_q_heads=32, num_kv_heads=8, batch=64, capacity_tokens=32768)
    assert b.workspace_bytes(big) > b.NOALLOC_SCRATCH_BYTES
    assert L.readkv_decode_attn_noalloc(ctypes.byref(big), fake, fake, 1.0, 1.0, 0, 0, fake, None, None,
                                        None, None) == -7
    assert L.readkv_decode_attn_noalloc(ctypes.byref(bad), fake, fake, 1.0, 1.0, 0, 0, fake, None, None,
                                        None, None) == -5
    assert "fixed scratch" in L.readkv_strerror(-7).decode()
    ev = (ctypes.c_void_p * 4)(fake, fake, None, fake)
    assert L.readkv_decode_attn_timed(by, fake, fake, 1.0, 1.0, 0, 0, fake, fake, ws, None, None, None,
                                      ctypes.cast(ev, ctypes.c_void_p), None) == -1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from query_adaptive_decode_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()
