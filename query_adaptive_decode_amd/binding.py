"""Thin ctypes binding of libreadkv.so (the C ABI in include/readkv.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the computation runs in the library's
kernels.  There is no fallback: if the library is missing, or a call
fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libreadkv.so")

BF16, F32 = 0, 1
VSCALE_PHYSICAL, VSCALE_UNIT = 0, 1
SCOPE_KV_HEAD, SCOPE_LAYER = 0, 1
RESTRICT_MIN_DEPTH1, RESTRICT_VALUE_PAIRS = 0x10, 0x20   # OR'ed into a policy
SINGLE_LAUNCH = 0x40   # OR'ed into a policy: the whole step as one cooperative launch
NUM_COUNTERS = 4   # key payload, value payload, metadata, open group (bits)
CODEC_UNIFORM, CODEC_LLOYD = 0, 1
FLAG_NONFINITE, FLAG_OVERFLOW = 1, 2

EXPORTED = ["readkv_validate_config", "readkv_store_bytes", "readkv_workspace_bytes",
            "readkv_store_init", "readkv_encode_append", "readkv_decode_attn",
            "readkv_decode_attn_timed", "readkv_decode_attn_noalloc", "readkv_store_status",
            "readkv_strerror", "readkv_codec_init", "readkv_codec_tables"]


class Config(ctypes.Structure):
    _fields_ = [("W", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("group_tokens", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("capacity_tokens", ctypes.c_int64), ("kv_dtype", ctypes.c_int32),
                ("codec", ctypes.c_int32)]


class ReadKVError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed: {msg} ({code})")
        self.code = code


_lib = None


def lib():
    """Load libreadkv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m query_adaptive_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        CP = ctypes.POINTER(Config)
        sig = {
            "readkv_validate_config": [CP],
            "readkv_store_bytes": [CP, P, ctypes.POINTER(SZ)],
            "readkv_workspace_bytes": [CP, ctypes.POINTER(SZ)],
            "readkv_store_init": [CP, P, SZ, P, P],
            "readkv_encode_append": [CP, P, P, P, P, I32, P],
            "readkv_decode_attn": [CP, P, P, ctypes.c_float, ctypes.c_float, I32, I32,
                                   P, P, SZ, P, P, P, P],
            "readkv_decode_attn_timed": [CP, P, P, ctypes.c_float, ctypes.c_float, I32, I32,
                                         P, P, SZ, P, P, P, P, P],
            "readkv_decode_attn_noalloc": [CP, P, P, ctypes.c_float, ctypes.c_float, I32, I32,
                                           P, P, P, P, P],
            "readkv_store_status": [CP, P, ctypes.POINTER(ctypes.c_uint32), P],
            "readkv_codec_init": [CP, P, P, P, P, P, I64, P],
            "readkv_codec_tables": [P, P, P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.readkv_strerror.argtypes = [ctypes.c_int]
        L.readkv_strerror.restype = ctypes.c_char_p
        _ = I64
        _lib = L
    return _lib


def _check(fn, rc):
    if rc != 0:
        raise ReadKVError(fn, rc, lib().readkv_strerror(rc).decode())


def make_config(W=8, head_dim=128, num_q_heads=32, num_kv_heads=8, batch=1,
                capacity_tokens=1024, kv_dtype=BF16, group_tokens=32, codec=CODEC_UNIFORM) -> Config:
    return Config(W, head_dim, num_q_heads, num_kv_heads, group_tokens, batch,
                  capacity_tokens, kv_dtype, codec)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _caps(cfg, req_capacity):
    if req_capacity is None:
        return None, None
    arr = (ctypes.c_int64 * cfg.batch)(*[int(x) for x in req_capacity])
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def validate_config(cfg: Config) -> int:
    return lib().readkv_validate_config(ctypes.byref(cfg))


def store_bytes(cfg: Config, req_capacity=None) -> int:
    n = ctypes.c_size_t()
    keep, p = _caps(cfg, req_capacity)
    _check("readkv_store_bytes", lib().readkv_store_bytes(ctypes.byref(cfg), p, ctypes.byref(n)))
    return n.value


def workspace_bytes(cfg: Config) -> int:
    n = ctypes.c_size_t()
    _check("readkv_workspace_bytes", lib().readkv_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("expected contiguous device tensors")


def store_init(cfg: Config, store: torch.Tensor, req_capacity=None):
    _need_cuda(store)
    keep, p = _caps(cfg, req_capacity)
    _check("readkv_store_init", lib().readkv_store_init(
        ctypes.byref(cfg), _ptr(store), store.numel() * store.element_size(), p, _stream()))


def codec_init(cfg: Config, store, signs_k, signs_v, k_cal, v_cal):
    """Lloyd code: set the transform signs (host int8 sequences of +-1, or
    None) and calibrate from device tensors k_cal, v_cal [n][G][d] in the
    config's dtype.  Synchronises the stream."""
    _need_cuda(store, k_cal, v_cal)

    def signs(s):
        if s is None:
            return None, None
        arr = (ctypes.c_int8 * cfg.head_dim)(*[int(x) for x in s])
        return arr, ctypes.cast(arr, ctypes.c_void_p)
    ka, kp = signs(signs_k)
    va, vp = signs(signs_v)
    _check("readkv_codec_init", lib().readkv_codec_init(
        ctypes.byref(cfg), _ptr(store), kp, vp, _ptr(k_cal), _ptr(v_cal), int(k_cal.shape[0]),
        _stream()))


def codec_tables():
    """The library's Lloyd-tree table: (centroids float32 [511], boundaries
    float64 [255], gains float64 [9]) as Python lists.  Host only."""
    cent = (ctypes.c_float * 511)()
    bnd = (ctypes.c_double * 255)()
    gains = (ctypes.c_double * 9)()
    _check("readkv_codec_tables", lib().readkv_codec_tables(
        ctypes.cast(cent, ctypes.c_void_p), ctypes.cast(bnd, ctypes.c_void_p),
        ctypes.cast(gains, ctypes.c_void_p)))
    return list(cent), list(bnd), list(gains)


def encode_append(cfg: Config, store, k_new, v_new, n_new=None, n_max=None):
    """k_new, v_new: [B][G][n_max][d] device tensors in the config's dtype
    (bf16 or fp32); n_new: optional int32 device tensor [B]."""
    _need_cuda(store, k_new, v_new, n_new)
    if n_max is None:
        n_max = k_new.shape[2]
    _check("readkv_encode_append", lib().readkv_encode_append(
        ctypes.byref(cfg), _ptr(store), _ptr(k_new), _ptr(v_new), _ptr(n_new),
        int(n_max), _stream()))


def _out(cfg, q, out):
    if out is None:
        out = torch.empty((cfg.batch, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32,
                          device=q.device)
    return out


def decode_attn(cfg: Config, store, q, R_K, R_V, workspace, out=None,
                vscale=VSCALE_PHYSICAL, key_depths=None, value_depths=None,
                policy=SCOPE_KV_HEAD, counters=None):
    """q: [B][H][d] device tensor in the config's dtype.  Returns out
    [B][H][d] fp32.  policy: a budget scope OR'ed with RESTRICT_* flags
    and SINGLE_LAUNCH.
    counters: optional int64 device tensor of NUM_COUNTERS entries,
    overwritten with the call's logical reads in bits."""
    out = _out(cfg, q, out)
    _need_cuda(store, q, out, workspace, key_depths, value_depths, counters)
    _check("readkv_decode_attn", lib().readkv_decode_attn(
        ctypes.byref(cfg), _ptr(store), _ptr(q), float(R_K), float(R_V), int(policy),
        int(vscale), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(key_depths), _ptr(value_depths), _ptr(counters), _stream()))
    return out


def decode_attn_timed(cfg: Config, store, q, R_K, R_V, workspace, events, out=None,
                      vscale=VSCALE_PHYSICAL, key_depths=None, value_depths=None,
                      policy=SCOPE_KV_HEAD, counters=None):
    """decode_attn that records four caller-created hipEvent_t handles
    (``events``: sequence of ints) around its three stages (score, value
    allocation, value gather)."""
    out = _out(cfg, q, out)
    _need_cuda(store, q, out, workspace, key_depths, value_depths, counters)
    ev = (ctypes.c_void_p * 4)(*[int(e) for e in events])
    _check("readkv_decode_attn_timed", lib().readkv_decode_attn_timed(
        ctypes.byref(cfg), _ptr(store), _ptr(q), float(R_K), float(R_V), int(policy),
        int(vscale), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(key_depths), _ptr(value_depths), _ptr(counters), ctypes.cast(ev, ctypes.c_void_p),
        _stream()))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20


def decode_attn_noalloc(cfg: Config, store, q, R_K, R_V, out, vscale=VSCALE_PHYSICAL,
                        key_depths=None, value_depths=None, policy=SCOPE_KV_HEAD, counters=None):
    """decode_attn without a workspace: the library's fixed per-GPU scratch
    is used, nothing is allocated (``out`` must be given)."""
    _need_cuda(store, q, out, key_depths, value_depths, counters)
    _check("readkv_decode_attn_noalloc", lib().readkv_decode_attn_noalloc(
        ctypes.byref(cfg), _ptr(store), _ptr(q), float(R_K), float(R_V), int(policy),
        int(vscale), _ptr(out), _ptr(key_depths), _ptr(value_depths), _ptr(counters),
        _stream()))
    return out


def store_status(cfg: Config, store):
    flags = ctypes.c_uint32()
    lens = (ctypes.c_int64 * cfg.batch)()
    _check("readkv_store_status", lib().readkv_store_status(
        ctypes.byref(cfg), _ptr(store), ctypes.byref(flags), ctypes.cast(lens, ctypes.c_void_p)))
    return flags.value, list(lens)


class ReadKVCache:
    """A store plus a workspace in device memory, with the library's calls."""

    def __init__(self, cfg: Config, device="cuda", req_capacity=None):
        self.cfg = cfg
        self.store = torch.empty(store_bytes(cfg, req_capacity), dtype=torch.uint8, device=device)
        self.workspace = torch.empty(workspace_bytes(cfg), dtype=torch.uint8, device=device)
        store_init(cfg, self.store, req_capacity)

    def append(self, k_new, v_new, n_new=None, n_max=None):
        encode_append(self.cfg, self.store, k_new, v_new, n_new, n_max)

    def decode(self, q, R_K, R_V, out=None, vscale=VSCALE_PHYSICAL, key_depths=None,
               value_depths=None, policy=SCOPE_KV_HEAD, counters=None):
        return decode_attn(self.cfg, self.store, q, R_K, R_V, self.workspace, out, vscale,
                           key_depths, value_depths, policy, counters)

    def status(self):
        return store_status(self.cfg, self.store)
