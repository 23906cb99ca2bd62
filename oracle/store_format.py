"""Byte layout of the packed KV store, written from its format description.

TEST INFRASTRUCTURE ONLY.  Used to turn the oracle's encoded streams into the
store's bytes (for bit-exact comparison with what the device encoder wrote)
and to read a device store back.  Shares no code with the device library.

Layout (all little-endian; every sub-array starts on a 256-byte boundary):

header (align_up(256 + 32*B, 4096) bytes)
  u32 magic 0x52564B31, u32 version 1, i32 W, i32 d, i32 H, i32 G,
  i32 group_tokens, i32 B, i32 kv_dtype (0 bf16, 1 f32), u32 flags,
  i64 capacity, i64 total_bytes, i32 codec (0 uniform, 1 Lloyd tree);
  at 256 + 32*b: i64 len, i64 cap, i64 offset, i64 reserved  for request b.
codec block (Lloyd tree only, right after the header; 256-byte aligned
  parts, total rounded up to 4096):
  cent   f32 [512]   centroid of depth-t cell P at 2^t - 1 + P (t = 0..8)
  bounds f64 [256]   boundary of depth-t cell P at 2^t - 1 + P (t = 0..7)
  gains  f64 [16]    Delta_t at t = 1..8
  sk, sv f64 [d]     transform signs
  vtab   f16 [9][256]  entry (t, X): centroid of depth-t cell X >> (8 - t)
  muk, sigk, muv, sigv f32 [G][d];  sphys f64 [G]
  (the first five parts are packed back to back, vtab then padded to 256)
request region b (cap = cap_b, a multiple of 32; ng = cap/32):
  Kplanes u32 [G][ntk][d][W][16]  bit i of word (g,tau,c,p,k) = plane p
                              (bit W-1-p of the code) of token
                              32*(16*tau+k)+i, channel c; ntk = ng/16
                              rounded up (tiles of 16 groups)
  Vplanes u32 [G][cap][W][d/32]  bit (c%32) of word (g,j,p,c/32) = plane p
                              of token j, channel c
  Kmeta   u32 [G][ng][d]      lo bf16 bits | rng bf16 bits << 16
  Vmeta   u32 [G][ng][d]
  EK      f64 [G][d]          sum over closed groups (in order) of rng_K^2
  EV      f64 [G][ng]         sum over channels (in order) of rng_V^2
  Ktail   elem [G][32][d]     open-group keys (slot i = token 32*floor(len/32)+i)
  Vtail   elem [G][32][d]
"""
from __future__ import annotations

import numpy as np

MAGIC = 0x52564B31


def _al(x: int, a: int) -> int:
    return (x + a - 1) // a * a


def header_bytes(B: int) -> int:
    return _al(256 + 32 * B, 4096)


def region_layout(G: int, d: int, W: int, cap: int, esize: int) -> dict:
    """Byte offsets (relative to the region start) and sizes of each
    sub-array of one request region."""
    ng = cap // 32
    ntk = (ng + 15) // 16
    parts = [
        ("Kplanes", G * ntk * d * W * 16 * 4),
        ("Vplanes", G * cap * W * (d // 32) * 4),
        ("Kmeta", G * ng * d * 4),
        ("Vmeta", G * ng * d * 4),
        ("EK", G * d * 8),
        ("EV", G * ng * 8),
        ("Ktail", G * 32 * d * esize),
        ("Vtail", G * 32 * d * esize),
    ]
    off = 0
    lay = {}
    for name, size in parts:
        off = _al(off, 256)
        lay[name] = (off, size)
        off += size
    lay["_size"] = _al(off, 4096)
    return lay


def codec_block_bytes(G: int, d: int) -> int:
    return _codec_parts(G, d)["_size"]


def _codec_parts(G: int, d: int) -> dict:
    off = 0
    lay = {}
    for name, size in [("cent", 512 * 4), ("bounds", 256 * 8), ("gains", 16 * 8),
                       ("sk", d * 8), ("sv", d * 8), ("vtab", 9 * 256 * 2)]:
        lay[name] = (off, size)
        off += size
    for name, size in [("muk", G * d * 4), ("sigk", G * d * 4), ("muv", G * d * 4),
                       ("sigv", G * d * 4), ("sphys", G * 8)]:
        off = _al(off, 256) if name == "muk" else off
        lay[name] = (off, size)
        off += size
    lay["_size"] = _al(off, 4096)
    return lay


def codec_block(codec, G: int, d: int) -> np.ndarray:
    """The bytes of a Lloyd-tree store's codec block for the oracle's codec
    state (oracle.lloyd.Codec with calibration arrays of G KV heads)."""
    lay = _codec_parts(G, d)
    out = np.zeros(lay["_size"], dtype=np.uint8)

    def put(name, arr):
        o, n = lay[name]
        raw = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        assert raw.size <= n
        out[o:o + raw.size] = raw

    T = codec.tree
    cent = np.zeros(512, dtype=np.float32)
    cent[:511] = T.flat_centroids32().astype(np.float32)
    put("cent", cent)
    bnd = np.zeros(256)
    bnd[:255] = np.concatenate([T.bounds[t] for t in range(8)])
    put("bounds", bnd)
    gains = np.zeros(16)
    gains[:9] = T.gains32
    put("gains", gains)
    ones = np.ones(d)
    put("sk", ones if codec.sK is None else np.asarray(codec.sK, dtype=np.float64))
    put("sv", ones if codec.sV is None else np.asarray(codec.sV, dtype=np.float64))
    vt = np.zeros((9, 256), dtype=np.float16)
    flat = T.flat_centroids32()
    for t in range(9):
        vt[t] = flat[(1 << t) - 1 + (np.arange(256) >> (8 - t))].astype(np.float32).astype(np.float16)
    put("vtab", vt)
    put("muk", np.asarray(codec.muK, dtype=np.float32))
    put("sigk", np.asarray(codec.sigK, dtype=np.float32))
    put("muv", np.asarray(codec.muV, dtype=np.float32))
    put("sigv", np.asarray(codec.sigV, dtype=np.float32))
    put("sphys", np.array([codec.s_phys(g) for g in range(G)]))
    return out


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint32)


def pack_unit(enc_k, enc_v, cap: int, dtype: str) -> dict:
    """Arrays one (request, KV head) unit occupies in a request region of
    capacity ``cap`` tokens, for the oracle's encoded key/value streams."""
    W = enc_k.W
    tp, d = enc_k.codes.shape
    ng = cap // 32
    ngc = enc_k.n_groups
    ntk = (ng + 15) // 16
    kpl = np.zeros((ntk, d, W, 16), dtype=np.uint32)
    ck = enc_k.codes.reshape(ngc, 32, d)
    for p in range(W):
        bits = ((ck >> (W - 1 - p)) & 1).astype(np.uint64)       # [ngc][32][d]
        word = (bits << np.arange(32, dtype=np.uint64)[None, :, None]).sum(axis=1)  # [ngc][d]
        for gam in range(ngc):
            kpl[gam // 16, :, p, gam % 16] = word[gam].astype(np.uint32)
    vpl = np.zeros((cap, W, d // 32), dtype=np.uint32)
    for p in range(W):
        bits = ((enc_v.codes >> (W - 1 - p)) & 1).astype(np.uint64)  # [tp][d]
        bits = bits.reshape(tp, d // 32, 32)
        word = (bits << np.arange(32, dtype=np.uint64)[None, None, :]).sum(axis=2)
        vpl[:tp, p, :] = word.astype(np.uint32)

    def meta(enc):
        m = np.zeros((ng, d), dtype=np.uint32)
        m[:ngc] = _bf16_bits(enc.lo) | (_bf16_bits(enc.rng) << 16)
        return m

    ek = np.zeros(d)
    for gam in range(ngc):
        ek = ek + enc_k.rng[gam] * enc_k.rng[gam]
    ev = np.zeros(ng)
    for c in range(d):
        ev[:ngc] = ev[:ngc] + enc_v.rng[:, c] * enc_v.rng[:, c]

    def tail(enc):
        r = enc.tail.shape[0]
        if dtype == "bf16":
            t = np.zeros((32, d), dtype=np.uint16)
            t[:r] = _bf16_bits(enc.tail).astype(np.uint16)
        else:
            t = np.zeros((32, d), dtype=np.float32)
            t[:r] = enc.tail.astype(np.float32)
        return t

    return dict(Kplanes=kpl, Vplanes=vpl, Kmeta=meta(enc_k), Vmeta=meta(enc_v),
                EK=ek, EV=ev, Ktail=tail(enc_k), Vtail=tail(enc_v))


def read_header(buf: np.ndarray) -> dict:
    """Parse the store header from raw bytes (uint8 array)."""
    b = np.asarray(buf, dtype=np.uint8)
    u32 = b[:64].view(np.uint32)
    i32 = b[:64].view(np.int32)
    i64 = b[:64].view(np.int64)
    hdr = dict(magic=int(u32[0]), version=int(u32[1]), W=int(i32[2]), d=int(i32[3]),
               H=int(i32[4]), G=int(i32[5]), group_tokens=int(i32[6]),
               B=int(i32[7]), kv_dtype=int(i32[8]), flags=int(u32[9]),
               capacity=int(i64[5]), codec=int(i32[14]))
    reqs = []
    for r in range(hdr["B"]):
        rec = b[256 + 32 * r: 256 + 32 * r + 32].view(np.int64)
        reqs.append(dict(len=int(rec[0]), cap=int(rec[1]), offset=int(rec[2])))
    hdr["requests"] = reqs
    return hdr


def unpack_unit(buf: np.ndarray, hdr: dict, b: int, g: int) -> dict:
    """The arrays of unit (b, g) from raw store bytes."""
    G, d, W = hdr["G"], hdr["d"], hdr["W"]
    req = hdr["requests"][b]
    cap = req["cap"]
    ng = cap // 32
    esize = 2 if hdr["kv_dtype"] == 0 else 4
    lay = region_layout(G, d, W, cap, esize)
    base = req["offset"]

    def sub(name, dt, shape):
        off, size = lay[name]
        per = size // G
        raw = np.asarray(buf[base + off + g * per: base + off + (g + 1) * per], dtype=np.uint8)
        return raw.view(dt).reshape(shape)

    edt = np.uint16 if esize == 2 else np.float32
    return dict(
        Kplanes=sub("Kplanes", np.uint32, ((ng + 15) // 16, d, W, 16)),
        Vplanes=sub("Vplanes", np.uint32, (cap, W, d // 32)),
        Kmeta=sub("Kmeta", np.uint32, (ng, d)),
        Vmeta=sub("Vmeta", np.uint32, (ng, d)),
        EK=sub("EK", np.float64, (d,)),
        EV=sub("EV", np.float64, (ng,)),
        Ktail=sub("Ktail", edt, (32, d)),
        Vtail=sub("Vtail", edt, (32, d)),
    )
