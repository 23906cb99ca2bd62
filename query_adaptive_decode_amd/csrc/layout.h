// Store and workspace layout shared by the host entry points and the kernels.
//
// Store = header + (Lloyd-tree code only) codec block + one region per
// request.  Header: 256 bytes of fields, then one 32-byte record {len, cap,
// offset, ticket} per request (ticket: the append's completion counter, zero
// between calls), rounded up to 4096 bytes.  The codec block (see
// codec_layout) follows the header.  A request region with capacity `cap` tokens
// (multiple of 32, ng = cap/32 groups) holds, each sub-array 256-byte
// aligned:
//   Kplanes u32 [G][ntk][d][W][16] token-packed, tile-major: bit i of word
//                                  (g,tau,c,p,k) is plane p of token
//                                  32*(16 tau + k) + i, channel c; ntk =
//                                  ceil(ng/16) tiles of 512 tokens.  A
//                                  channel's depth-t prefix over one tile is
//                                  t*64 contiguous bytes (planes 2k, 2k+1
//                                  share a 128 B line)
//   Vplanes u32 [G][cap][W][d/32]  channel-packed: a token's t-plane prefix
//                                  is t*d/8 contiguous bytes
//   Kmeta   u32 [G][ng][d]         lo bf16 | rng bf16 << 16
//   Vmeta   u32 [G][ng][d]
//   EK      f64 [G][d]             sum over closed groups of rng_K^2
//   EV      f64 [G][ng]            per group: sum over channels of rng_V^2
//   Ktail   elem [G][32][d]        open group, exact input values
//   Vtail   elem [G][32][d]
// Plane p holds bit (W-1-p) of the code (most significant first), so a
// depth-t read of a key channel is t whole lines and a depth-t read of a
// value token is one contiguous run.  Under the Lloyd-tree code the code is
// the scalar's tree path and Kmeta, Vmeta, EK and EV are not used.
#pragma once
#include <stdint.h>

#ifdef __HIPCC__
#define RKV_HD __host__ __device__ __forceinline__
#else
#define RKV_HD inline
#endif

namespace readkv {

constexpr uint32_t kMagic = 0x52564B31u;
constexpr uint32_t kVersion = 1u;
constexpr int kGroup = 32;      // tokens per quantiser group
constexpr int kDim = 128;       // head_dim supported by the kernels
constexpr int kTile = 256;      // tokens per score tile (8 groups, half of a
                                // key-plane tile); also the softmax
                                // split-context unit
constexpr int kChunk = 128;     // tokens per value-gather step (4 groups)

struct StoreHeader {          // first 256 bytes of a store
  uint32_t magic, version;
  int32_t W, d, H, G, group_tokens, B, kv_dtype;
  uint32_t flags;
  int64_t capacity, total_bytes;
  int32_t codec, reserved0;   // 0: uniform min/max code, 1: Lloyd tree
  int64_t reserved[24];
};
static_assert(sizeof(StoreHeader) == 256, "header size");

struct ReqRecord {            // at byte 256 + 32*b
  int64_t len, cap, offset, reserved;
};

RKV_HD int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

RKV_HD int64_t header_bytes(int B) { return align_up(256 + 32 * (int64_t)B, 4096); }

// Codec block of a Lloyd-tree store, at byte header_bytes(B):
//   cent   f32 [512]     centroid of depth-t cell P at (2^t - 1) + P, t = 0..8
//   bounds f64 [256]     boundary splitting depth-t cell P at (2^t - 1) + P,
//                        t = 0..7 (midpoint of the float32 child centroids)
//   gains  f64 [16]      gains[t] = Delta_t (float32 values), t = 1..8
//   sk, sv f64 [d]       signs of the key and value Hadamard-sign transforms
//   vtab   f16 [9][256]  vtab[t][X] = cent of depth-t cell X >> (8 - t)
//                        (X = an 8-bit code with its bits past depth t zero)
//   muk, sigk, muv, sigv f32 [G][d]   calibration means and scales
//   sphys  f64 [G]       sum over channels of sigv^2, left to right
constexpr int kTreeDepth = 8;
struct CodecLayout {
  int64_t cent, bounds, gains, sk, sv, vtab, muk, sigk, muv, sigv, sphys, size;
};
RKV_HD CodecLayout codec_layout(int G, int d) {
  CodecLayout L;
  int64_t off = 0;
  L.cent = off; off += 512 * 4;
  L.bounds = off; off += 256 * 8;
  L.gains = off; off += 16 * 8;
  L.sk = off; off += (int64_t)d * 8;
  L.sv = off; off += (int64_t)d * 8;
  L.vtab = off; off += 9 * 256 * 2; off = align_up(off, 256);
  L.muk = off; off += (int64_t)G * d * 4;
  L.sigk = off; off += (int64_t)G * d * 4;
  L.muv = off; off += (int64_t)G * d * 4;
  L.sigv = off; off += (int64_t)G * d * 4;
  L.sphys = off; off += (int64_t)G * 8;
  L.size = align_up(off, 4096);
  return L;
}
RKV_HD int64_t codec_bytes(int codec, int G, int d) { return codec ? codec_layout(G, d).size : 0; }

// 512-token tiles of the key planes (16 groups each)
RKV_HD int64_t key_tiles(int64_t cap) { return (cap / kGroup + 15) / 16; }

struct RegionLayout {
  int64_t kplanes, vplanes, kmeta, vmeta, ek, ev, ktail, vtail, size;
};

RKV_HD RegionLayout region_layout(int G, int d, int W, int64_t cap, int esize) {
  const int64_t ng = cap / kGroup;
  RegionLayout L;
  int64_t off = 0;
  L.kplanes = off; off += (int64_t)G * key_tiles(cap) * d * W * 16 * 4; off = align_up(off, 256);
  L.vplanes = off; off += (int64_t)G * cap * W * (d / 32) * 4; off = align_up(off, 256);
  L.kmeta = off; off += (int64_t)G * ng * d * 4; off = align_up(off, 256);
  L.vmeta = off; off += (int64_t)G * ng * d * 4; off = align_up(off, 256);
  L.ek = off; off += (int64_t)G * d * 8; off = align_up(off, 256);
  L.ev = off; off += (int64_t)G * ng * 8; off = align_up(off, 256);
  L.ktail = off; off += (int64_t)G * kGroup * d * esize; off = align_up(off, 256);
  L.vtail = off; off += (int64_t)G * kGroup * d * esize;
  L.size = align_up(off, 4096);
  return L;
}

// Pointers to one (request, KV head) unit's arrays.
struct Unit {
  uint32_t* kplanes;   // [ntk][d][W][16]
  uint32_t* vplanes;   // [cap][W][d/32]
  uint32_t* kmeta;     // [ng][d]
  uint32_t* vmeta;     // [ng][d]
  double* ek;          // [d]
  double* ev;          // [ng]
  uint8_t* ktail;      // [32][d] elements
  uint8_t* vtail;
  int64_t cap, ng, ntk;
};

RKV_HD Unit unit_of(uint8_t* store, const ReqRecord& r, int g, int G, int d, int W,
                    int esize) {
  const RegionLayout L = region_layout(G, d, W, r.cap, esize);
  uint8_t* base = store + r.offset;
  const int64_t ng = r.cap / kGroup;
  Unit u;
  u.cap = r.cap;
  u.ng = ng;
  u.ntk = key_tiles(r.cap);
  u.kplanes = (uint32_t*)(base + L.kplanes) + (int64_t)g * u.ntk * d * W * 16;
  u.vplanes = (uint32_t*)(base + L.vplanes) + (int64_t)g * r.cap * W * (d / 32);
  u.kmeta = (uint32_t*)(base + L.kmeta) + (int64_t)g * ng * d;
  u.vmeta = (uint32_t*)(base + L.vmeta) + (int64_t)g * ng * d;
  u.ek = (double*)(base + L.ek) + (int64_t)g * d;
  u.ev = (double*)(base + L.ev) + (int64_t)g * ng;
  u.ktail = base + L.ktail + (int64_t)g * kGroup * d * esize;
  u.vtail = base + L.vtail + (int64_t)g * kGroup * d * esize;
  return u;
}

// Decode workspace (one call).  capmax = largest request capacity.
//   tk     u8  [B][G][d]          key depths
//   tv     u8  [B][G][capmax]     value depths
//   ebuf   u32 [B][H][capmax]     exp(s - m_tile) per token (tile = kTile),
//                                 fp64 bits 61..30 (enc_e); Lloyd-tree code:
//                                 f64, the logit s itself
//   tilepart f64 [B][H][ntile][2] (m_tile, sum of exp) per tile
//   ftile  f64 [B][H][ntile]      exp(m_tile - m) / Z
//   aval   f64 [B][G][capmax]     value weights (only when they do not fit
//                                 in the allocator's registers)
//   opart  f32 [B][H][nchunk][d]  partial outputs, one per run of chunks
//                                 (at most nchunk runs)
//   Lloyd-tree code only:
//   qp     f64 [B][G][d][H/G]     the score's weights q'_hc sigma^K_c, q' = U_K q
//   qb     f64 [B][H]             sum_c q'_c mu^K_c
//   otail  f32 [B][H][d]          the open group's share of the output
// Per selection domain of the multi-block value selection: two 2048-bin
// histograms (exponent fields of regular items and of odd gains), two
// alternating 8192-bin radix-digit histograms and the search state.
constexpr int64_t kSelDomainBytes = (2 * 2048 + 2 * 8192) * 4 + 256;

struct WsLayout {
  int64_t tk, tv, ebuf, tilepart, ftile, aval, opart, qp, qb, otail, sel, size;
  int ntile, nchunk;
};

RKV_HD WsLayout ws_layout(int B, int H, int G, int d, int64_t capmax, int codec) {
  WsLayout L;
  L.ntile = (int)((capmax + kTile - 1) / kTile);
  L.nchunk = (int)((capmax + kChunk - 1) / kChunk);
  int64_t off = 0;
  L.tk = off; off = align_up(off + (int64_t)B * G * d, 256);
  L.tv = off; off = align_up(off + (int64_t)B * G * capmax, 256);
  L.ebuf = off; off = align_up(off + (int64_t)B * H * capmax * (codec ? 8 : 4), 256);
  L.tilepart = off; off = align_up(off + (int64_t)B * H * L.ntile * 16, 256);
  L.ftile = off; off = align_up(off + (int64_t)B * H * L.ntile * 8, 256);
  L.aval = off; off = align_up(off + (int64_t)B * G * capmax * 8, 256);
  L.opart = off; off = align_up(off + (int64_t)B * H * L.nchunk * d * 4, 256);
  L.qp = off; off = align_up(off + (int64_t)B * H * d * 8, 256);
  L.qb = off; off = align_up(off + (int64_t)B * H * 8, 256);
  L.otail = off; off = align_up(off + (int64_t)B * H * d * 4, 256);
  L.sel = off; off = align_up(off + (int64_t)B * G * kSelDomainBytes, 256);
  L.size = off;
  return L;
}

}  // namespace readkv
