// Encoder: append tokens, and quantise + bit-plane pack every group that
// closes ("Read What Matters", Sec. 3.1 / Algorithm 1 encoder; uniform
// quantiser of "KV Cache Compression Through the Lens of Transform Coding",
// Sec. III-C, Definition 2, in cell form).
//
// Per closed group (32 tokens) and channel c:
//   lo   = largest bf16 <= min x                      (directed rounding)
//   rng  = smallest bf16 >= fl64(max x - lo)
//   code = min(floor(fl64(x - lo) * 2^W / rng), 2^W - 1), exact; 0 if rng = 0
// The floor is exact: the fp64 quotient is corrected by comparing q*rng
// with the numerator, both of which are exact in fp64 (q <= 2^W has at
// most 9 bits and rng 8 significant bits).
//
// Under the pages' own codec (Sec. 3.1, App. D.1; the store's codec block
// holds the tree and calibration) each token of a closing group is mapped
// through the Hadamard-sign transform x' = H (s . x) / sqrt(d) (in-place
// Walsh-Hadamard butterflies over the block, float64: the sums of +-x are
// exact for bf16 inputs), standardised z = (x' - mu_c) / sigma_c, and coded
// as its path down the Lloyd tree: at each node the upper child when
// z >= the node's boundary, the first W levels of the depth-8 walk.
#include "kernels_common.h"
#include "readkv_internal.h"

namespace readkv {

constexpr int kSmallAppend = 64;  // tokens per request up to which one launch appends

__device__ __forceinline__ int64_t clamp_n(const ReqRecord& r, const int32_t* n_new, int b,
                                           int n_max) {
  int64_t n = n_new ? (int64_t)n_new[b] : (int64_t)n_max;
  if (n < 0) n = 0;
  if (n > n_max) n = n_max;
  if (r.len + n > r.cap) n = r.cap - r.len;
  return n;
}

// Encode closed group gam of unit (b, g) with one block of 256 threads:
// threads 0..127 take the key channels, 128..255 the value channels.  Rows
// j < len0 of the group come from the tail buffer, the others from the new
// tokens (row0 = the unit's first new-token row).  Returns rng^2 of the
// thread's channel (0 for a non-finite group).  Contains block barriers:
// every thread of the block must call it.
// The group's value planes (32 rows of W x 16 contiguous bytes) are staged
// in vst (LDS, 32 W 4 words) and written with one 16-byte store per thread.
// Its key-plane words (one word of each (channel, plane) line of its
// 512-token tile) go to kst (LDS, the tile's d W 16 words) when the caller
// writes the whole tile out afterwards, else straight to the store.
// Lloyd-tree code (LL): cb = the codec block, g / G the KV head, xs = LDS
// [2][32][d] doubles (the group's tokens while they are transformed), bnd =
// the tree's boundaries in LDS; no metadata, E^K or E^V.
template <int DT, bool LL>
__device__ __forceinline__ double encode_group(uint8_t* store, const Unit& u, const void* knew,
                                               const void* vnew, int64_t row0, int64_t len0,
                                               int64_t gam, int W, int* bad_s, double* rv2,
                                               uint32_t* vst, uint32_t* kst, const uint8_t* cb,
                                               int g, int G, double* xs, const double* bnd) {
  const int tid = threadIdx.x;
  const bool isv = tid >= 128;
  const int c = tid & 127;
  const void* src = isv ? vnew : knew;
  const uint8_t* tail = isv ? u.vtail : u.ktail;
  if (tid < 2) bad_s[tid] = 0;
  __syncthreads();

  double x[kGroup];
  bool finite = true;
  double mn = 0.0, mx = 0.0;
#pragma unroll
  for (int s = 0; s < kGroup; ++s) {
    const int64_t j = gam * kGroup + s;
    x[s] = (j < len0) ? load_elem<DT>(tail, (int64_t)s * kDim + c)
                      : load_elem<DT>(src, (row0 + (j - len0)) * kDim + c);
    finite = finite && isfinite(x[s]);
  }
  if (!finite) atomicOr(&bad_s[isv], 1);
  if (finite) {
    mn = x[0];
    mx = x[0];
#pragma unroll
    for (int s = 1; s < kGroup; ++s) {
      mn = fmin(mn, x[s]);
      mx = fmax(mx, x[s]);
    }
  }
  uint32_t code[kGroup];
  uint32_t meta = 0u;
  double r2 = 0.0;
  if constexpr (LL) {
    const CodecLayout C = codec_layout(G, kDim);
    const double sgn = reinterpret_cast<const double*>(cb + (isv ? C.sv : C.sk))[c];
    const double mu = (double)reinterpret_cast<const float*>(cb + (isv ? C.muv : C.muk))[g * kDim + c];
    const double sd = (double)reinterpret_cast<const float*>(cb + (isv ? C.sigv : C.sigk))[g * kDim + c];
    __syncthreads();
    const bool bad = bad_s[isv] != 0;
    double* xb = xs + (isv ? kGroup * kDim : 0);
#pragma unroll
    for (int s = 0; s < kGroup; ++s) xb[s * kDim + c] = bad ? 0.0 : x[s] * sgn;
    for (int h = 1; h < kDim; h <<= 1) {
      __syncthreads();
#pragma unroll
      for (int s = 0; s < kGroup; ++s) {
        const double a = xb[s * kDim + c], o = xb[s * kDim + (c ^ h)];
        x[s] = (c & h) ? o - a : a + o;
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < kGroup; ++s) xb[s * kDim + c] = x[s];
    }
#pragma unroll
    for (int s = 0; s < kGroup; ++s) {
      const double z = __ddiv_rn(__dsub_rn(__dmul_rn(x[s], kInvSqrt128), mu), sd);
      uint32_t P = 0;
      for (int t = 0; t < kTreeDepth; ++t) P = 2 * P + (z >= bnd[(1 << t) - 1 + P] ? 1u : 0u);
      code[s] = bad ? 0u : P >> (kTreeDepth - W);
    }
    if (bad && c == 0) atomicOr(&header_of(store)->flags, 1u);
  } else {
    const uint32_t lo_b = bf16_round_dir(mn, false);
    const double lo = (double)bf16_to_float(lo_b);
    const uint32_t rng_b = bf16_round_dir(mx - lo, true);
    const double rng = (double)bf16_to_float(rng_b);
    if (!(isfinite(lo) && isfinite(rng))) atomicOr(&bad_s[isv], 1);
    __syncthreads();
    const bool bad = bad_s[isv] != 0;

    const double scale = (double)(1u << W);
    const double cmax = (double)((1u << W) - 1u);
#pragma unroll
    for (int s = 0; s < kGroup; ++s) {
      double q = 0.0;
      if (!bad && rng > 0.0) {
        const double num = (x[s] - lo) * scale;  // fl64(x - lo) * 2^W, exact scaling
        q = floor(num / rng);
        if (q * rng > num) q -= 1.0;             // q*rng exact: <= 9 x 8 significant bits
        else if ((q + 1.0) * rng <= num) q += 1.0;
        q = fmin(q, cmax);
      }
      code[s] = (uint32_t)q;
    }
    meta = bad ? 0u : (lo_b | (rng_b << 16));
    r2 = bad ? 0.0 : rng * rng;
    if (bad && c == 0) atomicOr(&header_of(store)->flags, 1u);
  }

  if (!isv) {
    if constexpr (!LL) u.kmeta[gam * kDim + c] = meta;
    for (int p = 0; p < W; ++p) {
      uint32_t word = 0;
#pragma unroll
      for (int s = 0; s < kGroup; ++s) word |= ((code[s] >> (W - 1 - p)) & 1u) << s;
      if (kst) kst[(c * W + p) * 16 + (gam & 15)] = word;
      else u.kplanes[(((gam >> 4) * kDim + c) * W + p) * 16 + (gam & 15)] = word;
    }
  } else {
    if constexpr (!LL) {
      u.vmeta[gam * kDim + c] = meta;
      rv2[c] = r2;
    }
    const int half = c >> 6;  // which 64-channel half this wave holds
    for (int s = 0; s < kGroup; ++s) {
      for (int p = 0; p < W; ++p) {
        const uint64_t m = __ballot((code[s] >> (W - 1 - p)) & 1u);
        if ((c & 63) == 0) {
          vst[(s * W + p) * 4 + 2 * half] = (uint32_t)m;
          vst[(s * W + p) * 4 + 2 * half + 1] = (uint32_t)(m >> 32);
        }
      }
    }
  }
  __syncthreads();
  if (tid < kGroup * W)  // the group's value rows: 16 bytes per thread
    reinterpret_cast<uint4*>(u.vplanes + gam * kGroup * W * (kDim / 32))[tid] =
        reinterpret_cast<const uint4*>(vst)[tid];
  if (!LL && tid == 128) {
    double e = 0.0;
    for (int cc = 0; cc < kDim; ++cc) e = e + rv2[cc];
    u.ev[gam] = e;
  }
  return r2;
}

// grid (tiles touched, G, B), 256 threads: block i encodes the closing
// groups of the unit's i-th 512-token key tile touched by this append, in
// group order.  When it encodes all 16 groups of the tile, the key planes
// are staged in LDS and written as whole 64-byte lines (else word by word:
// the tile's other groups are already stored).
template <int DT, bool LL>
__global__ __launch_bounds__(256) void k_encode_tiles(uint8_t* store, const void* knew,
                                                      const void* vnew, const int32_t* n_new,
                                                      int n_max, int G, int W, const uint8_t* cb) {
  constexpr int esize = DT == 0 ? 2 : 4;
  const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const ReqRecord r = req_of(store, b);
  const int64_t len0 = r.len;
  const int64_t n = clamp_n(r, n_new, b, n_max);
  const int64_t first = len0 / kGroup, last = (len0 + n) / kGroup;
  if (last == first) return;
  const int64_t tile = (first >> 4) + i;
  if (tile > ((last - 1) >> 4)) return;
  const int64_t g0 = first > 16 * tile ? first : 16 * tile;
  const int64_t g1 = last < 16 * tile + 16 ? last : 16 * tile + 16;
  const bool whole = g0 == 16 * tile && g1 == 16 * tile + 16;
  __shared__ int bad_s[2];
  __shared__ double rv2[128];
  __shared__ __attribute__((aligned(16))) uint32_t vst[kGroup * 8 * 4];
  __shared__ __attribute__((aligned(16))) uint32_t kst[kDim * 8 * 16];
  __shared__ double xs[LL ? 2 * kGroup * kDim : 1];
  __shared__ double bnd[LL ? 256 : 1];
  if constexpr (LL) {
    const double* bsrc = reinterpret_cast<const double*>(cb + codec_layout(G, kDim).bounds);
    bnd[threadIdx.x] = bsrc[threadIdx.x];  // read after encode_group's first barrier
  }
  const Unit u = unit_of(store, r, g, G, kDim, W, esize);
  for (int64_t gam = g0; gam < g1; ++gam)
    encode_group<DT, LL>(store, u, knew, vnew, ((int64_t)b * G + g) * n_max, len0, gam, W, bad_s,
                         rv2, vst, whole ? kst : nullptr, cb, g, G, xs, bnd);
  if (whole) {
    __syncthreads();
    uint4* dst = reinterpret_cast<uint4*>(u.kplanes + tile * kDim * W * 16);
    for (int k = threadIdx.x; k < kDim * W * 4; k += 256) dst[k] = reinterpret_cast<const uint4*>(kst)[k];
  }
}

// grid (G, B), 128 threads: E^K[c] += rng^2 of every newly closed group,
// in group order.
template <int DT>
__global__ __launch_bounds__(128) void k_ek_update(uint8_t* store, const int32_t* n_new, int n_max,
                                                   int G, int W) {
  constexpr int esize = DT == 0 ? 2 : 4;
  const int g = blockIdx.x, b = blockIdx.y;
  const ReqRecord r = req_of(store, b);
  const int64_t n = clamp_n(r, n_new, b, n_max);
  const int64_t first = r.len / kGroup;
  const int64_t last = (r.len + n) / kGroup;
  if (last == first) return;
  const Unit u = unit_of(store, r, g, G, kDim, W, esize);
  const int c = threadIdx.x;
  double e = u.ek[c];
  for (int64_t gam = first; gam < last; ++gam) {
    const double rng = (double)bf16_to_float(u.kmeta[gam * kDim + c] >> 16);
    e = e + rng * rng;
  }
  u.ek[c] = e;
}

// grid (B), 256 threads: move the still-open tokens into the tail buffer and
// publish the new length.
template <int DT>
__global__ __launch_bounds__(256) void k_tail_update(uint8_t* store, const void* knew,
                                                     const void* vnew, const int32_t* n_new,
                                                     int n_max, int G, int W) {
  constexpr int esize = DT == 0 ? 2 : 4;
  const int b = blockIdx.x;
  ReqRecord* rp = reinterpret_cast<ReqRecord*>(store + 256 + 32 * (int64_t)b);
  const ReqRecord r = *rp;
  const int64_t want = n_new ? (int64_t)n_new[b] : (int64_t)n_max;
  const int64_t n = clamp_n(r, n_new, b, n_max);
  const int64_t len1 = r.len + n;
  const int64_t base = (len1 / kGroup) * kGroup;
  const int64_t from = base > r.len ? base : r.len;  // older tail tokens stay in place
  const int64_t cnt = len1 - from;
  const int64_t per_g = cnt * kDim;
  for (int64_t e = threadIdx.x; e < (int64_t)G * per_g; e += blockDim.x) {
    const int g = (int)(e / per_g);
    const int64_t rem = e - (int64_t)g * per_g;
    const int64_t j = from + rem / kDim;
    const int c = (int)(rem % kDim);
    const Unit u = unit_of(store, r, g, G, kDim, W, esize);
    const int64_t src = (((int64_t)b * G + g) * n_max + (j - r.len)) * kDim + c;
    const int64_t dst = (j - base) * kDim + c;
    if constexpr (DT == 0) {
      ((uint16_t*)u.ktail)[dst] = ((const uint16_t*)knew)[src];
      ((uint16_t*)u.vtail)[dst] = ((const uint16_t*)vnew)[src];
    } else {
      ((float*)u.ktail)[dst] = ((const float*)knew)[src];
      ((float*)u.vtail)[dst] = ((const float*)vnew)[src];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    rp->len = len1;
    if (n < want) atomicOr(&header_of(store)->flags, 2u);
  }
}

// Small appends (n_max <= kSmallAppend tokens per request), one launch: grid
// (G, B), 256 threads per (request, KV head): encode the closing groups in
// group order, add their rng_K^2 to E^K in that order, move the still-open
// tokens into the tail.  The request's last block to finish (a ticket
// counter in the request record's spare field, reset by that block)
// publishes the new length, after every block has read the old one.
template <int DT, bool LL>
__global__ __launch_bounds__(256) void k_append_small(uint8_t* store, const void* knew,
                                                      const void* vnew, const int32_t* n_new,
                                                      int n_max, int G, int W, const uint8_t* cb) {
  constexpr int esize = DT == 0 ? 2 : 4;
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  __shared__ int bad_s[2];
  __shared__ double rv2[128];
  __shared__ __attribute__((aligned(16))) uint32_t vst[kGroup * 8 * 4];
  __shared__ int last_s;
  __shared__ double xs[LL ? 2 * kGroup * kDim : 1];
  __shared__ double bnd[LL ? 256 : 1];
  if constexpr (LL) {
    const double* bsrc = reinterpret_cast<const double*>(cb + codec_layout(G, kDim).bounds);
    bnd[tid] = bsrc[tid];  // read after encode_group's first barrier
  }
  ReqRecord* rp = reinterpret_cast<ReqRecord*>(store + 256 + 32 * (int64_t)b);
  const ReqRecord r = *rp;
  const int64_t want = n_new ? (int64_t)n_new[b] : (int64_t)n_max;
  const int64_t n = clamp_n(r, n_new, b, n_max);
  const int64_t len0 = r.len, len1 = len0 + n;
  const int64_t first = len0 / kGroup, last = len1 / kGroup;
  const int64_t base = last * kGroup;
  const int64_t from = base > len0 ? base : len0;  // older tail tokens stay in place
  const Unit u = unit_of(store, r, g, G, kDim, W, esize);
  const int64_t row0 = ((int64_t)b * G + g) * n_max;
  for (int64_t gam = first; gam < last; ++gam) {
    const double r2 = encode_group<DT, LL>(store, u, knew, vnew, row0, len0, gam, W, bad_s, rv2, vst,
                                           nullptr, cb, g, G, xs, bnd);
    if (!LL && tid < kDim) u.ek[tid] = u.ek[tid] + r2;
    __syncthreads();  // the group's tail rows are read before they are replaced
  }
  const int64_t per = (len1 - from) * kDim;
  for (int64_t e = tid; e < per; e += 256) {
    const int64_t j = from + e / kDim;
    const int c = (int)(e % kDim);
    const int64_t srow = (row0 + (j - len0)) * kDim + c, drow = (j - base) * kDim + c;
    if constexpr (DT == 0) {
      ((uint16_t*)u.ktail)[drow] = ((const uint16_t*)knew)[srow];
      ((uint16_t*)u.vtail)[drow] = ((const uint16_t*)vnew)[srow];
    } else {
      ((float*)u.ktail)[drow] = ((const float*)knew)[srow];
      ((float*)u.vtail)[drow] = ((const float*)vnew)[srow];
    }
  }
  __syncthreads();
  if (tid == 0) {
    // the ticket only orders this block's reads of the record (all done:
    // their values are in use) before the length changes; the data written
    // here reaches the next launch through the kernel boundary, so no
    // device-scope fence (which would write back the L2) is needed
    unsigned long long* ticket = reinterpret_cast<unsigned long long*>(&rp->reserved);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    last_s = atomicAdd(ticket, 1ull) == (unsigned long long)(G - 1);
  }
  __syncthreads();
  if (tid == 0 && last_s) {
    *reinterpret_cast<unsigned long long*>(&rp->reserved) = 0ull;
    rp->len = len1;
    if (n < want) atomicOr(&header_of(store)->flags, 2u);
  }
}

__global__ void k_fill_zero(uint32_t* p, int64_t nwords) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nwords;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

int launch_store_zero(void* store, size_t bytes, hipStream_t st) {
  const int64_t nw = (int64_t)(bytes / 4);
  int blocks = (int)((nw + 255) / 256);
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_fill_zero, dim3(blocks), dim3(256), 0, st, (uint32_t*)store, nw);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

template <int DT, bool LL>
static void launch_encode_t(const EncodeArgs& a, hipStream_t st) {
  if (a.n_max <= kSmallAppend) {
    hipLaunchKernelGGL((k_append_small<DT, LL>), dim3(a.G, a.B), dim3(256), 0, st, (uint8_t*)a.store,
                       a.knew, a.vnew, a.n_new, a.n_max, a.G, a.W, a.cblock);
    return;
  }
  // key tiles an append of n_max tokens can touch: its groups, plus one
  // for a start inside a tile
  const int max_tiles = (int)((a.n_max + kGroup - 1) / kGroup + 15) / 16 + 1;
  hipLaunchKernelGGL((k_encode_tiles<DT, LL>), dim3(max_tiles, a.G, a.B), dim3(256), 0, st,
                     (uint8_t*)a.store, a.knew, a.vnew, a.n_new, a.n_max, a.G, a.W, a.cblock);
  if (!LL)
    hipLaunchKernelGGL((k_ek_update<DT>), dim3(a.G, a.B), dim3(128), 0, st, (uint8_t*)a.store,
                       a.n_new, a.n_max, a.G, a.W);
  hipLaunchKernelGGL((k_tail_update<DT>), dim3(a.B), dim3(256), 0, st, (uint8_t*)a.store, a.knew,
                     a.vnew, a.n_new, a.n_max, a.G, a.W);
}

int launch_encode(const EncodeArgs& a, hipStream_t st) {
  if (a.n_max <= 0) return 0;
  if (a.codec) {
    if (a.dtype == 0) launch_encode_t<0, true>(a, st);
    else launch_encode_t<1, true>(a, st);
  } else {
    if (a.dtype == 0) launch_encode_t<0, false>(a, st);
    else launch_encode_t<1, false>(a, st);
  }
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace readkv
