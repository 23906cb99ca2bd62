// One ReadKV decode step ("Read What Matters: Query-Adaptive Quantization
// for KV Caches", Sec. 3.2-3.3, Algorithm 1) as five launches on one stream:
//
//   k_key_alloc   (B*G waves)         key weights (Eq. (2)) and ChooseDepths
//                                     over the d_h channels -> t^K
//   k_score       (B*G x tiles)       prefix-gather of the chosen key planes
//                                     through LDS, reconstructed logits in
//                                     fp64, per-tile max and sum of exp
//                                     (split-context softmax)
//   k_value_alloc (B*G blocks)        softmax statistics, value weights
//                                     (Eq. (3)) and ChooseDepths over the
//                                     packed tokens -> t^V
//   k_gather      (B*G x chunks)      prefix-gather of the chosen value
//                                     planes, attention-weighted sums per
//                                     chunk
//   k_out_reduce  (B*H*d threads)     chunk partials summed in chunk order
//
// The k_value_alloc -> k_gather boundary is the staged(2) reader's second
// batch: value reads depend on attention computed from the first batch.
//
// Reconstruction of a depth-t prefix P (t MSB-first planes) of a group with
// metadata (lo, rng): x_hat = lo + rng (2P + 1) / 2^(t+1).  The kernels
// un-plane an 8-element bit column into X = P 2^(8-t) (missing planes read
// as zero) and use x_hat = lo + rng 2^-(t+1) + rng X / 256.
#include <math.h>

#include "kernels_common.h"
#include "readkv_internal.h"
#include "select.h"

namespace readkv {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr double kInvSqrtD = 0.088388347648318440550;  // 1/sqrt(128)

// byte `ob` of each of 8 plane words (plane p -> byte 7-p of hi:lo), then
// the 8x8 bit transpose: byte i of hi:lo becomes element 8*ob+i's code
// prefix, MSB-first (missing planes must be passed as zero words)
__device__ __forceinline__ void unplane8(const uint32_t (&w)[8], uint32_t sel, uint32_t& lo,
                                         uint32_t& hi) {
  const uint32_t r01 = __builtin_amdgcn_perm(w[0], w[1], sel);
  const uint32_t r23 = __builtin_amdgcn_perm(w[2], w[3], sel);
  const uint32_t r45 = __builtin_amdgcn_perm(w[4], w[5], sel);
  const uint32_t r67 = __builtin_amdgcn_perm(w[6], w[7], sel);
  hi = __builtin_amdgcn_perm(r01, r23, 0x05040100u);
  lo = __builtin_amdgcn_perm(r45, r67, 0x05040100u);
  transpose8_halves(lo, hi);
}

// ---------------------------------------------------------------------------
// Key allocation: one wave per (request, KV head).  Lane l holds channels l
// and l+64 and their W candidate gains w_c 4^-t (t = 1..W).  The B_K largest
// positive gains are chosen, ties to the lowest channel (App. E.2.1: with
// strictly decreasing per-item gains this is ChooseDepths' result).  The
// threshold is found in two steps on the 64-bit patterns of the fp64 gains:
// bisection on the 12-bit sign+exponent field, then an exact rank among the
// candidates in the threshold's exponent class.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(64) void k_key_alloc(const uint8_t* store, const void* q, int H, int G,
                                                  int W, float RK, uint8_t* tk) {
  constexpr int esize = DT == 0 ? 2 : 4;
  const int unit = blockIdx.x;
  const int b = unit / G, g = unit - b * G;
  const int gqa = H / G;
  const ReqRecord r = req_of(store, b);
  const Unit u = unit_of(const_cast<uint8_t*>(store), r, g, G, kDim, W, esize);
  const int lane = threadIdx.x;
  __shared__ uint64_t ck[2 * 64 * 8];
  __shared__ uint32_t cc[2 * 64 * 8];

  uint64_t key[2][8];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    double qsq = 0.0;
    for (int hh = 0; hh < gqa; ++hh) {
      const double qv = load_elem<DT>(q, ((int64_t)b * H + (int64_t)g * gqa + hh) * kDim + c);
      qsq = __dadd_rn(qsq, __dmul_rn(qv, qv));
    }
    const double w = __dmul_rn(qsq, u.ek[c]);
#pragma unroll
    for (int t = 1; t <= 8; ++t) {
      const double gt = __dmul_rn(w, ldexp_pow2(-2 * t));
      key[k][t - 1] = (t <= W && gt > 0.0) ? dbits(gt) : 0ull;
    }
  }
  const uint32_t Bk = (uint32_t)floor((double)RK * (double)kDim);
  // wave-wide counts are sums of ballot popcounts over the 16 candidate slots
  uint32_t npos = 0;
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int t = 0; t < 8; ++t) npos += (uint32_t)__popcll(__ballot(key[k][t] != 0ull));

  uint32_t sel[2] = {0u, 0u};
  if (npos <= Bk) {
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int t = 0; t < 8; ++t) sel[k] += key[k][t] != 0ull;
  } else if (Bk > 0) {
    // largest exponent class E with count(key >> 52 >= E) >= Bk
    int lo = 0, hi = 2047;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      uint32_t c_ = 0;
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int t = 0; t < 8; ++t)
          c_ += (uint32_t)__popcll(__ballot(key[k][t] != 0ull && (int)(key[k][t] >> 52) >= mid));
      if (c_ >= Bk) lo = mid;
      else hi = mid - 1;
    }
    const int Es = lo;
    uint32_t above = 0, at = 0;
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int e = (int)(key[k][t] >> 52);
        above += (uint32_t)__popcll(__ballot(key[k][t] != 0ull && e > Es));
        at += key[k][t] != 0ull && e == Es;
      }
    const uint32_t rem = Bk - above;  // >= 1 by the choice of Es
    // candidates in class Es: with normal gains at most one level per
    // channel; lane slot k holds channel lane + 64 k
    uint32_t atc[2] = {0u, 0u};
    uint64_t atm[2] = {0ull, 0ull};
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (key[k][t] != 0ull && (int)(key[k][t] >> 52) == Es) {
          ++atc[k];
          atm[k] = key[k][t] & 0x000FFFFFFFFFFFFFull;
        }
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int t = 0; t < 8; ++t) sel[k] += key[k][t] != 0ull && (int)(key[k][t] >> 52) > Es;
    if (!__any(atc[0] > 1u || atc[1] > 1u)) {
      // MSB-first search for the rem-th largest mantissa in the class
      uint64_t pre = 0ull;
      uint32_t rm = rem;
      for (int bit = 51; bit >= 0; --bit) {
        const uint64_t hi_mask = ~((2ull << bit) - 1ull);  // bits above `bit`
        const bool f0 = atc[0] && ((atm[0] ^ pre) & hi_mask) == 0ull && ((atm[0] >> bit) & 1ull);
        const bool f1 = atc[1] && ((atm[1] ^ pre) & hi_mask) == 0ull && ((atm[1] >> bit) & 1ull);
        const uint32_t c1 = (uint32_t)(__popcll(__ballot(f0)) + __popcll(__ballot(f1)));
        if (c1 >= rm) pre |= 1ull << bit;
        else rm -= c1;
      }
      // above the threshold mantissa: taken; equal: the first rm in channel order
      const bool e0 = atc[0] && atm[0] == pre, e1 = atc[1] && atm[1] == pre;
      const uint64_t b0 = __ballot(e0), b1 = __ballot(e1);
      const uint64_t below = (1ull << lane) - 1ull;
      if (atc[0] && atm[0] > pre) ++sel[0];
      if (atc[1] && atm[1] > pre) ++sel[1];
      if (e0 && (uint32_t)__popcll(b0 & below) < rm) ++sel[0];
      if (e1 && (uint32_t)(__popcll(b0) + __popcll(b1 & below)) < rm) ++sel[1];
    } else {
      // several levels of one channel in the class (subnormal gains): rank
      // every class member against the compacted list
      const uint32_t incl = wave_incl_scan_u32(at);
      const uint32_t nat = __shfl(incl, 63, 64);
      uint32_t pos = incl - at;
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (key[k][t] != 0ull && (int)(key[k][t] >> 52) == Es) {
            ck[pos] = key[k][t];
            cc[pos] = (uint32_t)(lane + 64 * k);
            ++pos;
          }
      __syncthreads();
      for (int k = 0; k < 2; ++k) {
        const uint32_t c = (uint32_t)(lane + 64 * k);
        for (int t = 0; t < 8; ++t) {
          const uint64_t kk = key[k][t];
          if (kk == 0ull || (int)(kk >> 52) != Es) continue;
          uint32_t beats = 0;
          for (uint32_t m = 0; m < nat; ++m) {
            const uint64_t k2 = ck[m];
            beats += (k2 > kk) || (k2 == kk && cc[m] < c);
          }
          if (beats < rem) ++sel[k];
        }
      }
    }
  }
  tk[(int64_t)unit * kDim + lane] = (uint8_t)sel[0];
  tk[(int64_t)unit * kDim + lane + 64] = (uint8_t)sel[1];
}

// ---------------------------------------------------------------------------
// Score: one block of 256 threads per 512-token tile (16 groups) of one
// (request, KV head).
//  1. Stage in LDS the tile's segment of every chosen key line (channel c,
//     plane p < t^K_c): 16 words = 64 B per line, loaded as 16 B pieces, and
//     the tile's key metadata.  LDS layout planes[group][slot], slot =
//     (sum over channels below c of t^K) + p.
//  2. Per-group constants
//       C_h = sum_c q_hc (lo_c + rng_c 2^-(t_c+1)) - 4096 sum_{t_c>0} beta_hc
//     with beta_hc = q_hc rng_c / 256 (exact products of bf16 values).
//  3. Wave w takes channels w, w+4, ... (so a channel's depth t is uniform
//     in the wave), lane o its 8 tokens 8o..8o+7 of the tile.  Per channel
//     the lane gathers byte o%4 of its group's t plane words, transposes the
//     8x8 bit block into the tokens' prefix codes X and accumulates
//     beta_hc (4096 + X) in fp64; 4096 + X is assembled as a double straight
//     from the code byte (one byte permute), the 4096 part cancels against C.
//  4. The four waves' sums are added in wave order through LDS; logits
//     s = (C + sum) / sqrt(d); open-group tokens use exact keys.  Each thread
//     finishes two tokens: e = exp(s - m_tile) (fp64, and rounded to fp16 for
//     the value gather) and the block writes (m_tile, sum e) per head.
// Grid (unit, tile): consecutive blocks are different units, so all tiles
// of a unit run on one XCD and share its L2 (a 128 B line holds two tiles'
// 64 B segments of a key line).
// Dynamic LDS: max(16 * (max slots | 1) words, the 64 x 8 x GQA fp64 wave
// reduction buffer).
// ---------------------------------------------------------------------------
// transpose8_halves for lo == 0 (at most 4 planes present)
__device__ __forceinline__ void transpose8_hi4(uint32_t& lo, uint32_t& hi) {
  uint32_t t;
  t = (hi ^ (hi >> 7)) & 0x00AA00AAu;
  hi ^= t ^ (t << 7);
  t = (hi ^ (hi >> 14)) & 0x0000CCCCu;
  hi ^= t ^ (t << 14);
  t = (hi << 4) & 0xF0F0F0F0u;
  lo = t;
  hi ^= t >> 4;
}

// the double 4096 + (byte i of y), built from its bit pattern
__device__ __forceinline__ double code_plus_4096(uint32_t y, int i) {
  const uint32_t hi = __builtin_amdgcn_perm(0x40B00000u, y, 0x0706000Cu | ((uint32_t)i << 8));
  return __hiloint2double((int)hi, 0);
}

template <int GQA, int DT>
__global__ __launch_bounds__(256) void k_score(const uint8_t* store, const void* q, const uint8_t* tk,
                                               int H, int G, int W, int64_t capmax, int ntile_ws,
                                               double* ebuf, _Float16* e16, double* tilepart) {
  constexpr int esize = DT == 0 ? 2 : 4;
  constexpr int NG = kTile / kGroup;  // 16
  extern __shared__ uint32_t planes[];
  __shared__ double qs[GQA][kDim];
  __shared__ uint32_t meta[NG][kDim + 1];  // padded: the 16 groups fall in distinct banks
  __shared__ double Cs[NG][GQA];
  __shared__ double tails[kGroup][GQA];
  __shared__ double red[4][GQA];
  __shared__ uint16_t offs[kDim + 1];
  __shared__ uint8_t tks[kDim];
  __shared__ uint8_t s2c[kDim * 8];
  __shared__ uint32_t wtot[2];

  const int tile = blockIdx.y, b = blockIdx.x / G, g = blockIdx.x % G;
  const ReqRecord r = req_of(store, b);
  const int64_t len = r.len;
  const int64_t t0 = (int64_t)tile * kTile;
  if (t0 >= len) return;
  const int64_t Tp = len & ~(int64_t)(kGroup - 1);
  const Unit u = unit_of(const_cast<uint8_t*>(store), r, g, G, kDim, W, esize);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t gam0 = t0 / kGroup;
  int64_t ngp64 = Tp / kGroup - gam0;
  const int ngp = (int)(ngp64 < 0 ? 0 : (ngp64 > NG ? NG : ngp64));  // packed groups in tile

  for (int i = tid; i < GQA * kDim; i += 256)
    qs[i / kDim][i % kDim] = load_elem<DT>(q, ((int64_t)b * H + (int64_t)g * GQA) * kDim + i);
  if (tid < kDim) tks[tid] = tk[((int64_t)b * G + g) * kDim + tid];
  for (int i = tid; i < NG * kDim; i += 256) {
    const int gl = i / kDim, c = i % kDim;
    meta[gl][c] = (gl < ngp) ? u.kmeta[(gam0 + gl) * kDim + c] : 0u;
  }
  __syncthreads();
  uint32_t tv_ = 0, inc = 0;
  if (tid < kDim) {
    tv_ = tks[tid];
    inc = wave_incl_scan_u32(tv_);
    if (lane == 63) wtot[wv] = inc;
  }
  __syncthreads();
  if (tid < kDim) {
    if (wv == 1) inc += wtot[0];
    offs[tid + 1] = (uint16_t)inc;
    if (tid == 0) offs[0] = 0;
    const uint32_t o = inc - tv_;
    for (uint32_t p = 0; p < tv_; ++p) s2c[o + p] = (uint8_t)tid;
  }
  __syncthreads();
  const int ns = offs[kDim];
  const int nsp = ns | 1;

  // ---- 1. stage key plane segments: (slot, quad) -> 16 B global loads ----
  {
    const int nq = ns * 4;
    const uint32_t* kpl = u.kplanes;
    for (int base = 0; base < nq; base += 256 * 8) {
      uint4 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int idx = base + k * 256 + tid;
        v[k] = make_uint4(0u, 0u, 0u, 0u);
        if (idx < nq) {
          const int s = idx >> 2, q4 = idx & 3;
          const int c = s2c[s];
          const int p = s - offs[c];
          if (4 * q4 < ngp)
            v[k] = *reinterpret_cast<const uint4*>(kpl + ((int64_t)c * W + p) * u.ngk + gam0 + 4 * q4);
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int idx = base + k * 256 + tid;
        if (idx < nq) {
          const int s = idx >> 2, q4 = idx & 3;
          planes[(4 * q4 + 0) * nsp + s] = v[k].x;
          planes[(4 * q4 + 1) * nsp + s] = v[k].y;
          planes[(4 * q4 + 2) * nsp + s] = v[k].z;
          planes[(4 * q4 + 3) * nsp + s] = v[k].w;
        }
      }
    }
  }
  // ---- 2. per-group constants ----
  {
    const int gl = tid >> 4, cs = tid & 15;
    double ca[GQA];
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) ca[hh] = 0.0;
    if (gl < ngp) {
      for (int k = 0; k < kDim / 16; ++k) {
        const int c = cs + 16 * k;
        const uint32_t m = meta[gl][c];
        const int t = tks[c];
        const double lo = (double)bf16_to_float(m & 0xFFFFu);
        const double rng = (double)bf16_to_float(m >> 16);
        const double base = lo + rng * ldexp_pow2(-t - 1) - (t > 0 ? 16.0 * rng : 0.0);
#pragma unroll
        for (int hh = 0; hh < GQA; ++hh) ca[hh] = fma(qs[hh][c], base, ca[hh]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) ca[hh] = group_sum<16>(ca[hh]);
    if (cs == 0)
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) Cs[gl][hh] = ca[hh];
  }
  __syncthreads();

  // ---- 3. un-plane and accumulate: wave wv, channels wv, wv+4, ... ----
  double acc[8][GQA];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) acc[i][hh] = 0.0;
  {
    const int gl = lane >> 2, ob = lane & 3;
    const uint32_t sel = 0x0C0C0000u | ((4u + (uint32_t)ob) << 8) | (uint32_t)ob;
    const uint32_t* pl = planes + gl * nsp;
    for (int c = wv; c < kDim; c += 4) {
      const int t = tks[c];
      if (t == 0) continue;
      const int s0 = offs[c];
      const double rs = (double)bf16_to_float(meta[gl][c] >> 16) * (1.0 / 256.0);
      double beta[GQA];
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) beta[hh] = qs[hh][c] * rs;
      uint32_t lo, hi;
      if (t <= 4) {
        const uint32_t w0 = pl[s0];
        const uint32_t w1 = t > 1 ? pl[s0 + 1] : 0u;
        const uint32_t w2 = t > 2 ? pl[s0 + 2] : 0u;
        const uint32_t w3 = t > 3 ? pl[s0 + 3] : 0u;
        hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(w0, w1, sel), __builtin_amdgcn_perm(w2, w3, sel),
                                   0x05040100u);
        transpose8_hi4(lo, hi);
      } else {
        uint32_t w[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) w[p] = (p < t) ? pl[s0 + p] : 0u;
        unplane8(w, sel, lo, hi);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double X = code_plus_4096(e < 4 ? lo : hi, e & 3);
#pragma unroll
        for (int hh = 0; hh < GQA; ++hh) acc[e][hh] = fma(beta[hh], X, acc[e][hh]);
      }
    }
  }
  // ---- the four waves' partial sums: waves 0,1 store, waves 2,3 add; the
  // epilogue adds the two buffers (fixed order (w0 + w2) + (w1 + w3)) ----
  double* wred = reinterpret_cast<double*>(planes);  // [2][8 * GQA][64]
  __syncthreads();
  if (wv < 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) wred[(wv * 8 * GQA + e * GQA + hh) * 64 + lane] = acc[e][hh];
  }
  __syncthreads();
  if (wv >= 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) {
        double* p = wred + ((wv - 2) * 8 * GQA + e * GQA + hh) * 64 + lane;
        *p = *p + acc[e][hh];
      }
  }
  __syncthreads();

  // ---- 4. open group (exact keys) ----
  const int64_t ntail = len - Tp;
  const bool tail_here = ntail > 0 && Tp >= t0 && Tp < t0 + kTile;
  if (tail_here) {
    const int rr = tid >> 3, part = tid & 7;
    double st[GQA];
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) st[hh] = 0.0;
    if (rr < ntail) {
      for (int c = part * 16; c < part * 16 + 16; ++c) {
        const double kv = load_elem<DT>(u.ktail, (int64_t)rr * kDim + c);
#pragma unroll
        for (int hh = 0; hh < GQA; ++hh) st[hh] = fma(qs[hh][c], kv, st[hh]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) st[hh] = group_sum<8>(st[hh]);
    if (part == 0 && rr < ntail)
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) tails[rr][hh] = st[hh] * kInvSqrtD;
  }
  __syncthreads();

  // ---- softmax partials: thread (oc = tid % 64, pair = tid / 64) finishes
  // tokens 8 oc + 2 pair and 8 oc + 2 pair + 1 of the tile ----
  const int oc = lane, e0 = 2 * wv;
  const int glt = oc >> 2;
  const bool pk = glt < ngp;
  const bool has_tail = tail_here && tid < ntail;
  double sv[2][GQA];
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh)
      sv[k][hh] = pk ? (Cs[glt][hh] + (wred[((e0 + k) * GQA + hh) * 64 + oc] +
                                        wred[(8 * GQA + (e0 + k) * GQA + hh) * 64 + oc])) * kInvSqrtD
                     : 0.0;
  double mt[GQA];
#pragma unroll
  for (int hh = 0; hh < GQA; ++hh) {
    double m = has_tail ? tails[tid][hh] : -INFINITY;
    if (pk) m = fmax(m, fmax(sv[0][hh], sv[1][hh]));
    m = wave_max(m);
    if (lane == 0) red[wv][hh] = m;
  }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < GQA; ++hh) mt[hh] = fmax(fmax(red[0][hh], red[1][hh]), fmax(red[2][hh], red[3][hh]));
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < GQA; ++hh) {
    const int64_t row = ((int64_t)b * H + (int64_t)g * GQA + hh) * capmax;
    double z = 0.0;
    if (pk) {
      const int64_t j = t0 + 8 * oc + e0;  // even: the pair is 16 B / 4 B aligned
      const double ea = exp(sv[0][hh] - mt[hh]), eb = exp(sv[1][hh] - mt[hh]);
      *reinterpret_cast<double2*>(ebuf + row + j) = make_double2(ea, eb);
      f16x2 hp;
      hp.x = (_Float16)(float)ea;
      hp.y = (_Float16)(float)eb;
      *reinterpret_cast<f16x2*>(e16 + row + j) = hp;
      z = ea + eb;
    }
    if (has_tail) {
      const double ev = exp(tails[tid][hh] - mt[hh]);
      ebuf[row + Tp + tid] = ev;
      e16[row + Tp + tid] = (_Float16)(float)ev;
      z += ev;
    }
    z = wave_sum(z);
    if (lane == 0) red[wv][hh] = z;
  }
  __syncthreads();
  if (tid < GQA) {
    double* tp = tilepart + (((int64_t)b * H + (int64_t)g * GQA + tid) * ntile_ws + tile) * 2;
    tp[0] = mt[tid];
    tp[1] = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
  }
}

// ---------------------------------------------------------------------------
// Value allocation: one block of 1024 threads per (request, KV head); token
// j is owned by thread j mod 1024 (coalesced reads).
//   m_h = max_tile m_tile, Z_h = sum_tile z_tile exp(m_tile - m_h)
//   f_{h,tile} = exp(m_tile - m_h) / Z_h         (alpha_hat = e * f)
//   a_j = (sum_h alpha_hat_hj^2) * s_gamma(j)     (Eq. (3))
// then ChooseDepths with B_V = floor(R_V * T_packed) over the (token, level)
// gains a_j 4^-t, ties to the lowest token.  A token with a normal a_j
// whose exponent field E exceeds 2W has its W gains at exponents E-2t with
// a_j's mantissa; smaller ("tiny") ones are multiplied out.  Threshold
// search: the exponent class E* of the B_V-th largest gain from an exponent
// histogram (E* and the count above it), then 11/11/10/10/10-bit radix
// passes over the mantissas of the candidates in class E*.
// ---------------------------------------------------------------------------
constexpr int kVNT = 1024;
constexpr int kVPMAX = 16;  // tokens per thread held in registers

// hist[bin] += 1 for every active lane, one LDS atomic per distinct bin of
// the wave: a lane's peers with the same 11-bit bin are found by matching
// the ballots of each bin bit; the lowest peer adds the peer count.
__device__ __forceinline__ void agg_add(uint32_t* hist, uint32_t bin, bool act) {
  uint64_t same = __ballot(act);
#pragma unroll
  for (int bit = 0; bit < 11; ++bit) {
    const uint64_t ones = __ballot(act && ((bin >> bit) & 1u));
    same &= ((bin >> bit) & 1u) ? ones : ~ones;
  }
  if (act && (same & ((1ull << __lane_id()) - 1ull)) == 0ull)
    atomicAdd(&hist[bin & 2047u], (uint32_t)__popcll(same));
}

template <int GQA, bool REG>
__global__ __launch_bounds__(1024) void k_value_alloc(const uint8_t* store, int H, int G, int W,
                                                      int esize, float RV, int vscale,
                                                      int64_t capmax, int ntile_ws,
                                                      const double* ebuf, const double* tilepart,
                                                      double* ftile, double* aval, uint8_t* tv) {
  constexpr int NT = kVNT;
  const int b = blockIdx.x / G, g = blockIdx.x % G;
  const ReqRecord r = req_of(store, b);
  const int64_t len = r.len;
  const int64_t Tp = len & ~(int64_t)(kGroup - 1);
  const int ntile_b = (int)((len + kTile - 1) / kTile);
  const Unit u = unit_of(const_cast<uint8_t*>(store), r, g, G, kDim, W, esize);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  __shared__ uint32_t hA[2048];
  __shared__ uint32_t hB[2048];
  __shared__ uint32_t wsum[NT / 64 + 1];
  __shared__ uint32_t sh[2];

  // ---- softmax statistics -> per-tile factors (wave h handles head h) ----
  if (wv < GQA) {
    const int h = g * GQA + wv;
    const double* tp = tilepart + ((int64_t)b * H + h) * ntile_ws * 2;
    double m = -INFINITY;
    for (int t = lane; t < ntile_b; t += 64) m = fmax(m, tp[2 * t]);
    m = wave_max(m);
    double Z = 0.0;
    for (int t = lane; t < ntile_b; t += 64) Z += tp[2 * t + 1] * exp(tp[2 * t] - m);
    Z = wave_sum(Z);
    double* f = ftile + ((int64_t)b * H + h) * ntile_ws;
    for (int t = lane; t < ntile_b; t += 64) f[t] = exp(tp[2 * t] - m) / Z;
  }
  for (int i = tid; i < 2048; i += NT) { hA[i] = 0u; hB[i] = 0u; }
  __threadfence_block();
  __syncthreads();

  // ---- value weights ----
  const int per = (int)((Tp + NT - 1) / NT);
  // loop bound over owned-token rounds: a compile-time constant when the
  // weights live in registers (so that the loops unroll and index them
  // statically), the actual count otherwise
  const int kmax = REG ? kVPMAX : per;
  const double* fb = ftile + ((int64_t)b * H + (int64_t)g * GQA) * ntile_ws;
  const double* eb = ebuf + ((int64_t)b * H + (int64_t)g * GQA) * capmax;
  double* ab = aval + ((int64_t)b * G + g) * capmax;
  uint8_t* tvb = tv + ((int64_t)b * G + g) * capmax;
  double areg[REG ? kVPMAX : 1];
#pragma unroll
  for (int k = 0; k < kmax; ++k) {
    if (k >= per) break;
    const int64_t j = tid + (int64_t)NT * k;
    double a = 0.0;
    if (j < Tp) {
      const int tl = (int)(j / kTile);
      double asq = 0.0;
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) {
        const double al = __dmul_rn(eb[(int64_t)hh * capmax + j], fb[(int64_t)hh * ntile_ws + tl]);
        asq = __dadd_rn(asq, __dmul_rn(al, al));
      }
      a = (vscale == 0) ? __dmul_rn(asq, u.ev[j / kGroup]) : asq;
    }
    if constexpr (REG) areg[k] = a;
    else if (j < Tp) ab[j] = a;
  }
  auto aof = [&](int k) -> double {
    const int64_t j = tid + (int64_t)NT * k;
    if (j >= Tp) return 0.0;
    if constexpr (REG) return areg[k];
    else return ab[j];
  };

  const uint32_t Bv = (uint32_t)floor((double)RV * (double)Tp);
  const int twoW = 2 * W;

  // ---- exponent histogram: hA[E] regular tokens, hB[E] tiny tokens' gains ----
  uint32_t npos_l = 0;
#pragma unroll
  for (int k = 0; k < kmax; ++k) {
    if (k >= per) break;
    const double a = aof(k);
    const bool posv = a > 0.0;
    const int E = (int)(dbits(a) >> 52);
    const bool reg = posv && E > twoW;
    agg_add(hA, (uint32_t)E, reg);
    if (reg) npos_l += W;
    if (posv && !reg) {
      for (int t = 1; t <= W; ++t) {
        const uint64_t kk = dbits(__dmul_rn(a, ldexp_pow2(-2 * t)));
        if (kk) { atomicAdd(&hB[(uint32_t)(kk >> 52)], 1u); ++npos_l; }
      }
    }
  }
  block_excl_scan<NT>(npos_l, wsum);
  const uint32_t npos = wsum[NT / 64];
  __syncthreads();
  // hB[E] += sum_t hA[E + 2t]: the gain-exponent histogram of all candidates
  for (int E = tid; E < 2048; E += NT) {
    uint32_t s = hB[E];
    for (int t = 1; t <= W; ++t)
      if (E + 2 * t < 2048) s += hA[E + 2 * t];
    hB[E] = s;
  }
  __syncthreads();

  const bool all_pos = npos <= Bv;
  int Es = -1;
  uint64_t prefix = 0, mask = 0;  // over the 52 mantissa bits
  uint32_t rem = 0, n_eq = 0;
  if (!all_pos && Bv > 0) {
    if (tid < 64) wave_find_digit<2048>(hB, Bv, &sh[0], &sh[1]);
    __syncthreads();
    Es = (int)sh[0];
    rem = Bv - sh[1];
    n_eq = hB[Es];
    __syncthreads();
    // digits of the 52 mantissa bits: 11, 11, 10, 10, 10 (MSB first)
    for (int pass = 0; pass < 5 && n_eq != rem; ++pass) {
      const int width = pass < 2 ? 11 : 10;
      const int shift = pass < 2 ? 41 - 11 * pass : 40 - 10 * pass;
      const uint32_t dmask = (1u << width) - 1u;
      for (int i = tid; i < 2048; i += NT) hA[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kmax; ++k) {
        if (k >= per) break;
        const double a = aof(k);
        if (!(a > 0.0)) continue;
        const uint64_t ab_ = dbits(a);
        const int E = (int)(ab_ >> 52);
        if (E > twoW) {
          const int d = E - Es;
          if (d >= 2 && d <= twoW && !(d & 1)) {
            const uint64_t mnt = ab_ & 0x000FFFFFFFFFFFFFull;
            if ((mnt & mask) == prefix) atomicAdd(&hA[(uint32_t)(mnt >> shift) & dmask], 1u);
          }
        } else {
          for (int t = 1; t <= W; ++t) {
            const uint64_t kk = dbits(__dmul_rn(a, ldexp_pow2(-2 * t)));
            if (kk && (int)(kk >> 52) == Es) {
              const uint64_t mnt = kk & 0x000FFFFFFFFFFFFFull;
              if ((mnt & mask) == prefix) atomicAdd(&hA[(uint32_t)(mnt >> shift) & dmask], 1u);
            }
          }
        }
      }
      __syncthreads();
      if (tid < 64) {
        if (width == 11) wave_find_digit<2048>(hA, rem, &sh[0], &sh[1]);
        else wave_find_digit<1024>(hA, rem, &sh[0], &sh[1]);
      }
      __syncthreads();
      const uint32_t dg = sh[0];
      n_eq = hA[dg];
      rem -= sh[1];
      prefix |= (uint64_t)dg << shift;
      mask |= (uint64_t)dmask << shift;
      __syncthreads();
    }
  }

  // ---- depths: levels above the threshold, plus ties in token order ----
  // returns (levels above the threshold) | (levels equal to it) << 16
  auto count_levels = [&](double a) -> uint32_t {
    uint32_t above = 0, tie = 0;
    if (!(a > 0.0)) return 0u;
    const uint64_t ab_ = dbits(a);
    const int E = (int)(ab_ >> 52);
    if (all_pos) {
      if (E > twoW) above = (uint32_t)W;
      else
        for (int t = 1; t <= W; ++t) above += dbits(__dmul_rn(a, ldexp_pow2(-2 * t))) != 0ull;
      return above;
    }
    if (Bv == 0) return 0u;
    if (E > twoW) {
      const int d = E - Es;
      if (d > 0) {
        int n = (d - 1) >> 1;
        above = (uint32_t)(n > W ? W : n);
      }
      if (d >= 2 && d <= twoW && !(d & 1)) {
        const uint64_t mnt = (ab_ & 0x000FFFFFFFFFFFFFull) & mask;
        if (mnt > prefix) ++above;
        else if (mnt == prefix) ++tie;
      }
    } else {
      for (int t = 1; t <= W; ++t) {
        const uint64_t kk = dbits(__dmul_rn(a, ldexp_pow2(-2 * t)));
        if (!kk) continue;
        const int e = (int)(kk >> 52);
        if (e > Es) ++above;
        else if (e == Es) {
          const uint64_t mnt = (kk & 0x000FFFFFFFFFFFFFull) & mask;
          if (mnt > prefix) ++above;
          else if (mnt == prefix) ++tie;
        }
      }
    }
    return above | (tie << 16);
  };
  const bool rank_ties = !all_pos && Bv > 0 && rem < n_eq;
  uint32_t running = 0;  // ties in earlier rounds (token order = round, thread)
#pragma unroll
  for (int k = 0; k < kmax; ++k) {
    if (k >= per) break;
    const int64_t j = tid + (int64_t)NT * k;
    const uint32_t lv = count_levels(aof(k));
    uint32_t above = lv & 0xFFFFu;
    const uint32_t tie = lv >> 16;
    if (rank_ties) {
      const uint32_t before = block_excl_scan<NT>(tie, wsum) + running;
      running += wsum[NT / 64];
      __syncthreads();
      if (tie && before < rem) ++above;
    } else {
      above += tie;
    }
    if (j < Tp) tvb[j] = (uint8_t)above;
  }
}

// ---------------------------------------------------------------------------
// Gather: one block of 256 threads per 256-token chunk (8 groups) of one
// (request, KV head).
//  1. The chosen value plane rows (16 B per token and plane) are staged in
//     LDS.
//  2. Every refined token (t > 0) is un-planed: 16 lanes per token, one per
//     8-channel octet, byte gather + 8x8 bit transpose, and its prefix codes
//     X (= P 2^(8-t)) are written token-major to an LDS code tile (tokens
//     with t = 0 keep X = 0).  Deep (t > 4) and shallow tokens are processed
//     from two separate lists so that the code path is uniform per wave.
//  3. Per group gamma and head h, with e = exp(s - m_tile) rounded to fp16,
//       sum_j e_j v_hat_jc = lo_c A + rng_c (Bh + U_c / 256),
//     A = sum e, Bh = sum e 2^-(t+1), U_c = sum e X_c.  U comes from
//     v_mfma_f32_16x16x32_f16: A operand = codes of 16 channels x 32 tokens
//     (one group), read channel-major from the code tile with the LDS
//     transpose read and turned into the fp16 values 1024 + X by one byte
//     permute per pair; B operand = e for 16 columns (head, group) with
//     zeros off the column's own group, so one column set covers 16/GQA
//     groups; the 1024 A part is removed when the group is folded in.
//  4. Column partials are added per head in group order, open-group tokens
//     (exact values) are added, and the chunk partial f_{h,tile} O is
//     written.  Grid (unit, chunk): all chunks of a unit on one XCD.
// ---------------------------------------------------------------------------
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

template <int GQA, int DT>
__global__ __launch_bounds__(256) void k_gather(const uint8_t* store, const uint8_t* tv, int H, int G,
                                                int W, int64_t capmax, int ntile_ws, int nchunk_ws,
                                                const _Float16* e16, const double* ftile,
                                                float* opart) {
  constexpr int esize = DT == 0 ? 2 : 4;
  constexpr int NG = kChunk / kGroup;                       // 8 groups per chunk
  constexpr int GS = (16 / GQA < NG) ? 16 / GQA : NG;       // groups per MFMA column set
  constexpr int NSET = (NG + GS - 1) / GS;
  constexpr int XS = kDim + 8;  // code-tile row stride: rows 2 apart fall in different banks
  __shared__ uint4 vrows[kChunk * 8];                       // staged rows; reused below
  __shared__ __attribute__((aligned(16))) uint8_t xl[kChunk * XS];    // codes [token][channel]
  __shared__ __attribute__((aligned(16))) _Float16 es[GQA][kChunk];
  __shared__ uint32_t vmeta_s[NG][kDim];
  __shared__ float Ag[NG][GQA], Bg[NG][GQA];
  __shared__ uint16_t offs[kChunk];
  __shared__ uint8_t tvs[kChunk];
  __shared__ uint8_t s2t[kChunk * 8];
  __shared__ uint8_t lst[kChunk];
  __shared__ float fs[GQA];
  __shared__ uint32_t wsum[256 / 64 + 1];

  const int chunk = blockIdx.y, b = blockIdx.x / G, g = blockIdx.x % G;
  const ReqRecord r = req_of(store, b);
  const int64_t len = r.len;
  const int64_t c0 = (int64_t)chunk * kChunk;
  if (c0 >= len) return;
  const int64_t Tp = len & ~(int64_t)(kGroup - 1);
  const Unit u = unit_of(const_cast<uint8_t*>(store), r, g, G, kDim, W, esize);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tile = (int)(c0 / kTile);
  const int64_t hrow0 = (int64_t)b * H + (int64_t)g * GQA;
  const int64_t gam0 = c0 / kGroup;

  {
    const int64_t j = c0 + tid;
    tvs[tid] = (j < Tp) ? tv[((int64_t)b * G + g) * capmax + j] : (uint8_t)0;
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh)
      es[hh][tid] = (j < len) ? e16[(hrow0 + hh) * capmax + j] : (_Float16)0.0f;
    for (int i = tid; i < NG * kDim; i += 256) {
      const int gl = i / kDim, c = i % kDim;
      const int64_t gam = gam0 + gl;
      vmeta_s[gl][c] = ((gam + 1) * kGroup <= Tp) ? u.vmeta[gam * kDim + c] : 0u;
    }
    if (tid < GQA) fs[tid] = (float)ftile[(hrow0 + tid) * ntile_ws + tile];
    uint2* xz = reinterpret_cast<uint2*>(xl);
    for (int i = tid; i < kChunk * XS / 8; i += 256) xz[i] = make_uint2(0u, 0u);
  }
  __syncthreads();
  // one scan for three prefix sums: slots (12 bits), deep tokens (9 bits)
  // and shallow tokens (9 bits), packed in one word
  const uint32_t tj = tvs[tid];
  const uint32_t deep = tj > 4u ? 1u : 0u, shallow = (tj >= 1u && tj <= 4u) ? 1u : 0u;
  const uint32_t pk3 = block_excl_scan<256>(tj | (deep << 12) | (shallow << 21), wsum);
  const uint32_t tot3 = wsum[256 / 64];
  const uint32_t ex = pk3 & 0xFFFu, pd = (pk3 >> 12) & 0x1FFu, ps = pk3 >> 21;
  const int nslots = (int)(tot3 & 0xFFFu);
  const int ndeep = (int)((tot3 >> 12) & 0x1FFu);
  const int nref = ndeep + (int)(tot3 >> 21);
  offs[tid] = (uint16_t)ex;
  for (uint32_t p = 0; p < tj; ++p) s2t[ex + p] = (uint8_t)tid;
  if (deep) lst[pd] = (uint8_t)tid;
  if (shallow) lst[ndeep + ps] = (uint8_t)tid;
  __syncthreads();

  // ---- 1. stage the chosen rows ----
  {
    const uint4* vp = reinterpret_cast<const uint4*>(u.vplanes);
    for (int base = 0; base < nslots; base += 256 * 8) {
      uint4 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int s = base + k * 256 + tid;
        v[k] = make_uint4(0u, 0u, 0u, 0u);
        if (s < nslots) {
          const int jl = s2t[s];
          const int p = s - offs[jl];
          v[k] = vp[(c0 + jl) * W + p];
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int s = base + k * 256 + tid;
        if (s < nslots) vrows[s] = v[k];
      }
    }
  }
  // per-group sums of e (A) and of e 2^-(t+1) (Bh): TPP threads per
  // (group, head), each over 32/TPP tokens, then a shuffle reduction
  {
    constexpr int NP = NG * GQA;
    constexpr int TPP = NP <= 8 ? 32 : (NP <= 16 ? 16 : (NP <= 32 ? 8 : 4));
    constexpr int TK = kGroup / TPP;
    const int pr = tid / TPP, part = tid % TPP;
    float a = 0.f, bh = 0.f;
    if (pr < NP) {
      const int gl = pr / GQA, hh = pr % GQA;
#pragma unroll
      for (int k = 0; k < TK; ++k) {
        const int jl = kGroup * gl + part * TK + k;
        const float e = (float)es[hh][jl];
        a += e;
        bh = fmaf(e, ldexp_pow2f(-(int)tvs[jl] - 1), bh);
      }
    }
    a = group_sum<TPP>(a);
    bh = group_sum<TPP>(bh);
    if (pr < NP && part == 0) {
      Ag[pr / GQA][pr % GQA] = a;
      Bg[pr / GQA][pr % GQA] = bh;
    }
  }
  __syncthreads();

  // ---- 2. un-plane refined tokens into the code tile ----
  {
    const int bo = lane & 15, wb = bo >> 2, ob = bo & 3;
    const uint32_t sel = 0x0C0C0000u | ((4u + (uint32_t)ob) << 8) | (uint32_t)ob;
    const uint32_t* rows = reinterpret_cast<const uint32_t*>(vrows);
    for (int i = 4 * wv + (lane >> 4); i < ndeep; i += 16) {
      const int jl = lst[i];
      const int t = tvs[jl], s0 = offs[jl];
      uint32_t w[8];
#pragma unroll
      for (int p = 0; p < 8; ++p) w[p] = (p < t) ? rows[(s0 + p) * 4 + wb] : 0u;
      uint32_t lo, hi;
      unplane8(w, sel, lo, hi);
      *reinterpret_cast<uint2*>(xl + jl * XS + 8 * bo) = make_uint2(lo, hi);
    }
    for (int i = ndeep + 4 * wv + (lane >> 4); i < nref; i += 16) {
      const int jl = lst[i];
      const int t = tvs[jl], s0 = offs[jl];
      const uint32_t w0 = rows[s0 * 4 + wb];
      const uint32_t w1 = t > 1 ? rows[(s0 + 1) * 4 + wb] : 0u;
      const uint32_t w2 = t > 2 ? rows[(s0 + 2) * 4 + wb] : 0u;
      const uint32_t w3 = t > 3 ? rows[(s0 + 3) * 4 + wb] : 0u;
      uint32_t lo, hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(w0, w1, sel),
                                              __builtin_amdgcn_perm(w2, w3, sel), 0x05040100u);
      transpose8_hi4(lo, hi);
      *reinterpret_cast<uint2*>(xl + jl * XS + 8 * bo) = make_uint2(lo, hi);
    }
  }
  __syncthreads();

  // ---- 3. MFMA per (16-channel block, column set); wave wv: blocks 2wv, 2wv+1 ----
  const int m = lane & 15, kb = lane >> 4;
  const int gp = m / GQA, hn = m % GQA;
  const bool colv = m < GS * GQA;
  float Oacc[2][4];
#pragma unroll
  for (int bl = 0; bl < 2; ++bl)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) Oacc[bl][rr] = 0.f;
  for (int set = 0; set < NSET; ++set) {
    const int gbase = set * GS;
#pragma unroll
    for (int bl = 0; bl < 2; ++bl) {
      const int cb = 16 * (2 * wv + bl);
      f32x4 D = {0.f, 0.f, 0.f, 0.f};
      for (int gi = 0; gi < GS; ++gi) {
        const int gl = gbase + gi;
        if (gl >= NG || (gam0 + gl + 1) * kGroup > Tp) continue;
        const int t0 = kGroup * gl + 8 * kb;
        const uint8_t* src = xl + (t0 + (m >> 1)) * XS + cb + 8 * (m & 1);
        const i32x2 xv = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)src);
        uint32_t ap[4];
        ap[0] = __builtin_amdgcn_perm(0x64646464u, (uint32_t)xv.x, 0x04010400u);
        ap[1] = __builtin_amdgcn_perm(0x64646464u, (uint32_t)xv.x, 0x04030402u);
        ap[2] = __builtin_amdgcn_perm(0x64646464u, (uint32_t)xv.y, 0x04010400u);
        ap[3] = __builtin_amdgcn_perm(0x64646464u, (uint32_t)xv.y, 0x04030402u);
        const f16x8 av = __builtin_bit_cast(f16x8, ap);
        f16x8 bv = {0, 0, 0, 0, 0, 0, 0, 0};
        if (colv && gp == gi) bv = *reinterpret_cast<const f16x8*>(&es[hn][t0]);
        D = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, D, 0, 0, 0);
      }
      // fold: D row = channel cb + 4 kb + rr, column m = (gp, hn)
      const int gl = gbase + gp;
      if (colv && gl < NG && (gam0 + gl + 1) * kGroup <= Tp) {
        const float A = Ag[gl][hn], Bh = Bg[gl][hn];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const uint32_t mt = vmeta_s[gl][cb + 4 * kb + rr];
          const float lo = bf16_to_float(mt & 0xFFFFu), rng = bf16_to_float(mt >> 16);
          Oacc[bl][rr] += fmaf(lo, A, rng * (Bh + (D[rr] - 1024.f * A) * (1.f / 256.f)));
        }
      }
    }
  }
  __syncthreads();
  float* red2 = reinterpret_cast<float*>(vrows);  // [16 columns][128 channels]
#pragma unroll
  for (int bl = 0; bl < 2; ++bl)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) red2[m * kDim + 16 * (2 * wv + bl) + 4 * kb + rr] = Oacc[bl][rr];
  __syncthreads();

  // ---- 4. per-head sums over the column groups, open group, chunk partial ----
  const int64_t jt0 = Tp > c0 ? Tp : c0;
  const int64_t jt1 = len < c0 + kChunk ? len : c0 + kChunk;
  for (int o = tid; o < GQA * kDim; o += 256) {
    const int hh = o / kDim, c = o % kDim;
    float s = 0.f;
    for (int q = 0; q < GS; ++q) s += red2[(q * GQA + hh) * kDim + c];
    for (int64_t j = jt0; j < jt1; ++j)
      s = fmaf((float)es[hh][j - c0], load_elem_f<DT>(u.vtail, (j - Tp) * kDim + c), s);
    opart[((hrow0 + hh) * nchunk_ws + chunk) * kDim + c] = s * fs[hh];
  }
}

// out[b][h][c] = sum over the request's chunks, in chunk order.  One thread
// per output element; the chunk loads are independent.
__global__ __launch_bounds__(256) void k_out_reduce(const uint8_t* store, int H, int nchunk_ws,
                                                    int64_t nout, const float* opart, float* out) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= nout) return;
  const int64_t bh = o / kDim;
  const int c = (int)(o - bh * kDim);
  const int b = (int)(bh / H);
  const ReqRecord r = req_of(store, b);
  const int nch = (int)((r.len + kChunk - 1) / kChunk);
  const float* p = opart + bh * nchunk_ws * kDim + c;
  float s = 0.f;
  int ch = 0;
  for (; ch + 4 <= nch; ch += 4) {
    const float v0 = p[(int64_t)ch * kDim], v1 = p[(int64_t)(ch + 1) * kDim];
    const float v2 = p[(int64_t)(ch + 2) * kDim], v3 = p[(int64_t)(ch + 3) * kDim];
    s += v0;
    s += v1;
    s += v2;
    s += v3;
  }
  for (; ch < nch; ++ch) s += p[(int64_t)ch * kDim];
  out[o] = s;
}

// ---------------------------------------------------------------------------
static inline void mark(const DecodeArgs& a, int i, hipStream_t st) {
  if (a.events) hipEventRecord((hipEvent_t)a.events[i], st);
}

template <int GQA, int DT>
static int launch_all(const DecodeArgs& a, const WsLayout& L, hipStream_t st) {
  uint8_t* ws = a.ws;
  uint8_t* tk = a.key_depths_out ? a.key_depths_out : ws + L.tk;
  uint8_t* tv = a.value_depths_out ? a.value_depths_out : ws + L.tv;
  const int esize = DT == 0 ? 2 : 4;

  mark(a, 0, st);
  hipLaunchKernelGGL((k_key_alloc<DT>), dim3(a.B * a.G), dim3(64), 0, st, (const uint8_t*)a.store,
                     a.q, a.H, a.G, a.W, a.RK, tk);
  mark(a, 1, st);
  // slots staged per score tile: at most min(B_K, 128 W) chosen key lines
  double bk = floor((double)a.RK * (double)kDim);
  if (bk > (double)(kDim * a.W)) bk = (double)(kDim * a.W);
  size_t dyn = (size_t)(kTile / kGroup) * (size_t)(((int)bk) | 1) * 4;
  const size_t dyn_red = (size_t)2 * 64 * 8 * GQA * 8;  // wave reduction buffers
  if (dyn < dyn_red) dyn = dyn_red;
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(&k_score<GQA, DT>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, 16 * 1025 * 4 + 64);
    attr_set = true;
  }
  hipLaunchKernelGGL((k_score<GQA, DT>), dim3(a.B * a.G, L.ntile), dim3(256), dyn, st,
                     (const uint8_t*)a.store, a.q, (const uint8_t*)tk, a.H, a.G, a.W, a.capmax,
                     L.ntile, (double*)(ws + L.ebuf), (_Float16*)(ws + L.e16),
                     (double*)(ws + L.tilepart));
  mark(a, 2, st);
  if (a.capmax <= (int64_t)kVNT * kVPMAX)
    hipLaunchKernelGGL((k_value_alloc<GQA, true>), dim3(a.B * a.G), dim3(kVNT), 0, st,
                       (const uint8_t*)a.store, a.H, a.G, a.W, esize, a.RV, a.vscale, a.capmax,
                       L.ntile, (const double*)(ws + L.ebuf), (const double*)(ws + L.tilepart),
                       (double*)(ws + L.ftile), (double*)(ws + L.aval), tv);
  else
    hipLaunchKernelGGL((k_value_alloc<GQA, false>), dim3(a.B * a.G), dim3(kVNT), 0, st,
                       (const uint8_t*)a.store, a.H, a.G, a.W, esize, a.RV, a.vscale, a.capmax,
                       L.ntile, (const double*)(ws + L.ebuf), (const double*)(ws + L.tilepart),
                       (double*)(ws + L.ftile), (double*)(ws + L.aval), tv);
  mark(a, 3, st);
  hipLaunchKernelGGL((k_gather<GQA, DT>), dim3(a.B * a.G, L.nchunk), dim3(256), 0, st,
                     (const uint8_t*)a.store, (const uint8_t*)tv, a.H, a.G, a.W, a.capmax, L.ntile,
                     L.nchunk, (const _Float16*)(ws + L.e16), (const double*)(ws + L.ftile),
                     (float*)(ws + L.opart));
  const int64_t nout = (int64_t)a.B * a.H * kDim;
  hipLaunchKernelGGL(k_out_reduce, dim3((unsigned)((nout + 255) / 256)), dim3(256), 0, st,
                     (const uint8_t*)a.store, a.H, L.nchunk, nout, (const float*)(ws + L.opart),
                     a.out);
  mark(a, 4, st);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

template <int DT>
static int dispatch_gqa(const DecodeArgs& a, const WsLayout& L, hipStream_t st) {
  switch (a.H / a.G) {
    case 1: return launch_all<1, DT>(a, L, st);
    case 2: return launch_all<2, DT>(a, L, st);
    case 3: return launch_all<3, DT>(a, L, st);
    case 4: return launch_all<4, DT>(a, L, st);
    case 5: return launch_all<5, DT>(a, L, st);
    case 6: return launch_all<6, DT>(a, L, st);
    case 7: return launch_all<7, DT>(a, L, st);
    case 8: return launch_all<8, DT>(a, L, st);
    default: return -5;
  }
}

int launch_decode(const DecodeArgs& a, hipStream_t st) {
  const WsLayout L = ws_layout(a.B, a.H, a.G, kDim, a.capmax);
  return a.dtype == 0 ? dispatch_gqa<0>(a, L, st) : dispatch_gqa<1>(a, L, st);
}

}  // namespace readkv
