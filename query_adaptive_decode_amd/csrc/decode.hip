// One ReadKV decode step ("Read What Matters: Query-Adaptive Quantization
// for KV Caches", Sec. 3.2-3.3, Algorithm 1) as five launches on one stream:
//
//   k_key_alloc   (B*G blocks)        key weights (Eq. (2)) and ChooseDepths
//                                     over the d_h channels -> t^K
//   k_score       (tiles x G x B)     prefix-gather of the chosen key planes,
//                                     reconstructed logits, per-tile max and
//                                     sum of exp (split-context softmax)
//   k_value_alloc (B*G blocks)        softmax statistics, value weights
//                                     (Eq. (3)) and ChooseDepths over the
//                                     packed tokens -> t^V
//   k_gather      (chunks x G x B)    prefix-gather of the chosen value planes
//                                     and attention-weighted sum per chunk
//   k_out_reduce  (B*H blocks)        fixed-order sum of the chunk partials
//
// The k_value_alloc -> k_gather boundary is the staged(2) reader's second
// batch: value reads depend on attention computed from the first batch.
//
// Reconstruction of a depth-t prefix P (t MSB-first planes) of a group with
// metadata (lo, rng): x_hat = lo + rng * (2P + 1) / 2^(t+1).  The kernels
// un-plane an 8-element byte column into X = P * 2^(8-t) (missing planes
// read as zero) and use x_hat = lo + rng * (2X + 2^(8-t)) / 512.
#include <math.h>

#include "kernels_common.h"
#include "readkv_internal.h"
#include "select.h"

namespace readkv {

// ---------------------------------------------------------------------------
// Key allocation: one block of 256 threads per (request, KV head).  Thread
// 2c+h holds the gains of channel c at levels 4h+1 .. 4h+4.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void k_key_alloc(const uint8_t* store, const void* q, int H, int G,
                                                   int W, float RK, uint8_t* tk) {
  constexpr int NT = 256;
  constexpr int esize = DT == 0 ? 2 : 4;
  const int b = blockIdx.x / G, g = blockIdx.x % G;
  const int gqa = H / G;
  const ReqRecord r = req_of(store, b);
  const Unit u = unit_of(const_cast<uint8_t*>(store), r, g, G, kDim, W, esize);
  const int tid = threadIdx.x;
  const int c = tid >> 1, half = tid & 1;

  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[NT / 64 + 1];
  __shared__ uint32_t sh[2];

  // key weight, Eq. (2): (sum_h q_hc^2) * (sum over groups of rng_c^2)
  double qsq = 0.0;
  for (int hh = 0; hh < gqa; ++hh) {
    const double qv = load_elem<DT>(q, ((int64_t)b * H + (int64_t)g * gqa + hh) * kDim + c);
    qsq = qsq + qv * qv;
  }
  const double w = qsq * u.ek[c];
  uint64_t key[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int t = half * 4 + m + 1;
    key[m] = (t <= W) ? dbits(w * ldexp_pow2(-2 * t)) : 0ull;
  }
  const uint32_t k = (uint32_t)floor((double)RK * (double)kDim);

  // ---- threshold search (8 passes of 8 bits) ----
  uint32_t npos_l = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) npos_l += key[m] > 0;
  block_excl_scan<NT>(npos_l, wsum);
  const uint32_t npos = wsum[NT / 64];
  __syncthreads();
  uint64_t prefix = 0, mask = 0;
  uint32_t rem = k, n_eq = 0;
  const bool all_pos = npos <= k;
  if (!all_pos && k > 0) {
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      hist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (key[m] > 0 && (key[m] & mask) == prefix)
          atomicAdd(&hist[(uint32_t)(key[m] >> shift) & 255u], 1u);
      __syncthreads();
      if (tid < 64) wave_find_digit<256>(hist, rem, &sh[0], &sh[1]);
      __syncthreads();
      const uint32_t d = sh[0];
      const uint32_t cnt = hist[d];
      rem -= sh[1];
      prefix |= (uint64_t)d << shift;
      mask |= 0xFFull << shift;
      n_eq = cnt;
      __syncthreads();
      if (cnt == rem) break;
    }
  }
  // ---- count chosen levels ----
  uint32_t sel = 0, tie = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (key[m] == 0) continue;
    if (all_pos) { ++sel; continue; }
    if (k == 0) continue;
    const uint64_t km = key[m] & mask;
    if (km > prefix) ++sel;
    else if (km == prefix) ++tie;
  }
  if (!all_pos && k > 0 && rem < n_eq) {
    // ties resolved toward the lowest channel (thread order = channel order)
    const uint32_t before = block_excl_scan<NT>(tie, wsum);
    if (tie && before < rem) ++sel;
  } else {
    sel += tie;
  }
  sel += __shfl_xor(sel, 1, 64);
  if (half == 0) tk[((int64_t)b * G + g) * kDim + c] = (uint8_t)sel;
}

// ---------------------------------------------------------------------------
// Score: block of 128 threads per 1024-token tile of one (request, KV head).
// Thread (gs, k) = (tid/4, tid%4) owns tokens 8k..8k+7 of group gs of the
// tile and loops over the channels with t^K_c > 0.  Logits are fp64:
//   s_hj = [ sum_c q_hc (lo + rng 2^-(t_c+1)) + sum_c (q_hc rng / 256) X_jc ] / sqrt(d)
// The block writes e_hj = exp(s_hj - m_tile) and (m_tile, sum_j e_hj).
// ---------------------------------------------------------------------------
template <int GQA, int DT>
__global__ __launch_bounds__(128) void k_score(const uint8_t* store, const void* q, const uint8_t* tk,
                                               int H, int G, int W, int64_t capmax, int ntile_ws,
                                               double* ebuf, double* tilepart) {
  constexpr int esize = DT == 0 ? 2 : 4;
  const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const ReqRecord r = req_of(store, b);
  const int64_t len = r.len;
  const int64_t t0 = (int64_t)tile * kKeyTile;
  if (t0 >= len) return;
  const int64_t Tp = len & ~(int64_t)(kGroup - 1);
  const Unit u = unit_of(const_cast<uint8_t*>(store), r, g, G, kDim, W, esize);
  const int tid = threadIdx.x;

  __shared__ double qs[GQA][kDim];
  __shared__ uint8_t ts[kDim];
  __shared__ uint8_t act[kDim];
  __shared__ int nact_s[2];
  __shared__ double red[2][GQA];

  for (int hh = 0; hh < GQA; ++hh)
    qs[hh][tid] = load_elem<DT>(q, ((int64_t)b * H + (int64_t)g * GQA + hh) * kDim + tid);
  const uint8_t tc = tk[((int64_t)b * G + g) * kDim + tid];
  ts[tid] = tc;
  {
    const uint64_t bal = __ballot(tc > 0);
    const int lane = tid & 63, w = tid >> 6;
    const uint32_t rank = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) nact_s[w] = __popcll(bal);
    __syncthreads();
    if (tc > 0) act[rank + (w ? nact_s[0] : 0)] = (uint8_t)tid;
  }
  __syncthreads();
  const int nact = nact_s[0] + nact_s[1];
  const double inv_sqrt_d = 0.088388347648318440550;  // 1/sqrt(128)

  const int gs = tid >> 2, k = tid & 3;
  const int64_t gam = (int64_t)tile * (kKeyTile / kGroup) + gs;
  const bool packed = (gam + 1) * kGroup <= Tp;
  double sv[8][GQA];

  if (packed) {
    double C[GQA];
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) C[hh] = 0.0;
    for (int c = k; c < kDim; c += 4) {
      const uint32_t m = u.kmeta[gam * kDim + c];
      const double lo = (double)bf16_to_float(m & 0xFFFFu);
      const double rng = (double)bf16_to_float(m >> 16);
      const double base = lo + rng * ldexp_pow2(-(int)ts[c] - 1);
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) C[hh] = fma(qs[hh][c], base, C[hh]);
    }
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) {
      C[hh] += __shfl_xor(C[hh], 1, 64);
      C[hh] += __shfl_xor(C[hh], 2, 64);
    }
    double acc[8][GQA];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) acc[i][hh] = 0.0;
    for (int ai = 0; ai < nact; ++ai) {
      const int c = act[ai];
      const int t = ts[c];
      const double rng = (double)bf16_to_float(u.kmeta[gam * kDim + c] >> 16);
      double beta[GQA];
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) beta[hh] = qs[hh][c] * rng * (1.0 / 256.0);
      const uint32_t* line = u.kplanes + (int64_t)c * W * u.ng + gam;
      uint64_t x = 0;
      for (int p = 0; p < t; ++p) {
        const uint32_t wd = line[(int64_t)p * u.ng];
        x |= (uint64_t)((wd >> (8 * k)) & 0xFFu) << (8 * (7 - p));
      }
      const uint64_t y = transpose8(x);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double xv = (double)(uint32_t)((y >> (8 * i)) & 0xFFu);
#pragma unroll
        for (int hh = 0; hh < GQA; ++hh) acc[i][hh] = fma(beta[hh], xv, acc[i][hh]);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) sv[i][hh] = (C[hh] + acc[i][hh]) * inv_sqrt_d;
  }

  // open-group tokens: exact keys.  The open group is group Tp/32, which
  // lies in tile Tp/1024; thread (rr, k) takes slot rr, channels 32k..32k+31.
  const int64_t ntail = len - Tp;
  const bool tail_tile = ntail > 0 && Tp / kKeyTile == tile;
  const int rr = tid >> 2;
  const bool has_tail = tail_tile && rr < ntail && k == 0;
  double st[GQA];
#pragma unroll
  for (int hh = 0; hh < GQA; ++hh) st[hh] = 0.0;
  if (tail_tile) {
    if (rr < ntail) {
      for (int c = k * 32; c < k * 32 + 32; ++c) {
        const double kv = load_elem<DT>(u.ktail, (int64_t)rr * kDim + c);
#pragma unroll
        for (int hh = 0; hh < GQA; ++hh) st[hh] = fma(qs[hh][c], kv, st[hh]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) {
      st[hh] += __shfl_xor(st[hh], 1, 64);
      st[hh] += __shfl_xor(st[hh], 2, 64);
      st[hh] *= inv_sqrt_d;
    }
  }

  // ---- split-context softmax partials for this tile ----
  double mloc[GQA];
#pragma unroll
  for (int hh = 0; hh < GQA; ++hh) {
    double m = has_tail ? st[hh] : -INFINITY;
    if (packed)
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmax(m, sv[i][hh]);
    m = wave_max(m);
    if ((tid & 63) == 0) red[tid >> 6][hh] = m;
  }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < GQA; ++hh) mloc[hh] = fmax(red[0][hh], red[1][hh]);
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < GQA; ++hh) {
    double z = 0.0;
    double* ep = ebuf + ((int64_t)b * H + (int64_t)g * GQA + hh) * capmax;
    if (packed) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double e = exp(sv[i][hh] - mloc[hh]);
        ep[gam * kGroup + 8 * k + i] = e;
        z += e;
      }
    }
    if (has_tail) {
      const double e = exp(st[hh] - mloc[hh]);
      ep[Tp + rr] = e;
      z += e;
    }
    z = wave_sum(z);
    if ((tid & 63) == 0) red[tid >> 6][hh] = z;
  }
  __syncthreads();
  if (tid < GQA) {
    double* tp = tilepart + (((int64_t)b * H + (int64_t)g * GQA + tid) * ntile_ws + tile) * 2;
    tp[0] = mloc[tid];
    tp[1] = red[0][tid] + red[1][tid];
  }
}

// ---------------------------------------------------------------------------
// Value allocation: one block of 1024 threads per (request, KV head).
//   m_h = max_tile m_tile, Z_h = sum_tile z_tile exp(m_tile - m_h)
//   f_{h,tile} = exp(m_tile - m_h) / Z_h       (alpha_hat = e * f)
//   a_j = (sum_h alpha_hat_hj^2) * s_gamma(j)  (Eq. (3))
// then ChooseDepths with B_V = floor(R_V * T_packed) over (token, level)
// gains a_j 4^-t.  Threshold search: first pass on the 11-bit exponent of
// the gains (a token's W gains land in bins e_j - 2, ..., e_j - 2W), then
// 9,9,9,9,8,8-bit mantissa passes.
// ---------------------------------------------------------------------------
constexpr int kVNT = 1024;

template <bool REG>
__global__ __launch_bounds__(1024) void k_value_alloc(const uint8_t* store, int H, int G, int W,
                                                      int esize, float RV, int vscale,
                                                      int64_t capmax, int ntile_ws,
                                                      const double* ebuf, const double* tilepart,
                                                      double* ftile, double* aval, uint8_t* tv) {
  constexpr int NT = kVNT;
  constexpr int PMAX = 16;
  const int b = blockIdx.x / G, g = blockIdx.x % G;
  const int gqa = H / G;
  const ReqRecord r = req_of(store, b);
  const int64_t len = r.len;
  const int64_t Tp = len & ~(int64_t)(kGroup - 1);
  const int ntile_b = (int)((len + kKeyTile - 1) / kKeyTile);
  const Unit u = unit_of(const_cast<uint8_t*>(store), r, g, G, kDim, W, esize);
  const int tid = threadIdx.x;

  __shared__ uint32_t hA[2048];
  __shared__ uint32_t hB[2048];
  __shared__ uint32_t wsum[NT / 64 + 1];
  __shared__ uint32_t sh[2];

  // ---- softmax statistics -> per-tile factors ----
  if (tid < gqa) {
    const int h = g * gqa + tid;
    const double* tp = tilepart + ((int64_t)b * H + h) * ntile_ws * 2;
    double m = -INFINITY;
    for (int t = 0; t < ntile_b; ++t) m = fmax(m, tp[2 * t]);
    double Z = 0.0;
    for (int t = 0; t < ntile_b; ++t) Z += tp[2 * t + 1] * exp(tp[2 * t] - m);
    double* f = ftile + ((int64_t)b * H + h) * ntile_ws;
    for (int t = 0; t < ntile_b; ++t) f[t] = exp(tp[2 * t] - m) / Z;
  }
  __syncthreads();

  // ---- value weights for owned tokens (blocked ownership) ----
  const int64_t per = (Tp + NT - 1) / NT;
  const int64_t j0 = (int64_t)tid * per;
  const int64_t j1 = (j0 + per < Tp) ? j0 + per : Tp;
  const double* fb = ftile + ((int64_t)b * H + (int64_t)g * gqa) * ntile_ws;
  const double* eb = ebuf + ((int64_t)b * H + (int64_t)g * gqa) * capmax;
  double* ab = aval + ((int64_t)b * G + g) * capmax;
  uint8_t* tvb = tv + ((int64_t)b * G + g) * capmax;
  double areg[REG ? PMAX : 1];
  for (int64_t j = j0; j < j1; ++j) {
    double asq = 0.0;
    const int tl = (int)(j / kKeyTile);
    for (int hh = 0; hh < gqa; ++hh) {
      const double al = eb[(int64_t)hh * capmax + j] * fb[(int64_t)hh * ntile_ws + tl];
      asq = asq + al * al;
    }
    const double a = (vscale == 0) ? asq * u.ev[j / kGroup] : asq;
    if constexpr (REG) areg[j - j0] = a; else ab[j] = a;
  }
  auto aof = [&](int64_t j) -> double {
    if constexpr (REG) return areg[j - j0]; else return ab[j];
  };

  const uint32_t k = (uint32_t)floor((double)RV * (double)Tp);
  const uint32_t twoW = 2u * (uint32_t)W;

  // ---- pass 1: exponent histogram of all candidate gains ----
  for (int i = tid; i < 2048; i += NT) { hA[i] = 0; hB[i] = 0; }
  __syncthreads();
  uint32_t npos_l = 0;
  for (int64_t j = j0; j < j1; ++j) {
    const double a = aof(j);
    if (!(a > 0.0)) continue;
    const uint32_t e = (uint32_t)(dbits(a) >> 52);
    if (e > twoW) {
      atomicAdd(&hA[e], 1u);
      npos_l += W;
    } else {
      for (int t = 1; t <= W; ++t) {
        const uint64_t kk = dbits(a * ldexp_pow2(-2 * t));
        if (kk) { atomicAdd(&hB[(uint32_t)(kk >> 52)], 1u); ++npos_l; }
      }
    }
  }
  block_excl_scan<NT>(npos_l, wsum);
  const uint32_t npos = wsum[NT / 64];
  __syncthreads();
  // combine: hB[E] += sum_t hA[E + 2t]
  for (int E = tid; E < 2048; E += NT) {
    uint32_t s = hB[E];
    for (int t = 1; t <= W; ++t)
      if (E + 2 * t < 2048) s += hA[E + 2 * t];
    hB[E] = s;  // each thread only touches its own E; hA is read-only here
  }
  __syncthreads();

  uint64_t prefix = 0, mask = 0;
  uint32_t rem = k, n_eq = 0;
  const bool all_pos = npos <= k;
  if (!all_pos && k > 0) {
    if (tid < 64) wave_find_digit<2048>(hB, rem, &sh[0], &sh[1]);
    __syncthreads();
    {
      const uint32_t d = sh[0];
      n_eq = hB[d];
      rem -= sh[1];
      prefix = (uint64_t)d << 52;
      mask = 0xFFFull << 52;
    }
    __syncthreads();
    const int shifts[6] = {43, 34, 25, 16, 8, 0};
    const int widths[6] = {9, 9, 9, 9, 8, 8};
    for (int pass = 0; pass < 6 && n_eq != rem; ++pass) {
      const int shift = shifts[pass];
      const uint32_t dmask = (1u << widths[pass]) - 1u;
      for (int i = tid; i < 512; i += NT) hA[i] = 0;
      __syncthreads();
      const uint32_t Estar = (uint32_t)(prefix >> 52);
      for (int64_t j = j0; j < j1; ++j) {
        const double a = aof(j);
        if (!(a > 0.0)) continue;
        const uint64_t ab_ = dbits(a);
        const uint32_t e = (uint32_t)(ab_ >> 52);
        if (e > twoW) {
          const int dd = (int)e - (int)Estar;
          if (dd < 2 || dd > (int)twoW || (dd & 1)) continue;
          const uint64_t kk = ab_ - ((uint64_t)dd << 52);
          if ((kk & mask) == prefix) atomicAdd(&hA[(uint32_t)(kk >> shift) & dmask], 1u);
        } else {
          for (int t = 1; t <= W; ++t) {
            const uint64_t kk = dbits(a * ldexp_pow2(-2 * t));
            if (kk && (kk & mask) == prefix) atomicAdd(&hA[(uint32_t)(kk >> shift) & dmask], 1u);
          }
        }
      }
      __syncthreads();
      if (tid < 64) {
        if (widths[pass] == 9) wave_find_digit<512>(hA, rem, &sh[0], &sh[1]);
        else wave_find_digit<256>(hA, rem, &sh[0], &sh[1]);
      }
      __syncthreads();
      const uint32_t d = sh[0];
      n_eq = hA[d];
      rem -= sh[1];
      prefix |= (uint64_t)d << shift;
      mask |= (uint64_t)dmask << shift;
      __syncthreads();
    }
  }

  // ---- depths ----
  auto count_levels = [&](double a, uint32_t& sel, uint32_t& tie) {
    sel = 0;
    tie = 0;
    if (!(a > 0.0)) return;
    for (int t = 1; t <= W; ++t) {
      const uint64_t kk = dbits(a * ldexp_pow2(-2 * t));
      if (!kk) continue;
      if (all_pos) { ++sel; continue; }
      if (k == 0) continue;
      const uint64_t km = kk & mask;
      if (km > prefix) ++sel;
      else if (km == prefix) ++tie;
    }
  };
  uint32_t before = 0;
  const bool rank_ties = !all_pos && k > 0 && rem < n_eq;
  if (rank_ties) {
    uint32_t mytie = 0;
    for (int64_t j = j0; j < j1; ++j) {
      uint32_t s_, t_;
      count_levels(aof(j), s_, t_);
      mytie += t_;
    }
    before = block_excl_scan<NT>(mytie, wsum);
  }
  for (int64_t j = j0; j < j1; ++j) {
    uint32_t s_, t_;
    count_levels(aof(j), s_, t_);
    if (t_) {
      if (!rank_ties) s_ += t_;
      else if (before < rem) ++s_;
      before += t_;
    }
    tvb[j] = (uint8_t)s_;
  }
}

// ---------------------------------------------------------------------------
// Gather: block of 256 threads per 256-token chunk of one (request, KV head).
// Thread (s, k) = (tid/16, tid%16) handles tokens s, s+16, ... of the chunk
// and channels 8k..8k+7: it reads byte k of each of the token's t^V_j plane
// rows, un-planes them and accumulates alpha_hat * v_hat in fp32.
// ---------------------------------------------------------------------------
template <int GQA, int DT>
__global__ __launch_bounds__(256) void k_gather(const uint8_t* store, const uint8_t* tv, int H, int G,
                                                int W, int64_t capmax, int ntile_ws, int nchunk_ws,
                                                const double* ebuf, const double* ftile,
                                                float* opart) {
  constexpr int esize = DT == 0 ? 2 : 4;
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const ReqRecord r = req_of(store, b);
  const int64_t len = r.len;
  const int64_t c0 = (int64_t)chunk * kValChunk;
  if (c0 >= len) return;
  const int64_t Tp = len & ~(int64_t)(kGroup - 1);
  const Unit u = unit_of(const_cast<uint8_t*>(store), r, g, G, kDim, W, esize);
  const int tid = threadIdx.x;

  __shared__ float al_s[GQA][kValChunk];
  __shared__ float lo_s[kValChunk / kGroup][kDim];
  __shared__ float rs_s[kValChunk / kGroup][kDim];
  __shared__ uint8_t tv_s[kValChunk];
  __shared__ float red[4][GQA][kDim];

  {
    const int64_t j = c0 + tid;
    if (j < len) {
      tv_s[tid] = (j < Tp) ? tv[((int64_t)b * G + g) * capmax + j] : 0;
      const int tl = (int)(j / kKeyTile);
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) {
        const int64_t hrow = (int64_t)b * H + (int64_t)g * GQA + hh;
        al_s[hh][tid] = (float)(ebuf[hrow * capmax + j] * ftile[hrow * ntile_ws + tl]);
      }
    }
    for (int i = tid; i < (kValChunk / kGroup) * kDim; i += 256) {
      const int gl = i / kDim, c = i % kDim;
      const int64_t gam = c0 / kGroup + gl;
      if ((gam + 1) * kGroup <= Tp) {
        const uint32_t m = u.vmeta[gam * kDim + c];
        lo_s[gl][c] = bf16_to_float(m & 0xFFFFu);
        rs_s[gl][c] = bf16_to_float(m >> 16) * (1.0f / 512.0f);
      }
    }
  }
  __syncthreads();

  const int s = tid >> 4, k = tid & 15;
  float acc[8][GQA];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) acc[i][hh] = 0.f;
  const uint8_t* vbytes = reinterpret_cast<const uint8_t*>(u.vplanes);
  for (int it = 0; it < kValChunk / 16; ++it) {
    const int jl = s + 16 * it;
    const int64_t j = c0 + jl;
    if (j >= len) break;
    float v[8];
    if (j < Tp) {
      const int t = tv_s[jl];
      const int gl = jl >> 5;
      uint64_t x = 0;
      const uint8_t* row = vbytes + (j * W) * (kDim / 8) + k;
      for (int p = 0; p < t; ++p) x |= (uint64_t)row[p * (kDim / 8)] << (8 * (7 - p));
      const uint64_t y = transpose8(x);
      const float half = (float)(256 >> t);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float X = (float)(uint32_t)((y >> (8 * i)) & 0xFFu);
        v[i] = fmaf(rs_s[gl][8 * k + i], fmaf(2.0f, X, half), lo_s[gl][8 * k + i]);
      }
    } else {
      const int64_t slot = j - Tp;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = load_elem_f<DT>(u.vtail, slot * kDim + 8 * k + i);
    }
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) {
      const float a = al_s[hh][jl];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i][hh] = fmaf(a, v[i], acc[i][hh]);
    }
  }
  // reduce the 4 token slots of each wave, then the 4 waves
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) {
      float vv = acc[i][hh];
      vv += __shfl_xor(vv, 16, 64);
      vv += __shfl_xor(vv, 32, 64);
      acc[i][hh] = vv;
    }
  if ((tid & 63) < 16) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) red[tid >> 6][hh][8 * k + i] = acc[i][hh];
  }
  __syncthreads();
  for (int o = tid; o < GQA * kDim; o += 256) {
    const int hh = o / kDim, c = o % kDim;
    const float sum = (red[0][hh][c] + red[1][hh][c]) + (red[2][hh][c] + red[3][hh][c]);
    opart[(((int64_t)b * H + (int64_t)g * GQA + hh) * nchunk_ws + chunk) * kDim + c] = sum;
  }
}

// out[b][h][c] = sum over the request's chunks, in chunk order.
__global__ __launch_bounds__(128) void k_out_reduce(const uint8_t* store, int H, int nchunk_ws,
                                                    const float* opart, float* out) {
  const int bh = blockIdx.x;
  const int b = bh / H;
  const ReqRecord r = req_of(store, b);
  const int nch = (int)((r.len + kValChunk - 1) / kValChunk);
  const float* p = opart + (int64_t)bh * nchunk_ws * kDim + threadIdx.x;
  float s = 0.f;
  for (int ch = 0; ch < nch; ++ch) s += p[(int64_t)ch * kDim];
  out[(int64_t)bh * kDim + threadIdx.x] = s;
}

// ---------------------------------------------------------------------------
template <int GQA, int DT>
static void launch_score_gather(const DecodeArgs& a, const WsLayout& L, const uint8_t* tk,
                                const uint8_t* tv, hipStream_t st, int phase) {
  uint8_t* ws = a.ws;
  if (phase == 0) {
    hipLaunchKernelGGL((k_score<GQA, DT>), dim3(L.ntile, a.G, a.B), dim3(128), 0, st,
                       (const uint8_t*)a.store, a.q, tk, a.H, a.G, a.W, a.capmax, L.ntile,
                       (double*)(ws + L.logits), (double*)(ws + L.tilepart));
  } else {
    hipLaunchKernelGGL((k_gather<GQA, DT>), dim3(L.nchunk, a.G, a.B), dim3(256), 0, st,
                       (const uint8_t*)a.store, tv, a.H, a.G, a.W, a.capmax, L.ntile, L.nchunk,
                       (const double*)(ws + L.logits), (const double*)(ws + L.ftile),
                       (float*)(ws + L.opart));
  }
}

template <int DT>
static bool dispatch_gqa(const DecodeArgs& a, const WsLayout& L, const uint8_t* tk,
                         const uint8_t* tv, hipStream_t st, int phase) {
  switch (a.H / a.G) {
    case 1: launch_score_gather<1, DT>(a, L, tk, tv, st, phase); return true;
    case 2: launch_score_gather<2, DT>(a, L, tk, tv, st, phase); return true;
    case 3: launch_score_gather<3, DT>(a, L, tk, tv, st, phase); return true;
    case 4: launch_score_gather<4, DT>(a, L, tk, tv, st, phase); return true;
    case 5: launch_score_gather<5, DT>(a, L, tk, tv, st, phase); return true;
    case 6: launch_score_gather<6, DT>(a, L, tk, tv, st, phase); return true;
    case 7: launch_score_gather<7, DT>(a, L, tk, tv, st, phase); return true;
    case 8: launch_score_gather<8, DT>(a, L, tk, tv, st, phase); return true;
    default: return false;
  }
}

static inline void mark(const DecodeArgs& a, int i, hipStream_t st) {
  if (a.events) hipEventRecord((hipEvent_t)a.events[i], st);
}

int launch_decode(const DecodeArgs& a, hipStream_t st) {
  const WsLayout L = ws_layout(a.B, a.H, a.G, kDim, a.capmax);
  mark(a, 0, st);
  uint8_t* ws = a.ws;
  uint8_t* tk = a.key_depths_out ? a.key_depths_out : ws + L.tk;
  uint8_t* tv = a.value_depths_out ? a.value_depths_out : ws + L.tv;
  const int esize = a.dtype == 0 ? 2 : 4;
  if (a.dtype == 0)
    hipLaunchKernelGGL((k_key_alloc<0>), dim3(a.B * a.G), dim3(256), 0, st,
                       (const uint8_t*)a.store, a.q, a.H, a.G, a.W, a.RK, tk);
  else
    hipLaunchKernelGGL((k_key_alloc<1>), dim3(a.B * a.G), dim3(256), 0, st,
                       (const uint8_t*)a.store, a.q, a.H, a.G, a.W, a.RK, tk);
  mark(a, 1, st);
  bool ok = a.dtype == 0 ? dispatch_gqa<0>(a, L, tk, tv, st, 0) : dispatch_gqa<1>(a, L, tk, tv, st, 0);
  if (!ok) return -5;
  mark(a, 2, st);
  const bool reg = a.capmax <= (int64_t)kVNT * 16;
  if (reg)
    hipLaunchKernelGGL((k_value_alloc<true>), dim3(a.B * a.G), dim3(kVNT), 0, st,
                       (const uint8_t*)a.store, a.H, a.G, a.W, esize, a.RV, a.vscale, a.capmax,
                       L.ntile, (const double*)(ws + L.logits), (const double*)(ws + L.tilepart),
                       (double*)(ws + L.ftile), (double*)(ws + L.aval), tv);
  else
    hipLaunchKernelGGL((k_value_alloc<false>), dim3(a.B * a.G), dim3(kVNT), 0, st,
                       (const uint8_t*)a.store, a.H, a.G, a.W, esize, a.RV, a.vscale, a.capmax,
                       L.ntile, (const double*)(ws + L.logits), (const double*)(ws + L.tilepart),
                       (double*)(ws + L.ftile), (double*)(ws + L.aval), tv);
  mark(a, 3, st);
  ok = a.dtype == 0 ? dispatch_gqa<0>(a, L, tk, tv, st, 1) : dispatch_gqa<1>(a, L, tk, tv, st, 1);
  if (!ok) return -5;
  mark(a, 4, st);
  hipLaunchKernelGGL(k_out_reduce, dim3(a.B * a.H), dim3(128), 0, st, (const uint8_t*)a.store, a.H,
                     L.nchunk, (const float*)(ws + L.opart), a.out);
  mark(a, 5, st);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace readkv
