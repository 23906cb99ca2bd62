// Block code of two value-allocation stages ("Read What Matters:
// Query-Adaptive Quantization for KV Caches", Sec. 3.2 Eq. (3), Sec. 3.3):
// the softmax statistics with the value weights, and ChooseDepths over the
// packed tokens.  Shared by their own launches (alloc.hip) and the
// single-launch reader (decode.hip).
#pragma once
#include <math.h>

#include "kernels_common.h"
#include "select.h"

namespace readkv {

// ---------------------------------------------------------------------------
// Value weights.  Block (unit, y) takes tokens [1024 y, 1024 y + 1024) of the
// unit (four score tiles); thread t takes tokens 4t .. 4t + 3 of the chunk.
//   m_h = max_tile m_tile, Z_h = sum_tile z_tile exp(m_tile - m_h)
//   f_{h,tile} = exp(m_tile - m_h) / Z_h         (alpha_hat = e * f)
//   a_j = (sum_h alpha_hat_hj^2) * s_gamma(j)     (Eq. (3); s = 1 for UNIT)
// Every block of a unit computes (m_h, Z_h) from the same partials in the
// same order, so all get identical factors; each writes the factors of its
// own tiles (the value gather reads them).  A unit with a non-finite query
// has NaN partials, so its factors and weights are NaN: no value gains.
// ---------------------------------------------------------------------------
constexpr int kVChunk = 1024;

template <int GQA>
struct ValueWeightsShared {
  double fs[GQA][kVChunk / kTile];
  double mh[GQA], zh[GQA];
};

template <int GQA, bool LL>
__device__ __forceinline__ void value_weights_block(ValueWeightsShared<GQA>& sh,
    const VBlock& vb, const uint8_t* store, int ub0, int H, int G, int W, int esize, int vscale,
    int64_t capmax, int ntile_ws, const uint32_t* ebuf, const double* tilepart, double* ftile,
    double* aval, const uint8_t* cb) {
  constexpr int TPC = kVChunk / kTile;  // score tiles per chunk
  static_assert(kVChunk == 4 * 256, "four tokens per thread");
  auto& fs = sh.fs;
  const int ux = ub0 + vb.x;
  const int b = ux / G, g = ux % G;
  const ReqRecord r = req_of(store, b);
  const int64_t len = r.len;
  const int64_t Tp = len & ~(int64_t)(kGroup - 1);
  const int ntile_b = (int)((len + kTile - 1) / kTile);
  const int t0 = vb.y * TPC;
  if (t0 >= ntile_b) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t hrow0 = (int64_t)b * H + (int64_t)g * GQA;
  // the thread's exponentials and group scale do not depend on the softmax
  // statistics: they are in flight while those are formed (a thread past
  // the packed tokens loads token 0's and drops them)
  const int64_t j0 = (int64_t)t0 * kTile + 4 * tid;
  const bool act = j0 < Tp;  // Tp is a multiple of 32: all four tokens or none
  const int64_t jc = act ? j0 : 0;
  uint4 ev[GQA];
  double2 ld[GQA][2];  // Lloyd code: the logits of the four tokens
#pragma unroll
  for (int hh = 0; hh < GQA; ++hh) {
    if constexpr (LL) {
      const double2* lp = reinterpret_cast<const double2*>(
          reinterpret_cast<const double*>(ebuf) + (hrow0 + hh) * capmax + jc);
      ld[hh][0] = lp[0];
      ld[hh][1] = lp[1];
    } else {
      ev[hh] = *reinterpret_cast<const uint4*>(ebuf + (hrow0 + hh) * capmax + jc);
    }
  }
  const Unit u = unit_of(const_cast<uint8_t*>(store), r, g, G, kDim, W, esize);
  const double sg = vscale != 0 ? 1.0
                    : LL ? reinterpret_cast<const double*>(cb + codec_layout(G, kDim).sphys)[g]
                         : u.ev[jc / kGroup];
  auto& mh = sh.mh;
  auto& zh = sh.zh;
  for (int hh = wv; hh < GQA; hh += 4) {
    const double* tp = tilepart + (hrow0 + hh) * ntile_ws * 2;
    double m = -INFINITY;
    for (int t = lane; t < ntile_b; t += 64) m = fmax(m, tp[2 * t]);
    m = wave_max(m);
    double Z = 0.0;
    for (int t = lane; t < ntile_b; t += 64) Z += tp[2 * t + 1] * exp(tp[2 * t] - m);
    Z = wave_sum(Z);
    if (lane == 0) {
      mh[hh] = m;
      zh[hh] = 1.0 / Z;
    }
    if (lane < TPC && t0 + lane < ntile_b) {
      const double f = exp(tp[2 * (t0 + lane)] - m) / Z;
      fs[hh][lane] = f;
      ftile[(hrow0 + hh) * ntile_ws + t0 + lane] = f;
    }
  }
  __syncthreads();
  if (!act) return;
  const int tl = (4 * tid) / kTile;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int hh = 0; hh < GQA; ++hh) {
    if constexpr (LL) {
      // alpha = exp(s - m) (1/Z) from the logit: equal logits, equal weights
      const double lg[4] = {ld[hh][0].x, ld[hh][0].y, ld[hh][1].x, ld[hh][1].y};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const double x = __dmul_rn(exp_nonpos(lg[k] - mh[hh]), zh[hh]);
        s[k] = __dadd_rn(s[k], __dmul_rn(x, x));
      }
    } else {
      const double f = fs[hh][tl];
      const uint32_t e4[4] = {ev[hh].x, ev[hh].y, ev[hh].z, ev[hh].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const double x = __dmul_rn(dec_e(e4[k]), f);
        s[k] = __dadd_rn(s[k], __dmul_rn(x, x));
      }
    }
  }
  if (vscale == 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) s[k] = __dmul_rn(s[k], sg);
  }
  double2* const ap = reinterpret_cast<double2*>(aval + ((int64_t)b * G + g) * capmax + j0);
  ap[0] = make_double2(s[0], s[1]);
  ap[1] = make_double2(s[2], s[3]);
}

// ---------------------------------------------------------------------------
// Value selection: ChooseDepths over the domain's packed tokens with
// B_V = floor(R_V * N), N = NU * T_packed; item i = (KV head g0 + i / T_p,
// token i % T_p).  Then the call's logical reads of the domain ([ReadKV]
// App. A.1): key payload T_p * sum_c t^K_c, value payload d * sum_j t^V_j,
// metadata (lo and rng of every closed group and channel of keys and values,
// E^K, E^V), the open group's keys and values.
// ---------------------------------------------------------------------------
constexpr int kVSelNT = 1024;

// Lloyd code: one load per call of the layer's calibration arrays (mu and
// sigma of keys and values, 32 bits per KV head and channel), charged to the
// first request's domains, and of the decoder table (510 centroids and 8
// gains, 32 bits each), charged to the first domain ([ReadKV] App. A.1).
__device__ __forceinline__ unsigned long long lloyd_meta_bits(bool first_request, bool first_domain,
                                                              unsigned long long nu) {
  return (first_request ? nu * 4ull * kDim * 32ull : 0ull) + (first_domain ? 518ull * 32ull : 0ull);
}
// domains of up to this many tokens are copied to LDS once (8 bytes each)
constexpr int kVSelLocal = 16384;

template <int NT>
struct ValueSelectShared {
  ChooseShared<NT> S;
  double gt[16];
};

// NT threads; acache: LDS of the domain's weights when LOCAL
template <int NT, bool LOCAL, bool LL>
__device__ __forceinline__ void value_select_block(ValueSelectShared<NT>& sh, double* acache,
    const VBlock& vb, const uint8_t* store, int ub0, int G, int W, int esize, float RV, int NU,
    int min1, int pairs, int64_t capmax, const double* aval, uint8_t* tv, const uint8_t* tk,
    uint64_t* counters, const uint8_t* cb) {
  auto& S = sh.S;
  auto& gt = sh.gt;
  if (LL && threadIdx.x < 16)
    gt[threadIdx.x] = reinterpret_cast<const double*>(cb + codec_layout(G, kDim).gains)[threadIdx.x];
  const int tid = threadIdx.x, lane = tid & 63;
  const int u0 = ub0 + vb.x * NU;
  const int b = u0 / G;
  const ReqRecord r = req_of(store, b);
  const int64_t len = r.len;
  const int64_t Tp = len & ~(int64_t)(kGroup - 1);
  const int64_t NT_ = (int64_t)NU * Tp;  // tokens of the domain
  const double* const ab = aval + (int64_t)u0 * capmax;
  uint8_t* const tvb = tv + (int64_t)u0 * capmax;
  auto at = [&](int64_t i) -> int64_t {  // token -> offset in the unit-major arrays
    if (NU == 1) return i;
    const int64_t k = i / Tp;
    return k * capmax + (i - k * Tp);
  };
  // items: tokens, or pairs of tokens (2m, 2m + 1) with summed weights; the
  // minimum depth one: weights / 4 over levels 1..W-1, budget less N
  const int64_t N = pairs ? NT_ / 2 : NT_;
  uint32_t Bv = (uint32_t)floor((double)RV * (double)NT_);
  if (pairs) Bv /= 2u;
  if (min1) Bv = (int64_t)Bv > N ? Bv - (uint32_t)N : 0u;
  const double sc = (min1 && !LL) ? 0.25 : 1.0;
  uint32_t mine = 0;  // this thread's token depths
  auto put = [&](int64_t i, uint32_t t) {
    t += (uint32_t)min1;
    if (pairs) {
      tvb[at(2 * i)] = (uint8_t)t;
      tvb[at(2 * i + 1)] = (uint8_t)t;
      mine += 2 * t;
    } else {
      tvb[at(i)] = (uint8_t)t;
      mine += t;
    }
  };
  auto select = [&](auto&& geta) {
    if constexpr (LL) {
      __syncthreads();  // gt
      block_choose_depths<NT>(N, Bv, W - min1, geta, put, S, TableGains{gt + min1});
    } else {
      block_choose_depths<NT>(N, Bv, W - min1, geta, put, S);
    }
  };
  if constexpr (LOCAL) {
    // eight loads in flight per thread, then their LDS stores
    for (int64_t i0 = 0; i0 < NT_; i0 += 8 * NT) {
      double v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t i = i0 + k * NT + tid;
        v[k] = i < NT_ ? ab[at(i)] : 0.0;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t i = i0 + k * NT + tid;
        if (i < NT_) acache[i] = v[k];
      }
    }
    __syncthreads();
    select([&](int64_t i) {
      return (pairs ? __dadd_rn(acache[2 * i], acache[2 * i + 1]) : acache[i]) * sc;
    });
  } else {
    select([&](int64_t i) {
      return (pairs ? __dadd_rn(ab[at(2 * i)], ab[at(2 * i + 1)]) : ab[at(i)]) * sc;
    });
  }
  if (counters) {
    const uint32_t vtot = block_sum_u32<NT>(mine, S.wsum);
    if (tid < 64) {
      int ks = 0;
      for (int i = lane; i < NU * kDim; i += 64) ks += tk[(int64_t)u0 * kDim + i];
      ks = wave_sum_i32(ks);
      if (lane == 0) {
        const unsigned long long ng = (unsigned long long)(Tp / kGroup), nu = (unsigned long long)NU;
        atomicAdd(reinterpret_cast<unsigned long long*>(counters), (unsigned long long)ks * (unsigned long long)Tp);
        atomicAdd(reinterpret_cast<unsigned long long*>(counters + 1), (unsigned long long)vtot * kDim);
        const unsigned long long meta =
            LL ? lloyd_meta_bits(b == 0, u0 == 0, nu)
               : nu * (2ull * ng * kDim * 32ull + kDim * 64ull + ng * 64ull);
        atomicAdd(reinterpret_cast<unsigned long long*>(counters + 2), meta);
        atomicAdd(reinterpret_cast<unsigned long long*>(counters + 3),
                  nu * 2ull * (unsigned long long)(len - Tp) * kDim * (unsigned long long)esize * 8ull);
      }
    }
  }
}

template <int NT, int GQA>
struct ValueAllocUnitShared {
  ChooseShared<NT> S;
  double gt[16];
  double fs[GQA][kVSelLocal / kTile];
  double mh[GQA], zh[GQA];
};

// NT threads; acache: the unit's weights [T_p], in LDS, or (GCACHE) in
// device memory that only this block touches
template <int NT, int GQA, bool LL, bool GCACHE>
__device__ __forceinline__ void value_alloc_unit_block(ValueAllocUnitShared<NT, GQA>& sh,
    double* acache, const VBlock& vb, const uint8_t* store, int ub0, int H, int G, int W, int esize,
    int vscale, float RV, int min1, int pairs, int64_t capmax, int ntile_ws, const uint32_t* ebuf,
    const double* tilepart, double* ftile, uint8_t* tv, const uint8_t* tk, uint64_t* counters,
    const uint8_t* cb) {
  constexpr int RT = 4 * NT;  // tokens per round
  auto& S = sh.S;
  auto& gt = sh.gt;
  auto& fs = sh.fs;
  const int ux = ub0 + vb.x;
  const int b = ux / G, g = ux % G;
  const ReqRecord r = req_of(store, b);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t hrow0 = (int64_t)b * H + (int64_t)g * GQA;
  const int64_t len = r.len;
  const int64_t Tp = len & ~(int64_t)(kGroup - 1);
  const int ntile_b = (int)((len + kTile - 1) / kTile);
  const Unit u = unit_of(const_cast<uint8_t*>(store), r, g, G, kDim, W, esize);
  // Lloyd code: one scale per KV head, the tree's gains
  const double sg_ll = LL && vscale == 0
                           ? reinterpret_cast<const double*>(cb + codec_layout(G, kDim).sphys)[g]
                           : 1.0;
  if (LL && tid < 16) gt[tid] = reinterpret_cast<const double*>(cb + codec_layout(G, kDim).gains)[tid];
  // the four tokens' exponentials (uniform code) or logits (Lloyd code)
  auto load_round = [&](int k, uint4 (&ev)[GQA], double2 (&ld)[GQA][2], double& sg)
                        __attribute__((always_inline)) {
    const int64_t j0 = (int64_t)k * RT + 4 * tid;
    const int64_t jc = j0 < Tp ? j0 : 0;  // (a thread past the tokens loads token 0's)
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) {
      if constexpr (LL) {
        const double2* lp = reinterpret_cast<const double2*>(
            reinterpret_cast<const double*>(ebuf) + (hrow0 + hh) * capmax + jc);
        ld[hh][0] = lp[0];
        ld[hh][1] = lp[1];
      } else {
        ev[hh] = *reinterpret_cast<const uint4*>(ebuf + (hrow0 + hh) * capmax + jc);
      }
    }
    sg = LL ? sg_ll : vscale == 0 ? u.ev[jc / kGroup] : 1.0;
  };
  uint4 ev[GQA];
  double2 ld[GQA][2];
  double sg;
  auto& mh = sh.mh;
  auto& zh = sh.zh;
  load_round(0, ev, ld, sg);
  choose_clear<NT>(S);  // while the first round's exponentials are in flight
  for (int hh = wv; hh < GQA; hh += NT / 64) {
    const double* tp = tilepart + (hrow0 + hh) * ntile_ws * 2;
    // one tile per lane (at most 64 tiles in a unit that fits LDS)
    const double mt = lane < ntile_b ? tp[2 * lane] : -INFINITY;
    const double zt = lane < ntile_b ? tp[2 * lane + 1] : 0.0;
    const double m = wave_max(mt);
    const double x = lane < ntile_b ? exp(mt - m) : 0.0;
    const double Z = wave_sum(zt * x);
    if (lane == 0) {
      mh[hh] = m;
      zh[hh] = 1.0 / Z;
    }
    if (lane < ntile_b) {
      const double f = x / Z;
      fs[hh][lane] = f;
      ftile[(hrow0 + hh) * ntile_ws + lane] = f;
    }
  }
  lds_barrier();
  // items: tokens, or pairs of tokens (2m, 2m + 1) with summed weights; the
  // minimum depth one: weights / 4 over levels 1..W-1, budget less N.  The
  // selection's histograms are built here from the weights in registers, in
  // exactly the form the selection reads them back from LDS.
  const int64_t N = pairs ? Tp / 2 : Tp;
  const double sc = (min1 && !LL) ? 0.25 : 1.0;
  const int Wc = W - min1;
  ChooseLocal CL;
  const TableGains tg{gt + min1};
  auto add = [&](double a) __attribute__((always_inline)) {
    if constexpr (LL) choose_add<NT>(a, Wc, S, CL, tg);
    else choose_add<NT>(a, Wc, S, CL);
  };
  const int nr = (int)((Tp + RT - 1) / RT);
  for (int k = 0; k < nr; ++k) {
    if (k > 0) load_round(k, ev, ld, sg);
    const int64_t j0 = (int64_t)k * RT + 4 * tid;
    if (j0 < Tp) {  // Tp is a multiple of 32: all four tokens or none
      const int tl = (int)(j0 / kTile);
      double sa[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) {
        if constexpr (LL) {
          // alpha = exp(s - m) (1/Z) from the logit: equal logits, equal weights
          const double lg[4] = {ld[hh][0].x, ld[hh][0].y, ld[hh][1].x, ld[hh][1].y};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const double xq = __dmul_rn(exp_nonpos(lg[q] - mh[hh]), zh[hh]);
            sa[q] = __dadd_rn(sa[q], __dmul_rn(xq, xq));
          }
        } else {
          const double f = fs[hh][tl];
          const uint32_t e4[4] = {ev[hh].x, ev[hh].y, ev[hh].z, ev[hh].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const double xq = __dmul_rn(dec_e(e4[q]), f);
            sa[q] = __dadd_rn(sa[q], __dmul_rn(xq, xq));
          }
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sa[q] = vscale == 0 ? __dmul_rn(sa[q], sg) : sa[q];
        acache[j0 + q] = sa[q];
      }
      if (pairs) {
        add(__dadd_rn(sa[0], sa[1]) * sc);
        add(__dadd_rn(sa[2], sa[3]) * sc);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) add(sa[q] * sc);
      }
    }
  }
  choose_flush<NT>(CL, S);
  if constexpr (GCACHE) __syncthreads();  // the weights in memory, for every thread
  else lds_barrier();
  uint32_t Bv = (uint32_t)floor((double)RV * (double)Tp);
  if (pairs) Bv /= 2u;
  if (min1) Bv = (int64_t)Bv > N ? Bv - (uint32_t)N : 0u;
  uint8_t* const tvb = tv + ((int64_t)b * G + g) * capmax;
  uint32_t mine = 0;  // this thread's token depths
  auto geta = [&](int64_t i) {
    return (pairs ? __dadd_rn(acache[2 * i], acache[2 * i + 1]) : acache[i]) * sc;
  };
  auto put = [&](int64_t i, uint32_t t) {
    t += (uint32_t)min1;
    if (pairs) {
      tvb[2 * i] = (uint8_t)t;
      tvb[2 * i + 1] = (uint8_t)t;
      mine += 2 * t;
    } else {
      tvb[i] = (uint8_t)t;
      mine += t;
    }
  };
  if constexpr (LL) block_choose_depths_hist<NT>(N, Bv, Wc, geta, put, S, tg);
  else block_choose_depths_hist<NT>(N, Bv, Wc, geta, put, S);
  if (counters) {
    const uint32_t vtot = block_sum_u32<NT>(mine, S.wsum);
    if (tid < 64) {
      const uint8_t* tkb = tk + ((int64_t)b * G + g) * kDim;
      const int ks = wave_sum_i32((int)tkb[lane] + (int)tkb[lane + 64]);
      if (lane == 0) {
        const unsigned long long ng = (unsigned long long)(Tp / kGroup);
        atomicAdd(reinterpret_cast<unsigned long long*>(counters), (unsigned long long)ks * (unsigned long long)Tp);
        atomicAdd(reinterpret_cast<unsigned long long*>(counters + 1), (unsigned long long)vtot * kDim);
        const unsigned long long meta = LL ? lloyd_meta_bits(b == 0, ux == 0, 1ull)
                                           : 2ull * ng * kDim * 32ull + kDim * 64ull + ng * 64ull;
        atomicAdd(reinterpret_cast<unsigned long long*>(counters + 2), meta);
        atomicAdd(reinterpret_cast<unsigned long long*>(counters + 3),
                  2ull * (unsigned long long)(len - Tp) * kDim * (unsigned long long)esize * 8ull);
      }
    }
  }
}

}  // namespace readkv
