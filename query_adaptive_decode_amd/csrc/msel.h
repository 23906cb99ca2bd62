// ChooseDepths over a large selection domain by many blocks ("Read What
// Matters: Query-Adaptive Quantization for KV Caches", Sec. 3.3; exactness
// App. E.2.1, Prop. 8): a request's pooled tokens under per-layer budgets,
// or a unit whose weights do not fit in LDS.  The threshold search is the one
// of block_choose_depths_hist (select.h) -- exponent-field histograms, then
// 11/11/10/10/10-bit radix digits of the mantissas in the threshold field,
// ties ranked by item index -- with each histogram summed in memory by all
// blocks that hold the domain's items and each decision taken by one block
// per domain; the mantissas are ranked in four 13-bit digits (fewer passes
// than the single block's 11/11/10/10/10, each a launch here).  A chain of
// launches on one stream, so it can be captured:
//   k_value_weights  (also zeroes the domain's histograms and state)
//   k_sel_hist       field histograms
//   k_sel_field      positive-gain count, top field, the field of the B-th
//                    largest gain
//   k_sel_radix<p>, k_sel_digit<p>, p = 0..3   one digit per pass (the
//                    last digit's launch also finds the index cut of the
//                    exact ties, when they are ranked)
//   k_sel_depths     every item's depth, and the read counters
// Item i of a domain is token i of the flat (KV head, token) order, or the
// pair of tokens 2i, 2i + 1 under value packets; item-parallel launches take
// 4096 (histograms) or 1024 (depths) tokens of one unit per block, 4 per
// thread at a time (a pair never straddles threads or units: T_packed is a
// multiple of 32).
#pragma once
#include <math.h>

#include "kernels_common.h"
#include "layout.h"
#include "select.h"

namespace readkv {

// tokens of one unit per block in the histogram passes (fewer blocks, so
// fewer flushes of each block's histogram into the domain's)
constexpr int kSelBlockTokens = 4096;

struct SelState {
  uint32_t npos;     // positive gains of the domain
  int etop;          // largest gain field + 2 (-1: none)
  uint32_t any_odd;  // some positive weight is not regular
  uint32_t flags;    // kSel*
  int Es;            // the threshold's field
  uint32_t rem, n_eq;
  uint32_t pad;
  uint64_t prefix, mask;  // the threshold's mantissa digits settled so far
  int64_t tie_cut;        // ranked ties: taken iff item index < tie_cut
};
constexpr uint32_t kSelDone = 1u;  // no further radix pass
constexpr uint32_t kSelRank = 2u;  // every bit settled, fewer to take than equal gains

struct SelDomain {
  uint32_t* hA;   // regular items by field
  uint32_t* hB;   // odd gains by field
  uint32_t* hC0;  // radix digits, even passes (8192 bins)
  uint32_t* hC1;  // radix digits, odd passes
  SelState* st;
};
constexpr int kSelDigitBits = 13;
constexpr int kSelDigitBins = 1 << kSelDigitBits;
constexpr int kSelPasses = 4;  // 4 x 13 = the 52 mantissa bits
__device__ __forceinline__ SelDomain sel_domain(uint8_t* sel, int64_t dom) {
  uint32_t* h = reinterpret_cast<uint32_t*>(sel + dom * kSelDomainBytes);
  return SelDomain{h, h + 2048, h + 4096, h + 4096 + kSelDigitBins,
                   reinterpret_cast<SelState*>(h + 4096 + 2 * kSelDigitBins)};
}

// One block (NT threads): the digit (of kSelDigitBins bins, in memory) where
// the count from the top reaches rem (>= 1, at most the bins' total); out[0]
// = digit, out[1] = count above it.  Thread t holds the t-th group of
// bins from the top; a block scan in thread order ranks the groups.
template <int NT>
__device__ __forceinline__ void block_find_digit(const uint32_t* hist, uint32_t rem, uint32_t* wsum,
                                                 uint32_t* out) {
  constexpr int PER = kSelDigitBins / NT;
  static_assert(PER % 4 == 0, "whole 16-byte reads per thread");
  const int tid = threadIdx.x;
  const int base = kSelDigitBins - (tid + 1) * PER;  // bins base .. base + PER - 1
  uint32_t h[PER];
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < PER / 4; ++i) {
    const uint4 v = *reinterpret_cast<const uint4*>(hist + base + 4 * i);
    h[4 * i] = v.x;
    h[4 * i + 1] = v.y;
    h[4 * i + 2] = v.z;
    h[4 * i + 3] = v.w;
    tot += (v.x + v.y) + (v.z + v.w);
  }
  const uint32_t excl = block_excl_scan<NT>(tot, wsum);
  if (excl < rem && excl + tot >= rem) {
    uint32_t c = excl;
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      if (c + h[i] >= rem) {
        out[0] = (uint32_t)(base + i);
        out[1] = c;
        break;
      }
      c += h[i];
    }
  }
  __syncthreads();
}

// A domain's budget and item form (as value_select_block): B_V =
// floor(R_V * NU * T_packed) (halved for packets); the minimum depth one
// selects over levels 2..W (weights / 4 under the uniform code, the table
// from Delta_2 on under the Lloyd code) with budget B_V - N.
struct SelParams {
  int64_t N;    // items
  uint32_t bud;
  int Wc;       // levels selected
  double sc;    // weight scale
};
__device__ __forceinline__ SelParams sel_params(int64_t Tp, int NU, float RV, int W, int min1, int pairs,
                                                bool LL) {
  SelParams p;
  const int64_t nt = (int64_t)NU * Tp;
  p.N = pairs ? nt / 2 : nt;
  uint32_t Bv = (uint32_t)floor((double)RV * (double)nt);
  if (pairs) Bv /= 2u;
  if (min1) Bv = (int64_t)Bv > p.N ? Bv - (uint32_t)p.N : 0u;
  p.bud = Bv;
  p.Wc = W - min1;
  p.sc = (min1 && !LL) ? 0.25 : 1.0;
  return p;
}

// The items of tokens j0 .. j0 + 3 of unit ux (j0 a multiple of 4): their
// weights (in the selection's form) and flat indices in the domain; n = 0
// (past the packed tokens), 2 (packets) or 4.
struct SelItems {
  double a[4];
  int64_t idx[4];
  int n;
  int64_t j0;  // first token (unit-local)
};
__device__ __forceinline__ SelItems sel_items(const double* aval, int64_t capmax, int ux, int NU, int64_t j0,
                                              int64_t Tp, int pairs, double sc) {
  SelItems it;
  it.j0 = j0;
  it.n = 0;
  if (it.j0 >= Tp) return it;
  const double2* ap = reinterpret_cast<const double2*>(aval + (int64_t)ux * capmax + it.j0);
  const double2 v0 = ap[0], v1 = ap[1];
  const int64_t flat = (int64_t)(ux % NU) * Tp + it.j0;  // token index in the domain
  if (pairs) {
    it.a[0] = __dadd_rn(v0.x, v0.y) * sc;
    it.a[1] = __dadd_rn(v1.x, v1.y) * sc;
    it.idx[0] = flat / 2;
    it.idx[1] = flat / 2 + 1;
    it.n = 2;
  } else {
    it.a[0] = v0.x * sc;
    it.a[1] = v0.y * sc;
    it.a[2] = v1.x * sc;
    it.a[3] = v1.y * sc;
#pragma unroll
    for (int q = 0; q < 4; ++q) it.idx[q] = flat + q;
    it.n = 4;
  }
  return it;
}

// One item's weight into field histograms (the counts of choose_add).
template <class GP>
__device__ __forceinline__ void sel_add_fields(double a, int W, uint32_t* hA, uint32_t* hB, ChooseLocal& L,
                                               const GP& gp) {
  const int ef = gp.regular(a, 2 * W);
  if (ef != kNoField) {
    atomicAdd(&hA[ef], 1u);
    L.npos += (uint32_t)W;
    L.etop = max(L.etop, ef);
  } else if (a > 0.0) {
    L.odd = true;
    for (int t = 1; t <= W; ++t) {
      const uint64_t kk = gp.gain(a, t);
      if (kk) {
        const int f = (int)(kk >> 52);
        atomicAdd(&hB[f], 1u);
        ++L.npos;
        L.etop = max(L.etop, f + 2);
      }
    }
  }
}

// fn(mantissa) for every gain of the item at field Es (as block_choose_depths_hist)
template <class GP, class Fn>
__device__ __forceinline__ void sel_gains_at(double a, int W, int Es, bool any_odd, const GP& gp, Fn&& fn) {
  const int ef = gp.regular(a, 2 * W);
  if (ef != kNoField) {
    const uint32_t d2 = (uint32_t)(ef - Es - 2);
    if (d2 <= (uint32_t)(2 * W - 2) && !(d2 & 1u)) fn(dbits(a) & kMant);
  } else if (any_odd && a > 0.0) {
    for (int t = 1; t <= W; ++t) {
      const uint64_t kk = gp.gain(a, t);
      if (kk && (int)(kk >> 52) == Es) fn(kk & kMant);
    }
  }
}

// Levels of the item above the threshold | (levels equal to it) << 16 (the
// count_levels of block_choose_depths_hist)
template <class GP>
__device__ __forceinline__ uint32_t sel_levels(double a, int W, const SelState& S, uint32_t bud, const GP& gp) {
  if (!(a > 0.0) || bud == 0) return 0u;
  if (S.npos <= bud) {  // every positive gain is taken
    const int ef = gp.regular(a, 2 * W);
    if (ef != kNoField) return (uint32_t)W;
    uint32_t n = 0;
    for (int t = 1; t <= W; ++t) n += gp.gain(a, t) != 0ull;
    return n;
  }
  uint32_t above = 0, tie = 0;
  const int ef = gp.regular(a, 2 * W);
  if (ef != kNoField) {
    const int d = ef - S.Es;
    above = (uint32_t)min(max((d - 1) >> 1, 0), W);
    if (d >= 2 && d <= 2 * W && !(d & 1)) {
      const uint64_t mnt = (dbits(a) & kMant) & S.mask;
      if (mnt > S.prefix) ++above;
      else if (mnt == S.prefix) ++tie;
    }
  } else {
    for (int t = 1; t <= W; ++t) {
      const uint64_t kk = gp.gain(a, t);
      if (!kk) continue;
      const int e = (int)(kk >> 52);
      if (e > S.Es) {
        ++above;
      } else if (e == S.Es) {
        const uint64_t mnt = (kk & kMant) & S.mask;
        if (mnt > S.prefix) ++above;
        else if (mnt == S.prefix) ++tie;
      }
    }
  }
  return above | (tie << 16);
}

}  // namespace readkv
