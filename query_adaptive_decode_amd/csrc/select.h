// Block-level top-k threshold search over 64-bit keys (the bit patterns of
// non-negative doubles, which order like the doubles themselves).
//
// ChooseDepths ("Read What Matters", Sec. 3.3) takes the B largest positive
// refinement gains, ties to the lowest item index.  Because every item's
// gains strictly decrease with depth, the chosen set is exactly "every gain
// above a threshold tau, plus the lowest-index items whose gain equals tau"
// (App. E.2.1, Prop. 8).  tau is found by an MSB-first radix descent:
// each pass histograms one digit of the keys that still match the chosen
// prefix and keeps the digit where the running count from the top crosses
// the number still to be chosen.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels_common.h"

namespace readkv {

// Outcome of a threshold search: a key is chosen iff it is positive and
// (key & mask) > prefix, or (key & mask) == prefix and it is among the
// `take_eq` lowest-index keys with that masked value (`n_eq` of them exist).
// all_pos: every positive key is chosen.
struct Threshold {
  uint64_t prefix, mask;
  uint32_t take_eq, n_eq;
  int all_pos;
};

// inclusive prefix sum over the wave: DPP row shifts inside each 16-lane
// row, then the row totals broadcast to the following rows
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += dpp_u32<kDppRowShr1>(v);
  v += dpp_u32<kDppRowShr2>(v);
  v += dpp_u32<kDppRowShr4>(v);
  v += dpp_u32<kDppRowShr8>(v);
  v += dpp_u32<kDppRowBcast15, 0xA>(v);
  v += dpp_u32<kDppRowBcast31, 0xC>(v);
  return v;
}

// One wave scans NB bins (LDS) from the highest digit down and finds the
// digit where the cumulative count reaches `rem` (>= 1): writes the digit
// and the count strictly above it.  If the bins hold fewer than `rem` in
// all, nothing is written.  `out_total` (may be null) gets the sum of all
// bins.  Each lane reads PER consecutive bins with 16-byte LDS reads.
template <int NB>
__device__ __forceinline__ void wave_find_digit(const uint32_t* hist, uint32_t rem, uint32_t* out_digit,
                                                uint32_t* out_above, uint32_t* out_total = nullptr) {
  constexpr int PER = NB / 64;
  static_assert(PER % 4 == 0, "whole 16-byte reads per lane");
  const int l = __lane_id();
  const int base = NB - (l + 1) * PER;  // lane l holds bins base .. base + PER - 1
  uint32_t h[PER];                      // h[i] = bin base + PER - 1 - i (descending)
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < PER / 4; ++i) {
    const uint4 v = *reinterpret_cast<const uint4*>(hist + base + 4 * i);
    h[PER - 1 - 4 * i] = v.x;
    h[PER - 2 - 4 * i] = v.y;
    h[PER - 3 - 4 * i] = v.z;
    h[PER - 4 - 4 * i] = v.w;
    tot += (v.x + v.y) + (v.z + v.w);
  }
  const uint32_t incl = wave_incl_scan_u32(tot);
  const uint32_t excl = incl - tot;
  if (out_total && l == 63) *out_total = incl;
  const uint64_t bal = __ballot(incl >= rem);
  const int L = bal ? __ffsll((unsigned long long)bal) - 1 : -1;
  if (l == L) {
    uint32_t c = excl;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (c + h[i] >= rem) {
        *out_digit = (uint32_t)(base + PER - 1 - i);
        *out_above = c;
        break;
      }
      c += h[i];
    }
  }
}

// Exclusive prefix sum over the threads of a block, in thread order.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum /*LDS NT/64+1*/) {
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const uint32_t incl = wave_incl_scan_u32(v);
  if ((tid & 63) == 63) wsum[w] = incl;
  lds_barrier();
  if (tid == 0) {
    uint32_t acc = 0;
    for (int i = 0; i < NT / 64; ++i) {
      const uint32_t t = wsum[i];
      wsum[i] = acc;
      acc += t;
    }
    wsum[NT / 64] = acc;
  }
  lds_barrier();
  const uint32_t r = wsum[w] + incl - v;
  lds_barrier();
  return r;
}

template <int NT>
__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, uint32_t* wsum) {
  const uint32_t e = block_excl_scan<NT>(v, wsum);
  (void)e;
  return wsum[NT / 64];  // total is left in wsum[NT/64] until the next scan
}

// ---------------------------------------------------------------------------
// ChooseDepths over N items by one block ([ReadKV] Sec. 3.3; exactness App.
// E.2.1, Prop. 8).  Item i has a weight a_i >= 0 (NaN or 0: no gains) and W
// candidate gains a_i 4^-t, t = 1..W; the Bud largest positive gains are
// chosen, ties to the lowest item index.
//
// Gain fields.  When a_i is a normal double with exponent field E in
// (2W, 2047) ("regular"), every gain is exact, with field E - 2t and a_i's
// mantissa, so a regular item holds min(W, max(0, floor((E - L) / 2))) gains
// at field L or above.  Other positive weights ("odd": some gains are
// subnormal) have their gains formed one by one.  An LDS histogram of the
// regular items' fields (hA) and of the odd gains' fields (hB), with the
// count of positive gains and the top field, gives the count at every field;
// one wave scans down from the top field for the field L* of the Bud-th
// largest gain; within L* the gains are ranked by mantissa with
// 11/11/10/10/10-bit radix passes that stop once the gains sharing the
// chosen digits are exactly the ones still to be taken; once at most
// kChooseBig gains share the digits their mantissas are copied to a list in
// LDS (over the field histograms, no longer needed), so that later passes
// read the list instead of every item, and once at most kChooseList are left
// one wave settles the remaining bits with ballots.  The remaining equal
// gains are ranked by item index.  A thread takes 4 consecutive items per
// round.  Barriers here order LDS only (global stores are not waited for).
// ---------------------------------------------------------------------------
constexpr int kNoField = -8192;
constexpr uint64_t kMant = 0x000FFFFFFFFFFFFFull;
constexpr int kChooseList = 64;
constexpr int kChooseBig = 2048;  // mantissas, 16 KB: hA and hB

__device__ __forceinline__ int regular_field(double a, int twoW) {
  const int E = (int)(dbits(a) >> 52);
  return (a > 0.0 && E > twoW && E < 2047) ? E : kNoField;
}
__device__ __forceinline__ uint64_t gain_bits(double a, int t) {
  return dbits(__dmul_rn(a, bitsd((uint64_t)(1023 - 2 * t) << 52)));
}

// Gain tables.  Pow4Gains: gain of level t = a 4^-t (uniform code; regular
// items use the shared-mantissa fields above).  TableGains: gain = a g[t]
// with a caller's table of decreasing positive g[1..W] (the Lloyd tree's
// Delta_t): every positive item forms its W gains one by one (the "odd"
// path), each an fp64 product rounded to nearest.
struct Pow4Gains {
  __device__ __forceinline__ int regular(double a, int twoW) const { return regular_field(a, twoW); }
  __device__ __forceinline__ uint64_t gain(double a, int t) const { return gain_bits(a, t); }
};
struct TableGains {
  const double* g;  // g[t], t = 1..W
  __device__ __forceinline__ int regular(double, int) const { return kNoField; }
  __device__ __forceinline__ uint64_t gain(double a, int t) const { return dbits(__dmul_rn(a, g[t])); }
};

template <int NT>
struct ChooseShared {
  union {
    struct {
      uint32_t hA[2048];  // regular items by field
      uint32_t hB[2048];  // odd gains by field
    };
    uint64_t big[kChooseBig];  // candidate mantissas, once the field is found
  };
  uint32_t hC[2048];  // radix digits
  uint32_t wsum[NT / 64 + 1];
  uint32_t sh[4];
  uint32_t npos;      // positive gains
  int etop;           // largest gain field + 2 (-1: no positive gain)
  uint32_t any_odd;   // some positive weight is not regular
  uint32_t nlist;     // candidates collected for the last bits
  uint32_t nbig;      // candidates in big
  uint64_t rprefix, rmask;  // the threshold's mantissa digits, once settled by one wave
  uint64_t list[kChooseList];
};

// All threads: zero the histograms and counts (a barrier must follow).
template <int NT>
__device__ __forceinline__ void choose_clear(ChooseShared<NT>& S) {
  for (int i = threadIdx.x; i < 2048; i += NT) {
    S.hA[i] = 0u;
    S.hB[i] = 0u;
    S.hC[i] = 0u;
  }
  if (threadIdx.x == 0) {
    S.npos = 0u;
    S.etop = -1;
    S.any_odd = 0u;
    S.nlist = 0u;
    S.nbig = 0u;
  }
}

// One item's weight into the histograms; the thread's count of positive
// gains and top field are kept in L until choose_flush.
struct ChooseLocal {
  uint32_t npos = 0u;
  int etop = -1;
  bool odd = false;
};
template <int NT, class GP = Pow4Gains>
__device__ __forceinline__ void choose_add(double a, int W, ChooseShared<NT>& S, ChooseLocal& L,
                                           const GP& gp = GP()) {
  const int ef = gp.regular(a, 2 * W);
  if (ef != kNoField) {
    atomicAdd(&S.hA[ef], 1u);
    L.npos += (uint32_t)W;
    L.etop = max(L.etop, ef);
  } else if (a > 0.0) {
    L.odd = true;
    for (int t = 1; t <= W; ++t) {
      const uint64_t kk = gp.gain(a, t);
      if (kk) {
        const int f = (int)(kk >> 52);
        atomicAdd(&S.hB[f], 1u);
        ++L.npos;
        L.etop = max(L.etop, f + 2);
      }
    }
  }
}
// All threads (every lane active): publish the counts of choose_add.
template <int NT>
__device__ __forceinline__ void choose_flush(const ChooseLocal& L, ChooseShared<NT>& S) {
  const int n = wave_sum_i32((int)L.npos);
  const int e = wave_max_i32(L.etop);
  const bool odd = __ballot(L.odd) != 0ull;
  if ((threadIdx.x & 63) == 0) {
    atomicAdd(&S.npos, (uint32_t)n);
    atomicMax(&S.etop, e);
    if (odd) S.any_odd = 1u;
  }
}

// One wave: the field of the rem-th largest gain (1 <= rem <= number of
// positive gains), scanning down from field `top` 64 fields at a time: lane l
// forms G[f] = hB[f] + sum_{t=1..W} hA[f + 2t] of field f = f0 - l.  out[0]
// = field, out[1] = count above it, out[2] = G[field].
__device__ __forceinline__ void wave_find_gain_field(const uint32_t* hA, const uint32_t* hB, int W,
                                                     int top, uint32_t rem, uint32_t* out) {
  const int l = __lane_id();
  uint32_t above = 0;
  for (int f0 = top; f0 >= 0; f0 -= 64) {
    const int f = f0 - l;
    uint32_t g = 0;
    if (f >= 0) {
      g = hB[f];
      for (int t = 1; t <= W; ++t) {
        const int fa = f + 2 * t;
        if (fa < 2048) g += hA[fa];
      }
    }
    const uint32_t incl = wave_incl_scan_u32(g);  // lanes in descending field order
    const uint64_t bal = __ballot(above + incl >= rem);
    if (bal) {
      const int L = __ffsll((unsigned long long)bal) - 1;
      if (l == L) {
        out[0] = (uint32_t)f;
        out[1] = above + incl - g;
        out[2] = g;
      }
      return;
    }
    above += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  }
}

// One wave: n <= 64 candidate mantissas (list) that agree with prefix under
// mask, of which the rem largest are to be taken (1 <= rem <= n).  Settles
// the bits below the mask MSB first with ballots, until the candidates that
// share the settled bits are exactly the ones still to be taken, or every
// bit is settled (then the equal ones are ties).  Writes the new prefix and
// mask, and out[0] = number still to take among the equal ones, out[1] = how
// many are equal.
__device__ __forceinline__ void wave_settle_bits(const uint64_t* list, uint32_t n, uint32_t rem,
                                                 uint64_t prefix, uint64_t mask, uint64_t* pm,
                                                 uint32_t* out) {
  const int l = __lane_id();
  const uint64_t m = l < (int)n ? list[l] : 0ull;
  uint64_t live = __ballot(l < (int)n);
  uint32_t r = rem;
  const int low = mask ? __builtin_ctzll(mask) : 52;  // lowest settled bit
  for (int b = low - 1; b >= 0; --b) {
    if ((uint32_t)__popcll(live) == r) break;
    const uint64_t ones = live & __ballot((m >> b) & 1ull);
    const uint32_t c1 = (uint32_t)__popcll(ones);
    if (c1 >= r) {
      live = ones;
      prefix |= 1ull << b;
    } else {
      r -= c1;
      live &= ~ones;
    }
    mask |= 1ull << b;
  }
  if (l == 0) {
    pm[0] = prefix;
    pm[1] = mask;
    out[0] = r;
    out[1] = (uint32_t)__popcll(live);
  }
}

// Items are visited in rounds of 4 NT: thread t takes items 4t .. 4t + 3 of
// a round (so the tie ranking in index order is a block scan per round).
// geta(i) returns a_i (i < N); put(i, t) stores item i's depth.  Returns the
// sum of this thread's depths.  Every thread of the block must call it
// (block barriers inside).  The histograms must have been built (choose_clear,
// choose_add of every item's geta value, choose_flush, a barrier).
template <int NT, class GetA, class PutT, class GP = Pow4Gains>
__device__ uint32_t block_choose_depths_hist(int64_t N, uint32_t Bud, int W, GetA&& geta, PutT&& put,
                                             ChooseShared<NT>& S, const GP& gp = GP()) {
  constexpr int NW = NT / 64;
  constexpr int IPT = 4;
  constexpr int64_t RT = (int64_t)NT * IPT;
  const int tid = threadIdx.x;
  const int twoW = 2 * W;
  const int64_t nr = (N + RT - 1) / RT;
  // fn(i, a, field, in_range) for every item of the thread (all threads,
  // uniform count)
  auto for_items = [&](auto&& fn) __attribute__((always_inline)) {
    for (int64_t k = 0; k < nr; ++k) {
      const int64_t i0 = k * RT + (int64_t)IPT * tid;
      double a[IPT];
#pragma unroll
      for (int q = 0; q < IPT; ++q) a[q] = i0 + q < N ? geta(i0 + q) : 0.0;
#pragma unroll
      for (int q = 0; q < IPT; ++q) fn(i0 + q, a[q], gp.regular(a[q], twoW), i0 + q < N);
    }
  };

  const uint32_t npos = S.npos;
  const bool any_odd = S.any_odd != 0u;
  const bool all_pos = npos <= Bud;
  int Es = -1;
  uint64_t prefix = 0, mask = 0;  // over the 52 mantissa bits
  uint32_t rem = 0, n_eq = 0;
  if (!all_pos && Bud > 0) {
    if (tid < 64) wave_find_gain_field(S.hA, S.hB, W, S.etop - 2, Bud, S.sh);
    lds_barrier();  // (hA and hB are free from here on)
    Es = (int)S.sh[0];
    rem = Bud - S.sh[1];  // >= 1
    n_eq = S.sh[2];       // >= rem
    const uint32_t dspan = (uint32_t)(twoW - 2);
    // fn(mantissa) for every gain at field Es (a regular item's candidate:
    // d = E - Es even in [2, 2W])
    auto for_gains_at_Es = [&](double a, int ef, auto&& fn) __attribute__((always_inline)) {
      if (ef != kNoField) {
        const uint32_t d2 = (uint32_t)(ef - Es - 2);
        if (d2 <= dspan && !(d2 & 1u)) fn(dbits(a) & kMant);
      } else if (any_odd && a > 0.0) {
        for (int t = 1; t <= W; ++t) {
          const uint64_t kk = gp.gain(a, t);
          if (kk && (int)(kk >> 52) == Es) fn(kk & kMant);
        }
      }
    };
    // fn(mantissa) for every gain that shares the digits so far: from the
    // list once it exists, else from the items
    int nbig = -1;
    auto for_candidates = [&](auto&& fn) __attribute__((always_inline)) {
      if (nbig >= 0) {
        for (int i = tid; i < nbig; i += NT) {
          const uint64_t mnt = S.big[i];
          if ((mnt & mask) == prefix) fn(mnt);
        }
      } else {
        for_items([&](int64_t, double a, int ef, bool) __attribute__((always_inline)) {
          for_gains_at_Es(a, ef, [&](uint64_t mnt) __attribute__((always_inline)) {
            if ((mnt & mask) == prefix) fn(mnt);
          });
        });
      }
    };
    // digits of the 52 mantissa bits: 11, 11, 10, 10, 10 (MSB first)
    for (int pass = 0; pass < 5 && n_eq != rem; ++pass) {
      if (n_eq <= (uint32_t)kChooseList) {
        // the last candidates: one wave settles the remaining bits
        for_candidates([&](uint64_t mnt) __attribute__((always_inline)) { S.list[atomicAdd(&S.nlist, 1u)] = mnt; });
        lds_barrier();
        if (tid < 64) wave_settle_bits(S.list, n_eq, rem, prefix, mask, &S.rprefix, S.sh);
        lds_barrier();
        prefix = S.rprefix;
        mask = S.rmask;
        rem = S.sh[0];
        n_eq = S.sh[1];
        break;
      }
      if (nbig < 0 && n_eq <= (uint32_t)kChooseBig) {
        for_candidates([&](uint64_t mnt) __attribute__((always_inline)) { S.big[atomicAdd(&S.nbig, 1u)] = mnt; });
        lds_barrier();
        nbig = (int)n_eq;
      }
      const int width = pass < 2 ? 11 : 10;
      const int shift = pass < 2 ? 41 - 11 * pass : 40 - 10 * pass;
      const uint32_t dmask = (1u << width) - 1u;
      if (pass > 0) {
        for (int i = tid; i < 2048; i += NT) S.hC[i] = 0u;
        lds_barrier();
      }
      for_candidates([&](uint64_t mnt) __attribute__((always_inline)) {
        atomicAdd(&S.hC[(uint32_t)(mnt >> shift) & dmask], 1u);
      });
      lds_barrier();
      if (tid < 64) {
        if (width == 11) wave_find_digit<2048>(S.hC, rem, &S.sh[0], &S.sh[1]);
        else wave_find_digit<1024>(S.hC, rem, &S.sh[0], &S.sh[1]);
      }
      lds_barrier();
      const uint32_t dg = S.sh[0];
      n_eq = S.hC[dg];
      rem -= S.sh[1];
      prefix |= (uint64_t)dg << shift;
      mask |= (uint64_t)dmask << shift;
      lds_barrier();
    }
  }

  // ---- depths: levels above the threshold, plus ties in index order ----
  // (levels above) | (levels equal to the threshold) << 16
  auto count_levels = [&](double a, int ef) __attribute__((always_inline)) -> uint32_t {
    if (!(a > 0.0) || Bud == 0) return 0u;
    if (all_pos) {
      if (ef != kNoField) return (uint32_t)W;
      uint32_t n = 0;
      for (int t = 1; t <= W; ++t) n += gp.gain(a, t) != 0ull;
      return n;
    }
    uint32_t above = 0, tie = 0;
    if (ef != kNoField) {
      const int d = ef - Es;
      above = (uint32_t)min(max((d - 1) >> 1, 0), W);
      if (d >= 2 && d <= twoW && !(d & 1)) {
        const uint64_t mnt = (dbits(a) & kMant) & mask;
        if (mnt > prefix) ++above;
        else if (mnt == prefix) ++tie;
      }
    } else {
      for (int t = 1; t <= W; ++t) {
        const uint64_t kk = gp.gain(a, t);
        if (!kk) continue;
        const int e = (int)(kk >> 52);
        if (e > Es) {
          ++above;
        } else if (e == Es) {
          const uint64_t mnt = (kk & kMant) & mask;
          if (mnt > prefix) ++above;
          else if (mnt == prefix) ++tie;
        }
      }
    }
    return above | (tie << 16);
  };
  // Ties are ranked only when not all equal gains are taken, which needs
  // all 52 bits settled: then an item has at most one gain equal to the
  // threshold (its gains differ from each other).
  const bool rank_ties = !all_pos && Bud > 0 && rem < n_eq;
  uint32_t running = 0;  // ties in earlier rounds
  uint32_t mine = 0;
  for (int64_t k = 0; k < nr; ++k) {
    const int64_t i0 = k * RT + (int64_t)IPT * tid;
    uint32_t t[IPT], tie[IPT];
#pragma unroll
    for (int q = 0; q < IPT; ++q) {
      const double a = i0 + q < N ? geta(i0 + q) : 0.0;
      const uint32_t lv = count_levels(a, gp.regular(a, twoW));
      t[q] = lv & 0xFFFFu;
      tie[q] = lv >> 16;
    }
    if (rank_ties) {
      uint32_t before = block_excl_scan<NT>((tie[0] + tie[1]) + (tie[2] + tie[3]), S.wsum) + running;
      running += S.wsum[NW];
#pragma unroll
      for (int q = 0; q < IPT; ++q) {
        if (tie[q] && before < rem) ++t[q];
        before += tie[q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < IPT; ++q) t[q] += tie[q];
    }
#pragma unroll
    for (int q = 0; q < IPT; ++q) {
      if (i0 + q < N) {
        put(i0 + q, t[q]);
        mine += t[q];
      }
    }
  }
  return mine;
}

// ChooseDepths with the histograms built here from geta.
template <int NT, class GetA, class PutT, class GP = Pow4Gains>
__device__ uint32_t block_choose_depths(int64_t N, uint32_t Bud, int W, GetA&& geta, PutT&& put,
                                        ChooseShared<NT>& S, const GP& gp = GP()) {
  const int tid = threadIdx.x;
  choose_clear<NT>(S);
  lds_barrier();
  ChooseLocal L;
  for (int64_t i = tid; i < N; i += NT) choose_add<NT>(geta(i), W, S, L, gp);
  choose_flush<NT>(L, S);
  lds_barrier();
  return block_choose_depths_hist<NT>(N, Bud, W, geta, put, S, gp);
}

}  // namespace readkv
