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
  __syncthreads();
  if (tid == 0) {
    uint32_t acc = 0;
    for (int i = 0; i < NT / 64; ++i) {
      const uint32_t t = wsum[i];
      wsum[i] = acc;
      acc += t;
    }
    wsum[NT / 64] = acc;
  }
  __syncthreads();
  const uint32_t r = wsum[w] + incl - v;
  __syncthreads();
  return r;
}

template <int NT>
__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, uint32_t* wsum) {
  const uint32_t e = block_excl_scan<NT>(v, wsum);
  (void)e;
  return wsum[NT / 64];  // total is left in wsum[NT/64] until the next scan
}

}  // namespace readkv
