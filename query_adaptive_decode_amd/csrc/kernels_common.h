// Device-side helpers shared by the encoder and decoder kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "bitops.h"
#include "layout.h"

namespace readkv {

// 1/sqrt(128), the double nearest to it (the attention scale 1/sqrt(d_h) and
// the Hadamard-sign transforms' normalisation)
constexpr double kInvSqrt128 = 0.088388347648318440550;

// A block's coordinates in the grid of one stage: its own launch's
// (blockIdx, gridDim), or a virtual block of a persistent launch that walks
// the stage's grid.
struct VBlock {
  int x, y, nx, ny;
};
__device__ __forceinline__ VBlock launch_block() {
  return VBlock{(int)blockIdx.x, (int)blockIdx.y, (int)gridDim.x, (int)gridDim.y};
}

__device__ __forceinline__ const ReqRecord& req_of(const uint8_t* store, int b) {
  return *reinterpret_cast<const ReqRecord*>(store + 256 + 32 * (int64_t)b);
}

__device__ __forceinline__ StoreHeader* header_of(uint8_t* store) {
  return reinterpret_cast<StoreHeader*>(store);
}

// element load in the store's input type (0 = bf16 bits, 1 = f32)
template <int DT>
__device__ __forceinline__ double load_elem(const void* p, int64_t i) {
  if constexpr (DT == 0) {
    return (double)bf16_to_float(((const uint16_t*)p)[i]);
  } else {
    return (double)((const float*)p)[i];
  }
}
template <int DT>
__device__ __forceinline__ float load_elem_f(const void* p, int64_t i) {
  if constexpr (DT == 0) {
    return bf16_to_float(((const uint16_t*)p)[i]);
  } else {
    return ((const float*)p)[i];
  }
}

__device__ __forceinline__ double ldexp_pow2(int e) {
  // 2^e for -1022 <= e <= 1023
  return bitsd((uint64_t)(e + 1023) << 52);
}

__device__ __forceinline__ float ldexp_pow2f(int e) {
  // 2^e for -126 <= e <= 127
  return __uint_as_float((uint32_t)(e + 127) << 23);
}

// Attention weights e = exp(s - m) in [0, 1] kept in 32 bits: bits 61..30
// of the fp64 pattern (bits 63 and 62 are zero for every value in [0, 1]),
// rounded to nearest.  The full fp64 exponent range survives (every e down
// to 2^-1074 keeps a non-zero code) with 22 mantissa bits, a relative
// rounding error below 2^-23.
__device__ __forceinline__ uint32_t enc_e(double e) {
  return (uint32_t)((dbits(e) + (1ull << 29)) >> 30);
}
__device__ __forceinline__ double dec_e(uint32_t b) { return bitsd((uint64_t)b << 30); }

// e^x for x <= 0 (or -inf), relative error below 1e-9.  Cody-Waite range
// reduction x = k ln2 + r (k = rint(x / ln2), ln2 in two parts, so r is
// exact to ~1e-17 and |r| <= ln2 / 2), then
//   e^r = 1 + r + r^2 (1/2 + r P(r)),  P(r) = sum_{i>=0} r^i / (i + 3)!
// with P's Taylor polynomial (degree 5: truncation r^9 / 9! below 3e-10) evaluated
// in fp32: its rounding error, weighted by |r|^3 <= 0.042, stays below
// 1e-9 of the result.  Then the exact scaling 2^k.
__device__ __forceinline__ double exp_nonpos(double x) {
  const double xc = fmax(x, -745.0);
  const double k = rint(xc * 1.4426950408889634074);
  const double r = fma(k, -1.9082149292705877000e-10, fma(k, -6.9314718036912381649e-01, xc));
  const float rf = (float)r;
  float pp = 2.4801587e-05f;                 // 1/8!
  pp = fmaf(pp, rf, 1.9841270e-04f);         // 1/7!
  pp = fmaf(pp, rf, 1.3888889e-03f);         // 1/6!
  pp = fmaf(pp, rf, 8.3333333e-03f);         // 1/5!
  pp = fmaf(pp, rf, 4.1666668e-02f);         // 1/4!
  pp = fmaf(pp, rf, 1.6666667e-01f);         // 1/3!
  const double e = fma(r * r, fma(r, (double)pp, 0.5), 1.0 + r);
  const double v = ldexp(e, (int)k);
  return x > -745.0 ? v : 0.0;
}


// Raw buffer resources (stride 0): the fourth descriptor word of the GFX9
// family for untyped 32-bit data, and an offset past any buffer this code
// builds (a load there returns zeros and makes no memory access).
constexpr int kBufWord3 = 0x00020000;
constexpr int kBufOff = (int)0x80000000u;

// wave64 helpers built on DPP lane moves (no LDS round trips).
// DPP control codes of the GFX9 family.
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = dbits(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return bitsd(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = dbits(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return bitsd(((uint64_t)hi << 32) | lo);
}

// op-reduction over each 16-lane row; every lane of the row gets the result
template <typename T, typename Op>
__device__ __forceinline__ T row_reduce(T v, Op op) {
  if constexpr (sizeof(T) == 8) {
    v = op(v, dpp_f64<kDppQuadXor1>(v));
    v = op(v, dpp_f64<kDppQuadXor2>(v));
    v = op(v, dpp_f64<kDppRowHalfMirror>(v));
    v = op(v, dpp_f64<kDppRowMirror>(v));
  } else {
    v = op(v, dpp_f32<kDppQuadXor1>(v));
    v = op(v, dpp_f32<kDppQuadXor2>(v));
    v = op(v, dpp_f32<kDppRowHalfMirror>(v));
    v = op(v, dpp_f32<kDppRowMirror>(v));
  }
  return v;
}

// sum over groups of P consecutive lanes (P = 2, 4, 8, 16, 32, 64); every
// lane of a group gets its group's sum
template <int P, typename T>
__device__ __forceinline__ T group_sum(T v) {
  auto dpp = [](T x, auto ctrl) {
    if constexpr (sizeof(T) == 8) return dpp_f64<decltype(ctrl)::value>(x);
    else return dpp_f32<decltype(ctrl)::value>(x);
  };
  if constexpr (P >= 2) v += dpp(v, std::integral_constant<int, kDppQuadXor1>{});
  if constexpr (P >= 4) v += dpp(v, std::integral_constant<int, kDppQuadXor2>{});
  if constexpr (P >= 8) v += dpp(v, std::integral_constant<int, kDppRowHalfMirror>{});
  if constexpr (P >= 16) v += dpp(v, std::integral_constant<int, kDppRowMirror>{});
  if constexpr (P >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (P >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its outstanding global loads or stores (a full
// __syncthreads() would also drain loads in flight and stores not yet
// acknowledged).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// orders this wave's LDS accesses before and after it (no block barrier)
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// integer max over the wave, every lane gets it
__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, (int)dpp_u32<kDppQuadXor1>((uint32_t)v));
  v = max(v, (int)dpp_u32<kDppQuadXor2>((uint32_t)v));
  v = max(v, (int)dpp_u32<kDppRowHalfMirror>((uint32_t)v));
  v = max(v, (int)dpp_u32<kDppRowMirror>((uint32_t)v));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// integer sum over the wave, every lane gets it
__device__ __forceinline__ int wave_sum_i32(int v) {
  v += (int)dpp_u32<kDppQuadXor1>((uint32_t)v);
  v += (int)dpp_u32<kDppQuadXor2>((uint32_t)v);
  v += (int)dpp_u32<kDppRowHalfMirror>((uint32_t)v);
  v += (int)dpp_u32<kDppRowMirror>((uint32_t)v);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// sum / max over the wave (rows combined in fixed order 0,1,2,3)
__device__ __forceinline__ double wave_sum(double v) {
  v = row_reduce(v, [](double a, double b) { return a + b; });
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}
__device__ __forceinline__ double wave_max(double v) {
  v = row_reduce(v, [](double a, double b) { return fmax(a, b); });
  return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)), fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row_reduce(v, [](float a, float b) { return a + b; });
  auto rl = [](float x, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l)); };
  return (rl(v, 0) + rl(v, 16)) + (rl(v, 32) + rl(v, 48));
}

}  // namespace readkv
