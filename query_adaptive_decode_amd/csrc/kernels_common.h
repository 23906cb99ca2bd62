// Device-side helpers shared by the encoder and decoder kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bitops.h"
#include "layout.h"

namespace readkv {

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

// wave64 helpers
__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace readkv
