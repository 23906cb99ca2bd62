// Host-side launch interface between the C ABI and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace readkv {

struct EncodeArgs {
  void* store;
  const void* knew;
  const void* vnew;
  const int32_t* n_new;
  int n_max, B, G, W, dtype;
};

struct DecodeArgs {
  const void* store;
  const void* q;
  float RK, RV;
  int vscale;
  float* out;
  uint8_t* ws;
  uint8_t* key_depths_out;
  uint8_t* value_depths_out;
  uint64_t* counters;   // NULL, or 4 device words (readkv_decode_attn)
  int scope;
  int B, H, G, W, dtype;
  int64_t capmax;
  void* const* events;  // NULL, or 5 hipEvent_t recorded around the 4 kernels
};

int launch_store_zero(void* store, size_t bytes, hipStream_t st);
int launch_encode(const EncodeArgs& a, hipStream_t st);
int launch_decode(const DecodeArgs& a, hipStream_t st);

}  // namespace readkv
