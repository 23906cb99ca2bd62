// Host-side launch interface between the C ABI and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "layout.h"

namespace readkv {

// Per-layer (pooled) budgets: at most this many KV heads per request.
constexpr int kMaxPooledKV = 32;

struct EncodeArgs {
  void* store;
  const void* knew;
  const void* vnew;
  const int32_t* n_new;
  int n_max, B, G, W, dtype;
  int codec;                 // 0: uniform min/max, 1: Lloyd tree
  const uint8_t* cblock;     // the Lloyd-tree store's codec block (device)
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
  int scope;            // 0: per (request, KV head) budgets, 1: per request
  int min1;             // 1: minimum depth one in both stages
  int pairs;            // 1: two-token value packets
  int B, H, G, W, dtype;
  int64_t capmax;
  void* const* events;  // NULL, or 4 hipEvent_t recorded around the 3 stages
  int codec;            // 0: uniform min/max, 1: Lloyd tree
  const uint8_t* cblock;  // the Lloyd-tree store's codec block (device)
  int fused;            // 1: the single-launch reader
};

// The Lloyd tree's float32 table ("Read What Matters", App. D.1), built on
// the host once: cent[(2^t - 1) + P] (t = 0..8), bounds[(2^t - 1) + P]
// (t = 0..7), gains[t] (t = 1..8).
struct TreeTables {
  float cent[512];
  double bounds[256];
  double gains[16];
};
const TreeTables& lloyd_tables();
// codec.hip: the codec block of a new Lloyd-tree store (host image: tables,
// signs +1, mean 0, scale 1), and the calibration launch.
void codec_block_image(int G, uint8_t* img);
int launch_calibrate(uint8_t* cblock, int G, int dtype, const void* kcal, const void* vcal,
                     int64_t ncal, hipStream_t st);

int launch_store_zero(void* store, size_t bytes, hipStream_t st);
int launch_encode(const EncodeArgs& a, hipStream_t st);
int launch_decode(const DecodeArgs& a, hipStream_t st);
// A part of a decode call: the units [ub0, ub0 + nunits) (whole requests).
struct Part {
  int ub0, nunits;
};
// the allocation stages (alloc.hip); tk, tv: the depth arrays of the call
int launch_key_alloc(const DecodeArgs& a, const Part& P, uint8_t* tk, hipStream_t st);
int launch_value_alloc(const DecodeArgs& a, const Part& P, const WsLayout& L, const uint8_t* tk,
                       uint8_t* tv, hipStream_t st);
int launch_key_alloc_lloyd(const DecodeArgs& a, const WsLayout& L, uint8_t* tk, hipStream_t st);

}  // namespace readkv
