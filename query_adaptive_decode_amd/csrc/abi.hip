// C ABI entry points: argument checks on the host, then enqueue.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/readkv.h"
#include "layout.h"
#include "readkv_internal.h"

using namespace readkv;

namespace {

int esize_of(int dt) { return dt == READKV_BF16 ? 2 : 4; }

int64_t cap_of(const readkv_config* cfg, const int64_t* req_capacity, int b) {
  const int64_t c = req_capacity ? req_capacity[b] : cfg->capacity_tokens;
  return align_up(c, kGroup);
}

// Per-request capacities may be smaller than cfg->capacity_tokens, which is
// the largest one (workspace sizes follow it).
int check_caps(const readkv_config* cfg, const int64_t* req_capacity) {
  if (!req_capacity) return READKV_OK;
  for (int b = 0; b < cfg->batch; ++b)
    if (req_capacity[b] <= 0 || req_capacity[b] > cfg->capacity_tokens) return READKV_EINVAL;
  return READKV_OK;
}

int64_t capmax_of(const readkv_config* cfg) { return align_up(cfg->capacity_tokens, kGroup); }

// Build the host image of the header + request table.
std::vector<uint8_t> header_image(const readkv_config* cfg, const int64_t* req_capacity,
                                  int64_t* total) {
  const int64_t hb = header_bytes(cfg->batch);
  std::vector<uint8_t> img((size_t)hb, 0);
  StoreHeader h;
  memset(&h, 0, sizeof(h));
  h.magic = kMagic;
  h.version = kVersion;
  h.W = cfg->W;
  h.d = cfg->head_dim;
  h.H = cfg->num_q_heads;
  h.G = cfg->num_kv_heads;
  h.group_tokens = cfg->group_tokens;
  h.B = cfg->batch;
  h.kv_dtype = cfg->kv_dtype;
  h.flags = 0;
  h.capacity = capmax_of(cfg);
  h.codec = cfg->codec;
  int64_t off = hb + codec_bytes(cfg->codec, cfg->num_kv_heads, cfg->head_dim);
  for (int b = 0; b < cfg->batch; ++b) {
    ReqRecord r;
    r.len = 0;
    r.cap = cap_of(cfg, req_capacity, b);
    r.offset = off;
    r.reserved = 0;
    memcpy(img.data() + 256 + 32 * (size_t)b, &r, sizeof(r));
    off += region_layout(cfg->num_kv_heads, cfg->head_dim, cfg->W, r.cap,
                         esize_of(cfg->kv_dtype)).size;
  }
  h.total_bytes = off;
  memcpy(img.data(), &h, sizeof(h));
  *total = off;
  return img;
}

// Scratch of readkv_decode_attn_noalloc: one fixed array per GPU, in place
// of a caller-provided workspace.  In host code `scratch` names a host-side
// stand-in, never the device memory: the device address comes from
// hipGetSymbolAddress, once per device (with that device current), and only
// that address is handed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return READKV_ELAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return READKV_ELAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return READKV_OK;
}

}  // namespace

extern "C" {

int readkv_validate_config(const readkv_config* cfg) {
  if (!cfg) return READKV_EINVAL;
  if (cfg->kv_dtype != READKV_BF16 && cfg->kv_dtype != READKV_F32) return READKV_EDTYPE;
  if (cfg->W < 1 || cfg->W > 8) return READKV_EINVAL;
  if (cfg->head_dim <= 0 || cfg->num_q_heads <= 0 || cfg->num_kv_heads <= 0 ||
      cfg->batch <= 0 || cfg->group_tokens <= 0 || cfg->capacity_tokens <= 0)
    return READKV_EINVAL;
  if (cfg->num_q_heads % cfg->num_kv_heads != 0) return READKV_EINVAL;
  if (cfg->capacity_tokens > (int64_t(1) << 26)) return READKV_EINVAL;
  if (cfg->codec != READKV_CODEC_UNIFORM && cfg->codec != READKV_CODEC_LLOYD) return READKV_EINVAL;
  if (cfg->head_dim != kDim) return READKV_EUNSUPPORTED;
  if (cfg->group_tokens != kGroup) return READKV_EUNSUPPORTED;
  if (cfg->num_q_heads / cfg->num_kv_heads > 8) return READKV_EUNSUPPORTED;
  return READKV_OK;
}

int readkv_store_bytes(const readkv_config* cfg, const int64_t* req_capacity, size_t* bytes) {
  int rc = readkv_validate_config(cfg);
  if (rc) return rc;
  if (!bytes) return READKV_EINVAL;
  if ((rc = check_caps(cfg, req_capacity))) return rc;
  int64_t total = 0;
  header_image(cfg, req_capacity, &total);
  *bytes = (size_t)total;
  return READKV_OK;
}

int readkv_workspace_bytes(const readkv_config* cfg, size_t* bytes) {
  int rc = readkv_validate_config(cfg);
  if (rc) return rc;
  if (!bytes) return READKV_EINVAL;
  const WsLayout L = ws_layout(cfg->batch, cfg->num_q_heads, cfg->num_kv_heads, cfg->head_dim,
                               capmax_of(cfg), cfg->codec);
  *bytes = (size_t)L.size;
  return READKV_OK;
}

int readkv_store_init(const readkv_config* cfg, void* store, size_t store_bytes,
                      const int64_t* req_capacity, void* stream) {
  int rc = readkv_validate_config(cfg);
  if (rc) return rc;
  if (!store) return READKV_EINVAL;
  if ((rc = check_caps(cfg, req_capacity))) return rc;
  int64_t total = 0;
  std::vector<uint8_t> img = header_image(cfg, req_capacity, &total);
  if ((int64_t)store_bytes < total) return READKV_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (launch_store_zero(store, (size_t)total, st)) return READKV_ELAUNCH;
  if (hipMemcpyAsync(store, img.data(), img.size(), hipMemcpyHostToDevice, st) != hipSuccess)
    return READKV_ELAUNCH;
  std::vector<uint8_t> cimg;
  if (cfg->codec == READKV_CODEC_LLOYD) {
    cimg.resize((size_t)codec_bytes(1, cfg->num_kv_heads, cfg->head_dim));
    codec_block_image(cfg->num_kv_heads, cimg.data());
    if (hipMemcpyAsync((uint8_t*)store + img.size(), cimg.data(), cimg.size(),
                       hipMemcpyHostToDevice, st) != hipSuccess)
      return READKV_ELAUNCH;
  }
  if (hipStreamSynchronize(st) != hipSuccess) return READKV_ELAUNCH;
  return READKV_OK;
}

int readkv_codec_init(const readkv_config* cfg, void* store, const int8_t* signs_k,
                      const int8_t* signs_v, const void* k_cal, const void* v_cal, int64_t n_cal,
                      void* stream) {
  int rc = readkv_validate_config(cfg);
  if (rc) return rc;
  if (cfg->codec != READKV_CODEC_LLOYD || !store || !k_cal || !v_cal || n_cal < 1 ||
      n_cal > (int64_t(1) << 24))
    return READKV_EINVAL;
  std::vector<double> sg(2 * (size_t)kDim, 1.0);
  for (int c = 0; c < kDim; ++c) {
    if (signs_k) {
      if (signs_k[c] != 1 && signs_k[c] != -1) return READKV_EINVAL;
      sg[c] = (double)signs_k[c];
    }
    if (signs_v) {
      if (signs_v[c] != 1 && signs_v[c] != -1) return READKV_EINVAL;
      sg[kDim + c] = (double)signs_v[c];
    }
  }
  hipStream_t st = (hipStream_t)stream;
  const CodecLayout C = codec_layout(cfg->num_kv_heads, kDim);
  uint8_t* cb = (uint8_t*)store + header_bytes(cfg->batch);
  static_assert(sizeof(double) * kDim * 2 == 2048, "sk and sv are adjacent");
  if (C.sv != C.sk + kDim * 8) return READKV_ELAUNCH;
  if (hipMemcpyAsync(cb + C.sk, sg.data(), sg.size() * sizeof(double), hipMemcpyHostToDevice, st) !=
      hipSuccess)
    return READKV_ELAUNCH;
  if (launch_calibrate(cb, cfg->num_kv_heads, cfg->kv_dtype, k_cal, v_cal, n_cal, st))
    return READKV_ELAUNCH;
  if (hipStreamSynchronize(st) != hipSuccess) return READKV_ELAUNCH;
  return READKV_OK;
}

int readkv_codec_tables(float* cent_out, double* bounds_out, double* gains_out) {
  if (!cent_out || !bounds_out || !gains_out) return READKV_EINVAL;
  const TreeTables& T = lloyd_tables();
  for (int i = 0; i < 511; ++i) cent_out[i] = T.cent[i];
  for (int i = 0; i < 255; ++i) bounds_out[i] = T.bounds[i];
  for (int t = 0; t <= kTreeDepth; ++t) gains_out[t] = T.gains[t];
  return READKV_OK;
}

int readkv_encode_append(const readkv_config* cfg, void* store, const void* k_new,
                         const void* v_new, const int32_t* n_new, int32_t n_max, void* stream) {
  int rc = readkv_validate_config(cfg);
  if (rc) return rc;
  if (!store || n_max < 0) return READKV_EINVAL;
  if (n_max == 0) return READKV_OK;
  if (!k_new || !v_new) return READKV_EINVAL;
  if ((int64_t)n_max > align_up(cfg->capacity_tokens, kGroup)) return READKV_ENOSPC;
  EncodeArgs a;
  a.store = store;
  a.knew = k_new;
  a.vnew = v_new;
  a.n_new = n_new;
  a.n_max = n_max;
  a.B = cfg->batch;
  a.G = cfg->num_kv_heads;
  a.W = cfg->W;
  a.dtype = cfg->kv_dtype;
  a.codec = cfg->codec;
  a.cblock = (const uint8_t*)store + header_bytes(cfg->batch);
  return launch_encode(a, (hipStream_t)stream) ? READKV_ELAUNCH : READKV_OK;
}

static int decode_impl(const readkv_config* cfg, const void* store, const void* q, float R_K,
                       float R_V, int32_t policy, int32_t vscale, float* out, void* workspace,
                       size_t workspace_bytes, uint8_t* key_depths_out,
                       uint8_t* value_depths_out, uint64_t* counters_out, void* const* events,
                       void* stream) {
  int rc = readkv_validate_config(cfg);
  if (rc) return rc;
  if (!store || !q || !out || !workspace) return READKV_EINVAL;
  if (!isfinite(R_K) || !isfinite(R_V) || R_K < 0.f || R_V < 0.f) return READKV_EINVAL;
  if (vscale != READKV_VSCALE_PHYSICAL && vscale != READKV_VSCALE_UNIT) return READKV_EINVAL;
  if (policy & ~(READKV_SCOPE_LAYER | READKV_RESTRICT_MIN_DEPTH1 | READKV_RESTRICT_VALUE_PAIRS |
                 READKV_SINGLE_LAUNCH))
    return READKV_EINVAL;
  const int scope = policy & READKV_SCOPE_LAYER;
  if (scope == READKV_SCOPE_LAYER && cfg->num_kv_heads > kMaxPooledKV) return READKV_EUNSUPPORTED;
  const int fused = (policy & READKV_SINGLE_LAUNCH) ? 1 : 0;
  if (fused && (scope == READKV_SCOPE_LAYER || cfg->codec != READKV_CODEC_UNIFORM))
    return READKV_EUNSUPPORTED;
  // budgets must fit the 32-bit counters: R * (items of a domain) <= 2^31
  const double nu = scope == READKV_SCOPE_LAYER ? (double)cfg->num_kv_heads : 1.0;
  if ((double)R_V * (double)align_up(cfg->capacity_tokens, kGroup) * nu > 2147483647.0 ||
      (double)R_K * cfg->head_dim * nu > 2147483647.0)
    return READKV_EINVAL;
  const int64_t capmax = capmax_of(cfg);
  const WsLayout L = ws_layout(cfg->batch, cfg->num_q_heads, cfg->num_kv_heads, cfg->head_dim,
                               capmax, cfg->codec);
  if ((int64_t)workspace_bytes < L.size) return READKV_EWORKSPACE;
  DecodeArgs a;
  a.store = store;
  a.q = q;
  a.RK = R_K;
  a.RV = R_V;
  a.vscale = vscale;
  a.out = out;
  a.ws = (uint8_t*)workspace;
  a.key_depths_out = key_depths_out;
  a.value_depths_out = value_depths_out;
  a.counters = counters_out;
  a.scope = scope;
  a.min1 = (policy & READKV_RESTRICT_MIN_DEPTH1) ? 1 : 0;
  a.pairs = (policy & READKV_RESTRICT_VALUE_PAIRS) ? 1 : 0;
  a.B = cfg->batch;
  a.H = cfg->num_q_heads;
  a.G = cfg->num_kv_heads;
  a.W = cfg->W;
  a.dtype = cfg->kv_dtype;
  a.capmax = capmax;
  a.events = events;
  a.codec = cfg->codec;
  a.cblock = (const uint8_t*)store + header_bytes(cfg->batch);
  a.fused = fused;
  rc = launch_decode(a, (hipStream_t)stream);
  if (rc == -5) return READKV_EUNSUPPORTED;
  return rc ? READKV_ELAUNCH : READKV_OK;
}

int readkv_decode_attn(const readkv_config* cfg, const void* store, const void* q, float R_K,
                       float R_V, int32_t policy, int32_t vscale, float* out, void* workspace,
                       size_t workspace_bytes, uint8_t* key_depths_out,
                       uint8_t* value_depths_out, uint64_t* counters_out, void* stream) {
  return decode_impl(cfg, store, q, R_K, R_V, policy, vscale, out, workspace, workspace_bytes,
                     key_depths_out, value_depths_out, counters_out, nullptr, stream);
}

int readkv_decode_attn_timed(const readkv_config* cfg, const void* store, const void* q,
                             float R_K, float R_V, int32_t policy, int32_t vscale, float* out,
                             void* workspace, size_t workspace_bytes, uint8_t* key_depths_out,
                             uint8_t* value_depths_out, uint64_t* counters_out,
                             void* const* events, void* stream) {
  if (!events) return READKV_EINVAL;
  for (int i = 0; i < 4; ++i)
    if (!events[i]) return READKV_EINVAL;
  return decode_impl(cfg, store, q, R_K, R_V, policy, vscale, out, workspace, workspace_bytes,
                     key_depths_out, value_depths_out, counters_out, events, stream);
}

int readkv_decode_attn_noalloc(const readkv_config* cfg, const void* store, const void* q,
                               float R_K, float R_V, int32_t policy, int32_t vscale, float* out,
                               uint8_t* key_depths_out, uint8_t* value_depths_out,
                               uint64_t* counters_out, void* stream) {
  int rc = readkv_validate_config(cfg);
  if (rc) return rc;
  const WsLayout L = ws_layout(cfg->batch, cfg->num_q_heads, cfg->num_kv_heads, cfg->head_dim,
                               capmax_of(cfg), cfg->codec);
  if ((size_t)L.size > kScratchBytes) return READKV_ESCRATCH;
  void* ws = nullptr;
  if ((rc = scratch_of_current_device(&ws))) return rc;
  return decode_impl(cfg, store, q, R_K, R_V, policy, vscale, out, ws, kScratchBytes,
                     key_depths_out, value_depths_out, counters_out, nullptr, stream);
}

int readkv_store_status(const readkv_config* cfg, const void* store, uint32_t* flags_out,
                        int64_t* lengths_out) {
  int rc = readkv_validate_config(cfg);
  if (rc) return rc;
  if (!store || !flags_out) return READKV_EINVAL;
  std::vector<uint8_t> img((size_t)header_bytes(cfg->batch));
  if (hipMemcpy(img.data(), store, img.size(), hipMemcpyDeviceToHost) != hipSuccess)
    return READKV_ELAUNCH;
  StoreHeader h;
  memcpy(&h, img.data(), sizeof(h));
  if (h.magic != kMagic || h.B != cfg->batch) return READKV_EINVAL;
  *flags_out = h.flags;
  if (lengths_out)
    for (int b = 0; b < cfg->batch; ++b) {
      ReqRecord r;
      memcpy(&r, img.data() + 256 + 32 * (size_t)b, sizeof(r));
      lengths_out[b] = r.len;
    }
  return READKV_OK;
}

const char* readkv_strerror(int code) {
  switch (code) {
    case READKV_OK: return "ok";
    case READKV_EINVAL: return "invalid argument or configuration";
    case READKV_ENOSPC: return "append larger than the store capacity";
    case READKV_EWORKSPACE: return "store or workspace buffer too small";
    case READKV_EDTYPE: return "unknown element type";
    case READKV_EUNSUPPORTED: return "configuration not supported by this build";
    case READKV_ELAUNCH: return "HIP launch or copy failed";
    case READKV_ESCRATCH: return "the call needs more workspace than the fixed scratch holds";
    default: return "unknown error";
  }
}

}  // extern "C"
