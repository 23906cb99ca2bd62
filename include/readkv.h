/*
 * readkv.h -- C ABI of the ReadKV decode-attention library for AMD MI355X
 * (gfx950).
 *
 * The method ("Read What Matters: Query-Adaptive Quantization for KV
 * Caches", arXiv 2610.11245): every cached key and value scalar is stored
 * once as a W-bit progressive code whose every prefix is decodable (Sec. 3.1).
 * At each decode step the query chooses how many prefix bits of every key
 * channel to read under a read budget, attention is computed from the
 * reconstructed keys, and that attention chooses how many prefix bits of
 * every value token to read (Sec. 3.2-3.3, Algorithm 1; a staged(2) reader
 * in the sense of Sec. 2).  Stored records are never rewritten.
 *
 * Two codes (readkv_config.codec):
 * READKV_CODEC_UNIFORM: per (request, KV head, channel, 32-token group)
 *   uniform min/max quantiser; lo = bf16 group minimum rounded down, rng =
 *   bf16 range rounded up; code = min(floor((x - lo) * 2^W / rng), 2^W - 1);
 *   stored as W MSB-first bit-planes.  A depth-t prefix P reconstructs to
 *   lo + rng * (2P + 1) / 2^(t+1).  Refinement gains follow D(t) ~ 4^-t.
 * READKV_CODEC_LLOYD: the pages' own code (Sec. 3.1, App. D.1).  Keys and
 *   queries pass through a Hadamard-sign transform U_K x = H (s_K . x) /
 *   sqrt(d_h), values through U_V (the output is mapped back by U_V^T);
 *   every transformed scalar is standardised with its KV head's calibrated
 *   channel mean and scale, z = (x' - mu) / sigma, and stored as its path
 *   in the depth-8 Gaussian Lloyd tree (first W levels), as W MSB-first
 *   bit-planes.  A depth-t prefix reconstructs to mu + sigma * (float32
 *   centroid of its depth-t cell); gains are the tree's float32 Delta_t
 *   (Lemma 7).  The store carries the tree, the signs and the calibration
 *   (readkv_codec_init) in a codec block after its header.
 *
 * Ownership: the caller allocates every buffer (store, workspace, inputs,
 * outputs) in device memory and keeps it alive until the enqueued work
 * completes.  The library allocates no device memory (apart from the fixed
 * scratch of readkv_decode_attn_noalloc), never synchronises the stream
 * (except readkv_store_init and readkv_store_status, which say so), and
 * keeps no state beyond its loaded kernels and that scratch.  Calls on
 * different streams are independent if they use different stores and
 * workspaces.
 *
 * Errors: every entry point returns 0 on success or a negative READKV_E*
 * code.  All argument checks happen on the host before anything is
 * enqueued; on error nothing is enqueued.  READKV_ELAUNCH reports a failed
 * kernel launch.  Device-side conditions (non-finite input, append beyond
 * capacity) set sticky flags in the store header, read with
 * readkv_store_status.
 *
 * `stream` arguments are hipStream_t values passed as void* (NULL = the
 * default stream).
 */
#ifndef READKV_H
#define READKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define READKV_OK 0
#define READKV_EINVAL (-1)       /* bad argument or config                  */
#define READKV_ENOSPC (-2)       /* append larger than the store capacity   */
#define READKV_EWORKSPACE (-3)   /* store or workspace buffer too small     */
#define READKV_EDTYPE (-4)       /* unknown element type                    */
#define READKV_EUNSUPPORTED (-5) /* valid but not built (d_h != 128, ...)   */
#define READKV_ELAUNCH (-6)      /* a HIP launch or copy failed             */
#define READKV_ESCRATCH (-7)     /* workspace need above the fixed scratch of
                                    readkv_decode_attn_noalloc              */

#define READKV_BF16 0
#define READKV_F32 1

#define READKV_CODEC_UNIFORM 0
#define READKV_CODEC_LLOYD 1

/* Value-item scale s in the value weight (Sec. 3.2, Eq. (3); App. D.2):
 * PHYSICAL = sum over channels of the token group's squared range (uniform
 * code) or of the KV head's squared calibrated scales sigma^V (Lloyd code),
 * UNIT = 1 (standardised units). */
#define READKV_VSCALE_PHYSICAL 0
#define READKV_VSCALE_UNIT 1

/* Budget scope (Sec. 3.3; Sec. 5.1 and App. F.8 for the per-head policy):
 * KV_HEAD = one key budget over the d_h channels and one value budget over
 * the packed tokens of every (request, KV head); LAYER = one key budget over
 * the G * d_h channels and one value budget over the G * T_packed tokens of
 * every request (all KV heads of the layer pooled). */
#define READKV_SCOPE_KV_HEAD 0
#define READKV_SCOPE_LAYER 1

/* Restrictions of the pages' GPU reader (Sec. 5.1, App. F.8), OR'ed into
 * the policy argument of readkv_decode_attn:
 * MIN_DEPTH1: every key channel and value token is read to depth >= 1; those
 *   N levels count against the budget (App. F.6), max(0, B - N) remain, and
 *   the minimum is kept even when B < N.
 * VALUE_PAIRS: tokens 2m and 2m + 1 of a KV head share one value depth; a
 *   pair is one item whose weight is the sum of its tokens' weights, and a
 *   pair level costs two token levels (floor(B_V / 2) pair levels). */
#define READKV_RESTRICT_MIN_DEPTH1 0x10
#define READKV_RESTRICT_VALUE_PAIRS 0x20

/* The single-launch reader (Sec. 7 names fusing the reader's launches as the
 * way to close its latency gap), OR'ed into the policy argument: the whole
 * step as one cooperative launch of as many blocks as fit on the GPU at once,
 * its stages (score with key allocation, value weights, value selection,
 * gather, output reduction) separated by grid-wide barriers instead of launch
 * boundaries.  Results are bitwise those of the split launches.  Uniform code
 * and READKV_SCOPE_KV_HEAD only, on a device with cooperative launch
 * (EUNSUPPORTED otherwise); the READKV_RESTRICT_* flags apply.  Not for
 * stream capture (a cooperative launch). */
#define READKV_SINGLE_LAUNCH 0x40

/* Logical-read counters of one decode call (App. A.1: payload and metadata
 * bits the reader asks for; workspace and schedules are not counted), summed
 * over every request and KV head:
 *   [READKV_CTR_KEY_PAYLOAD]   sum over units of T_packed * sum_c t^K_c
 *   [READKV_CTR_VALUE_PAYLOAD] sum over units of d_h * sum_j t^V_j
 *   [READKV_CTR_METADATA]      uniform code: lo and rng (16 bits each) of
 *                              every closed group and channel of keys and
 *                              values, E^K (d_h x 64 bits) and E^V (64 bits
 *                              per closed group); Lloyd code: one load per
 *                              call of the layer's calibration arrays (mu,
 *                              sigma of keys and values, 32 bits per KV head
 *                              and channel) and of the decoder table (510
 *                              centroids and 8 gains, 32 bits each)
 *   [READKV_CTR_OPEN_GROUP]    keys and values of the open group in kv_dtype */
#define READKV_CTR_KEY_PAYLOAD 0
#define READKV_CTR_VALUE_PAYLOAD 1
#define READKV_CTR_METADATA 2
#define READKV_CTR_OPEN_GROUP 3
#define READKV_NUM_COUNTERS 4

/* Store flags (readkv_store_status) */
#define READKV_FLAG_NONFINITE 1u /* a group held a non-finite value; it was
                                    stored with codes 0 (and lo = rng = 0)   */
#define READKV_FLAG_OVERFLOW 2u  /* an append ran past a request's capacity;
                                    the tokens beyond it were dropped        */

typedef struct readkv_config {
  int32_t W;               /* stored bits per scalar, 1..8 (Sec. 2: W)     */
  int32_t head_dim;        /* d_h; this build supports 128                 */
  int32_t num_q_heads;     /* H query heads                                */
  int32_t num_kv_heads;    /* G KV heads; H % G == 0, H/G <= 8 (GQA map
                              g(h) = h / (H/G), Sec. 3.1)                  */
  int32_t group_tokens;    /* quantiser group along tokens; must be 32     */
  int32_t batch;           /* B requests                                   */
  int64_t capacity_tokens; /* largest per-request capacity, tokens (also
                              the default capacity of every request);
                              at most 2^26                                 */
  int32_t kv_dtype;        /* READKV_BF16 or READKV_F32: element type of
                              appended K/V, of the open-group buffer and of
                              queries                                      */
  int32_t codec;           /* READKV_CODEC_UNIFORM or READKV_CODEC_LLOYD   */
} readkv_config;

/* Check a config.  Returns 0, EINVAL, EDTYPE or EUNSUPPORTED. */
int readkv_validate_config(const readkv_config* cfg);

/* Bytes of device memory a store needs.  req_capacity: host array [batch]
 * of per-request capacities in tokens, each in 1..capacity_tokens (ragged
 * batches get per-request regions), or NULL to give every request
 * cfg->capacity_tokens.  Capacities round up to a multiple of 32.  Host only. */
int readkv_store_bytes(const readkv_config* cfg, const int64_t* req_capacity,
                       size_t* bytes);

/* Bytes of device workspace one readkv_decode_attn call needs (scores,
 * probabilities, weights, depth schedules, partial outputs; sized for
 * capacity_tokens per request).  Host only. */
int readkv_workspace_bytes(const readkv_config* cfg, size_t* bytes);

/* Format a store: writes the header (per-request lengths 0) and zeroes every
 * record.  store_bytes must be >= readkv_store_bytes.  Synchronises
 * `stream` before returning (the header is staged from host memory). */
int readkv_store_init(const readkv_config* cfg, void* store,
                      size_t store_bytes, const int64_t* req_capacity,
                      void* stream);

/* Lloyd code only: set the store's transform signs and calibrate it
 * (Sec. 3.1; App. D.1: means and scales per KV head and transformed
 * channel from held-out data).  Call after readkv_store_init and before the
 * first append (until then the signs are +1, means 0 and scales 1).
 * signs_k, signs_v: host int8 [head_dim] of +1 / -1 (the signs s_K, s_V of
 *   U_K and U_V, drawn once by the caller), or NULL for all +1.
 * k_cal, v_cal: device [n_cal][num_kv_heads][head_dim] calibration keys and
 *   values in kv_dtype, 1 <= n_cal <= 2^24.
 * Per KV head g and channel c: x' = U x of every calibration token;
 * mu = (sum x') / n_cal and sigma = sqrt(sum (x' - mu)^2 / n_cal), sums in
 * token order in float64, then rounded to float32; a zero or non-finite
 * sigma becomes 1.  Also stores s_g = sum_c sigma^V_{g,c}^2.  EINVAL for a
 * uniform-code store or a bad argument.  Synchronises `stream`. */
int readkv_codec_init(const readkv_config* cfg, void* store,
                      const int8_t* signs_k, const int8_t* signs_v,
                      const void* k_cal, const void* v_cal, int64_t n_cal,
                      void* stream);

/* The library's Lloyd-tree table (App. D.1), host arrays: cent_out [511]
 * float32 centroids, depth-t cell P at (2^t - 1) + P (t = 0..8, depth 0 is
 * 0); bounds_out [255] the encoder's boundary of depth-t cell P at
 * (2^t - 1) + P (t = 0..7, the midpoint of the two float32 child
 * centroids); gains_out [9] the float32 gains Delta_t = D(t-1) - D(t),
 * t = 1..8 (gains_out[0] = 0).  Host only, no device access. */
int readkv_codec_tables(float* cent_out, double* bounds_out, double* gains_out);

/* Append new tokens (the encoder of Sec. 3.1 / Algorithm 1).
 * k_new, v_new: device [batch][num_kv_heads][n_max][head_dim] in kv_dtype;
 *   request b contributes its first n_new[b] rows (ragged prefill).
 * n_new: device int32 [batch], or NULL for n_max rows in every request.
 * When a request's open group reaches 32 tokens the group is quantised and
 * its bit-planes (uniform code: also its metadata and energy sums) are
 * written once; tokens of a still-open group are kept exactly.  Returns ENOSPC if n_max exceeds the
 * store's default capacity. */
int readkv_encode_append(const readkv_config* cfg, void* store,
                         const void* k_new, const void* v_new,
                         const int32_t* n_new, int32_t n_max, void* stream);

/* One decode step of ReadKV attention for every request and query head
 * (Sec. 3.2-3.3, Algorithm 1).
 * q: device [batch][num_q_heads][head_dim] in kv_dtype.  A unit (request,
 *   KV head) any of whose query values is not finite reads nothing: its
 *   depths are 0 and its outputs NaN.  A request that holds no token reads
 *   nothing and its outputs are 0 (the empty sum), whatever its query; its
 *   key depths are the minimum under the uniform code (no key energy) and
 *   are allocated as for any request under the Lloyd code (its key weights
 *   hold no context term).
 * R_K, R_V: read bits per scalar for the key and value stages (finite,
 *   >= 0; the nominal rate is R = (R_K + R_V)/2, Sec. 3.3).  Budgets (R as
 *   float32, product in double): B_K = floor(R_K * d_h) key refinements over
 *   the d_h channels, B_V = floor(R_V * T_packed) value refinements over the
 *   tokens of closed groups, per (request, KV head) for
 *   READKV_SCOPE_KV_HEAD; for READKV_SCOPE_LAYER one B_K = floor(R_K * G *
 *   d_h) over the G * d_h channels and one B_V = floor(R_V * G * T_packed)
 *   over the G * T_packed tokens of each request, items ordered by KV head
 *   then channel / token (ties to the lowest in that order).
 * policy: READKV_SCOPE_KV_HEAD or READKV_SCOPE_LAYER (the latter needs
 *   num_kv_heads <= 32, else EUNSUPPORTED), OR'ed with any of the
 *   READKV_RESTRICT_* flags and READKV_SINGLE_LAUNCH; other bits give
 *   EINVAL.
 * vscale: READKV_VSCALE_PHYSICAL or READKV_VSCALE_UNIT.
 * out: device fp32 [batch][num_q_heads][head_dim].
 * workspace: device, >= readkv_workspace_bytes.
 * key_depths_out: device u8 [batch][num_kv_heads][head_dim] or NULL.
 * value_depths_out: device u8 [batch][num_kv_heads][capacity_max] or NULL
 *   (entries beyond a request's packed length are unspecified).
 * counters_out: device u64 [READKV_NUM_COUNTERS] or NULL; overwritten with
 *   this call's logical reads in bits (see READKV_CTR_*).
 * Allocation is ChooseDepths (Sec. 3.3) with gains a_i * 4^-t (uniform
 * code) or a_i * Delta_t (Lloyd code), exact under diminishing gains (App.
 * E.2.1, Prop. 8); ties go to the lowest channel / token index; only
 * positive gains are taken.  Lloyd code: key weights (q'_c sigma^K_c)^2
 * summed over the KV head's query heads with q' = U_K q, logits
 * q' . k_hat' / sqrt(d_h), output U_V^T (sum alpha v_hat'); tokens of the
 * open group use q . k / sqrt(d_h) and their exact values.  Results are bitwise
 * reproducible from call to call. */
int readkv_decode_attn(const readkv_config* cfg, const void* store,
                       const void* q, float R_K, float R_V, int32_t policy,
                       int32_t vscale, float* out, void* workspace,
                       size_t workspace_bytes, uint8_t* key_depths_out,
                       uint8_t* value_depths_out, uint64_t* counters_out,
                       void* stream);

/* readkv_decode_attn with timing hooks: `events` points to 4 hipEvent_t
 * handles created by the caller (as void*); events[0] is recorded on
 * `stream` before the first kernel and events[i] after stage i of the
 * step, in the order score (with the key allocation in its prologue and
 * the split-context softmax partials), value allocation (with the softmax
 * statistics), value gather (with the output reduction); under
 * READKV_SINGLE_LAUNCH events[1..3] are all recorded after the one launch.
 * Arguments and results are otherwise those of readkv_decode_attn (EINVAL
 * if events or any of the 4 handles is NULL). */
int readkv_decode_attn_timed(const readkv_config* cfg, const void* store,
                             const void* q, float R_K, float R_V,
                             int32_t policy, int32_t vscale, float* out,
                             void* workspace, size_t workspace_bytes,
                             uint8_t* key_depths_out,
                             uint8_t* value_depths_out,
                             uint64_t* counters_out, void* const* events,
                             void* stream);

/* readkv_decode_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and arguments, minus the workspace,
 * which is a fixed array of READKV_NOALLOC_SCRATCH_BYTES per GPU held by the
 * library until the process ends.  Calls whose readkv_workspace_bytes
 * exceeds it return READKV_ESCRATCH before enqueuing anything.  The call
 * allocates nothing; its first call on a device looks the array's address
 * up (make one call before capturing a graph).  Every call on a GPU uses
 * that GPU's one array: calls that overlap in time on one GPU (different
 * streams, or graphs replayed concurrently) race and give wrong results. */
#define READKV_NOALLOC_SCRATCH_BYTES (64u << 20)
int readkv_decode_attn_noalloc(const readkv_config* cfg, const void* store,
                               const void* q, float R_K, float R_V,
                               int32_t policy, int32_t vscale, float* out,
                               uint8_t* key_depths_out,
                               uint8_t* value_depths_out,
                               uint64_t* counters_out, void* stream);

/* Read the store's sticky flags and per-request lengths (host arrays;
 * lengths_out [batch] may be NULL).  Synchronous device-to-host copy. */
int readkv_store_status(const readkv_config* cfg, const void* store,
                        uint32_t* flags_out, int64_t* lengths_out);

/* Static description of an error code. */
const char* readkv_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* READKV_H */
