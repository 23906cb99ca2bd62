// The two allocation stages of a ReadKV decode step ("Read What Matters:
// Query-Adaptive Quantization for KV Caches", Sec. 3.2-3.3, Algorithm 1):
//
//   k_key_alloc     (one block per request; per-layer budgets only)
//                   key weights (Eq. (2)) and ChooseDepths over the request's
//                   G * d_h key channels -> t^K (per-KV-head budgets are
//                   allocated in the score kernel's block prologue)
//   k_value_weights (B*G x chunks of 1024 tokens, all compute units)
//                   softmax statistics from the score tiles' partials, the
//                   per-tile factors exp(m_tile - m)/Z, and the value weights
//                   (Eq. (3)) of every packed token
//   k_value_select  (one block per selection domain, when its weights fit
//                   in LDS) ChooseDepths over the domain's packed tokens ->
//                   t^V, and the call's logical-read counters
//   k_sel_*         (otherwise) the same ChooseDepths and counters by many
//                   blocks per domain, in a chain of launches (msel.h)
//
// (The block code of the last two is in valloc.h, which the single-launch
// reader shares.)  A selection domain is one (request, KV head) under
// per-KV-head budgets, or one request (its G KV heads pooled, item index =
// KV head * N + item) under per-layer budgets.
#include <math.h>

#include "kernels_common.h"
#include "readkv_internal.h"
#include "msel.h"
#include "select.h"
#include "valloc.h"

namespace readkv {

// ---------------------------------------------------------------------------
// Key allocation under per-layer budgets (per-KV-head budgets are allocated
// in the score kernel's prologue).  Item i = (KV head g0 + i / d, channel
// i % d) of the request; w = (sum_{h in S(g)} q_hc^2) * E^K_gc in head order
// (Eq. (2) with sigma^2 read as the channel's summed squared group range).
// A KV head with a non-finite query value gets zero weights (it reads
// nothing).
// ---------------------------------------------------------------------------
template <int GQA, int DT, int NUMAX>
__global__ __launch_bounds__(256) void k_key_alloc(const uint8_t* store, int ub0, const void* q, int H,
                                                   int G, int W, float RK, int NU, int min1,
                                                   uint8_t* tk) {
  constexpr int NT = 256;
  constexpr int esize = DT == 0 ? 2 : 4;
  __shared__ ChooseShared<NT> S;
  __shared__ double wl[NUMAX * kDim];
  __shared__ int bad[NUMAX];
  const int tid = threadIdx.x;
  const int u0 = ub0 + (int)blockIdx.x * NU;
  const int b = u0 / G, g0 = u0 % G;
  const ReqRecord r = req_of(store, b);
  if (tid < NU) bad[tid] = 0;
  __syncthreads();
  const int N = NU * kDim;
  for (int i = tid; i < N; i += NT) {
    const int k = i / kDim, c = i % kDim;
    const Unit u = unit_of(const_cast<uint8_t*>(store), r, g0 + k, G, kDim, W, esize);
    double qsq = 0.0;
    bool nf = false;
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) {
      const double qv = load_elem<DT>(q, ((int64_t)b * H + (int64_t)(g0 + k) * GQA + hh) * kDim + c);
      nf |= !isfinite(qv);
      qsq = __dadd_rn(qsq, __dmul_rn(qv, qv));
    }
    wl[i] = __dmul_rn(qsq, u.ek[c]);
    if (nf) bad[k] = 1;
  }
  __syncthreads();
  // the minimum depth one: levels 2..W of w are levels 1..W-1 of w/4
  // (exact), over the budget left after the N forced levels
  const double sc = min1 ? 0.25 : 1.0;
  for (int i = tid; i < N; i += NT) wl[i] = bad[i / kDim] ? 0.0 : wl[i] * sc;
  __syncthreads();
  uint32_t Bk = (uint32_t)floor((double)RK * (double)N);
  if (min1) Bk = Bk > (uint32_t)N ? Bk - (uint32_t)N : 0u;
  uint8_t* const tkd = tk + (int64_t)u0 * kDim;
  block_choose_depths<NT>(
      N, Bk, W - min1, [&](int64_t i) { return wl[i]; },
      [&](int64_t i, uint32_t t) { tkd[i] = (uint8_t)(t + (uint32_t)min1); }, S);
}

// ---------------------------------------------------------------------------
// Key allocation under the Lloyd-tree code ([ReadKV] Sec. 3.1-3.2), one
// block per selection domain (a unit, or a request's NU = G KV heads under
// per-layer budgets).  Per KV head: the query heads' rows q' = U_K q
// (Walsh-Hadamard butterflies over the block in fp64, times 1/sqrt(d));
// written to the workspace: the score's channel weights q'_hc sigma^K_c
// ([unit][channel][head]) and qb_h = sum_c q'_hc mu^K_c (channel order);
// weights w_c = sum_h (q'_hc sigma^K_c)^2 in head order (Eq. (2)); then
// ChooseDepths with the tree's gains Delta_t.  A KV head with a non-finite
// query value gets zero weights and qb = NaN (the score reads nothing for
// it).  Block 0 zeroes the call's read counters.
// ---------------------------------------------------------------------------
template <int GQA, int DT, int NUMAX>
__global__ __launch_bounds__(256) void k_key_alloc_lloyd(const uint8_t* cb, const void* q, int H,
                                                         int G, int W, float RK, int NU, int min1,
                                                         uint8_t* tk, double* qw, double* qb,
                                                         uint64_t* counters) {
  constexpr int NT = 256;
  constexpr int PER = (GQA * kDim + NT - 1) / NT;
  __shared__ ChooseShared<NT> S;
  __shared__ double wl[NUMAX * kDim];
  __shared__ double xb[GQA * kDim];
  __shared__ double gt[16];
  const CodecLayout C = codec_layout(G, kDim);
  const int tid = threadIdx.x;
  if (counters && blockIdx.x == 0 && tid < 4) counters[tid] = 0ull;
  const int u0 = (int)blockIdx.x * NU;
  const int b = u0 / G, g0 = u0 % G;
  if (tid < 16) gt[tid] = reinterpret_cast<const double*>(cb + C.gains)[tid];
  const double* sk = reinterpret_cast<const double*>(cb + C.sk);
  for (int k = 0; k < NU; ++k) {
    const int g = g0 + k;
    const int64_t hrow = (int64_t)b * H + (int64_t)g * GQA;
    int nf = 0;
    for (int i = tid; i < GQA * kDim; i += NT) {
      const double v = load_elem<DT>(q, hrow * kDim + i);
      nf |= !isfinite(v);
      xb[i] = v * sk[i % kDim];
    }
    nf = __syncthreads_or(nf);
    for (int h = 1; h < kDim; h <<= 1) {
      double y[PER];
#pragma unroll
      for (int n = 0; n < PER; ++n) {
        const int i = tid + n * NT;
        if (i < GQA * kDim) {
          const double a = xb[i], o = xb[i ^ h];  // (h < d: the partner is in the same row)
          y[n] = (i & h) ? o - a : a + o;
        }
      }
      __syncthreads();
#pragma unroll
      for (int n = 0; n < PER; ++n) {
        const int i = tid + n * NT;
        if (i < GQA * kDim) xb[i] = y[n];
      }
      __syncthreads();
    }
    for (int i = tid; i < GQA * kDim; i += NT) xb[i] = __dmul_rn(xb[i], kInvSqrt128);
    __syncthreads();
    if (tid < kDim) {
      const int c = tid;
      const double sg = (double)reinterpret_cast<const float*>(cb + C.sigk)[g * kDim + c];
      double a = 0.0;
      double* const qwc = qw + ((int64_t)(b * G + g) * kDim + c) * GQA;
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) {
        const double x = __dmul_rn(xb[hh * kDim + c], sg);
        qwc[hh] = x;
        a = __dadd_rn(a, __dmul_rn(x, x));
      }
      wl[k * kDim + c] = nf ? 0.0 : a;
    } else if (tid < kDim + GQA) {
      const int hh = tid - kDim;
      const float* mu = reinterpret_cast<const float*>(cb + C.muk) + g * kDim;
      double sacc = 0.0;
      for (int c = 0; c < kDim; ++c) sacc = __dadd_rn(sacc, __dmul_rn(xb[hh * kDim + c], (double)mu[c]));
      qb[hrow + hh] = nf ? __builtin_nan("") : sacc;
    }
    __syncthreads();
  }
  const int N = NU * kDim;
  uint32_t Bk = (uint32_t)floor((double)RK * (double)N);
  if (min1) Bk = Bk > (uint32_t)N ? Bk - (uint32_t)N : 0u;
  uint8_t* const tkd = tk + (int64_t)u0 * kDim;
  // the minimum depth one: levels 2..W, i.e. the table from Delta_2 on
  block_choose_depths<NT>(
      N, Bk, W - min1, [&](int64_t i) { return wl[i]; },
      [&](int64_t i, uint32_t t) { tkd[i] = (uint8_t)(t + (uint32_t)min1); }, S,
      TableGains{gt + min1});
}

// (sel, when not null: the first block of each selection domain of NU units
// zeroes the domain's histograms and search state for the k_sel_* chain)
template <int GQA, bool LL>
__global__ __launch_bounds__(256) void k_value_weights(
    const uint8_t* store, int ub0, int H, int G, int W, int esize, int vscale, int64_t capmax,
    int ntile_ws, const uint32_t* ebuf, const double* tilepart, double* ftile, double* aval,
    const uint8_t* cb, int NU, uint8_t* sel) {
  __shared__ ValueWeightsShared<GQA> sh;
  const int ux = ub0 + (int)blockIdx.x;
  if (sel && blockIdx.y == 0 && ux % NU == 0) {
    const SelDomain D = sel_domain(sel, ux / NU);
    for (int i = threadIdx.x; i < 4096; i += 256) D.hA[i] = 0u;               // hA and hB
    for (int i = threadIdx.x; i < 2 * kSelDigitBins; i += 256) D.hC0[i] = 0u;  // hC0 and hC1
    if (threadIdx.x == 0) {
      SelState z = {};
      z.etop = -1;
      *D.st = z;
    }
  }
  value_weights_block<GQA, LL>(sh, launch_block(), store, ub0, H, G, W, esize, vscale, capmax,
                               ntile_ws, ebuf, tilepart, ftile, aval, cb);
}

template <bool LOCAL, bool LL>
__global__ __launch_bounds__(kVSelNT) void k_value_select(
    const uint8_t* store, int ub0, int G, int W, int esize, float RV, int NU, int min1, int pairs,
    int64_t capmax, const double* aval, uint8_t* tv, const uint8_t* tk, uint64_t* counters,
    const uint8_t* cb) {
  __shared__ ValueSelectShared<kVSelNT> sh;
  extern __shared__ double acache[];  // [tokens] when LOCAL
  value_select_block<kVSelNT, LOCAL, LL>(sh, acache, launch_block(), store, ub0, G, W, esize, RV,
                                         NU, min1, pairs, capmax, aval, tv, tk, counters, cb);
}

// ---------------------------------------------------------------------------
// Value allocation under per-KV-head budgets when the unit's capacity fits
// LDS (up to kVSelLocal tokens): one block per (request, KV head) forms the
// softmax statistics and factors, the weights a_j of every packed token
// straight into LDS (exactly as k_value_weights), then ChooseDepths over
// them (as k_value_select) and the read counters.  Thread t takes tokens
// 4t .. 4t + 3 of each round of 4096; the first round's exponentials are in
// flight while the statistics are formed.
// ---------------------------------------------------------------------------
template <int GQA, bool LL>
__global__ __launch_bounds__(kVSelNT) void k_value_alloc_unit(
    const uint8_t* store, int ub0, int H, int G, int W, int esize, int vscale, float RV, int min1,
    int pairs, int64_t capmax, int ntile_ws, const uint32_t* ebuf, const double* tilepart,
    double* ftile, uint8_t* tv, const uint8_t* tk, uint64_t* counters, const uint8_t* cb) {
  __shared__ ValueAllocUnitShared<kVSelNT, GQA> sh;
  extern __shared__ double acache[];  // [T_p]
  value_alloc_unit_block<kVSelNT, GQA, LL, false>(sh, acache, launch_block(), store, ub0, H, G, W,
                                                  esize, vscale, RV, min1, pairs, capmax, ntile_ws,
                                                  ebuf, tilepart, ftile, tv, tk, counters, cb);
}

// ---------------------------------------------------------------------------
template <int GQA, int DT>
static void key_alloc_gqa(const DecodeArgs& a, const Part& P, uint8_t* tk, hipStream_t st) {
  const int NU = a.G;  // per-layer budgets: one selection per request
  hipLaunchKernelGGL((k_key_alloc<GQA, DT, kMaxPooledKV>), dim3(P.nunits / NU), dim3(256), 0, st,
                     (const uint8_t*)a.store, P.ub0, a.q, a.H, a.G, a.W, a.RK, NU, a.min1, tk);
}

template <int DT>
static int key_alloc_dt(const DecodeArgs& a, const Part& P, uint8_t* tk, hipStream_t st) {
  switch (a.H / a.G) {
    case 1: key_alloc_gqa<1, DT>(a, P, tk, st); return 0;
    case 2: key_alloc_gqa<2, DT>(a, P, tk, st); return 0;
    case 3: key_alloc_gqa<3, DT>(a, P, tk, st); return 0;
    case 4: key_alloc_gqa<4, DT>(a, P, tk, st); return 0;
    case 5: key_alloc_gqa<5, DT>(a, P, tk, st); return 0;
    case 6: key_alloc_gqa<6, DT>(a, P, tk, st); return 0;
    case 7: key_alloc_gqa<7, DT>(a, P, tk, st); return 0;
    case 8: key_alloc_gqa<8, DT>(a, P, tk, st); return 0;
    default: return -5;
  }
}

int launch_key_alloc(const DecodeArgs& a, const Part& P, uint8_t* tk, hipStream_t st) {
  return a.dtype == 0 ? key_alloc_dt<0>(a, P, tk, st) : key_alloc_dt<1>(a, P, tk, st);
}

template <int GQA, int DT>
static void key_alloc_lloyd_gqa(const DecodeArgs& a, const WsLayout& L, uint8_t* tk, hipStream_t st) {
  const int NU = a.scope == 1 ? a.G : 1;
  const int nd = a.B * a.G / NU;
  if (NU > 1)
    hipLaunchKernelGGL((k_key_alloc_lloyd<GQA, DT, kMaxPooledKV>), dim3(nd), dim3(256), 0, st, a.cblock,
                       a.q, a.H, a.G, a.W, a.RK, NU, a.min1, tk, (double*)(a.ws + L.qp),
                       (double*)(a.ws + L.qb), a.counters);
  else
    hipLaunchKernelGGL((k_key_alloc_lloyd<GQA, DT, 1>), dim3(nd), dim3(256), 0, st, a.cblock, a.q,
                       a.H, a.G, a.W, a.RK, NU, a.min1, tk, (double*)(a.ws + L.qp),
                       (double*)(a.ws + L.qb), a.counters);
}

template <int DT>
static int key_alloc_lloyd_dt(const DecodeArgs& a, const WsLayout& L, uint8_t* tk, hipStream_t st) {
  switch (a.H / a.G) {
    case 1: key_alloc_lloyd_gqa<1, DT>(a, L, tk, st); return 0;
    case 2: key_alloc_lloyd_gqa<2, DT>(a, L, tk, st); return 0;
    case 3: key_alloc_lloyd_gqa<3, DT>(a, L, tk, st); return 0;
    case 4: key_alloc_lloyd_gqa<4, DT>(a, L, tk, st); return 0;
    case 5: key_alloc_lloyd_gqa<5, DT>(a, L, tk, st); return 0;
    case 6: key_alloc_lloyd_gqa<6, DT>(a, L, tk, st); return 0;
    case 7: key_alloc_lloyd_gqa<7, DT>(a, L, tk, st); return 0;
    case 8: key_alloc_lloyd_gqa<8, DT>(a, L, tk, st); return 0;
    default: return -5;
  }
}

int launch_key_alloc_lloyd(const DecodeArgs& a, const WsLayout& L, uint8_t* tk, hipStream_t st) {
  return a.dtype == 0 ? key_alloc_lloyd_dt<0>(a, L, tk, st) : key_alloc_lloyd_dt<1>(a, L, tk, st);
}

// per-KV-head budgets and a capacity that fits LDS: one fused launch;
// otherwise value weights (all compute units) then the selection
// ---------------------------------------------------------------------------
// The multi-block selection (msel.h).  Item-parallel launches: block (unit,
// 4096 tokens for the histograms, 1024 for the depths), 256 threads, 4 tokens
// at a time; per-domain launches: one block of 256 decides (k_sel_field,
// k_sel_digit; the last digit's block of 1024 also cuts the ties).
// ---------------------------------------------------------------------------
template <bool LL>
__device__ __forceinline__ void sel_load_gains(double* gt, const uint8_t* cb, int G) {
  if (LL && threadIdx.x < 16)
    gt[threadIdx.x] = reinterpret_cast<const double*>(cb + codec_layout(G, kDim).gains)[threadIdx.x];
}

template <bool LL>
__global__ __launch_bounds__(256) void k_sel_hist(const uint8_t* store, int ub0, int G, int W, int NU,
                                                  float RV, int min1, int pairs, int64_t capmax,
                                                  const double* aval, uint8_t* sel, const uint8_t* cb) {
  __shared__ uint32_t hA[2048], hB[2048];
  __shared__ double gt[16];
  const int tid = threadIdx.x;
  const int ux = ub0 + (int)blockIdx.x;
  const ReqRecord r = req_of(store, ux / G);
  const int64_t Tp = r.len & ~(int64_t)(kGroup - 1);
  const int64_t c0 = (int64_t)blockIdx.y * kSelBlockTokens;
  if (c0 >= Tp) return;  // (the whole block)
  for (int i = tid; i < 2048; i += 256) {
    hA[i] = 0u;
    hB[i] = 0u;
  }
  sel_load_gains<LL>(gt, cb, G);
  __syncthreads();
  const SelParams P = sel_params(Tp, NU, RV, W, min1, pairs, LL);
  ChooseLocal L;  // (the counts come from the histograms in k_sel_field)
  for (int64_t j0 = c0 + 4 * tid; j0 < c0 + kSelBlockTokens; j0 += 1024) {
    const SelItems it = sel_items(aval, capmax, ux, NU, j0, Tp, pairs, P.sc);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q >= it.n) break;
      if constexpr (LL) sel_add_fields(it.a[q], P.Wc, hA, hB, L, TableGains{gt + min1});
      else sel_add_fields(it.a[q], P.Wc, hA, hB, L, Pow4Gains{});
    }
  }
  const SelDomain D = sel_domain(sel, ux / NU);
  __syncthreads();
  for (int i = tid; i < 2048; i += 256) {
    if (hA[i]) atomicAdd(&D.hA[i], hA[i]);
    if (hB[i]) atomicAdd(&D.hB[i], hB[i]);
  }
}

template <bool LL>
__global__ __launch_bounds__(256) void k_sel_field(const uint8_t* store, int ub0, int G, int W, int NU,
                                                   float RV, int min1, int pairs, uint8_t* sel) {
  __shared__ uint32_t out[4];
  __shared__ uint32_t wnp[4], wodd[4];
  __shared__ int wet[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int dom = ub0 / NU + (int)blockIdx.x;
  const ReqRecord r = req_of(store, dom * NU / G);
  const int64_t Tp = r.len & ~(int64_t)(kGroup - 1);
  const SelParams P = sel_params(Tp, NU, RV, W, min1, pairs, LL);
  const SelDomain D = sel_domain(sel, dom);
  // positive gains, top field (+2) and odd gains, from the histograms (a
  // regular item at field f holds Wc gains, the top one at f - 2); thread t
  // reads bins 8t .. 8t + 7 of both with 16-byte loads
  uint32_t np = 0u, odd = 0u;
  int et = -1;
  {
    const uint4* a4 = reinterpret_cast<const uint4*>(D.hA) + 2 * tid;
    const uint4* b4 = reinterpret_cast<const uint4*>(D.hB) + 2 * tid;
    const uint4 av[2] = {a4[0], a4[1]}, ov[2] = {b4[0], b4[1]};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint4& x = av[k >> 2];
      const uint4& y = ov[k >> 2];
      const uint32_t a = (k & 3) == 0 ? x.x : (k & 3) == 1 ? x.y : (k & 3) == 2 ? x.z : x.w;
      const uint32_t o = (k & 3) == 0 ? y.x : (k & 3) == 1 ? y.y : (k & 3) == 2 ? y.z : y.w;
      const int f = 8 * tid + k;
      np += a * (uint32_t)P.Wc + o;
      odd |= o;
      if (a) et = max(et, f);
      if (o) et = max(et, f + 2);
    }
  }
  {
    const uint32_t n = (uint32_t)wave_sum_i32((int)np);
    const int e = wave_max_i32(et);
    const bool o = __ballot(odd != 0u) != 0ull;
    if (lane == 0) {
      wnp[wv] = n;
      wet[wv] = e;
      wodd[wv] = o ? 1u : 0u;
    }
  }
  __syncthreads();
  if (wv != 0) return;
  const uint32_t npos = (wnp[0] + wnp[1]) + (wnp[2] + wnp[3]);
  const int etop = max(max(wet[0], wet[1]), max(wet[2], wet[3]));
  const uint32_t any_odd = (wodd[0] | wodd[1] | wodd[2] | wodd[3]) ? 1u : 0u;
  uint32_t flags = 0u, rem = 0u, n_eq = 0u;
  int Es = 0;
  if (P.bud == 0u || npos <= P.bud) {
    flags = kSelDone;  // nothing, or every positive gain, is taken
  } else {
    if (lane == 0) out[0] = out[1] = out[2] = 0u;
    wave_lds_fence();
    wave_find_gain_field(D.hA, D.hB, P.Wc, etop - 2, P.bud, out);
    wave_lds_fence();
    Es = (int)out[0];
    rem = P.bud - out[1];
    n_eq = out[2];
    if (n_eq == rem) flags = kSelDone;
  }
  if (lane == 0) {
    SelState* s = D.st;
    s->npos = npos;
    s->etop = etop;
    s->any_odd = any_odd;
    s->flags = flags;
    s->Es = Es;
    s->rem = rem;
    s->n_eq = n_eq;
    s->prefix = 0ull;
    s->mask = 0ull;
    s->tie_cut = 0;
  }
}

template <bool LL, int PASS>
__global__ __launch_bounds__(256) void k_sel_radix(const uint8_t* store, int ub0, int G, int W, int NU,
                                                   float RV, int min1, int pairs, int64_t capmax,
                                                   const double* aval, uint8_t* sel, const uint8_t* cb) {
  constexpr int shift = 52 - kSelDigitBits * (PASS + 1);
  constexpr uint32_t dmask = (uint32_t)kSelDigitBins - 1u;
  __shared__ uint32_t hC[kSelDigitBins];
  __shared__ double gt[16];
  const int tid = threadIdx.x;
  const int ux = ub0 + (int)blockIdx.x;
  const SelDomain D = sel_domain(sel, ux / NU);
  const SelState S = *D.st;
  if (S.flags & kSelDone) return;  // (the whole block)
  const ReqRecord r = req_of(store, ux / G);
  const int64_t Tp = r.len & ~(int64_t)(kGroup - 1);
  const int64_t c0 = (int64_t)blockIdx.y * kSelBlockTokens;
  if (c0 >= Tp) return;
  for (int i = tid; i < kSelDigitBins; i += 256) hC[i] = 0u;
  sel_load_gains<LL>(gt, cb, G);
  __syncthreads();
  const SelParams P = sel_params(Tp, NU, RV, W, min1, pairs, LL);
  auto bin = [&](uint64_t mnt) __attribute__((always_inline)) {
    if ((mnt & S.mask) == S.prefix) atomicAdd(&hC[(uint32_t)(mnt >> shift) & dmask], 1u);
  };
  for (int64_t j0 = c0 + 4 * tid; j0 < c0 + kSelBlockTokens; j0 += 1024) {
    const SelItems it = sel_items(aval, capmax, ux, NU, j0, Tp, pairs, P.sc);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q >= it.n) break;
      if constexpr (LL) sel_gains_at(it.a[q], P.Wc, S.Es, S.any_odd != 0u, TableGains{gt + min1}, bin);
      else sel_gains_at(it.a[q], P.Wc, S.Es, S.any_odd != 0u, Pow4Gains{}, bin);
    }
  }
  __syncthreads();
  uint32_t* const g = (PASS & 1) ? D.hC1 : D.hC0;
  for (int i = tid; i <= (int)dmask; i += 256)
    if (hC[i]) atomicAdd(&g[i], hC[i]);
}

// Ranked ties (block of 1024): the items whose gain equals the threshold
// are taken in index order while fewer than rem are; tie_cut = the index
// after the rem-th.
template <bool LL>
__device__ void sel_tie_cut(const uint8_t* store, int G, int W, int NU, float RV, int min1, int pairs,
                            int64_t capmax, const double* aval, const SelDomain& D, const SelState& S,
                            int dom, const double* gt, uint32_t* wsum, int* found) {
  constexpr int NT = 1024;
  const int tid = threadIdx.x;
  const int u0 = dom * NU;
  const ReqRecord r = req_of(store, u0 / G);
  const int64_t Tp = r.len & ~(int64_t)(kGroup - 1);
  const SelParams P = sel_params(Tp, NU, RV, W, min1, pairs, LL);
  uint32_t running = 0;  // ties in earlier rounds
  for (int k = 0; k < NU; ++k) {
    for (int64_t r0 = 0; r0 < Tp; r0 += 4 * NT) {
      const SelItems it = sel_items(aval, capmax, u0 + k, NU, r0 + 4 * tid, Tp, pairs, P.sc);
      uint32_t tie[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q >= it.n) break;
        const uint32_t lv = LL ? sel_levels(it.a[q], P.Wc, S, P.bud, TableGains{gt + min1})
                               : sel_levels(it.a[q], P.Wc, S, P.bud, Pow4Gains{});
        tie[q] = lv >> 16;
      }
      uint32_t c = block_excl_scan<NT>((tie[0] + tie[1]) + (tie[2] + tie[3]), wsum) + running;
      running += wsum[NT / 64];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (tie[q]) {
          if (c + 1u == S.rem) {
            D.st->tie_cut = it.idx[q] + 1;
            *found = 1;
          }
          ++c;
        }
      }
      __syncthreads();
      if (*found) return;
    }
  }
}

// Digit PASS of every domain by one block; the last pass's launch (1024
// threads) then cuts the ties when they are ranked.
template <bool LL, int PASS>
__global__ __launch_bounds__(PASS == kSelPasses - 1 ? 1024 : 256) void k_sel_digit(
    const uint8_t* store, int ub0, int G, int W, int NU, float RV, int min1, int pairs, int64_t capmax,
    const double* aval, uint8_t* sel, const uint8_t* cb) {
  constexpr bool LAST = PASS == kSelPasses - 1;
  constexpr int NT = LAST ? 1024 : 256;
  constexpr int shift = 52 - kSelDigitBits * (PASS + 1);
  constexpr uint32_t dmask = (uint32_t)kSelDigitBins - 1u;
  __shared__ uint32_t out[2];
  __shared__ uint32_t wsum[NT / 64 + 1];
  __shared__ double gt[16];
  __shared__ int found;
  const int dom = ub0 / NU + (int)blockIdx.x;
  const SelDomain D = sel_domain(sel, dom);
  SelState S = *D.st;
  uint32_t* const g = (PASS & 1) ? D.hC1 : D.hC0;
  uint32_t* const gnext = (PASS & 1) ? D.hC0 : D.hC1;
  if (!(S.flags & kSelDone)) {  // (the whole block)
    if (threadIdx.x == 0) out[0] = out[1] = 0u;
    __syncthreads();
    block_find_digit<NT>(g, S.rem, wsum, out);
    const uint32_t dg = min(out[0], dmask);
    S.n_eq = g[dg];
    S.rem -= out[1];
    S.prefix |= (uint64_t)dg << shift;
    S.mask |= (uint64_t)dmask << shift;
    if (S.n_eq == S.rem) S.flags |= kSelDone;
    else if (LAST) S.flags |= kSelDone | kSelRank;  // every bit settled: rank the ties
    if (threadIdx.x == 0) {
      D.st->flags = S.flags;
      D.st->rem = S.rem;
      D.st->n_eq = S.n_eq;
      D.st->prefix = S.prefix;
      D.st->mask = S.mask;
    }
    if constexpr (LAST) {
      if (S.flags & kSelRank) {  // (the whole block)
        sel_load_gains<LL>(gt, cb, G);
        if (threadIdx.x == 0) found = 0;
        __syncthreads();
        sel_tie_cut<LL>(store, G, W, NU, RV, min1, pairs, capmax, aval, D, S, dom, gt, wsum, &found);
      }
    }
  }
  // the next pass's histogram starts from zero (this one's is not touched)
  if (!LAST)
    for (int i = threadIdx.x; i < kSelDigitBins; i += NT) gnext[i] = 0u;
}

template <bool LL>
__global__ __launch_bounds__(256) void k_sel_depths(const uint8_t* store, int ub0, int G, int W, int esize,
                                                    int NU, float RV, int min1, int pairs, int64_t capmax,
                                                    const double* aval, uint8_t* sel, uint8_t* tv,
                                                    const uint8_t* tk, uint64_t* counters,
                                                    const uint8_t* cb) {
  __shared__ uint32_t wsum[256 / 64 + 1];
  __shared__ double gt[16];
  const int tid = threadIdx.x, lane = tid & 63;
  sel_load_gains<LL>(gt, cb, G);
  __syncthreads();
  const int ux = ub0 + (int)blockIdx.x;
  const int b = ux / G;
  const ReqRecord r = req_of(store, b);
  const int64_t len = r.len;
  const int64_t Tp = len & ~(int64_t)(kGroup - 1);
  const SelParams P = sel_params(Tp, NU, RV, W, min1, pairs, LL);
  const SelDomain D = sel_domain(sel, ux / NU);
  const SelState S = *D.st;
  const bool rank = (S.flags & kSelRank) != 0u;
  const SelItems it = sel_items(aval, capmax, ux, NU, (int64_t)blockIdx.y * 1024 + 4 * tid, Tp, pairs, P.sc);
  uint8_t* const tvb = tv + (int64_t)ux * capmax;
  uint32_t mine = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q >= it.n) break;
    const uint32_t lv = LL ? sel_levels(it.a[q], P.Wc, S, P.bud, TableGains{gt + min1})
                           : sel_levels(it.a[q], P.Wc, S, P.bud, Pow4Gains{});
    const uint32_t tie = lv >> 16;
    uint32_t t = (lv & 0xFFFFu) + (rank ? (tie && it.idx[q] < S.tie_cut ? 1u : 0u) : tie) + (uint32_t)min1;
    if (pairs) {
      tvb[it.j0 + 2 * q] = (uint8_t)t;
      tvb[it.j0 + 2 * q + 1] = (uint8_t)t;
      mine += 2 * t;
    } else {
      tvb[it.j0 + q] = (uint8_t)t;
      mine += t;
    }
  }
  if (!counters) return;
  const uint32_t vtot = block_sum_u32<256>(mine, wsum);
  if (tid == 0 && vtot) atomicAdd(reinterpret_cast<unsigned long long*>(counters + 1),
                                  (unsigned long long)vtot * kDim);
  // the domain's other reads, once (as value_select_block)
  if (blockIdx.y == 0 && ux % NU == 0 && tid < 64) {
    int ks = 0;
    for (int i = lane; i < NU * kDim; i += 64) ks += tk[(int64_t)ux * kDim + i];
    ks = wave_sum_i32(ks);
    if (lane == 0) {
      const unsigned long long ng = (unsigned long long)(Tp / kGroup), nu = (unsigned long long)NU;
      atomicAdd(reinterpret_cast<unsigned long long*>(counters), (unsigned long long)ks * (unsigned long long)Tp);
      const unsigned long long meta =
          LL ? lloyd_meta_bits(b == 0, ux == 0, nu) : nu * (2ull * ng * kDim * 32ull + kDim * 64ull + ng * 64ull);
      atomicAdd(reinterpret_cast<unsigned long long*>(counters + 2), meta);
      atomicAdd(reinterpret_cast<unsigned long long*>(counters + 3),
                nu * 2ull * (unsigned long long)(len - Tp) * kDim * (unsigned long long)esize * 8ull);
    }
  }
}

template <bool LL>
static void launch_sel_chain(const DecodeArgs& a, const Part& P, const WsLayout& L, const uint8_t* tk,
                             uint8_t* tv, int NU, hipStream_t st) {
  const int nch = (int)((a.capmax + kVChunk - 1) / kVChunk);
  const int ndom = P.nunits / NU;
  uint8_t* const sel = a.ws + L.sel;
  const double* const aval = (const double*)(a.ws + L.aval);
  const uint8_t* const store = (const uint8_t*)a.store;
  const dim3 gi(P.nunits, nch);
  const dim3 gh(P.nunits, (unsigned)((a.capmax + kSelBlockTokens - 1) / kSelBlockTokens));
  hipLaunchKernelGGL((k_sel_hist<LL>), gh, dim3(256), 0, st, store, P.ub0, a.G, a.W, NU, a.RV, a.min1,
                     a.pairs, a.capmax, aval, sel, a.cblock);
  hipLaunchKernelGGL((k_sel_field<LL>), dim3(ndom), dim3(256), 0, st, store, P.ub0, a.G, a.W, NU, a.RV,
                     a.min1, a.pairs, sel);
#define READKV_SEL_PASS(p)                                                                              \
  hipLaunchKernelGGL((k_sel_radix<LL, p>), gh, dim3(256), 0, st, store, P.ub0, a.G, a.W, NU, a.RV, a.min1, \
                     a.pairs, a.capmax, aval, sel, a.cblock);                                            \
  hipLaunchKernelGGL((k_sel_digit<LL, p>), dim3(ndom), dim3(p == kSelPasses - 1 ? 1024 : 256), 0, st, store, \
                     P.ub0, a.G, a.W, NU, a.RV, a.min1, a.pairs, a.capmax, aval, sel, a.cblock);
  static_assert(kSelPasses == 4, "one launch pair per digit below");
  READKV_SEL_PASS(0)
  READKV_SEL_PASS(1)
  READKV_SEL_PASS(2)
  READKV_SEL_PASS(3)
#undef READKV_SEL_PASS
  hipLaunchKernelGGL((k_sel_depths<LL>), gi, dim3(256), 0, st, store, P.ub0, a.G, a.W, a.dtype == 0 ? 2 : 4,
                     NU, a.RV, a.min1, a.pairs, a.capmax, aval, sel, tv, tk, a.counters, a.cblock);
}

template <int GQA, bool LL>
static bool value_first_gqa(const DecodeArgs& a, const Part& P, const WsLayout& L, const uint8_t* tk,
                            uint8_t* tv, hipStream_t st) {
  if (a.scope == 0 && a.capmax <= kVSelLocal) {
    static bool attr_set = false;
    if (!attr_set) {
      hipFuncSetAttribute(reinterpret_cast<const void*>(&k_value_alloc_unit<GQA, LL>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kVSelLocal * 8);
      attr_set = true;
    }
    hipLaunchKernelGGL((k_value_alloc_unit<GQA, LL>), dim3(P.nunits), dim3(kVSelNT), (size_t)a.capmax * 8,
                       st, (const uint8_t*)a.store, P.ub0, a.H, a.G, a.W, a.dtype == 0 ? 2 : 4, a.vscale, a.RV,
                       a.min1, a.pairs, a.capmax, L.ntile, (const uint32_t*)(a.ws + L.ebuf),
                       (const double*)(a.ws + L.tilepart), (double*)(a.ws + L.ftile), tv, tk,
                       a.counters, a.cblock);
    return true;
  }
  const int nch = (int)((a.capmax + kVChunk - 1) / kVChunk);
  const int NU = a.scope == 1 ? a.G : 1;
  const bool chain = (int64_t)NU * a.capmax > kVSelLocal;  // the multi-block selection follows
  hipLaunchKernelGGL((k_value_weights<GQA, LL>), dim3(P.nunits, nch), dim3(256), 0, st,
                     (const uint8_t*)a.store, P.ub0, a.H, a.G, a.W, a.dtype == 0 ? 2 : 4, a.vscale, a.capmax,
                     L.ntile, (const uint32_t*)(a.ws + L.ebuf), (const double*)(a.ws + L.tilepart),
                     (double*)(a.ws + L.ftile), (double*)(a.ws + L.aval), a.cblock, NU,
                     chain ? a.ws + L.sel : nullptr);
  return false;
}

template <bool LL>
static int launch_value_alloc_t(const DecodeArgs& a, const Part& P, const WsLayout& L, const uint8_t* tk,
                                uint8_t* tv, hipStream_t st) {
  bool done;
  switch (a.H / a.G) {
    case 1: done = value_first_gqa<1, LL>(a, P, L, tk, tv, st); break;
    case 2: done = value_first_gqa<2, LL>(a, P, L, tk, tv, st); break;
    case 3: done = value_first_gqa<3, LL>(a, P, L, tk, tv, st); break;
    case 4: done = value_first_gqa<4, LL>(a, P, L, tk, tv, st); break;
    case 5: done = value_first_gqa<5, LL>(a, P, L, tk, tv, st); break;
    case 6: done = value_first_gqa<6, LL>(a, P, L, tk, tv, st); break;
    case 7: done = value_first_gqa<7, LL>(a, P, L, tk, tv, st); break;
    case 8: done = value_first_gqa<8, LL>(a, P, L, tk, tv, st); break;
    default: return -5;
  }
  if (done) return 0;
  const int NU = a.scope == 1 ? a.G : 1;
  const int64_t nmax = (int64_t)NU * a.capmax;  // items of a domain, at most
  const bool local = nmax <= kVSelLocal;
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(&k_value_select<true, LL>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, kVSelLocal * 8);
    attr_set = true;
  }
  if (!local) {
    launch_sel_chain<LL>(a, P, L, tk, tv, NU, st);
    return 0;
  }
  auto* const ksel = &k_value_select<true, LL>;
  hipLaunchKernelGGL(ksel, dim3(P.nunits / NU),
                     dim3(kVSelNT), (size_t)nmax * 8, st,
                     (const uint8_t*)a.store, P.ub0, a.G, a.W, a.dtype == 0 ? 2 : 4, a.RV, NU, a.min1,
                     a.pairs, a.capmax,
                     (const double*)(a.ws + L.aval), tv, tk, a.counters, a.cblock);
  return 0;
}

int launch_value_alloc(const DecodeArgs& a, const Part& P, const WsLayout& L, const uint8_t* tk,
                       uint8_t* tv, hipStream_t st) {
  return a.codec ? launch_value_alloc_t<true>(a, P, L, tk, tv, st)
                 : launch_value_alloc_t<false>(a, P, L, tk, tv, st);
}

}  // namespace readkv
