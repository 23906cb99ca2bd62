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
//   k_value_select  (one block per selection domain)
//                   ChooseDepths over the domain's packed tokens -> t^V, and
//                   the call's logical-read counters
//
// (The block code of the last two is in valloc.h, which the single-launch
// reader shares.)  A selection domain is one (request, KV head) under
// per-KV-head budgets, or one request (its G KV heads pooled, item index =
// KV head * N + item) under per-layer budgets.
#include <math.h>

#include "kernels_common.h"
#include "readkv_internal.h"
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

template <int GQA, bool LL>
__global__ __launch_bounds__(256) void k_value_weights(
    const uint8_t* store, int ub0, int H, int G, int W, int esize, int vscale, int64_t capmax,
    int ntile_ws, const uint32_t* ebuf, const double* tilepart, double* ftile, double* aval,
    const uint8_t* cb) {
  __shared__ ValueWeightsShared<GQA> sh;
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
  hipLaunchKernelGGL((k_value_weights<GQA, LL>), dim3(P.nunits, nch), dim3(256), 0, st,
                     (const uint8_t*)a.store, P.ub0, a.H, a.G, a.W, a.dtype == 0 ? 2 : 4, a.vscale, a.capmax,
                     L.ntile, (const uint32_t*)(a.ws + L.ebuf), (const double*)(a.ws + L.tilepart),
                     (double*)(a.ws + L.ftile), (double*)(a.ws + L.aval), a.cblock);
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
  auto* const ksel = local ? &k_value_select<true, LL> : &k_value_select<false, LL>;
  hipLaunchKernelGGL(ksel, dim3(P.nunits / NU),
                     dim3(kVSelNT), local ? (size_t)nmax * 8 : 0, st,
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
