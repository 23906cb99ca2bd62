// The pages' own codec ("Read What Matters: Query-Adaptive Quantization for
// KV Caches", Sec. 3.1 and App. D.1): a binary tree fitted to Z ~ N(0, 1),
// each node's interval cut where the boundary equals the average of the two
// children's conditional means (the Lloyd condition), behind a
// Hadamard-sign transform with per-channel calibration.
//
// Host: the depth-8 tree in float64, rounded to the float32 table the
// decoder reads (centroids, the eight gains Delta_t = D(t-1) - D(t)), and
// the encoder's boundaries (midpoints of the float32 child centroids, exact
// in float64).  Built on the positive half line and mirrored: the density is
// even, so the table is exactly symmetric.
//
// Device: calibration of a Lloyd-tree store from a held-out split (App.
// D.1): per KV head and transformed channel, the mean and root-mean-square
// deviation, summed in token order in float64 and rounded to float32; a
// zero or non-finite scale becomes 1.
#include <math.h>
#include <string.h>

#include <vector>

#include "kernels_common.h"
#include "readkv_internal.h"

// every operation below rounds on its own (no fused multiply-adds), as
// written
#pragma clang fp contract(off)

namespace readkv {

namespace {

double npdf(double x) { return isinf(x) ? 0.0 : exp(-0.5 * x * x) / sqrt(2.0 * M_PI); }
// P(Z > x)
double upper(double x) { return 0.5 * erfc(x / sqrt(2.0)); }
// P(a < Z < b) and E[Z | a < Z < b] for 0 <= a < b <= inf
double cell_mass(double a, double b) { return upper(a) - upper(b); }
double cell_mean(double a, double b) { return (npdf(a) - npdf(b)) / cell_mass(a, b); }

// the x in (a, b) where x equals the mean of the two children's centroids
// (x minus that mean is negative near a and positive near b): bisection to
// the last bit
double lloyd_split(double a, double b) {
  double lo = a, hi = isinf(b) ? cell_mean(a, b) + 40.0 : b;
  for (int it = 0; it < 400; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    const double f = mid - 0.5 * (cell_mean(a, mid) + cell_mean(mid, b));
    if (f < 0.0) lo = mid;
    else hi = mid;
  }
  return 0.5 * (lo + hi);
}

TreeTables build_tables() {
  TreeTables T;
  memset(&T, 0, sizeof(T));
  // edges of the positive half at depths 1..8: level t has 2^(t-1) cells
  std::vector<std::vector<double>> half(kTreeDepth + 1);
  half[1] = {0.0, INFINITY};
  for (int t = 2; t <= kTreeDepth; ++t) {
    const std::vector<double>& e = half[t - 1];
    std::vector<double> n{e[0]};
    for (size_t i = 0; i + 1 < e.size(); ++i) {
      n.push_back(lloyd_split(e[i], e[i + 1]));
      n.push_back(e[i + 1]);
    }
    half[t] = n;
  }
  double energy_prev = 0.0;  // sum over cells of P(cell) c^2 (whole line)
  for (int t = 1; t <= kTreeDepth; ++t) {
    const std::vector<double>& e = half[t];
    const int nh = (int)e.size() - 1;  // cells of the positive half
    double energy = 0.0;
    for (int i = 0; i < nh; ++i) {
      const double c = cell_mean(e[i], e[i + 1]);
      energy += cell_mass(e[i], e[i + 1]) * (c * c);
      const float c32 = (float)c;
      T.cent[(1 << t) - 1 + nh + i] = c32;       // upper half, left to right
      T.cent[(1 << t) - 1 + nh - 1 - i] = -c32;  // its mirror image
    }
    energy *= 2.0;
    T.gains[t] = (double)(float)(energy - energy_prev);
    energy_prev = energy;
  }
  for (int t = 0; t < kTreeDepth; ++t)
    for (int P = 0; P < (1 << t); ++P) {
      const int ch = (1 << (t + 1)) - 1 + 2 * P;
      T.bounds[(1 << t) - 1 + P] = ((double)T.cent[ch] + (double)T.cent[ch + 1]) / 2.0;
    }
  return T;
}

// mean and root-mean-square deviation of one (KV head, side) over the
// calibration tokens: block (g, side), thread c = transformed channel.
template <int DT>
__global__ __launch_bounds__(128) void k_calibrate(uint8_t* cb, int G, const void* kcal,
                                                   const void* vcal, int64_t n) {
  const CodecLayout C = codec_layout(G, kDim);
  const int g = blockIdx.x, side = blockIdx.y, c = threadIdx.x;
  const void* src = side ? vcal : kcal;
  const double sg = reinterpret_cast<const double*>(cb + (side ? C.sv : C.sk))[c];
  __shared__ double buf[kDim];
  __shared__ float sigs[kDim];
  // channel c of U x_j = H (s . x_j) / sqrt(d): the in-place Walsh-Hadamard
  // butterflies (Sylvester order) over the block
  auto xform = [&](int64_t j) -> double {
    buf[c] = load_elem<DT>(src, (j * G + g) * kDim + c) * sg;
    __syncthreads();
    for (int h = 1; h < kDim; h <<= 1) {
      const double a = buf[c], o = buf[c ^ h];
      __syncthreads();
      buf[c] = (c & h) ? o - a : a + o;
      __syncthreads();
    }
    const double r = __dmul_rn(buf[c], kInvSqrt128);
    __syncthreads();
    return r;
  };
  double s = 0.0;
  for (int64_t j = 0; j < n; ++j) s = __dadd_rn(s, xform(j));
  const double mu = s / (double)n;
  double s2 = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    const double dv = __dsub_rn(xform(j), mu);
    s2 = __dadd_rn(s2, __dmul_rn(dv, dv));
  }
  double sd = sqrt(s2 / (double)n);
  if (!(isfinite(sd) && sd > 0.0)) sd = 1.0;
  const float mu32 = (float)mu, sd32 = (float)sd;
  reinterpret_cast<float*>(cb + (side ? C.muv : C.muk))[g * kDim + c] = mu32;
  reinterpret_cast<float*>(cb + (side ? C.sigv : C.sigk))[g * kDim + c] = sd32;
  if (side == 1) {
    sigs[c] = sd32;
    __syncthreads();
    if (c == 0) {
      double e = 0.0;
      for (int k = 0; k < kDim; ++k) e = __dadd_rn(e, __dmul_rn((double)sigs[k], (double)sigs[k]));
      reinterpret_cast<double*>(cb + C.sphys)[g] = e;
    }
  }
}

}  // namespace

const TreeTables& lloyd_tables() {
  static const TreeTables T = build_tables();
  return T;
}

void codec_block_image(int G, uint8_t* img) {
  const CodecLayout C = codec_layout(G, kDim);
  memset(img, 0, (size_t)C.size);
  const TreeTables& T = lloyd_tables();
  memcpy(img + C.cent, T.cent, sizeof(T.cent));
  memcpy(img + C.bounds, T.bounds, sizeof(T.bounds));
  memcpy(img + C.gains, T.gains, sizeof(T.gains));
  double* sk = reinterpret_cast<double*>(img + C.sk);
  double* sv = reinterpret_cast<double*>(img + C.sv);
  for (int c = 0; c < kDim; ++c) sk[c] = sv[c] = 1.0;
  _Float16* vt = reinterpret_cast<_Float16*>(img + C.vtab);
  for (int t = 0; t <= kTreeDepth; ++t)
    for (int X = 0; X < 256; ++X) vt[t * 256 + X] = (_Float16)T.cent[(1 << t) - 1 + (X >> (8 - t))];
  float* mk = reinterpret_cast<float*>(img + C.muk);
  float* sgk = reinterpret_cast<float*>(img + C.sigk);
  float* mv = reinterpret_cast<float*>(img + C.muv);
  float* sgv = reinterpret_cast<float*>(img + C.sigv);
  double* sp = reinterpret_cast<double*>(img + C.sphys);
  for (int i = 0; i < G * kDim; ++i) {
    mk[i] = mv[i] = 0.f;
    sgk[i] = sgv[i] = 1.f;
  }
  for (int g = 0; g < G; ++g) sp[g] = (double)kDim;
}

int launch_calibrate(uint8_t* cblock, int G, int dtype, const void* kcal, const void* vcal,
                     int64_t ncal, hipStream_t st) {
  if (dtype == 0)
    hipLaunchKernelGGL(k_calibrate<0>, dim3(G, 2), dim3(kDim), 0, st, cblock, G, kcal, vcal, ncal);
  else
    hipLaunchKernelGGL(k_calibrate<1>, dim3(G, 2), dim3(kDim), 0, st, cblock, G, kcal, vcal, ncal);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace readkv
