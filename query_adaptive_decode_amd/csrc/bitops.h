// Scalar helpers used by the kernels, written so they also compile for the
// host (unit-tested there on the CPU).
#pragma once
#include <stdint.h>
#include <string.h>

#ifdef __HIPCC__
#define RKV_HDI __host__ __device__ __forceinline__
#else
#define RKV_HDI inline
#endif

namespace readkv {

RKV_HDI uint64_t dbits(double v) {
  uint64_t u;
  memcpy(&u, &v, 8);
  return u;
}
RKV_HDI double bitsd(uint64_t u) {
  double v;
  memcpy(&v, &u, 8);
  return v;
}
RKV_HDI float bf16_to_float(uint32_t b) {
  uint32_t u = b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// Round a finite double to bfloat16 (8 significant bits) toward +inf (up)
// or -inf (!up); returns the bf16 bit pattern.  Magnitudes past the bf16
// range give +-inf (0x7F80 / 0xFF80).  Zero results are +0.
RKV_HDI uint32_t bf16_round_dir(double v, bool up) {
  const uint64_t u = dbits(v);
  const uint32_t sign = (uint32_t)(u >> 63);
  const uint64_t mag = u & 0x7FFFFFFFFFFFFFFFull;
  if (mag == 0) return 0u;
  // rounding the magnitude away from zero when the direction and the sign
  // agree (up for positives, down for negatives), else toward zero
  const bool away = (up && !sign) || (!up && sign);
  const int e = (int)(mag >> 52);           // biased double exponent (>= 1 here for normals)
  uint32_t bmag;                            // bf16 magnitude bits
  if (e >= 1023 - 126) {
    // normal bf16 range: keep 7 mantissa bits
    const int be = e - 1023 + 127;          // bf16 biased exponent
    const uint64_t m = mag & 0x000FFFFFFFFFFFFFull;
    uint32_t keep = (uint32_t)(m >> 45);    // top 7 mantissa bits
    const bool rest = (m & ((1ull << 45) - 1)) != 0;
    if (be >= 255) return sign ? 0xFF80u : 0x7F80u;
    bmag = ((uint32_t)be << 7) | keep;
    if (rest && away) bmag += 1;            // carry into the exponent is correct
    if (bmag >= 0x7F80u) bmag = 0x7F80u;
  } else {
    // below 2^-126: bf16 subnormal grid of spacing 2^-133
    const double s = bitsd(mag) * 0x1p133;  // exact scaling (result >= 2^-941)
    double k = (double)(uint64_t)s;         // floor for positives
    if (k != s && away) k += 1.0;
    bmag = (uint32_t)k;                     // <= 128 (128 == smallest normal)
    if (bmag == 0) return 0u;
  }
  return (sign << 15) | bmag;
}

// 8x8 bit-matrix transpose of x, where bit (8r + c) is element (r, c):
// the result has bit (8c + r) = element (r, c).
RKV_HDI uint64_t transpose8(uint64_t x) {
  uint64_t t;
  t = (x ^ (x >> 7)) & 0x00AA00AA00AA00AAull;
  x = x ^ t ^ (t << 7);
  t = (x ^ (x >> 14)) & 0x0000CCCC0000CCCCull;
  x = x ^ t ^ (t << 14);
  t = (x ^ (x >> 28)) & 0x00000000F0F0F0F0ull;
  x = x ^ t ^ (t << 28);
  return x;
}

// transpose8 on the two 32-bit halves of x (lo = bits 0..31, hi = 32..63),
// the form the kernels use: the first two exchange stages stay inside each
// half, the last one crosses them through a 64-bit funnel shift.
RKV_HDI void transpose8_halves(uint32_t& lo, uint32_t& hi) {
  uint32_t t;
  t = (lo ^ (lo >> 7)) & 0x00AA00AAu;
  lo ^= t ^ (t << 7);
  t = (hi ^ (hi >> 7)) & 0x00AA00AAu;
  hi ^= t ^ (t << 7);
  t = (lo ^ (lo >> 14)) & 0x0000CCCCu;
  lo ^= t ^ (t << 14);
  t = (hi ^ (hi >> 14)) & 0x0000CCCCu;
  hi ^= t ^ (t << 14);
  const uint32_t fun = (uint32_t)(((((uint64_t)hi) << 32) | lo) >> 28);
  t = (lo ^ fun) & 0xF0F0F0F0u;
  lo ^= t;
  hi ^= t >> 4;
}

// Byte permute with the semantics of the gfx950 v_perm_b32 instruction:
// byte i of the result is byte sel_i of the 8-byte value {a (bytes 4..7),
// b (bytes 0..3)}; selector 0x0C gives 0x00.  (Host model for tests; the
// kernels call the instruction.)
RKV_HDI uint32_t perm_bytes(uint32_t a, uint32_t b, uint32_t sel) {
  const uint64_t v = ((uint64_t)a << 32) | b;
  uint32_t r = 0;
  for (int i = 0; i < 4; ++i) {
    const uint32_t s = (sel >> (8 * i)) & 0xFFu;
    uint32_t byte = 0;
    if (s < 8) byte = (uint32_t)(v >> (8 * s)) & 0xFFu;
    else if (s == 0x0C) byte = 0;
    else if (s >= 0x0D) byte = 0xFF;
    r |= byte << (8 * i);
  }
  return r;
}

// Un-plane: `planes` holds plane p (bit i = element i) in byte 7-p.  The
// result's byte i is element i's code prefix with plane p at bit 7-p
// (missing planes are zero), i.e. X = P * 2^(8-t) for a depth-t prefix P.
RKV_HDI uint64_t unplane8(uint64_t planes_rev) { return transpose8(planes_rev); }

}  // namespace readkv
