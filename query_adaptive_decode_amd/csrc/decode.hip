// One ReadKV decode step ("Read What Matters: Query-Adaptive Quantization
// for KV Caches", Sec. 3.2-3.3, Algorithm 1) as five launches on one stream
// (six under per-layer budgets):
//
//   k_key_alloc      (requests)           per-layer budgets only: key
//                                         weights (Eq. (2)) and ChooseDepths
//                                         over a request's G*d_h channels
//                                         -> t^K (alloc.hip)
//   k_score          (B*G x runs)         per-KV-head budgets: key weights and
//                                         ChooseDepths over the unit's d_h
//                                         channels (block prologue); then the
//                                         prefix-gather of the chosen key
//                                         planes through LDS, reconstructed
//                                         logits in fp64, per-tile max and
//                                         sum of exp (split-context softmax)
//   k_value_weights  (B*G x chunks)       softmax statistics and value
//                                         weights (Eq. (3)) (alloc.hip)
//   k_value_select   (domains)            ChooseDepths over the packed
//                                         tokens -> t^V (alloc.hip)
//   k_gather         (B*G x runs)         prefix-gather of the chosen value
//                                         planes, attention-weighted sums per
//                                         run of chunks
//   k_out_reduce     (B*H*d threads)      run partials summed in run order
//
// The value selection -> gather boundary is the staged(2) reader's second
// batch: value reads depend on attention computed from the first batch.
// Each kernel is a thin launch around a block function (its LDS struct and
// a block index as arguments), so that k_reader_fused can run the same block
// code as one cooperative launch with grid barriers between the stages.
//
// Reconstruction of a depth-t prefix P (t MSB-first planes) of a group with
// metadata (lo, rng): x_hat = lo + rng (2P + 1) / 2^(t+1).  The kernels
// un-plane an 8-element bit column into X = P 2^(8-t) (missing planes read
// as zero) and use x_hat = lo + rng 2^-(t+1) + rng X / 256.
#include <hip/hip_cooperative_groups.h>
#include <math.h>

#include <algorithm>

#include "kernels_common.h"
#include "readkv_internal.h"
#include "select.h"
#include "valloc.h"

namespace readkv {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr double kInvSqrtD = kInvSqrt128;

// ---------------------------------------------------------------------------
// Key allocation.  ChooseDepths for one unit's d_h = 128 key channels by one
// wave: lane l holds channels l and l + 64 with weights wv[0], wv[1]; the W
// candidate gains of a channel are w_c 4^-t, t = 1..W, and the B_K largest
// positive ones are chosen, ties to the lowest channel (with strictly
// decreasing per-item gains this is ChooseDepths' result, [ReadKV] App.
// E.2.1).  Returns the depths of the lane's two channels.  cc: LDS scratch of
// 258 words.  Wave-level only (no block barrier).
//
// Every positive weight has a normal exponent field E_c in [2W + 1, 2046]:
// with finite bf16 or fp32 queries (|q| in [2^-149, 2^128)) and ranges (bf16,
// in [2^-133, 2^128), at most 2^21 groups), w_c = (sum of at most 8 q^2)
// E^K_c lies in [2^-564, 2^537).  A non-finite query never reaches this
// function (its unit's weights are zero).  So each gain w_c 4^-(t+1) is exact,
// with field E_c - 2t - 2 and the mantissa M_c of w_c.  Gains order by that
// field first; the B_K-th largest lies at the highest field level L with
//   count(L) = sum_c #{t < W : E_c - 2t - 2 >= L} >= B_K,
// and at that level each channel has at most one candidate, ranked by (M_c
// descending, c ascending).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void key_depths_wave(const double (&wv)[2], int W, uint32_t Bk,
    uint32_t* cc, uint32_t (&sel)[2]) {
  const int lane = __lane_id();
  sel[0] = 0u;
  sel[1] = 0u;
  int ec[2];
  uint64_t mc[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint64_t wb = dbits(wv[k]);
    ec[k] = wv[k] > 0.0 ? (int)(wb >> 52) : -1;  // no candidate unless w_c > 0
    mc[k] = wb & 0x000FFFFFFFFFFFFFull;
  }
  auto cnt_ge = [&](int k, int lvl) -> int {  // #{t < W : E - 2t - 2 >= lvl} for slot k
    if (ec[k] < 0) return 0;
    const int d = ec[k] - 2 - lvl;
    return d < 0 ? 0 : min(d / 2 + 1, W);
  };
  const uint32_t nposf = (uint32_t)W * (uint32_t)(__popcll(__ballot(ec[0] >= 0)) +
                                                  __popcll(__ballot(ec[1] >= 0)));
  if (nposf <= Bk) {
    sel[0] = ec[0] >= 0 ? (uint32_t)W : 0u;
    sel[1] = ec[1] >= 0 ? (uint32_t)W : 0u;
    return;
  }
  if (Bk == 0) return;
  const int emax = wave_max_i32(max(ec[0], ec[1]));
  // Lane l evaluates count(L) at level L = emax - 2 - l: with n_i the
  // number of channels with E_c = emax - i and S_i = n_0 + ... + n_i,
  //   count(L) = sum_{k=1..W} #{c : E_c >= L + 2k} = sum_k S_{l + 2 - 2k}
  // (S of a negative index is 0; a channel with E_c < emax - 63 has no
  // candidate at these levels).  The highest such level with count >= B_K
  // is the first lane's; when it lies below them all, a bisection over
  // [min E - 2W, max E - 2] finds it.
  uint32_t* const hE = cc;       // n_i, i < 64
  uint32_t* const hS = cc + 64;  // S_i at hS[16 + i], zeros below
  hE[lane] = 0u;
  if (lane < 16) hS[lane] = 0u;
  wave_lds_fence();
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (ec[k] >= 0 && emax - ec[k] < 64) atomicAdd(&hE[emax - ec[k]], 1u);
  wave_lds_fence();
  hS[16 + lane] = wave_incl_scan_u32(hE[lane]);
  wave_lds_fence();
  uint32_t cntl = 0;
#pragma unroll
  for (int k = 1; k <= 8; ++k)
    if (k <= W) cntl += hS[16 + lane + 2 - 2 * k];
  const uint64_t okb = __ballot(cntl >= Bk);
  int Ls;
  uint32_t above;
  if (okb) {
    const int ls = __ffsll((unsigned long long)okb) - 1;
    Ls = emax - 2 - ls;
    above = ls > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)cntl, ls - 1) : 0u;
  } else {
    const int lo0 = min(ec[0] >= 0 ? ec[0] : 4096, ec[1] >= 0 ? ec[1] : 4096);
    const int emin = -wave_max_i32(-lo0);  // some channel is positive here
    int lo_l = max(1, emin - 2 * W), hi_l = emax - 2;
    while (lo_l < hi_l) {
      const int mid = (lo_l + hi_l + 1) >> 1;
      if ((uint32_t)wave_sum_i32(cnt_ge(0, mid) + cnt_ge(1, mid)) >= Bk) lo_l = mid;
      else hi_l = mid - 1;
    }
    Ls = lo_l;
    above = (uint32_t)wave_sum_i32(cnt_ge(0, Ls + 1) + cnt_ge(1, Ls + 1));
  }
  const uint32_t rem = Bk - above;  // >= 1
  bool at[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    sel[k] = (uint32_t)cnt_ge(k, Ls + 1);
    const int d = ec[k] - 2 - Ls;
    at[k] = ec[k] >= 0 && d >= 0 && (d & 1) == 0 && d / 2 < W;
  }
  // the rem largest at the level by (M_c descending, c ascending): an
  // MSB-first search over the 52 mantissa bits (wave ballots) that stops
  // as soon as the candidates still equal to the threshold on the decided
  // bits are exactly the ones left to take
  uint64_t pre = 0ull, hm = 0ull;  // threshold bits decided so far, their mask
  uint32_t rm = rem;
  bool early = false;
  {
    // the top 8 mantissa bits in one step: a 256-bin histogram of the
    // candidates' top digits, scanned from the top (splitting further
    // never changes which candidates end up taken)
    uint32_t* const hD = cc;
    *reinterpret_cast<uint4*>(hD + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
    wave_lds_fence();
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if (at[k]) atomicAdd(&hD[(uint32_t)(mc[k] >> 44)], 1u);
    wave_lds_fence();
    wave_find_digit<256>(hD, rm, cc + 256, cc + 257);
    wave_lds_fence();
    pre = (uint64_t)cc[256] << 44;
    hm = 0xFFull << 44;
    rm -= cc[257];
  }
  for (int bit = 43; bit >= 0; --bit) {
    const bool a0 = at[0] && ((mc[0] ^ pre) & hm) == 0ull;
    const bool a1 = at[1] && ((mc[1] ^ pre) & hm) == 0ull;
    if ((uint32_t)(__popcll(__ballot(a0)) + __popcll(__ballot(a1))) == rm) {
      early = true;
      break;
    }
    const uint64_t bm = 1ull << bit;
    const uint32_t c1 = (uint32_t)(__popcll(__ballot(a0 && (mc[0] & bm))) +
                                   __popcll(__ballot(a1 && (mc[1] & bm))));
    if (c1 >= rm) pre |= bm;
    else rm -= c1;
    hm |= bm;
  }
  // above the threshold on the decided bits: taken; equal to it: all of
  // them after an early stop, else (equal mantissas) the first rm in
  // channel order
  bool eq[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint64_t hv = mc[k] & hm;
    eq[k] = at[k] && hv == pre;
    if (at[k] && hv > pre) ++sel[k];
  }
  if (early) {
    sel[0] += eq[0];
    sel[1] += eq[1];
  } else {
    const uint64_t b0 = __ballot(eq[0]), b1 = __ballot(eq[1]);
    const uint64_t below = (1ull << lane) - 1ull;
    if (eq[0] && (uint32_t)__popcll(b0 & below) < rm) ++sel[0];
    if (eq[1] && (uint32_t)(__popcll(b0) + __popcll(b1 & below)) < rm) ++sel[1];
  }
}

// ---------------------------------------------------------------------------
// Score: a block of 256 threads takes every ny-th 256-token tile (8 groups;
// half of a 512-token key-plane tile) of one (request, KV head), ny = the
// unit's block count, starting at its own index.  The logit of token j and
// query head h is
//   s_hj = (C_gh + sum_c beta_hc X'_jc) / sqrt(d),
//   beta_hc = q_hc rng_gc / 256,  X' = X - 128 (X = P 2^(8-t), the prefix
//   code in the top bits of a byte),
//   C_gh = sum_c q_hc (lo_gc + rng_gc 2^-(t_c+1) + [t_c > 0] rng_gc / 2)
// (the reconstruction x_hat = lo + rng 2^-(t+1) + rng X / 256 with the -128
// offset folded into C; channels with t_c = 0 contribute only to C).
// The sum over channels is an exact integer matrix product on the int8
// matrix cores: with a per-head power of two 2^sig_h (so that every
// |q_hc rng_gc| 2^sig_h < 2^46), the integer N_hc = rint(q_hc rng_gc 2^sig_h)
// is split into six signed 8-bit digits, and
//   sum_c beta_hc X'_jc = 2^(-sig_h - 8) sum_k 2^(8k) sum_c digit_k(N_hc) X'_jc
// with every inner sum exact in int32.  One fp64 FMA produces the digits:
// q 2^sig * rng + (2^52 + 0x808080808080) rounds q rng 2^sig to an integer
// N and leaves N + 0x808080808080 in the low 48 mantissa bits, whose byte k
// is digit_k + 128 (flipping bit 7 gives the two's-complement digit).
// The rounding error of N is below 2^-46 of the per-head bound, far below
// the float64 rounding of the reconstructed logits it replaces.
//
// Once per block: depths, query, per-head scales, the slot table.  Per tile:
//  1. The tile's segment of every chosen key line (channel c, plane p < t_c;
//     8 words = 32 B, one per group) sits in LDS as planes[slot][group],
//     slot = (sum of t over channels below c) + p.  The next tile's segments
//     and metadata are in flight to registers while this tile is computed;
//     they are written to LDS after its last un-plane, and the loads for the
//     tile after are issued at once (the first tile's go out as soon as the
//     slot table is known).  Barriers inside the tile loop wait for LDS
//     traffic only, never for those loads.
//  2. Per-group constants C_gh: a 16 x 128 x GQA fp64 contraction on the
//     matrix cores (v_mfma_f64_16x16x4_f64).
//  3. Four slabs of 32 channels.  Un-plane: wave w takes the slab's channels
//     w, w+4, ... in pairs (channels sorted by depth, deepest first; depths
//     from a scalar table), lane o of a half-wave the tile's tokens
//     8o..8o+7: one transposing LDS read gives their 8 plane bytes, an 8x8
//     bit transpose the 8 codes (the top plane inverted first, which makes
//     them X'), stored as a code tile [channel][token].
//     MFMA: wave w takes groups 2w and 2w+1; per group it writes the digit
//     words of its 32 channels x GQA heads, then v_mfma_i32_16x16x32_i8 with
//     A = digits and B = codes (16 tokens x 32 channels), both read with the
//     transposing ds_read_b64_tr_b8, accumulating over the slabs.  An A chunk
//     holds digits 4m..4m+3 of two heads, so the 16 rows of one MFMA are
//     (4 heads) x (4 digits) and lane l of the result holds all its digits of
//     head l/16 for token l%16: the digit sums are combined in-lane.
//  4. Digit sums -> logits (fp64) in registers; open-group tokens use exact
//     keys; per head the tile max m, e = exp(s - m) (fp64; stored as bits
//     61..30 of its fp64 pattern, read by the value allocation and the value
//     gather) and sum e (split-context softmax).
// Grid (unit, ny): consecutive blocks are different units, so all blocks of
// a unit are on one XCD and share its L2; as they take neighbouring tiles at
// the same time, the two halves of a key-plane tile are read from HBM once.
// Dynamic LDS: 32 B per staged slot (at most min(B_K, 128 W) slots).
// ---------------------------------------------------------------------------
// transpose8_halves for lo == 0 (at most 4 planes present)
__device__ __forceinline__ void transpose8_hi4(uint32_t& lo, uint32_t& hi) {
  uint32_t t;
  t = (hi ^ (hi >> 7)) & 0x00AA00AAu;
  hi ^= t ^ (t << 7);
  t = (hi ^ (hi >> 14)) & 0x0000CCCCu;
  hi ^= t ^ (t << 14);
  t = (hi << 4) & 0xF0F0F0F0u;
  lo = t;
  hi ^= t >> 4;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef int i32x2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2v lds_i32x2v;

// 2^52 + sum_{k<6} 128 * 2^(8k)
constexpr double kDigitBias = 4503599627370496.0 + 141289400074368.0;
constexpr int kSigTop = 46;  // |q rng 2^sig| < 2^46
constexpr int kStagePre = 4;  // 16 B pieces per thread loaded ahead of the tile

__device__ __forceinline__ long tr8_read(const uint8_t* p) {
  const i32x2v v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2v*)p);
  return __builtin_bit_cast(long, v);
}

__device__ __forceinline__ double swizzle_xor16(double v) {
  const uint64_t u = dbits(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(uint32_t)u, 0x401F);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(uint32_t)(u >> 32), 0x401F);
  return bitsd(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int ilogb_bits(double v) {  // exponent of |v| (subnormals: -1023)
  return (int)((dbits(v) >> 52) & 0x7FFu) - 1023;
}

// Issue priority of the calling wave from a block's progress: level 3
// (highest) over the first quarter of its work down to 0 over the last.
// The SIMD's arbiter prefers older waves among equal priorities, so blocks
// that share a compute unit would otherwise finish one after another (the
// youngest up to a third later, with the unit under-occupied meanwhile);
// dropping the priority of a block that is ahead lets the others catch up,
// and they end together.
__device__ __forceinline__ void set_progress_priority(int done, int total) {
  const int lv = total > 0 ? 3 - (4 * done) / total : 0;
  switch (lv) {
    case 3: __builtin_amdgcn_s_setprio(3); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
  }
}

// fp64 -> fp16 through an fp32 value the optimiser cannot fold away (a
// direct f64 -> f16 truncation is a long software sequence on this target)
__device__ __forceinline__ _Float16 to_half(double v) {
  float f = (float)v;
  asm volatile("" : "+v"(f));
  return (_Float16)f;
}

// max over the 32-lane half of the wave (lanes 0..31 / 32..63), in every lane
__device__ __forceinline__ double half_max(double v) {
  v = row_reduce(v, [](double a, double b) { return fmax(a, b); });
  return fmax(v, swizzle_xor16(v));
}
__device__ __forceinline__ double half_sum(double v) {
  v = row_reduce(v, [](double a, double b) { return a + b; });
  const double o = swizzle_xor16(v);
  return (threadIdx.x & 16) ? o + v : v + o;  // rows in order 0 + 1, 2 + 3
}

// LDS of one score block (members ordered largest first)
// Mask of the plane bytes of a depth-t channel in a transposing plane read
// (plane p in byte 7 - p: bytes 7 .. 8 - t kept).
__device__ __forceinline__ uint64_t plane_keep(uint32_t t) {
  return t >= 8u ? ~0ull : (t == 0u ? 0ull : ~0ull << (64u - 8u * t));
}

template <int GQA>
struct ScoreShared {
  static constexpr int NG = kTile / kGroup;  // 8 groups; wave w owns groups 2w, 2w + 1
  static constexpr int NHQ = (GQA + 3) / 4;  // head quads: two MFMA row blocks each
  static constexpr int CXS = kTile + 16;     // code-tile row stride (bytes)
  static constexpr int AOS = 2 * 8 * 2 * 8 + 16;  // digit chunks of a channel octet: [j][set] x 8 B, padded
  static constexpr int AMS = 4 * AOS;        // one (head quad, digit half) block of 32 channels
  static constexpr int AGS = NHQ * 2 * AMS;  // one group's digit chunks
  __attribute__((aligned(16))) uint8_t at[4][AGS];
  __attribute__((aligned(16))) uint8_t cx[32 * CXS];
  uint32_t meta[NG][kDim + 1];
  double qd[GQA][kDim];
  double kap[kDim];                          // 2^-(t_c+1) + [t_c > 0] / 2
  uint8_t s2c[kDim * 8];
  double Cpart[4][NG][GQA];                  // per-wave partial constants
  double tails[kGroup][GQA];
  uint16_t offs[kDim + 1];
  uint32_t wtot[2];
  __attribute__((aligned(4))) uint8_t tks[kDim];
  double redm[4][GQA], redz[4][GQA];
  uint8_t cperm[kDim];
  // un-plane descriptors of wave w, channel pair r of slab s, half-wave hw
  // at [32 w + 2 (4 s + r) + hw]: first slot's byte offset, plane mask
  // (low word, high word), the pair's larger depth
  uint4 udesc[128];
  uint32_t dcnt[2][9];                       // channels per depth value, per wave
  uint32_t qflag[2];                         // a non-finite query value, per wave
  int emx[2][GQA];
  double mfin[GQA];
};

template <int GQA, int DT>
__device__ __forceinline__ void score_block(ScoreShared<GQA>& sh, uint32_t* planes,
    const VBlock& vb, const uint8_t* store, int ub0, const void* q, uint8_t* tk, int tk_ready,
    int min1, int H, int G, int W, float RK, int64_t capmax, int ntile_ws, uint32_t* ebuf,
    double* tilepart, uint64_t* counters) {
  constexpr int esize = DT == 0 ? 2 : 4;
  constexpr int NG = kTile / kGroup;  // 8 groups; wave w owns groups 2w, 2w + 1
  static_assert(NG == 8, "a score tile is half of a 16-group key-plane tile");
  constexpr int NHQ = (GQA + 3) / 4;  // head quads: two MFMA row blocks each
  constexpr int CXS = kTile + 16;     // code-tile row stride (bytes)
  constexpr int AOS = 2 * 8 * 2 * 8 + 16;  // digit chunks of a channel octet: [j][set] x 8 B, padded
  constexpr int AMS = 4 * AOS;        // one (head quad, digit half) block of 32 channels
  constexpr int AGS = NHQ * 2 * AMS;  // one group's digit chunks
  constexpr int PRE = kStagePre;
  constexpr int MPT = NG * kDim / 256;
  auto& qd = sh.qd;
  auto& meta = sh.meta;
  auto& cx = sh.cx;
  auto& at = sh.at;
  auto& Cpart = sh.Cpart;
  auto& kap = sh.kap;
  auto& tails = sh.tails;
  auto& redm = sh.redm;
  auto& redz = sh.redz;
  auto& mfin = sh.mfin;
  auto& emx = sh.emx;
  auto& offs = sh.offs;
  auto& tks = sh.tks;
  auto& cperm = sh.cperm;
  auto& s2c = sh.s2c;
  auto& wtot = sh.wtot;
  auto& dcnt = sh.dcnt;
  auto& qflag = sh.qflag;
  auto& udesc = sh.udesc;

  // the call's read counters start from zero (the value selection, a later
  // launch, adds to them)
  if (counters && vb.x == 0 && vb.y == 0 && threadIdx.x < 4) counters[threadIdx.x] = 0ull;
  const int ux = ub0 + vb.x;  // the unit (request, KV head)
  const int b = ux / G, g = ux % G;
  const ReqRecord r = req_of(store, b);
  const int64_t len = r.len;
  const int ntl = (int)((len + kTile - 1) / kTile);
  // this block's share of the unit's tiles: every ny-th one from y, so that
  // the blocks of a unit (all on one XCD) work on neighbouring tiles at the
  // same time and the two halves of a key-plane tile meet in its L2
  const int ny = vb.ny;
  const int tile_begin = vb.y;
  if (tile_begin >= ntl) {
    // an empty request has no closed group (E^K = 0): all key depths are 0
    // (or the minimum depth)
    if (!tk_ready && ntl == 0 && vb.y == 0 && threadIdx.x < kDim)
      tk[((int64_t)b * G + g) * kDim + threadIdx.x] = (uint8_t)min1;
    return;
  }
  const int64_t Tp = len & ~(int64_t)(kGroup - 1);
  const Unit u = unit_of(const_cast<uint8_t*>(store), r, g, G, kDim, W, esize);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  auto tile_ngp = [&](int tile) -> int {
    const int64_t n = Tp / kGroup - (int64_t)tile * NG;
    return (int)(n < 0 ? 0 : (n > NG ? NG : n));
  };
  // metadata word k of this thread: group k * 256 / kDim + tid / kDim of
  // the tile, channel tid % kDim; buffer loads, zero past the closed groups
  uint32_t pmeta[MPT];
  const __amdgpu_buffer_rsrc_t rs_meta = __builtin_amdgcn_make_buffer_rsrc(
      u.kmeta, (short)0, (int)(Tp / kGroup) * kDim * 4, kBufWord3);
  auto load_meta = [&](int tile) {
#pragma unroll
    for (int k = 0; k < MPT; ++k)
      pmeta[k] = __builtin_amdgcn_raw_buffer_load_b32(rs_meta, (tile * NG * kDim + k * 256 + tid) * 4, 0, 0);
  };

  // ---- once per block: depths, query, per-head digit scale, slot table ----
  // Key allocation of the unit: under per-layer budgets it comes from the
  // key allocation launch (tk_ready); otherwise every block of the unit
  // computes it (w_c = (sum_h q_hc^2) E^K_c in head order, then ChooseDepths
  // over the channels by wave 0) and the unit's first block writes it out.
  // A query with a non-finite value reads nothing: its unit's key weights are
  // zero (depths 0) and its softmax statistics NaN, so that no value is
  // refined and every output of the unit is NaN.
  // (the query and E^K loads go out before the first tile's metadata, so
  // that waiting for them does not wait for the metadata)
  double ek = 0.0;
  bool qnf = false;
  double qv[GQA];
  uint8_t tkr = 0;
  if (tid < kDim) {
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh)
      qv[hh] = load_elem<DT>(q, ((int64_t)b * H + (int64_t)g * GQA + hh) * kDim + tid);
    ek = u.ek[tid];
    if (tk_ready) tkr = tk[((int64_t)b * G + g) * kDim + tid];
  }
  load_meta(tile_begin);  // independent of the depths: in flight during the setup
  if (tid < kDim) {
    const int c = tid;
    double qsq = 0.0;
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) {
      qd[hh][c] = qv[hh];
      qnf |= !isfinite(qv[hh]);
      qsq = __dadd_rn(qsq, __dmul_rn(qv[hh], qv[hh]));
    }
    if (tk_ready) tks[c] = tkr;
    else kap[c] = __dmul_rn(qsq, ek);  // the key weight, until kap is set below
    const bool any = __ballot(qnf) != 0ull;  // (waves 0 and 1: every channel)
    if (lane == 0) qflag[wv] = any ? 1u : 0u;
  }
  // barriers in the set-up order LDS only: the loads of the first tile in
  // flight (and the depths written out) are not waited for
  lds_barrier();
  const bool qbad = (qflag[0] | qflag[1]) != 0u;
  if (!tk_ready) {
    if (wv == 0) {
      // the minimum depth one: levels 2..W of w are levels 1..W-1 of w/4
      // (exact), over the budget left after the d_h forced levels
      const double sc = min1 ? 0.25 : 1.0;
      const double w2[2] = {qbad ? 0.0 : kap[lane] * sc, qbad ? 0.0 : kap[lane + 64] * sc};
      uint32_t Bk = (uint32_t)floor((double)RK * (double)kDim);
      if (min1) Bk = Bk > (uint32_t)kDim ? Bk - (uint32_t)kDim : 0u;
      uint32_t sel[2];
      key_depths_wave(w2, W - min1, Bk, reinterpret_cast<uint32_t*>(planes), sel);
      sel[0] += (uint32_t)min1;
      sel[1] += (uint32_t)min1;
      tks[lane] = (uint8_t)sel[0];
      tks[lane + 64] = (uint8_t)sel[1];
      if (tile_begin == 0) {  // the unit's first block writes the depths out
        tk[((int64_t)b * G + g) * kDim + lane] = (uint8_t)sel[0];
        tk[((int64_t)b * G + g) * kDim + lane + 64] = (uint8_t)sel[1];
      }
    }
    lds_barrier();
  }
  uint32_t tv_ = 0, inc = 0, below = 0;
  if (tid < kDim) {
    const int c = tid;
    tv_ = tks[c];
    // 2^er >= sqrt(E_c) >= every closed group's rng_c
    const int er = ek > 0.0 ? ((ilogb_bits(ek) + 2) >> 1) : 0;
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) {
      const double qv = qd[hh][c];
      const int e = (qv != 0.0 && ek > 0.0 && tv_ > 0u) ? ilogb_bits(qv) + 1 + er : -100000;
      const int em = wave_max_i32(e);
      if (lane == 0) emx[wv][hh] = em;
    }
    inc = wave_incl_scan_u32(tv_);
    if (lane == 63) wtot[wv] = inc;
    // depth histogram of the wave, and this channel's rank among equal
    // depths below it in the wave
    uint64_t mine = 0ull;
#pragma unroll
    for (int v = 0; v <= 8; ++v) {
      const uint64_t bv = __ballot(tv_ == (uint32_t)v);
      if (tv_ == (uint32_t)v) mine = bv;
      if (lane == v) dcnt[wv][v] = (uint32_t)__popcll(bv);
    }
    below = (uint32_t)__popcll(mine & ((1ull << lane) - 1ull));
  }
  lds_barrier();
  if (tid < kDim) {
    if (wv == 1) inc += wtot[0];
    offs[tid + 1] = (uint16_t)inc;
    if (tid == 0) offs[0] = 0;
    const uint32_t o = inc - tv_;
    for (uint32_t p = 0; p < tv_; ++p) s2c[o + p] = (uint8_t)tid;
    // channel order by depth, deepest first (stable): the slabs then hold
    // channels of similar depth, and trailing depth-0 slabs are skipped
    uint32_t rank = below + (wv == 1 ? dcnt[0][tv_] : 0u);
#pragma unroll
    for (int v = 1; v <= 8; ++v)
      if ((uint32_t)v > tv_) rank += dcnt[0][v] + dcnt[1][v];
    cperm[rank] = (uint8_t)tid;
    kap[tid] = ldexp_pow2(-(int)tv_ - 1) + (tv_ > 0u ? 0.5 : 0.0);
  }
  lds_barrier();
  const int ns = offs[kDim];
  const int nq = ns * 2;  // 16 B pieces per tile
  // Staging.  A score tile is half (h = tile & 1) of a 16-group key-plane
  // tile: its segment of a chosen line (channel c, plane p) is words
  // 8 h .. 8 h + 7 of the line's 16.  Piece idx = (slot s, half q2) is
  // words 4 q2 .. 4 q2 + 3 of it -> planes[s][4 q2 .. 4 q2 + 3].
  auto seg_base = [&](int tile) -> const uint32_t* {
    return u.kplanes + (int64_t)(tile >> 1) * kDim * W * 16 + 8 * (tile & 1);
  };
  auto piece = [&](int idx, int tile, int ngp) -> uint4 {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    const int s = idx >> 1, q2 = idx & 1;
    const int c = s2c[s];
    const int p = s - offs[c];
    if (4 * q2 < ngp) v = *reinterpret_cast<const uint4*>(seg_base(tile) + (c * W + p) * 16 + 4 * q2);
    return v;
  };
  // Piece k of this thread is idx = k * 256 + tid.  Its byte offset from a
  // tile's segment base and its place in LDS do not depend on the tile, so
  // both are set up once; the segment base is the scalar base of a buffer
  // (pieces past the chosen lines take an offset outside it and read as
  // zeros, and the groups of a partial tile past the closed ones are read
  // but unused).
  uint32_t poff[PRE];
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const int idx = k * 256 + tid;
    int o = kBufOff;
    if (idx < nq) {
      const int s = idx >> 1, c = s2c[s], p = s - offs[c];
      o = ((c * W + p) * 16 + 4 * (idx & 1)) * 4;
    }
    poff[k] = (uint32_t)o;
  }
  uint4 pre[PRE];
  auto load_pieces = [&](int tile) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(seg_base(tile)), (short)0, kDim * W * 64 - 32 * (tile & 1), kBufWord3);
#pragma unroll
    for (int k = 0; k < PRE; ++k) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)poff[k], 0, 0);
      pre[k] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  auto load_ahead = [&](int tile) {
    load_pieces(tile);
    load_meta(tile);
  };
  // slot s is 32 B at planes + 32 s; piece k of this thread sits in slot
  // 128 k + tid / 2
  auto stage_put = [&](int idx, uint4 v) __attribute__((always_inline)) {
    *reinterpret_cast<uint4*>(planes + (idx >> 1) * 8 + (idx & 1) * 4) = v;
  };
  uint8_t* const pl0 = reinterpret_cast<uint8_t*>(planes) + (tid >> 1) * 32 + (tid & 1) * 16;
  auto store_ahead = [&](int tile) {
#pragma unroll
    for (int k = 0; k < PRE; ++k)
      if (k * 256 + tid < nq) *reinterpret_cast<uint4*>(pl0 + k * 4096) = pre[k];
#pragma unroll
    for (int k = 0; k < MPT; ++k) {
      const int i = k * 256 + tid;
      meta[i / kDim][i % kDim] = pmeta[k];
    }
    // pieces past the prefetched ones (deep reads only)
    const int ngp = tile_ngp(tile);
    for (int idx = PRE * 256 + tid; idx < nq; idx += 256) stage_put(idx, piece(idx, tile, ngp));
  };
  // the first tile's pieces go out as soon as the slot table is known (its
  // metadata is already in flight); the per-block set-up below overlaps them
  load_pieces(tile_begin);
  // scalar table: lane 8 s + i of wave w describes the channel at sorted
  // position 32 s + w + 4 i (depth | first slot << 8; slot 0 when depth 0)
  // the un-plane descriptors (entry e: wave e / 32, slab (e / 8) % 4, pair
  // (e / 2) % 4, half-wave e % 2; the sorted position 32 slab + wave +
  // 4 (e % 8)); a depth-0 channel reads slot 0, masked
  if (tid < 128) {
    const int pos = 32 * ((tid >> 3) & 3) + (tid >> 5) + 4 * (tid & 7);
    const int c = cperm[pos], c2 = cperm[pos ^ 4];
    const uint32_t t = tks[c];
    const uint64_t keep = plane_keep(t);
    udesc[tid] = make_uint4((t ? (uint32_t)offs[c] : 0u) * 32u, (uint32_t)keep, (uint32_t)(keep >> 32),
                            max(t, (uint32_t)tks[c2]));
  }
  // digit scale 2^sig of head h: lane quad q of head quad hq is head 4 hq + q
  auto head_sig = [&](int hh) -> int {
    const int e = max(emx[0][hh], emx[1][hh]);
    return e > -100000 ? kSigTop - e : 0;
  };
  // Per block, for the digit build of each slab: this lane's channel
  // (sorted position 32 s + lane % 32), whether it has depth, and the live
  // slabs (deepest first, so the live ones come first)
  int cAs[4];
  int nslab = 0;
  // the per-group constants' query operand (column lane % 16 = (channel set
  // z, head h) = (n / 8, n % 8), channel 32 w + 8 st + 4 z + lane / 16) for
  // the 4 steps
  static_assert(GQA <= 8, "a channel set's heads fit 8 columns");
  double qbs[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int hB = lane & 7, c = 32 * wv + 8 * st + 4 * ((lane >> 3) & 1) + (lane >> 4);
    qbs[st] = hB < GQA ? qd[min(hB, GQA - 1)][c] : 0.0;
  }
  // the logit scale exponent -(sig + 8) of the lane's epilogue head per head quad
  int lsg[NHQ];
#pragma unroll
  for (int hq = 0; hq < NHQ; ++hq) lsg[hq] = -head_sig(min(4 * hq + (lane >> 4), GQA - 1)) - 8;
  double qas[4][NHQ][2];  // q 2^sig of the lane's channel and two heads, per slab
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    cAs[sb] = cperm[32 * sb + (lane & 31)];
    const bool live = tks[cAs[sb]] > 0;
    nslab += tks[cperm[32 * sb]] != 0 ? 1 : 0;
#pragma unroll
    for (int hq = 0; hq < NHQ; ++hq)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int hh = 4 * hq + 2 * (lane >> 5) + e;
        qas[sb][hq][e] = (hh < GQA && live) ? qd[min(hh, GQA - 1)][cAs[sb]] * ldexp_pow2(head_sig(min(hh, GQA - 1))) : 0.0;
      }
  }

  store_ahead(tile_begin);
  lds_barrier();
  // the register prefetch runs one tile ahead; it is issued right after the
  // previous staging write, before the epilogue's global stores, so that no
  // wait on those stores delays it
  if (tile_begin + ny < ntl) load_ahead(tile_begin + ny);

  const int kq = lane >> 4, jj = (lane & 15) >> 1, ss = lane & 1;
  // transposing plane read of two channels: the half-wave hw = lane / 32
  // takes one; lane 2j + s of its quarter q2 = (lane / 16) % 2 addresses
  // plane 7 - j, groups 4 q2 + 2 s and 4 q2 + 2 s + 1 (8-byte chunk
  // 2 q2 + s of the 32-byte slot); lane o of the half-wave then holds the
  // plane bytes of octet o (tokens 8 o .. 8 o + 7 of the tile)
  const int hw = lane >> 5;
  const int c8 = 2 * (kq & 1) + ss;
  // this lane's plane-read address less the channel's first slot, and its
  // descriptors (channel 2 r + hw of the slab's pair r)
  const uint8_t* const lane_pl = reinterpret_cast<const uint8_t*>(planes) + (7 - jj) * 32 + (c8 << 3);
  const uint4* const ldesc = &udesc[32 * wv + hw];
  // digit chunk (channel octet co, channel j, set s) of block (hq, half m)
  auto achunk = [&](int hq, int m, int co, int j, int s) -> int {
    return (2 * hq + m) * AMS + co * AOS + (2 * j + s) * 8;
  };
  const int c32 = lane & 31, sA = lane >> 5;  // A-build: channel, head pair of the quad

  const int my_tiles = (ntl - tile_begin + ny - 1) / ny;
  for (int tile = tile_begin; tile < ntl; tile += ny) {
    set_progress_priority((tile - tile_begin) / ny, my_tiles);
    const int64_t t0 = (int64_t)tile * kTile;
    const int ngp = tile_ngp(tile);
    const bool more = tile + ny < ntl;

    // ---- per-group constants C[g][h] = sum_c base[g][c] q[h][c] on the fp64
    // matrix cores: wave w contracts its 32 channels in 4 steps of two
    // channel sets z = 0, 1 of 4 channels each.  Rows m = (z, group) =
    // (m / 8, m % 8), columns n = (z, head) = (n / 8, n % 8); A: lane l =
    // (row l % 16, channel l / 16 of the row's set), B: (channel l / 16 of
    // the column's set, column l % 16).  Result lane l, register i = (row
    // 4 i + l / 16, column l % 16); only the blocks with equal sets are
    // wanted: set z's sums are registers 2 z, 2 z + 1 of the lanes with
    // (l / 8) % 2 = z, and the lanes of set 1 add those of set 0, 8 lanes
    // below in the same row ----
    {
      const int mA = lane & 15, kk = lane >> 4;
      const int gA = mA & 7, zA = mA >> 3;
      f64x4 cd = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int c = 32 * wv + 8 * st + 4 * zA + kk;
        const uint32_t m = meta[gA][c];
        const double lo = (double)bf16_to_float(m & 0xFFFFu);
        const double rng = (double)bf16_to_float(m >> 16);
        const double base = fma(rng, kap[c], lo);
        cd = __builtin_amdgcn_mfma_f64_16x16x4f64(base, qbs[st], cd, 0, 0, 0);
      }
      const double c0 = cd[2] + dpp_f64<kDppRowShr8>(cd[0]);  // groups kk, 4 + kk
      const double c1 = cd[3] + dpp_f64<kDppRowShr8>(cd[1]);
      const int hB = lane & 7;
      if ((lane & 8) && hB < GQA) {
        Cpart[wv][kk][hB] = c0;
        Cpart[wv][4 + kk][hB] = c1;
      }
    }
    const int64_t ntail = len - Tp;
    const bool tail_here = ntail > 0 && Tp >= t0 && Tp < t0 + kTile;
    if (tail_here) {
      const int rr = tid >> 3, part = tid & 7;
      double st[GQA];
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) st[hh] = 0.0;
      if (rr < ntail) {
        for (int c = part * 16; c < part * 16 + 16; ++c) {
          const double kv = load_elem<DT>(u.ktail, (int64_t)rr * kDim + c);
#pragma unroll
          for (int hh = 0; hh < GQA; ++hh) st[hh] = fma(qd[hh][c], kv, st[hh]);
        }
      }
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) st[hh] = group_sum<8>(st[hh]);
      if (part == 0 && rr < ntail)
#pragma unroll
        for (int hh = 0; hh < GQA; ++hh) tails[rr][hh] = st[hh] * kInvSqrtD;
    }
    lds_barrier();  // constants and open-group logits (the slab loop may not run)

    // ---- un-plane + int8 MFMA, one 32-channel slab at a time ----
    i32x4 acc[4][NHQ][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int hq = 0; hq < NHQ; ++hq) acc[i][hq][0] = acc[i][hq][1] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int slab = 0; slab < 4; ++slab) {
      if (slab >= nslab) break;  // deepest first: the rest is depth 0
      // The wave's 8 channels of the slab (sorted positions w + 4 k, nearly
      // equal depth) in pairs (2 r, 2 r + 1): one transposing LDS read per
      // pair gives lane o of half-wave hw the 8 plane bytes of octet o of
      // channel 2 r + hw (plane p in byte 7 - p; planes past the depth are
      // read from the padding and masked).
      uint2 pb[4];
      uint32_t kl[4], kh[4];
      int tmxr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint4 d = ldesc[2 * (4 * slab + r)];
        pb[r] = __builtin_bit_cast(uint2, tr8_read(lane_pl + d.x));
        kl[r] = d.y;
        kh[r] = d.z;
        tmxr[r] = __builtin_amdgcn_readfirstlane((int)d.w);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tmx = tmxr[r];
        if (tmx == 0) continue;  // both depth 0: their codes meet zero digits
        uint32_t lo = pb[r].x & kl[r];
        uint32_t hi = (pb[r].y & kh[r]) ^ 0xFF000000u;
        if (tmx <= 4) transpose8_hi4(lo, hi);
        else transpose8_halves(lo, hi);
        const int cl = wv + 4 * (2 * r + hw);
        *reinterpret_cast<uint2*>(cx + cl * CXS + 8 * (lane & 31)) = make_uint2(lo, hi);
      }
      lds_barrier();
      // digit words of this lane's channel (sorted position c32), heads
      // 4 hq + 2 sA and 4 hq + 2 sA + 1: the chunk of digit half m holds
      // digits 4m .. 4m + 3 of both heads
      const int cA = cAs[slab];
      const double (&qa)[NHQ][2] = qas[slab];
      // the ranges of the wave's groups for this lane's channel, read together
      uint32_t rmeta[2];
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) rmeta[gi] = meta[2 * wv + gi][cA];
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int gw = 2 * wv + gi;
        if (gw >= ngp) break;
        {
          const double rng = (double)bf16_to_float(rmeta[gi] >> 16);
#pragma unroll
          for (int hq = 0; hq < NHQ; ++hq) {
            const uint64_t d0 = dbits(fma(qa[hq][0], rng, kDigitBias)) ^ 0x8080808080808080ull;
            const uint64_t d1 = dbits(fma(qa[hq][1], rng, kDigitBias)) ^ 0x8080808080808080ull;
            *reinterpret_cast<uint2*>(&at[wv][achunk(hq, 0, c32 >> 3, c32 & 7, sA)]) =
                make_uint2((uint32_t)d0, (uint32_t)d1);
            *reinterpret_cast<uint2*>(&at[wv][achunk(hq, 1, c32 >> 3, c32 & 7, sA)]) =
                make_uint2((uint32_t)(d0 >> 32), (uint32_t)(d1 >> 32));
          }
        }
        wave_lds_fence();
        long A[NHQ][2];
#pragma unroll
        for (int hq = 0; hq < NHQ; ++hq)
#pragma unroll
          for (int m = 0; m < 2; ++m) A[hq][m] = tr8_read(&at[wv][achunk(hq, m, kq, jj, ss)]);
#pragma unroll
        for (int tl = 0; tl < 2; ++tl) {
          const int tb = 2 * gi + tl;         // the wave's token block
          const int oct = 2 * (4 * wv + tb);  // first octet of the block
          const long Bv = tr8_read(cx + (8 * kq + jj) * CXS + 8 * (oct + ss));
#pragma unroll
          for (int hq = 0; hq < NHQ; ++hq)
#pragma unroll
            for (int m = 0; m < 2; ++m)
              acc[tb][hq][m] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A[hq][m], Bv, acc[tb][hq][m], 0, 0, 0);
        }
        wave_lds_fence();
      }
      lds_barrier();
    }
    // the staged planes and metadata of this tile are dead: next tile in
    if (more) store_ahead(tile + ny);
    if (tile + 2 * ny < ntl) load_ahead(tile + 2 * ny);

    // ---- logits in registers: lane -> (token 16 (4 w + tb) + lane % 16,
    // head 4 hq + lane / 16); its digits sit in its own accumulators ----
    const int toff = (int)(Tp - t0);  // tile-local first open-group token (if here)
    const int hl = lane >> 4;
    double sv[4][NHQ];
#pragma unroll
    for (int hq = 0; hq < NHQ; ++hq) {
      const int hh = 4 * hq + hl;
      const int hc = min(hh, GQA - 1);

#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const int gw = 2 * wv + (tb >> 1);
        const int tok = 16 * (4 * wv + tb) + (lane & 15);
        double s = -INFINITY;
        if (hh < GQA) {
          if (gw < ngp) {
            const i32x4 d0 = acc[tb][hq][0], d1 = acc[tb][hq][1];
            // digit sums are below 2^21 in magnitude (128 channels of
            // byte x byte products), so digit pairs combine exactly in int32
            const int p01 = d0[0] + d0[1] * 256, p23 = d0[2] + d0[3] * 256, p45 = d1[0] + d1[1] * 256;
            const double P = fma((double)p45, 0x1p32, fma((double)p23, 0x1p16, (double)p01));
            const double C = (Cpart[0][gw][hc] + Cpart[1][gw][hc]) + (Cpart[2][gw][hc] + Cpart[3][gw][hc]);
            s = (C + ldexp(P, lsg[hq])) * kInvSqrtD;
          } else if (tail_here && tok >= toff && tok < toff + ntail) {
            s = tails[tok - toff][hc];
          }
        }
        sv[tb][hq] = s;
      }
    }
    // tile max per head: lanes of a quad share the head
#pragma unroll
    for (int hq = 0; hq < NHQ; ++hq) {
      double m = sv[0][hq];
#pragma unroll
      for (int tb = 1; tb < 4; ++tb) m = fmax(m, sv[tb][hq]);
      m = row_reduce(m, [](double a, double c) { return fmax(a, c); });
      const int hh = 4 * hq + hl;
      if ((lane & 15) == 0 && hh < GQA) redm[wv][hh] = m;
    }
    lds_barrier();
#pragma unroll
    for (int hq = 0; hq < NHQ; ++hq) {
      const int hh = 4 * hq + hl;
      const int hc = min(hh, GQA - 1);
      const double mt = fmax(fmax(redm[0][hc], redm[1][hc]), fmax(redm[2][hc], redm[3][hc]));
      const int64_t lane0 = ((int64_t)b * H + (int64_t)g * GQA + hc) * capmax + t0 + 64 * wv + (lane & 15);
      uint32_t* const ep = ebuf + lane0;
      double z = 0.0;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const double e = exp_nonpos(sv[tb][hq] - mt);
        if (sv[tb][hq] != -INFINITY) {  // a token of the request (logit NaN if qbad)
          ep[16 * tb] = qbad ? 0u : enc_e(e);
          z += e;
        }
      }
      z = row_reduce(z, [](double a, double c) { return a + c; });
      if ((lane & 15) == 0 && hh < GQA) {
        redz[wv][hh] = z;
        if (wv == 0) mfin[hh] = mt;
      }
    }
    lds_barrier();
    if (tid < GQA) {
      double* tp = tilepart + (((int64_t)b * H + (int64_t)g * GQA + tid) * ntile_ws + tile) * 2;
      tp[0] = qbad ? __builtin_nan("") : mfin[tid];
      tp[1] = qbad ? __builtin_nan("") : (redz[0][tid] + redz[1][tid]) + (redz[2][tid] + redz[3][tid]);
    }
  }
}

// The score launch: one block per (unit, run).
template <int GQA, int DT>
__global__ __launch_bounds__(256, GQA <= 4 ? 3 : 2) void k_score(
    const uint8_t* store, int ub0, const void* q, uint8_t* tk, int tk_ready, int min1, int H, int G,
    int W, float RK, int64_t capmax, int ntile_ws, uint32_t* ebuf, double* tilepart,
    uint64_t* counters) {
  __shared__ ScoreShared<GQA> sh;
  extern __shared__ __attribute__((aligned(16))) uint32_t planes[];  // [slot][8]
  score_block<GQA, DT>(sh, planes, launch_block(), store, ub0, q, tk, tk_ready, min1, H, G, W, RK,
                       capmax, ntile_ws, ebuf, tilepart, counters);
}

// ---------------------------------------------------------------------------
// Score under the Lloyd-tree code ([ReadKV] Sec. 3.1-3.2).  Block (unit, y)
// takes every ny-th 256-token tile from y; thread j takes token j of the
// tile and forms, for every query head h of the unit,
//   s_hj = (qb_h + sum_c w_hc C(t_c, P_jc)) / sqrt(d)   packed tokens
//   s_hj = (sum_c q_hc k_jc) / sqrt(d)                  open group (exact)
// in fp64, with w_hc = q'_hc sigma^K_c and qb_h = sum_c q'_hc mu^K_c (both
// from the key allocation), C(t, P) the float32 centroid of depth-t cell P,
// P = the token's first t planes of channel c; a channel at depth 0
// reconstructs to its mean and appears only in qb.  Per tile:
//  1. un-plane: thread (channel quad, 32-token word) loads the chosen plane
//     words of its four channels, and 8x8 bit transposes turn them into code
//     bytes X = P 2^(8-t); one 32-bit LDS word per (token, channel quad);
//  2. thread j reads its code word per channel quad, looks the four centroids
//     up in an LDS table indexed by (depth, X), and accumulates with the
//     weights, which the scalar unit loads (the channel loop is uniform).
// Then the split-context softmax partials as the uniform code's score
// (per-tile max and sum of exp(s - m)), but every token's fp64 logit is kept
// in place of its exponential: the value allocation forms alpha = exp(s -
// m) / Z from it, so that equal logits anywhere in the context give
// bitwise-equal weights (every token shares the calibrated mean at depth 0,
// so ties across tiles are common here).  A unit whose query is not finite
// (qb NaN) writes NaN partials and NaN logits.  Barriers order LDS only: the
// next tile's plane words stay in flight across them.
// ---------------------------------------------------------------------------
typedef const double __attribute__((address_space(4)))* cdptr;
typedef const uint32_t __attribute__((address_space(4)))* cuptr;

template <int GQA, int DT>
__global__ __launch_bounds__(256, 3) void k_score_lloyd(const uint8_t* store, const uint8_t* cb,
                                                        const void* q, const uint8_t* tk,
                                                        const double* qw, const double* qb, int H,
                                                        int G, int W, int64_t capmax, int ntile_ws,
                                                        uint32_t* ebuf, double* tilepart) {
  constexpr int CS = kDim / 4 + 1;  // code-word row stride (words): rows 33 banks apart
  __shared__ uint32_t codes[kTile * CS];
  // centroid of depth-t cell P at (2^t - 1) + P: a depth's cells are
  // contiguous, so the up to 2^t distinct entries a lookup at depth t can
  // touch sit in distinct banks for t <= 5
  __shared__ float ftab[512];
  __shared__ uint32_t tk4s[kDim / 4];
  __shared__ double redm[4][GQA], redz[4][GQA];
  const CodecLayout C = codec_layout(G, kDim);
  const int ux = (int)blockIdx.x;
  const int b = ux / G, g = ux % G;
  const ReqRecord r = req_of(store, b);
  const int64_t len = r.len;
  const int ntl = (int)((len + kTile - 1) / kTile);
  const int ny = (int)gridDim.y;
  if ((int)blockIdx.y >= ntl) return;
  const int64_t Tp = len & ~(int64_t)(kGroup - 1);
  const int esize = DT == 0 ? 2 : 4;
  const Unit u = unit_of(const_cast<uint8_t*>(store), r, g, G, kDim, W, esize);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t hrow0 = (int64_t)b * H + (int64_t)g * GQA;

  // ---- once per block: depths, the centroid table ----
  const float* cent = reinterpret_cast<const float*>(cb + C.cent);
  for (int i = tid; i < 512; i += 256) ftab[i] = cent[i];
  if (tid < kDim / 4) tk4s[tid] = reinterpret_cast<const uint32_t*>(tk + (int64_t)ux * kDim)[tid];
  double qbv[GQA];
  bool qbad = false;
#pragma unroll
  for (int hh = 0; hh < GQA; ++hh) {
    qbv[hh] = qb[hrow0 + hh];
    qbad |= !isfinite(qbv[hh]);
  }
  // weights and depths through the scalar unit (bases forced uniform: a
  // per-lane use of the same address elsewhere would otherwise move them to
  // vector registers and the loads to the vector memory path)
  auto uniform_ptr = [](const void* p) -> uint64_t {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
  };
  const cdptr wsc = (cdptr)uniform_ptr(qw + (int64_t)ux * kDim * GQA);
  const cuptr tsc = (cuptr)uniform_ptr(tk + (int64_t)ux * kDim);
  lds_barrier();
  // un-plane role: channels 4 cq .. 4 cq + 3, 32-token word kwd of the tile
  const int cq = tid >> 3, kwd = tid & 7;
  const uint32_t t4u = tk4s[cq];

  // the plane words of this thread's four channels and word of tile `tile`
  // (buffer loads: planes past a channel's depth take an offset beyond the
  // buffer and read zero), loaded one tile ahead
  uint32_t w[4][8];
  auto load_words = [&](int tile) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        u.kplanes + (int64_t)(tile >> 1) * kDim * W * 16, (short)0, kDim * W * 16 * 4, kBufWord3);
    const int wo = 8 * (tile & 1) + kwd;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int t = (t4u >> (8 * s4)) & 0xFF;
#pragma unroll
      for (int p = 0; p < 8; ++p)
        w[s4][p] = __builtin_amdgcn_raw_buffer_load_b32(
            rs, p < t ? (((4 * cq + s4) * W + p) * 16 + wo) * 4 : kBufOff, 0, 0);
    }
  };
  load_words((int)blockIdx.y);

  for (int tile = (int)blockIdx.y; tile < ntl; tile += ny) {
    const int64_t t0 = (int64_t)tile * kTile;
    // ---- 1. un-plane this half of key tile tile / 2 ----
    {
      lds_barrier();  // the previous tile's codes are done with
      // per octet o of the word: code bytes of tokens 32 kwd + 8 o + i
#pragma unroll
      for (int o = 0; o < 4; ++o) {
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          // byte 7 - p = byte o of plane p's word
          const uint32_t b76 = __builtin_amdgcn_perm(w[s4][6], w[s4][7], (uint32_t)(o | ((o + 4) << 8)) | 0x0C0C0000u);
          const uint32_t b54 = __builtin_amdgcn_perm(w[s4][4], w[s4][5], (uint32_t)(o | ((o + 4) << 8)) | 0x0C0C0000u);
          const uint32_t b32 = __builtin_amdgcn_perm(w[s4][2], w[s4][3], (uint32_t)(o | ((o + 4) << 8)) | 0x0C0C0000u);
          const uint32_t b10 = __builtin_amdgcn_perm(w[s4][0], w[s4][1], (uint32_t)(o | ((o + 4) << 8)) | 0x0C0C0000u);
          lo[s4] = b76 | (b54 << 16);  // bytes: plane 7, 6, 5, 4
          hi[s4] = b32 | (b10 << 16);  // bytes: plane 3, 2, 1, 0
          transpose8_halves(lo[s4], hi[s4]);
        }
        // 4 x 4 byte transposes: token i's word holds the four channels' codes
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const uint32_t* v = half ? hi : lo;
          const uint32_t a01l = __builtin_amdgcn_perm(v[1], v[0], 0x05010400u);  // x0 y0 x1 y1 (bytes 0,1)
          const uint32_t a01h = __builtin_amdgcn_perm(v[1], v[0], 0x07030602u);  // bytes 2,3
          const uint32_t a23l = __builtin_amdgcn_perm(v[3], v[2], 0x05010400u);
          const uint32_t a23h = __builtin_amdgcn_perm(v[3], v[2], 0x07030602u);
          const uint32_t tok0 = __builtin_amdgcn_perm(a23l, a01l, 0x05040100u);
          const uint32_t tok1 = __builtin_amdgcn_perm(a23l, a01l, 0x07060302u);
          const uint32_t tok2 = __builtin_amdgcn_perm(a23h, a01h, 0x05040100u);
          const uint32_t tok3 = __builtin_amdgcn_perm(a23h, a01h, 0x07060302u);
          const int j0 = 32 * kwd + 8 * o + 4 * half;
          codes[(j0 + 0) * CS + cq] = tok0;
          codes[(j0 + 1) * CS + cq] = tok1;
          codes[(j0 + 2) * CS + cq] = tok2;
          codes[(j0 + 3) * CS + cq] = tok3;
        }
      }
      if (tile + ny < ntl) load_words(tile + ny);  // lands during this tile's logits
      lds_barrier();
    }
    // ---- 2. logits (uniform control flow: the channel loop's depths and
    // weights are scalar loads) ----
    const int64_t tok = t0 + tid;
    double sv[GQA];
    {
      double acc[GQA];
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) acc[hh] = 0.0;
      // software pipeline over the channel quads: quad c's centroid lookups
      // and weights are in flight during quad c - 1's multiply-adds, its code
      // word and depths two quads ahead, so that one wait per quad covers
      // loads issued a quad earlier.  (A channel at depth 0 looks up the
      // table's entry 0, which is zero; a quad at depth 0 is skipped.)
      auto lookup = [&](uint32_t t4, uint32_t x4, float (&cv)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const uint32_t t = (t4 >> (8 * s4)) & 0xFFu;
          cv[s4] = ftab[((1u << t) - 1u) + (((x4 >> (8 * s4)) & 0xFFu) >> (8u - t))];
        }
      };
      auto weights = [&](int c4, double (&wq)[4][GQA]) __attribute__((always_inline)) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
          for (int hh = 0; hh < GQA; ++hh) wq[s4][hh] = wsc[(4 * c4 + s4) * GQA + hh];
      };
      constexpr int NQ = kDim / 4;
      uint32_t t4c = tsc[0], t4n = tsc[1];
      uint32_t x4n = codes[tid * CS + 1];
      float cvc[4];
      double wqc[4][GQA];
      lookup(t4c, codes[tid * CS], cvc);
      weights(0, wqc);
      // (the prologue's loads complete before the loop: otherwise the loop
      // head, which merges the first entry with the back edge, waits for them
      // in every iteration)
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
#pragma unroll 2
      for (int c4 = 0; c4 < NQ; ++c4) {
        float cvn[4] = {0.f, 0.f, 0.f, 0.f};
        double wqn[4][GQA];
        if (c4 + 1 < NQ) {
          lookup(t4n, x4n, cvn);
          weights(c4 + 1, wqn);
        }
        uint32_t t4nn = 0u, x4nn = 0u;
        if (c4 + 2 < NQ) {
          t4nn = tsc[c4 + 2];
          x4nn = codes[tid * CS + c4 + 2];
        }
        if (t4c != 0u) {
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
            for (int hh = 0; hh < GQA; ++hh) acc[hh] = fma(wqc[s4][hh], (double)cvc[s4], acc[hh]);
        }
        t4c = t4n;
        t4n = t4nn;
        x4n = x4nn;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          cvc[s4] = cvn[s4];
#pragma unroll
          for (int hh = 0; hh < GQA; ++hh) wqc[s4][hh] = wqn[s4][hh];
        }
      }
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) sv[hh] = __dmul_rn(__dadd_rn(qbv[hh], acc[hh]), kInvSqrt128);
    }
    if (t0 + kTile > Tp) {
      // the open group's tokens are in this tile: exact keys and query,
      // staged in the code tile's LDS (dead by now) as fp32 keys [32][d]
      // (exact for both input types) and fp64 query rows [GQA][d]
      float* tkey = reinterpret_cast<float*>(codes);
      double* tq = reinterpret_cast<double*>(codes + kGroup * kDim);
      static_assert(kGroup * kDim + 2 * GQA * kDim <= kTile * CS, "fits the code tile");
      const int ntl_tok = (int)(len - Tp);
      lds_barrier();  // every thread is done with the codes
      for (int i = tid; i < ntl_tok * kDim; i += 256) tkey[i] = (float)load_elem<DT>(u.ktail, i);
      for (int i = tid; i < GQA * kDim; i += 256) tq[i] = load_elem<DT>(q, hrow0 * kDim + i);
      lds_barrier();
      if (tok >= Tp && tok < len) {
        const float* kr = tkey + (tok - Tp) * kDim;
        double acc[GQA];
#pragma unroll
        for (int hh = 0; hh < GQA; ++hh) acc[hh] = 0.0;
        for (int c = 0; c < kDim; ++c) {
          const double kv = (double)kr[c];
#pragma unroll
          for (int hh = 0; hh < GQA; ++hh) acc[hh] = fma(tq[hh * kDim + c], kv, acc[hh]);
        }
#pragma unroll
        for (int hh = 0; hh < GQA; ++hh) sv[hh] = __dmul_rn(acc[hh], kInvSqrt128);
      } else if (tok >= len) {
#pragma unroll
        for (int hh = 0; hh < GQA; ++hh) sv[hh] = -INFINITY;
      }
    }
    // ---- 3. tile max and sum of exp per head; the logits out ----
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) {
      const double m = wave_max(sv[hh]);
      if (lane == 0) redm[wv][hh] = m;
    }
    lds_barrier();
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) {
      const double mt = fmax(fmax(redm[0][hh], redm[1][hh]), fmax(redm[2][hh], redm[3][hh]));
      double e = 0.0;
      if (tok < len) {
        e = exp_nonpos(sv[hh] - mt);
        reinterpret_cast<double*>(ebuf)[(hrow0 + hh) * capmax + tok] = qbad ? __builtin_nan("") : sv[hh];
      }
      const double z = wave_sum(e);
      if (lane == 0) redz[wv][hh] = z;
    }
    lds_barrier();
    if (tid < GQA) {
      const double mt = fmax(fmax(redm[0][tid], redm[1][tid]), fmax(redm[2][tid], redm[3][tid]));
      double* tp = tilepart + ((hrow0 + tid) * ntile_ws + tile) * 2;
      tp[0] = qbad ? __builtin_nan("") : mt;
      tp[1] = qbad ? __builtin_nan("") : (redz[0][tid] + redz[1][tid]) + (redz[2][tid] + redz[3][tid]);
    }
  }
}

// ---------------------------------------------------------------------------
// Gather: a block of 256 threads takes a run of consecutive 128-token chunks
// (4 groups each) of one (request, KV head) and accumulates its share of
//   O_h = sum_j alpha_hj v_hat_j,  alpha_hj = e_hj f_{h,tile(j)}
// (e = exp(s - m_tile), rounded to fp16 for the matrix cores, f_{h,tile} =
// exp(m_tile - m) / Z in fp32).
// Per chunk:
//  1. The chosen value plane rows (16 B per token and plane) sit in LDS as
//     rows[plane][token]; depths, weights and metadata of the chunk too.  All
//     of it was loaded into registers while the previous chunk was computed
//     (the depths one chunk further ahead, as the row loads need them).
//  2. Un-plane: a 16-lane quarter takes one token; one transposing LDS read
//     (ds_read_b64_tr_b8) gives lane o the 8 plane bytes of channel octet o,
//     planes past the token's depth are masked, an 8x8 bit transpose gives
//     the 8 prefix codes X = P 2^(8-t) (depth-0 tokens give zeros), written
//     token-major to a code tile.
//  3. Per group gamma and head h,
//       sum_j e_j v_hat_jc = lo_c A + rng_c (Bh + U_c / 256),
//     A = sum e, Bh = sum e 2^-(t+1), U_c = sum e X_c.  U comes from
//     v_mfma_f32_16x16x32_f16: A operand = codes of 16 channels x 32 tokens
//     (one group), read channel-major from the code tile with the transposing
//     LDS read and turned into the fp16 values 1024 + X by one byte permute
//     per pair; B operand = e for 16 columns (head, group) with zeros off the
//     column's own group; the 1024 A part is removed when the group is
//     folded into the block's running sums (scaled by f of the chunk's tile).
// At the end of the run: column sums per head, the open group's tokens
// (exact values), one partial output per run.  Barriers inside the chunk
// loop wait for LDS traffic only, never for the loads in flight.
// Grid (unit, run): all runs of a unit on one XCD.
// ---------------------------------------------------------------------------
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Lloyd-tree code (LL): the un-planed codes X of a token at depth t become
// the fp16 centroids vtab[t][X] in a channel-major tile (xh), which is the
// MFMA's A operand directly; per group and head
//   sum_j e_j v_hat'_jc = mu_c A + sigma_c U_c,  U_c = sum_j e_j C(t_j, P_jc),
// so the fold uses the channel's calibration (mu, sigma) in place of the
// group's (lo, rng).  The score kept logits s (fp64) in place of the
// exponentials: e = exp(s - m_tile) is formed here (fp32).  The partial
// outputs are in the transformed space; the open group's exact values go to
// otail instead (written by the last run).
// LDS of one gather block, uniform code (members ordered largest first)
template <int GQA, bool LL>
struct GatherShared {
  static constexpr int NG = kChunk / kGroup;  // 4 groups per chunk
  static constexpr int XS = kDim + 16;
  static constexpr int RS = kChunk + 1;
  __attribute__((aligned(16))) uint8_t xl[kChunk * XS];  // codes [token][channel]
  __attribute__((aligned(16))) uint4 rows[8 * RS];        // [plane][token]; reused at the end
  uint32_t vmeta_s[NG][kDim + 1];
  __attribute__((aligned(16))) _Float16 es[GQA][kChunk + 8];
  __attribute__((aligned(4))) uint8_t tvs[kChunk];
  float Ag[NG][GQA], Bg[NG][GQA];
  float fs[GQA];
  __attribute__((aligned(16))) _Float16 ezero[8];         // a zero weight operand
  // (Lloyd code only)
  __attribute__((aligned(16))) _Float16 xh[8];
  _Float16 vts[1];
  float mus[1], sgs[1];
};

// Lloyd code: reconstructed values in fp16 instead of codes, the value
// table, the calibration arrays; no group metadata
template <int GQA>
struct GatherShared<GQA, true> {
  static constexpr int NG = kChunk / kGroup;
  static constexpr int RS = kChunk + 1;
  static constexpr int XHS = kChunk;
  __attribute__((aligned(16))) _Float16 xh[kDim * XHS];
  __attribute__((aligned(16))) uint4 rows[8 * RS];
  _Float16 vts[512];                  // value centroids, compacted per depth
  __attribute__((aligned(16))) _Float16 es[GQA][kChunk + 8];
  float mus[kDim], sgs[kDim];
  __attribute__((aligned(4))) uint8_t tvs[kChunk];
  float Ag[NG][GQA], Bg[NG][GQA];
  float fs[GQA];
  __attribute__((aligned(16))) _Float16 ezero[8];
  // (uniform code only)
  __attribute__((aligned(16))) uint8_t xl[16];
  uint32_t vmeta_s[1][kDim + 1];
};

template <int GQA, int DT, bool LL>
__device__ __forceinline__ void gather_block(GatherShared<GQA, LL>& sh, const VBlock& vb,
    const uint8_t* store, int ub0, const uint8_t* tv, int H, int G, int W, int64_t capmax,
    int ntile_ws, int nrun_ws, const uint32_t* ebuf, const double* ftile, float* opart,
    const uint8_t* cblk, float* otail, const double* tilepart) {
  constexpr int esize = DT == 0 ? 2 : 4;
  constexpr int NG = kChunk / kGroup;                  // 4 groups per chunk
  constexpr int GS = (16 / GQA < NG) ? 16 / GQA : NG;  // groups per MFMA column set
  constexpr int NSET = (NG + GS - 1) / GS;
  // code-tile row stride 144 B (36 words): the 8 rows an MFMA operand read
  // touches start 4 banks apart
  constexpr int XS = kDim + 16;
  // plane-row stride kChunk + 1 chunks: the 8 planes a transposing read
  // touches start 4 banks apart (an unpadded 2 KB stride puts them all on
  // the same banks)
  constexpr int RS = kChunk + 1;
  constexpr int MPT = NG * kDim / 256;  // metadata words per thread
  auto& rows = sh.rows;
  auto& xl = sh.xl;
  // rows padded so that the heads' weight rows (es) and the groups'
  // metadata rows (vmeta_s) read by one MFMA fold start on different banks
  auto& es = sh.es;
  auto& vmeta_s = sh.vmeta_s;
  auto& Ag = sh.Ag;
  auto& Bg = sh.Bg;
  auto& tvs = sh.tvs;
  auto& fs = sh.fs;
  auto& ezero = sh.ezero;
  // Lloyd code: centroid tile [channel][token] (8-token blocks XOR-swizzled
  // per row, see xh_at), the fp16 table, mu and sigma
  constexpr int XHS = kChunk;
  auto& xh = sh.xh;
  auto& vts = sh.vts;
  auto& mus = sh.mus;
  auto& sgs = sh.sgs;

  const int ux = ub0 + vb.x;
  const int b = ux / G, g = ux % G;
  const ReqRecord r = req_of(store, b);
  const int64_t len = r.len;
  const int64_t Tp = len & ~(int64_t)(kGroup - 1);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t hrow0 = (int64_t)b * H + (int64_t)g * GQA;
  const int nch = (int)((len + kChunk - 1) / kChunk);
  const int cb = (int)(((int64_t)vb.y * nch) / vb.ny);
  const int ce = (int)(((int64_t)(vb.y + 1) * nch) / vb.ny);
  if (cb >= ce) {  // empty run: its partial output is zero
    for (int o = tid; o < GQA * kDim; o += 256) {
      opart[((hrow0 + o / kDim) * nrun_ws + vb.y) * kDim + o % kDim] = 0.f;
      if (LL && vb.y == vb.ny - 1) otail[hrow0 * kDim + o] = 0.f;
    }
    return;
  }
  const Unit u = unit_of(const_cast<uint8_t*>(store), r, g, G, kDim, W, esize);
  const uint8_t* tvu = tv + ((int64_t)b * G + g) * capmax;
  if (tid < 4) reinterpret_cast<uint32_t*>(ezero)[tid] = 0u;  // read after the first barrier
  // element (row, token j) of the centroid tile: block j / 8 of the row is
  // stored at block (j / 8) ^ f(row), f(row) = (row / 8) ^ 2 (row % 8), so
  // that the un-plane's stores (16 rows 8 apart) and the MFMA operand reads
  // (16 consecutive rows) each touch 16 different 16-byte blocks
  auto xh_at = [](int row, int j) __attribute__((always_inline)) -> int {
    const int f = ((row >> 3) & 15) ^ ((row & 7) << 1);
    return row * XHS + ((((j >> 3) ^ f) << 3) | (j & 7));
  };
  if constexpr (LL) {  // (read after the first barrier)
    const CodecLayout CL = codec_layout(G, kDim);
    const _Float16* vt = reinterpret_cast<const _Float16*>(cblk + CL.vtab);
    // the table compacted per depth: cell P of depth t at (2^t - 1) + P
    // (a depth's cells contiguous, so that a lookup's distinct entries
    // spread over the banks)
    for (int i = tid; i < 511; i += 256) {
      const int t = 31 - __builtin_clz(i + 1), P = i + 1 - (1 << t);
      vts[i] = vt[256 * t + (P << (8 - t))];
    }
    if (tid < kDim) {
      mus[tid] = reinterpret_cast<const float*>(cblk + CL.muv)[g * kDim + tid];
      sgs[tid] = reinterpret_cast<const float*>(cblk + CL.sigv)[g * kDim + tid];
    }
  }
  // row loads: plane pl of tokens tq .. tq + 3, so that the 8 lanes of a
  // token read its 128-byte row (all planes) together and one load
  // instruction covers 8 whole rows
  const int tq = 4 * (tid >> 3), pl = tid & 7;

  // ---- register prefetch of one chunk ----
  uint32_t pes[GQA];  // encoded e of token tid (tid < kChunk) per head
  double pls[GQA], pmt[GQA];  // Lloyd code: its logit and its tile's maximum
  uint32_t pmeta[MPT];
  double pfs = 0.0;  // converted when stored: no wait right after its load
  uint4 prow[4];     // plane pl of tokens tq .. tq + 3
  // Buffer loads whose range check supplies the zeros past the data (offset
  // kBufOff lies outside every buffer): no branches around the loads.
  const __amdgpu_buffer_rsrc_t rs_tv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(tvu), (short)0, (int)Tp, kBufWord3);
  const __amdgpu_buffer_rsrc_t rs_meta = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(u.vmeta), (short)0, (int)(Tp / kGroup) * kDim * 4, kBufWord3);
  const __amdgpu_buffer_rsrc_t rs_ft = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<double*>(ftile + hrow0 * ntile_ws), (short)0, GQA * ntile_ws * 8, kBufWord3);
  // the depths of tokens tq .. tq + 3 (one byte each; Tp is a multiple of
  // 32, so the four are all inside the buffer or all past it)
  auto tv_of = [&](int chunk) __attribute__((always_inline)) -> uint32_t {
    return __builtin_amdgcn_raw_buffer_load_b32(rs_tv, chunk * kChunk + tq, 0, 0);
  };
  auto load_small = [&](int chunk) __attribute__((always_inline)) {
    const int c0 = chunk * kChunk;
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) {
      if constexpr (LL) {
        const __amdgpu_buffer_rsrc_t rs_e = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t*>(ebuf) + (hrow0 + hh) * capmax * 2, (short)0, (int)len * 8, kBufWord3);
        pls[hh] = __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(
                                                 rs_e, tid < kChunk ? (c0 + tid) * 8 : kBufOff, 0, 0));
        pmt[hh] = tilepart[((hrow0 + hh) * ntile_ws + c0 / kTile) * 2];
      } else {
        const __amdgpu_buffer_rsrc_t rs_e = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t*>(ebuf + (hrow0 + hh) * capmax), (short)0, (int)len * 4, kBufWord3);
        pes[hh] = __builtin_amdgcn_raw_buffer_load_b32(rs_e, tid < kChunk ? (c0 + tid) * 4 : kBufOff, 0, 0);
      }
    }
    if constexpr (!LL) {
#pragma unroll
      for (int k = 0; k < MPT; ++k)
        pmeta[k] = __builtin_amdgcn_raw_buffer_load_b32(rs_meta, ((c0 / kGroup) * kDim + k * 256 + tid) * 4, 0, 0);
    }
    pfs = __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(
                                         rs_ft, tid < GQA ? (tid * ntile_ws + c0 / kTile) * 8 : kBufOff, 0, 0));
  };
  auto load_rows = [&](int chunk, uint32_t t4) __attribute__((always_inline)) {
    // buffer loads over the chunk's plane rows: planes past the depth take
    // an offset beyond the buffer's size, which reads zeros without a
    // memory access, so a token costs only the lines its prefix touches
    // (nothing at depth 0)
    const uint8_t* cbase = reinterpret_cast<const uint8_t*>(u.vplanes) + (int64_t)chunk * kChunk * W * 16;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(cbase), (short)0, kChunk * W * 16, kBufWord3);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t t = (t4 >> (8 * r)) & 0xFFu;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(
          rs, (uint32_t)pl < t ? ((tq + r) * W + pl) * 16 : kBufOff, 0, 0);
      prow[r] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  auto store_chunk = [&](uint32_t t4) __attribute__((always_inline)) {
    if (pl == 0) *reinterpret_cast<uint32_t*>(&tvs[tq]) = t4;
    if (tid < kChunk) {
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) {
        if constexpr (LL) es[hh][tid] = (_Float16)__expf((float)(pls[hh] - pmt[hh]));
        else es[hh][tid] = to_half(dec_e(pes[hh]));
      }
    }
    if constexpr (!LL) {
#pragma unroll
      for (int k = 0; k < MPT; ++k) {
        const int i = k * 256 + tid;
        vmeta_s[i / kDim][i % kDim] = pmeta[k];
      }
    }
    if (tid < GQA) fs[tid] = (float)pfs;
    // (rows past a token's depth hold zeros)
#pragma unroll
    for (int r = 0; r < 4; ++r) rows[pl * RS + tq + r] = prow[r];
  };

  // depths of tokens tq .. tq + 3: tA of the chunk whose rows are in
  // flight, tB of the next one (loaded a chunk ahead); the loop runs two
  // chunks per turn with the roles swapped, so a depth load never has to
  // land in another register
  uint32_t tA = tv_of(cb), tB = tv_of(cb + 1);  // past the run: unused
  load_small(cb);
  load_rows(cb, tA);

  const int m = lane & 15, kb = lane >> 4;
  const int gp = m / GQA, hn = m % GQA;
  const bool colv = m < GS * GQA;
  float Oacc[2][4];
#pragma unroll
  for (int bl = 0; bl < 2; ++bl)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) Oacc[bl][rr] = 0.f;
  const int q4 = lane >> 4, L = lane & 15;
  // transposing plane read: lane 2e + s of a quarter addresses plane 7 - e,
  // bytes 8s .. 8s + 7 of the quarter's token row; lane L then holds the
  // plane bytes of channel octet L
  const int troff = (7 - (L >> 1)) * (RS * 16) + 8 * (L & 1);

  auto chunk_step = [&](int chunk, uint32_t& tcur, uint32_t& tnext) __attribute__((always_inline)) {
    set_progress_priority(chunk - cb, ce - cb);
    const int64_t c0 = (int64_t)chunk * kChunk;
    const int64_t gam0 = c0 / kGroup;
    store_chunk(tcur);
    lds_barrier();
    // next chunk's loads go out now and land while this one is computed
    if (chunk + 1 < ce) {
      load_small(chunk + 1);
      load_rows(chunk + 1, tnext);
      tcur = tv_of(chunk + 2);  // tcur is free once stored
    }
    // per-group sums of e (A) and of e 2^-(t+1) (Bh): TPP threads per
    // (group, head), each over 32/TPP tokens, then a shuffle reduction
    {
      constexpr int NP = NG * GQA;
      constexpr int TPP = NP <= 8 ? 32 : (NP <= 16 ? 16 : (NP <= 32 ? 8 : 4));
      constexpr int TK = kGroup / TPP;
      const int pr = tid / TPP, part = tid % TPP;
      float a = 0.f, bh = 0.f;
      if (pr < NP) {
        const int gl = pr / GQA, hh = pr % GQA;
#pragma unroll
        for (int k = 0; k < TK; ++k) {
          const int j = kGroup * gl + part * TK + k;
          const float e = (float)es[hh][j];
          a += e;
          bh = fmaf(e, ldexp_pow2f(-(int)tvs[j] - 1), bh);
        }
      }
      a = group_sum<TPP>(a);
      bh = group_sum<TPP>(bh);
      if (pr < NP && part == 0) {
        // with the tile factor f folded in: f A and f (Bh - 4 A) (the codes
        // reach the MFMA as 1024 + X, whose 1024 part is f 4 A after the
        // 1/256 scale)
        const float f = fs[pr % GQA], fa = f * a;
        Ag[pr / GQA][pr % GQA] = fa;
        Bg[pr / GQA][pr % GQA] = fmaf(f, bh, -4.f * fa);
      }
    }
    // ---- un-plane: wave w, step i -> tokens 32 w + 4 i + quarter.  The
    // rows of planes past a token's depth were loaded as zeros, so the
    // codes need no mask; the deepest of the 4 tokens (a scalar) picks the
    // transpose (at most 4 planes: the upper half only) ----
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int j0 = 32 * wv + 4 * it;
      const uint32_t t4 = (uint32_t)__builtin_amdgcn_readfirstlane(
          (int)*reinterpret_cast<const uint32_t*>(&tvs[j0]));  // the 4 tokens' depths
      // all four depths <= 4 (depths are <= 8: adding 123 sets bit 7 of a
      // byte exactly when it is >= 5, with no carry between bytes)
      const bool shallow = ((t4 + 0x7B7B7B7Bu) & 0x80808080u) == 0u;
      const int j = j0 + q4;
      const long v = tr8_read(reinterpret_cast<const uint8_t*>(rows) + j * 16 + troff);
      const uint2 pb = __builtin_bit_cast(uint2, v);
      uint32_t lo = pb.x, hi = pb.y;
      if (shallow) transpose8_hi4(lo, hi);
      else transpose8_halves(lo, hi);
      if constexpr (LL) {
        const uint32_t tj = tvs[j];
        const int tb = (1 << tj) - 1;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t X = ((i < 4 ? lo : hi) >> (8 * (i & 3))) & 0xFFu;
          xh[xh_at(8 * L + i, j)] = vts[tb + (int)(X >> (8u - tj))];
        }
      } else {
        *reinterpret_cast<uint2*>(xl + j * XS + 8 * L) = make_uint2(lo, hi);
      }
    }
    lds_barrier();

    // ---- MFMA per (16-channel block, column set); wave w: blocks 2w, 2w+1 ----
    // closed groups of the chunk (a scalar); the weight operand of group gi
    // is the same for both channel blocks, so it is read once, from a zero
    // block for the lanes whose column belongs to another group
    const int ngc = (int)min(max((Tp - c0) / kGroup, (int64_t)0), (int64_t)NG);
    for (int set = 0; set < NSET; ++set) {
      const int gbase = set * GS;
      f16x8 bvs[GS];
#pragma unroll
      for (int gi = 0; gi < GS; ++gi) {
        const int gl = gbase + gi;
        const bool mine = colv && gp == gi && gl < NG;
        const _Float16* src = mine ? &es[hn][kGroup * gl + 8 * kb] : ezero;
        bvs[gi] = *reinterpret_cast<const f16x8*>(src);
      }
#pragma unroll
      for (int bl = 0; bl < 2; ++bl) {
        const int cbk = 16 * (2 * wv + bl);
        f32x4 D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int gi = 0; gi < GS; ++gi) {
          const int gl = gbase + gi;
          if (gl >= ngc) break;
          const int t0 = kGroup * gl + 8 * kb;
          f16x8 av;
          if constexpr (LL) {
            av = *reinterpret_cast<const f16x8*>(&xh[xh_at(cbk + m, t0)]);
          } else {
            const uint2 xv = __builtin_bit_cast(uint2, tr8_read(xl + (t0 + (m >> 1)) * XS + cbk + 8 * (m & 1)));
            uint32_t ap[4];
            ap[0] = __builtin_amdgcn_perm(0x64646464u, xv.x, 0x04010400u);
            ap[1] = __builtin_amdgcn_perm(0x64646464u, xv.x, 0x04030402u);
            ap[2] = __builtin_amdgcn_perm(0x64646464u, xv.y, 0x04010400u);
            ap[3] = __builtin_amdgcn_perm(0x64646464u, xv.y, 0x04030402u);
            av = __builtin_bit_cast(f16x8, ap);
          }
          D = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bvs[gi], D, 0, 0, 0);
        }
        // fold: D row = channel cbk + 4 kb + rr, column m = (gp, hn)
        const int gl = gbase + gp;
        if (colv && gl < ngc) {
          if constexpr (LL) {
            const float fA = Ag[gl][hn], fD = fs[hn];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int c = cbk + 4 * kb + rr;
              Oacc[bl][rr] = fmaf(sgs[c], D[rr] * fD, fmaf(mus[c], fA, Oacc[bl][rr]));
            }
          } else {
            const float fA = Ag[gl][hn], fB = Bg[gl][hn], fD = fs[hn] * (1.f / 256.f);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const uint32_t mt = vmeta_s[gl][cbk + 4 * kb + rr];
              const float lo = bf16_to_float(mt & 0xFFFFu), rng = bf16_to_float(mt >> 16);
              Oacc[bl][rr] = fmaf(rng, fmaf(D[rr], fD, fB), fmaf(lo, fA, Oacc[bl][rr]));
            }
          }
        }
      }
    }
    lds_barrier();
  };
  for (int chunk = cb; chunk < ce; chunk += 2) {
    chunk_step(chunk, tA, tB);
    if (chunk + 1 >= ce) break;
    chunk_step(chunk + 1, tB, tA);
  }

  // ---- column sums per head, open group, partial output of the run ----
  float* red2 = reinterpret_cast<float*>(rows);  // [16 columns][128 channels]
#pragma unroll
  for (int bl = 0; bl < 2; ++bl)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) red2[m * kDim + 16 * (2 * wv + bl) + 4 * kb + rr] = Oacc[bl][rr];
  lds_barrier();
  const int64_t cl0 = (int64_t)(ce - 1) * kChunk;  // the last chunk (es, fs still in LDS)
  const int64_t jt0 = Tp > cl0 ? Tp : cl0;
  const int64_t jt1 = len < cl0 + kChunk ? len : cl0 + kChunk;
  for (int o = tid; o < GQA * kDim; o += 256) {
    const int hh = o / kDim, c = o % kDim;
    float s = 0.f;
    for (int qq = 0; qq < GS; ++qq) s += red2[(qq * GQA + hh) * kDim + c];
    float st = 0.f;
    for (int64_t j = jt0; j < jt1; ++j)
      st = fmaf((float)es[hh][j - cl0], load_elem_f<DT>(u.vtail, (j - Tp) * kDim + c), st);
    if constexpr (LL) {
      opart[((hrow0 + hh) * nrun_ws + vb.y) * kDim + c] = s;
      if (vb.y == vb.ny - 1) otail[(hrow0 + hh) * kDim + c] = st * fs[hh];
    } else {
      opart[((hrow0 + hh) * nrun_ws + vb.y) * kDim + c] = fmaf(st, fs[hh], s);
    }
  }
}

// The gather launch: one block per (unit, run); four blocks per compute
// unit where the registers allow it (the uniform code's LDS does).
template <int GQA, int DT, bool LL>
__global__ __launch_bounds__(256, (LL || GQA > 4) ? 2 : 4) void k_gather(
    const uint8_t* store, int ub0, const uint8_t* tv, int H, int G, int W, int64_t capmax,
    int ntile_ws, int nrun_ws, const uint32_t* ebuf, const double* ftile, float* opart,
    const uint8_t* cblk, float* otail, const double* tilepart) {
  __shared__ GatherShared<GQA, LL> sh;
  gather_block<GQA, DT, LL>(sh, launch_block(), store, ub0, tv, H, G, W, capmax, ntile_ws, nrun_ws,
                            ebuf, ftile, opart, cblk, otail, tilepart);
}

// out[b][h][c] = sum over the unit's runs, in run order, for output element
// o = (b H + h) d + c.
__device__ __forceinline__ void out_reduce_elem(int64_t o, int nrun, int nrun_ws, const float* opart,
                                                float* out) {
  const int64_t bh = o / kDim;
  const int c = (int)(o - bh * kDim);
  const float* p = opart + bh * nrun_ws * kDim + c;
  float s = 0.f;
  int k = 0;
  // eight loads in flight at a time, summed in run order
  for (; k + 8 <= nrun; k += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[(int64_t)(k + i) * kDim];
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[i];
  }
  for (; k < nrun; ++k) s += p[(int64_t)k * kDim];
  out[o] = s;
}

// one thread per output element
__global__ __launch_bounds__(256) void k_out_reduce(int nrun, int nrun_ws, int64_t nout,
                                                    const float* opart, float* out) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (o < nout) out_reduce_elem(o, nrun, nrun_ws, opart, out);
}

// Lloyd code: one block of d_h threads per (request, query head): the run
// partials summed in run order (transformed space), then
//   o = U_V^T o' + o_open = s_V . (H o') / sqrt(d) + o_open
// with in-place Walsh-Hadamard butterflies over the block (fp32).
__global__ __launch_bounds__(kDim) void k_out_reduce_lloyd(int nrun, int nrun_ws, const float* opart,
                                                           const float* otail, const uint8_t* cb,
                                                           int G, float* out) {
  __shared__ float y[kDim];
  const int64_t bh = blockIdx.x;
  const int c = threadIdx.x;
  const float* p = opart + bh * nrun_ws * kDim + c;
  float s = 0.f;
  int k = 0;
  for (; k + 8 <= nrun; k += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[(int64_t)(k + i) * kDim];
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[i];
  }
  for (; k < nrun; ++k) s += p[(int64_t)k * kDim];
  y[c] = s;
  __syncthreads();
  for (int h = 1; h < kDim; h <<= 1) {
    const float a = y[c], o = y[c ^ h];
    __syncthreads();
    y[c] = (c & h) ? o - a : a + o;
    __syncthreads();
  }
  const double sv = reinterpret_cast<const double*>(cb + codec_layout(G, kDim).sv)[c];
  out[bh * kDim + c] = y[c] * ((float)kInvSqrt128 * (float)sv) + otail[bh * kDim + c];
}

// ---------------------------------------------------------------------------
// Single-launch reader ([ReadKV] Sec. 7 names fusing the reader's launches
// as the way to close its latency gap).  One cooperative launch of as many
// 256-thread blocks as fit on the chip at once walks the grids of the split
// path's launches in turn, a grid-wide barrier standing where a launch
// boundary stood:
//   score, key allocation in the block prologue   (units x score runs)
//   value allocation of a unit in one block       (units; capacities up to
//     16,384 tokens), or value weights            (units x 1024-token chunks)
//     then value selection                        (units)
//   value gather                                  (units x gather runs)
//   output reduction                              (B H d / 256)
// Every stage runs the block code of its own launch; the score and gather
// split each unit's tiles and chunks over (blocks / units) runs.  Key and
// value depths and read counters are the split path's exactly; outputs
// differ from it only in the order the gather runs' partial sums are added.
// Uniform code, per-KV-head budgets, at most as many units as blocks.  LDS:
// one dynamic region holding the current stage's block state (the score's
// staged key planes after it).
// ---------------------------------------------------------------------------
constexpr int kFusedSelNT = 256;

struct FusedArgs {
  const uint8_t* store;
  const void* q;
  uint8_t* tk;
  uint8_t* tv;
  uint32_t* ebuf;
  double* tilepart;
  double* ftile;
  double* aval;
  float* opart;
  float* out;
  uint64_t* counters;
  float RK, RV;
  int H, G, W, esize, vscale, min1, pairs;
  int nunits, nrun, nch, nrun_g, ntile_ws, nchunk_ws;
  int unit_alloc;  // 1: the unit's value allocation in one block (capacity <= kVSelLocal)
  int reserved;
  int64_t capmax, nout;
};

template <int GQA>
constexpr size_t fused_planes_offset() {
  return (sizeof(ScoreShared<GQA>) + 15) / 16 * 16;
}

// The score and gather stages give each block at most one of their blocks:
// a loop around their block code would keep its loop-invariant values in
// registers across the iterations and spill.
// The launch's arguments, read afresh from the kernel-argument segment by
// each stage: the pointer passes through an empty asm statement, so that no
// stage's arguments stay in registers through the other stages.
typedef const FusedArgs __attribute__((address_space(4)))* fused_args_ptr;
__device__ __forceinline__ fused_args_ptr fused_args() {
  fused_args_ptr p = (fused_args_ptr)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return p;
}

template <int GQA, int DT>
__global__ __launch_bounds__(256, GQA <= 4 ? 3 : 2) void k_reader_fused(FusedArgs) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  cooperative_groups::grid_group grid = cooperative_groups::this_grid();
  const int nb = (int)gridDim.x;
  const int bid = (int)blockIdx.x;
  if (const auto A = fused_args(); bid < A->nunits * A->nrun) {
    auto& sh = *reinterpret_cast<ScoreShared<GQA>*>(lds);
    uint32_t* const planes = reinterpret_cast<uint32_t*>(lds + fused_planes_offset<GQA>());
    score_block<GQA, DT>(sh, planes, VBlock{bid % A->nunits, bid / A->nunits, A->nunits, A->nrun},
                         A->store, 0, A->q, A->tk, 0, A->min1, A->H, A->G, A->W, A->RK, A->capmax,
                         A->ntile_ws, A->ebuf, A->tilepart, A->counters);
  }
  grid.sync();
  if (fused_args()->unit_alloc) {
    // capacities up to 16,384 tokens: the value allocation of a unit in one
    // block, its weights kept in the workspace (read back by the same block)
    const auto A = fused_args();
    auto& sh = *reinterpret_cast<ValueAllocUnitShared<kFusedSelNT, GQA>*>(lds);
    for (int v = bid; v < A->nunits; v += nb) {
      value_alloc_unit_block<kFusedSelNT, GQA, false, true>(
          sh, A->aval + (int64_t)v * A->capmax, VBlock{v, 0, A->nunits, 1}, A->store, 0, A->H, A->G,
          A->W, A->esize, A->vscale, A->RV, A->min1, A->pairs, A->capmax, A->ntile_ws, A->ebuf,
          A->tilepart, A->ftile, A->tv, A->tk, A->counters, nullptr);
      __syncthreads();
    }
  } else {
    {
      const auto A = fused_args();
      auto& sh = *reinterpret_cast<ValueWeightsShared<GQA>*>(lds);
      for (int v = bid; v < A->nunits * A->nch; v += nb) {
        value_weights_block<GQA, false>(sh, VBlock{v % A->nunits, v / A->nunits, A->nunits, A->nch},
                                        A->store, 0, A->H, A->G, A->W, A->esize, A->vscale,
                                        A->capmax, A->ntile_ws, A->ebuf, A->tilepart, A->ftile,
                                        A->aval, nullptr);
        __syncthreads();
      }
    }
    grid.sync();
    {
      const auto A = fused_args();
      auto& sh = *reinterpret_cast<ValueSelectShared<kFusedSelNT>*>(lds);
      for (int v = bid; v < A->nunits; v += nb) {
        value_select_block<kFusedSelNT, false, false>(sh, nullptr, VBlock{v, 0, A->nunits, 1},
                                                      A->store, 0, A->G, A->W, A->esize, A->RV, 1,
                                                      A->min1, A->pairs, A->capmax, A->aval, A->tv,
                                                      A->tk, A->counters, nullptr);
        __syncthreads();
      }
    }
  }
  grid.sync();
  if (const auto A = fused_args(); bid < A->nunits * A->nrun_g) {
    auto& sh = *reinterpret_cast<GatherShared<GQA, false>*>(lds);
    gather_block<GQA, DT, false>(sh, VBlock{bid % A->nunits, bid / A->nunits, A->nunits, A->nrun_g},
                                 A->store, 0, A->tv, A->H, A->G, A->W, A->capmax, A->ntile_ws, A->nchunk_ws,
                                 A->ebuf, A->ftile, A->opart, nullptr, nullptr, nullptr);
  }
  grid.sync();
  const auto A = fused_args();
  for (int64_t o = (int64_t)bid * 256 + threadIdx.x; o < A->nout; o += (int64_t)nb * 256)
    out_reduce_elem(o, A->nrun_g, A->nchunk_ws, A->opart, A->out);
}

// ---------------------------------------------------------------------------
static int device_cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

static inline void mark(const DecodeArgs& a, int i, hipStream_t st) {
  if (a.events) hipEventRecord((hipEvent_t)a.events[i], st);
}

// Dynamic LDS of a score block: the key-line segments staged per tile, at
// most min(B_K of the domain, 128 W) chosen segments of one unit, 32 B each
// (+8 slots: un-plane reads of a batch may run past a shallower channel's
// last slot; those words are masked).  NU: KV heads per selection domain.
static size_t score_planes_bytes(const DecodeArgs& a, int NU) {
  double bk = floor((double)a.RK * (double)(kDim * NU));
  if (a.min1 && bk < (double)kDim) bk = (double)kDim;  // every channel at depth >= 1
  if (bk > (double)(kDim * a.W)) bk = (double)(kDim * a.W);
  if (bk < 0.0) bk = 0.0;
  size_t dyn = ((size_t)bk + 8) * 32;
  if (NU == 1 && dyn < 258 * 4) dyn = 258 * 4;  // the key allocation's scratch
  return dyn;
}

// Gather runs per unit: runs of consecutive chunks, about four blocks per
// compute unit over the whole call (37 KB of LDS each).
static int gather_runs(const DecodeArgs& a, const WsLayout& L) {
  const int64_t total = (int64_t)a.B * a.G * L.nchunk;
  const int64_t gslots = 4 * (int64_t)device_cu_count();
  int grun = (int)((total + gslots - 1) / gslots);
  if (grun < 1) grun = 1;
  return (L.nchunk + grun - 1) / grun;
}

// The launches for the units P.ub0 .. P.ub0 + P.nunits - 1 (whole
// requests): key allocation (per-layer budgets), score, value allocation,
// value gather.  The score of the part that starts at unit 0 zeroes the
// read counters.
template <int GQA, int DT>
static int launch_part(const DecodeArgs& a, const WsLayout& L, const Part& P, uint8_t* tk, uint8_t* tv,
                       int nrun_g, hipStream_t st) {
  uint8_t* ws = a.ws;
  const int NU = a.scope == 1 ? a.G : 1;  // KV heads per selection domain
  // per-layer budgets: one key selection per request in its own launch;
  // per-KV-head budgets: inside the score kernel's blocks
  if (NU > 1 && launch_key_alloc(a, P, tk, st)) return -5;
  const size_t dyn = score_planes_bytes(a, NU);
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(&k_score<GQA, DT>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (kDim * 8 + 8) * 32);
    attr_set = true;
  }
  // each unit's tiles split evenly over nrun blocks, as many blocks as fit
  // on the chip at once (three per compute unit at most: two for more than
  // 4 query heads per KV head, or when the staged lines of a large key
  // budget take more LDS)
  const int64_t total_tiles = (int64_t)P.nunits * L.ntile;
  static size_t occ_dyn = 0;
  static int occ_n = 0;
  if (occ_n == 0 || occ_dyn != dyn) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&k_score<GQA, DT>), 256,
                                                     dyn) != hipSuccess || n < 1)
      n = 1;
    occ_n = min(n, GQA <= 4 ? 3 : 2);
    occ_dyn = dyn;
  }
  const int64_t slots = (int64_t)occ_n * device_cu_count();
  int run = (int)((total_tiles + slots - 1) / slots);
  if (run < 1) run = 1;
  const int nrun = (L.ntile + run - 1) / run;
  hipLaunchKernelGGL((k_score<GQA, DT>), dim3(P.nunits, nrun), dim3(256), dyn, st,
                     (const uint8_t*)a.store, P.ub0, a.q, tk, NU > 1 ? 1 : 0, a.min1, a.H, a.G, a.W, a.RK,
                     a.capmax, L.ntile, (uint32_t*)(ws + L.ebuf), (double*)(ws + L.tilepart),
                     P.ub0 == 0 ? a.counters : nullptr);
  if (P.ub0 == 0) mark(a, 1, st);
  if (launch_value_alloc(a, P, L, tk, tv, st)) return -5;
  if (P.ub0 == 0) mark(a, 2, st);
  hipLaunchKernelGGL((k_gather<GQA, DT, false>), dim3(P.nunits, nrun_g), dim3(256), 0, st,
                     (const uint8_t*)a.store, P.ub0, (const uint8_t*)tv, a.H, a.G, a.W, a.capmax,
                     L.ntile, L.nchunk, (const uint32_t*)(ws + L.ebuf), (const double*)(ws + L.ftile),
                     (float*)(ws + L.opart), nullptr, nullptr, nullptr);
  return 0;
}

template <int GQA, int DT>
static int launch_all(const DecodeArgs& a, const WsLayout& L, hipStream_t st) {
  uint8_t* tk = a.key_depths_out ? a.key_depths_out : a.ws + L.tk;
  uint8_t* tv = a.value_depths_out ? a.value_depths_out : a.ws + L.tv;
  const int nrun_g = gather_runs(a, L);
  mark(a, 0, st);
  const Part P{0, a.B * a.G};
  const int rc = launch_part<GQA, DT>(a, L, P, tk, tv, nrun_g, st);
  if (rc) return rc;
  const int64_t nout = (int64_t)a.B * a.H * kDim;
  hipLaunchKernelGGL(k_out_reduce, dim3((unsigned)((nout + 255) / 256)), dim3(256), 0, st, nrun_g,
                     L.nchunk, nout, (const float*)(a.ws + L.opart), a.out);
  mark(a, 3, st);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// The single-launch reader (uniform code, per-KV-head budgets): one
// cooperative launch of as many blocks as fit on the chip at once (units
// beyond that number: unsupported).
template <int GQA, int DT>
static int launch_fused(const DecodeArgs& a, const WsLayout& L, hipStream_t st) {
  if (a.codec != 0 || a.scope != 0) return -5;
  static int coop = -1;
  if (coop < 0) {
    int dev = 0, v = 0;
    coop = (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess && v)
               ? 1
               : 0;
  }
  if (!coop) return -5;
  const void* const kfn = reinterpret_cast<const void*>(&k_reader_fused<GQA, DT>);
  size_t dyn = fused_planes_offset<GQA>() + score_planes_bytes(a, 1);
  dyn = std::max(dyn, sizeof(ValueWeightsShared<GQA>));
  dyn = std::max(dyn, sizeof(ValueSelectShared<kFusedSelNT>));
  dyn = std::max(dyn, sizeof(ValueAllocUnitShared<kFusedSelNT, GQA>));
  dyn = std::max(dyn, sizeof(GatherShared<GQA, false>));
  static bool attr_set = false;
  if (!attr_set) {
    const size_t most = std::max({fused_planes_offset<GQA>() + (size_t)(kDim * 8 + 8) * 32,
                                  sizeof(GatherShared<GQA, false>),
                                  sizeof(ValueAllocUnitShared<kFusedSelNT, GQA>),
                                  sizeof(ValueSelectShared<kFusedSelNT>)});
    if (hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)most) != hipSuccess)
      return -6;
    attr_set = true;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kfn, 256, dyn) != hipSuccess || per_cu < 1)
    return -6;
  const int nunits = a.B * a.G;
  FusedArgs A;
  A.store = (const uint8_t*)a.store;
  A.q = a.q;
  A.tk = a.key_depths_out ? a.key_depths_out : a.ws + L.tk;
  A.tv = a.value_depths_out ? a.value_depths_out : a.ws + L.tv;
  A.ebuf = (uint32_t*)(a.ws + L.ebuf);
  A.tilepart = (double*)(a.ws + L.tilepart);
  A.ftile = (double*)(a.ws + L.ftile);
  A.aval = (double*)(a.ws + L.aval);
  A.opart = (float*)(a.ws + L.opart);
  A.out = a.out;
  A.counters = a.counters;
  A.RK = a.RK;
  A.RV = a.RV;
  A.H = a.H;
  A.G = a.G;
  A.W = a.W;
  A.esize = a.dtype == 0 ? 2 : 4;
  A.vscale = a.vscale;
  A.min1 = a.min1;
  A.pairs = a.pairs;
  A.nunits = nunits;
  const int64_t slots = (int64_t)per_cu * device_cu_count();
  if (nunits > slots) return -5;
  // runs per unit: one block each
  const int per_unit = (int)(slots / nunits);
  A.nrun = std::min(per_unit, L.ntile);
  A.nch = (int)((a.capmax + kVChunk - 1) / kVChunk);
  A.unit_alloc = a.capmax <= kVSelLocal ? 1 : 0;
  A.reserved = 0;
  A.nrun_g = std::min(per_unit, L.nchunk);
  A.ntile_ws = L.ntile;
  A.nchunk_ws = L.nchunk;
  A.capmax = a.capmax;
  A.nout = (int64_t)a.B * a.H * kDim;
  // no more blocks than the largest stage has
  int64_t most = std::max<int64_t>((int64_t)nunits * A.nrun, (int64_t)nunits * A.nch);
  most = std::max<int64_t>(most, (int64_t)nunits * A.nrun_g);
  most = std::max<int64_t>(most, (A.nout + 255) / 256);
  const int grid = (int)std::min<int64_t>(slots, most);
  void* args[] = {&A};
  mark(a, 0, st);
  if (hipLaunchCooperativeKernel(kfn, dim3(grid), dim3(256), args, (unsigned)dyn, st) != hipSuccess)
    return -6;
  // (the stages have no events of their own)
  mark(a, 1, st);
  mark(a, 2, st);
  mark(a, 3, st);
  return 0;
}

// Lloyd code: key allocation (own launch, per domain), score, value
// allocation, gather, output reduction with the inverse value transform.
template <int GQA, int DT>
static int launch_all_lloyd(const DecodeArgs& a, const WsLayout& L, hipStream_t st) {
  uint8_t* ws = a.ws;
  uint8_t* tk = a.key_depths_out ? a.key_depths_out : ws + L.tk;
  uint8_t* tv = a.value_depths_out ? a.value_depths_out : ws + L.tv;
  const int nunits = a.B * a.G;
  mark(a, 0, st);
  if (launch_key_alloc_lloyd(a, L, tk, st)) return -5;
  const int64_t total_tiles = (int64_t)nunits * L.ntile;
  const int64_t slots = 3 * (int64_t)device_cu_count();
  int run = (int)((total_tiles + slots - 1) / slots);
  if (run < 1) run = 1;
  const int nrun = (L.ntile + run - 1) / run;
  hipLaunchKernelGGL((k_score_lloyd<GQA, DT>), dim3(nunits, nrun), dim3(256), 0, st,
                     (const uint8_t*)a.store, a.cblock, a.q, (const uint8_t*)tk,
                     (const double*)(ws + L.qp), (const double*)(ws + L.qb), a.H, a.G, a.W, a.capmax,
                     L.ntile, (uint32_t*)(ws + L.ebuf), (double*)(ws + L.tilepart));
  mark(a, 1, st);
  const Part P{0, nunits};
  if (launch_value_alloc(a, P, L, tk, tv, st)) return -5;
  mark(a, 2, st);
  const int64_t total = (int64_t)nunits * L.nchunk;
  const int64_t gslots = 4 * (int64_t)device_cu_count();
  int grun = (int)((total + gslots - 1) / gslots);
  if (grun < 1) grun = 1;
  const int nrun_g = (L.nchunk + grun - 1) / grun;
  hipLaunchKernelGGL((k_gather<GQA, DT, true>), dim3(nunits, nrun_g), dim3(256), 0, st,
                     (const uint8_t*)a.store, 0, (const uint8_t*)tv, a.H, a.G, a.W, a.capmax,
                     L.ntile, L.nchunk, (const uint32_t*)(ws + L.ebuf), (const double*)(ws + L.ftile),
                     (float*)(ws + L.opart), a.cblock, (float*)(ws + L.otail),
                     (const double*)(ws + L.tilepart));
  hipLaunchKernelGGL(k_out_reduce_lloyd, dim3(a.B * a.H), dim3(kDim), 0, st, nrun_g, L.nchunk,
                     (const float*)(ws + L.opart), (const float*)(ws + L.otail), a.cblock, a.G, a.out);
  mark(a, 3, st);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

template <int DT>
static int dispatch_gqa(const DecodeArgs& a, const WsLayout& L, hipStream_t st) {
  if (a.codec) {
    switch (a.H / a.G) {
      case 1: return launch_all_lloyd<1, DT>(a, L, st);
      case 2: return launch_all_lloyd<2, DT>(a, L, st);
      case 3: return launch_all_lloyd<3, DT>(a, L, st);
      case 4: return launch_all_lloyd<4, DT>(a, L, st);
      case 5: return launch_all_lloyd<5, DT>(a, L, st);
      case 6: return launch_all_lloyd<6, DT>(a, L, st);
      case 7: return launch_all_lloyd<7, DT>(a, L, st);
      case 8: return launch_all_lloyd<8, DT>(a, L, st);
      default: return -5;
    }
  }
  if (a.fused) {
    switch (a.H / a.G) {
      case 1: return launch_fused<1, DT>(a, L, st);
      case 2: return launch_fused<2, DT>(a, L, st);
      case 3: return launch_fused<3, DT>(a, L, st);
      case 4: return launch_fused<4, DT>(a, L, st);
      case 5: return launch_fused<5, DT>(a, L, st);
      case 6: return launch_fused<6, DT>(a, L, st);
      case 7: return launch_fused<7, DT>(a, L, st);
      case 8: return launch_fused<8, DT>(a, L, st);
      default: return -5;
    }
  }
  switch (a.H / a.G) {
    case 1: return launch_all<1, DT>(a, L, st);
    case 2: return launch_all<2, DT>(a, L, st);
    case 3: return launch_all<3, DT>(a, L, st);
    case 4: return launch_all<4, DT>(a, L, st);
    case 5: return launch_all<5, DT>(a, L, st);
    case 6: return launch_all<6, DT>(a, L, st);
    case 7: return launch_all<7, DT>(a, L, st);
    case 8: return launch_all<8, DT>(a, L, st);
    default: return -5;
  }
}

int launch_decode(const DecodeArgs& a, hipStream_t st) {
  const WsLayout L = ws_layout(a.B, a.H, a.G, kDim, a.capmax, a.codec);
  return a.dtype == 0 ? dispatch_gqa<0>(a, L, st) : dispatch_gqa<1>(a, L, st);
}

}  // namespace readkv
