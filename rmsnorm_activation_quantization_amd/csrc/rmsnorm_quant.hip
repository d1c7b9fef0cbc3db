// rmsnorm_quant.hip -- gfx950 kernels and the C ABI of librmsnorm_quant.so.
//
// The fused step (sglang PR #29723, Motivation / Key changes / Accuracy
// Tests): residual add -> RMSNorm -> quantize, equal to the unfused sequence
// with bf16 tensors between its launches, in ONE pass over HBM:
//   read x, residual (and the L2-resident weight) once, write residual_out,
//   the codes and the scales once.  The row stays in VGPRs from load to store.
// The same kernel template also runs the two launches of the unfused sequence
// (norm alone, quantize alone: a stage parameter), with bit-identical results,
// and takes bf16 or fp16 rows (an element-type parameter).
// The QK variant (sglang PR #27656, Motivation / Modifications): GemmaRMSNorm
// of q and k heads read through their strides plus the gate de-interleave, in
// one launch.
//
// Work mapping (CDNA4: 64-lane waves, 16-byte loads):
//   a lane owns 8 consecutive elements (one 16-byte load per tensor) per
//   "chunk"; the lanes of a row cover 8 * lanes consecutive columns per chunk,
//   so every wave-level load and store is fully coalesced.  A row is spread
//   over WPR waves (1, 2, 4, 8 or 16) of one workgroup, and NC = chunks per
//   lane is a template parameter, so the row lives in registers from load to
//   store and is never re-read.  For many rows the host picks WPR so that a
//   lane holds at most two chunks: few registers, hence up to 8 waves per SIMD
//   in flight, which measured best on MI355X at prefill sizes (a wave per row
//   with the row in 115 VGPRs ran at 68 % of HBM peak, a workgroup per row at
//   74 %).  For a decode batch, which cannot fill the chip, it picks one chunk
//   per lane (more waves per row, a shorter chain per lane).  Waves of a row
//   combine their partial sums and maxima through LDS with one barrier each;
//   the row's sum of squares is added up in one order whatever the tiling, so
//   a row gives the same bits in any batch.
// Reductions: the sum of squares over the row, and max |y| per token, per
// group or per 32-element block, use DPP row operations inside 16-lane rows,
// a swizzle across rows and readlane across wave halves.  Every butterfly step
// is symmetric, so every lane ends with the bit-identical result.
//
// Arithmetic (matches the oracle's definition exactly except rstd, which is
// fp32 here):
//   residual_out = round(f32(x) + f32(res))   exact: the fp32 sum of two bf16
//                  (fp16) values rounded to bf16 (fp16) is the correctly
//                  rounded sum (24 >= 2*8 + 2 and 24 >= 2*11 + 2, so the
//                  double rounding is innocuous).
//   ss = sum of r^2 in fp32; rstd = rsq(ss * (1/H) + eps) (hardware
//        reciprocal square root; the oracle's rstd is fp64, and y may differ
//        by one ulp where r * rstd * w lies next to a rounding boundary).
//   y = round((r * rstd) * w), to nearest even.
//   FP8: scale = amax / 448 exactly (IEEE-equal); the quotient y / scale is
//        formed with the correctly rounded reciprocal of the scale and one
//        Markstein correction (q0 = y*inv, e = scale*q0 - y, q = q0 - e*inv),
//        which equals the IEEE fp32 quotient for every bf16 or fp16 y and
//        fp32 scale >= 2^-64 (checked exhaustively on the host by the test
//        suite); the hardware converter then rounds to E4M3FN (nearest-even).
//   MXFP4: E8M0 byte from the fp32 exponent of amax; the hardware converter
//        divides y by the block scale 2^(byte - 127), exactly, and rounds to
//        E2M1 (nearest-even, saturating at 6).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <utility>

#include "rmsnorm_quant.h"

#define RQ_QUOTIENT_QUALIFIERS __device__ __forceinline__
#include "fp8_quotient.h"
#define RQ_HEAD_INDEX_QUALIFIERS __device__ __forceinline__
#include "head_index.h"

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxChunks = 2;  // chunks per lane; rows need at most 16 waves * 64 lanes * 8 * 2 = 16384

enum QuantMode { kFp8Token = 0, kFp8Group = 1, kMxfp4 = 2 };
// kStageFusedColScales: the fused step with column-major scales (the layout is a
// compile-time choice, so the row-major kernels never read the scale stride),
// each scale stored by the lane that computes it; kStageFusedColScalesStaged:
// the same with the scales staged in LDS and stored as runs along M, MXFP4's
// multi-wave rows two in turn a workgroup (the host's choice for large
// batches, see kStagedColScaleRows).
enum Stage { kStageFused = 0, kStageNorm = 1, kStageQuantize = 2, kStageFusedColScales = 3, kStageFusedColScalesStaged = 4 };

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// v_cvt_pk_bf16_f32: two fp32 -> packed bf16, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
// Element types of the activation rows, two 16-bit values packed per 32-bit
// word (element 2j in the low half).  bf16 is the pages' type; fp16 rows are
// carried through the step unchanged in type (fp16 in, fp16 residual_out and
// y out) for consumers that hold fp16 activations.
struct Bf16 {
  __device__ static float lo(uint32_t w) { return bf_lo(w); }
  __device__ static float hi(uint32_t w) { return bf_hi(w); }
  __device__ static uint32_t pack(float a, float b) { return pack_bf16(a, b); }
  __device__ static float value(uint32_t h) { return __uint_as_float(h << 16); }  // one element's bits
  // v_cvt_scalef32_pk_fp4_bf16: the pair's two E2M1 codes, each element divided
  // by s, into byte kSel of old.
  template <int kSel>
  __device__ static uint32_t fp4x2(uint32_t old, uint32_t w, float s) {
    return (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, __builtin_bit_cast(bf16x2_t, w), s, kSel);
  }
};
struct F16 {
  __device__ static float lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
  __device__ static float hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
  // v_cvt_pk_f16_f32: round to nearest even
  __device__ static uint32_t pack(float a, float b) {
    f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  }
  __device__ static float value(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }
  // v_cvt_scalef32_pk_fp4_f16, as the bf16 one
  template <int kSel>
  __device__ static uint32_t fp4x2(uint32_t old, uint32_t w, float s) {
    return (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f16(old, __builtin_bit_cast(f16x2_t, w), s, kSel);
  }
};

// Largest |bf16| or |fp16| bit pattern of a packed pair per half (integer max of the
// magnitude bits orders finite < Inf < NaN, so a NaN propagates).
__device__ __forceinline__ uint32_t abs_max2(uint32_t acc, uint32_t w) {
  u16x2_t a = __builtin_bit_cast(u16x2_t, acc);
  u16x2_t b = __builtin_bit_cast(u16x2_t, w & 0x7FFF7FFFu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}
__device__ __forceinline__ uint32_t halves_max(uint32_t w) {
  uint32_t lo = w & 0xFFFFu, hi = w >> 16;
  return lo > hi ? lo : hi;
}

// ---------------------------------------------------------------------------
// Global memory.  Streaming rows (read once, written once) use non-temporal
// loads and stores: measured on MI355X they raise the sustained bandwidth of
// this read-2 / write-1.5 pattern by about 5 % of peak.  The weight, re-read by
// every row, uses ordinary cached loads.
// ---------------------------------------------------------------------------
template <bool kNT>
__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  if (!kNT) return *reinterpret_cast<const uint4*>(p);
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <bool kNT, typename T>
__device__ __forceinline__ void store16(T* p, const uint4& v) {
  if (!kNT) {
    *reinterpret_cast<uint4*>(p) = v;
    return;
  }
  const u32x4_t u = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(u, reinterpret_cast<u32x4_t*>(p));
}
template <bool kNT>
__device__ __forceinline__ void store8(uint8_t* p, const uint2& v) {
  if (!kNT) {
    *reinterpret_cast<uint2*>(p) = v;
    return;
  }
  const u32x2_t u = {v.x, v.y};
  __builtin_nontemporal_store(u, reinterpret_cast<u32x2_t*>(p));
}
template <bool kNT>
__device__ __forceinline__ void store4(uint8_t* p, uint32_t v) {
  if (!kNT) {
    *reinterpret_cast<uint32_t*>(p) = v;
    return;
  }
  __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}

// ---------------------------------------------------------------------------
// Cross-lane exchange
// ---------------------------------------------------------------------------
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i inside each 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i inside each 16
constexpr int kSwizzleXor16 = 0x401F; // ds_swizzle bit mode: lane ^ 16 inside each 32

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t swz16(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, kSwizzleXor16);
}
__device__ __forceinline__ uint32_t rdlane(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// Max over aligned groups of 2^log2n lanes (log2n in 0..6, uniform).
__device__ __forceinline__ uint32_t group_max(uint32_t v, int log2n) {
  if (log2n >= 1) v = umax(v, dpp<kDppXor1>(v));
  if (log2n >= 2) v = umax(v, dpp<kDppXor2>(v));
  if (log2n >= 3) v = umax(v, dpp<kDppHalfMirror>(v));
  if (log2n >= 4) v = umax(v, dpp<kDppMirror>(v));
  if (log2n >= 5) v = umax(v, swz16(v));
  if (log2n >= 6) v = umax(rdlane(v, 0), rdlane(v, 32));
  return v;
}
template <int kLog2n>
__device__ __forceinline__ uint32_t group_max_c(uint32_t v) { return group_max(v, kLog2n); }

__device__ __forceinline__ float addf(float a, uint32_t b) { return a + __uint_as_float(b); }
// Sum over aligned groups of 2^log2n lanes, identical in every lane of a group.
__device__ __forceinline__ float group_sum(float v, int log2n) {
  if (log2n >= 1) v = addf(v, dpp<kDppXor1>(__float_as_uint(v)));
  if (log2n >= 2) v = addf(v, dpp<kDppXor2>(__float_as_uint(v)));
  if (log2n >= 3) v = addf(v, dpp<kDppHalfMirror>(__float_as_uint(v)));
  if (log2n >= 4) v = addf(v, dpp<kDppMirror>(__float_as_uint(v)));
  if (log2n == 5) v = addf(v, swz16(__float_as_uint(v)));
  if (log2n >= 6) {
    float a = __uint_as_float(rdlane(__float_as_uint(v), 0));
    float b = __uint_as_float(rdlane(__float_as_uint(v), 16));
    float c = __uint_as_float(rdlane(__float_as_uint(v), 32));
    float d = __uint_as_float(rdlane(__float_as_uint(v), 48));
    v = (a + b) + (c + d);
  }
  return v;
}

// ---------------------------------------------------------------------------
// Quantization helpers
// ---------------------------------------------------------------------------
// Per-granule constants of the FP8 quotient y / scale.
struct Fp8Granule {
  float scale;  // stored scale = amax / 448
  float sc;     // divisor used by the correction step
  float inv;    // correctly rounded 1 / sc
  bool slow;    // scale below 2^-62 or amax not finite: plain IEEE division
};

// No division on the fast path: the scale is the exact quotient amax / 448
// (correction step with the constant 1/448), and its reciprocal is the hardware
// estimate refined by one Newton step, which is the correctly rounded value for
// every scale that can occur (fp8_quotient.h).  Both depend only on amax, so
// they issue in parallel: two short chains instead of two IEEE divisions.
template <typename E>
__device__ __forceinline__ Fp8Granule fp8_granule(uint32_t amax_bits) {
  Fp8Granule g;
  const float amax = E::value(amax_bits);     // exact: every bf16 and fp16 value is an fp32 value
  const uint32_t e = __float_as_uint(amax) >> 23;  // its fp32 exponent field (sign is clear)
  g.slow = false;
  if (amax_bits == 0) {
    // All-zero granule: scale 0; q = y * 0 keeps the sign of each zero.
    g.scale = 0.0f;
    g.sc = 1.0f;
    g.inv = 0.0f;
  } else if (e >= 73u && e < 255u) {  // amax >= 2^-54: the scale and every intermediate stay normal
    g.scale = rq_fp8_scale(amax);
    g.sc = g.scale;
    g.inv = rq_recip_refine(g.scale, __builtin_amdgcn_rcpf(g.scale));
  } else {
    g.scale = amax / 448.0f;
    g.sc = g.scale;
    g.inv = 0.0f;
    g.slow = true;
  }
  return g;
}

// fp32 quotient y / sc, correctly rounded (fp8_quotient.h).
__device__ __forceinline__ float fp8_quotient(float y, const Fp8Granule& g) {
  return rq_fp8_quotient(y, g.sc, g.inv);
}

// Eight values (packed in a uint4) -> eight E4M3FN codes (a uint2).
template <typename E>
__device__ __forceinline__ uint2 fp8_codes(const uint4& y, const Fp8Granule& g) {
  const uint32_t w[4] = {y.x, y.y, y.z, y.w};
  float q[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    q[2 * j] = fp8_quotient(E::lo(w[j]), g);
    q[2 * j + 1] = fp8_quotient(E::hi(w[j]), g);
  }
  // Tiny or non-finite granule: plain IEEE division instead.  The branch is
  // marked unlikely so that it stays a branch: evaluating the eight divisions
  // unconditionally and selecting cost about 0.4 us a decode call.
  if (__builtin_expect(g.slow, false)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      q[2 * j] = E::lo(w[j]) / g.sc;
      q[2 * j + 1] = E::hi(w[j]) / g.sc;
    }
  }
  uint32_t d0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  d0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], (int)d0, true);
  uint32_t d1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  d1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], (int)d1, true);
  return make_uint2(d0, d1);
}

// E8M0 byte for a block whose largest magnitude is amax (a bf16 or fp16 value,
// exact in fp32): floor(log2 amax) - 2 + 127 clamped to [0, 254] is the fp32
// exponent field minus 2, and 0 below that (fp32-subnormal or zero amax); 255
// for Inf / NaN.
__device__ __forceinline__ uint32_t e8m0_byte(float amax) {
  const uint32_t e = __float_as_uint(amax) >> 23;
  if (e == 255u) return 255u;
  return e >= 2u ? e - 2u : 0u;
}

// Eight values -> eight E2M1 codes (one uint32, element i in nibble i): each
// value over the block scale 2^(byte - 127), rounded once to nearest even,
// saturating.  The converter takes the packed 16-bit elements as they are and
// divides by its fp32 scale operand, which holds that scale itself (byte 0 is
// 2^-127, an fp32 subnormal; a finite block's byte is at most 252).  Measured
// on MI355X over every bf16 and every fp16 pair at every such byte, the codes
// are those of scaling in fp32 first (exact: a power of two) and converting at
// scale 1.  A non-finite block (byte 255) passes +Inf; its codes are left
// unspecified.
template <typename E>
__device__ __forceinline__ uint32_t mxfp4_codes(const uint4& y, uint32_t byte) {
  const float s = __uint_as_float(byte != 0u ? byte << 23 : 0x00400000u);
  uint32_t d = 0;
  d = E::template fp4x2<0>(d, y.x, s);
  d = E::template fp4x2<1>(d, y.y, s);
  d = E::template fp4x2<2>(d, y.z, s);
  d = E::template fp4x2<3>(d, y.w, s);
  return d;
}

__device__ __forceinline__ uint32_t chunk_abs_max(const uint4& y) {
  uint32_t m = abs_max2(0u, y.x);
  m = abs_max2(m, y.y);
  m = abs_max2(m, y.z);
  m = abs_max2(m, y.w);
  return halves_max(m);
}

// ---------------------------------------------------------------------------
// The fused row kernel
// ---------------------------------------------------------------------------
struct RowArgs {
  const uint16_t* x;
  const uint16_t* res;
  const uint16_t* w;
  uint16_t* res_out;
  uint8_t* q;
  void* scale;
  uint16_t* y_out;
  int64_t ldx;
  int64_t ldr;
  int64_t row0;          // first row of this launch (a batch too large for one grid takes several)
  int M;
  int H;
  float eps;
  float inv_h;           // 1 / H, rounded on the host
  int group_log2_lanes;  // per-group FP8: log2(group / 8)
  int groups_per_row;    // per-group FP8: H / group
  int64_t scale_ld;      // column-major scales (kStageFusedColScales): scale (m, g) at g * scale_ld + m
};

// Sum of a row from per-lane piece sums (one per chunk): each 64-lane block
// by the wave butterfly, then the blocks in column order (block b = chunk
// b / kWPR of wave b % kWPR).  A multi-wave row exchanges the block sums
// through LDS (one barrier); the loop runs over every block slot, and those
// past the row's end hold +0, which leaves a sum of squares unchanged.
template <int kNC, int kWPR>
__device__ __forceinline__ float row_sum(float (&part)[kNC], float* lds, int lane, int wrow) {
#pragma unroll
  for (int c = 0; c < kNC; ++c) part[c] = group_sum(part[c], 6);  // independent chains
  if (kWPR == 1) {
    float s = part[0];
#pragma unroll
    for (int c = 1; c < kNC; ++c) s += part[c];
    return s;
  }
  if (lane == 0) {
#pragma unroll
    for (int c = 0; c < kNC; ++c) lds[c * kWPR + wrow] = part[c];
  }
  __syncthreads();
  float s = lds[0];
#pragma unroll
  for (int b = 1; b < kNC * kWPR; ++b) s += lds[b];  // one fixed order: every lane agrees
  return s;
}

// Rows a workgroup holds at once: four one-wave rows, or one row of several
// waves (so every barrier of a multi-wave row is uniform over its workgroup).
constexpr int rows_per_block_of(int wpr) { return wpr == 1 ? 4 : 1; }
// Rows a workgroup takes in turn: two multi-wave MXFP4 rows one after the
// other in the staged column-major kernels, so that each scale column receives
// its two bytes in one store (the scattered one-byte stores of a column-major
// scale are what such a launch spends its extra time on); otherwise one.
// Measured on MI355X over 1024-8192 rows at H = 2048-8192: 1.5-8 % faster than
// one row a workgroup (1.4 % slower at [2048, 7168]).  Four rows in turn were
// slower at H = 4096 and mixed at wider rows, two rows at once slower
// throughout.
constexpr int rows_in_turn_of(int wpr, int mode, int stage) {
  return stage == kStageFusedColScalesStaged && mode == kMxfp4 && wpr > 1 ? 2 : 1;
}

// Column-major scales: batches of at least this many rows, whose launch also
// fills the chip's wave slots (M x waves per row >= kResidentWaves), take the
// staged kernels (scales stored as runs along M, MXFP4 rows in turn); smaller
// ones store each scale from the lane that computes it.  Measured on MI355X at
// H = 2048-7168: in smaller batches the staged kernels' final barrier, and the
// second turn's latency when the pairs of rows leave fewer than two
// workgroups or sixteen waves a CU, cost more than the scattered stores
// (MXFP4 up to 1.69x the row-major call's time at 4-512 rows, 1.24x at
// [1024, 2048], against 0.99-1.08x stored directly; per-group FP8 1.04-1.09x
// against 1.00-1.05x); beyond, the runs along M win (MXFP4 [1024, 4096]
// 7.33 against 7.57 us).
constexpr int64_t kStagedColScaleRows = 1024;
template <int kWPR>
constexpr int block_threads() { return kWave * kWPR * rows_per_block_of(kWPR); }

// Column-major scales: the order in which workgroups take rows.  Workgroups are
// dealt to the 8 XCDs in turn (workgroup b runs on XCD b % 8), so in dispatch
// order consecutive rows land on different XCDs, and every line of a scale
// column (32 fp32 or 128 E8M0 values of consecutive rows) collects its values
// in eight L2s, each writing back its part of the line.  This order hands each
// XCD runs of 128 consecutive rows instead, so that one L2 fills each line.
// Measured on MI355X at [8192, 4096]: per-group FP8 goes from 41.3 to 39.5 us
// (row-major scales: 39.5 us) and the extra 64-byte write requests of the
// partial lines disappear.  The tail of the grid past the last whole span of
// 8 runs keeps dispatch order.  A bijection on [0, n).
template <int kRows>
__device__ __forceinline__ uint32_t xcd_run_order(uint32_t b, uint32_t n) {
  constexpr uint32_t kXcds = 8, kRun = 128 / kRows;  // workgroups per run of 128 rows
  constexpr uint32_t kSpan = kXcds * kRun;
  if (b >= n / kSpan * kSpan) return b;
  const uint32_t x = b % kXcds, k = b / kXcds;
  return ((k / kRun) * kXcds + x) * kRun + k % kRun;
}

// kStage selects what one launch does: the fused step (norm + quantize; with
// row-major or column-major scales), or one launch of the unfused sequence (norm
// alone writing y, or quantize alone reading y from a.x with stride a.ldx).
template <typename E, int kMode, int kNC, int kWPR, int kStage>
__global__ __launch_bounds__((block_threads<kWPR>())) void fused_rows(const RowArgs a) {
  constexpr int kLanes = kWave * kWPR;
  constexpr int kChunk = kLanes * 8;
  constexpr int kRPB = rows_per_block_of(kWPR);                  // rows at once
  constexpr int kTurns = rows_in_turn_of(kWPR, kMode, kStage);   // rows in turn
  constexpr int kRows = kRPB * kTurns;                           // rows a workgroup covers
  constexpr bool kNT = true;
  constexpr bool kColScales = kStage == kStageFusedColScales || kStage == kStageFusedColScalesStaged;
  // Only multi-wave MXFP4 rows take turns; every other barrier below is
  // written for one row's turn.
  static_assert(kTurns == 1 || (kMode == kMxfp4 && kRPB == 1), "rows in turn");
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;            // wave in the workgroup
  const int rloc = wave / kWPR;                     // row of the current turn
  const int wrow = wave % kWPR;                     // wave in the row
  const uint32_t blk = kColScales ? xcd_run_order<kRows>(blockIdx.x, gridDim.x) : blockIdx.x;
  const int64_t row_first = a.row0 + (int64_t)blk * kRows;
  const int t = (int)threadIdx.x % kLanes;          // lane in the row
  // A row past the end only happens in the last workgroup of a launch; its
  // waves still reach every barrier (loads and stores are masked).  A
  // workgroup's rows increase with its turns, so its first turn is live
  // whenever any is.
  const int64_t row_of_first_turn = row_first + rloc;
  const bool live_first = row_of_first_turn < a.M;
  const int H = a.H;
  if constexpr (kWPR <= 8) {
    // Left to itself the compiler loads the row pointers in three rounds (the
    // weight's, then x's and the residual's, each behind its own wait) and the
    // output pointers later still.  An empty use of each puts them all in the
    // first batch of argument loads: 1-5 % faster from 1 to 256 rows on MI355X.
    // Rows of 16 waves (1024-thread workgroups) measured 2-3 % slower with it,
    // so they keep the compiler's order.  No instruction is emitted.
    asm volatile("" ::"s"(a.x), "s"(a.res), "s"(a.w), "s"(a.res_out));
    asm volatile("" ::"s"(a.q), "s"(a.scale), "s"(a.y_out));
  }

  // One buffer of block sums per turn, so that a wave's next turn never writes
  // the sums another wave of the row may still be reading.
  __shared__ float lds_sum[kTurns][kRPB][kWPR * kNC];
  __shared__ float lds_sum_tiny[kTurns][kRPB][kWPR * kNC];
  __shared__ uint32_t lds_max[kRPB][kWPR];
  // Staged column-major scales of multi-wave rows (and of MXFP4's four
  // one-wave rows) wait here until the workgroup's last row has its own, then
  // leave as one run of kRows consecutive rows per scale column (one store per
  // column instead of one per row).  At most H / 32 scales a row (E8M0 bytes,
  // or fp32 for groups of 32 or more).  Per-group FP8 in one-wave rows stores
  // its scales directly: those workgroups have no barrier of their own, and
  // the one the stage needs measured 3 % slower on MI355X at [8192, 256].
  constexpr bool kStaged = kStage == kStageFusedColScalesStaged && (kMode == kMxfp4 || kWPR > 1);
  constexpr int kScaleWords = !kStaged ? 1 : kMode == kMxfp4 ? kLanes * kNC / 16 : kLanes * kNC / 4;
  __shared__ uint32_t lds_scales[kStaged ? kRows : 1][kScaleWords];

  // 1. Issue every load of a row before using any of it, the weight first.
  //    Loads return in order, so by the time x and the residual have arrived
  //    the weight has too, and within a turn no wait for data can be made to
  //    include the completion of a store (the one counter of vector memory
  //    operations counts both, and a wait behind a store waits for all); a
  //    second turn's loads do wait behind the first turn's stores.  Rows that
  //    take turns load the weight once, before the first.
  uint4 wv[kNC];
  if constexpr (kTurns > 1) {
#pragma unroll
    for (int c = 0; c < kNC; ++c) {
      const int col = c * kChunk + t * 8;
      wv[c] = (live_first && (c < kNC - 1 || col < H)) ? load16<false>(a.w + col) : make_uint4(0, 0, 0, 0);
    }
  }

  // Not unrolled: two unrolled turns of MXFP4 rows measured 0.5-2.2 us slower
  // at [8192, 4096], [8192, 7168] and [4096, 8192] on MI355X.
#pragma unroll 1
  for (int turn = 0; turn < kTurns; ++turn) {
    const int rw = turn * kRPB + rloc;                // row of the workgroup
    const int64_t row = kTurns == 1 ? row_of_first_turn : row_first + rw;
    const bool live = kTurns == 1 ? live_first : row < a.M;
    uint4 yp[kNC];
    if constexpr (kStage == kStageQuantize) {
      // The quantize launch of the unfused sequence: y comes from memory.
      const uint16_t* yr = a.x + (live ? row : 0) * a.ldx;
#pragma unroll
      for (int c = 0; c < kNC; ++c) {
        const int col = c * kChunk + t * 8;
        yp[c] = (live && (c < kNC - 1 || col < H)) ? load16<kNT>(yr + col) : make_uint4(0, 0, 0, 0);
      }
    } else {
      const uint16_t* xr = a.x + (live ? row : 0) * a.ldx;
      const uint16_t* rr = a.res + (live ? row : 0) * a.ldr;
      uint4 xv[kNC], rv[kNC];
      if constexpr (kTurns == 1) {
    #pragma unroll
        for (int c = 0; c < kNC; ++c) {
          const int col = c * kChunk + t * 8;
          // the weight is re-read by every row: keep it cached
          wv[c] = (live && (c < kNC - 1 || col < H)) ? load16<false>(a.w + col) : make_uint4(0, 0, 0, 0);
        }
      }
    #pragma unroll
      for (int c = 0; c < kNC; ++c) {
        const int col = c * kChunk + t * 8;
        if (live && (c < kNC - 1 || col < H)) {
          xv[c] = load16<kNT>(xr + col);
          rv[c] = load16<kNT>(rr + col);
        } else {
          xv[c] = make_uint4(0, 0, 0, 0);
          rv[c] = make_uint4(0, 0, 0, 0);
        }
      }

      // 2. Residual add (one bf16 rounding) and the sum of squares of each
      //    8-element piece; then the residual_out stores, after the last load.
      uint4 rp[kNC];
      float ssc[kNC];
    #pragma unroll
      for (int c = 0; c < kNC; ++c) {
        const uint32_t xs[4] = {xv[c].x, xv[c].y, xv[c].z, xv[c].w};
        const uint32_t rs[4] = {rv[c].x, rv[c].y, rv[c].z, rv[c].w};
        uint32_t p[4];
        ssc[c] = 0.0f;
    #pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[j] = E::pack(E::lo(xs[j]) + E::lo(rs[j]), E::hi(xs[j]) + E::hi(rs[j]));
          const float r0 = E::lo(p[j]), r1 = E::hi(p[j]);
          ssc[c] = __builtin_fmaf(r0, r0, ssc[c]);
          ssc[c] = __builtin_fmaf(r1, r1, ssc[c]);
        }
        rp[c] = make_uint4(p[0], p[1], p[2], p[3]);
      }
    #pragma unroll
      for (int c = 0; c < kNC; ++c) {
        const int col = c * kChunk + t * 8;
        if (live && (c < kNC - 1 || col < H)) store16<kNT>(a.res_out + row * H + col, rp[c]);
      }

      // 3. rstd over the whole row, summed in an order that does not depend on
      //    the tiling: the 64 pieces of each 512-column block by the wave
      //    butterfly, then the blocks' sums left to right.  Block b is chunk
      //    b / kWPR of wave b % kWPR, so every (kWPR, kNC) launch of a row gives
      //    the same bits, and the host may pick the tiling from the batch size.
      const float ss = row_sum<kNC, kWPR>(ssc, lds_sum[turn][rloc], lane, wrow);
      // rstd need not be correctly rounded (the tolerance on y is one bf16 ulp):
      // the hardware reciprocal square root keeps it off the critical path.
      const float t_ms = __builtin_fmaf(ss, a.inv_h, a.eps);
      float rstd;
      if (__builtin_expect(!(t_ms < 0x1p-100f) && t_ms != __builtin_huge_valf(), true)) {
        rstd = __builtin_amdgcn_rsqf(t_ms);  // NaN propagates through here
      } else {
        // The fp32 squares left their range; sum them again with r scaled by an
        // exact power of two k, in the same order.  A row this small (only with
        // eps < 2^-100; |r| < 2^-43) takes k = 2^100, so the scaled squares lie in
        // [2^-66, 2^114].  A row whose sum of squares overflowed (bf16 allows |r|
        // up to 2^128) takes k = 2^-80: scaled squares at most 2^96, their sum at
        // most 2^110; a row holding Inf still sums to Inf and gets rstd 0, as an
        // exact computation does.  Uniform over the row, and a multi-wave row has
        // its workgroup to itself for its turn.
        const float k = t_ms < 0x1p-100f ? 0x1p100f : 0x1p-80f;
        float s2c[kNC];
    #pragma unroll
        for (int c = 0; c < kNC; ++c) {
          const uint32_t rs[4] = {rp[c].x, rp[c].y, rp[c].z, rp[c].w};
          s2c[c] = 0.0f;
    #pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float r0 = E::lo(rs[j]) * k, r1 = E::hi(rs[j]) * k;
            s2c[c] = __builtin_fmaf(r0, r0, s2c[c]);
            s2c[c] = __builtin_fmaf(r1, r1, s2c[c]);
          }
        }
        const float s2 = row_sum<kNC, kWPR>(s2c, lds_sum_tiny[turn][rloc], lane, wrow);
        rstd = __builtin_amdgcn_rsqf(__builtin_fmaf(s2, a.inv_h, a.eps * k * k)) * k;
      }

      // 4. y = bf16((r * rstd) * w), optional bf16 side output.
    #pragma unroll
      for (int c = 0; c < kNC; ++c) {
        const uint32_t rs[4] = {rp[c].x, rp[c].y, rp[c].z, rp[c].w};
        const uint32_t ws[4] = {wv[c].x, wv[c].y, wv[c].z, wv[c].w};
        uint32_t p[4];
    #pragma unroll
        for (int j = 0; j < 4; ++j)
          p[j] = E::pack((E::lo(rs[j]) * rstd) * E::lo(ws[j]), (E::hi(rs[j]) * rstd) * E::hi(ws[j]));
        yp[c] = make_uint4(p[0], p[1], p[2], p[3]);
      }
      if (a.y_out) {
    #pragma unroll
        for (int c = 0; c < kNC; ++c) {
          const int col = c * kChunk + t * 8;
          if (live && (c < kNC - 1 || col < H)) store16<kNT>(a.y_out + row * H + col, yp[c]);
        }
      }
    }
    if constexpr (kStage == kStageNorm) continue;

    // 5. Absmax per granule, scale, quantize, pack, store.
    if (kMode == kFp8Token) {
      uint32_t m = 0;
#pragma unroll
      for (int c = 0; c < kNC; ++c) m = umax(m, chunk_abs_max(yp[c]));
      m = group_max(m, 6);
      if (kWPR > 1) {
        if (lane == 0) lds_max[rloc][wrow] = m;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kWPR; ++w) m = umax(m, lds_max[rloc][w]);
      }
      const Fp8Granule g = fp8_granule<E>(m);
      if (live && t == 0) reinterpret_cast<float*>(a.scale)[row] = g.scale;
#pragma unroll
      for (int c = 0; c < kNC; ++c) {
        const int col = c * kChunk + t * 8;
        const uint2 codes = fp8_codes<E>(yp[c], g);
        if (live && (c < kNC - 1 || col < H)) store8<kNT>(a.q + row * H + col, codes);
      }
    } else if (kMode == kFp8Group) {
      const int gl = a.group_log2_lanes;
#pragma unroll
      for (int c = 0; c < kNC; ++c) {
        const int col = c * kChunk + t * 8;
        const uint32_t m = group_max(chunk_abs_max(yp[c]), gl);
        const Fp8Granule g = fp8_granule<E>(m);
        const uint2 codes = fp8_codes<E>(yp[c], g);
        if (live && (c < kNC - 1 || col < H)) {
          store8<kNT>(a.q + row * H + col, codes);
          if ((t & ((1 << gl) - 1)) == 0) {
            const int64_t gi = col >> (gl + 3);
            if constexpr (kStaged)
              lds_scales[rw][gi] = __builtin_bit_cast(uint32_t, g.scale);
            else
              reinterpret_cast<float*>(a.scale)[kColScales ? gi * a.scale_ld + row : row * a.groups_per_row + gi] =
                  g.scale;
          }
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < kNC; ++c) {
        const int col = c * kChunk + t * 8;
        const uint32_t m = group_max_c<2>(chunk_abs_max(yp[c]));
        const uint32_t byte = e8m0_byte(E::value(m));
        const uint32_t codes = mxfp4_codes<E>(yp[c], byte);
        if (live && (c < kNC - 1 || col < H)) {
          store4<kNT>(a.q + row * (H / 2) + col / 2, codes);
          if ((t & 3) == 0) {
            const int64_t bi = col / 32;
            if constexpr (kStaged)
              reinterpret_cast<uint8_t*>(lds_scales[rw])[bi] = (uint8_t)byte;
            else
              reinterpret_cast<uint8_t*>(a.scale)[kColScales ? bi * a.scale_ld + row : row * (H / 32) + bi] =
                  (uint8_t)byte;
          }
        }
      }
    }
  }  // turns

  if constexpr (kStaged) {
    // Every row of the workgroup has its scales in LDS; each thread stores one,
    // consecutive threads taking consecutive rows of a scale column.
    __syncthreads();
    const int n = kMode == kMxfp4 ? H / 32 : a.groups_per_row;
    for (int i = threadIdx.x; i < n * kRows; i += kRPB * kLanes) {
      const int si = i / kRows, r = i % kRows;
      if (row_first + r < a.M) {
        const int64_t at = (int64_t)si * a.scale_ld + row_first + r;
        if constexpr (kMode == kMxfp4)
          reinterpret_cast<uint8_t*>(a.scale)[at] = reinterpret_cast<const uint8_t*>(lds_scales[r])[si];
        else
          reinterpret_cast<uint32_t*>(a.scale)[at] = lds_scales[r][si];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// QK GemmaRMSNorm + gate de-interleave
// ---------------------------------------------------------------------------
struct QKArgs {
  const uint16_t* qg;
  const uint16_t* k;
  const uint16_t* qw;
  const uint16_t* kw;
  uint16_t* q_out;     // bf16 outputs (kQKBf16)
  uint16_t* k_out;
  uint16_t* gate_out;
  uint8_t* q_codes;    // quantized outputs: FP8 codes (kQKFp8) or packed E2M1 (kQKMxfp4)
  uint8_t* k_codes;
  void* q_scale;       // fp32 per head (kQKFp8) or E8M0 bytes per 32 elements (kQKMxfp4)
  void* k_scale;
  int64_t ld_qg;
  int64_t ld_k;
  int64_t tok0;          // first token of this launch (a batch too large for one grid takes several)
  uint32_t units;         // heads this launch normalizes: its tokens * (Hq + Hk), below 2^31
  uint32_t heads_magic;   // division by Hq + Hk (head_index.h)
  uint32_t heads_shift;
  int Hq;
  int Hk;
  int D;
  float eps;
  float inv_d;  // 1 / D, rounded on the host
};

constexpr int64_t kMaxHeads = int64_t(1) << 16;  // q or k heads per token accepted by the QK entry points
enum QKOut { kQKBf16 = 0, kQKFp8 = 1, kQKMxfp4 = 2 };
constexpr int kQKBlock = 64;  // one wave a workgroup: spreads a small decode batch over many CUs

// kLog2Lanes: lanes per head = 2^kLog2Lanes >= D / 8; 64 >> kLog2Lanes heads a wave.
// q, k and the gate stream through non-temporal loads and stores (8 % faster
// than cached ones at 8192 tokens on MI355X, the same at decode sizes); the
// head weights use cached loads.
// kOut: bf16 heads; or each normalized head quantized, as E4M3FN codes with
// one fp32 scale (amax / 448) per head (kQKFp8), or as MXFP4 with one E8M0
// byte per 32 elements (kQKMxfp4).  The bf16 head a quantized variant
// quantizes is the one the bf16 variant writes, bit for bit.
template <int kLog2Lanes, int kOut>
__global__ __launch_bounds__(kQKBlock) void qk_gemma_gate(const QKArgs a) {
  constexpr int kLanesPerHead = 1 << kLog2Lanes;
  constexpr int kHeadsPerWave = kWave / kLanesPerHead;
  const int lane = threadIdx.x;
  // flat head index within the launch (token-major), below 2^31
  const uint32_t unit = blockIdx.x * (uint32_t)kHeadsPerWave + (uint32_t)(lane / kLanesPerHead);
  const int col = (lane % kLanesPerHead) * 8;
  const uint32_t heads = (uint32_t)(a.Hq + a.Hk);
  const bool active = unit < a.units && col < a.D;
  const uint32_t tl = rq_head_quotient(unit, a.heads_magic, a.heads_shift);
  const int64_t tok = active ? a.tok0 + tl : 0;
  const int h = active ? (int)(unit - tl * heads) : 0;
  const bool is_q = h < a.Hq;
  if constexpr (kOut != kQKBf16) {
    // Left to itself the compiler loads the gate, code and scale pointers just
    // before the stores, a scalar round trip at the end of every head; an empty
    // use here puts them in the first batch of argument loads (1-2 % faster
    // on MI355X at 64 and at 8192 tokens).  No instruction is emitted.
    asm volatile("" ::"s"(a.gate_out), "s"(a.q_codes), "s"(a.k_codes), "s"(a.q_scale), "s"(a.k_scale));
  }

  uint4 v = make_uint4(0, 0, 0, 0), w = make_uint4(0, 0, 0, 0), gate = make_uint4(0, 0, 0, 0);
  const uint16_t* src;
  if (is_q) {
    src = a.qg + tok * a.ld_qg + (int64_t)2 * a.D * h + col;
  } else {
    src = a.k + tok * a.ld_k + (int64_t)a.D * (h - a.Hq) + col;
  }
  if (active) {
    v = load16<true>(src);  // streaming: non-temporal
    w = *reinterpret_cast<const uint4*>((is_q ? a.qw : a.kw) + col);
    if (is_q) gate = load16<true>(src + a.D);
  }
  const uint32_t vs[4] = {v.x, v.y, v.z, v.w};
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ss = __builtin_fmaf(bf_lo(vs[j]), bf_lo(vs[j]), ss);
    ss = __builtin_fmaf(bf_hi(vs[j]), bf_hi(vs[j]), ss);
  }
  ss = group_sum(ss, kLog2Lanes);
  const float t_ms = __builtin_fmaf(ss, a.inv_d, a.eps);
  float rstd;
  if (!(t_ms < 0x1p-100f) && t_ms != __builtin_huge_valf()) {
    rstd = __builtin_amdgcn_rsqf(t_ms);
  } else {
    // Squares out of fp32 range: sum again with v scaled by k (exact), as in
    // the row kernel: k = 2^100 for a head this small (eps < 2^-100), 2^-80 for
    // a head whose sum of squares overflowed (an Inf in it still gives rstd 0).
    const float k = t_ms < 0x1p-100f ? 0x1p100f : 0x1p-80f;
    float s2 = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v0 = bf_lo(vs[j]) * k, v1 = bf_hi(vs[j]) * k;
      s2 = __builtin_fmaf(v0, v0, s2);
      s2 = __builtin_fmaf(v1, v1, s2);
    }
    s2 = group_sum(s2, kLog2Lanes);
    rstd = __builtin_amdgcn_rsqf(__builtin_fmaf(s2, a.inv_d, a.eps * k * k)) * k;
  }
  uint32_t p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    p[j] = pack_bf16((bf_lo(vs[j]) * rstd) * (1.0f + bf_lo(ws[j])),
                     (bf_hi(vs[j]) * rstd) * (1.0f + bf_hi(ws[j])));
  const uint4 out = make_uint4(p[0], p[1], p[2], p[3]);
  const int64_t head = is_q ? tok * a.Hq + h : tok * a.Hk + (h - a.Hq);  // in the contiguous q or k output
  const int64_t o = head * a.D + col;
  if constexpr (kOut == kQKBf16) {
    if (active) {
      store16<true>((is_q ? a.q_out : a.k_out) + o, out);
      if (is_q) store16<true>(a.gate_out + o, gate);
    }
  } else if constexpr (kOut == kQKFp8) {
    // The head's lanes form an aligned group; lanes past D (and heads past
    // the end) hold zeros, which leave the maximum unchanged.
    const uint32_t m = group_max(chunk_abs_max(out), kLog2Lanes);
    const Fp8Granule g = fp8_granule<Bf16>(m);
    const uint2 codes = fp8_codes<Bf16>(out, g);
    if (active) {
      store8<true>((is_q ? a.q_codes : a.k_codes) + o, codes);
      if (is_q) store16<true>(a.gate_out + o, gate);
      if (col == 0) reinterpret_cast<float*>(is_q ? a.q_scale : a.k_scale)[head] = g.scale;
    }
  } else {
    // A 32-element block is four aligned lanes (D is a multiple of 32).
    const uint32_t m = group_max_c<2>(chunk_abs_max(out));
    const uint32_t byte = e8m0_byte(Bf16::value(m));
    const uint32_t codes = mxfp4_codes<Bf16>(out, byte);
    if (active) {
      store4<true>((is_q ? a.q_codes : a.k_codes) + o / 2, codes);
      if (is_q) store16<true>(a.gate_out + o, gate);
      if ((col & 31) == 0) reinterpret_cast<uint8_t*>(is_q ? a.q_scale : a.k_scale)[o / 32] = (uint8_t)byte;
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel tables
// ---------------------------------------------------------------------------
using RowKernel = void (*)(RowArgs);
using QKKernel = void (*)(QKArgs);

template <typename E, int kMode, int kStage, int kWPR>
struct RowKernelsW {
  static constexpr RowKernel k[kMaxChunks] = {&fused_rows<E, kMode, 1, kWPR, kStage>,
                                              &fused_rows<E, kMode, 2, kWPR, kStage>};
};
template <typename E, int kMode, int kStage>
struct RowKernels {
  // [log2 waves per row][chunks per lane - 1]
  static constexpr const RowKernel* k[5] = {
      RowKernelsW<E, kMode, kStage, 1>::k, RowKernelsW<E, kMode, kStage, 2>::k, RowKernelsW<E, kMode, kStage, 4>::k,
      RowKernelsW<E, kMode, kStage, 8>::k, RowKernelsW<E, kMode, kStage, 16>::k};
};
template <int kOut>
struct QKKernels {
  static constexpr QKKernel k[7] = {&qk_gemma_gate<0, kOut>, &qk_gemma_gate<1, kOut>, &qk_gemma_gate<2, kOut>,
                                    &qk_gemma_gate<3, kOut>, &qk_gemma_gate<4, kOut>, &qk_gemma_gate<5, kOut>,
                                    &qk_gemma_gate<6, kOut>};
};

// ---------------------------------------------------------------------------
// Host-side preflight
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

// A device other than gfx950 is RQ_ERR_DEVICE, not RQ_ERR_UNSUPPORTED: no entry
// point of this library (fused or unfused) can run there, so "cannot fuse,
// run the unfused sequence" would send the caller to calls that fail the same
// way.
rq_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return RQ_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return RQ_ERR_DEVICE;
  int state = g_arch_state[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return RQ_ERR_HIP;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_state[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? RQ_OK : RQ_ERR_DEVICE;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

struct Span {
  uintptr_t lo, hi;  // [lo, hi) in bytes; empty when lo == hi
  bool ok;           // false when the extent cannot be a real buffer (it would overflow)
};
// No buffer spans 2^48 bytes or more; larger extents (absurd strides or
// counts) are refused rather than computed with overflow.
constexpr int64_t kMaxExtentBytes = int64_t(1) << 48;
Span span_of(const void* p, int64_t rows, int64_t ld, int64_t width, int64_t elem_bytes) {
  if (!p || rows <= 0 || width <= 0) return {0, 0, true};
  const int64_t limit = kMaxExtentBytes / elem_bytes;  // in elements
  if (width > limit || ld < 0 || (rows > 1 && ld > (limit - width) / (rows - 1))) return {0, 0, false};
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  const uintptr_t bytes = (uintptr_t)(((rows - 1) * ld + width) * elem_bytes);
  if (lo + bytes < lo) return {0, 0, false};
  return {lo, lo + bytes, true};
}
bool overlap(const Span& a, const Span& b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

// Every output must be disjoint from every other buffer, except residual_out
// aliasing residual exactly (ldr == H); every extent must be representable.
bool outputs_disjoint(const Span* outs, int n_out, const Span* ins, int n_in, int inplace_out, int inplace_in) {
  for (int i = 0; i < n_out; ++i)
    if (!outs[i].ok) return false;
  for (int j = 0; j < n_in; ++j)
    if (!ins[j].ok) return false;
  for (int i = 0; i < n_out; ++i) {
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outs[i], outs[j])) return false;
    for (int j = 0; j < n_in; ++j) {
      if (i == inplace_out && j == inplace_in && outs[i].lo == ins[j].lo && outs[i].hi == ins[j].hi) continue;
      if (overlap(outs[i], ins[j])) return false;
    }
  }
  return true;
}

// Shared checks of the three fused row entry points.  granule = elements per
// scale; code_bits = bits per element of q_out (8 for FP8, 4 for MXFP4).
rq_status row_preflight(const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
                        const uint16_t* weight, int64_t M, int64_t H, float eps,
                        const uint16_t* residual_out, const uint8_t* q_out, const void* scale_out,
                        int64_t scale_count, int64_t scale_bytes, const uint16_t* y_out,
                        int64_t granule, int code_bits, int64_t scale_ld = 0) {
  if (M < 0 || H <= 0 || !(eps >= 0.0f) || ldx < H || ldr < H) return RQ_ERR_INVALID;
  if (scale_ld < 0 || (scale_ld > 0 && scale_ld < M)) return RQ_ERR_INVALID;
  if (M > 0 && (!x || !residual || !weight || !residual_out || !q_out || !scale_out)) return RQ_ERR_INVALID;
  if (H % 8 != 0 || H > RQ_MAX_HIDDEN || M > INT32_MAX) return RQ_ERR_UNSUPPORTED;
  if (granule <= 0 || H % granule != 0) return RQ_ERR_UNSUPPORTED;
  if (M == 0) return RQ_OK;
  if (ldx % 8 != 0 || ldr % 8 != 0 || !aligned(x, 16) || !aligned(residual, 16) || !aligned(weight, 16) ||
      !aligned(residual_out, 16) || (y_out && !aligned(y_out, 16)) || !aligned(q_out, code_bits == 8 ? 8 : 4) ||
      !aligned(scale_out, scale_bytes))
    return RQ_ERR_UNSUPPORTED;
  const Span ins[3] = {span_of(x, M, ldx, H, 2), span_of(residual, M, ldr, H, 2), span_of(weight, 1, H, H, 2)};
  const Span scales = scale_ld > 0 ? span_of(scale_out, scale_count, scale_ld, M, scale_bytes)  // [G, scale_ld]
                                   : span_of(scale_out, M, scale_count, scale_count, scale_bytes);
  const Span outs[4] = {span_of(residual_out, M, H, H, 2), span_of(q_out, M, H * code_bits / 8, H * code_bits / 8, 1),
                        scales, span_of(y_out, M, H, H, 2)};
  if (!outputs_disjoint(outs, 4, ins, 3, /*inplace_out=*/0, /*inplace_in=*/1)) return RQ_ERR_INVALID;
  return check_device();
}

// Checks of the norm launch of the unfused sequence (x, residual, weight in;
// residual_out and y out).
rq_status norm_preflight(const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
                         const uint16_t* weight, int64_t M, int64_t H, float eps, const uint16_t* residual_out,
                         const uint16_t* y_out) {
  if (M < 0 || H <= 0 || !(eps >= 0.0f) || ldx < H || ldr < H) return RQ_ERR_INVALID;
  if (M > 0 && (!x || !residual || !weight || !residual_out || !y_out)) return RQ_ERR_INVALID;
  if (H % 8 != 0 || H > RQ_MAX_HIDDEN || M > INT32_MAX) return RQ_ERR_UNSUPPORTED;
  if (M == 0) return RQ_OK;
  if (ldx % 8 != 0 || ldr % 8 != 0 || !aligned(x, 16) || !aligned(residual, 16) || !aligned(weight, 16) ||
      !aligned(residual_out, 16) || !aligned(y_out, 16))
    return RQ_ERR_UNSUPPORTED;
  const Span ins[3] = {span_of(x, M, ldx, H, 2), span_of(residual, M, ldr, H, 2), span_of(weight, 1, H, H, 2)};
  const Span outs[2] = {span_of(residual_out, M, H, H, 2), span_of(y_out, M, H, H, 2)};
  if (!outputs_disjoint(outs, 2, ins, 3, /*inplace_out=*/0, /*inplace_in=*/1)) return RQ_ERR_INVALID;
  return check_device();
}

// Checks of the quantize launch of the unfused sequence (y in; codes and
// scales out).
rq_status quant_preflight(const uint16_t* y, int64_t ldy, int64_t M, int64_t H, const uint8_t* q_out,
                          const void* scale_out, int64_t scale_count, int64_t scale_bytes, int64_t granule,
                          int code_bits) {
  if (M < 0 || H <= 0 || ldy < H) return RQ_ERR_INVALID;
  if (M > 0 && (!y || !q_out || !scale_out)) return RQ_ERR_INVALID;
  if (H % 8 != 0 || H > RQ_MAX_HIDDEN || M > INT32_MAX) return RQ_ERR_UNSUPPORTED;
  if (granule <= 0 || H % granule != 0) return RQ_ERR_UNSUPPORTED;
  if (M == 0) return RQ_OK;
  if (ldy % 8 != 0 || !aligned(y, 16) || !aligned(q_out, code_bits == 8 ? 8 : 4) || !aligned(scale_out, scale_bytes))
    return RQ_ERR_UNSUPPORTED;
  const Span ins[1] = {span_of(y, M, ldy, H, 2)};
  const Span outs[2] = {span_of(q_out, M, H * code_bits / 8, H * code_bits / 8, 1),
                        span_of(scale_out, M, scale_count, scale_count, scale_bytes)};
  if (!outputs_disjoint(outs, 2, ins, 1, -1, -1)) return RQ_ERR_INVALID;
  return check_device();
}

int group_log2_lanes(int64_t group) {
  for (int l = 2; l <= 6; ++l)
    if (group == (int64_t)8 << l) return l;
  return -1;
}

rq_status launch(const void* kernel, dim3 grid, dim3 block, void* args, void* stream) {
  void* argv[1] = {args};
  hipError_t err = hipLaunchKernel(kernel, grid, block, argv, 0, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}

// Work-items one launch may hold.  A dispatch packet carries the grid size in
// work-items as a 32-bit count; a larger batch is split into launches of at
// most this many work-items each, every launch told its first row or head.
// A build may lower the limit (RQ_MAX_GRID_ITEMS, a multiple of 256) so that
// tests reach the split with small batches; the results do not change.
#ifndef RQ_MAX_GRID_ITEMS
#define RQ_MAX_GRID_ITEMS (int64_t(1) << 31)
#endif
constexpr int64_t kMaxGridItems = RQ_MAX_GRID_ITEMS;
static_assert(kMaxGridItems % 256 == 0 && kMaxGridItems <= (int64_t(1) << 31), "grid limit");

// Waves the chip holds at once: 256 CUs x 4 SIMDs x 8 wave slots per SIMD.
constexpr int64_t kResidentWaves = 256 * 4 * 8;

int chunks_per_lane(int H, int l) {
  const int lanes = kWave << l;
  return (H + lanes * 8 - 1) / (lanes * 8);
}

// Waves per row (a power of two, 1..16).  Many rows: the fewest for which a
// lane holds at most kMaxChunks chunks of 8 elements (few registers, and the
// waves of later rows take the slots that finished ones free), except that a
// row which one chunk of at most 8 waves covers exactly (H = 1024, 2048, 4096)
// takes those waves with one chunk a lane: measured on MI355X 0-2.5 % faster
// than two chunks from 2048 to 16384 rows at those widths, and not at widths
// that would leave lanes idle (3072) or need 16-wave rows (5120-8192).  Fewer
// rows, where the whole launch fits in the chip's wave slots at once: more
// waves, so that a lane holds one chunk, as long as the launch still fits; a
// lane's dependent chain from load to store is then as short as it gets, and
// there is no second generation of waves to wait for.  The column-major scale
// kernels take the same tiling (per-group FP8 with its scales staged in LDS:
// measured on MI355X from 1 % slower to 4 % faster than with the fewest waves,
// over 1024-8192 rows and H = 2048-8192), except that the staged ones give
// rows of 7168-8192 one chunk of 16 waves (launch_rows).  The row's sum is the
// same for every tiling.
int waves_per_row_log2(int64_t M, int H) {
  int l = 0;
  while (l < 4 && chunks_per_lane(H, l) > kMaxChunks) ++l;
  if (l < 3 && chunks_per_lane(H, l) == 2 && H == 8 * (kWave << (l + 1))) ++l;
  while (l < 4 && chunks_per_lane(H, l) > 1 && M * (int64_t)(2 << l) <= kResidentWaves) ++l;
  return l;
}

template <typename E, int kMode, int kStage = kStageFused>
rq_status launch_rows(RowArgs& a, void* stream) {
  int l = waves_per_row_log2(a.M, a.H);
  bool staged = false;
  if constexpr (kStage == kStageFusedColScales) {
    staged = a.M >= kStagedColScaleRows && a.M * (int64_t)(1 << l) >= kResidentWaves;
    // Staged column-major scales of wide rows take one chunk of 16 waves where
    // the row tiling gives two chunks of 8, when at most an eighth of the
    // lanes would sit idle (H >= 7168): measured on MI355X 0-11 % faster at
    // 2048-8192 rows of 7168 and 8192 (the row-major kernels measured up to 8 %
    // slower that way), 3-4 % slower at 5120 where 37.5 % of the lanes idle.
    if (staged && l == 3 && chunks_per_lane(a.H, 3) == 2 && 8 * a.H >= 7 * (kWave << 4) * 8) l = 4;
  }
  const int wpr = 1 << l;
  const int lanes = kWave * wpr;
  const int nc = chunks_per_lane(a.H, l);
  const int rpb = rows_per_block_of(wpr);
  const void* kernel = reinterpret_cast<const void*>(RowKernels<E, kMode, kStage>::k[l][nc - 1]);
  int turns = rows_in_turn_of(wpr, kMode, kStage);
  if constexpr (kStage == kStageFusedColScales) {
    if (staged) {
      kernel = reinterpret_cast<const void*>(RowKernels<E, kMode, kStageFusedColScalesStaged>::k[l][nc - 1]);
      turns = rows_in_turn_of(wpr, kMode, kStageFusedColScalesStaged);
    }
  }
  const int rows_per_wg = rpb * turns;
  // A power of two of at least rows_per_wg rows, so that no workgroup's rows
  // straddle two launches.
  const int64_t rows_per_launch = kMaxGridItems / lanes;
  for (int64_t row0 = 0; row0 < a.M; row0 += rows_per_launch) {
    const int64_t rows = std::min<int64_t>(a.M - row0, rows_per_launch);
    a.row0 = row0;
    const rq_status st = launch(kernel, dim3((unsigned)((rows + rows_per_wg - 1) / rows_per_wg)),
                                dim3((unsigned)(lanes * rpb)), &a, stream);
    if (st != RQ_OK) return st;
  }
  return RQ_OK;
}

RowArgs make_row_args(const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr, const uint16_t* weight,
                      int64_t M, int64_t H, float eps, uint16_t* residual_out, uint8_t* q_out, void* scale_out,
                      uint16_t* y_out) {
  RowArgs a = {};
  a.x = x;
  a.res = residual;
  a.w = weight;
  a.res_out = residual_out;
  a.q = q_out;
  a.scale = scale_out;
  a.y_out = y_out;
  a.ldx = ldx;
  a.ldr = ldr;
  a.M = (int)M;
  a.H = (int)H;
  a.eps = eps;
  a.inv_h = 1.0f / (float)H;
  a.group_log2_lanes = 0;
  a.groups_per_row = 0;
  a.scale_ld = 0;
  return a;
}

// One implementation per entry point, for either element type.
template <typename E>
rq_status fp8_per_token_impl(const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
                             const uint16_t* weight, int64_t M, int64_t H, float eps, uint16_t* residual_out,
                             uint8_t* q_out, float* scale_out, uint16_t* y_out, void* stream) {
  rq_status st = row_preflight(x, ldx, residual, ldr, weight, M, H, eps, residual_out, q_out, scale_out, 1, 4,
                               y_out, H, 8);
  if (st != RQ_OK || M == 0) return st;
  RowArgs a = make_row_args(x, ldx, residual, ldr, weight, M, H, eps, residual_out, q_out, scale_out, y_out);
  return launch_rows<E, kFp8Token>(a, stream);
}

// scale_ld: 0 for row-major scales [M, H / granule]; otherwise the leading
// dimension (>= M) of column-major scales [H / granule, scale_ld].
template <typename E>
rq_status fp8_per_group_impl(const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
                             const uint16_t* weight, int64_t M, int64_t H, float eps, int64_t group,
                             uint16_t* residual_out, uint8_t* q_out, float* scale_out, uint16_t* y_out,
                             void* stream, int64_t scale_ld = 0) {
  if (group <= 0) return RQ_ERR_INVALID;
  const int log2_lanes = group_log2_lanes(group);
  const int64_t granule = log2_lanes < 0 ? -1 : group;
  rq_status st = row_preflight(x, ldx, residual, ldr, weight, M, H, eps, residual_out, q_out, scale_out,
                               log2_lanes < 0 ? 1 : H / group, 4, y_out, granule, 8, scale_ld);
  if (st != RQ_OK || M == 0) return st;
  RowArgs a = make_row_args(x, ldx, residual, ldr, weight, M, H, eps, residual_out, q_out, scale_out, y_out);
  a.group_log2_lanes = log2_lanes;
  a.groups_per_row = (int)(H / group);
  a.scale_ld = scale_ld;
  return scale_ld ? launch_rows<E, kFp8Group, kStageFusedColScales>(a, stream) : launch_rows<E, kFp8Group>(a, stream);
}

template <typename E>
rq_status mxfp4_impl(const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr, const uint16_t* weight,
                     int64_t M, int64_t H, float eps, uint16_t* residual_out, uint8_t* q_out, uint8_t* scale_out,
                     uint16_t* y_out, void* stream, int64_t scale_ld = 0) {
  rq_status st = row_preflight(x, ldx, residual, ldr, weight, M, H, eps, residual_out, q_out, scale_out, H / 32, 1,
                               y_out, 32, 4, scale_ld);
  if (st != RQ_OK || M == 0) return st;
  RowArgs a = make_row_args(x, ldx, residual, ldr, weight, M, H, eps, residual_out, q_out, scale_out, y_out);
  a.scale_ld = scale_ld;
  return scale_ld ? launch_rows<E, kMxfp4, kStageFusedColScales>(a, stream) : launch_rows<E, kMxfp4>(a, stream);
}

template <typename E>
rq_status norm_impl(const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr, const uint16_t* weight,
                    int64_t M, int64_t H, float eps, uint16_t* residual_out, uint16_t* y_out, void* stream) {
  rq_status st = norm_preflight(x, ldx, residual, ldr, weight, M, H, eps, residual_out, y_out);
  if (st != RQ_OK || M == 0) return st;
  RowArgs a = make_row_args(x, ldx, residual, ldr, weight, M, H, eps, residual_out, nullptr, nullptr, y_out);
  return launch_rows<E, kFp8Token, kStageNorm>(a, stream);
}

template <typename E>
rq_status quant_fp8_token_impl(const uint16_t* y, int64_t ldy, int64_t M, int64_t H, uint8_t* q_out,
                               float* scale_out, void* stream) {
  rq_status st = quant_preflight(y, ldy, M, H, q_out, scale_out, 1, 4, H, 8);
  if (st != RQ_OK || M == 0) return st;
  RowArgs a = make_row_args(y, ldy, nullptr, 0, nullptr, M, H, 0.0f, nullptr, q_out, scale_out, nullptr);
  return launch_rows<E, kFp8Token, kStageQuantize>(a, stream);
}

template <typename E>
rq_status quant_fp8_group_impl(const uint16_t* y, int64_t ldy, int64_t M, int64_t H, int64_t group, uint8_t* q_out,
                               float* scale_out, void* stream) {
  if (group <= 0) return RQ_ERR_INVALID;
  const int l = group_log2_lanes(group);
  rq_status st = quant_preflight(y, ldy, M, H, q_out, scale_out, l < 0 ? 1 : H / group, 4, l < 0 ? -1 : group, 8);
  if (st != RQ_OK || M == 0) return st;
  RowArgs a = make_row_args(y, ldy, nullptr, 0, nullptr, M, H, 0.0f, nullptr, q_out, scale_out, nullptr);
  a.group_log2_lanes = l;
  a.groups_per_row = (int)(H / group);
  return launch_rows<E, kFp8Group, kStageQuantize>(a, stream);
}

template <typename E>
rq_status quant_mxfp4_impl(const uint16_t* y, int64_t ldy, int64_t M, int64_t H, uint8_t* q_out,
                           uint8_t* scale_out, void* stream) {
  rq_status st = quant_preflight(y, ldy, M, H, q_out, scale_out, H / 32, 1, 32, 4);
  if (st != RQ_OK || M == 0) return st;
  RowArgs a = make_row_args(y, ldy, nullptr, 0, nullptr, M, H, 0.0f, nullptr, q_out, scale_out, nullptr);
  return launch_rows<E, kMxfp4, kStageQuantize>(a, stream);
}

// Checks and launch of the QK variants.  q_dst / k_dst are the q and k
// outputs (bf16 rows, or codes with the scales already in `a`).
template <int kOut>
rq_status qk_impl(const uint16_t* qg, int64_t ld_qg, const uint16_t* k, int64_t ld_k, const uint16_t* q_w,
                  const uint16_t* k_w, int64_t T, int64_t Hq, int64_t Hk, int64_t D, float eps, QKArgs& a,
                  const void* q_dst, const void* k_dst, uint16_t* gate_out, void* stream) {
  constexpr bool kQuant = kOut != kQKBf16;
  if (T < 0 || Hq < 0 || Hk < 0 || D <= 0 || !(eps >= 0.0f)) return RQ_ERR_INVALID;
  // bounded first, so that the products below cannot overflow
  if (D > RQ_MAX_HEAD_DIM || Hq > kMaxHeads || Hk > kMaxHeads) return RQ_ERR_UNSUPPORTED;
  if (ld_qg < 2 * Hq * D || ld_k < Hk * D) return RQ_ERR_INVALID;
  const bool any_q = T > 0 && Hq > 0, any_k = T > 0 && Hk > 0;
  if (any_q && (!qg || !q_w || !q_dst || !gate_out || (kQuant && !a.q_scale))) return RQ_ERR_INVALID;
  if (any_k && (!k || !k_w || !k_dst || (kQuant && !a.k_scale))) return RQ_ERR_INVALID;
  if (D % (kOut == kQKMxfp4 ? 32 : 8) != 0 || T > INT32_MAX) return RQ_ERR_UNSUPPORTED;
  if (!any_q && !any_k) return RQ_OK;
  // Per head: output bytes, their store alignment, scale bytes and alignment.
  const int64_t out_b = kOut == kQKBf16 ? 2 * D : (kOut == kQKFp8 ? D : D / 2);
  const uintptr_t out_align = kOut == kQKBf16 ? 16 : (kOut == kQKFp8 ? 8 : 4);
  const int64_t sc_b = kOut == kQKFp8 ? 4 : (kOut == kQKMxfp4 ? D / 32 : 0);
  const uintptr_t sc_align = kOut == kQKFp8 ? 4 : 1;
  if ((any_q && (ld_qg % 8 != 0 || !aligned(qg, 16) || !aligned(q_w, 16) || !aligned(q_dst, out_align) ||
                 !aligned(gate_out, 16) || (kQuant && !aligned(a.q_scale, sc_align)))) ||
      (any_k && (ld_k % 8 != 0 || !aligned(k, 16) || !aligned(k_w, 16) || !aligned(k_dst, out_align) ||
                 (kQuant && !aligned(a.k_scale, sc_align)))))
    return RQ_ERR_UNSUPPORTED;
  const Span none{0, 0, true};
  const Span ins[4] = {any_q ? span_of(qg, T, ld_qg, 2 * Hq * D, 2) : none,
                       any_k ? span_of(k, T, ld_k, Hk * D, 2) : none,
                       any_q ? span_of(q_w, 1, D, D, 2) : none, any_k ? span_of(k_w, 1, D, D, 2) : none};
  const Span outs[5] = {any_q ? span_of(q_dst, T, Hq * out_b, Hq * out_b, 1) : none,
                        any_k ? span_of(k_dst, T, Hk * out_b, Hk * out_b, 1) : none,
                        any_q ? span_of(gate_out, T, Hq * D, Hq * D, 2) : none,
                        kQuant && any_q ? span_of(a.q_scale, T, Hq * sc_b, Hq * sc_b, 1) : none,
                        kQuant && any_k ? span_of(a.k_scale, T, Hk * sc_b, Hk * sc_b, 1) : none};
  if (!outputs_disjoint(outs, 5, ins, 4, -1, -1)) return RQ_ERR_INVALID;
  rq_status st = check_device();
  if (st != RQ_OK) return st;

  int log2_lanes = 0;
  while ((8 << log2_lanes) < D) ++log2_lanes;
  a.qg = qg;
  a.k = k;
  a.qw = q_w;
  a.kw = k_w;
  a.gate_out = gate_out;
  a.ld_qg = ld_qg;
  a.ld_k = ld_k;
  const int64_t heads = Hq + Hk;
  const rq_head_divisor div = rq_head_divisor_of((uint32_t)heads);
  a.heads_magic = div.magic;
  a.heads_shift = div.shift;
  a.Hq = (int)Hq;
  a.Hk = (int)Hk;
  a.D = (int)D;
  a.eps = eps;
  a.inv_d = 1.0f / (float)D;
  const int64_t heads_per_wave = kWave >> log2_lanes;
  // Whole tokens a launch, at most 2^31 work-items: the flat head index of a
  // launch stays below 2^31 (heads <= 2^17, so a launch holds >= 2^8 tokens).
  const int64_t tokens_per_launch = kMaxGridItems / kQKBlock * heads_per_wave / heads;
  if (tokens_per_launch < 1) return RQ_ERR_UNSUPPORTED;  // only under a lowered grid limit
  const void* kernel = reinterpret_cast<const void*>(QKKernels<kOut>::k[log2_lanes]);
  for (int64_t tok0 = 0; tok0 < T; tok0 += tokens_per_launch) {
    const int64_t units = std::min<int64_t>(T - tok0, tokens_per_launch) * heads;
    a.tok0 = tok0;
    a.units = (uint32_t)units;
    const rq_status st = launch(kernel, dim3((unsigned)((units + heads_per_wave - 1) / heads_per_wave)),
                                dim3(kQKBlock), &a, stream);
    if (st != RQ_OK) return st;
  }
  return RQ_OK;
}

}  // namespace

extern "C" {

#define RQ_ROW_EXPORTS(SUFFIX, E)                                                                                  \
  rq_status rmsnorm_quant_fp8_per_token##SUFFIX(                                                                   \
      const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr, const uint16_t* weight, int64_t M,    \
      int64_t H, float eps, uint16_t* residual_out, uint8_t* q_out, float* scale_out, uint16_t* y_out,             \
      void* stream) {                                                                                              \
    return fp8_per_token_impl<E>(x, ldx, residual, ldr, weight, M, H, eps, residual_out, q_out, scale_out, y_out,  \
                                 stream);                                                                          \
  }                                                                                                                \
  rq_status rmsnorm_quant_fp8_per_group##SUFFIX(                                                                   \
      const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr, const uint16_t* weight, int64_t M,    \
      int64_t H, float eps, int64_t group, uint16_t* residual_out, uint8_t* q_out, float* scale_out,               \
      uint16_t* y_out, void* stream) {                                                                             \
    return fp8_per_group_impl<E>(x, ldx, residual, ldr, weight, M, H, eps, group, residual_out, q_out, scale_out,  \
                                 y_out, stream);                                                                   \
  }                                                                                                                \
  rq_status rmsnorm_quant_mxfp4##SUFFIX(const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,     \
                                        const uint16_t* weight, int64_t M, int64_t H, float eps,                  \
                                        uint16_t* residual_out, uint8_t* q_out, uint8_t* scale_out,               \
                                        uint16_t* y_out, void* stream) {                                          \
    return mxfp4_impl<E>(x, ldx, residual, ldr, weight, M, H, eps, residual_out, q_out, scale_out, y_out, stream); \
  }                                                                                                                \
  rq_status quantize_fp8_per_token##SUFFIX(const uint16_t* y, int64_t ldy, int64_t M, int64_t H, uint8_t* q_out,  \
                                           float* scale_out, void* stream) {                                      \
    return quant_fp8_token_impl<E>(y, ldy, M, H, q_out, scale_out, stream);                                        \
  }                                                                                                                \
  rq_status quantize_fp8_per_group##SUFFIX(const uint16_t* y, int64_t ldy, int64_t M, int64_t H, int64_t group,   \
                                           uint8_t* q_out, float* scale_out, void* stream) {                      \
    return quant_fp8_group_impl<E>(y, ldy, M, H, group, q_out, scale_out, stream);                                 \
  }                                                                                                                \
  rq_status quantize_mxfp4##SUFFIX(const uint16_t* y, int64_t ldy, int64_t M, int64_t H, uint8_t* q_out,          \
                                   uint8_t* scale_out, void* stream) {                                            \
    return quant_mxfp4_impl<E>(y, ldy, M, H, q_out, scale_out, stream);                                            \
  }                                                                                                                \
  rq_status rmsnorm_quant_fp8_per_group_tscale##SUFFIX(                                                            \
      const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr, const uint16_t* weight, int64_t M,    \
      int64_t H, float eps, int64_t group, uint16_t* residual_out, uint8_t* q_out, float* scale_out,               \
      int64_t ld_scale, uint16_t* y_out, void* stream) {                                                           \
    if (ld_scale < 1) return RQ_ERR_INVALID;                                                                       \
    return fp8_per_group_impl<E>(x, ldx, residual, ldr, weight, M, H, eps, group, residual_out, q_out, scale_out,  \
                                 y_out, stream, ld_scale);                                                         \
  }                                                                                                                \
  rq_status rmsnorm_quant_mxfp4_tscale##SUFFIX(                                                                    \
      const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr, const uint16_t* weight, int64_t M,    \
      int64_t H, float eps, uint16_t* residual_out, uint8_t* q_out, uint8_t* scale_out, int64_t ld_scale,          \
      uint16_t* y_out, void* stream) {                                                                             \
    if (ld_scale < 1) return RQ_ERR_INVALID;                                                                       \
    return mxfp4_impl<E>(x, ldx, residual, ldr, weight, M, H, eps, residual_out, q_out, scale_out, y_out, stream,   \
                         ld_scale);                                                                                \
  }

RQ_ROW_EXPORTS(, Bf16)
RQ_ROW_EXPORTS(_f16, F16)

rq_status rmsnorm_residual_bf16(const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
                                const uint16_t* weight, int64_t M, int64_t H, float eps, uint16_t* residual_out,
                                uint16_t* y_out, void* stream) {
  return norm_impl<Bf16>(x, ldx, residual, ldr, weight, M, H, eps, residual_out, y_out, stream);
}

rq_status rmsnorm_residual_f16(const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
                               const uint16_t* weight, int64_t M, int64_t H, float eps, uint16_t* residual_out,
                               uint16_t* y_out, void* stream) {
  return norm_impl<F16>(x, ldx, residual, ldr, weight, M, H, eps, residual_out, y_out, stream);
}

rq_status qk_gemma_rmsnorm_gate(const uint16_t* qg, int64_t ld_qg, const uint16_t* k, int64_t ld_k,
                                const uint16_t* q_w, const uint16_t* k_w, int64_t T, int64_t Hq, int64_t Hk,
                                int64_t D, float eps, uint16_t* q_out, uint16_t* k_out, uint16_t* gate_out,
                                void* stream) {
  QKArgs a = {};
  a.q_out = q_out;
  a.k_out = k_out;
  return qk_impl<kQKBf16>(qg, ld_qg, k, ld_k, q_w, k_w, T, Hq, Hk, D, eps, a, q_out, k_out, gate_out, stream);
}

rq_status qk_gemma_rmsnorm_gate_fp8(const uint16_t* qg, int64_t ld_qg, const uint16_t* k, int64_t ld_k,
                                    const uint16_t* q_w, const uint16_t* k_w, int64_t T, int64_t Hq, int64_t Hk,
                                    int64_t D, float eps, uint8_t* q_codes, float* q_scale, uint8_t* k_codes,
                                    float* k_scale, uint16_t* gate_out, void* stream) {
  QKArgs a = {};
  a.q_codes = q_codes;
  a.k_codes = k_codes;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  return qk_impl<kQKFp8>(qg, ld_qg, k, ld_k, q_w, k_w, T, Hq, Hk, D, eps, a, q_codes, k_codes, gate_out, stream);
}

rq_status qk_gemma_rmsnorm_gate_mxfp4(const uint16_t* qg, int64_t ld_qg, const uint16_t* k, int64_t ld_k,
                                      const uint16_t* q_w, const uint16_t* k_w, int64_t T, int64_t Hq, int64_t Hk,
                                      int64_t D, float eps, uint8_t* q_codes, uint8_t* q_scale, uint8_t* k_codes,
                                      uint8_t* k_scale, uint16_t* gate_out, void* stream) {
  QKArgs a = {};
  a.q_codes = q_codes;
  a.k_codes = k_codes;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  return qk_impl<kQKMxfp4>(qg, ld_qg, k, ld_k, q_w, k_w, T, Hq, Hk, D, eps, a, q_codes, k_codes, gate_out, stream);
}

const char* rq_status_string(rq_status status) {
  switch (status) {
    case RQ_OK: return "RQ_OK";
    case RQ_ERR_INVALID: return "RQ_ERR_INVALID: invalid argument (null pointer, size, stride, eps or overlap)";
    case RQ_ERR_UNSUPPORTED:
      return "RQ_ERR_UNSUPPORTED: misaligned rows, or a shape this library does not fuse";
    case RQ_ERR_HIP: return "RQ_ERR_HIP: the HIP runtime rejected the launch";
    case RQ_ERR_DEVICE: return "RQ_ERR_DEVICE: the current device is not an MI355X (gfx950)";
  }
  return "unknown rq_status";
}

}  // extern "C"
