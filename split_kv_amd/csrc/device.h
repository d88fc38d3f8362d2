// Device-side helpers and the parameter block shared by the gfx950 kernels.
//
// Notation follows the split-KV pages: a decode step attends a few query
// tokens over a long KV history; each split yields a partial (m, l, o) that a
// combine merges ("vLLM 0.30.0 FA4 SplitKV Bug: H100 Decode Can Be 48%
// Slower", section "What SplitKV is trying to do").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "splitkv.h"

namespace splitkv {

typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Parameters of every partial kernel (plain values; built on the host).
struct PartialParams {
  const uint16_t* q;            // bf16 codes
  int64_t qsb, qst, qsh;        // element strides
  int32_t q_rows_linear;        // MLA: row r = t * Hq + h at r * qsh (qst == Hq * qsh), byte offsets < 2^31
  const uint8_t* k;             // cache base, as bytes
  const uint8_t* v;
  int64_t ksp, ksh, kst;        // byte strides
  int64_t vsp, vsh, vst;
  const int32_t* bt;
  int64_t bt_stride;
  const int32_t* seq_lens;
  const int32_t* num_splits;
  const int32_t* slot_offset;
  const int32_t* slot_info;     // [S][4]: b, (n << 16) | split, start, end
  int32_t T, Hq, Hkv, g, page_size, rows, row_blocks, total_wg;
  int32_t page_shift;           // log2(page_size) when it is a power of two, else -1
  float scale_log2;             // scale * k_scale * log2(e) (times q_scale for e4m3 queries)
  float q_scale;                // e4m3 queries: codes of q / q_scale
  float q_rcp;                  // RN(1 / q_scale) when 2^-64 <= q_scale <= 2^64, else 0
  float v_scale;
  float* part_m;                // [S][T*Hq]
  float* part_l;
  float* part_o;                // [S][T*Hq][d_v] (grouped-query kernels)
  float* part_s;                // MLA: [S][T*Hq][2] scales of the two 256-feature halves of o
  int16_t* part_q;              // MLA: [S][T*Hq][512] codes of o (o = code * scale of its half)
  void* out;
  int32_t out_f32;
  float* lse;
  int32_t* debug;
  int32_t* tickets;             // single launch: arrival counters per (sequence, KV head, row block)
  int32_t direct;               // single-split sequences write out/lse directly
};

struct CombineParams {
  const int32_t* num_splits;
  const int32_t* slot_offset;
  const float* part_m;
  const float* part_l;
  const float* part_o;
  void* out;
  int32_t out_f32;
  float* lse;
  int32_t B, R, d_v;            // R = T * Hq rows per sequence
  int32_t skip_single;          // rows of single-split sequences were written by the partial kernel
  int32_t uniform_splits;       // > 0: every sequence has this many splits (no plan reads)
  int32_t max_seq_splits;       // > 0: no sequence has more splits (sizes the launch); 0: unknown
};

// Parameters of the KV append kernel (index 0: keys, 1: values).
struct AppendParams {
  const uint16_t* src[2];            // new keys, new values (bf16 codes)
  int64_t ssb[2], sst[2], ssh[2];    // their element strides
  uint8_t* dst[2];                   // key and value caches, as bytes
  int64_t dsp[2], dsh[2], dsk[2];    // cache byte strides: page, head, token
  int32_t d[2];                      // row widths
  const int32_t* bt;
  int64_t bt_stride;
  const int32_t* positions;
  int32_t T, Hkv, page_size, num_pages, fp8;
  float scale[2];
};

typedef short bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Two fp32 values to a bf16 pair (lo in the low half) with one
// v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Widen four e4m3 codes (one dword) to four bf16 codes (two dwords).  Every
// e4m3 value is a bf16 value, so the conversion is exact with scale 1.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, lo);
  r.y = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// e4m3 encoding of bf16 values x / s (fp32 division), saturated to the largest
// finite magnitude and rounded to the nearest code by the hardware conversion
// (v_cvt_pk_fp8_f32: OCP e4m3fn on gfx950, round to nearest even).
constexpr float kE4m3Max = 448.f;

// x / s saturated to +-448 (NaN passes through: both comparisons are false).
__device__ __forceinline__ float scaled_sat(float x, float s) {
  const float y = x / s;
  return y > kE4m3Max ? kE4m3Max : (y < -kE4m3Max ? -kE4m3Max : y);
}

// Eight bf16 values (four dwords) -> eight e4m3 codes (two dwords).
__device__ __forceinline__ u32x2 quantise8(u32x4 w, float s) {
  u32x2 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t a = h ? w.z : w.x, b = h ? w.w : w.y;
    const float f0 = scaled_sat(__uint_as_float(a << 16), s);
    const float f1 = scaled_sat(__uint_as_float(a & 0xffff0000u), s);
    const float f2 = scaled_sat(__uint_as_float(b << 16), s);
    const float f3 = scaled_sat(__uint_as_float(b & 0xffff0000u), s);
    int c = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
    c = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, c, true);
    if (h) r.y = uint32_t(c); else r.x = uint32_t(c);
  }
  return r;
}

// The same codes without a division per value, given r = RN(1 / s) and
// 2^-64 <= s <= 2^64.  For x = |value| the quotient estimate q0 = RN(x r)
// is corrected once by the exact remainder: q1 = RN(q0 + RN(x - s q0) r),
// both steps fused multiply-adds.  For a numerator with at most 8 significant
// bits (every bf16 value) q1 is the correctly rounded fp32 quotient x / s:
// the check runs every fp32 significand of s against every bf16 significand
// of x (2^30 pairs, none differs), and the rounding steps scale with the
// exponents as long as the values that decide a code (quotients from 2^-12
// to 448, whose remainders are near x 2^-24) stay normal, which the bounds on
// s guarantee.  Quotient estimates above 448 (the exact quotient then rounds
// to the 448 code too; infinite x gives one) saturate; NaN stays NaN; the
// sign bit of each value is copied onto its code, so -0 keeps its own code.
__device__ __forceinline__ u32x2 quantise8_rcp(u32x4 w, float s, float r) {
  u32x2 res;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t a = h ? w.z : w.x, b = h ? w.w : w.y;
    float f[4] = {__uint_as_float((a << 16) & 0x7fffffffu), __uint_as_float(a & 0x7fff0000u),
                  __uint_as_float((b << 16) & 0x7fffffffu), __uint_as_float(b & 0x7fff0000u)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float q0 = f[i] * r;
      const float q1 = __builtin_fmaf(__builtin_fmaf(-s, q0, f[i]), r, q0);
      f[i] = q0 > kE4m3Max ? kE4m3Max : q1;
    }
    int c = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    c = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], c, true);
    // sign bits: bit 7 of bytes 1 and 3 of a and of b, to bytes 0 .. 3
    const uint32_t sg = __builtin_amdgcn_perm(b, a, 0x07050301u) & 0x80808080u;
    if (h) res.y = uint32_t(c) | sg; else res.x = uint32_t(c) | sg;
  }
  return res;
}

// Lane-exchange helpers within a 64-wide wavefront.
__device__ __forceinline__ float xor_shfl(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Max over the four lanes {l, l^16, l^32, l^48} (one MFMA output column),
// with the gfx950 lane-swap instructions instead of an LDS round trip.
__device__ __forceinline__ float column_max4(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float column_sum4(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 2^x with the hardware instruction (no denormal range reduction; the
// arguments here are <= 8 and tiny results may flush to zero).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Work record of one slot, read through the scalar cache in one load.
struct SlotWork {
  int b, split, nsplit, s, e;
};

typedef const __attribute__((address_space(4))) int32_t cint32;

__device__ __forceinline__ SlotWork load_slot(const int32_t* slot_info, int slot) {
  cint32* r = (cint32*)slot_info + 4 * slot;
  SlotWork w;
  w.b = r[0];
  w.split = r[1] & 0xffff;
  w.nsplit = r[1] >> 16;
  w.s = r[2];
  w.e = r[3];
  return w;
}

template <typename T>
__device__ __forceinline__ T uniform(T v) {
  return __builtin_amdgcn_readfirstlane(v);
}

}  // namespace splitkv
