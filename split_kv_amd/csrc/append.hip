// KV append for gfx950: the new tokens' key/value rows written into their
// cache pages, quantised to e4m3 for an FP8 cache.
//
// The step before decode attention.  An FP8 cache is read as code x scale
// with one fp32 scale per tensor ("Xqa decode kernels", section "Purpose":
// bf16 queries over an FP8 KV cache); writing stores the inverse: x / scale
// in fp32, saturated to the largest finite e4m3 magnitude and rounded to the
// nearest code by the hardware conversion (v_cvt_pk_fp8_f32, OCP e4m3fn on
// gfx950, round to nearest even).  One wave per (sequence, token, KV head,
// keys or values); each lane moves 16 bytes of the new row per step.
#include "device.h"

namespace splitkv {

namespace {

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

}  // namespace

__global__ __launch_bounds__(64) void append_kernel(AppendParams p) {
  const int which = blockIdx.y;          // 0: keys, 1: values
  int r = blockIdx.x;
  const int hk = r % p.Hkv;
  r /= p.Hkv;
  const int t = r % p.T;
  const int b = r / p.T;
  const int64_t pos = int64_t(p.positions[b]) + t;
  if (pos < 0) return;
  const int64_t col = pos / p.page_size;
  if (col >= p.bt_stride) return;
  const int page = p.bt[int64_t(b) * p.bt_stride + col];
  if (page < 0 || page >= p.num_pages) return;
  const int64_t slot = pos - col * p.page_size;
  const uint16_t* src = p.src[which] + int64_t(b) * p.ssb[which] + int64_t(t) * p.sst[which] +
                        int64_t(hk) * p.ssh[which];
  uint8_t* dst = p.dst[which] + int64_t(page) * p.dsp[which] + int64_t(hk) * p.dsh[which] +
                 slot * p.dsk[which];
  const int d = p.d[which];
  for (int i = 8 * int(threadIdx.x); i < d; i += 8 * 64) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(src + i);
    if (p.fp8)
      *reinterpret_cast<u32x2*>(dst + i) = quantise8(w, p.scale[which]);
    else
      *reinterpret_cast<u32x4*>(dst + 2 * i) = w;
  }
}

hipError_t launch_append(const AppendParams& p, int rows, int kinds, hipStream_t stream) {
  hipLaunchKernelGGL(append_kernel, dim3(unsigned(rows), unsigned(kinds)), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace splitkv
