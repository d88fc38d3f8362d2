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
