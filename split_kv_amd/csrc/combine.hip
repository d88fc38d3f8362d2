// Log-sum-exp combine of split partials, and the e4m3 widening check kernel.
//
// The combine merges the (m, l, o) partials of a sequence's splits into the
// softmax output: M = max_i m_i, w_i = exp(m_i - M), out = sum w_i o_i /
// sum w_i l_i, lse = M + ln(sum w_i l_i).  An empty split carries m = -inf and
// gets weight zero, which is why a split count that leaves ranges empty still
// gives the right answer ("vLLM 0.30.0 FA4 SplitKV Bug: H100 Decode Can Be 48%
// Slower", section "Why the result is still correct").  Its cost grows with
// the split count ("Shipped: 484.5 tok/s on one GB300 ...", section "Why 8
// splits lost"): it reads S * rows * (d_v + 2) * 4 bytes of partials.
//
// One wave per output row (b, t, h); lanes span the d_v features so every
// partial row is one coalesced read.
#include "device.h"

namespace splitkv {

template <int DV>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  constexpr int VEC = DV / 64;          // features per lane: 2, 4 or 8
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= int64_t(p.B) * p.R) return;
  const int b = int(row / p.R);
  const int64_t rix = row % p.R;
  const int n = p.num_splits[b];
  if (p.skip_single && n == 1) return;
  const int64_t base = p.slot_offset[b];

  float M = -INFINITY;
  for (int i = lane; i < n; i += 64) M = fmaxf(M, p.part_m[(base + i) * p.R + rix]);
  M = wave_max(M);
  float lam = 0.f;
  for (int i = lane; i < n; i += 64) {
    const float mi = p.part_m[(base + i) * p.R + rix];
    if (mi != -INFINITY) lam += expf(mi - M) * p.part_l[(base + i) * p.R + rix];
  }
  lam = wave_sum(lam);

  float acc[VEC];
#pragma unroll
  for (int k = 0; k < VEC; ++k) acc[k] = 0.f;
  if (M != -INFINITY) {
    for (int i = 0; i < n; ++i) {
      const float mi = p.part_m[(base + i) * p.R + rix];
      if (mi == -INFINITY) continue;
      const float w = expf(mi - M);
      const float* src = p.part_o + ((base + i) * p.R + rix) * DV + lane * VEC;
#pragma unroll
      for (int k = 0; k < VEC; k += 2) {
        const float2 v = *reinterpret_cast<const float2*>(src + k);
        acc[k] += w * v.x;
        acc[k + 1] += w * v.y;
      }
    }
  }
  const bool ok = M != -INFINITY && lam > 0.f;
  const float inv = ok ? 1.f / lam : 0.f;
  const int64_t o = row * DV + lane * VEC;
  if (p.out_f32) {
    float* dst = static_cast<float*>(p.out) + o;
#pragma unroll
    for (int k = 0; k < VEC; ++k) dst[k] = acc[k] * inv;
  } else {
    uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.out) + o);
#pragma unroll
    for (int k = 0; k < VEC; k += 2) dst[k / 2] = pack_bf16x2(acc[k] * inv, acc[k + 1] * inv);
  }
  if (p.lse && lane == 0) p.lse[row] = ok ? M + logf(lam) : -INFINITY;
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  const int64_t rows = int64_t(p.B) * p.R;
  const dim3 grid(unsigned((rows + 3) / 4)), block(256);
  switch (p.d_v) {
    case 128: hipLaunchKernelGGL(combine_kernel<128>, grid, block, 0, stream, p); break;
    case 256: hipLaunchKernelGGL(combine_kernel<256>, grid, block, 0, stream, p); break;
    case 512: hipLaunchKernelGGL(combine_kernel<512>, grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Widen e4m3 codes with the exact conversion the FP8 partial kernel uses.
__global__ void e4m3_to_bf16_kernel(const uint8_t* in, uint16_t* out, int64_t n) {
  const int64_t i = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i + 3 < n) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(in + i);
    const u32x2 r = e4m3x4_to_bf16x4(w);
    out[i + 0] = uint16_t(r.x & 0xffff);
    out[i + 1] = uint16_t(r.x >> 16);
    out[i + 2] = uint16_t(r.y & 0xffff);
    out[i + 3] = uint16_t(r.y >> 16);
  } else {
    for (int64_t k = i; k < n; ++k) {
      const u32x2 r = e4m3x4_to_bf16x4(uint32_t(in[k]));
      out[k] = uint16_t(r.x & 0xffff);
    }
  }
}

hipError_t launch_e4m3_to_bf16(const uint8_t* in, uint16_t* out, int64_t n, hipStream_t stream) {
  const int64_t quads = (n + 3) / 4;
  const dim3 grid(unsigned((quads + 255) / 256)), block(256);
  hipLaunchKernelGGL(e4m3_to_bf16_kernel, grid, block, 0, stream, in, out, n);
  return hipGetLastError();
}

}  // namespace splitkv
