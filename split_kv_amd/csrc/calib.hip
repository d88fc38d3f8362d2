// Measurement helpers of the benchmark: the floors a decode step is judged
// against.  A plain streaming read over the same bytes and the same number of
// workgroups shows what any read-only kernel of that grid reaches on this GPU,
// and an empty kernel shows what one graph node costs before any work -- the
// "same grid, thread count and shared memory" comparison that separates launch
// and occupancy effects from useful work ("vLLM 0.30.0 FA4 SplitKV Bug: H100
// Decode Can Be 48% Slower", section "The kernel profile isolates one
// operation").
#include "device.h"
#include "internal.h"

namespace splitkv {

__global__ void calib_empty_kernel() {}

// Workgroup w reads 16-byte words [w * per_wg, min(n16, (w + 1) * per_wg)),
// thirty-two loads in flight per thread (128 KiB per workgroup, as many bytes
// as a grouped-query decode workgroup keeps in flight), and stores the XOR of
// everything it read to sink[w] so that no load can be dropped.
constexpr int kCalibThreads = 256;
constexpr int kCalibUnroll = 32;

__global__ __launch_bounds__(kCalibThreads) void calib_stream_read_kernel(const u32x4* src, int64_t n16,
                                                                         int64_t per_wg, uint32_t* sink) {
  __shared__ uint32_t red[kCalibThreads / 64];
  const int64_t lo = int64_t(blockIdx.x) * per_wg;
  const int64_t hi = min(n16, lo + per_wg);
  u32x4 acc = {0u, 0u, 0u, 0u};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  // every load of a round is issued before any is used; loads past the
  // share's end are masked off
  for (int64_t base = lo + threadIdx.x; base < hi; base += kCalibUnroll * kCalibThreads) {
    u32x4 v[kCalibUnroll];
#pragma unroll
    for (int u = 0; u < kCalibUnroll; ++u) {
      const int64_t j = base + int64_t(u) * kCalibThreads;
      v[u] = j < hi ? src[j] : zero;
    }
#pragma unroll
    for (int u = 0; u < kCalibUnroll; ++u) acc ^= v[u];
  }
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= uint32_t(__shfl_xor(int(x), m, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < kCalibThreads / 64; ++w) r ^= red[w];
    sink[blockIdx.x] = r;
  }
}

}  // namespace splitkv

using namespace splitkv;

extern "C" {

splitkv_status splitkv_calib_empty(void* stream) {
  hipLaunchKernelGGL(calib_empty_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SPLITKV_ERR_LAUNCH, "splitkv_calib_empty: %s", hipGetErrorString(err));
  return SPLITKV_OK;
}

splitkv_status splitkv_calib_stream_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink,
                                         void* stream) {
  const char* fn = "splitkv_calib_stream_read";
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(sink) & 3) != 0 || workgroups < 1 || workgroups > (1 << 24))
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: bad arguments (bytes %zu, workgroups %d)", fn, bytes, workgroups);
  const int64_t n16 = int64_t(bytes / 16);
  const int64_t per_wg = (n16 + workgroups - 1) / workgroups;
  hipLaunchKernelGGL(calib_stream_read_kernel, dim3(unsigned(workgroups)), dim3(kCalibThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), n16, per_wg, sink);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SPLITKV_ERR_LAUNCH, "%s: %s", fn, hipGetErrorString(err));
  return SPLITKV_OK;
}

}  // extern "C"
