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
// everything it read to sink[w] so that no load can be dropped.  Like the
// grouped-query kernel, a grid with a workgroup per compute unit or more
// reads with non-temporal loads (NT), a smaller one with default ones.
constexpr int kCalibThreads = 256;
constexpr int kCalibUnroll = 32;

template <bool NT>
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
      if constexpr (NT)
        v[u] = j < hi ? __builtin_nontemporal_load(src + j) : zero;
      else
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

// Matrix-product rate: each wave runs `iters` rounds of four independent
// accumulation chains of v_mfma_f32_32x32x16_bf16 (32 x 32 x 16, 32,768
// FLOPs each) on register operands, so the matrix unit of its SIMD never
// waits for an operand; with four waves a workgroup, one per SIMD.  Wave w of
// workgroup g stores to sink[2 (4 g + w)] the low bits of its accumulators'
// sum (so nothing is dropped) and to sink[2 (4 g + w) + 1] the s_memtime
// cycles (core clocks) its loop took.
constexpr int kCalibMfmaWaves = 4;

__global__ __launch_bounds__(64 * kCalibMfmaWaves) void calib_mfma_kernel(int32_t iters, uint32_t* sink) {
  typedef float f32x16_t __attribute__((ext_vector_type(16)));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = short(0x3f80 + ((lane + i) & 7));       // bf16 values near 1
    b[i] = short(0x3f00 + ((lane * 3 + i) & 7));   // near 0.5
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  float sum = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) sum += c0[v] + c1[v] + c2[v] + c3[v];
  for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 64);
  if (lane == 0) {
    const int64_t i = (int64_t(blockIdx.x) * kCalibMfmaWaves + wave) * 2;
    sink[i] = __float_as_uint(sum);
    sink[i + 1] = uint32_t(t1 - t0);
  }
}

// LDS read bandwidth: each workgroup of four waves fills 64 KiB of LDS, then
// every wave runs `iters` rounds of sixteen reads -- mode 0: ds_read_b128, 16
// bytes a lane; mode 1: ds_read_b64_tr_b16, 8 bytes a lane -- at
// lane-consecutive, bank-conflict-free addresses that move by 1 KiB a read
// (wrapping inside the 64 KiB), XOR-accumulating what it read.  Wave w of
// workgroup g stores the XOR to sink[2 (4 g + w)] and the s_memtime cycles of
// its read loop to sink[2 (4 g + w) + 1].
constexpr int kCalibLdsBytes = 65536;

__global__ __launch_bounds__(256) void calib_lds_read_kernel(int32_t iters, int32_t mode, uint32_t* sink) {
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;
  typedef short v4i16_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kCalibLdsBytes];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kCalibLdsBytes / 16; i += 256)
    reinterpret_cast<u32x4*>(lds)[i] = u32x4{uint32_t(i), uint32_t(i * 3), uint32_t(i * 5), uint32_t(i * 7)};
  __syncthreads();
  u32x4 acc = {0u, 0u, 0u, 0u};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  if (mode == 0) {
    for (int it = 0; it < iters; ++it) {
      u32x4 v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t off = (uint32_t(it * 16 + j + wave * 4) * 1024u + 16u * lane) & (kCalibLdsBytes - 1);
        v[j] = *(const lds_u32x4_t*)((__attribute__((address_space(3))) uint8_t*)lds + off);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) acc ^= v[j];
    }
  } else {
    for (int it = 0; it < iters; ++it) {
      v4i16_t v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t off = (uint32_t(it * 16 + j + wave * 4) * 1024u + 8u * lane) & (kCalibLdsBytes - 1);
        v[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)((__attribute__((address_space(3))) uint8_t*)lds + off));
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        acc.x ^= uint32_t(uint16_t(v[j][0])) | (uint32_t(uint16_t(v[j][1])) << 16);
        acc.y ^= uint32_t(uint16_t(v[j][2])) | (uint32_t(uint16_t(v[j][3])) << 16);
      }
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int m = 32; m >= 1; m >>= 1) x ^= uint32_t(__shfl_xor(int(x), m, 64));
  if (lane == 0) {
    const int64_t i = (int64_t(blockIdx.x) * 4 + wave) * 2;
    sink[i] = x;
    sink[i + 1] = uint32_t(t1 - t0);
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
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return fail(SPLITKV_ERR_DEVICE, "%s: cannot query the compute-unit count", fn);
  if (workgroups >= cus)
    hipLaunchKernelGGL(calib_stream_read_kernel<true>, dim3(unsigned(workgroups)), dim3(kCalibThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), n16, per_wg, sink);
  else
    hipLaunchKernelGGL(calib_stream_read_kernel<false>, dim3(unsigned(workgroups)), dim3(kCalibThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), n16, per_wg, sink);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SPLITKV_ERR_LAUNCH, "%s: %s", fn, hipGetErrorString(err));
  return SPLITKV_OK;
}

splitkv_status splitkv_calib_mfma(int32_t workgroups, int32_t iters, uint32_t* sink, void* stream) {
  const char* fn = "splitkv_calib_mfma";
  if (!sink || (reinterpret_cast<uintptr_t>(sink) & 3) != 0 || workgroups < 1 || workgroups > (1 << 20) ||
      iters < 1 || iters > (1 << 24))
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: bad arguments (workgroups %d, iters %d)", fn, workgroups, iters);
  hipLaunchKernelGGL(calib_mfma_kernel, dim3(unsigned(workgroups)), dim3(64 * kCalibMfmaWaves), 0,
                     static_cast<hipStream_t>(stream), iters, sink);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SPLITKV_ERR_LAUNCH, "%s: %s", fn, hipGetErrorString(err));
  return SPLITKV_OK;
}

splitkv_status splitkv_calib_lds_read(int32_t workgroups, int32_t iters, int32_t mode, uint32_t* sink,
                                      void* stream) {
  const char* fn = "splitkv_calib_lds_read";
  if (!sink || (reinterpret_cast<uintptr_t>(sink) & 3) != 0 || workgroups < 1 || workgroups > (1 << 20) ||
      iters < 1 || iters > (1 << 24) || (mode != 0 && mode != 1))
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: bad arguments (workgroups %d, iters %d, mode %d)", fn, workgroups,
                iters, mode);
  hipLaunchKernelGGL(calib_lds_read_kernel, dim3(unsigned(workgroups)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, mode, sink);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(SPLITKV_ERR_LAUNCH, "%s: %s", fn, hipGetErrorString(err));
  return SPLITKV_OK;
}

}  // extern "C"
