// Pieces of the MLA partial kernel (bf16 cache; e4m3 cache with bf16 or e4m3
// queries): the direct global->LDS tile loads, the LDS barrier, the 32x32
// product and lane helpers of a 32-row wave, and the paged-addressing record.
#pragma once

#include "device.h"

namespace splitkv {
namespace mla {

constexpr int kDqk = 576;                        // latent row: 512 value features + 64 rope
constexpr int kDv = 512;
constexpr int kWRows = SPLITKV_ROWS_PER_WG_MLA;  // 128 query rows per workgroup
constexpr int kWWaves = 4;                       // one per SIMD, 32 rows each
static_assert(kWRows == 32 * kWWaves, "32 rows per wave");
constexpr int kTile = 32;                        // tokens per LDS tile
constexpr int kVb = kDv / 32;                    // 16 blocks of 32 value features
// Epilogue staging of the compact partial: 128 rows of 512 int16 codes, row
// pitch 1040 bytes.
constexpr int kCodeRowBytes = 1040;
constexpr int kStageBytes = kWRows * kCodeRowBytes;   // 133120

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Direct global->LDS load of 16 bytes per lane into the 1 KiB at LDS byte
// address lds (lane j at lds + 16 j), issued as inline assembly so that the
// compiler does not track it: it would otherwise make every LDS read of the
// tile ring wait for all such loads in flight (it cannot tell which slot a
// load fills).  The kernels wait for these loads explicitly (s_waitcnt vmcnt
// and a workgroup barrier before a slot is read), and loads complete in
// order, so the compiler's own waits for other loads stay correct.  M0 holds
// the LDS address; nothing else in the kernels uses M0.
__device__ __forceinline__ void dma16(const uint8_t* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory");
}
// The same with a uniform 64-bit base and a 32-bit per-lane offset.
__device__ __forceinline__ void dma16_sbase(const uint8_t* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory");
}

// Workgroup barrier after this wave's LDS operations have completed (a bare
// s_barrier does not wait for them); the signal fences keep the compiler from
// moving memory operations across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt immediate for vmcnt(n) alone (n < 64).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Max and sum over the two lanes l and l ^ 32 (one row of the 32x32 result).
__device__ __forceinline__ float pair_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// acc *= a for an accumulator held in the accumulation registers, one
// register at a time (read, multiply, write back): written as whole-vector
// arithmetic, the compiler copies every accumulator out at once, which does
// not fit beside the query.
__device__ __forceinline__ void scale_acc(f32x16& acc, float a) {
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float tmp;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(acc[v]), "=&v"(tmp)
                 : "v"(a));
  }
}

// The paged-addressing record of a workgroup (its range and a digest of the
// pages its 16-token groups read), when the caller asked for it.
__device__ __forceinline__ void store_debug(const PartialParams& p, int slot, int rb, int b, int split, int s,
                                            int e, int groups, int pxor, uint32_t psum) {
  int32_t* rec = p.debug + (int64_t(slot) * p.row_blocks + rb) * 8;
  rec[0] = b;
  rec[1] = split;
  rec[2] = 0;
  rec[3] = s;
  rec[4] = e;
  rec[5] = groups;
  rec[6] = pxor;
  rec[7] = int(psum & 0x7fffffffu);
}

}  // namespace mla
}  // namespace splitkv
