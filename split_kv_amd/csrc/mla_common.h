// Pieces shared by the MLA partial kernels (bf16 and e4m3 queries): the
// direct global->LDS tile loads, the LDS barrier, and the epilogue that writes
// a workgroup's partial (m, l, o) or, for a single-split sequence, the final
// output and log-sum-exp.
#pragma once

#include "device.h"

namespace splitkv {
namespace mla {

constexpr int kDqk = 576;                        // latent row: 512 value features + 64 rope
constexpr int kDv = 512;
constexpr int kBlockRows = SPLITKV_ROWS_PER_WG_MLA;   // query rows of a row block of the plan
// The e4m3-query kernel's workgroups: 64 rows (half a row block), 8 waves.
constexpr int kRows = 64;
constexpr int kWaves = 8;
static_assert(kBlockRows == 2 * kRows, "a row block is two e4m3-query workgroups");

typedef __attribute__((address_space(3))) uint8_t lds_u8;

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

// Row pitch (floats) of the epilogue's LDS staging: 256 features plus 8, so
// that the sixteen rows of a 16-byte write land in distinct banks.
constexpr int kStagePitch = 264;
constexpr int kStageBytes = kWaves * 16 * kStagePitch * 4;    // 135168
// Row pitch (int16) of the staged partial codes: 256 plus 16, so that rows
// start 8 banks apart and the 8-byte writes of a row's 16 lanes and the
// 8-byte reads of a row are free of bank conflicts.
constexpr int kCodePitch = 272;
static_assert(kWaves * 16 * kCodePitch * 2 <= kStageBytes, "the code staging fits the float staging");

// Epilogue of one wave: lane (n16, qg) of wave half hf holds
// O[row][256 hf + 16 e + 4 qg + i] in o[e][i] (unnormalised, relative to the
// reference max m_ref), the running true max m_true and its part of the
// weight sum l_run (the row's four qg lanes hold parts that add up).  Both
// waves of a pair hold the same (m, l); the hf == 0 wave writes them.
// A single-split sequence's rows go straight to out/lse (normalised).
// Otherwise the partial o is written compactly: each wave's 256 features of
// a row as int16 codes of o / s, with s = (largest |o| of those 256) / 32767
// stored beside them, so a value is off by at most s / 2 = 2^-16 of that
// largest magnitude -- half the bytes of fp32, for the merge to read back.
// The rows go out through LDS (`stage`, kStageBytes of the kernel's tile
// pool, free once every wave has left the tile loop): written there in the
// MFMA layout, read back a row at a time, so that each store instruction
// writes one row's contiguous features -- in register layout a store would
// cover sixteen rows with a few bytes each.
// Must be reached by every wave of the workgroup (it holds a barrier).
__device__ __forceinline__ void store_rows(const PartialParams& p, const f32x4 (&o)[16], int rowv,
                                           int qg, int hf, int b, int slot, int nsplit, float m_ref,
                                           float m_true, float l_run, uint8_t* stage) {
  const bool direct = p.direct && nsplit == 1;
  const int64_t R = int64_t(p.T) * p.Hq;
  // bring (l, o) from the reference max to the true max of the row
  const float f = (m_ref == -INFINITY) ? 0.f : fast_exp2(m_ref - m_true);
  const float m_run = m_true;
  const float l_tot = column_sum4(l_run * f);
  const bool real = rowv < p.rows;
  const int64_t rix = rowv;              // row (t, h) of the sequence is t * Hq + h
  float mul = p.v_scale * f;
  if (direct) mul = l_tot > 0.f ? p.v_scale * f / l_tot : 0.f;
  const int lane = int(threadIdx.x & 63);
  const int wave = int(threadIdx.x >> 6);
  const int n16 = lane & 15;
  const int row0 = rowv - n16;           // the wave's first row
  if (direct) {
    float* st = reinterpret_cast<float*>(stage) + wave * 16 * kStagePitch;
    __syncthreads();                     // every wave is done with the tile pool
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      f32x4 v4 = o[e];
      v4 *= mul;
      *reinterpret_cast<f32x4*>(st + n16 * kStagePitch + 16 * e + 4 * qg) = v4;
    }
    // each wave reads back only what it wrote (no barrier; the LDS waits
    // suffice), all sixteen rows before the first store; rows are in (t, h)
    // order, so a row's index within the sequence is the row number itself
    f32x4 rv4[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) rv4[r] = *reinterpret_cast<const f32x4*>(st + r * kStagePitch + 4 * lane);
    const int d = 256 * hf + 4 * lane;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t rr = row0 + r;
      if (rr >= p.rows) continue;
      const f32x4 v4 = rv4[r];
      const int64_t oo = (int64_t(b) * R + rr) * kDv + d;
      if (p.out_f32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + oo) = v4;
      } else {
        u32x2 pk = {pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3])};
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + oo) = pk;
      }
    }
    if (real && qg == 0 && hf == 0 && p.lse)
      p.lse[int64_t(b) * R + rix] = (m_run == -INFINITY || !(l_tot > 0.f)) ? -INFINITY
                                                                           : (m_run + log2f(l_tot)) * kLn2;
    return;
  }
  // the row's largest |o| over this wave's 256 features (its four qg lanes)
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e)
#pragma unroll
    for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(o[e][i]));
  amax = column_max4(amax) * fabsf(mul);
  const float k = amax > 0.f ? mul * (32767.f / amax) : 0.f;   // code = nearest integer to o * k
  int16_t* st = reinterpret_cast<int16_t*>(stage) + wave * 16 * kCodePitch;
  __syncthreads();                       // every wave is done with the tile pool
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    int c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = int(fminf(fmaxf(rintf(o[e][i] * k), -32767.f), 32767.f));
    const u32x2 w = {(uint32_t(c[0]) & 0xffffu) | (uint32_t(c[1]) << 16),
                     (uint32_t(c[2]) & 0xffffu) | (uint32_t(c[3]) << 16)};
    *reinterpret_cast<u32x2*>(st + n16 * kCodePitch + 16 * e + 4 * qg) = w;
  }
  u32x2 rc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) rc[r] = *reinterpret_cast<const u32x2*>(st + r * kCodePitch + 4 * lane);
  const int d = 256 * hf + 4 * lane;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t rr = row0 + r;
    if (rr >= p.rows) continue;
    *reinterpret_cast<u32x2*>(p.part_q + (int64_t(slot) * R + rr) * kDv + d) = rc[r];
  }
  if (real && qg == 0) {
    p.part_s[(int64_t(slot) * R + rix) * 2 + hf] = amax * (1.f / 32767.f);
    if (hf == 0) {
      p.part_m[int64_t(slot) * R + rix] = m_run == -INFINITY ? -INFINITY : m_run * kLn2;
      p.part_l[int64_t(slot) * R + rix] = l_tot;
    }
  }
}

// The paged-addressing record of a workgroup (its range and a digest of the
// pages its 16-token groups read), when the caller asked for it.
__device__ __forceinline__ void store_debug(const PartialParams& p, int slot, int rb, int b, int split,
                                            int s, int e, int groups, int pxor, uint32_t psum) {
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
