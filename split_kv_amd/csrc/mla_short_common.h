// Pieces of the short-range MLA partial kernels (64 query rows and eight
// waves per workgroup; bf16 and e4m3 queries): the epilogue that writes a
// workgroup's partial (m, l, o) or, for a single-split sequence, the final
// output and log-sum-exp, and the paged-addressing record.  The direct
// global->LDS loads and the LDS barrier are the 128-row kernel's.
#pragma once

#include "mla_common.h"

namespace splitkv {
namespace mla_short {

using mla::dma16;
using mla::dma16_sbase;
using mla::lds_barrier;
using mla::lds_u8;

constexpr int kDqk = 576;                        // latent row: 512 value features + 64 rope
constexpr int kDv = 512;
constexpr int kRows = 64;                        // query rows per workgroup
constexpr int kWaves = 8;
static_assert(2 * kRows == SPLITKV_ROWS_PER_WG_MLA, "a plan row block is two of these workgroups");

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
  // o * kq lies in [-1, 1]; v_cvt_pknorm_i16_f32 takes two such values to
  // the nearest multiples of 1/32767, as int16 codes
  const float kq = amax > 0.f ? mul / amax : 0.f;
  int16_t* st = reinterpret_cast<int16_t*>(stage) + wave * 16 * kCodePitch;
  __syncthreads();                       // every wave is done with the tile pool
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const u32x2 w = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(o[e][0] * kq, o[e][1] * kq)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(o[e][2] * kq, o[e][3] * kq))};
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
// pages its 16-token groups read), when the caller asked for it: records are
// kept in the plan's 128-row blocks, each two of these 64-row workgroups,
// and the first of the two writes it.
__device__ __forceinline__ void store_debug(const PartialParams& p, int slot, int rb, int b, int split,
                                            int s, int e, int groups, int pxor, uint32_t psum) {
  if (rb & 1) return;
  int32_t* rec = p.debug + (int64_t(slot) * ((p.row_blocks + 1) >> 1) + (rb >> 1)) * 8;
  rec[0] = b;
  rec[1] = split;
  rec[2] = 0;
  rec[3] = s;
  rec[4] = e;
  rec[5] = groups;
  rec[6] = pxor;
  rec[7] = int(psum & 0x7fffffffu);
}

}  // namespace mla_short
}  // namespace splitkv
