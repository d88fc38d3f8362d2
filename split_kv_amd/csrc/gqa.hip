// Grouped-query split-KV partial kernel for gfx950 (bf16 or e4m3 paged cache).
//
// One workgroup serves one (slot, KV head, block of 16 query rows); a slot is
// one split of one sequence ("vLLM 0.30.0 FA4 SplitKV Bug: H100 Decode Can Be
// 48% Slower", section "What SplitKV is trying to do": each split computes a
// partial attention result over its own KV range).  The four waves of the
// workgroup take interleaved 32-token blocks of the range, keep their own
// running (m, l, o) and merge through LDS at the end, so a split streams its
// range with four independent load streams and writes one partial.
//
// Data path per 32-token block (two 16-token groups), all in registers:
//   * K rows go straight from HBM into the MFMA A-operand layout (lane = token,
//     16 bytes of the feature dimension per load); e4m3 codes widen exactly to
//     bf16 on the way ("Xqa decode kernels", section "Purpose": bf16 queries
//     over an FP8 KV cache).
//   * S^T[token][row] = K Q^T with v_mfma_f32_16x16x32_bf16; tokens sit on M so
//     a row's scores land in one lane column and the row max needs two lane
//     exchanges.
//   * online softmax in base 2 (scale * log2 e folded into one multiply).
//   * O^T[d][row] += V^T P^T: each lane loads 16 contiguous bytes of V for each
//     of its 8 tokens (fully coalesced per quarter-wave) and transposes them in
//     registers with v_perm_b32, so P never leaves the register file and the
//     per-row rescale factor is local to the lane.
// The kernel is bound by HBM bandwidth for these shapes: per token it does
// 2*g*(d_qk + d_v) FLOPs against (d_qk + d_v) * elem bytes.
#include "device.h"

namespace splitkv {

namespace {

template <bool FP8>
__device__ __forceinline__ int q_chunk_d0(int it, int qg) {
  // Feature offset of the 8 elements lane-group qg holds in k-iteration it.
  // It must match how the K operand is loaded (see load_k_group).
  return FP8 ? 64 * (it >> 1) + 16 * qg + 8 * (it & 1) : 32 * it + 8 * qg;
}

// K operand of one 16-token group: lane (token n16, group qg).
template <int D, bool FP8>
__device__ __forceinline__ void load_k_group(const uint8_t* krow, bf16x8 (&kop)[D / 32], int qg) {
  if constexpr (!FP8) {
#pragma unroll
    for (int it = 0; it < D / 32; ++it)
      kop[it] = *reinterpret_cast<const bf16x8*>(krow + 2 * (32 * it + 8 * qg));
  } else {
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(krow + 64 * kk + 16 * qg);
      const u32x2 a = e4m3x4_to_bf16x4(w.x), b = e4m3x4_to_bf16x4(w.y);
      const u32x2 c = e4m3x4_to_bf16x4(w.z), d = e4m3x4_to_bf16x4(w.w);
      u32x4 lo = {a.x, a.y, b.x, b.y}, hi = {c.x, c.y, d.x, d.y};
      kop[2 * kk] = __builtin_bit_cast(bf16x8, lo);
      kop[2 * kk + 1] = __builtin_bit_cast(bf16x8, hi);
    }
  }
}

// 8 consecutive V features of one token, as 4 dwords of bf16 pairs.
template <bool FP8>
__device__ __forceinline__ u32x4 load_v8(const uint8_t* p) {
  if constexpr (!FP8) {
    return *reinterpret_cast<const u32x4*>(p);
  } else {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    const u32x2 a = e4m3x4_to_bf16x4(w.x), b = e4m3x4_to_bf16x4(w.y);
    u32x4 r = {a.x, a.y, b.x, b.y};
    return r;
  }
}

// Transpose 8 tokens x 8 features (bf16) held as w[token] into 8 MFMA
// operands op[feature] of 8 tokens each.
__device__ __forceinline__ void transpose8x8(const u32x4 (&w)[8], bf16x8 (&op)[8]) {
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    u32x4 ev, od;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const uint32_t a = w[2 * y][x], b = w[2 * y + 1][x];
      ev[y] = __builtin_amdgcn_perm(b, a, 0x05040100u);
      od[y] = __builtin_amdgcn_perm(b, a, 0x07060302u);
    }
    op[2 * x] = __builtin_bit_cast(bf16x8, ev);
    op[2 * x + 1] = __builtin_bit_cast(bf16x8, od);
  }
}

}  // namespace

template <int D, bool FP8>
__global__ __launch_bounds__(256) void gqa_partial_kernel(PartialParams p) {
  constexpr int NIT = D / 32;           // QK k-iterations
  constexpr int NC = D / 128;           // V feature chunks of 128 per lane-row
  constexpr int ELEM = FP8 ? 1 : 2;
  constexpr int LDS_STRIDE = D + 4;     // floats; padding against bank conflicts
  __shared__ float sm_o[4][16][LDS_STRIDE];
  __shared__ float sm_m[4][16], sm_l[4][16];
  __shared__ int sm_dbg[4][3];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(int(threadIdx.x >> 6));
  const int n16 = lane & 15, qg = lane >> 4;

  int wg = blockIdx.x;
  const int rb = wg % p.row_blocks;
  wg /= p.row_blocks;
  const int hk = wg % p.Hkv;
  const int slot = wg / p.Hkv;
  const int packed = p.slot_seq[slot];
  const int b = packed >> 8, split = packed & 255;
  const int L = p.seq_lens[b];
  const int nsplit = p.num_splits[b];
  int s, e;
  split_bounds(L, nsplit, split, &s, &e);

  // This lane's query row (column of the S^T tile).
  const int row = rb * 16 + n16;
  const bool row_ok = row < p.rows;
  const int t = row_ok ? row / p.g : 0;
  const int h = hk * p.g + (row_ok ? row % p.g : 0);
  const int limit = L - p.T + t;        // last visible key position

  bf16x8 qop[NIT];
  {
    const uint16_t* qrow = p.q + b * p.qsb + t * p.qst + h * p.qsh;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      if (row_ok)
        qop[it] = *reinterpret_cast<const bf16x8*>(qrow + q_chunk_d0<FP8>(it, qg));
      else
        qop[it] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  f32x4 oacc[NC * 8];
#pragma unroll
  for (int c = 0; c < NC * 8; ++c) oacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  int dbg_groups = 0, dbg_xor = 0;
  uint32_t dbg_sum = 0;

  const int P = p.page_size;
  const int32_t* bt_row = p.bt + b * p.bt_stride;
  const uint8_t* kbase = p.k + hk * p.ksh;
  const uint8_t* vbase = p.v + hk * p.vsh;

  for (int blk = s + 32 * wave; blk < e; blk += 128) {
    const int tok1 = blk + 16;
    const bool has1 = tok1 < e;
    const int64_t pg0 = bt_row[blk / P];
    const int64_t pg1 = has1 ? int64_t(bt_row[tok1 / P]) : pg0;
    const int sl0 = blk % P, sl1 = tok1 % P;
    dbg_groups += has1 ? 2 : 1;
    dbg_xor ^= int(pg0) ^ (has1 ? int(pg1) : 0);
    dbg_sum += uint32_t(pg0) + (has1 ? uint32_t(pg1) : 0u);

    // ---- K operands (lane = token n16 of each group)
    bf16x8 k0[NIT], k1[NIT];
    load_k_group<D, FP8>(kbase + pg0 * p.ksp + (sl0 + n16) * p.kst, k0, qg);
    if (has1) load_k_group<D, FP8>(kbase + pg1 * p.ksp + (sl1 + n16) * p.kst, k1, qg);

    // ---- V rows: lane (n16, qg) owns tokens 4qg..4qg+3 of each group
    u32x4 vw[NC][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool g1 = j >= 4;
      const int tok_in = 4 * qg + (j & 3);
      if (!g1 || has1) {
        const uint8_t* vrow = vbase + (g1 ? pg1 : pg0) * p.vsp + ((g1 ? sl1 : sl0) + tok_in) * p.vst;
#pragma unroll
        for (int c = 0; c < NC; ++c) vw[c][j] = load_v8<FP8>(vrow + ELEM * (128 * c + 8 * n16));
      } else {
#pragma unroll
        for (int c = 0; c < NC; ++c) vw[c][j] = u32x4{0u, 0u, 0u, 0u};
      }
    }

    // ---- scores S^T = K Q^T (lane holds row n16, tokens 4qg+i of each group)
    f32x4 sc0 = {0.f, 0.f, 0.f, 0.f}, sc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < NIT; ++it) sc0 = mfma16x16x32(k0[it], qop[it], sc0);
    if (has1) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) sc1 = mfma16x16x32(k1[it], qop[it], sc1);
    }
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ta = blk + 4 * qg + i, tb = tok1 + 4 * qg + i;
      sv[i] = (ta < e && ta <= limit) ? sc0[i] * p.scale_log2 : -INFINITY;
      sv[4 + i] = (has1 && tb < e && tb <= limit) ? sc1[i] * p.scale_log2 : -INFINITY;
    }
    float mx = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
    mx = fmaxf(mx, xor_shfl(mx, 16));
    mx = fmaxf(mx, xor_shfl(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float pv[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = exp2f(sv[i] - m_use);
      psum += pv[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    u32x4 pw = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
    const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);

    // Tokens past the range end sit in the same (valid) page but may hold
    // anything, NaN included; P is zero there but 0 * NaN is not, so clear V.
    if (blk + 32 > e) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tk = (j < 4 ? blk : tok1) + 4 * qg + (j & 3);
        if (tk >= e) {
#pragma unroll
          for (int c = 0; c < NC; ++c) vw[c][j] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 vop[8];
      transpose8x8(vw[c], vop);
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        f32x4 acc = oacc[c * 8 + e8] * alpha;
        oacc[c * 8 + e8] = mfma16x16x32(vop[e8], pop, acc);
      }
    }
  }

  // ---- per-wave row totals; then merge the four waves through LDS
  l_run += xor_shfl(l_run, 16);
  l_run += xor_shfl(l_run, 32);
  // lane (n16, qg) holds O[row n16][128c + 32qg + 8i + e8] in oacc[c*8+e8][i]
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e4 = 0; e4 < 2; ++e4) {
        f32x4 v4 = {oacc[c * 8 + 4 * e4 + 0][i], oacc[c * 8 + 4 * e4 + 1][i],
                    oacc[c * 8 + 4 * e4 + 2][i], oacc[c * 8 + 4 * e4 + 3][i]};
        *reinterpret_cast<f32x4*>(&sm_o[wave][n16][128 * c + 32 * qg + 8 * i + 4 * e4]) = v4;
      }
  if (qg == 0) {
    sm_m[wave][n16] = m_run;
    sm_l[wave][n16] = l_run;
  }
  if (lane == 0) {
    sm_dbg[wave][0] = dbg_groups;
    sm_dbg[wave][1] = dbg_xor;
    sm_dbg[wave][2] = int(dbg_sum);
  }
  __syncthreads();

  const bool direct = p.direct && nsplit == 1;
  {
    const int r = threadIdx.x >> 4;       // row within the block
    const int part = threadIdx.x & 15;    // D/16 features each
    const int grow = rb * 16 + r;
    if (grow < p.rows) {
      float M = sm_m[0][r];
#pragma unroll
      for (int w = 1; w < 4; ++w) M = fmaxf(M, sm_m[w][r]);
      float wgt[4], Lsum = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        wgt[w] = sm_m[w][r] == -INFINITY ? 0.f : exp2f(sm_m[w][r] - M);
        Lsum += wgt[w] * sm_l[w][r];
      }
      const int tt = grow / p.g, hh = hk * p.g + grow % p.g;
      const int64_t R = int64_t(p.T) * p.Hq;
      const int64_t rix = int64_t(tt) * p.Hq + hh;
      float mul = p.v_scale;
      if (direct) mul = Lsum > 0.f ? p.v_scale / Lsum : 0.f;
      constexpr int PER = D / 16;
#pragma unroll
      for (int k4 = 0; k4 < PER / 4; ++k4) {
        const int d = part * PER + 4 * k4;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < 4; ++w)
          acc += wgt[w] * *reinterpret_cast<const f32x4*>(&sm_o[w][r][d]);
        acc *= mul;
        if (direct) {
          const int64_t o = (int64_t(b) * R + rix) * D + d;
          if (p.out_f32) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + o) = acc;
          } else {
            u32x2 pk = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + o) = pk;
          }
        } else {
          const int64_t o = (int64_t(slot) * R + rix) * D + d;
          *reinterpret_cast<f32x4*>(p.part_o + o) = acc;
        }
      }
      if (part == 0) {
        const bool empty = M == -INFINITY;
        if (direct) {
          if (p.lse)
            p.lse[int64_t(b) * R + rix] =
                (empty || !(Lsum > 0.f)) ? -INFINITY : (M + log2f(Lsum)) * kLn2;
        } else {
          p.part_m[int64_t(slot) * R + rix] = empty ? -INFINITY : M * kLn2;
          p.part_l[int64_t(slot) * R + rix] = Lsum;
        }
      }
    }
  }
  if (p.debug && threadIdx.x == 0) {
    int groups = 0, x = 0;
    uint32_t sum = 0;
    for (int w = 0; w < 4; ++w) {
      groups += sm_dbg[w][0];
      x ^= sm_dbg[w][1];
      sum += uint32_t(sm_dbg[w][2]);
    }
    int32_t* rec = p.debug + ((int64_t(slot) * p.Hkv + hk) * p.row_blocks + rb) * 8;
    rec[0] = b;
    rec[1] = split;
    rec[2] = hk;
    rec[3] = s;
    rec[4] = e;
    rec[5] = groups;
    rec[6] = x;
    rec[7] = int(sum & 0x7fffffffu);
  }
}

// Host launcher: grid = slots x KV heads x row blocks, 256 threads.
hipError_t launch_gqa_partial(const PartialParams& p, int D, bool fp8, hipStream_t stream) {
  const dim3 grid(p.total_wg), block(256);
  if (D == 128 && !fp8) hipLaunchKernelGGL((gqa_partial_kernel<128, false>), grid, block, 0, stream, p);
  else if (D == 256 && !fp8) hipLaunchKernelGGL((gqa_partial_kernel<256, false>), grid, block, 0, stream, p);
  else if (D == 128 && fp8) hipLaunchKernelGGL((gqa_partial_kernel<128, true>), grid, block, 0, stream, p);
  else if (D == 256 && fp8) hipLaunchKernelGGL((gqa_partial_kernel<256, true>), grid, block, 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace splitkv
