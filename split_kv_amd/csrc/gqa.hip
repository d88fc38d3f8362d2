// Grouped-query split-KV partial kernel for gfx950 (bf16 or e4m3 paged cache).
//
// One workgroup serves one (slot, KV head, block of 16 query rows); a slot is
// one split of one sequence ("vLLM 0.30.0 FA4 SplitKV Bug: H100 Decode Can Be
// 48% Slower", section "What SplitKV is trying to do": each split computes a
// partial attention result over its own KV range).  The four waves of the
// workgroup take interleaved 16-token groups of the range, keep their own
// running (m, l, o) and merge through LDS at the end, so a split streams its
// range with four independent load streams and writes one partial.
//
// Decode attention is memory-bound here (per token 2*g*(d_qk+d_v) FLOPs
// against (d_qk+d_v)*elem bytes), and at decode sizes mostly memory-latency
// bound, so the kernel is organised around keeping loads in flight:
//   * block-table entries come through the scalar cache, one group ahead, so
//     waiting for them never waits for K/V vector loads;
//   * every K/V load is a uniform base plus a loop-invariant lane offset;
//   * the next group's K and V are loaded into a second register set while
//     the current group is computed (software pipelining, distance one), in a
//     loop shaped so the compiler's load-completion waits stay exact.
// Per 16-token group, all in registers:
//   * K rows go straight from HBM into the MFMA A-operand layout (lane = token,
//     16 bytes of the feature dimension per load); e4m3 codes widen exactly to
//     bf16 on the way ("Xqa decode kernels", section "Purpose": bf16 queries
//     over an FP8 KV cache);
//   * S^T[token][row] = K Q^T with v_mfma_f32_16x16x32_bf16; tokens sit on M so
//     a row's scores land in one lane column and the row max needs two lane
//     exchanges;
//   * online softmax in base 2 (scale * log2 e folded into one multiply); the
//     exponentials use a reference max that moves only when a row max grows
//     by more than 2^8, so O is rarely rescaled (the true max is tracked
//     separately and the merge brings every wave to it);
//   * O^T[d][row] += V^T P^T with v_mfma_f32_16x16x16_bf16: each lane loads 16
//     contiguous bytes of V for each of its 4 tokens (a quarter-wave reads 256
//     contiguous bytes) and transposes them in registers with v_perm_b32, so P
//     never leaves the register file.
#include "device.h"

namespace splitkv {

namespace {

template <bool FP8>
__device__ __forceinline__ int q_chunk_d0(int it, int qg) {
  // Feature offset of the 8 elements lane-group qg holds in k-iteration it.
  // It must match how the K operand is loaded (the load lambda of the kernel).
  return FP8 ? 64 * (it >> 1) + 16 * qg + 8 * (it & 1) : 32 * it + 8 * qg;
}

template <int D>
__device__ __forceinline__ void widen_k_fp8(bf16x8 (&kop)[D / 32]) {
#pragma unroll
  for (int kk = D / 64 - 1; kk >= 0; --kk) {
    const u32x4 w = __builtin_bit_cast(u32x4, kop[2 * kk]);
    const u32x2 a = e4m3x4_to_bf16x4(w.x), b = e4m3x4_to_bf16x4(w.y);
    const u32x2 c = e4m3x4_to_bf16x4(w.z), d = e4m3x4_to_bf16x4(w.w);
    u32x4 lo = {a.x, a.y, b.x, b.y}, hi = {c.x, c.y, d.x, d.y};
    kop[2 * kk] = __builtin_bit_cast(bf16x8, lo);
    kop[2 * kk + 1] = __builtin_bit_cast(bf16x8, hi);
  }
}

// 8 consecutive V features of one token: 4 dwords of bf16 pairs (bf16 cache)
// or 2 dwords of e4m3 codes (FP8 cache, widened later).
template <bool FP8>
__device__ __forceinline__ u32x4 load_v8(const uint8_t* p) {
  if constexpr (!FP8) {
    return *reinterpret_cast<const u32x4*>(p);
  } else {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    u32x4 r = {w.x, w.y, 0u, 0u};
    return r;
  }
}

template <bool FP8>
__device__ __forceinline__ u32x4 widen_v8(u32x4 w) {
  if constexpr (!FP8) {
    return w;
  } else {
    const u32x2 a = e4m3x4_to_bf16x4(w.x), b = e4m3x4_to_bf16x4(w.y);
    u32x4 r = {a.x, a.y, b.x, b.y};
    return r;
  }
}

// Transpose 4 tokens x 8 features (bf16) held as w[token] into 8 MFMA
// operands op[feature] of 4 tokens each.  sel_ev/sel_od are the v_perm byte
// selectors for even/odd features of the token pairs (0,1) and (2,3); a
// selector byte of 0x0C yields 0x00, which is how tokens past the end of the
// range are zeroed at no extra cost.
__device__ __forceinline__ void transpose4x8(const u32x4 (&w)[4], bf16x4 (&op)[8],
                                             const uint32_t (&sel_ev)[2], const uint32_t (&sel_od)[2]) {
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    u32x2 ev, od;
    ev.x = __builtin_amdgcn_perm(w[1][x], w[0][x], sel_ev[0]);
    ev.y = __builtin_amdgcn_perm(w[3][x], w[2][x], sel_ev[1]);
    od.x = __builtin_amdgcn_perm(w[1][x], w[0][x], sel_od[0]);
    od.y = __builtin_amdgcn_perm(w[3][x], w[2][x], sel_od[1]);
    op[2 * x] = __builtin_bit_cast(bf16x4, ev);
    op[2 * x + 1] = __builtin_bit_cast(bf16x4, od);
  }
}

template <int D, bool FP8>
struct GroupRegs {
  bf16x8 k[D / 32];
  u32x4 v[D / 128][4];
};

}  // namespace

template <int D, bool FP8>
__global__ __launch_bounds__(256) void gqa_partial_kernel(PartialParams p) {
  constexpr int NIT = D / 32;           // QK k-iterations
  constexpr int NC = D / 128;           // V feature chunks of 128 per lane-row
  constexpr int ELEM = FP8 ? 1 : 2;
  constexpr int LDS_STRIDE = D + 4;     // floats; padding against bank conflicts
  constexpr bool Q_IN_LDS = D >= 256;   // frees 32 VGPRs for the wide head dim
  constexpr int QROW = D + 8;           // bf16 elements per LDS query row (padded)
  constexpr float kRescaleMargin = 8.f; // base-2 growth of a row max before O is rescaled
  __shared__ float sm_o[4][16][LDS_STRIDE];
  __shared__ float sm_m[4][16], sm_r[4][16], sm_l[4][16];
  __shared__ int sm_dbg[4][3];
  __shared__ __attribute__((aligned(16))) uint16_t sm_q[Q_IN_LDS ? 16 : 1][QROW];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(int(threadIdx.x >> 6));
  const int n16 = lane & 15, qg = lane >> 4;

  int wg = blockIdx.x;
  const int rb = wg % p.row_blocks;
  wg /= p.row_blocks;
  const int hk = wg % p.Hkv;
  const int slot = wg / p.Hkv;
  // One scalar load gives the slot's sequence, split and token range.
  const SlotWork work = load_slot(p.slot_info, slot);
  const int b = work.b, split = work.split, nsplit = work.nsplit, s = work.s, e = work.e;

  // This lane's query row (column of the S^T tile).
  const int row = rb * 16 + n16;
  const int t = row < p.rows ? row / p.g : 0;
  // Causal limit: with one query token every key of the range is visible, so
  // only multi-token decode reads the sequence length.
  int limit = 0x7fffffff;
  if (p.T > 1) limit = ((cint32*)p.seq_lens)[b] - p.T + t;

  // Query operand: issued now, consumed after the first K/V loads are in flight.
  bf16x8 qop[Q_IN_LDS ? 1 : NIT];
  constexpr int QCH = Q_IN_LDS ? (16 * (D / 8)) / 256 : 1;   // 16-byte chunks per thread
  bf16x8 qstage[QCH];
  if constexpr (Q_IN_LDS) {
#pragma unroll
    for (int k = 0; k < QCH; ++k) {
      const int c = threadIdx.x + 256 * k;
      const int r = c / (D / 8), d8 = c % (D / 8);
      // Rows past the last query row load row rows-1 and are zeroed when
      // staged: an unconditional load keeps the completion count exact.
      const int gr = min(rb * 16 + r, p.rows - 1);
      const int tt = gr / p.g, hh = hk * p.g + gr % p.g;
      qstage[k] = *reinterpret_cast<const bf16x8*>(p.q + b * p.qsb + tt * p.qst + hh * p.qsh + 8 * d8);
    }
  } else {
    const int rc = min(row, p.rows - 1);
    const uint16_t* qrow = p.q + b * p.qsb + (rc / p.g) * p.qst + (hk * p.g + rc % p.g) * p.qsh;
#pragma unroll
    for (int it = 0; it < NIT; ++it)
      qop[it] = *reinterpret_cast<const bf16x8*>(qrow + q_chunk_d0<FP8>(it, qg));
  }

  const int P = p.page_size;
  const int32_t* bt_row = p.bt + b * p.bt_stride;
  const uint8_t* kbase = p.k + hk * p.ksh;
  const uint8_t* vbase = p.v + hk * p.vsh;

  // groups of the range: wave w takes groups w, w+4, w+8, ...
  const int ngroups = (e - s + 15) >> 4;
  const int ngw = ngroups > wave ? (ngroups - wave + 3) >> 2 : 0;

  // Block-table reads go through the scalar cache (constant address space:
  // the table is read-only while the kernel runs), so their completion
  // counter is not the one the in-flight K/V vector loads use.  Each group's
  // page is fetched one group ahead.
  cint32* cbt = (cint32*)bt_row;
  const int psh = p.page_shift;
  auto page_of = [&](int j) -> int {
    const int tok = s + 16 * (wave + 4 * j);
    return cbt[psh >= 0 ? tok >> psh : tok / P];
  };

  f32x4 oacc[NC * 8];
#pragma unroll
  for (int c = 0; c < NC * 8; ++c) oacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  // m_ref: reference max the exponentials use (moves only when a row max grows
  // by more than kRescaleMargin); m_true: the row's true running max.
  float m_ref = -INFINITY, m_true = -INFINITY, l_run = 0.f;
  int dbg_groups = 0, dbg_xor = 0;
  uint32_t dbg_sum = 0;

  // Per-lane byte offsets inside a 16-token group are loop-invariant; each
  // load is a uniform (scalar) base plus one of them, so the loop needs no
  // per-iteration vector address arithmetic.
  const uint32_t koff = uint32_t(n16 * p.kst) + 16u * qg;
  uint32_t voff[4];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) voff[jt] = uint32_t((4 * qg + jt) * p.vst) + uint32_t(ELEM * 8 * n16);

  auto load = [&](int j, int64_t pg, GroupRegs<D, FP8>& r) {
    const int tok = s + 16 * (wave + 4 * j);
    const int sl = psh >= 0 ? tok & (P - 1) : tok % P;
    const uint8_t* kb = kbase + pg * p.ksp + int64_t(sl) * p.kst;
    const uint8_t* vb = vbase + pg * p.vsp + int64_t(sl) * p.vst;
    if constexpr (!FP8) {
#pragma unroll
      for (int it = 0; it < NIT; ++it)
        r.k[it] = *reinterpret_cast<const bf16x8*>(kb + koff + 64 * it);
    } else {
#pragma unroll
      for (int kk = 0; kk < D / 64; ++kk)
        r.k[2 * kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kb + koff + 64 * kk));
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int c = 0; c < NC; ++c)
        r.v[c][jt] = load_v8<FP8>(vb + voff[jt] + ELEM * 128 * c);
  };

  auto compute = [&](int j, GroupRegs<D, FP8>& r) {
    const int g0 = s + 16 * (wave + 4 * j);
    if constexpr (FP8) widen_k_fp8<D>(r.k);
    // two independent accumulation chains halve the dependent MFMA latency
    f32x4 sca = {0.f, 0.f, 0.f, 0.f}, scb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      bf16x8 qv;
      if constexpr (Q_IN_LDS)
        qv = *reinterpret_cast<const bf16x8*>(&sm_q[n16][q_chunk_d0<FP8>(it, qg)]);
      else
        qv = qop[it];
      if (it & 1)
        scb = mfma16x16x32(r.k[it], qv, scb);
      else
        sca = mfma16x16x32(r.k[it], qv, sca);
    }
    const f32x4 sc = sca + scb;
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tk = g0 + 4 * qg + i;
      sv[i] = (tk < e && tk <= limit) ? sc[i] * p.scale_log2 : -INFINITY;
    }
    const float mx = column_max4(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    m_true = fmaxf(m_true, mx);
    const bool bump = mx > m_ref + kRescaleMargin;
    if (__any(bump)) {
      const float m_new = bump ? mx : m_ref;
      const float alpha = fast_exp2(m_ref - m_new);   // 0 on the first visible group
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < NC * 8; ++c) oacc[c] *= alpha;
      m_ref = m_new;
    }
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = fast_exp2(sv[i] - m_use);
    l_run += (pv[0] + pv[1]) + (pv[2] + pv[3]);
    u32x2 pw = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
    const bf16x4 pop = __builtin_bit_cast(bf16x4, pw);

    // Tokens past the range end sit in the same (valid) page but may hold
    // anything, NaN included; P is zero there but 0 * NaN is not, so their V
    // bytes are replaced by zeros inside the transpose.
    uint32_t sel_ev[2] = {0x05040100u, 0x05040100u}, sel_od[2] = {0x07060302u, 0x07060302u};
    if (g0 + 16 > e) {
      const int tb = g0 + 4 * qg;
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        const bool lo = tb + 2 * y < e, hi = tb + 2 * y + 1 < e;
        sel_ev[y] = (lo ? 0x0100u : 0x0C0Cu) | (hi ? 0x05040000u : 0x0C0C0000u);
        sel_od[y] = (lo ? 0x0302u : 0x0C0Cu) | (hi ? 0x07060000u : 0x0C0C0000u);
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 w[4];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) w[jt] = widen_v8<FP8>(r.v[c][jt]);
      bf16x4 vop[8];
      transpose4x8(w, vop, sel_ev, sel_od);
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) oacc[c * 8 + e8] = mfma16x16x16(vop[e8], pop, oacc[c * 8 + e8]);
    }
  };

  auto visit = [&](int64_t pg) {
    dbg_groups += 1;
    dbg_xor ^= int(pg);
    dbg_sum += uint32_t(pg);
  };

  // Software pipeline over two register sets: groups j and j+1 are in
  // flight before group j is computed, and each set is refilled (group j+2,
  // j+3) as soon as its group has been consumed, so a wave always has one or
  // two groups of loads outstanding.  Prefetches are unconditional (clamped
  // to the last group, whose lines they then re-read from cache) and the loop
  // has a single exit at its end, so no control-flow path reaches the loop
  // head with loads the compiler cannot account for -- otherwise it waits for
  // every load at the top of each iteration.  sched_barrier keeps the
  // scheduler from hoisting compute (and its waits) above a prefetch.  The
  // first two groups are issued before the query is staged, so the query
  // and block-table latencies overlap them.  A wave without groups issues
  // the same loads from page 0 (which always exists) and never uses them:
  // the loads stay unconditional, so the wait for the query stays exact.
  GroupRegs<D, FP8> ra, rb2;
  int pg_cur = 0, pg_nxt = 0, pg_a = 0, pg_b = 0;   // pages of groups j, j+1, j+2, j+3
  if (ngw > 0) {
    pg_cur = page_of(0);
    pg_nxt = page_of(min(1, ngw - 1));
  }
  load(0, pg_cur, ra);
  load(min(1, max(ngw - 1, 0)), pg_nxt, rb2);
  if (ngw > 0) {
    pg_a = page_of(min(2, ngw - 1));
    pg_b = page_of(min(3, ngw - 1));
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (Q_IN_LDS) {
#pragma unroll
    for (int k = 0; k < QCH; ++k) {
      const int c = threadIdx.x + 256 * k;
      const int r = c / (D / 8);
      const bf16x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
      *reinterpret_cast<bf16x8*>(&sm_q[r][8 * (c % (D / 8))]) = rb * 16 + r < p.rows ? qstage[k] : zero;
    }
    __syncthreads();
  }
  for (int j = 0; j < ngw; j += 2) {
    visit(pg_cur);
    compute(j, ra);
    load(min(j + 2, ngw - 1), pg_a, ra);
    pg_cur = pg_a;
    pg_a = page_of(min(j + 4, ngw - 1));
    __builtin_amdgcn_sched_barrier(0);
    if (j + 1 < ngw) {
      visit(pg_nxt);
      compute(j + 1, rb2);
    }
    load(min(j + 3, ngw - 1), pg_b, rb2);
    pg_nxt = pg_b;
    pg_b = page_of(min(j + 5, ngw - 1));
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- per-wave row totals; then merge the four waves through LDS
  l_run = column_sum4(l_run);
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
    sm_m[wave][n16] = m_true;
    sm_r[wave][n16] = m_ref;
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
      // each wave's (l, o) is relative to its reference max; bring all four
      // to the block's true max
      float M = sm_m[0][r];
#pragma unroll
      for (int w = 1; w < 4; ++w) M = fmaxf(M, sm_m[w][r]);
      float wgt[4], Lsum = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mr = sm_r[w][r];
        wgt[w] = mr == -INFINITY ? 0.f : exp2f(mr - M);
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
