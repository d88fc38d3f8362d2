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
// against (d_qk+d_v)*elem bytes), and at decode sizes mostly bound by memory
// latency: a workgroup's critical path is a chain of dependent loads
// (split record -> block table -> K/V).  The kernel keeps that chain short:
//   * the first argument dwords (cache, table, query and plan pointers, the
//     table stride and the launch geometry) are preloaded into scalar
//     registers at wave launch, so the split record is the first memory
//     access;
//   * block-table entries come through the scalar cache, one group ahead, so
//     waiting for them never waits for K/V vector loads;
//   * every K/V load is a uniform base plus a loop-invariant lane offset;
//   * two groups of K and V are in flight per wave while one is computed
//     (software pipelining over two register sets), in a loop shaped so the
//     compiler's load-completion waits stay exact;
//   * the query goes straight to registers in MFMA operand layout.
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
#include <type_traits>

#include "device.h"

namespace splitkv {

namespace {

// Arguments read after the preloaded ones (they are not on the first load's
// critical path).
struct GqaRest {
  int32_t qsb, qst, qsh;          // query element strides
  int32_t ksp, ksh, kst;          // key byte strides: page, head, token
  int32_t vsp, vsh, vst;          // value byte strides
  int32_t T, Hq, g, page_size, rows, R;   // R = T * Hq output rows per sequence
  float scale_log2;               // scale * k_scale * log2(e)
  float v_scale;
  const int32_t* seq_lens;
  float* part_m;
  float* part_l;
  float* part_o;
  void* out;
  float* lse;
  int32_t* debug;
  int32_t* tickets;               // single launch: [B][Hkv][row blocks] arrival counters
  int32_t out_f32, direct;
};

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

// Buffer resource over the bytes of one 16-token group.  A group past the
// end of the range gets a resource of zero bytes: its loads are still issued
// (so the load-completion counts stay static) but return zeros without a
// memory access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t group_rsrc(const uint8_t* base, bool valid) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, valid ? 0x7fffffff : 0,
                                           0x00020000);
}

// 8 consecutive V features of one token: 4 dwords of bf16 pairs (bf16 cache)
// or 2 dwords of e4m3 codes (FP8 cache, widened later).
// Cache policy of the K/V loads: 0, or 2 (non-temporal, `nt`) for launches
// with a workgroup per compute unit or more.
template <bool FP8, int AUX>
__device__ __forceinline__ u32x4 load_v8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (!FP8) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
  } else {
    const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX));
    u32x4 v = {w.x, w.y, 0u, 0u};
    return v;
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
  u32x4 v[(D + 127) / 128][4];
};


}  // namespace

// Launch geometry packed into one preloaded dword: Hkv (bits 0-15), row
// blocks (16-23), log2(page size) + 1 (24-31; 0 when not a power of two).
template <int D, bool FP8, bool FUSED, bool NT>
__global__ __launch_bounds__(256) void gqa_partial_kernel(
    const int32_t* bt, const int32_t* slot_info, const uint16_t* q, const uint8_t* kc,
    const uint8_t* vc, int32_t bt_stride, int32_t geom, GqaRest a) {
  constexpr int NIT = D / 32;           // QK k-iterations
  constexpr int NC = (D + 127) / 128;   // V feature chunks of 128 per lane-row (D = 64: half of one)
  constexpr int ELEM = FP8 ? 1 : 2;
  constexpr int LDS_STRIDE = D + 4;     // floats; padding against bank conflicts
  constexpr float kRescaleMargin = 8.f; // base-2 growth of a row max before O is rescaled
  __shared__ float sm_o[4][16][LDS_STRIDE];
  __shared__ f32x4 sm_ml[4][16];      // per wave and row: true max, reference max, sum
  __shared__ int sm_dbg[4][3];
  __shared__ int sm_last;

  const int lane = threadIdx.x & 63;
  const int wave = uniform(int(threadIdx.x >> 6));
  const int n16 = lane & 15, qg = lane >> 4;

  const int Hkv = geom & 0xffff;
  const int RB = (geom >> 16) & 0xff;
  const int psh = (geom >> 24) - 1;
  int wg = blockIdx.x;
  const int rb = RB == 1 ? 0 : wg % RB;
  wg = RB == 1 ? wg : wg / RB;
  const int hk = wg % Hkv;
  const int slot = wg / Hkv;
  // One scalar load gives the slot's sequence, split and token range.
  const SlotWork work = load_slot(slot_info, slot);
  const int b = work.b, split = work.split, nsplit = work.nsplit, s = work.s, e = work.e;

  const int P = a.page_size;
  const int32_t* bt_row = bt + int64_t(b) * bt_stride;
  // groups of the range: wave w takes groups w, w+4, w+8, ...
  const int ngroups = (e - s + 15) >> 4;
  const int ngw = ngroups > wave ? (ngroups - wave + 3) >> 2 : 0;

  // Block-table reads go through the scalar cache (constant address space:
  // the table is read-only while the kernel runs), so their completion
  // counter is not the one the in-flight K/V vector loads use.
  cint32* cbt = (cint32*)bt_row;
  auto page_of = [&](int j) -> int {
    const int tok = s + 16 * (wave + 4 * j);
    return cbt[psh >= 0 ? tok >> psh : tok / P];
  };
  int pg_cur = 0, pg_nxt = 0, pg_a = 0, pg_b = 0;   // pages of groups j, j+1, j+2, j+3
  if (ngw > 0) pg_cur = page_of(0);
  if (ngw > 1) pg_nxt = page_of(1);

  // This lane's query row (column of the S^T tile).  Rows past the last query
  // row read row rows-1: their columns are computed and never stored.
  const int row = rb * 16 + n16;
  const int rc = min(row, a.rows - 1);
  const int t = rc / a.g;
  // Causal limit: with one query token every key of the range is visible, so
  // only multi-token decode reads the sequence length.
  int limit = 0x7fffffff;
  if (a.T > 1) limit = ((cint32*)a.seq_lens)[b] - a.T + t;
  bf16x8 qop[NIT];
  {
    const uint16_t* qrow = q + int64_t(b) * a.qsb + int64_t(t) * a.qst + int64_t(hk * a.g + rc % a.g) * a.qsh;
#pragma unroll
    for (int it = 0; it < NIT; ++it)
      qop[it] = *reinterpret_cast<const bf16x8*>(qrow + q_chunk_d0<FP8>(it, qg));
  }

  const uint8_t* kbase = kc + int64_t(hk) * a.ksh;
  const uint8_t* vbase = vc + int64_t(hk) * a.vsh;

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
  const uint32_t koff = uint32_t(n16 * a.kst) + 16u * qg;
  // lane n16 holds value features 8 n16 .. +7 of each 128; with D = 64 the
  // lanes past the row read a copy of the first half (their output rows are
  // never stored)
  const int vl = D >= 128 ? n16 : (n16 & 7);
  uint32_t voff[4];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) voff[jt] = uint32_t((4 * qg + jt) * a.vst) + uint32_t(ELEM * 8 * vl);

  // Group j of this wave (j < ngw loads; later j only keep the counts static).
  // Non-temporal loads (NT) stream faster once the grid fills the chip (a
  // 1 GiB read: 6.7-6.8 against 5.8-6.0 TB/s) but slow a partly filled one
  // (few-KV L=5900, 124 workgroups: 6.8 -> 7.2 us), so the host picks them
  // by the grid size.
  constexpr int kAux = NT ? 2 : 0;
  auto load = [&](int j, int64_t pg, GroupRegs<D, FP8>& r) {
    const bool valid = j < ngw;
    const int tok = s + 16 * (wave + 4 * j);
    const int sl = psh >= 0 ? tok & (P - 1) : tok % P;
    const auto rk = group_rsrc(kbase + pg * a.ksp + int64_t(sl) * a.kst, valid);
    const auto rv = group_rsrc(vbase + pg * a.vsp + int64_t(sl) * a.vst, valid);
    if constexpr (!FP8) {
#pragma unroll
      for (int it = 0; it < NIT; ++it)
        r.k[it] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, koff + 64 * it, 0, kAux));
    } else {
#pragma unroll
      for (int kk = 0; kk < D / 64; ++kk)
        r.k[2 * kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, koff + 64 * kk, 0, kAux));
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int c = 0; c < NC; ++c)
        r.v[c][jt] = load_v8<FP8, kAux>(rv, voff[jt] + ELEM * 128 * c);
  };

  auto compute = [&](int j, GroupRegs<D, FP8>& r) {
    const int g0 = s + 16 * (wave + 4 * j);
    if constexpr (FP8) widen_k_fp8<D>(r.k);
    // two independent accumulation chains halve the dependent MFMA latency
    f32x4 sca = {0.f, 0.f, 0.f, 0.f}, scb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      if (it & 1)
        scb = mfma16x16x32(r.k[it], qop[it], scb);
      else
        sca = mfma16x16x32(r.k[it], qop[it], sca);
    }
    const f32x4 sc = sca + scb;
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tk = g0 + 4 * qg + i;
      sv[i] = (tk < e && tk <= limit) ? sc[i] * a.scale_log2 : -INFINITY;
    }
    const float mx = column_max4(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    m_true = fmaxf(m_true, mx);
    const bool bump = mx > m_ref + kRescaleMargin;
    if (__any(bump)) {
      const float m_new = bump ? mx : m_ref;
      // a row that does not move keeps alpha = 1 exactly: computing it would
      // give exp2(-inf - -inf) = NaN for a row with nothing visible yet
      const float alpha = bump ? fast_exp2(m_ref - m_new) : 1.f;   // 0 on the first visible group
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
  // two groups of loads outstanding.  Inside the steady-state loop every load
  // is unconditional (the loop runs only while groups j+2 and j+3 exist), so
  // the compiler's load-completion waits stay exact; the first two groups are
  // issued unconditionally too (through an empty buffer range when the wave
  // has fewer groups, which costs no memory traffic).  The at most three
  // groups after the loop need at most one more load, issued in the tail, so
  // no load is left in flight when the wave reaches the merge.
  // sched_barrier keeps the scheduler from hoisting compute (and its waits)
  // above a prefetch.
  GroupRegs<D, FP8> ra, rb2;
  load(0, pg_cur, ra);
  load(1, pg_nxt, rb2);
  if (ngw > 2) pg_a = page_of(2);
  if (ngw > 3) pg_b = page_of(3);
  __builtin_amdgcn_sched_barrier(0);
  int j = 0;
  for (; j + 3 < ngw; j += 2) {
    visit(pg_cur);
    compute(j, ra);
    load(j + 2, pg_a, ra);
    pg_cur = pg_a;
    __builtin_amdgcn_sched_barrier(0);
    visit(pg_nxt);
    compute(j + 1, rb2);
    load(j + 3, pg_b, rb2);
    pg_nxt = pg_b;
    if (j + 4 < ngw) pg_a = page_of(j + 4);
    if (j + 5 < ngw) pg_b = page_of(j + 5);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (j < ngw) {
    visit(pg_cur);
    compute(j, ra);
    if (j + 2 < ngw) load(j + 2, pg_a, ra);
  }
  if (j + 1 < ngw) {
    visit(pg_nxt);
    compute(j + 1, rb2);
  }
  if (j + 2 < ngw) {
    visit(pg_a);
    compute(j + 2, ra);
  }

  // ---- per-wave row totals; then merge the four waves through LDS (only
  // the block's real query rows: a KV head with g < 16 query rows leaves
  // the rest of the MFMA block unused)
  l_run = column_sum4(l_run);
  const int nrow = min(16, a.rows - rb * 16);
  // lane (n16, qg) holds O[row n16][128c + 32qg + 8i + e8] in oacc[c*8+e8][i]
  if (n16 < nrow && (D >= 128 || 32 * qg < D)) {
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
  }
  if (qg == 0) {
    sm_ml[wave][n16] = f32x4{m_true, m_ref, l_run, 0.f};
  }
  if (lane == 0) {
    sm_dbg[wave][0] = dbg_groups;
    sm_dbg[wave][1] = dbg_xor;
    sm_dbg[wave][2] = int(dbg_sum);
  }
  __syncthreads();

  const bool direct = a.direct && nsplit == 1;
  const int64_t R = a.R;
  // Thread t merges row t / TPR of the block, float4 columns (t % TPR) +
  // TPR*q, TPR = 256 / RR threads per row for a block of RR rows (8 when
  // the block has at most 8 real rows, else 16): the row's weights are
  // computed by its threads in parallel, and they read (and store) 256 or 512
  // contiguous bytes at a time.
  auto merge = [&](auto rows_c) __attribute__((always_inline)) {
    constexpr int RR = decltype(rows_c)::value;
    constexpr int TPR = 256 / RR < D / 4 ? 256 / RR : D / 4;
    constexpr int NQ = D / 4 / TPR;        // float4 columns per thread
    const int t = threadIdx.x;
    const int row = t / TPR, cl = t % TPR;   // threads past RR * TPR have row >= RR: no store
    f32x4 mlw[4];
    f32x4 ov[4][NQ];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mlw[w] = sm_ml[w][row];
#pragma unroll
      for (int q = 0; q < NQ; ++q) ov[w][q] = *reinterpret_cast<const f32x4*>(&sm_o[w][row][4 * (cl + TPR * q)]);
    }
    // each wave's (l, o) is relative to its reference max; bring all four to
    // the block's true max (reference maxima never exceed the true one)
    const float M = fmaxf(fmaxf(mlw[0][0], mlw[1][0]), fmaxf(mlw[2][0], mlw[3][0]));
    float wgt[4], Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wgt[w] = mlw[w][1] == -INFINITY ? 0.f : fast_exp2(mlw[w][1] - M);
      Lsum += wgt[w] * mlw[w][2];
    }
    if (row < nrow) {
      const int grow = rb * 16 + row;
      const int tt = grow / a.g, hh = hk * a.g + grow - tt * a.g;
      const int64_t rix = int64_t(tt) * a.Hq + hh;
      const bool empty = M == -INFINITY;
      const float mul = direct ? (Lsum > 0.f ? a.v_scale / Lsum : 0.f) : a.v_scale;
      const int64_t obase = ((direct ? int64_t(b) : int64_t(slot)) * R + rix) * D;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        f32x4 acc = wgt[0] * ov[0][q];
#pragma unroll
        for (int w = 1; w < 4; ++w) acc += wgt[w] * ov[w][q];
        acc *= mul;
        const int64_t o = obase + 4 * (cl + TPR * q);
        if (direct) {
          if (a.out_f32) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + o) = acc;
          } else {
            u32x2 pk = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + o) = pk;
          }
        } else {
          *reinterpret_cast<f32x4*>(a.part_o + o) = acc;
        }
      }
      if (cl == 0) {
        if (direct) {
          if (a.lse)
            a.lse[int64_t(b) * R + rix] = (empty || !(Lsum > 0.f)) ? -INFINITY : (M + log2f(Lsum)) * kLn2;
        } else {
          a.part_m[int64_t(slot) * R + rix] = empty ? -INFINITY : M * kLn2;
          a.part_l[int64_t(slot) * R + rix] = Lsum;
        }
      }
    }
  };
  if (nrow <= 8)
    merge(std::integral_constant<int, 8>{});
  else
    merge(std::integral_constant<int, 16>{});
  if (a.debug && threadIdx.x == 0) {
    int groups = 0, x = 0;
    uint32_t sum = 0;
    for (int w = 0; w < 4; ++w) {
      groups += sm_dbg[w][0];
      x ^= sm_dbg[w][1];
      sum += uint32_t(sm_dbg[w][2]);
    }
    int32_t* rec = a.debug + ((int64_t(slot) * Hkv + hk) * RB + rb) * 8;
    rec[0] = b;
    rec[1] = split;
    rec[2] = hk;
    rec[3] = s;
    rec[4] = e;
    rec[5] = groups;
    rec[6] = x;
    rec[7] = int(sum & 0x7fffffffu);
  }
  if constexpr (FUSED) {
    if (nsplit > 1) {
      // Single launch: the workgroups of one (sequence, KV head, row block)
      // count their arrivals in a ticket; the one that arrives last merges
      // the group's partials, so no second kernel is launched.  Each
      // workgroup's partial stores complete before thread 0 releases them at
      // device scope with the ticket increment (the partials of one group are
      // written on every XCD, whose L2 caches are not coherent with each
      // other); the last arriver acquires before it reads them.
      __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0): this wave's stores are done
      __syncthreads();
      if (threadIdx.x == 0) {
        int32_t* ctr = a.tickets + (int64_t(b) * Hkv + hk) * RB + rb;
        const int arrived = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        const int last = arrived == nsplit - 1;
        if (last) {
          // every arrival of this call is in: the counter is left at zero for the next call
          __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        sm_last = last;
      }
      __syncthreads();
      if (sm_last) {
        // log-sum-exp merge of the group's nsplit partials (slots slot - split
        // .. of the sequence), in split order, eight loads in flight per thread;
        // thread t takes (row, float4 column) pairs t, t + 256, ...
        const int base = slot - split;
        constexpr int NCOL = D / 4;
        const int64_t R = a.R;
        for (int pr = threadIdx.x; pr < nrow * NCOL; pr += 256) {
          const int r = pr / NCOL, cq = pr - r * NCOL;
          const int grow = rb * 16 + r;
          const int tt = grow / a.g, hh = hk * a.g + grow - tt * a.g;
          const int64_t rix = int64_t(tt) * a.Hq + hh;
          float M2 = -INFINITY, lam = 0.f;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          for (int i0 = 0; i0 < nsplit; i0 += 8) {
            float mi[8], li[8];
            f32x4 oi[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const int64_t sl = base + min(i0 + u, nsplit - 1);
              mi[u] = a.part_m[sl * R + rix];
              li[u] = a.part_l[sl * R + rix];
              oi[u] = *reinterpret_cast<const f32x4*>(a.part_o + (sl * R + rix) * D + 4 * cq);
              if (i0 + u >= nsplit) mi[u] = -INFINITY;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              if (mi[u] == -INFINITY) continue;          // empty split: zero weight
              const f32x4 ov = oi[u];
              const float m2 = mi[u] * kLog2e;
              const float Mn = fmaxf(M2, m2);
              const float al = fast_exp2(M2 - Mn);
              const float w = fast_exp2(m2 - Mn);
              lam = lam * al + w * li[u];
              acc = acc * al + w * ov;
              M2 = Mn;
            }
          }
          const bool ok = M2 != -INFINITY && lam > 0.f;
          acc *= ok ? 1.f / lam : 0.f;
          const int64_t o = (int64_t(b) * R + rix) * D + 4 * cq;
          if (a.out_f32) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + o) = acc;
          } else {
            u32x2 pk = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + o) = pk;
          }
          if (a.lse && cq == 0) a.lse[int64_t(b) * R + rix] = ok ? (M2 + log2f(lam)) * kLn2 : -INFINITY;
        }
      }
    }
  }
}

// Compute units of the current device, queried once per device.
static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1 << 30;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      return 1 << 30;
    cus[dev] = n;
  }
  return cus[dev];
}

// Host launcher: grid = slots x KV heads x row blocks, 256 threads.
hipError_t launch_gqa_partial(const PartialParams& p, int D, bool fp8, bool fused, hipStream_t stream) {
  GqaRest a;
  a.qsb = int32_t(p.qsb);
  a.qst = int32_t(p.qst);
  a.qsh = int32_t(p.qsh);
  a.ksp = int32_t(p.ksp);
  a.ksh = int32_t(p.ksh);
  a.kst = int32_t(p.kst);
  a.vsp = int32_t(p.vsp);
  a.vsh = int32_t(p.vsh);
  a.vst = int32_t(p.vst);
  a.T = p.T;
  a.Hq = p.Hq;
  a.g = p.g;
  a.page_size = p.page_size;
  a.rows = p.rows;
  a.R = p.T * p.Hq;
  a.scale_log2 = p.scale_log2;
  a.v_scale = p.v_scale;
  a.seq_lens = p.seq_lens;
  a.part_m = p.part_m;
  a.part_l = p.part_l;
  a.part_o = p.part_o;
  a.out = p.out;
  a.lse = p.lse;
  a.debug = p.debug;
  a.tickets = p.tickets;
  a.out_f32 = p.out_f32;
  a.direct = p.direct;
  const int32_t geom = (p.Hkv & 0xffff) | ((p.row_blocks & 0xff) << 16) | ((p.page_shift + 1) << 24);
  const int32_t bt_stride = int32_t(p.bt_stride);
  const dim3 grid(p.total_wg), block(256);
  // non-temporal K/V loads for a grid with a workgroup per compute unit or
  // more (the single launch runs only small grids)
  const bool nt = !fused && p.total_wg >= device_cus();
#define SPLITKV_LAUNCH(DD, F8, FU, NTV)                                                                       \
  hipLaunchKernelGGL((gqa_partial_kernel<DD, F8, FU, NTV>), grid, block, 0, stream, p.bt, p.slot_info, p.q, \
                     p.k, p.v, bt_stride, geom, a)
#define SPLITKV_LAUNCH_D(DD)                                       \
  do {                                                             \
    if (fused) {                                                   \
      if (fp8) SPLITKV_LAUNCH(DD, true, true, false);              \
      else SPLITKV_LAUNCH(DD, false, true, false);                 \
    } else if (nt) {                                               \
      if (fp8) SPLITKV_LAUNCH(DD, true, false, true);              \
      else SPLITKV_LAUNCH(DD, false, false, true);                 \
    } else {                                                       \
      if (fp8) SPLITKV_LAUNCH(DD, true, false, false);             \
      else SPLITKV_LAUNCH(DD, false, false, false);                \
    }                                                              \
  } while (0)
  if (D == 64) SPLITKV_LAUNCH_D(64);
  else if (D == 128) SPLITKV_LAUNCH_D(128);
  else if (D == 256) SPLITKV_LAUNCH_D(256);
  else return hipErrorInvalidValue;
#undef SPLITKV_LAUNCH_D
#undef SPLITKV_LAUNCH
  return hipGetLastError();
}

}  // namespace splitkv
