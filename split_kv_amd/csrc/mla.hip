// MLA split-KV partial kernel for gfx950: one 576-wide latent KV head shared
// by every query head; the value is the first 512 columns of the same row
// ("Shipped: 484.5 tok/s on one GB300 ...", table "What shipped": split-KV
// MLA decode of one request at six speculative tokens, causal within them).
//
// Unlike the grouped-query kernel this one is bound by matrix throughput:
// every cached token meets all T*Hq query rows (768 in the six-token,
// 128-head shape), about 1.67 MFLOP per 1152-byte row.  So a workgroup keeps
// 64 query rows (four waves of 16) and streams the split's tokens through LDS
// in 32-token tiles that all four waves reuse:
//   * tile load: 256 threads fetch 32 x 1152 bytes (16 bytes each, nine
//     per thread) into registers one tile ahead, then store them to LDS;
//   * S^T[token][row] = K Q^T with v_mfma_f32_16x16x32_bf16, Q (16 rows x 576)
//     resident in registers, K read from LDS in the A-operand layout;
//   * online softmax in base 2 as in the grouped kernel;
//   * O^T[d][row] += V^T P^T with V read from LDS 16 bytes per token and
//     transposed in registers (v_perm_b32); O (16 x 512 fp32) stays in
//     accumulator registers.
// Workgroups of one split are placed on one XCD (dispatch is round-robin over
// the eight XCDs) so their re-reads of the split's tiles hit that XCD's L2.
#include "device.h"

namespace splitkv {

namespace {

constexpr int kMlaDqk = 576;
constexpr int kMlaDv = 512;
constexpr int kTile = 32;
constexpr int kRowBytes = kMlaDqk * 2 + 16;      // LDS row pitch, padded
constexpr int kChunks = kMlaDqk * 2 / 16;        // 72 16-byte chunks per row
constexpr int kPerThread = kTile * kChunks / 256; // 9 chunks per thread per tile

__device__ __forceinline__ void transpose8x8_m(const u32x4 (&w)[8], bf16x8 (&op)[8]) {
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

__global__ __launch_bounds__(256) void mla_partial_kernel(PartialParams p, int per_xcd) {
  __shared__ __attribute__((aligned(16))) uint8_t smk[kTile * kRowBytes];

  // XCD-aware placement: block id i runs on XCD i % 8; give each XCD a
  // contiguous run of (slot, row block) work items.
  const int xcd = blockIdx.x & 7;
  const int gidx = xcd * per_xcd + int(blockIdx.x >> 3);
  if (gidx >= p.total_wg) return;
  const int rb = gidx % p.row_blocks;
  const int slot = gidx / p.row_blocks;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int n16 = lane & 15, qg = lane >> 4;

  const SlotWork work = load_slot(p.slot_info, slot);
  const int b = work.b, split = work.split, nsplit = work.nsplit, s = work.s, e = work.e;
  const int L = ((cint32*)p.seq_lens)[b];

  const int row = rb * 64 + wave * 16 + n16;   // row = t * Hq + h
  const bool row_ok = row < p.rows;
  const int t = row_ok ? row / p.Hq : 0;
  const int h = row_ok ? row % p.Hq : 0;
  const int limit = L - p.T + t;

  bf16x8 qop[kMlaDqk / 32];
  {
    const uint16_t* qrow = p.q + b * p.qsb + t * p.qst + h * p.qsh;
#pragma unroll
    for (int it = 0; it < kMlaDqk / 32; ++it)
      qop[it] = row_ok ? *reinterpret_cast<const bf16x8*>(qrow + 32 * it + 8 * qg)
                       : bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }

  f32x4 oacc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) oacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  // m_ref: reference max of the exponentials (moves only when a row max grows
  // by more than kRescaleMargin, so the accumulators are rarely touched by
  // vector ALU code); m_true: the row's true running max.
  constexpr float kRescaleMargin = 8.f;
  float m_ref = -INFINITY, m_true = -INFINITY, l_run = 0.f;

  const int P = p.page_size;
  const int psh = p.page_shift;
  const int32_t* bt_row = p.bt + b * p.bt_stride;
  cint32* cbt = (cint32*)bt_row;

  // Tile fetch into registers: thread (token tid / 8, lane-in-row tid % 8)
  // copies 16-byte chunks j, j+8, ..., j+64 of its token's 1152-byte row, so a
  // thread needs one page lookup per tile.
  const int ftok = tid >> 3, fj = tid & 7;
  auto fetch = [&](int tile, u32x4 (&regs)[kPerThread]) {
    const int gt = tile + ftok;
    if (gt < e) {
      const int64_t pg = bt_row[psh >= 0 ? gt >> psh : gt / P];
      const int sl = psh >= 0 ? gt & (P - 1) : gt % P;
      const uint8_t* src = p.k + pg * p.ksp + int64_t(sl) * p.kst + 16 * fj;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) regs[k] = *reinterpret_cast<const u32x4*>(src + 128 * k);
    } else {
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) regs[k] = u32x4{0u, 0u, 0u, 0u};   // past the range: zeros
    }
  };

  int dbg_groups = 0, dbg_xor = 0;
  uint32_t dbg_sum = 0;
  u32x4 regs[kPerThread];
  if (s < e) fetch(s, regs);
  for (int tile = s; tile < e; tile += kTile) {
    __syncthreads();                           // previous tile fully consumed
#pragma unroll
    for (int k = 0; k < kPerThread; ++k)
      *reinterpret_cast<u32x4*>(smk + ftok * kRowBytes + 16 * (fj + 8 * k)) = regs[k];
    __syncthreads();
    if (tile + kTile < e) fetch(tile + kTile, regs);

    const bool has1 = tile + 16 < e;
    {
      const int pg0 = cbt[psh >= 0 ? tile >> psh : tile / P];
      const int pg1 = has1 ? cbt[psh >= 0 ? (tile + 16) >> psh : (tile + 16) / P] : 0;
      dbg_groups += has1 ? 2 : 1;
      dbg_xor ^= pg0 ^ pg1;
      dbg_sum += uint32_t(pg0) + uint32_t(pg1);
    }

    // ---- S^T = K Q^T for the two 16-token groups (two accumulation chains each)
    f32x4 sc0 = {0.f, 0.f, 0.f, 0.f}, sc1 = {0.f, 0.f, 0.f, 0.f};
    f32x4 sc0b = {0.f, 0.f, 0.f, 0.f}, sc1b = {0.f, 0.f, 0.f, 0.f};
    const uint8_t* k0 = smk + n16 * kRowBytes + 16 * qg;
    const uint8_t* k1 = k0 + 16 * kRowBytes;
#pragma unroll
    for (int it = 0; it < kMlaDqk / 32; it += 2) {
      sc0 = mfma16x16x32(*reinterpret_cast<const bf16x8*>(k0 + 64 * it), qop[it], sc0);
      sc1 = mfma16x16x32(*reinterpret_cast<const bf16x8*>(k1 + 64 * it), qop[it], sc1);
      sc0b = mfma16x16x32(*reinterpret_cast<const bf16x8*>(k0 + 64 * (it + 1)), qop[it + 1], sc0b);
      sc1b = mfma16x16x32(*reinterpret_cast<const bf16x8*>(k1 + 64 * (it + 1)), qop[it + 1], sc1b);
    }
    sc0 += sc0b;
    sc1 += sc1b;
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ta = tile + 4 * qg + i, tb = tile + 16 + 4 * qg + i;
      sv[i] = (ta < e && ta <= limit) ? sc0[i] * p.scale_log2 : -INFINITY;
      sv[4 + i] = (tb < e && tb <= limit) ? sc1[i] * p.scale_log2 : -INFINITY;
    }
    float mx = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
    mx = column_max4(mx);
    m_true = fmaxf(m_true, mx);
    const bool bump = mx > m_ref + kRescaleMargin;
    if (__any(bump)) {
      const float m_new = bump ? mx : m_ref;
      const float alpha = fast_exp2(m_ref - m_new);   // 0 on the first visible tile
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < 32; ++c) oacc[c] *= alpha;
      m_ref = m_new;
    }
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pv[i] = fast_exp2(sv[i] - m_use);
    l_run += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
    u32x4 pw = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
    const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);

    // ---- O^T += V^T P^T; V = first 512 columns of the tile rows
#pragma unroll
    for (int c = 0; c < kMlaDv / 128; ++c) {
      u32x4 vw[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tk = (j < 4 ? 0 : 16) + 4 * qg + (j & 3);
        vw[j] = *reinterpret_cast<const u32x4*>(smk + tk * kRowBytes + 2 * (128 * c + 8 * n16));
      }
      bf16x8 vop[8];
      transpose8x8_m(vw, vop);
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) oacc[c * 8 + e8] = mfma16x16x32(vop[e8], pop, oacc[c * 8 + e8]);
    }
  }

  // bring (l, o) from the reference max to the true max of the row
  {
    const float f = (m_ref == -INFINITY) ? 0.f : fast_exp2(m_ref - m_true);
    l_run *= f;
#pragma unroll
    for (int c = 0; c < 32; ++c) oacc[c] *= f;
  }
  const float m_run = m_true;
  l_run = column_sum4(l_run);
  const bool direct = p.direct && nsplit == 1;
  if (row_ok) {
    const int64_t R = int64_t(p.T) * p.Hq;
    const int64_t rix = int64_t(t) * p.Hq + h;
    float mul = p.v_scale;
    if (direct) mul = l_run > 0.f ? p.v_scale / l_run : 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e4 = 0; e4 < 2; ++e4) {
          const int d = 128 * c + 32 * qg + 8 * i + 4 * e4;
          f32x4 v4 = {oacc[c * 8 + 4 * e4 + 0][i], oacc[c * 8 + 4 * e4 + 1][i],
                      oacc[c * 8 + 4 * e4 + 2][i], oacc[c * 8 + 4 * e4 + 3][i]};
          v4 *= mul;
          if (direct) {
            const int64_t o = (int64_t(b) * R + rix) * kMlaDv + d;
            if (p.out_f32) {
              *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + o) = v4;
            } else {
              u32x2 pk = {pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3])};
              *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + o) = pk;
            }
          } else {
            *reinterpret_cast<f32x4*>(p.part_o + (int64_t(slot) * R + rix) * kMlaDv + d) = v4;
          }
        }
    if (qg == 0) {
      const bool empty = m_run == -INFINITY;
      if (direct) {
        if (p.lse)
          p.lse[int64_t(b) * R + rix] =
              (empty || !(l_run > 0.f)) ? -INFINITY : (m_run + log2f(l_run)) * kLn2;
      } else {
        p.part_m[int64_t(slot) * R + rix] = empty ? -INFINITY : m_run * kLn2;
        p.part_l[int64_t(slot) * R + rix] = l_run;
      }
    }
  }
  if (p.debug && tid == 0) {
    int32_t* rec = p.debug + (int64_t(slot) * p.row_blocks + rb) * 8;
    rec[0] = b;
    rec[1] = split;
    rec[2] = 0;
    rec[3] = s;
    rec[4] = e;
    rec[5] = dbg_groups;
    rec[6] = dbg_xor;
    rec[7] = int(dbg_sum & 0x7fffffffu);
  }
}

hipError_t launch_mla_partial(const PartialParams& p, hipStream_t stream) {
  const int per_xcd = (p.total_wg + 7) / 8;
  const dim3 grid(unsigned(per_xcd * 8)), block(256);
  hipLaunchKernelGGL(mla_partial_kernel, grid, block, 0, stream, p, per_xcd);
  return hipGetLastError();
}

}  // namespace splitkv
