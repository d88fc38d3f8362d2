// MLA split-KV partial kernel for gfx950: one 576-wide latent KV head shared
// by every query head; the value is the first 512 columns of the same row
// ("Shipped: 484.5 tok/s on one GB300 ...", table "What shipped": split-KV
// MLA decode of one request at six speculative tokens, causal within them).
//
// Unlike the grouped-query kernel this one is bound by matrix throughput:
// every cached token meets all T*Hq query rows (768 in the six-token,
// 128-head shape), 1,671,168 FLOPs per 1152-byte row.  A workgroup keeps 64
// query rows and streams the split's tokens through LDS in 32-token tiles:
//   * tiles arrive by direct global->LDS loads (16 bytes per lane, no
//     register staging) into a ring of three, two tiles ahead of the one
//     being computed;
//   * a token's 1152 bytes sit at a pitch of 73 16-byte chunks, which makes
//     both operand reads conflict-free: sixteen lanes reading one chunk of
//     sixteen tokens fall in sixteen different bank groups (73 = 9 mod 16),
//     and sixteen lanes reading sixteen chunks of one token are contiguous;
//   * the four waves form two pairs; a pair owns 32 query rows (two blocks
//     of 16), and its two waves split the feature dimension: each computes
//     the partial scores over half of the 576 key features for all 32 rows,
//     the two swap partials through LDS (fp32, summed in the same order by
//     both, so both hold bit-identical scores and softmax state), and each
//     accumulates O over half of the 512 value features.  Every operand read
//     from LDS feeds two MFMAs (one per block), so LDS traffic per FLOP is
//     half that of 16 rows per wave, while the query (32 rows x 288, 72
//     VGPRs) and O (32 rows x 256 fp32, 128 accumulation registers) fit;
//   * per tile: every K operand read of the tile is issued before its MFMAs
//     (LDS latency otherwise stalls the single wave per SIMD), S^T[token][row]
//     = K Q^T with v_mfma_f32_16x16x32_bf16, one partial exchange, then the
//     online softmax in base 2 (lazily moved reference max) over the tile's
//     32 tokens, and O^T[d][row] += V^T P^T with v_mfma_f32_16x16x32_bf16 over
//     all 32 tokens at once, V read from LDS 16 bytes per token and
//     transposed in registers (v_perm_b32).
// Workgroups of one split are placed on one XCD (dispatch is round-robin over
// the eight XCDs), so the row blocks' reads of a tile share that XCD's L2.
#include "device.h"

namespace splitkv {

namespace {

constexpr int kMlaDqk = 576;
constexpr int kMlaDv = 512;
constexpr int kTile = 32;                        // tokens per LDS tile
constexpr int kPitch = 73;                       // 16-byte chunks per token row (72 + 1 pad)
constexpr int kChunks = kMlaDqk * 2 / 16;        // 72 chunks of a token's row
constexpr int kTileChunks = kTile * kPitch;      // 2336
constexpr int kTileLoads = (kTileChunks + 63) / 64;   // 37 wave-level 1 KB loads
constexpr int kLoadsPerWave = (kTileLoads + 3) / 4;   // 10: every wave issues the same count
constexpr int kSlotBytes = kTileLoads * 1024;    // 37888
constexpr int kRing = 3;
constexpr int kRows = 64;                        // query rows per workgroup
constexpr int kQk = kMlaDqk / 32 / 2;            // 9 k-steps of 32 key features per half
constexpr int kPv = kMlaDv / 128 / 2;            // 2 chunks of 128 value features per half
static_assert(kSlotBytes >= kTileChunks * 16, "slot holds a tile");
static_assert(SPLITKV_ROWS_PER_WG_MLA == kRows, "rows per workgroup");

typedef __attribute__((address_space(3))) void lds_void;

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

// Workgroup barrier after this wave's LDS operations have completed (a bare
// s_barrier does not wait for them); the signal fences keep the compiler from
// moving memory operations across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace

__global__ __launch_bounds__(256) void mla_partial_kernel(PartialParams p, int per_xcd) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRing][kSlotBytes];
  // partial-score exchange: [wave][group][block][lane]
  __shared__ f32x4 xch[4][2][2][64];

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
  const int pair = wave >> 1, hf = wave & 1;      // hf: which half of the features
  const int n16 = lane & 15, qg = lane >> 4;

  const SlotWork work = load_slot(p.slot_info, slot);
  const int b = work.b, split = work.split, nsplit = work.nsplit, s = work.s, e = work.e;
  const int L = ((cint32*)p.seq_lens)[b];

  // This lane's two query rows (columns of the S^T tiles of the two blocks);
  // rows past the last one read row rows-1 and are never stored.  The wave
  // holds its half of their key features.
  int rowv[2], limit[2];
  bf16x8 q0[kQk], q1[kQk];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    rowv[sb] = rb * kRows + pair * 32 + sb * 16 + n16;
    const int rc = min(rowv[sb], p.rows - 1);
    const int t = rc / p.Hq, h = rc % p.Hq;
    limit[sb] = L - p.T + t;
    const uint16_t* qrow = p.q + b * p.qsb + t * p.qst + h * p.qsh + 32 * kQk * hf + 8 * qg;
#pragma unroll
    for (int it = 0; it < kQk; ++it) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 32 * it);
      if (sb == 0) q0[it] = v;
      else q1[it] = v;
    }
  }

  // The page size is a power of two for this kernel (checked on the host).
  const int psh = p.page_shift;
  const int pmask = p.page_size - 1;
  cint32* cbt = (cint32*)(p.bt + b * p.bt_stride);
  const uint32_t ksp = uint32_t(p.ksp), kst = uint32_t(p.kst);   // < 2^31, checked on the host

  // Tile fill: wave w issues the wave-level loads w, w+4, ..., w+36 of the
  // 37 a tile needs; a wave with fewer repeats its last load (same lanes,
  // same addresses, same bytes), so every wave issues ten per tile and the
  // completion counts are the same for all.  Lane j of load i fills the
  // 16-byte chunk q = 64*i + j of the slot: token q / 73, chunk q % 73.  The
  // pad chunk and the chunks past the tile reload a valid chunk; tokens past
  // the range end load the range's last token (finite, masked later).  A
  // 32-token tile starting on a multiple of 16 spans at most two pages.
  const int nt = (e - s + kTile - 1) / kTile;      // tiles of the range
  // (token, byte offset) of every chunk this lane fills, the same for every tile
  uint32_t fl[kLoadsPerWave];
#pragma unroll
  for (int u = 0; u < kLoadsPerWave; ++u) {
    int i = wave + 4 * u;
    if (i >= kTileLoads) i -= 4;
    const uint32_t q = uint32_t(64 * i + lane);
    uint32_t tk = (q * 1796u) >> 17;                  // q / 73 for q < 3640
    uint32_t c = q - tk * kPitch;
    if (tk >= uint32_t(kTile)) tk = kTile - 1;
    if (c >= uint32_t(kChunks)) c = 0;
    fl[u] = (tk << 16) | (16u * c);
  }
  auto fill = [&](int k, uint8_t* slotp) __attribute__((always_inline)) {
    const int t0 = s + kTile * min(k, nt - 1);      // beyond the last tile: reload it
    const int last = min(t0 + kTile - 1, e - 1);
    const int pi0 = t0 >> psh;
    const uint64_t base0 = uint64_t(uint32_t(cbt[pi0])) * ksp;
    const uint64_t base1 = uint64_t(uint32_t(cbt[last >> psh])) * ksp;
#pragma unroll
    for (int u = 0; u < kLoadsPerWave; ++u) {
      int i = wave + 4 * u;
      if (i >= kTileLoads) i -= 4;
      const int tok = min(t0 + int(fl[u] >> 16), last);
      const uint64_t base = (tok >> psh) == pi0 ? base0 : base1;
      const uint8_t* src = p.k + (base + uint64_t(uint32_t(tok & pmask) * kst + (fl[u] & 0xffffu)));
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(slotp + 1024 * i), 16, 0, 0);
    }
  };

  // O^T accumulators of the two blocks over this wave's value half: lane
  // (n16, qg) holds O[row n16][256hf + 128c + 32qg + 8i + e8] in o[c*8+e8][i].
  f32x4 o0[kPv * 8], o1[kPv * 8];
#pragma unroll
  for (int c = 0; c < kPv * 8; ++c) {
    o0[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    o1[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  constexpr float kRescaleMargin = 8.f;
  float m_ref[2] = {-INFINITY, -INFINITY}, m_true[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  int dbg_groups = 0, dbg_xor = 0;
  uint32_t dbg_sum = 0;

  // One 32-token tile in slotp, tokens t0 .. t0+31 of the range.
  auto tile = [&](const uint8_t* slotp, int t0) __attribute__((always_inline)) {
    // ---- partial S^T = K Q^T over this wave's key half for both 16-token
    // groups and both blocks: all eighteen operand reads first, then the
    // MFMAs, four independent accumulation chains.
    const uint8_t* krow = slotp + n16 * (kPitch * 16) + 16 * qg + 64 * kQk * hf;
    bf16x8 k0[kQk], k1[kQk];
#pragma unroll
    for (int it = 0; it < kQk; ++it) {
      k0[it] = *reinterpret_cast<const bf16x8*>(krow + 64 * it);
      k1[it] = *reinterpret_cast<const bf16x8*>(krow + 16 * (kPitch * 16) + 64 * it);
    }
    f32x4 s00 = {0.f, 0.f, 0.f, 0.f}, s01 = {0.f, 0.f, 0.f, 0.f};
    f32x4 s10 = {0.f, 0.f, 0.f, 0.f}, s11 = {0.f, 0.f, 0.f, 0.f};   // s[group][block]
#pragma unroll
    for (int it = 0; it < kQk; ++it) {
      s00 = mfma16x16x32(k0[it], q0[it], s00);
      s01 = mfma16x16x32(k0[it], q1[it], s01);
      s10 = mfma16x16x32(k1[it], q0[it], s10);
      s11 = mfma16x16x32(k1[it], q1[it], s11);
    }
    // ---- swap partials with the pair's other wave; both sum own + other,
    // the same two values, so both hold identical scores
    xch[wave][0][0][lane] = s00;
    xch[wave][0][1][lane] = s01;
    xch[wave][1][0][lane] = s10;
    xch[wave][1][1][lane] = s11;
    lds_barrier();
    const int w2 = wave ^ 1;
    const f32x4 sc[2][2] = {{s00 + xch[w2][0][0][lane], s01 + xch[w2][0][1][lane]},
                            {s10 + xch[w2][1][0][lane], s11 + xch[w2][1][1][lane]}};
    // ---- online softmax over the tile: lane (n16, qg) holds tokens
    // 4qg..4qg+3 of each group for row n16 of each block
    float sv[2][8], mx[2];
    bool bump[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tk = t0 + 16 * g + 4 * qg + i;
          sv[sb][4 * g + i] = (tk < e && tk <= limit[sb]) ? sc[g][sb][i] * p.scale_log2 : -INFINITY;
        }
      float m8 = sv[sb][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) m8 = fmaxf(m8, sv[sb][i]);
      mx[sb] = column_max4(m8);
      m_true[sb] = fmaxf(m_true[sb], mx[sb]);
      bump[sb] = mx[sb] > m_ref[sb] + kRescaleMargin;
    }
    if (__any(bump[0] || bump[1])) {
      float alpha[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const float m_new = bump[sb] ? mx[sb] : m_ref[sb];
        alpha[sb] = fast_exp2(m_ref[sb] - m_new);   // 0 on the first visible tile, 1 if unmoved
        l_run[sb] *= alpha[sb];
        m_ref[sb] = m_new;
      }
#pragma unroll
      for (int c = 0; c < kPv * 8; ++c) {
        o0[c] *= alpha[0];
        o1[c] *= alpha[1];
      }
    }
    bf16x8 pop[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const float m_use = m_ref[sb] == -INFINITY ? 0.f : m_ref[sb];
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pv[i] = fast_exp2(sv[sb][i] - m_use);
      l_run[sb] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
      u32x4 pw = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                  pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
      pop[sb] = __builtin_bit_cast(bf16x8, pw);
    }
    // ---- O^T += V^T P^T over this wave's value half, all 32 tokens per MFMA:
    // k index 8qg + j is token (j < 4 ? 0 : 16) + 4qg + (j & 3), for V and P
    // alike.  The next chunk's eight rows are read while the current chunk is
    // multiplied.
    const uint8_t* vrow = slotp + (4 * qg) * (kPitch * 16) + 16 * n16 + 256 * kPv * hf;
    auto vld = [&](int c, u32x4 (&w)[8]) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        w[j] = *reinterpret_cast<const u32x4*>(vrow + ((j < 4 ? 0 : 16) + (j & 3)) * (kPitch * 16) + 256 * c);
    };
    u32x4 wcur[8];
    vld(0, wcur);
#pragma unroll
    for (int c = 0; c < kPv; ++c) {
      bf16x8 vop[8];
      transpose8x8(wcur, vop);
      if (c + 1 < kPv) vld(c + 1, wcur);
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        o0[c * 8 + e8] = mfma16x16x32(vop[e8], pop[0], o0[c * 8 + e8]);
        o1[c * 8 + e8] = mfma16x16x32(vop[e8], pop[1], o1[c * 8 + e8]);
      }
    }
  };

  // Tile k: wait until this wave's loads of tile k are done (the ten loads
  // of tile k+1 may still be in flight), then a barrier so every wave's part
  // of the tile has landed -- which also means every wave has finished tile
  // k-1 (its LDS reads and its partial exchange), so its slot can be
  // refilled with tile k+2 and the exchange buffer reused.  Tiles past the range
  // reload the last tile (never computed), so the counts stay static.
  auto step = [&](int k) __attribute__((always_inline)) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70 | 10);               // vmcnt(10)
    lds_barrier();
    fill(k + 2, ring[(k + 2) % kRing]);
    const uint8_t* cur = ring[k % kRing];
    const int t0 = s + kTile * k;
    {
      const int pg0 = cbt[t0 >> psh];
      const bool has1 = t0 + 16 < e;
      const int pg1 = has1 ? cbt[(t0 + 16) >> psh] : 0;
      dbg_groups += has1 ? 2 : 1;
      dbg_xor ^= pg0 ^ pg1;
      dbg_sum += uint32_t(pg0) + uint32_t(pg1);
    }
    tile(cur, t0);
  };

  if (nt > 0) {
    fill(0, ring[0]);
    fill(1, ring[1]);
    for (int k = 0; k < nt; ++k) step(k);
  }
  // no wave leaves while loads it issued may still write LDS
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);                      // vmcnt(0)

  const bool direct = p.direct && nsplit == 1;
  const int64_t R = int64_t(p.T) * p.Hq;
  auto finish = [&](int sb, const f32x4 (&oacc)[kPv * 8]) __attribute__((always_inline)) {
    // bring (l, o) from the reference max to the true max of the row
    const float f = (m_ref[sb] == -INFINITY) ? 0.f : fast_exp2(m_ref[sb] - m_true[sb]);
    const float m_run = m_true[sb];
    const float l_tot = column_sum4(l_run[sb] * f);
    const int row = rowv[sb];
    if (row >= p.rows) return;
    const int t = row / p.Hq, h = row % p.Hq;
    const int64_t rix = int64_t(t) * p.Hq + h;
    float mul = p.v_scale * f;
    if (direct) mul = l_tot > 0.f ? p.v_scale * f / l_tot : 0.f;
#pragma unroll
    for (int c = 0; c < kPv; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e4 = 0; e4 < 2; ++e4) {
          const int d = 256 * hf + 128 * c + 32 * qg + 8 * i + 4 * e4;
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
    // both waves of the pair hold the same (m, l); one writes them
    if (qg == 0 && hf == 0) {
      const bool empty = m_run == -INFINITY;
      if (direct) {
        if (p.lse)
          p.lse[int64_t(b) * R + rix] =
              (empty || !(l_tot > 0.f)) ? -INFINITY : (m_run + log2f(l_tot)) * kLn2;
      } else {
        p.part_m[int64_t(slot) * R + rix] = empty ? -INFINITY : m_run * kLn2;
        p.part_l[int64_t(slot) * R + rix] = l_tot;
      }
    }
  };
  finish(0, o0);
  finish(1, o1);

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
