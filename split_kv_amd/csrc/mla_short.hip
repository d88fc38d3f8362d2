// Short-range MLA split-KV partial kernel for gfx950: one 576-wide latent KV
// head shared by every query head; the value is the first 512 columns of the
// same row ("Shipped: 484.5 tok/s on one GB300 ...", table "What shipped":
// split-KV MLA decode of one request at six speculative tokens, causal within
// them).  The host runs it instead of the 128-row kernel (mla.hip) when the
// step is short: every split at most eight 32-token tiles and the 64-row
// workgroups all on the compute units at once.  There its two waves per SIMD
// hide the fixed costs of a workgroup (query in, partial out) that the
// 128-row kernel's one wave per SIMD cannot; per tile it does less work per
// byte of LDS read, so long ranges go to the 128-row kernel.
//
// Unlike the grouped-query kernel this one is bound by matrix throughput:
// every cached token meets all T*Hq query rows (768 in the six-token,
// 128-head shape), 1,671,168 FLOPs per 1152-byte row.  A workgroup keeps 64
// query rows and streams the split's tokens through LDS in 32-token tiles:
//   * tiles arrive by direct global->LDS loads (16 bytes per lane, no
//     register staging) into a ring of four, three tiles ahead of the one
//     being computed (the loads of a tile take longer than two tiles of
//     compute), issued after a tile's partial-score exchange so that the
//     tile's own K reads and QK go first;
//   * a token's 72 16-byte chunks are stored unpadded with chunk c of tile
//     token t at position c ^ swz(t) -- a permutation inside each aligned
//     group of eight, swz(t) a 3-bit table entry for t mod 16 -- which keeps
//     both operand reads (K: one chunk of sixteen tokens per sixteen lanes;
//     V: the transposing reads below) free of bank conflicts; the unpadded
//     tile is what lets four of them fit in LDS;
//   * eight waves, two per SIMD, so that one wave's LDS reads, exchange and
//     softmax overlap the other's matrix work; they form four pairs, a pair
//     owns 16 query rows, and its two waves split the feature dimension: each
//     computes the partial scores over half of the 576 key features, the two
//     swap partials through LDS (fp32, summed in the same order by both, so
//     both hold bit-identical scores and softmax state; a wave takes every
//     other 32-feature k-step, which keeps its K reads on one swizzle
//     pattern), and each accumulates
//     O over half of the 512 value features.  The query (16 rows x 288, 36
//     VGPRs) and O (16 rows x 256 fp32, 64 registers) leave room for two
//     waves per SIMD;
//   * per tile: every K operand read of the tile is issued before its MFMAs
//     (so no MFMA waits on a read issued just before it), S^T[token][row]
//     = K Q^T with v_mfma_f32_16x16x32_bf16, one partial exchange, then the
//     online softmax in base 2 (lazily moved reference max) over the tile's
//     32 tokens, and O^T[d][row] += V^T P^T with v_mfma_f32_16x16x32_bf16 over
//     all 32 tokens at once, the V^T operand read straight from the
//     token-major tile with the gfx950 transposing LDS read
//     (ds_read_b64_tr_b16): a 16-lane group that points at 4 tokens x 4
//     consecutive features receives, in lane x, feature x of the 4 tokens.
// An e4m3 latent cache (bf16 queries, "Xqa decode kernels", section
// "Purpose") runs the same tile code: its codes, half the bytes, arrive the
// same way into a four-deep code ring and are widened exactly to bf16 at the
// start of each step into a two-deep ring of bf16 tiles laid out as above.
// Workgroups of one split are placed on one XCD (dispatch is round-robin over
// the eight XCDs), so the row blocks' reads of a tile share that XCD's L2.
// The block-table entries a tile fill needs are read one step ahead, so the
// fill's address computation never waits for them.
#include "mla_short_common.h"

namespace splitkv {

namespace {

using namespace mla_short;
constexpr int kMlaDqk = kDqk;
constexpr int kMlaDv = kDv;
constexpr int kTile = 32;                        // tokens per LDS tile
constexpr int kPitch = kMlaDqk * 2 / 16;         // 72 16-byte chunks per token row, unpadded
constexpr int kTileChunks = kTile * kPitch;      // 2304
constexpr int kTileLoads = kTileChunks / 64;          // 36 wave-level 1 KB loads
constexpr int kLoadsPerWave = (kTileLoads + kWaves - 1) / kWaves;   // 5: every wave issues the same count
constexpr int kSlotBytes = kTileLoads * 1024;    // 36864
constexpr int kRing = 4;
// e4m3 cache: a tile's codes (32 x 576 bytes) are 18 wave-level loads; waves
// 0-1 issue three, the others two plus a repeat of their second, so every
// wave issues three.  The codes land in a four-deep staging ring and are
// widened into a two-deep ring of bf16 tiles laid out as above.
constexpr int kF8Pitch = kMlaDqk / 16;                // 36 16-byte chunks per code row
constexpr int kF8TileLoads = kTile * kMlaDqk / 1024;  // 18
constexpr int kF8LoadsPerWave = 3;
constexpr int kF8StageBytes = kF8TileLoads * 1024;    // 18432
constexpr int kPoolBytes = kRing * kSlotBytes;        // 147456 either way
static_assert(2 * kSlotBytes + 4 * kF8StageBytes == kPoolBytes, "e4m3 rings fill the pool");
static_assert((kF8LoadsPerWave - 1) * kWaves < kF8TileLoads && kF8LoadsPerWave * kWaves >= kF8TileLoads,
              "three loads per wave cover an e4m3 tile");
constexpr int kQk = kMlaDqk / 32 / 2;            // 9 k-steps of 32 key features per half
constexpr int kPv = kMlaDv / 128 / 2;            // 2 chunks of 128 value features per half
static_assert(kSlotBytes == kTileChunks * 16 && kTileChunks % 64 == 0, "slot holds a tile");
static_assert(kStageBytes <= kPoolBytes, "the epilogue's staging fits the tile pool");

typedef __attribute__((address_space(3))) void lds_void;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Position swizzle of a tile token's 16-byte chunks: entry t & 15 of a
// 16-entry table of 3-bit values, chosen (by search against measured gfx950
// LDS behaviour: 16-byte reads are served 32 lanes at a time from 128
// four-byte banks, transposing 8-byte reads 32 lanes at a time from 64) so
// that both the K reads and the transposing value reads are conflict-free.
__device__ __forceinline__ uint32_t swz(uint32_t t) {
  return uint32_t((0x8c87fc16ec52ull >> (3 * (t & 15u))) & 7u);
}

}  // namespace

template <bool FP8>
__global__ __launch_bounds__(512) void mla_short_partial_kernel(PartialParams p, int per_xcd) {
  // bf16: four tile slots.  e4m3: two bf16 tile slots, then four code slots.
  __shared__ __attribute__((aligned(1024))) uint8_t pool[kPoolBytes];
  constexpr int kLPW = FP8 ? kF8LoadsPerWave : kLoadsPerWave;   // loads per wave and tile
  auto tile_slot = [&](int k) __attribute__((always_inline)) {
    return pool + (FP8 ? (k & 1) : (k & 3)) * kSlotBytes;
  };
  auto fill_slot = [&](int k) __attribute__((always_inline)) {
    return FP8 ? pool + 2 * kSlotBytes + (k & 3) * kF8StageBytes : pool + (k & 3) * kSlotBytes;
  };
  // partial-score exchange: [wave][group][lane]
  __shared__ f32x4 xch[kWaves][2][64];

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

  // This lane's query row (column of the S^T tiles); rows past the last one
  // read row rows-1 and are never stored.  The wave holds its half of the
  // row's key features.
  const int rowv = rb * kRows + pair * 16 + n16;
  int limit;
  bf16x8 q[kQk];
  {
    const int rc = min(rowv, p.rows - 1);
    const int t = rc / p.Hq, h = rc % p.Hq;
    limit = L - p.T + t;      // last key position this row sees
    // k-step it of this wave is k-step 2*it + hf of the row: features 64*it + 32*hf + 8*qg ..
    const uint16_t* qrow = p.q + b * p.qsb + t * p.qst + h * p.qsh + 32 * hf + 8 * qg;
#pragma unroll
    for (int it = 0; it < kQk; ++it) q[it] = *reinterpret_cast<const bf16x8*>(qrow + 64 * it);
  }
  // The query's loads stay in flight while the first tile fills are issued
  // (below); the wait for all of them comes before the tile loop.

  // Tiles that end at or before full_end need no mask: every token is in the
  // range and visible to every row of the wave (its first row has the
  // smallest causal limit).
  const int full_end = min(e, L - p.T + min(rb * kRows + pair * 16, p.rows - 1) / p.Hq + 1);

  // The page size is a power of two for this kernel (checked on the host).
  const int psh = p.page_shift;
  const int pmask = p.page_size - 1;
  cint32* cbt = (cint32*)(p.bt + b * p.bt_stride);
  const uint32_t ksp = uint32_t(p.ksp), kst = uint32_t(p.kst);   // < 2^31, checked on the host

  // Tile fill: wave w issues the wave-level loads w, w+8, ..., w+32 of the
  // 36 a tile needs; a wave with fewer repeats its last load (same lanes,
  // same addresses, same bytes), so every wave issues five per tile and the
  // completion counts are the same for all.  Lane j of load i fills the
  // 16-byte position q = 64*i + j of the slot: token q / 72, holding chunk
  // (q % 72) ^ swz(token) of that token's row.  Tokens past the range
  // end load the range's last token (finite, masked later).  A 32-token tile
  // starting on a multiple of 16 spans at most two pages.
  const int nt = (e - s + kTile - 1) / kTile;      // tiles of the range
  // (token, byte offset) of every chunk this lane fills, the same for every tile
  // Loads 0-17 hold tokens 0-15 and loads 18-35 tokens 16-31 (16 x 72 =
  // 18 x 64 chunks), and a 16-token half of a tile lies in one page (tiles
  // start on multiples of 16, pages hold a power of two >= 16 tokens), so for
  // a tile inside the range a load reads one page: its address is a uniform
  // page base plus the lane's offset inside the half, lo[u].
  // For an e4m3 cache, lane j of load i fills 16-byte position q = 64*i + j
  // of the code slot in plain order: token q / 36, code bytes 16*(q % 36)
  // .. +15 of its row; loads 0-8 hold tokens 0-15, loads 9-17 tokens 16-31.
  auto load_index = [&](int u) __attribute__((always_inline)) {
    int i = wave + kWaves * u;
    if (i >= (FP8 ? kF8TileLoads : kTileLoads)) i -= kWaves;
    return i;
  };
  uint32_t fl[kLPW], lo[kLPW];
#pragma unroll
  for (int u = 0; u < kLPW; ++u) {
    const uint32_t qc = uint32_t(64 * load_index(u) + lane);
    uint32_t tk, c;
    if constexpr (FP8) {
      tk = qc / uint32_t(kF8Pitch);
      c = qc - tk * kF8Pitch;
    } else {
      tk = qc / uint32_t(kPitch);
      c = (qc - tk * kPitch) ^ swz(tk);
    }
    fl[u] = (tk << 16) | (16u * c);
    lo[u] = (tk & 15u) * kst + 16u * c;
  }
  // Pages of tile k's first and last token (the tile past the range: the last
  // tile's), read ahead of the fill that needs them.
  auto tile_pages = [&](int k, int& pa, int& pb) __attribute__((always_inline)) {
    const int t0 = s + kTile * min(k, nt - 1);
    const int last = min(t0 + kTile - 1, e - 1);
    pa = cbt[t0 >> psh];
    pb = cbt[last >> psh];
  };
  auto fill = [&](int k, uint8_t* slotp, int pa, int pb) __attribute__((always_inline)) {
    const int t0 = s + kTile * k;                   // k < nt
    if (t0 + kTile <= e) {
      // whole tile in the range: half 0 in page pa, half 1 in page pb
      const uint8_t* half0 = p.k + uint64_t(uint32_t(pa)) * ksp + uint32_t(t0 & pmask) * kst;
      const uint8_t* half1 = p.k + uint64_t(uint32_t(pb)) * ksp + uint32_t((t0 + 16) & pmask) * kst;
#pragma unroll
      for (int u = 0; u < kLPW; ++u) {
        const int i = load_index(u);
        dma16_sbase(i < (FP8 ? kF8TileLoads : kTileLoads) / 2 ? half0 : half1, lo[u],
                    uint32_t(size_t((lds_u8*)(slotp + 1024 * i))));
      }
      return;
    }
    const int last = min(t0 + kTile - 1, e - 1);
    const int pi0 = t0 >> psh;
    const uint64_t base0 = uint64_t(uint32_t(pa)) * ksp;
    const uint64_t base1 = uint64_t(uint32_t(pb)) * ksp;
#pragma unroll
    for (int u = 0; u < kLPW; ++u) {
      const int i = load_index(u);
      const int tok = min(t0 + int(fl[u] >> 16), last);
      const uint64_t base = (tok >> psh) == pi0 ? base0 : base1;
      const uint8_t* src = p.k + (base + uint64_t(uint32_t(tok & pmask) * kst + (fl[u] & 0xffffu)));
      dma16(src, uint32_t(size_t((lds_u8*)(slotp + 1024 * i))));
    }
  };

  // O^T accumulators over this wave's value half: lane (n16, qg) holds
  // O[row n16][256hf + 128c + 16e8 + 4qg + i] in o[c*8+e8][i].
  f32x4 o[kPv * 8];
#pragma unroll
  for (int c = 0; c < kPv * 8; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr float kRescaleMargin = 8.f;
  float m_ref = -INFINITY, m_true = -INFINITY, l_run = 0.f;
  int dbg_groups = 0, dbg_xor = 0;
  uint32_t dbg_sum = 0;

  // Byte offsets (inside a 128-feature chunk of the wave's value half) of
  // this lane's transposing reads for the four values of e8 & 3.
  uint32_t vofs[4];
  {
    const uint32_t vt = 4 * qg + (n16 >> 2);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      vofs[m] = vt * (kPitch * 16) + 16 * ((2 * m + ((n16 & 3) >> 1)) ^ swz(vt)) + 8 * (n16 & 1);
  }

  // e4m3: widen tile k's codes (exactly; the scales are applied to the scores
  // and the output) into its bf16 slot, 16-byte chunk c of token t at
  // position c ^ swz(t) as the bf16 fills place it.
  // Thread tid widens chunks tid, tid + 512, ... of the tile's 2304 (waves
  // 0-3 five, waves 4-7 four); the byte offsets are the same every tile.
  constexpr int kWidenMax = (kTile * kPitch + kWaves * 64 - 1) / (kWaves * 64);   // 5
  const int widen_n = (kTile * kPitch - int(tid) + kWaves * 64 - 1) / (kWaves * 64);
  uint32_t wsrc[kWidenMax], wdst[kWidenMax];
#pragma unroll
  for (int j = 0; j < kWidenMax; ++j) {
    const uint32_t u = min(uint32_t(tid) + uint32_t(kWaves * 64 * j), uint32_t(kTile * kPitch - 1));
    const uint32_t t = u / kPitch, c = u - t * kPitch;
    wsrc[j] = t * kMlaDqk + 8 * c;
    wdst[j] = t * (kPitch * 16) + 16 * (c ^ swz(t));
  }
  auto widen_tile = [&](int k) __attribute__((always_inline)) {
    const lds_u8* src = (const lds_u8*)fill_slot(k);
    lds_u8* dst = (lds_u8*)tile_slot(k);
#pragma unroll
    for (int j = 0; j < kWidenMax; ++j) {
      if (j < widen_n) {
        const u32x2 w = *(const __attribute__((address_space(3))) u32x2*)(src + wsrc[j]);
        const u32x2 a = e4m3x4_to_bf16x4(w.x), b2 = e4m3x4_to_bf16x4(w.y);
        const u32x4 r = {a.x, a.y, b2.x, b2.y};
        *(__attribute__((address_space(3))) u32x4*)(dst + wdst[j]) = r;
      }
    }
  };
  int fill_k = 0;          // the tile the current step fills
  int pa = 0, pb = 0;      // its pages (the tile after it's, once read ahead)
  // One 32-token tile in slotp, tokens t0 .. t0+31 of the range.
  auto tile = [&](const uint8_t* slotp, int t0) __attribute__((always_inline)) {
    // ---- partial S^T = K Q^T over this wave's key half for both 16-token
    // groups: all eighteen operand reads first, then the MFMAs, two
    // independent accumulation chains.
    // k-step it: chunk 8*it + 4*hf + qg of token n16 (and 16 + n16, same
    // swizzle), stored at 8*it + ((4*hf + qg) ^ swz(n16))
    const uint8_t* krow = slotp + n16 * (kPitch * 16) + 16 * ((4 * hf + qg) ^ swz(n16));
    bf16x8 k0[kQk], k1[kQk];
#pragma unroll
    for (int it = 0; it < kQk; ++it) {
      k0[it] = *reinterpret_cast<const bf16x8*>(krow + 128 * it);
      k1[it] = *reinterpret_cast<const bf16x8*>(krow + 16 * (kPitch * 16) + 128 * it);
    }
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};   // s[group]
#pragma unroll
    for (int it = 0; it < kQk; ++it) {
      s0 = mfma16x16x32(k0[it], q[it], s0);
      s1 = mfma16x16x32(k1[it], q[it], s1);
    }
    // the first value chunk's operands do not depend on the scores: their
    // reads overlap the exchange and the softmax
    const lds_u8* vbase = (const lds_u8*)slotp + 512 * hf;
    v4i16 vpre[16];
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      const lds_u8* a = vbase + vofs[e8 & 3] + 128 * (e8 >> 2);
      vpre[2 * e8] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)a);
      vpre[2 * e8 + 1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(a + 16 * (kPitch * 16)));
    }
    // ---- swap partials with the pair's other wave; both sum own + other,
    // the same two values, so both hold identical scores
    xch[wave][0][lane] = s0;
    xch[wave][1][lane] = s1;
    lds_barrier();
    // tile k+3's loads into the slot tile k-1 left (every wave finished tile
    // k-1 before the step barrier): issued here rather than at the step start,
    // so the tile's K reads and QK go first and the loads queue under the
    // softmax and PV; past the range's last tile nothing is loaded
    if (fill_k >= 0) fill(fill_k, fill_slot(fill_k), pa, pb);
    const int w2 = wave ^ 1;
    const f32x4 sc[2] = {s0 + xch[w2][0][lane], s1 + xch[w2][1][lane]};
    // ---- online softmax over the tile: lane (n16, qg) holds tokens
    // 4qg..4qg+3 of each group for row n16
    float sv[8];
    if (t0 + kTile <= full_end) {
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[4 * g + i] = sc[g][i] * p.scale_log2;
    } else {
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tk = t0 + 16 * g + 4 * qg + i;
          sv[4 * g + i] = (tk < e && tk <= limit) ? sc[g][i] * p.scale_log2 : -INFINITY;
        }
    }
    float m8 = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) m8 = fmaxf(m8, sv[i]);
    const float mx = column_max4(m8);
    m_true = fmaxf(m_true, mx);
    const bool bump = mx > m_ref + kRescaleMargin;
    if (__any(bump)) {
      const float m_new = bump ? mx : m_ref;
      // a row that does not move keeps alpha = 1 exactly: computing it would
      // give exp2(-inf - -inf) = NaN for a row with nothing visible yet
      const float alpha = bump ? fast_exp2(m_ref - m_new) : 1.f;   // 0 on the first visible tile
      l_run *= alpha;
      m_ref = m_new;
#pragma unroll
      for (int c = 0; c < kPv * 8; ++c) o[c] *= alpha;
    }
    bf16x8 pop;
    {
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pv[i] = fast_exp2(sv[i] - m_use);
      l_run += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
      u32x4 pw = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                  pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
      pop = __builtin_bit_cast(bf16x8, pw);
    }
    // ---- O^T += V^T P^T over this wave's value half, all 32 tokens per MFMA:
    // k index 8qg + j is token (j < 4 ? 0 : 16) + 4qg + (j & 3), for V and P
    // alike.  Block e8 of chunk c is features fb = 256hf + 128c + 16e8 ..
    // +15; lane (x, qg) points at features fb + 4(x&3) .. +3 of token
    // 4qg + (x >> 2) (then 16 + that), i.e. at chunk 2e8 + ((x&3) >> 1) of
    // the chunk's 16, half x & 1.
#pragma unroll
    for (int c = 0; c < kPv; ++c)
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const lds_u8* a = vbase + vofs[e8 & 3] + 128 * (e8 >> 2) + 256 * c;
        const v4i16 lo = c == 0 ? vpre[2 * e8] : __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)a);
        const v4i16 hi = c == 0 ? vpre[2 * e8 + 1]
                                : __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(a + 16 * (kPitch * 16)));
        u32x4 w = {__builtin_bit_cast(u32x2, lo).x, __builtin_bit_cast(u32x2, lo).y,
                   __builtin_bit_cast(u32x2, hi).x, __builtin_bit_cast(u32x2, hi).y};
        o[c * 8 + e8] = mfma16x16x32(__builtin_bit_cast(bf16x8, w), pop, o[c * 8 + e8]);
      }
  };

  // Tile k: wait until this wave's loads of tile k are done (the loads of
  // tiles k+1 and k+2, where the range has them, may still be in flight),
  // then a barrier so every wave's part of the tile has landed -- which also
  // means every wave has finished tile k-1 (its LDS reads and its partial
  // exchange), so its slot can be refilled with tile k+3 (issued inside the
  // tile, after the exchange) and the exchange buffer reused.  Tiles past the
  // range are never loaded: the wait allows as many loads in flight as the
  // range has tiles after k, up to two.
  // e4m3: the same three-ahead fills into the code ring; tile k+1 is widened
  // at the start of step k, so at step k this wave waits for its loads of
  // tile k+1 (those of tile k+2 may still be in flight) and the barrier makes
  // tile k's widened slot and tile k+1's codes visible (widening at the step
  // start measured faster than after the exchange or split around it).
  // The steps of the loop's last three tiles (TAIL) take these counts from
  // the range; the others, all but the last three, have two tiles in flight
  // behind theirs and a tile to fill.
  auto step = [&](int k, auto TAIL) __attribute__((always_inline)) {
    constexpr bool tail = decltype(TAIL)::value;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if constexpr (FP8) {
      if (!tail || k + 2 < nt)
        __builtin_amdgcn_s_waitcnt(0x0F70 | kLPW);         // vmcnt(3)
      else
        __builtin_amdgcn_s_waitcnt(0x0F70);                // vmcnt(0)
    } else {
      if (!tail || k + 2 < nt)
        __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * kLPW));   // vmcnt(10)
      else if (k + 1 < nt)
        __builtin_amdgcn_s_waitcnt(0x0F70 | kLPW);         // vmcnt(5)
      else
        __builtin_amdgcn_s_waitcnt(0x0F70);                // vmcnt(0)
    }
    lds_barrier();
    fill_k = tail ? -1 : k + 3;
    // e4m3: widen tile k+1 (its codes have landed) into the slot tile k-1 left
    if constexpr (FP8) {
      if (!tail || k + 1 < nt) widen_tile(k + 1);
    }
    const uint8_t* cur = tile_slot(k);
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
    // pages for the next step's fill; their wait is the next step's barrier
    tile_pages(k + 4, pa, pb);
  };

  if (nt > 0) {
    tile_pages(0, pa, pb);
    fill(0, fill_slot(0), pa, pb);
    tile_pages(1, pa, pb);
    if (nt > 1) fill(1, fill_slot(1), pa, pb);
    tile_pages(2, pa, pb);
    if (nt > 2) fill(2, fill_slot(2), pa, pb);
    tile_pages(3, pa, pb);
    // Wait here for the query (and with it, loads completing in order, the
    // three fills): the compiler does not see the fills, and a wait for the
    // query placed inside the tile loop would drain the fills in flight there.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);                    // vmcnt(0)
#pragma unroll
    for (int it = 0; it < kQk; ++it) asm volatile("" ::"v"(q[it]));
    if constexpr (FP8) {
      // tile 0 (landed with the wait above) widened before the loop; tile
      // k+1 is widened in step k
      lds_barrier();
      widen_tile(0);
    }
    int k = 0;
    for (; k + 3 < nt; ++k) step(k, std::false_type());
    for (; k < nt; ++k) step(k, std::true_type());
  }
  // no wave leaves while loads it issued may still write LDS
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);                      // vmcnt(0)

  store_rows(p, o, rowv, qg, hf, b, slot, nsplit, m_ref, m_true, l_run, pool);

  if (p.debug && tid == 0) store_debug(p, slot, rb, b, split, s, e, dbg_groups, dbg_xor, dbg_sum);
}

hipError_t launch_mla_short_partial(const PartialParams& p, bool fp8, hipStream_t stream) {
  const int per_xcd = (p.total_wg + 7) / 8;
  const dim3 grid(unsigned(per_xcd * 8)), block(512);
  if (fp8)
    hipLaunchKernelGGL(mla_short_partial_kernel<true>, grid, block, 0, stream, p, per_xcd);
  else
    hipLaunchKernelGGL(mla_short_partial_kernel<false>, grid, block, 0, stream, p, per_xcd);
  return hipGetLastError();
}

}  // namespace splitkv
