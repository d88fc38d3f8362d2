// MLA split-KV partial kernel for gfx950: one 576-wide latent KV head shared
// by every query head; the value is the first 512 columns of the same row
// ("Shipped: 484.5 tok/s on one GB300 ...", table "What shipped": split-KV
// MLA decode of one request at six speculative tokens, causal within them).
//
// Unlike the grouped-query kernel this one is bound by matrix throughput:
// every cached token meets all T*Hq query rows (768 in the six-token,
// 128-head shape), 1,671,168 FLOPs per 1152-byte row.  What limits such a
// kernel is how many FLOPs each byte moved into and out of LDS buys, so a
// workgroup keeps 128 query rows -- each cache tile is brought on chip once
// for twice as many rows as with 64 -- and each of its four waves (one per
// SIMD) owns 32 whole rows: the query's 576 features (144 VGPRs) and the
// output's 512 (256 accumulation registers).  A 32-row wave multiplies on the
// 32x32x16 bf16 matrix instruction, whose operands are twice as wide as the
// 16x16 form's, so one 16-byte read from LDS feeds twice the work, and no
// wave shares a row with another: no partial-score exchange, one workgroup
// barrier per tile.
//   * Tiles of 32 tokens arrive by direct global->LDS loads (16 bytes per
//     lane, no register staging) into a ring of four, three tiles ahead of
//     the one being computed.
//   * A token's 72 16-byte chunks are stored unpadded, chunk c of tile token
//     t at position c ^ swz(t) (a permutation inside each aligned group of
//     eight), which keeps both operand reads free of bank conflicts: the
//     key reads (one chunk of 32 tokens per 32 lanes) and the transposing
//     value reads (4 tokens x 64 bytes per 32 lanes).
//   * Per tile: S^T[token][row] = K Q^T (36 products over 16 features each,
//     the K operand read from LDS a few products ahead), the online softmax
//     in base 2 (lazily moved reference max) over the tile's 32 tokens, then
//     O^T[d][row] += V^T P^T (32 products, 16 tokens each), the V^T operand
//     read straight from the token-major tile with the gfx950 transposing
//     LDS read (ds_read_b64_tr_b16: a 16-lane group that points at 4 tokens
//     x 16 consecutive features receives, in lane x, feature x of the 4
//     tokens).  P needs no data movement: the inner dimension of the second
//     product may list the tokens in any order shared by both operands, and
//     the order chosen is the one the scores come out in.
// An e4m3 latent cache (bf16 queries, "Xqa decode kernels", section
// "Purpose") runs the same tile code: its codes, half the bytes, arrive the
// same way into a four-deep code ring and are widened exactly to bf16 at the
// start of each step into a two-deep ring of bf16 tiles laid out as above.
// Workgroups of one split are placed on one XCD (dispatch is round-robin over
// the eight XCDs), so the row blocks' reads of a tile share that XCD's L2.
// The block-table entries a tile fill needs are read one step ahead, so the
// fill's address computation never waits for them.
#include "mla_common.h"

namespace splitkv {

namespace {

using namespace mla;
constexpr int kWRows = SPLITKV_ROWS_PER_WG_MLA;  // 128 query rows per workgroup
constexpr int kWWaves = 4;                       // one per SIMD, 32 rows each
static_assert(kWRows == 32 * kWWaves, "32 rows per wave");
constexpr int kTile = 32;                        // tokens per LDS tile
constexpr int kPitch = kDqk * 2 / 16;            // 72 16-byte chunks per token row, unpadded
constexpr int kTileLoads = kTile * kPitch / 64;  // 36 wave-level 1 KiB loads
constexpr int kLoadsPerWave = kTileLoads / kWWaves;   // 9
static_assert(kLoadsPerWave * kWWaves == kTileLoads, "every wave issues the same loads per tile");
constexpr int kSlotBytes = kTileLoads * 1024;    // 36864
constexpr int kRing = 4;
// e4m3 cache: a tile's codes (32 x 576 bytes) are 18 wave-level loads; waves
// 0-1 issue five, waves 2-3 four plus a repeat of their fourth, so every wave
// issues five.  The codes land in a four-deep staging ring and are widened
// into a two-deep ring of bf16 tiles laid out as above.
constexpr int kF8Pitch = kDqk / 16;                   // 36 16-byte chunks per code row
constexpr int kF8TileLoads = kTile * kDqk / 1024;     // 18
constexpr int kF8LoadsPerWave = 5;
constexpr int kF8StageBytes = kF8TileLoads * 1024;    // 18432
constexpr int kPoolBytes = kRing * kSlotBytes;        // 147456 either way
static_assert(2 * kSlotBytes + 4 * kF8StageBytes == kPoolBytes, "e4m3 rings fill the pool");
static_assert((kF8LoadsPerWave - 1) * kWWaves < kF8TileLoads && kF8LoadsPerWave * kWWaves >= kF8TileLoads,
              "five loads per wave cover an e4m3 tile");
constexpr int kQk = kDqk / 16;                   // 36 products of 16 key features
constexpr int kQkReg = kDv / 16;                 // 32 of them take the query from registers; the
                                                 // rope features' 4 take it from LDS
constexpr int kVb = kDv / 32;                    // 16 blocks of 32 value features
constexpr int kKAhead = 4;                       // K operand reads in flight ahead of their product
constexpr int kVAhead = 4;                       // products whose V operands are in flight
// Epilogue staging of the compact partial: 128 rows of 512 int16 codes, row
// pitch 1040 bytes.
constexpr int kCodeRowBytes = 1040;
static_assert(kWRows * kCodeRowBytes <= kPoolBytes, "the code staging fits the tile pool");
constexpr int kQRopeBytes = kWWaves * (kQk - kQkReg) * 1024;   // 16384
static_assert(kPoolBytes + kQRopeBytes <= 160 * 1024, "tile pool and rope query fit the LDS");

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Position swizzle of tile token t's chunks (t in 0..31, 3 bits): the eight
// tokens of one residue mod 4 (whose rows start on the same bank, the row
// pitch being 1152 bytes) take eight different values, so the 32 lanes of a
// key read hit 32 different 16-byte bank groups; and tokens t and t + 2 of
// an aligned group of four differ in bit 2, so the four 64-byte pieces of a
// transposing read land in the four different quarters of the 256 bytes of
// banks it is served from.
__device__ __forceinline__ uint32_t swz(uint32_t t) { return ((t >> 2) ^ ((t & 2u) << 1)) & 7u; }

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

// s_waitcnt immediate for vmcnt(n) alone (n < 64).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

}  // namespace

template <bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_partial_kernel(PartialParams p, int per_xcd) {
  // bf16: four tile slots.  e4m3: two bf16 tile slots, then four code slots.
  __shared__ __attribute__((aligned(1024))) uint8_t pool[kPoolBytes];
  // the query's 64 rope features, in the operand layout: wave w, product
  // it - 32, lane j at qrope + 1024 (4 w + it - 32) + 16 j
  __shared__ __attribute__((aligned(1024))) uint8_t qrope[kQRopeBytes];
  constexpr int kLPW = FP8 ? kF8LoadsPerWave : kLoadsPerWave;   // loads per wave and tile
  auto tile_slot = [&](int k) __attribute__((always_inline)) {
    return pool + (FP8 ? (k & 1) : (k & 3)) * kSlotBytes;
  };
  auto fill_slot = [&](int k) __attribute__((always_inline)) {
    return FP8 ? pool + 2 * kSlotBytes + (k & 3) * kF8StageBytes : pool + (k & 3) * kSlotBytes;
  };

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
  const int r32 = lane & 31, h = lane >> 5;

  const SlotWork work = load_slot(p.slot_info, slot);
  const int b = work.b, split = work.split, nsplit = work.nsplit, s = work.s, e = work.e;
  const int L = ((cint32*)p.seq_lens)[b];

  // This lane's query row (column of the S^T tiles); rows past the last one
  // read row rows-1 and are never stored.  Lane (r32, h) holds features
  // 16 it + 8 h .. +7 of the row for the product it: in registers for the
  // 512 latent features, in LDS for the 64 rope features (the registers are
  // what bounds this layout).
  const int rowv = rb * kWRows + wave * 32 + r32;
  int limit;
  bf16x8 q[kQkReg];
  const lds_u8* qr = (const lds_u8*)qrope + wave * ((kQk - kQkReg) * 1024) + 16 * lane;
  {
    const int rc = min(rowv, p.rows - 1);
    const int t = rc / p.Hq, hq = rc % p.Hq;
    limit = L - p.T + t;      // last key position this row sees
    const uint16_t* qrow = p.q + b * p.qsb + t * p.qst + hq * p.qsh + 8 * h;
#pragma unroll
    for (int it = 0; it < kQkReg; ++it) q[it] = *reinterpret_cast<const bf16x8*>(qrow + 16 * it);
    // the rope part goes straight to LDS, so nothing waits for it here
#pragma unroll
    for (int it = kQkReg; it < kQk; ++it)
      dma16(reinterpret_cast<const uint8_t*>(qrow + 16 * it),
            uint32_t(size_t(qrope + wave * ((kQk - kQkReg) * 1024) + 1024 * (it - kQkReg))));
  }

  // Tiles that end at or before full_end need no mask: every token is in the
  // range and visible to every row of the wave (its first row has the
  // smallest causal limit).
  const int full_end = min(e, L - p.T + min(rb * kWRows + wave * 32, p.rows - 1) / p.Hq + 1);

  // The page size is a power of two for this kernel (checked on the host).
  const int psh = p.page_shift;
  const int pmask = p.page_size - 1;
  cint32* cbt = (cint32*)(p.bt + b * p.bt_stride);
  const uint32_t ksp = uint32_t(p.ksp), kst = uint32_t(p.kst);   // < 2^31, checked on the host

  // Tile fill: wave w issues the wave-level loads w, w+4, ..., w+32 of the 36
  // a tile needs.  Lane j of load i fills the 16-byte position q = 64*i + j of
  // the slot: token q / 72, holding chunk (q % 72) ^ swz(token) of that
  // token's row.  Tokens past the range end load the range's last token
  // (finite, masked later).  Loads 0-17 hold tokens 0-15 and loads 18-35
  // tokens 16-31 (16 x 72 = 18 x 64 chunks), and a 16-token half of a tile
  // lies in one page (tiles start on multiples of 16, pages hold a power of
  // two >= 16 tokens), so for a tile inside the range a load reads one page:
  // its address is a uniform page base plus the lane's offset inside the
  // half, lo[u].
  // For an e4m3 cache, lane j of load i fills 16-byte position q = 64*i + j
  // of the code slot in plain order: token q / 36, code bytes 16*(q % 36)
  // .. +15 of its row; loads 0-8 hold tokens 0-15, loads 9-17 tokens 16-31;
  // a wave with only four loads repeats its fourth (same lanes, same
  // addresses, same bytes), so every wave's completion counts are the same.
  const int nt = (e - s + kTile - 1) / kTile;      // tiles of the range
  auto load_index = [&](int u) __attribute__((always_inline)) {
    int i = wave + kWWaves * u;
    if (FP8 && i >= kF8TileLoads) i -= kWWaves;
    return i;
  };
  // (token, byte offset in its row) of the chunk lane fills in load u
  auto chunk_of = [&](int u, uint32_t& tk, uint32_t& c16) __attribute__((always_inline)) {
    const uint32_t qc = uint32_t(64 * load_index(u) + lane);
    if constexpr (FP8) {
      tk = qc / uint32_t(kF8Pitch);
      c16 = 16u * (qc - tk * kF8Pitch);
    } else {
      tk = qc / uint32_t(kPitch);
      c16 = 16u * ((qc - tk * kPitch) ^ swz(tk));
    }
  };
  uint32_t lo[kLPW];
#pragma unroll
  for (int u = 0; u < kLPW; ++u) {
    uint32_t tk, c16;
    chunk_of(u, tk, c16);
    lo[u] = (tk & 15u) * kst + c16;
  }
  // Pages of tile k's first and last token (past the range: the last tile's),
  // read ahead of the fill that needs them.
  auto tile_pages = [&](int k, int& pa, int& pb) __attribute__((always_inline)) {
    const int t0 = s + kTile * min(k, nt - 1);
    const int last = min(t0 + kTile - 1, e - 1);
    pa = cbt[t0 >> psh];
    pb = cbt[last >> psh];
  };
  // The paged-addressing digest of the range (pages of its 16-token groups),
  // taken as each tile is filled: a 16-token group lies in one page, so the
  // group [t0 + 16, t0 + 32) is in the page of the tile's last token.
  int dbg_groups = 0, dbg_xor = 0;
  uint32_t dbg_sum = 0;
  auto digest = [&](int k, int pa, int pb) __attribute__((always_inline)) {
    const bool has1 = s + kTile * k + 16 < e;
    dbg_groups += has1 ? 2 : 1;
    dbg_xor ^= pa ^ (has1 ? pb : 0);
    dbg_sum += uint32_t(pa) + (has1 ? uint32_t(pb) : 0u);
  };
  constexpr int kHalf = (FP8 ? kF8TileLoads : kTileLoads) / 2;
  // A tile inside the range: half 0 in page pa, half 1 in page pb; load u of
  // this wave is a uniform page base plus lo[u].  Split into single loads so
  // that the steps can spread them over their products.
  struct WholeFill {
    const uint8_t* half0;
    const uint8_t* half1;
    uint8_t* slotp;
  };
  auto whole_fill = [&](int k, uint8_t* slotp, int pa, int pb) __attribute__((always_inline)) {
    const int t0 = s + kTile * k;                   // t0 + kTile <= e
    digest(k, pa, pb);
    return WholeFill{p.k + uint64_t(uint32_t(pa)) * ksp + uint32_t(t0 & pmask) * kst,
                     p.k + uint64_t(uint32_t(pb)) * ksp + uint32_t((t0 + 16) & pmask) * kst, slotp};
  };
  auto whole_load = [&](const WholeFill& f, int u) __attribute__((always_inline)) {
    const int i = load_index(u);
    dma16_sbase(i < kHalf ? f.half0 : f.half1, lo[u], uint32_t(size_t((lds_u8*)(f.slotp + 1024 * i))));
  };
  // Any tile of the range (the last may be cut by the range end): tokens past
  // the end load the range's last token.
  auto fill = [&](int k, uint8_t* slotp, int pa, int pb) __attribute__((always_inline)) {
    const int t0 = s + kTile * k;                   // k < nt
    if (t0 + kTile <= e) {
      const WholeFill f = whole_fill(k, slotp, pa, pb);
#pragma unroll
      for (int u = 0; u < kLPW; ++u) whole_load(f, u);
      return;
    }
    digest(k, pa, pb);
    // half 0 lies in page pa; half 1, when the range reaches it, in page pb,
    // else its tokens all load the range's last token, which is in page pa
    const int last = min(t0 + kTile - 1, e - 1);
    const uint8_t* b0 = p.k + uint64_t(uint32_t(pa)) * ksp;
    const uint8_t* b1 = t0 + 16 < e ? p.k + uint64_t(uint32_t(pb)) * ksp : b0;
#pragma unroll
    for (int u = 0; u < kLPW; ++u) {
      const int i = load_index(u);
      uint32_t tk, c16;
      chunk_of(u, tk, c16);
      const uint32_t off = uint32_t(min(t0 + int(tk), last) & pmask) * kst + c16;
      dma16_sbase(i < kHalf ? b0 : b1, off, uint32_t(size_t((lds_u8*)(slotp + 1024 * i))));
    }
  };

  // O^T accumulators: lane (r32, h) holds O[row r32][32 blk + 8 (v / 4) +
  // 4 h + v % 4] in o[blk][v].
  f32x16 o[kVb];
#pragma unroll
  for (int c = 0; c < kVb; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[c][v] = 0.f;
  constexpr float kRescaleMargin = 8.f;
  float m_ref = -INFINITY, m_true = -INFINITY, l_run = 0.f;

  // Byte offsets of this lane's K operand reads: product it reads chunk
  // 2 it + h of token r32, at kofs[it & 3] + 128 (it >> 2).
  uint32_t kofs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) kofs[j] = uint32_t(r32) * (kPitch * 16) + 16u * ((2u * j + h) ^ swz(r32));
  // Byte offsets of this lane's transposing V reads.  The score result leaves
  // lane (r32, h) the tokens 8 (v / 4) + 4 h + v % 4 of row r32 in item v, so
  // the second product's inner index 8 h + u of 16-token step kb is token
  // 16 kb + 8 (u / 4) + 4 h + u % 4.  Its V^T operand: lane (x, g1, h)
  // (x = lane & 15, g1 = bit 4) holds feature 32 blk + 16 g1 + x of those
  // tokens; read r (u / 4) of step kb points the lane at token tv = 16 kb +
  // 8 r + 4 h + x / 4, features 32 blk + 16 g1 + 4 (x & 3) .. +3: chunk
  // c = 4 blk + 2 g1 + (x & 3) / 2, half x & 1, at position c ^ swz(tv).
  // With swz(tv) = (4 kb + 2 r + h) ^ 4 (x >> 3), the position's offset
  // inside the 128 bytes of blk >> 1 is 64 ((blk & 1) ^ kb ^ (x >> 3)) +
  // 16 ((2 g1 + (x & 3) / 2) ^ (2 r + h)): four per-lane offsets
  // vofs[(blk & 1) ^ kb][r], the rest (16 kb + 8 r tokens, 128 (blk >> 1)
  // bytes) a constant.
  uint32_t vofs[2][2];
  {
    const uint32_t x = lane & 15, g1 = (lane >> 4) & 1;
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int r = 0; r < 2; ++r)
        vofs[bk][r] = (4u * h + (x >> 2)) * (kPitch * 16) + 64u * (bk ^ (x >> 3)) +
                      16u * ((2u * g1 + ((x & 3u) >> 1)) ^ (2u * r + h)) + 8u * (x & 1u);
  }

  // e4m3: widen tile k's codes (exactly; the scales are applied to the scores
  // and the output) into its bf16 slot, 16-byte chunk c of token t at
  // position c ^ swz(t) as the bf16 fills place it.  Thread tid widens token
  // tid / 8, chunks tid % 8 + 8 j (j = 0..8): 8 code bytes at wsrc + 64 j,
  // 16 bf16 bytes at wdst + 128 j (the swizzle stays inside the aligned
  // group of eight).
  constexpr int kWiden = kPitch / 8;               // 9
  static_assert(kWWaves * 64 == 8 * kTile, "eight threads per tile token");
  uint32_t wsrc = 0, wdst = 0;
  if constexpr (FP8) {
    const uint32_t t = uint32_t(tid) >> 3, c = uint32_t(tid) & 7u;
    wsrc = t * kDqk + 8u * c;
    wdst = t * (kPitch * 16) + 16u * (c ^ swz(t));
  }
  // All nine reads go out before the first conversion (one wave per SIMD:
  // nothing else would hide their latency), and a scheduling barrier keeps
  // them and the writes out of the score products' read pattern.
  auto widen_tile = [&](int k) __attribute__((always_inline)) {
    const lds_u8* src = (const lds_u8*)fill_slot(k) + wsrc;
    lds_u8* dst = (lds_u8*)tile_slot(k) + wdst;
    u32x2 w[FP8 ? kWiden : 1];
#pragma unroll
    for (int j = 0; j < (FP8 ? kWiden : 0); ++j) w[j] = *(const __attribute__((address_space(3))) u32x2*)(src + 64 * j);
#pragma unroll
    for (int j = 0; j < (FP8 ? kWiden : 0); ++j) {
      const u32x2 a = e4m3x4_to_bf16x4(w[j].x), b2 = e4m3x4_to_bf16x4(w[j].y);
      const u32x4 r = {a.x, a.y, b2.x, b2.y};
      *(__attribute__((address_space(3))) u32x4*)(dst + 128 * j) = r;
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // One 32-token tile in slotp, tokens t0 .. t0+31 of the range; load u of
  // the next tile's fill (fill_u, which may do nothing) goes out after
  // product 4 u + 2 of the scores.
  auto tile = [&](const uint8_t* slotp, int t0, auto&& fill_u) __attribute__((always_inline)) {
    const lds_u8* ls = (const lds_u8*)slotp;
    // ---- S^T = K Q^T: 36 products into one accumulator, each K operand
    // read kKAhead products ahead
    f32x16 sacc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
    bf16x8 kr[kQk], qrr[kQk];
    auto kread = [&](int it) __attribute__((always_inline)) {
      kr[it] = *(const lds_bf16x8*)(ls + kofs[it & 3] + 128 * (it >> 2));
      if (it >= kQkReg) qrr[it] = *(const lds_bf16x8*)(qr + 1024 * (it - kQkReg));
    };
#pragma unroll
    for (int it = 0; it < kKAhead; ++it) kread(it);
#pragma unroll
    for (int it = 0; it < kQk; ++it) {
      if (it + kKAhead < kQk) kread(it + kKAhead);
      if (it % 4 == 2 && it / 4 < kLPW) fill_u(it / 4);
      sacc = mfma32(kr[it], it < kQkReg ? q[it] : qrr[it], sacc);
    }
    // Hold the scheduler to that order (left alone it issues each read just
    // before its product, which then waits out the LDS latency): the first
    // kKAhead reads, then read (two for a rope product), product, ...
    __builtin_amdgcn_sched_group_barrier(0x100, kKAhead, 0);
#pragma unroll
    for (int it = 0; it < kQkReg - kKAhead; ++it) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int it = kQkReg - kKAhead; it < kQk - kKAhead; ++it) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#pragma unroll
    for (int it = kQk - kKAhead; it < kQk; ++it) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    // the first value products' operands do not depend on the scores: their
    // reads overlap the softmax
    auto vread = [&](int n, v4i16& a0, v4i16& a1) __attribute__((always_inline)) {
      const int kb = n / kVb, blk = n % kVb;
      const lds_u8* base = ls + 16 * kb * (kPitch * 16) + 128 * (blk >> 1);
      a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + vofs[(blk & 1) ^ kb][0]));
      a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16*)(base + 8 * (kPitch * 16) + vofs[(blk & 1) ^ kb][1]));
    };
    v4i16 va[2 * kVb], vb[2 * kVb];
#pragma unroll
    for (int n = 0; n < kVAhead; ++n) vread(n, va[n], vb[n]);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVAhead, 0);
    // ---- online softmax over the tile: lane (r32, h) holds tokens
    // 8 (v / 4) + 4 h + v % 4 of row r32
    float sv[16];
    if (t0 + kTile <= full_end) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sv[v] = sacc[v] * p.scale_log2;
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int tk = t0 + 8 * (v >> 2) + 4 * h + (v & 3);
        sv[v] = (tk < e && tk <= limit) ? sacc[v] * p.scale_log2 : -INFINITY;
      }
    }
    float m16 = sv[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) m16 = fmaxf(m16, sv[v]);
    const float mx = pair_max(m16);
    m_true = fmaxf(m_true, mx);
    const bool bump = mx > m_ref + kRescaleMargin;
    if (__any(bump)) {
      const float m_new = bump ? mx : m_ref;
      // a row that does not move keeps alpha = 1 exactly: computing it would
      // give exp2(-inf - -inf) = NaN for a row with nothing visible yet
      const float alpha = bump ? fast_exp2(m_ref - m_new) : 1.f;   // 0 on the first visible tile
      // a row whose reference max was -inf has o = 0 (every weight so far
      // was 0), so only rows that had one need their o rescaled
      const bool moved = bump && m_ref != -INFINITY;
      l_run *= alpha;
      m_ref = m_new;
      if (__any(moved)) {
#pragma unroll
        for (int c = 0; c < kVb; ++c) scale_acc(o[c], alpha);
      }
    }
    bf16x8 pk[2];
    {
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      float pv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) pv[v] = fast_exp2(sv[v] - m_use);
      float ls4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) ls4[j] = (pv[4 * j] + pv[4 * j + 1]) + (pv[4 * j + 2] + pv[4 * j + 3]);
      l_run += (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 pw = {pack_bf16x2(pv[8 * kb + 0], pv[8 * kb + 1]), pack_bf16x2(pv[8 * kb + 2], pv[8 * kb + 3]),
                          pack_bf16x2(pv[8 * kb + 4], pv[8 * kb + 5]), pack_bf16x2(pv[8 * kb + 6], pv[8 * kb + 7])};
        pk[kb] = __builtin_bit_cast(bf16x8, pw);
      }
    }
    // ---- O^T += V^T P^T: product n = kb * 16 + blk accumulates value block
    // blk over the 16 tokens of step kb; the V operands run kVAhead products
    // ahead
#pragma unroll
    for (int n = 0; n < 2 * kVb; ++n) {
      if (n + kVAhead < 2 * kVb) vread(n + kVAhead, va[n + kVAhead], vb[n + kVAhead]);
      const u32x4 w = {__builtin_bit_cast(u32x2, va[n]).x, __builtin_bit_cast(u32x2, va[n]).y,
                       __builtin_bit_cast(u32x2, vb[n]).x, __builtin_bit_cast(u32x2, vb[n]).y};
      o[n % kVb] = mfma32(__builtin_bit_cast(bf16x8, w), pk[n / kVb], o[n % kVb]);
    }
    // as for the scores: read two ahead, product, ...
#pragma unroll
    for (int n = 0; n < 2 * kVb - kVAhead; ++n) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
#pragma unroll
    for (int n = 2 * kVb - kVAhead; n < 2 * kVb; ++n) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  };

  int pa = 0, pb = 0;      // pages of the tile the next fill loads
  // Step k: wait until this wave's loads of tile k are done (those of tiles
  // k+1 and k+2, where the range has them, may still be in flight), then a
  // barrier so every wave's part of the tile has landed -- which also means
  // every wave has finished tile k-1, so its slot can be refilled with tile
  // k+3.  Tiles past the range are never loaded: the wait allows as many
  // loads in flight as the range has tiles after k, up to two.
  // e4m3: the same three-ahead fills into the code ring; tile k+1 is widened
  // at the start of step k, so at step k this wave waits for its loads of
  // tile k+1 (those of tile k+2 may still be in flight) and the barrier makes
  // tile k's widened slot and tile k+1's codes visible.
  // The steps of the loop's last three tiles (TAIL) take these counts from
  // the range; the others have two tiles in flight behind theirs and a tile
  // to fill.
  // Steps whose fill is a tile before the range's last (all but the last
  // four) spread its loads over the score products; the last four (TAIL)
  // fill the range's last tile, which may be cut by the range end, up front,
  // or nothing.
  auto step = [&](int k, auto TAIL) __attribute__((always_inline)) {
    constexpr bool tail = decltype(TAIL)::value;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if constexpr (FP8) {
      if (!tail || k + 2 < nt)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLPW));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    } else {
      if (!tail || k + 2 < nt)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLPW));
      else if (k + 1 < nt)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLPW));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    lds_barrier();
    if (tail && k + 3 < nt) fill(k + 3, fill_slot(k + 3), pa, pb);
    // e4m3: widen tile k+1 (its codes have landed) into the slot tile k-1 left
    if constexpr (FP8) {
      if (!tail || k + 1 < nt) widen_tile(k + 1);
    }
    const uint8_t* cur = tile_slot(k);
    const int t0 = s + kTile * k;
    if constexpr (!tail) {
      const WholeFill f = whole_fill(k + 3, fill_slot(k + 3), pa, pb);
      tile(cur, t0, [&](int u) __attribute__((always_inline)) { whole_load(f, u); });
    } else {
      tile(cur, t0, [](int) {});
    }
    // pages for the next step's fill; their wait is the next step's barrier.
    // The scheduling barrier keeps these scalar loads behind every value read
    // of the tile: while one is in flight the compiler can only wait for LDS
    // reads with lgkmcnt(0), which would drain the reads in flight.
    __builtin_amdgcn_sched_barrier(0);
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
    // Wait here for the query and tile 0 (loads complete in order; tiles 1
    // and 2 may still be in flight): the compiler does not see the fills, and
    // a wait for the query placed inside the tile loop would drain the fills
    // in flight there.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (nt > 2)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLPW));
    else if (nt > 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLPW));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
#pragma unroll
    for (int it = 0; it < kQkReg; ++it) asm volatile("" ::"v"(q[it]));
    if constexpr (FP8) {
      // tile 0 (landed with the wait above) widened before the loop; tile
      // k+1 is widened in step k
      lds_barrier();
      widen_tile(0);
    }
    // tiles k + 3 < nt - 1 are inside the range; tile nt - 1 may be cut
    int k = 0;
    for (; k + 4 < nt; ++k) step(k, std::false_type());
    for (; k < nt; ++k) step(k, std::true_type());
  }
  // no wave leaves while loads it issued may still write LDS
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // ---- epilogue: bring (l, o) from the reference max to the true max
  const bool direct = p.direct && nsplit == 1;
  const int64_t R = int64_t(p.T) * p.Hq;
  const float f = (m_ref == -INFINITY) ? 0.f : fast_exp2(m_ref - m_true);
  const float l_tot = pair_sum(l_run * f);
  const bool real = rowv < p.rows;
  float mul = p.v_scale * f;
  if (direct) mul = l_tot > 0.f ? p.v_scale * f / l_tot : 0.f;
  if (direct) {
    // a single-split sequence's rows go straight to out (normalised) and lse
    if (real) {
      const int64_t ob = (int64_t(b) * R + rowv) * kDv + 4 * h;
#pragma unroll
      for (int c = 0; c < kVb; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t oo = ob + 32 * c + 8 * j;
          const f32x4 v4 = {o[c][4 * j] * mul, o[c][4 * j + 1] * mul, o[c][4 * j + 2] * mul, o[c][4 * j + 3] * mul};
          if (p.out_f32) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + oo) = v4;
          } else {
            const u32x2 pk2 = {pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3])};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + oo) = pk2;
          }
        }
      if (h == 0 && p.lse)
        p.lse[int64_t(b) * R + rowv] = (m_true == -INFINITY || !(l_tot > 0.f)) ? -INFINITY
                                                                               : (m_true + log2f(l_tot)) * kLn2;
    }
  } else {
    // Compact partial: each 256-feature half of a row as int16 codes of
    // o / s, s = (largest |o| of the half) / 32767, written beside them.
    // The codes go out through LDS (the tile pool, free once every wave has
    // left the tile loop): written in the product layout, read back a row at
    // a time, so each store writes one row's 1 KiB.
    // Largest |o| of each half from the bit patterns: the signed maximum of
    // the patterns is the largest positive value, the unsigned maximum the
    // negative value of largest magnitude (or, with none, the largest
    // positive), so the larger of their magnitudes is the answer -- two
    // three-operand integer maxima per pair of values.
    float amax[2], kq[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      int32_t smax = INT32_MIN;
      uint32_t umax = 0;
#pragma unroll
      for (int c = 8 * hf; c < 8 * hf + 8; ++c)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const int32_t x = __float_as_int(o[c][v]), y = __float_as_int(o[c][v + 1]);
          smax = max(smax, max(x, y));
          umax = max(umax, max(uint32_t(x), uint32_t(y)));
        }
      const float a = pair_max(fmaxf(fabsf(__int_as_float(smax)), fabsf(__uint_as_float(umax))));
      amax[hf] = a * fabsf(mul);
      // o * kq lies in [-1, 1]; its code is the nearest integer to 32767 times it
      kq[hf] = amax[hf] > 0.f ? mul / amax[hf] : 0.f;
    }
    lds_u8* st = (lds_u8*)pool + (wave * 32) * kCodeRowBytes;
    __syncthreads();                       // every wave is done with the tile pool
#pragma unroll
    for (int c = 0; c < kVb; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // v_cvt_pknorm_i16_f32: two values in [-1, 1] to the nearest multiples
        // of 1/32767, as int16 codes
        const float kk = kq[c / 8];
        const u32x2 w = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(o[c][4 * j] * kk, o[c][4 * j + 1] * kk)),
                         __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(o[c][4 * j + 2] * kk, o[c][4 * j + 3] * kk))};
        *(__attribute__((address_space(3))) u32x2*)(st + r32 * kCodeRowBytes + 2 * (32 * c + 8 * j + 4 * h)) = w;
      }
    // each wave reads back only what it wrote (no barrier; the LDS waits
    // suffice); rows are in (t, h) order, so a row's index within the
    // sequence is the row number itself
    const int row0 = rb * kWRows + wave * 32;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const u32x4 w = *(const __attribute__((address_space(3))) u32x4*)(st + r * kCodeRowBytes + 16 * lane);
      if (row0 + r < p.rows) *reinterpret_cast<u32x4*>(p.part_q + (int64_t(slot) * R + row0 + r) * kDv + 8 * lane) = w;
    }
    if (real && h == 0) {
      const int64_t ix = int64_t(slot) * R + rowv;
      p.part_s[2 * ix] = amax[0] * (1.f / 32767.f);
      p.part_s[2 * ix + 1] = amax[1] * (1.f / 32767.f);
      p.part_m[ix] = m_true == -INFINITY ? -INFINITY : m_true * kLn2;
      p.part_l[ix] = l_tot;
    }
  }

  if (p.debug && tid == 0) store_debug(p, slot, rb, b, split, s, e, dbg_groups, dbg_xor, dbg_sum);
}

hipError_t launch_mla_partial(const PartialParams& p, bool fp8, hipStream_t stream) {
  const int per_xcd = (p.total_wg + 7) / 8;
  const dim3 grid(unsigned(per_xcd * 8)), block(256);
  if (fp8)
    hipLaunchKernelGGL(mla_partial_kernel<true>, grid, block, 0, stream, p, per_xcd);
  else
    hipLaunchKernelGGL(mla_partial_kernel<false>, grid, block, 0, stream, p, per_xcd);
  return hipGetLastError();
}

}  // namespace splitkv
