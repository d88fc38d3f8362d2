// MLA split-KV partial kernel for gfx950: one 576-wide latent KV head shared
// by every query head; the value is the first 512 columns of the same row
// ("Shipped: 484.5 tok/s on one GB300 ...", table "What shipped": split-KV
// MLA decode of one request at six speculative tokens, causal within them).
// One kernel body, three cache/query kinds (KIND):
//   0: bf16 latent cache, bf16 queries;
//   1: e4m3 latent cache (one per-tensor scale, "Xqa decode kernels", section
//      "Purpose"), bf16 queries;
//   2: e4m3 latent cache and e4m3 queries, quantised here to codes of
//      q / q_scale, so the scores run on the FP8 matrix instruction (the
//      pages' FP8-Q path, "Xqa decode kernels", timeline: the FP8-Q selection).
//
// Every cached token meets all T*Hq query rows (768 in the six-token,
// 128-head shape), 1,671,168 FLOPs per latent row.  What bounds such a kernel
// on gfx950 is the bytes it reads out of LDS per FLOP (an LDS read returns
// ~100 bytes a clock per CU for 16-byte reads, ~80 for transposing ones,
// against 4096 FLOPs a clock of bf16 matrix work), so a workgroup keeps 128
// query rows -- each cache tile is brought on chip once for all of them --
// and each of its four waves (one per SIMD) owns 32 whole rows: the query in
// registers (the bf16 query's 64 rope features in LDS) and O's 32 rows x 512
// features in all 256 accumulation registers.  The products are the 32x32
// forms (v_mfma_f32_32x32x16_bf16, and v_mfma_f32_32x32x64_f8f6f4 for the
// e4m3-query scores), whose operands feed twice the work of the 16x16 forms
// per byte read.  No wave shares a row: no partial-score exchange, one
// workgroup barrier per tile.
//   * Tiles of 32 tokens arrive by direct global->LDS loads (16 bytes per
//     lane, no register staging) into a ring, several tiles ahead of the one
//     being computed.  An e4m3 tile holds the codes themselves, half the
//     bytes of bf16: the operands are read as codes and widened exactly to
//     bf16 in registers (v_cvt_scalef32_pk_bf16_fp8), which halves the LDS
//     reads; with e4m3 queries the score operands are the codes.
//   * Token rows are stored unpadded, 16-byte chunk c of tile token t at a
//     swizzled position inside an aligned group of chunks, which keeps every
//     operand read free of bank conflicts.
//   * Per tile: S^T[token][row] = K Q^T (the K operand read from LDS a few
//     products ahead), the online softmax in base 2 (lazily moved reference
//     max) over the tile's 32 tokens, then O^T[d][row] += V^T P^T (32
//     products of 16 tokens), the V^T operand read straight from the
//     token-major tile with the gfx950 transposing LDS reads
//     (ds_read_b64_tr_b16 for bf16: a 16-lane group that points at 4 tokens
//     x 16 features receives, in lane x, feature x of the 4 tokens;
//     ds_read_b64_tr_b8 for codes: lane x receives byte x & 7 of the 8-byte
//     vectors read by lanes 2j + (x >> 3), j = 0..7, i.e. one feature of 8
//     tokens).  P needs no data movement: the inner dimension of the value
//     product lists the tile's tokens in the order the scores come out in.
//     P enters it as bf16 in every kind: with e4m3 queries the FP8
//     instruction serves the scores, and the value product runs on bf16
//     operands like the others' (V widened from its codes).
//   * The bf16 query is staged through LDS in a bf16 tile's layout by loads
//     of 1 KiB of consecutive rows (loaded straight into the operand layout,
//     every load would touch 32 rows); e4m3 queries are quantised in
//     registers with an exact division-free quotient.
// Workgroups of one split are placed on one XCD (dispatch is round-robin over
// the eight XCDs), so the row blocks' reads of a tile share that XCD's L2.
// The block-table entries a tile fill needs are read one step ahead, so the
// fill's address computation never waits for them.
#include "mla_common.h"

namespace splitkv {

namespace {

using namespace mla;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// Tile geometry of each kind.
template <int KIND>
struct Geo {
  static constexpr bool kCodes = KIND != 0;                            // the tile holds e4m3 codes
  static constexpr int kChunks = kCodes ? kDqk / 16 : kDqk * 2 / 16;   // 36 or 72 16-byte chunks a row
  static constexpr int kRowBytes = 16 * kChunks;                       // 576 or 1152
  static constexpr int kLoads = kTile * kChunks / 64;                  // 18 or 36 wave-level 1 KiB loads
  static constexpr int kLPW = (kLoads + kWWaves - 1) / kWWaves;        // 5 or 9 loads per wave and tile
  static constexpr int kSlotBytes = kLoads * 1024;                     // 18432 or 36864
  static constexpr int kRing = kCodes ? 8 : 4;                         // tile slots
  static constexpr int kAhead = kCodes ? 6 : 3;                        // tiles filled ahead of the one computed
  static constexpr int kPoolBytes = kRing * kSlotBytes;                // 147456 either way
  static_assert(kAhead < kRing && kAhead * kLPW < 64, "fills in flight fit the ring and the counter");
  static_assert(kStageBytes <= kPoolBytes, "the epilogue's staging fits the tile pool");
};

// bf16 tiles: chunk c of token t at position c ^ swz_bf16(t) (3 bits, inside
// each aligned group of eight).  The eight tokens of one residue mod 4 (whose
// rows start on the same bank at the 1152-byte pitch) take eight different
// values, so the 32 lanes of a key read (one chunk of 32 tokens) hit 32
// different 16-byte bank groups; tokens t and t + 2 of an aligned group of
// four differ in bit 2, so the four 64-byte pieces of a transposing read
// land in the four different quarters of the 256 bytes of banks it is served
// from.
__device__ __forceinline__ uint32_t swz_bf16(uint32_t t) { return ((t >> 2) ^ ((t & 2u) << 1)) & 7u; }
// e4m3 tiles: chunk c of token t at position 4 (c >> 2) + ((c & 3) ^
// swz_e4m3(t)) (2 bits, inside each aligned group of four).  At the 576-byte
// pitch tokens t and t + 8 start on the same bank: tokens t, t + 8, t + 16,
// t + 24 take four different values, so a key read's 32 lanes (one chunk of
// 32 tokens) hit 32 bank groups; and tokens t and t + 8 differ in bit 1, so
// the eight 32-byte pieces of a transposing byte read (8 tokens x 32
// features) fill its 256 bytes of banks.
__device__ __forceinline__ uint32_t swz_e4m3(uint32_t t) { return (((t >> 3) & 1u) << 1) | ((t >> 4) & 1u); }

// D += A B over 64 e4m3 inner elements (both operands e4m3: format codes 0;
// with both scale operands zero the compiler emits the unscaled instruction).
__device__ __forceinline__ f32x16 mma64(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Eight e4m3 codes (two dwords) to eight bf16 values, exactly.
__device__ __forceinline__ bf16x8 widen8(uint32_t lo, uint32_t hi) {
  const u32x2 a = e4m3x4_to_bf16x4(lo), b = e4m3x4_to_bf16x4(hi);
  return __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
}

// s_waitcnt vmcnt(kLPW * n) for a uniform n in 0..6.
template <int kLPW>
__device__ __forceinline__ void wait_tiles(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLPW)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLPW)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * kLPW < 64 ? 3 * kLPW : 63)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * kLPW < 64 ? 4 * kLPW : 63)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5 * kLPW < 64 ? 5 * kLPW : 63)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(6 * kLPW < 64 ? 6 * kLPW : 63)); break;
  }
}

constexpr int kVAhead = 4;                       // value products whose operands are in flight
constexpr int kQRopeBytes = 16384;               // bf16 queries: 64 rope features x 32 rows x 4 waves

}  // namespace

template <int KIND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_partial_kernel(PartialParams p, int per_xcd) {
  using G = Geo<KIND>;
  constexpr bool kCodes = G::kCodes;
  constexpr bool kQ8 = KIND == 2;
  constexpr int kLPW = G::kLPW;
  constexpr int kAhead = G::kAhead;
  constexpr int kRowBytes = G::kRowBytes;
  // the tile ring; the epilogue's staging once the tile loop is done
  __shared__ __attribute__((aligned(1024))) uint8_t pool[G::kPoolBytes];
  // bf16 queries: the query's 64 rope features, in the score operand layout
  // (kept out of the registers, which bound this layout): wave w, operand
  // block i (0..3), lane j at qrope + 4096 w + 1024 i + 16 j
  __shared__ __attribute__((aligned(1024))) uint8_t qrope[kQ8 ? 16 : kQRopeBytes];
  static_assert(G::kPoolBytes + kQRopeBytes <= 160 * 1024, "tile pool and rope query fit the LDS");
  auto tile_slot = [&](int k) __attribute__((always_inline)) {
    return pool + (k & (G::kRing - 1)) * G::kSlotBytes;
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
  // read row rows-1 and are never stored.
  const int rowv = rb * kWRows + wave * 32 + r32;
  const int rc = min(rowv, p.rows - 1);
  const int limit = L - p.T + rc / p.Hq;           // last key position this row sees
  const uint16_t* qrow = p.q + b * p.qsb + (rc / p.Hq) * p.qst + (rc % p.Hq) * p.qsh;

  // Tiles that end at or before full_end need no mask: every token is in the
  // range and visible to every row of the wave (its first row has the
  // smallest causal limit).
  const int full_end = min(e, L - p.T + min(rb * kWRows + wave * 32, p.rows - 1) / p.Hq + 1);

  // The page size is a power of two for this kernel (checked on the host).
  const int psh = p.page_shift;
  const int pmask = p.page_size - 1;
  cint32* cbt = (cint32*)(p.bt + b * p.bt_stride);
  const uint32_t ksp = uint32_t(p.ksp), kst = uint32_t(p.kst);   // < 2^31, checked on the host

  // Tile fill: wave w issues the wave-level loads w, w+4, w+8, ... of those a
  // tile needs; a wave with one fewer repeats its last (same lanes, same
  // addresses, same bytes), so every wave issues kLPW and all waves' counts
  // agree.  Lane j of load i fills the 16-byte position q = 64*i + j of the
  // slot: token q / kChunks, position q % kChunks, which holds the chunk the
  // swizzle maps there.  Tokens past the range end load the range's last
  // token (finite, masked later).  The first half of the loads holds tokens
  // 0-15, the second tokens 16-31 (16 rows are a whole number of 1 KiB
  // loads), and a 16-token half of a tile lies in one page (tiles start on
  // multiples of 16, pages hold a power of two >= 16 tokens), so for a tile
  // inside the range a load reads one page: its address is a uniform page
  // base plus the lane's offset inside the half, lo[u].
  const int nt = (e - s + kTile - 1) / kTile;      // tiles of the range
  auto load_index = [&](int u) __attribute__((always_inline)) {
    int i = wave + kWWaves * u;
    if (i >= G::kLoads) i -= kWWaves;
    return i;
  };
  // (token, byte offset in its row) of the chunk lane fills in load u
  auto chunk_of = [&](int u, uint32_t& tk, uint32_t& c16) __attribute__((always_inline)) {
    const uint32_t qc = uint32_t(64 * load_index(u) + lane);
    tk = qc / uint32_t(G::kChunks);
    const uint32_t pos = qc - tk * G::kChunks;
    if constexpr (kCodes)
      c16 = 16u * ((pos & ~3u) | ((pos & 3u) ^ swz_e4m3(tk)));
    else
      c16 = 16u * (pos ^ swz_bf16(tk));
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
  constexpr int kHalf = G::kLoads / 2;
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

  // Pages of the first kAhead + 1 tiles: their scalar loads go out before
  // the query's loads and have landed when the first fills need them.
  int pg[2 * (kAhead + 1)];
#pragma unroll
  for (int k = 0; k <= kAhead; ++k) tile_pages(k, pg[2 * k], pg[2 * k + 1]);

  // The query, loaded before any tile.  bf16 (kinds 0, 1): lane (r32, h)
  // holds 8 features of the row for each 16-feature score product, in
  // registers for the 512 latent features and in LDS for the 64 rope features
  // -- kind 0: features 16 i + 8 h .. +7 for product i; kind 1 (a chunk of 16
  // codes feeds two products): features 32 m + 16 h .. +7 for product 2 m and
  // +8 .. +15 for product 2 m + 1.  e4m3 (kind 2): codes of features 64 p +
  // 32 h .. +31 for the 64-feature product p, all in registers.
  constexpr int kQOps = kQ8 ? 9 : 32;              // register operands
  bf16x8 qb[kQ8 ? 1 : kQOps];
  i32x8 qc8[kQ8 ? kQOps : 1];
  const lds_u8* qr = (const lds_u8*)qrope + wave * 4096 + 16 * lane;
  if constexpr (kQ8) {
    auto quantise_q = [&](auto FAST) __attribute__((always_inline)) {
      constexpr bool fast = decltype(FAST)::value;
#pragma unroll
      for (int pp = 0; pp < kQOps; ++pp) {
        const uint16_t* src = qrow + 64 * pp + 32 * h;
        u32x2 c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(src + 8 * j);
          c[j] = fast ? quantise8_rcp(w, p.q_scale, p.q_rcp) : quantise8(w, p.q_scale);
        }
        qc8[pp] = i32x8{int(c[0].x), int(c[0].y), int(c[1].x), int(c[1].y),
                        int(c[2].x), int(c[2].y), int(c[3].x), int(c[3].y)};
      }
    };
    // a division per value only for scales outside the fast path's bounds
    if (p.q_rcp != 0.f)
      quantise_q(std::true_type{});
    else
      quantise_q(std::false_type{});
  } else {
    // 16-byte chunk (8 features) of operand i
    auto qchunk = [&](int i) __attribute__((always_inline)) {
      return KIND == 0 ? 2 * i + h : 4 * (i >> 1) + 2 * h + (i & 1);
    };
    if (p.q_rows_linear) {
      // Row r of the sequence's query at r * qsh: the wave's 32 rows go
      // through its own 36 KiB of the tile pool, laid out as a bf16 key tile
      // (chunk c of row t at position c ^ swz_bf16(t)), with loads that read
      // 1 KiB of consecutive rows each -- loaded straight into the operand
      // layout, every load would touch 32 rows.  The operand reads then
      // follow the key reads' conflict-free pattern.
      const uint8_t* qbase = reinterpret_cast<const uint8_t*>(p.q + b * p.qsb);
      const uint32_t r0 = uint32_t(rb * kWRows + wave * 32), rlast = uint32_t(p.rows - 1);
      const uint32_t qrb = 2u * uint32_t(p.qsh);
      uint8_t* qs = pool + wave * (32 * 1152);
#pragma unroll
      for (int i = 0; i < 36; ++i) {
        const uint32_t qpos = 64u * i + lane;
        const uint32_t tk = qpos / 72u, c = (qpos - 72u * tk) ^ swz_bf16(tk);
        dma16_sbase(qbase, min(r0 + tk, rlast) * qrb + 16u * c, uint32_t(size_t((lds_u8*)(qs + 1024 * i))));
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      const lds_u8* qsl = (const lds_u8*)qs + r32 * 1152;
#pragma unroll
      for (int i = 0; i < kQOps; ++i) qb[i] = *(const lds_bf16x8*)(qsl + 16 * (qchunk(i) ^ swz_bf16(r32)));
#pragma unroll
      for (int i = kQOps; i < kQOps + 4; ++i)
        *(lds_u32x4*)(qrope + wave * 4096 + 1024 * (i - kQOps) + 16 * lane) =
            *(const lds_u32x4*)(qsl + 16 * (qchunk(i) ^ swz_bf16(r32)));
      // every wave has its query before the fills below reuse the pool
      lds_barrier();
    } else {
#pragma unroll
      for (int i = 0; i < kQOps; ++i) qb[i] = *reinterpret_cast<const bf16x8*>(qrow + 8 * qchunk(i));
      // the rope operands 32..35 go straight to LDS, so nothing waits for them
#pragma unroll
      for (int i = kQOps; i < kQOps + 4; ++i)
        dma16(reinterpret_cast<const uint8_t*>(qrow + 8 * qchunk(i)), uint32_t(size_t(qrope + wave * 4096 + 1024 * (i - kQOps))));
      // the wait for the query (and with it everything issued before it) here
#pragma unroll
      for (int i = 0; i < kQOps; ++i) asm volatile("" ::"v"(qb[i]));
    }
  }
  // the first kAhead tiles go out once the query has landed (a wait for it
  // issued after them would wait for them too)
#pragma unroll
  for (int k = 0; k < kAhead; ++k)
    if (k < nt) fill(k, tile_slot(k), pg[2 * k], pg[2 * k + 1]);
  int pa = pg[2 * kAhead], pb = pg[2 * kAhead + 1];     // pages of the tile the next fill loads

  // O^T accumulators: lane (r32, h) holds O[row r32][32 blk + 8 (v / 4) +
  // 4 h + v % 4] in o[blk][v].
  f32x16 o[kVb];
#pragma unroll
  for (int c = 0; c < kVb; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[c][v] = 0.f;
  constexpr float kRescaleMargin = 8.f;
  float m_ref = -INFINITY, m_true = -INFINITY, l_run = 0.f;

  // Byte offsets of this lane's K operand reads (token r32).  Kind 0: product
  // it reads chunk 2 it + h at kofs[it & 3] + 128 (it >> 2).  Kind 1: read m
  // takes chunk 2 m + h (16 codes: products 2 m and 2 m + 1) at
  // kofs[m & 1] + 64 (m >> 1).  Kind 2: product p takes chunks 4 p + 2 h + c
  // (c = 0, 1) at kofs[c] + 64 p.
  uint32_t kofs[KIND == 0 ? 4 : 2];
#pragma unroll
  for (int j = 0; j < (KIND == 0 ? 4 : 2); ++j) {
    if constexpr (KIND == 0)
      kofs[j] = uint32_t(r32) * kRowBytes + 16u * ((2u * j + h) ^ swz_bf16(r32));
    else if constexpr (KIND == 1)
      kofs[j] = uint32_t(r32) * kRowBytes + 16u * ((2u * j + h) ^ swz_e4m3(r32));
    else
      kofs[j] = uint32_t(r32) * kRowBytes + 16u * ((2u * h + j) ^ swz_e4m3(r32));
  }
  // Byte offsets of this lane's transposing V reads.  The score result leaves
  // lane (r32, h) the tokens 8 (v / 4) + 4 h + v % 4 of row r32 in item v, so
  // the value product's inner index 8 h + u of 16-token step kb is token
  // 16 kb + 8 (u / 4) + 4 h + u % 4, and its V^T operand gives lane (x, g1, h)
  // (x = lane & 15, g1 = bit 4) feature 32 blk + 16 g1 + x of those tokens.
  // Kind 0, two 16-bit transposing reads: read r (u / 4) of step kb points
  // the lane at token tv = 16 kb + 8 r + 4 h + x / 4, features 32 blk + 16 g1
  // + 4 (x & 3) .. +3: chunk c = 4 blk + 2 g1 + (x & 3) / 2, half x & 1, at
  // position c ^ swz_bf16(tv); with swz_bf16(tv) = (4 kb + 2 r + h) ^ 4 (x >> 3)
  // the offset inside the 128 bytes of blk >> 1 is 64 ((blk & 1) ^ kb ^ (x >> 3))
  // + 16 ((2 g1 + (x & 3) / 2) ^ (2 r + h)): vofs[(blk & 1) ^ kb][r], the rest
  // (16 kb + 8 r tokens, 128 (blk >> 1) bytes) a constant.
  // Codes, one byte transposing read: source lane x = 2 j + sh points at
  // token tv = 16 kb + 8 (j / 4) + 4 h + j % 4, codes 32 blk + 16 g1 + 8 sh
  // .. +7: chunk c = 2 blk + g1, half sh, at position 4 (c >> 2) + ((c & 3) ^
  // swz_e4m3(tv)); swz_e4m3(tv) = 2 (j / 4) + kb, so the offset is 576 tv +
  // 64 (blk >> 1) + 32 ((blk & 1) ^ (j / 4)) + 16 (g1 ^ kb) + 8 sh:
  // vofs[kb][blk & 1] plus 64 (blk >> 1).
  uint32_t vofs[2][2];
  {
    const uint32_t x = lane & 15, g1 = (lane >> 4) & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        if constexpr (KIND == 0) {
          vofs[i][j2] = (4u * h + (x >> 2)) * kRowBytes + 64u * (i ^ (x >> 3)) +
                        16u * ((2u * g1 + ((x & 3u) >> 1)) ^ (2u * j2 + h)) + 8u * (x & 1u);
        } else {
          const uint32_t j = x >> 1, sh = x & 1;
          const uint32_t tv = 16u * i + 8u * (j >> 2) + 4u * h + (j & 3u);
          vofs[i][j2] = tv * kRowBytes + 32u * (j2 ^ (j >> 2)) + 16u * (g1 ^ i) + 8u * sh;
        }
      }
  }

  // One 32-token tile in slotp, tokens t0 .. t0+31 of the range; fill_u(u)
  // issues load u of a later tile's fill (or nothing), spread over the score
  // products.
  auto tile = [&](const uint8_t* slotp, int t0, auto&& fill_u) __attribute__((always_inline)) {
    const lds_u8* ls = (const lds_u8*)slotp;
    f32x16 sacc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
    if constexpr (KIND == 0) {
      // ---- S^T = K Q^T: 36 products into one accumulator, each K operand
      // read four products ahead
      constexpr int kN = 36, kAh = 4;
      bf16x8 kr[kN], qrr[kN];
      auto kread = [&](int it) __attribute__((always_inline)) {
        kr[it] = *(const lds_bf16x8*)(ls + kofs[it & 3] + 128 * (it >> 2));
        if (it >= 32) qrr[it] = *(const lds_bf16x8*)(qr + 1024 * (it - 32));
      };
#pragma unroll
      for (int it = 0; it < kAh; ++it) kread(it);
#pragma unroll
      for (int it = 0; it < kN; ++it) {
        if (it + kAh < kN) kread(it + kAh);
        if (it % 4 == 2 && it / 4 < kLPW) fill_u(it / 4);
        sacc = mfma32(kr[it], it < 32 ? qb[it] : qrr[it], sacc);
      }
      // Hold the scheduler to that order (left alone it issues each read just
      // before its product, which then waits out the LDS latency): the first
      // reads, then product, read (two for a rope product), ...
      __builtin_amdgcn_sched_group_barrier(0x100, kAh, 0);
#pragma unroll
      for (int it = 0; it < 32 - kAh; ++it) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int it = 32 - kAh; it < kN - kAh; ++it) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int it = kN - kAh; it < kN; ++it) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    } else if constexpr (KIND == 1) {
      // ---- 18 reads of 16 codes, each widened into the operands of two
      // products; the reads run three ahead (with the rope query's two
      // operand reads for the last two)
      constexpr int kN = 18, kAh = 3;
      u32x4 kr[kN], qlo[kN], qhi[kN];
      auto kread = [&](int m) __attribute__((always_inline)) {
        kr[m] = *(const lds_u32x4*)(ls + kofs[m & 1] + 64 * (m >> 1));
        if (m >= 16) {
          qlo[m] = *(const lds_u32x4*)(qr + 1024 * (2 * (m - 16)));
          qhi[m] = *(const lds_u32x4*)(qr + 1024 * (2 * (m - 16) + 1));
        }
      };
#pragma unroll
      for (int m = 0; m < kAh; ++m) kread(m);
#pragma unroll
      for (int m = 0; m < kN; ++m) {
        if (m + kAh < kN) kread(m + kAh);
        if (m % 2 == 1 && m / 2 < kLPW) fill_u(m / 2);
        const bf16x8 qa = m < 16 ? qb[2 * m] : __builtin_bit_cast(bf16x8, qlo[m]);
        const bf16x8 qz = m < 16 ? qb[2 * m + 1] : __builtin_bit_cast(bf16x8, qhi[m]);
        sacc = mfma32(widen8(kr[m].x, kr[m].y), qa, sacc);
        sacc = mfma32(widen8(kr[m].z, kr[m].w), qz, sacc);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, kAh, 0);
#pragma unroll
      for (int m = 0; m < 16 - kAh; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int m = 16 - kAh; m < kN - kAh; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      }
#pragma unroll
      for (int m = kN - kAh; m < kN; ++m) __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    } else {
      // ---- e4m3 queries: nine 64-feature products on the codes, two
      // 16-byte reads each, two products ahead
      constexpr int kN = 9, kAh = 2;
      u32x4 kr[kN][2];
      auto kread = [&](int pp) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < 2; ++c) kr[pp][c] = *(const lds_u32x4*)(ls + kofs[c] + 64 * pp);
      };
#pragma unroll
      for (int pp = 0; pp < kAh; ++pp) kread(pp);
#pragma unroll
      for (int pp = 0; pp < kN; ++pp) {
        if (pp + kAh < kN) kread(pp + kAh);
        if (pp < kLPW) fill_u(pp);
        const i32x8 ka = {int(kr[pp][0].x), int(kr[pp][0].y), int(kr[pp][0].z), int(kr[pp][0].w),
                          int(kr[pp][1].x), int(kr[pp][1].y), int(kr[pp][1].z), int(kr[pp][1].w)};
        sacc = mma64(ka, qc8[pp], sacc);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAh, 0);
#pragma unroll
      for (int pp = 0; pp < kN - kAh; ++pp) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int pp = kN - kAh; pp < kN; ++pp) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    // the first value products' operands do not depend on the scores: their
    // reads overlap the softmax
    v4i16 va[2 * kVb], vb[2 * kVb];
    i32x2 vc[2 * kVb];
    auto vread = [&](int n) __attribute__((always_inline)) {
      const int kb = n / kVb, blk = n % kVb;
      if constexpr (KIND == 0) {
        const lds_u8* base = ls + 16 * kb * kRowBytes + 128 * (blk >> 1);
        va[n] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + vofs[(blk & 1) ^ kb][0]));
        vb[n] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + 8 * kRowBytes + vofs[(blk & 1) ^ kb][1]));
      } else {
        vc[n] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(ls + 64 * (blk >> 1) + vofs[kb][blk & 1]));
      }
    };
    auto vop = [&](int n) __attribute__((always_inline)) {
      if constexpr (KIND == 0)
        return __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(u32x2, va[n]).x, __builtin_bit_cast(u32x2, va[n]).y,
                                                __builtin_bit_cast(u32x2, vb[n]).x, __builtin_bit_cast(u32x2, vb[n]).y});
      else
        return widen8(uint32_t(vc[n].x), uint32_t(vc[n].y));
    };
    constexpr int kVReads = KIND == 0 ? 2 : 1;     // reads per value product
#pragma unroll
    for (int n = 0; n < kVAhead; ++n) vread(n);
    __builtin_amdgcn_sched_group_barrier(0x100, kVReads * kVAhead, 0);
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
      if (n + kVAhead < 2 * kVb) vread(n + kVAhead);
      o[n % kVb] = mfma32(vop(n), pk[n / kVb], o[n % kVb]);
    }
    // as for the scores: read ahead, product, ...
#pragma unroll
    for (int n = 0; n < 2 * kVb - kVAhead; ++n) {
      __builtin_amdgcn_sched_group_barrier(0x100, kVReads, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
#pragma unroll
    for (int n = 2 * kVb - kVAhead; n < 2 * kVb; ++n) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  };

  // Step k: wait until this wave's loads of tile k are done (those of the
  // next kAhead - 1 tiles, where the range has them, may still be in
  // flight), then a barrier so every wave's part of the tile has landed --
  // which also means every wave has finished tile k-1, whose slot (the ring
  // holds kAhead + 1 tiles or more) takes tile k + kAhead.  Tiles past the
  // range are never loaded: the wait allows as many loads in flight as the
  // range has tiles after k.
  // Steps whose fill is a tile before the range's last spread its loads over
  // the score products; the others (TAIL) fill the range's last tile, which
  // may be cut by the range end, up front, or nothing.
  auto step = [&](int k, auto TAIL) __attribute__((always_inline)) {
    constexpr bool tail = decltype(TAIL)::value;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if constexpr (!tail)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((kAhead - 1) * kLPW));
    else
      wait_tiles<kLPW>(min(kAhead - 1, nt - 1 - k));
    lds_barrier();
    if (tail && k + kAhead < nt) fill(k + kAhead, tile_slot(k + kAhead), pa, pb);
    const uint8_t* cur = tile_slot(k);
    const int t0 = s + kTile * k;
    if constexpr (!tail) {
      const WholeFill f = whole_fill(k + kAhead, tile_slot(k + kAhead), pa, pb);
      tile(cur, t0, [&](int u) __attribute__((always_inline)) { whole_load(f, u); });
    } else {
      tile(cur, t0, [](int) {});
    }
    // pages for the next step's fill; their wait is the next step's barrier.
    // The scheduling barrier keeps these scalar loads behind every value read
    // of the tile: while one is in flight the compiler can only wait for LDS
    // reads with lgkmcnt(0), which would drain the reads in flight.
    __builtin_amdgcn_sched_barrier(0);
    tile_pages(k + kAhead + 1, pa, pb);
  };

  if (nt > 0) {
    // tiles k + kAhead < nt - 1 are inside the range; tile nt - 1 may be cut
    int k = 0;
    for (; k + kAhead + 1 < nt; ++k) step(k, std::false_type());
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
    // three-operand integer maxima per pair of values.  A half's 128 values
    // per lane are copied out of the accumulation registers once and serve
    // both its maximum and its codes.
    float amax[2];
    lds_u8* st = (lds_u8*)pool + (wave * 32) * kCodeRowBytes;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      float xv[128];
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) xv[16 * c + v] = o[8 * hf + c][v];
      int32_t smax = INT32_MIN;
      uint32_t umax = 0;
#pragma unroll
      for (int v = 0; v < 128; v += 2) {
        const int32_t x = __float_as_int(xv[v]), y = __float_as_int(xv[v + 1]);
        smax = max(smax, max(x, y));
        umax = max(umax, max(uint32_t(x), uint32_t(y)));
      }
      const float a = pair_max(fmaxf(fabsf(__int_as_float(smax)), fabsf(__uint_as_float(umax))));
      amax[hf] = a * fabsf(mul);
      // o * kq lies in [-1, 1]; its code is the nearest integer to 32767 times it
      const float kq = amax[hf] > 0.f ? mul / amax[hf] : 0.f;
      if (hf == 0) __syncthreads();        // every wave is done with the tile pool
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // v_cvt_pknorm_i16_f32: two values in [-1, 1] to the nearest
          // multiples of 1/32767, as int16 codes
          const float* x4 = xv + 16 * c + 4 * j;
          const u32x2 w = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(x4[0] * kq, x4[1] * kq)),
                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(x4[2] * kq, x4[3] * kq))};
          *(__attribute__((address_space(3))) u32x2*)(st + r32 * kCodeRowBytes +
                                                      2 * (32 * (8 * hf + c) + 8 * j + 4 * h)) = w;
        }
    }
    // each wave reads back only what it wrote (no barrier; the LDS waits
    // suffice), eight rows in flight at a time; rows are in (t, h) order, so
    // a row's index within the sequence is the row number itself
    const int row0 = rb * kWRows + wave * 32;
    int16_t* qdst = p.part_q + (int64_t(slot) * R + row0) * kDv + 8 * lane;
    const lds_u8* qsrc = st + 16 * lane;
    if (row0 + 32 <= p.rows) {
#pragma unroll
      for (int r0 = 0; r0 < 32; r0 += 8) {
        u32x4 w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = *(const lds_u32x4*)(qsrc + (r0 + j) * kCodeRowBytes);
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(qdst + (r0 + j) * kDv) = w[j];
      }
    } else {
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const u32x4 w = *(const lds_u32x4*)(qsrc + r * kCodeRowBytes);
        if (row0 + r < p.rows) *reinterpret_cast<u32x4*>(qdst + r * kDv) = w;
      }
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

// kind: 0 bf16 cache, 1 e4m3 cache with bf16 queries, 2 e4m3 cache and queries.
hipError_t launch_mla_partial(const PartialParams& p, int kind, hipStream_t stream) {
  const int per_xcd = (p.total_wg + 7) / 8;
  const dim3 grid(unsigned(per_xcd * 8)), block(256);
  if (kind == 2)
    hipLaunchKernelGGL(mla_partial_kernel<2>, grid, block, 0, stream, p, per_xcd);
  else if (kind == 1)
    hipLaunchKernelGGL(mla_partial_kernel<1>, grid, block, 0, stream, p, per_xcd);
  else
    hipLaunchKernelGGL(mla_partial_kernel<0>, grid, block, 0, stream, p, per_xcd);
  return hipGetLastError();
}

}  // namespace splitkv
