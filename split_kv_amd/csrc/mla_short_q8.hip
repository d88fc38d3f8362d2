// Short-range MLA split-KV partial kernel with e4m3 queries over an e4m3
// latent cache, on gfx950's FP8 matrix instructions.  The host runs it
// instead of the 128-row kernel (mla.hip, kind 2) for short steps (every
// split at most eight 32-token tiles, the 64-row workgroups all on the compute
// units at once), where its two waves per SIMD hide a workgroup's fixed costs.
//
// FP8 queries let the scores run on the FP8 matrix path against an FP8 KV
// cache ("Xqa decode kernels", timeline: the FP8-Q selection, gated on the
// hardware and on the layer's cache being FP8).  The query is quantised here
// to e4m3 codes of q / q_scale (the correctly rounded fp32 quotient,
// saturating, round to nearest even, the same encoding as the cache write); the scores are
// sum(q code x k code) x q_scale x k_scale x softmax scale.  The
// probabilities enter P V as e4m3 too, as two terms: P (<= 2^8 against the
// reference max, inside e4m3's range) = hi + lo + r with hi and lo e4m3 codes
// and |r| <= 2^-8 P + 2^-10 (the weight sum adds P itself); one e4m3 term
// alone (3 mantissa bits, up to 2^-4 relative per weight) moves an output
// that averages a few values of comparable weight by several hundredths.
//
// Work layout (same row blocks, pairs and epilogue as the bf16-query kernel):
// a workgroup keeps 64 query rows, eight waves (two per SIMD) form four
// pairs, a pair owns 16 rows, and the pair's two waves split the key features
// for the scores (each takes 288 of 576, the two swap partial sums through
// LDS) and the value features for the output (256 of 512 each).
//   * Scores: v_mfma_f32_16x16x128_f8f6f4 (16 tokens x 16 rows x 128
//     features, twice the bf16 rate) for features 0..511, and the 32-wide
//     v_mfma_f32_16x16x32_fp8_fp8 for the 64 rope features; the e4m3 codes
//     are the operands, so nothing is widened.
//   * P V: v_mfma_f32_16x16x128_f8f6f4 with the 128 tokens as the inner
//     dimension: the softmax runs over windows of four 32-token sub-tiles,
//     after which each wave issues 32 such products (16 value features each,
//     hi and lo terms of P)
//     whose V^T operand comes from the token-major code tiles through the
//     gfx950 transposing byte read (ds_read_b64_tr_b8: in a 16-lane group,
//     lane x receives byte x & 7 of the 8-byte vectors read by lanes
//     2j + (x >> 3), j = 0..7, measured with an in-bounds probe).
//   * The inner-dimension order of both products is a free choice as long
//     as the two operands agree; here byte 8r + 4g + i of a lane's 32-byte
//     operand is token 32r + 16g + 4qg + i of the window (qg = lane / 16), which
//     is the order the score products leave the probabilities in.
//   * Sub-tiles (32 tokens x 576 code bytes) arrive by direct global->LDS
//     loads into a ring of eight, four ahead of the one being computed: the
//     window being multiplied holds four slots while the next window's four
//     are filled.  Chunk c (16 bytes) of sub-tile token t sits at position
//     c ^ swz8(t); the 2-bit swizzle keeps the score operand reads (16 tokens
//     x 2 chunks per 32 lanes) and the transposing value reads (16 tokens x 2
//     halves of a chunk per 32 lanes) free of bank conflicts, and stays
//     inside the aligned groups of four chunks a 36-chunk row is made of.
//   * Eight slots (144 KiB) and the 16 KiB exchange buffer fill the LDS.
#include "mla_short_common.h"

namespace splitkv {

namespace {

using namespace mla_short;

constexpr int kSub = 32;                          // tokens per sub-tile (one ring slot)
constexpr int kWin = 4;                           // sub-tiles per softmax window (128 tokens)
constexpr int kSlotBytes = kSub * kDqk;           // 18432
constexpr int kSlotLoads = kSlotBytes / 1024;     // 18 wave-level 1 KiB loads
constexpr int kChunks = kDqk / 16;                // 36 16-byte chunks per code row
constexpr int kLPW = 3;                           // loads per wave and sub-tile
constexpr int kRing = 8;
constexpr int kAhead = 4;                         // sub-tiles in flight ahead of the current one
static_assert((kLPW - 1) * kWaves < kSlotLoads && kLPW * kWaves >= kSlotLoads,
              "three loads per wave cover a sub-tile");
static_assert(kRing * kSlotBytes + kWaves * 2 * 64 * 16 == 160 * 1024, "ring and exchange fill the LDS");
static_assert(kChunks % 4 == 0, "the swizzle permutes aligned groups of four chunks");
static_assert(kRing == 2 * kAhead && kAhead == kWin, "one window computed while the next is filled");
static_assert(kStageBytes <= kRing * kSlotBytes, "the epilogue's staging fits the sub-tile ring");

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) uint64_t lds_u64;
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Position swizzle of sub-tile token t's chunks (t in 0..31).
__device__ __forceinline__ uint32_t swz8(uint32_t t) {
  return ((t >> 2) & 1u) | ((((t >> 3) ^ (t >> 4)) & 1u) << 1);
}

// D += A B over 128 e4m3 inner elements (A and B both e4m3: format codes 0;
// with both scale operands zero the compiler emits the unscaled instruction).
__device__ __forceinline__ f32x4 mma128(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(uint64_t a, uint64_t b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(long(a), long(b), c, 0, 0, 0);
}

}  // namespace

__global__ __launch_bounds__(512) void mla_short_q8_partial_kernel(PartialParams p, int per_xcd) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRing * kSlotBytes];
  __shared__ f32x4 xch[kWaves][2][64];              // partial scores: [wave][group][lane]
  auto slot_ptr = [&](int k) __attribute__((always_inline)) {
    return ring + (k & (kRing - 1)) * kSlotBytes;
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
  const int pair = wave >> 1, hf = wave & 1;
  const int n16 = lane & 15, qg = lane >> 4;

  const SlotWork work = load_slot(p.slot_info, slot);
  const int b = work.b, split = work.split, nsplit = work.nsplit, s = work.s, e = work.e;
  const int L = ((cint32*)p.seq_lens)[b];

  // This lane's query row, quantised: the 16x16x128 steps 2hf and 2hf+1 take
  // features 128 ks + 16 qg .. +15 (bytes 0-15 of the operand) and
  // 128 ks + 64 + 16 qg .. +15 (bytes 16-31); the 16x16x32 step takes
  // features 512 + 32 hf + 8 qg .. +7.  Rows past the last read row rows-1
  // and are never stored.
  const int rowv = rb * kRows + pair * 16 + n16;
  int limit;
  i32x8 qa[2];
  uint64_t qr;
  {
    const int rc = min(rowv, p.rows - 1);
    const int t = rc / p.Hq, h = rc % p.Hq;
    limit = L - p.T + t;      // last key position this row sees
    const uint16_t* qrow = p.q + b * p.qsb + t * p.qst + h * p.qsh;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint16_t* ca = qrow + 128 * (2 * hf + j) + 16 * qg;
      const uint16_t* cb = ca + 64;
      const u32x2 c0 = quantise8(*reinterpret_cast<const u32x4*>(ca), p.q_scale);
      const u32x2 c1 = quantise8(*reinterpret_cast<const u32x4*>(ca + 8), p.q_scale);
      const u32x2 c2 = quantise8(*reinterpret_cast<const u32x4*>(cb), p.q_scale);
      const u32x2 c3 = quantise8(*reinterpret_cast<const u32x4*>(cb + 8), p.q_scale);
      qa[j] = i32x8{int(c0.x), int(c0.y), int(c1.x), int(c1.y), int(c2.x), int(c2.y), int(c3.x), int(c3.y)};
    }
    const u32x2 cr = quantise8(*reinterpret_cast<const u32x4*>(qrow + 512 + 32 * hf + 8 * qg), p.q_scale);
    qr = (uint64_t(cr.y) << 32) | cr.x;
  }
  // The query has landed before the first fill is issued (the compiler's own
  // waits for it would otherwise also drain the fills in flight).
  __builtin_amdgcn_s_waitcnt(0x0F70);                      // vmcnt(0)

  // Sub-tiles that end at or before full_end need no mask.
  const int full_end = min(e, L - p.T + min(rb * kRows + pair * 16, p.rows - 1) / p.Hq + 1);

  const int psh = p.page_shift;                   // page size: a power of two >= 16
  const int pmask = p.page_size - 1;
  cint32* cbt = (cint32*)(p.bt + b * p.bt_stride);
  const uint32_t ksp = uint32_t(p.ksp), kst = uint32_t(p.kst);   // < 2^31, checked on the host

  // Sub-tile fill: wave w issues the wave-level loads w, w+8 and (waves 0
  // and 1) w+16 of the 18, so waves 0-1 issue three per sub-tile and the
  // others two; each waits with its own count.  Lane j of load i fills
  // 16-byte position q = 64 i + j: token q / 36, holding chunk
  // (q % 36) ^ swz8(token).  Loads 0-8 hold tokens 0-15 and loads 9-17
  // tokens 16-31; a 16-token half lies in one page, so a sub-tile inside the
  // range reads each half from a uniform page base plus a per-lane offset.
  // Tokens past the range end load the range's last token; sub-tiles past
  // the range but inside its last window reload the last one (finite codes,
  // never unmasked); nothing past the last window is loaded.
  const int nt = (e - s + kSub - 1) / kSub;
  const bool third = wave + kWaves * (kLPW - 1) < kSlotLoads;   // waves 0 and 1
  auto load_index = [&](int u) __attribute__((always_inline)) {
    int i = wave + kWaves * u;
    if (i >= kSlotLoads) i -= kWaves;      // (never issued: only the offsets are computed)
    return i;
  };
  uint32_t fl[kLPW], lo[kLPW];
#pragma unroll
  for (int u = 0; u < kLPW; ++u) {
    const uint32_t qc = uint32_t(64 * load_index(u) + lane);
    const uint32_t tk = qc / uint32_t(kChunks);
    const uint32_t c = (qc - tk * kChunks) ^ swz8(tk);
    fl[u] = (tk << 16) | (16u * c);
    lo[u] = (tk & 15u) * kst + 16u * c;
  }
  auto tile_pages = [&](int k, int& pa, int& pb) __attribute__((always_inline)) {
    const int t0 = s + kSub * min(k, nt - 1);
    const int last = min(t0 + kSub - 1, e - 1);
    pa = cbt[t0 >> psh];
    pb = cbt[last >> psh];
  };
  auto fill = [&](int k, int pa, int pb) __attribute__((always_inline)) {
    uint8_t* slotp = slot_ptr(k);
    const int t0 = s + kSub * min(k, nt - 1);
    if (t0 + kSub <= e) {
      const uint8_t* half0 = p.k + uint64_t(uint32_t(pa)) * ksp + uint32_t(t0 & pmask) * kst;
      const uint8_t* half1 = p.k + uint64_t(uint32_t(pb)) * ksp + uint32_t((t0 + 16) & pmask) * kst;
#pragma unroll
      for (int u = 0; u < kLPW; ++u) {
        if (u == kLPW - 1 && !third) break;
        const int i = load_index(u);
        dma16_sbase(i < kSlotLoads / 2 ? half0 : half1, lo[u], uint32_t(size_t((lds_u8*)(slotp + 1024 * i))));
      }
      return;
    }
    const int last = min(t0 + kSub - 1, e - 1);
    const int pi0 = t0 >> psh;
    const uint64_t base0 = uint64_t(uint32_t(pa)) * ksp;
    const uint64_t base1 = uint64_t(uint32_t(pb)) * ksp;
#pragma unroll
    for (int u = 0; u < kLPW; ++u) {
      if (u == kLPW - 1 && !third) break;
      const int i = load_index(u);
      const int tok = min(t0 + int(fl[u] >> 16), last);
      const uint64_t base = (tok >> psh) == pi0 ? base0 : base1;
      const uint8_t* src = p.k + (base + uint64_t(uint32_t(tok & pmask) * kst + (fl[u] & 0xffffu)));
      dma16(src, uint32_t(size_t((lds_u8*)(slotp + 1024 * i))));
    }
  };

  // Score operand offsets inside a slot, group g (tokens 16 g + n16):
  // 16x16x128 step ks reads chunk 8 ks + qg at kofs[g] + 128 ks and chunk
  // 8 ks + 4 + qg 64 bytes later; the 16x16x32 step reads 8 bytes at rofs[g].
  uint32_t kofs[2], rofs[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const uint32_t tt = 16u * g + n16, sw = swz8(tt);
    kofs[g] = tt * kDqk + 16u * (uint32_t(qg) ^ sw);
    rofs[g] = tt * kDqk + 16u * (32u + ((2u * hf + (uint32_t(qg) >> 1)) ^ sw)) + 8u * (qg & 1);
  }
  // Transposing value reads: lane x = n16 of group qg points at token
  // 16 (j >> 2) + 4 qg + (j & 3), j = x >> 1, bytes 8 (x & 1) .. +7 of the
  // 16-feature chunk being read; vofs[m] for a chunk index = m mod 4.
  uint32_t vofs[4];
  {
    const uint32_t j = uint32_t(n16) >> 1;
    const uint32_t tt = 16u * (j >> 2) + 4u * qg + (j & 3u), sw = swz8(tt);
#pragma unroll
    for (int m = 0; m < 4; ++m) vofs[m] = tt * kDqk + 16u * (uint32_t(m) ^ sw) + 8u * (n16 & 1);
  }

  // O^T accumulators over this wave's value half: lane (n16, qg) holds
  // O[row n16][256 hf + 16 e + 4 qg + i] in o[e][i].
  f32x4 o[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr float kRescaleMargin = 8.f;
  float m_ref = -INFINITY, m_true = -INFINITY, l_run = 0.f;
  float sv[kWin * 8];       // the window's scores (base 2): sub-tile r, group g, token 4qg + i at 8r + 4g + i
  int dbg_groups = 0, dbg_xor = 0;
  uint32_t dbg_sum = 0;
  int pa = 0, pb = 0;       // pages of the next fill

  // Step k (sub-tile r = k mod 4 of its window): wait for this wave's loads of
  // sub-tile k (those of k+1..k+3, three or two per sub-tile, may still be in
  // flight; in the last window only those up to its end, the last sub-tile
  // loaded), then a barrier so every wave's part has landed -- which also
  // means every wave has finished step k-1, so the exchange buffer can be
  // reused, and the previous window's products, so its slots can be refilled.
  auto step = [&](int k, auto R, auto LASTW) __attribute__((always_inline)) {
    constexpr int r = decltype(R)::value;
    constexpr bool lastw = decltype(LASTW)::value;
    constexpr int ahead_last = kWin - 1 - r;               // sub-tiles after k in the last window
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if constexpr (!lastw) {
      if (third)
        __builtin_amdgcn_s_waitcnt(0x0F70 | (3 * kLPW));         // vmcnt(9)
      else
        __builtin_amdgcn_s_waitcnt(0x0F70 | (3 * (kLPW - 1)));   // vmcnt(6)
    } else {
      if (third)
        __builtin_amdgcn_s_waitcnt(0x0F70 | (ahead_last * kLPW));
      else
        __builtin_amdgcn_s_waitcnt(0x0F70 | (ahead_last * (kLPW - 1)));
    }
    lds_barrier();
    const uint8_t* cur = slot_ptr(k);
    const int t0 = s + kSub * k;
    if (k < nt) {
      const int pg0 = cbt[t0 >> psh];
      const bool has1 = t0 + 16 < e;
      const int pg1 = has1 ? cbt[(t0 + 16) >> psh] : 0;
      dbg_groups += has1 ? 2 : 1;
      dbg_xor ^= pg0 ^ pg1;
      dbg_sum += uint32_t(pg0) + uint32_t(pg1);
    }
    // ---- partial S^T = K Q^T over this wave's key half, both 16-token groups
    const lds_u8* sp = (const lds_u8*)cur;
    i32x8 ka[2][2];
    uint64_t kr[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const lds_u8* a = sp + kofs[g] + 128 * (2 * hf + j);
        const u32x4 x0 = *(const lds_u32x4*)a;
        const u32x4 x1 = *(const lds_u32x4*)(a + 64);
        ka[g][j] = i32x8{int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
      }
      kr[g] = *(const lds_u64*)(sp + rofs[g]);
    }
    // every operand read is issued before the first product (the scheduler
    // would otherwise pair each read with its product and wait on each)
    __builtin_amdgcn_sched_barrier(0);
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    s0 = mma128(ka[0][0], qa[0], s0);
    s1 = mma128(ka[1][0], qa[0], s1);
    s0 = mma128(ka[0][1], qa[1], s0);
    s1 = mma128(ka[1][1], qa[1], s1);
    s0 = mma32(kr[0], qr, s0);
    s1 = mma32(kr[1], qr, s1);
    // ---- swap partials with the pair's other wave (both add the same two
    // values, so both hold identical scores)
    xch[wave][0][lane] = s0;
    xch[wave][1][lane] = s1;
    lds_barrier();
    // sub-tile k+4 into the slot sub-tile k-4 left (its window's products
    // finished before this step's first barrier); the last window loads none
    if constexpr (!lastw) fill(k + kAhead, pa, pb);
    const int w2 = wave ^ 1;
    const f32x4 sc[2] = {s0 + xch[w2][0][lane], s1 + xch[w2][1][lane]};
    if (t0 + kSub <= full_end) {
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[8 * r + 4 * g + i] = sc[g][i] * p.scale_log2;
    } else {
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tk = t0 + 16 * g + 4 * qg + i;
          sv[8 * r + 4 * g + i] = (tk < e && tk <= limit) ? sc[g][i] * p.scale_log2 : -INFINITY;
        }
    }
    // pages of the next step's fill; their wait is the next step's barrier
    tile_pages(k + kAhead + 1, pa, pb);
  };

  // Window w (sub-tiles 4w .. 4w+3): online softmax over its 128 tokens in
  // base 2 (lazily moved reference max), P as two e4m3 terms, then
  // O^T[d][row] += V^T P^T with two 128-deep products (hi, lo) per 16 value features.
  auto window = [&](int w) __attribute__((always_inline)) {
    float m32 = sv[0];
#pragma unroll
    for (int i = 1; i < kWin * 8; ++i) m32 = fmaxf(m32, sv[i]);
    const float mx = column_max4(m32);
    m_true = fmaxf(m_true, mx);
    const bool bump = mx > m_ref + kRescaleMargin;
    if (__any(bump)) {
      const float m_new = bump ? mx : m_ref;
      // a row that does not move keeps alpha = 1 exactly: computing it would
      // give exp2(-inf - -inf) = NaN for a row with nothing visible yet
      const float alpha = bump ? fast_exp2(m_ref - m_new) : 1.f;   // 0 on the first visible window
      l_run *= alpha;
      m_ref = m_new;
#pragma unroll
      for (int c = 0; c < 16; ++c) o[c] *= alpha;
    }
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    // P = hi + lo: hi the nearest e4m3 value, lo the nearest e4m3 value of the
    // (exactly computed) remainder, so hi + lo is within 2^-8 of P relative
    // (plus 2^-10 absolute where lo falls below e4m3's normal range)
    i32x8 ph, pl;
    float lsum = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const float p0 = fast_exp2(sv[4 * d] - m_use), p1 = fast_exp2(sv[4 * d + 1] - m_use);
      const float p2 = fast_exp2(sv[4 * d + 2] - m_use), p3 = fast_exp2(sv[4 * d + 3] - m_use);
      int c = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
      c = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, c, true);
      ph[d] = c;
      const f32x2 r01 = __builtin_amdgcn_cvt_pk_f32_fp8(c, false);
      const f32x2 r23 = __builtin_amdgcn_cvt_pk_f32_fp8(c, true);
      int c2 = __builtin_amdgcn_cvt_pk_fp8_f32(p0 - r01.x, p1 - r01.y, 0, false);
      c2 = __builtin_amdgcn_cvt_pk_fp8_f32(p2 - r23.x, p3 - r23.y, c2, true);
      pl[d] = c2;
      lsum += (p0 + p1) + (p2 + p3);
    }
    l_run += lsum;
    const lds_u8* vb[kWin];
#pragma unroll
    for (int r = 0; r < kWin; ++r) vb[r] = (const lds_u8*)slot_ptr(kWin * w + r) + 256 * hf;
    // V^T operand of value block e16: four transposing reads, one per sub-tile
    auto read_v = [&](int e16) __attribute__((always_inline)) {
      i32x8 a;
#pragma unroll
      for (int r = 0; r < kWin; ++r) {
        const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_i32x2*)(vb[r] + 64 * (e16 >> 2) + vofs[e16 & 3]));
        a[2 * r] = v.x;
        a[2 * r + 1] = v.y;
      }
      return a;
    };
    // two value blocks per stage: the next stage's reads are issued before
    // this stage's products, and the hi and lo products of a block are
    // separated by the other block's (no back-to-back dependent products)
    i32x8 a0 = read_v(0), a1 = read_v(1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      i32x8 n0 = a0, n1 = a1;
      if (j < 7) {
        n0 = read_v(2 * j + 2);
        n1 = read_v(2 * j + 3);
      }
      __builtin_amdgcn_sched_barrier(0);
      o[2 * j] = mma128(a0, ph, o[2 * j]);
      o[2 * j + 1] = mma128(a1, ph, o[2 * j + 1]);
      o[2 * j] = mma128(a0, pl, o[2 * j]);
      o[2 * j + 1] = mma128(a1, pl, o[2 * j + 1]);
      __builtin_amdgcn_sched_barrier(0);
      a0 = n0;
      a1 = n1;
    }
  };

  if (nt > 0) {
#pragma unroll
    for (int k = 0; k < kAhead; ++k) {
      tile_pages(k, pa, pb);
      fill(k, pa, pb);
    }
    tile_pages(kAhead, pa, pb);
    const int nw = (nt + kWin - 1) / kWin;
    auto win_steps = [&](int w, auto LASTW) __attribute__((always_inline)) {
      step(kWin * w + 0, std::integral_constant<int, 0>(), LASTW);
      step(kWin * w + 1, std::integral_constant<int, 1>(), LASTW);
      step(kWin * w + 2, std::integral_constant<int, 2>(), LASTW);
      step(kWin * w + 3, std::integral_constant<int, 3>(), LASTW);
      window(w);
    };
    for (int w = 0; w + 1 < nw; ++w) win_steps(w, std::false_type());
    win_steps(nw - 1, std::true_type());
  }
  // no wave leaves while loads it issued may still write LDS
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);                      // vmcnt(0)

  store_rows(p, o, rowv, qg, hf, b, slot, nsplit, m_ref, m_true, l_run, ring);
  if (p.debug && tid == 0) store_debug(p, slot, rb, b, split, s, e, dbg_groups, dbg_xor, dbg_sum);
}

hipError_t launch_mla_short_q8_partial(const PartialParams& p, hipStream_t stream) {
  const int per_xcd = (p.total_wg + 7) / 8;
  const dim3 grid(unsigned(per_xcd * 8)), block(512);
  hipLaunchKernelGGL(mla_short_q8_partial_kernel, grid, block, 0, stream, p, per_xcd);
  return hipGetLastError();
}

}  // namespace splitkv
