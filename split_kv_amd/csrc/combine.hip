// Log-sum-exp combine of split partials, and the e4m3 widening check kernel.
//
// The combine merges the (m, l, o) partials of a sequence's splits into the
// softmax output: M = max_i m_i, w_i = exp(m_i - M), out = sum w_i o_i /
// sum w_i l_i, lse = M + ln(sum w_i l_i).  An empty split carries m = -inf and
// gets weight zero, which is why a split count that leaves ranges empty still
// gives the right answer ("vLLM 0.30.0 FA4 SplitKV Bug: H100 Decode Can Be 48%
// Slower", section "Why the result is still correct").  Its cost grows with
// the split count ("Shipped: 484.5 tok/s on one GB300 ...", section "Why 8
// splits lost"): it reads S * rows * (d_v + 2) * 4 bytes of partials, or
// S * rows * (2 * d_v + 16) in the MLA kernels' compact layout (int16 codes
// of o with a scale per 256-feature half).
//
// fp32 partials: a workgroup merges one row's partials over C float4 columns
// (4C features) with G groups of threads over the splits: thread (g, c) takes
// splits g, g + G, g + 2G, ... of the row for column c, issuing the loads of
// up to U splits (m, l and a float4 of o each) before merging any, and the G
// groups meet in LDS (the same rescaling as across splits).  The host picks G
// for the plan's largest split count so that a thread has at most four
// splits while G <= 4, else at most eight (G = 1 needs no LDS step at all);
// C is 256 / G columns, or the whole
// row when that is narrower, so a row of the few-KV shape (256 features, ~62
// splits) is two workgroups of 8 x 32.  Every load of a row is in flight at
// once: at decode sizes the merge is latency-bound.  The MLA layout has a
// kernel of its own (combine_codes_kernel, below).
#include "device.h"

namespace splitkv {

// One thread's share of a row's splits: splits g, g+G, g+2G, ... of the n,
// U loads in flight per pass, merged into the running (M2, lam, acc) in base 2.
// po points at the thread's float4 of the row in slot 0 and step is a slot's
// stride.
template <int U>
__device__ __forceinline__ void merge_splits(const float* part_m, const float* part_l, const float* po,
                                             int64_t step, int R, int rix, int base, int n, int g, int G,
                                             float& M2, float& lam, f32x4& acc) {
  for (int i0 = g; i0 < n; i0 += U * G) {
    float mi[U], li[U];
    f32x4 oi[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * G;
      const int64_t sl = base + (i < n ? i : i0);   // past the end: reread a valid slot, weight 0
      mi[u] = part_m[sl * R + rix];
      li[u] = part_l[sl * R + rix];
      oi[u] = *reinterpret_cast<const f32x4*>(po + sl * step);
      if (i >= n) mi[u] = -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (mi[u] == -INFINITY) continue;                  // empty split: zero weight
      const float m2 = mi[u] * kLog2e;
      const float Mn = fmaxf(M2, m2);
      const float a = fast_exp2(M2 - Mn);                 // 0 while M2 is -inf
      const float w = fast_exp2(m2 - Mn);
      lam = lam * a + w * li[u];
      acc = acc * a + w * oi[u];
      M2 = Mn;
    }
  }
}

// All argument dwords (workspace, plan, output and log-sum-exp pointers, the
// row geometry and flags) are preloaded into scalar registers at wave launch,
// so the two plan reads of the row's sequence are the first memory accesses,
// issued together, and the stores need no argument load.  part_l and part_o
// follow part_m in the workspace: part_l at SR floats (SR = total_slots *
// rows per sequence), part_o at the next 256-byte boundary after 2 * SR
// floats.  The merge runs in base 2 on the hardware exponential (every
// argument is <= 0: a difference from the running max).
// flags: d_v (bits 0-15) | skip rows of single-split sequences (bit 16) |
// fp32 output (bit 17) | uniform split count (bits 18-26; 0: read the plan).
// With a uniform count the row's plan is n = that count and base = b * n, so
// the partial loads are the first memory accesses.  The workgroup has C * G
// threads (C = blockDim.x / G float4 columns).
template <int G>
__global__ __launch_bounds__(256) void combine_kernel(const float* part_m, const int32_t* num_splits,
                                                      const int32_t* slot_offset, void* out,
                                                      float* lse, int32_t R, int32_t dsplit,
                                                      int32_t flags, int32_t SR) {
  __shared__ float red_m[256], red_l[256];
  __shared__ f32x4 red_o[256];

  const int tid = threadIdx.x;
  const int C = int(blockDim.x) / G;
  const int row = int(blockIdx.x) / dsplit;
  const int part = int(blockIdx.x) - row * dsplit;
  const int b = row / R;
  const int rix = row - b * R;
  const int un = (flags >> 18) & 0x1ff;
  int n, base;
  if (un > 0) {
    n = un;
    base = b * un;
  } else {
    n = ((cint32*)num_splits)[b];
    base = ((cint32*)slot_offset)[b];
    asm volatile("" :: "s"(n), "s"(base));   // both reads in flight before either is used
  }
  if ((flags & (1 << 16)) && n == 1) return;
  const int DV = flags & 0xffff;
  const int c = tid % C, g = tid / C;
  const float* part_l = part_m + SR;

  // running state in base 2: M2 = max of m_i * log2(e)
  float M2 = -INFINITY, lam = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int f0 = 4 * (C * part + c);                  // this thread's first feature
  const int64_t step = int64_t(R) * DV;
  const float* po = part_m + (int64_t(2) * SR * 4 + 255) / 256 * 64 + int64_t(rix) * DV + f0;
  // loads per thread and pass: just enough for the row's splits (uniform
  // across the workgroup), so no pass issues loads it only masks away
  const int per = (n + G - 1) / G;
  if (per <= 1)
    merge_splits<1>(part_m, part_l, po, step, R, rix, base, n, g, G, M2, lam, acc);
  else if (per <= 2)
    merge_splits<2>(part_m, part_l, po, step, R, rix, base, n, g, G, M2, lam, acc);
  else if (per <= 4)
    merge_splits<4>(part_m, part_l, po, step, R, rix, base, n, g, G, M2, lam, acc);
  else
    merge_splits<8>(part_m, part_l, po, step, R, rix, base, n, g, G, M2, lam, acc);
  if constexpr (G > 1) {
    red_m[tid] = M2;
    red_l[tid] = lam;
    red_o[tid] = acc;
    __syncthreads();
    if (g != 0) return;
    float Mt = M2;
#pragma unroll
    for (int k = 1; k < G; ++k) Mt = fmaxf(Mt, red_m[k * C + c]);
    float lt = 0.f;
    f32x4 ot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const float mk = red_m[k * C + c];
      const float w = mk == -INFINITY ? 0.f : fast_exp2(mk - Mt);
      lt += w * red_l[k * C + c];
      ot += w * red_o[k * C + c];
    }
    M2 = Mt;
    lam = lt;
    acc = ot;
  }
  const bool ok = M2 != -INFINITY && lam > 0.f;
  acc *= ok ? 1.f / lam : 0.f;
  const int64_t o = int64_t(row) * DV + f0;
  if (flags & (1 << 17)) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + o) = acc;
  } else {
    u32x2 pk = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + o) = pk;
  }
  if (lse && part == 0 && c == 0) lse[row] = ok ? (M2 + log2f(lam)) * kLn2 : -INFINITY;
}

// The MLA layout (512 features: int16 codes of o, a scale per 256-feature
// half): one workgroup of four waves per row.  Wave w merges splits w, w + 4,
// w + 8, ...; lane j keeps features 8 j .. 8 j + 7, whose codes are one
// 16-byte load per split (the wave reads a split's row of codes in one 1 KiB
// load); a split's m, l and two scales are the same for the whole wave (one
// address per load; as scalar loads they measured slower).  U splits' loads
// per wave are in flight before any is merged, U the fewest of 1, 2, 4, 6, 8
// and 12 that hold the wave's share of the row's splits (the 42 splits of a
// long context in one pass, one memory trip); the four waves meet in LDS,
// and wave 0 writes the row.
template <int U>
__device__ __forceinline__ void merge_code_splits(const float* part_m, const float* part_l, const float* part_s,
                                                  const int16_t* pq, int64_t R, int rix, int base, int n,
                                                  int w, int hf, float& M2, float& lam, float (&acc)[8]) {
  for (int i0 = w; i0 < n; i0 += 4 * U) {
    float mi[U], li[U], si[U], s2[U][2];
    u32x4 ci[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + 4 * u;
      const int64_t ix = int64_t(base + (i < n ? i : i0)) * R + rix;   // past the end: a valid slot, weight 0
      mi[u] = part_m[ix];
      li[u] = part_l[ix];
      const float s0 = part_s[2 * ix], s1 = part_s[2 * ix + 1];
      ci[u] = *reinterpret_cast<const u32x4*>(pq + ix * 512);
      s2[u][0] = s0;
      s2[u][1] = s1;
    }
    // every load of the pass is in flight before the first wait
#pragma unroll
    for (int u = 0; u < U; ++u) asm volatile("" :: "v"(mi[u]), "v"(li[u]), "v"(s2[u][0]), "v"(s2[u][1]));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      si[u] = hf ? s2[u][1] : s2[u][0];
      if (i0 + 4 * u >= n) mi[u] = -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (mi[u] == -INFINITY) continue;                  // empty split: zero weight
      const float m2 = mi[u] * kLog2e;
      const float Mn = fmaxf(M2, m2);
      const float a = fast_exp2(M2 - Mn);                 // 0 while M2 is -inf
      const float wt = fast_exp2(m2 - Mn);
      lam = lam * a + wt * li[u];
      const float ws = wt * si[u];
      const uint32_t c4[4] = {ci[u].x, ci[u].y, ci[u].z, ci[u].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] = acc[2 * k] * a + ws * float(int16_t(c4[k] & 0xffffu));
        acc[2 * k + 1] = acc[2 * k + 1] * a + ws * float(int16_t(c4[k] >> 16));
      }
      M2 = Mn;
    }
  }
}

__global__ __launch_bounds__(256) void combine_codes_kernel(const float* part_m, const int32_t* num_splits,
                                                            const int32_t* slot_offset, void* out, float* lse,
                                                            int32_t R, int32_t flags, int32_t SR) {
  __shared__ float red_ml[4][2];
  __shared__ f32x4 red_o[3][2][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int row = blockIdx.x;
  const int b = row / R;
  const int rix = row - b * R;
  const int un = (flags >> 18) & 0x1ff;
  int n, base;
  if (un > 0) {
    n = un;
    base = b * un;
  } else {
    n = ((cint32*)num_splits)[b];
    base = ((cint32*)slot_offset)[b];
    asm volatile("" :: "s"(n), "s"(base));   // both reads in flight before either is used
  }
  if ((flags & (1 << 16)) && n == 1) return;
  const float* part_l = part_m + SR;
  const float* part_s = part_m + 2 * int64_t(SR);
  const int16_t* pq = reinterpret_cast<const int16_t*>(reinterpret_cast<const char*>(part_m) +
                                                       (int64_t(16) * SR + 255) / 256 * 256) + 8 * lane;
  float M2 = -INFINITY, lam = 0.f;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  const int hf = lane >> 5;                            // features 8 lane .. +7 lie in half lane / 32
  // loads per wave and pass: just enough for the row's splits
  const int per = (n + 3) / 4;
  if (per <= 1)
    merge_code_splits<1>(part_m, part_l, part_s, pq, R, rix, base, n, w, hf, M2, lam, acc);
  else if (per <= 2)
    merge_code_splits<2>(part_m, part_l, part_s, pq, R, rix, base, n, w, hf, M2, lam, acc);
  else if (per <= 4)
    merge_code_splits<4>(part_m, part_l, part_s, pq, R, rix, base, n, w, hf, M2, lam, acc);
  else if (per <= 6)
    merge_code_splits<6>(part_m, part_l, part_s, pq, R, rix, base, n, w, hf, M2, lam, acc);
  else if (per <= 8)
    merge_code_splits<8>(part_m, part_l, part_s, pq, R, rix, base, n, w, hf, M2, lam, acc);
  else
    merge_code_splits<12>(part_m, part_l, part_s, pq, R, rix, base, n, w, hf, M2, lam, acc);
  if (w > 0) {
    if (lane == 0) {
      red_ml[w][0] = M2;
      red_ml[w][1] = lam;
    }
    red_o[w - 1][0][lane] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    red_o[w - 1][1][lane] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
  __syncthreads();
  if (w > 0) return;
  float Mt = M2;
#pragma unroll
  for (int k = 1; k < 4; ++k) Mt = fmaxf(Mt, red_ml[k][0]);
  const float a0 = M2 == -INFINITY ? 0.f : fast_exp2(M2 - Mt);
  float lt = lam * a0;
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] *= a0;
#pragma unroll
  for (int k = 1; k < 4; ++k) {
    const float mk = red_ml[k][0];
    const float wk = mk == -INFINITY ? 0.f : fast_exp2(mk - Mt);
    lt += wk * red_ml[k][1];
    const f32x4 lo = red_o[k - 1][0][lane], hi = red_o[k - 1][1][lane];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] += wk * lo[j];
      acc[4 + j] += wk * hi[j];
    }
  }
  const bool ok = Mt != -INFINITY && lt > 0.f;
  const float inv = ok ? 1.f / lt : 0.f;
  const int64_t o = int64_t(row) * 512 + 8 * lane;
  if (flags & (1 << 17)) {
    float* of = static_cast<float*>(out) + o;
    *reinterpret_cast<f32x4*>(of) = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *reinterpret_cast<f32x4*>(of + 4) = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  } else {
    const u32x4 pk = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                      pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + o) = pk;
  }
  if (lse && lane == 0) lse[row] = ok ? (Mt + log2f(lt)) * kLn2 : -INFINITY;
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  if (p.d_v % 4 != 0 || p.d_v > 0xffff || p.uniform_splits < 0 || p.uniform_splits > 0x1ff)
    return hipErrorInvalidValue;
  // splits per row the launch is sized for: the plan's largest count when
  // known, else the most any plan can hold
  const int nmax = p.uniform_splits > 0 ? p.uniform_splits
                                        : (p.max_seq_splits > 0 ? p.max_seq_splits : SPLITKV_MAX_SPLITS_LIMIT);
  // thread groups over the splits: up to four, until a thread has at most
  // four splits (short chains for small counts: measured 0.1-0.25 µs faster
  // per step at 8 and 13 splits), then up to sixteen, until it has at most
  // eight (more groups at ~60 splits measured no faster)
  int G = 1;
  while (G < 4 && (nmax + G - 1) / G > 4) G *= 2;
  while (G < 16 && (nmax + G - 1) / G > 8) G *= 2;
  const int cols = p.d_v / 4;                       // float4 columns of a row
  int C = 256 / G;
  while (C > cols) C /= 2;
  if (cols % C != 0) return hipErrorInvalidValue;   // d_v a multiple of 4 * C
  const int dsplit = cols / C;
  const int64_t wgs = int64_t(p.B) * p.R * dsplit;
  const int64_t SR = p.part_l - p.part_m;
  const bool codes = p.d_v == 512;                  // the MLA layout
  if (wgs > INT32_MAX || SR > INT32_MAX / 16 ||
      (!codes && p.part_o != p.part_m + (2 * SR * 4 + 255) / 256 * 64))
    return hipErrorInvalidValue;
  const int32_t flags0 = p.d_v | (p.skip_single ? 1 << 16 : 0) | (p.out_f32 ? 1 << 17 : 0) |
                         (p.uniform_splits << 18);
  if (codes) {
    const int64_t rows = int64_t(p.B) * p.R;
    if (rows > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(combine_codes_kernel, dim3(unsigned(rows)), dim3(256), 0, stream, p.part_m, p.num_splits,
                       p.slot_offset, p.out, p.lse, p.R, flags0, int32_t(SR));
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>(wgs)), block(unsigned(C * G));
#define SPLITKV_COMBINE(GG)                                                                            \
  hipLaunchKernelGGL((combine_kernel<GG>), grid, block, 0, stream, p.part_m, p.num_splits,             \
                     p.slot_offset, p.out, p.lse, p.R, dsplit, flags0, int32_t(SR))
  switch (G) {
    case 1: SPLITKV_COMBINE(1); break;
    case 2: SPLITKV_COMBINE(2); break;
    case 4: SPLITKV_COMBINE(4); break;
    case 8: SPLITKV_COMBINE(8); break;
    default: SPLITKV_COMBINE(16); break;
  }
#undef SPLITKV_COMBINE
  return hipGetLastError();
}

// Widen e4m3 codes with the exact conversion the FP8 partial kernel uses.
__global__ void e4m3_to_bf16_kernel(const uint8_t* in, uint16_t* out, int64_t n) {
  const int64_t i = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i + 3 < n) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(in + i);
    const u32x2 r = e4m3x4_to_bf16x4(w);
    out[i + 0] = uint16_t(r.x & 0xffff);
    out[i + 1] = uint16_t(r.x >> 16);
    out[i + 2] = uint16_t(r.y & 0xffff);
    out[i + 3] = uint16_t(r.y >> 16);
  } else {
    for (int64_t k = i; k < n; ++k) {
      const u32x2 r = e4m3x4_to_bf16x4(uint32_t(in[k]));
      out[k] = uint16_t(r.x & 0xffff);
    }
  }
}

hipError_t launch_e4m3_to_bf16(const uint8_t* in, uint16_t* out, int64_t n, hipStream_t stream) {
  const int64_t quads = (n + 3) / 4;
  const dim3 grid(unsigned((quads + 255) / 256)), block(256);
  hipLaunchKernelGGL(e4m3_to_bf16_kernel, grid, block, 0, stream, in, out, n);
  return hipGetLastError();
}

}  // namespace splitkv
