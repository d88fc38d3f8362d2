// Host-side split planner and the host entry points that touch no device.
//
// The count the caller asks for is the count the kernels use: the partition
// is computed from the runtime value only, never from a stored default (the
// defect analysed in "vLLM 0.30.0 FA4 SplitKV Bug: H100 Decode Can Be 48%
// Slower", section "The actual bug is one missing constructor argument").
// Auto mode weighs the gain of more splits against their cost -- every extra
// split adds merge work ("Shipped: 484.5 tok/s on one GB300 ...", section "Why
// 8 splits lost") and every extra workgroup a fixed start-up latency -- by
// estimating two candidate plans with a list-scheduling model of the compute
// units and keeping the faster one.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <functional>
#include <queue>
#include <string>
#include <vector>

#include "internal.h"

namespace splitkv {

static thread_local std::string g_last_error;

splitkv_status fail(splitkv_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

static int32_t clamp_request(int64_t L, int64_t n, int64_t max_splits) {
  int64_t cap = num_granules(L);
  if (cap < 1) cap = 1;
  if (cap > max_splits) cap = max_splits;
  if (n > cap) n = cap;
  if (n < 1) n = 1;
  return static_cast<int32_t>(n);
}

// floor(sqrt(x)) for x >= 0.
static int64_t isqrt64(int64_t x) {
  int64_t r = static_cast<int64_t>(std::sqrt(static_cast<double>(x)));
  while (r > 0 && r * r > x) --r;
  while ((r + 1) * (r + 1) <= x) ++r;
  return r;
}

// Finish time of the busiest compute unit when the plan's workgroups are
// handed out in launch order (slot by slot, the units of a slot one after
// another), each to the unit that becomes free first; a workgroup costs
// `overhead` plus its range length, in tokens.
static int64_t list_schedule(const int32_t* seq_lens, const std::vector<int32_t>& ns,
                             int64_t units, int32_t num_cus, int64_t overhead) {
  std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> free_at;
  for (int32_t c = 0; c < num_cus; ++c) free_at.push(0);
  int64_t busiest = 0;
  for (size_t b = 0; b < ns.size(); ++b)
    for (int32_t i = 0; i < ns[b]; ++i) {
      int64_t s, e;
      split_range(seq_lens[b], ns[b], i, &s, &e);
      for (int64_t u = 0; u < units; ++u) {
        const int64_t t = free_at.top() + overhead + (e - s);
        free_at.pop();
        free_at.push(t);
        busiest = std::max(busiest, t);
      }
    }
  return busiest;
}

// The partials a plan writes and the merge reads back, in tokens of
// streaming spread over every compute unit (a single split writes the output
// directly and has none).  A partial row is (d_v + 2) fp32 values, or for the
// MLA kernels 2 * d_v bytes of codes and four fp32 values (m, l, two scales).
static int64_t merge_tokens(const std::vector<int32_t>& ns, int64_t T, int64_t Hq, int64_t d_v,
                            bool mla, int32_t num_cus, int64_t tb) {
  int64_t slots = 0;
  for (int32_t n : ns)
    if (n > 1) slots += n;
  const int64_t row_bytes = mla ? 2 * d_v + 16 : (d_v + 2) * 4;
  return ceil_div(2 * slots * T * Hq * row_bytes, int64_t(num_cus) * tb);
}

// Auto split counts (the rule documented at splitkv_plan).
static void auto_splits(const splitkv_plan_args& a, int32_t num_cus, const int32_t* seq_lens,
                        int32_t* num_splits) {
  const bool mla = a.kernel == SPLITKV_KERNEL_MLA;
  const int64_t rows_per_wg = mla ? SPLITKV_ROWS_PER_WG_MLA : SPLITKV_ROWS_PER_WG_GQA;
  const int64_t units = int64_t(a.Hkv) * ceil_div(int64_t(a.Hq / a.Hkv) * a.T, rows_per_wg);
  const int64_t elem = a.kv_dtype == SPLITKV_KV_E4M3 ? 1 : 2;
  // MLA: the cost of a token is the matrix work on bf16 operands, whatever the cache dtype
  const int64_t tb = mla ? int64_t(a.d_qk) * 2 : (int64_t(a.d_qk) + a.d_v) * elem;
  int64_t lmax = 0, sum_len = 0;
  for (int32_t b = 0; b < a.B; ++b) {
    lmax = std::max<int64_t>(lmax, seq_lens[b]);
    sum_len += seq_lens[b];
  }
  std::fill(num_splits, num_splits + a.B, 1);
  if (lmax * tb < SPLITKV_AUTO_SPLIT_MIN_BYTES) return;
  const int64_t c_lat =
      std::max<int64_t>(SPLITKV_GRANULE, isqrt64(lmax * SPLITKV_AUTO_LAT_NUM / SPLITKV_AUTO_LAT_DEN));
  const int64_t work = sum_len > (INT64_MAX / 4) / units ? INT64_MAX / 4 : sum_len * units;
  const int64_t c_one = std::max(c_lat, ceil_div(work, int64_t(num_cus)));
  const int64_t c_bal = std::max(c_lat, ceil_div(work, int64_t(SPLITKV_AUTO_BALANCE) * num_cus));
  const int64_t c_43 = ceil_div(4 * c_one, 3);
  // candidates in tie-break order: one round, balanced, one round at 4/3 and at 2x the chunk
  std::vector<std::vector<int32_t>> cand(4, std::vector<int32_t>(a.B));
  for (int32_t b = 0; b < a.B; ++b) {
    const int64_t L = seq_lens[b];
    cand[0][b] = clamp_request(L, L / c_one, a.max_splits);
    cand[1][b] = clamp_request(L, ceil_div(L, c_bal), a.max_splits);
    cand[2][b] = clamp_request(L, L / c_43, a.max_splits);
    cand[3][b] = clamp_request(L, L / (2 * c_one), a.max_splits);
  }
  const int64_t overhead = ceil_div(int64_t(SPLITKV_AUTO_WG_OVERHEAD_BYTES), tb);
  size_t best = 0;
  int64_t best_score = INT64_MAX;
  for (size_t k = 0; k < cand.size(); ++k) {
    const int64_t score = list_schedule(seq_lens, cand[k], units, num_cus, overhead) +
                          merge_tokens(cand[k], a.T, a.Hq, a.d_v, mla, num_cus, tb);
    if (score < best_score) {
      best = k;
      best_score = score;
    }
  }
  std::copy(cand[best].begin(), cand[best].end(), num_splits);
}

splitkv_status plan_host(const splitkv_plan_args& a, int32_t num_cus, const int32_t* seq_lens,
                         int32_t* num_splits, int32_t* slot_offset, int32_t* slot_info,
                         int32_t slot_info_capacity, int32_t* total_slots) {
  if (!seq_lens || !num_splits || !slot_offset || !total_slots)
    return fail(SPLITKV_ERR_INVALID_ARG, "splitkv_plan: null output or seq_lens pointer");
  if (a.B < 1 || a.T < 1 || a.Hq < 1 || a.Hkv < 1 || a.Hq % a.Hkv != 0)
    return fail(SPLITKV_ERR_INVALID_ARG, "splitkv_plan: bad shape B=%d T=%d Hq=%d Hkv=%d", a.B,
                a.T, a.Hq, a.Hkv);
  if (a.max_splits < 1 || a.max_splits > SPLITKV_MAX_SPLITS_LIMIT)
    return fail(SPLITKV_ERR_INVALID_ARG, "splitkv_plan: max_splits=%d outside [1, %d]",
                a.max_splits, SPLITKV_MAX_SPLITS_LIMIT);
  if (a.requested_splits < 0)
    return fail(SPLITKV_ERR_INVALID_ARG, "splitkv_plan: requested_splits=%d < 0",
                a.requested_splits);
  if (a.kernel != SPLITKV_KERNEL_GQA && a.kernel != SPLITKV_KERNEL_MLA)
    return fail(SPLITKV_ERR_INVALID_ARG, "splitkv_plan: unknown kernel %d", a.kernel);
  if (num_cus < 1) return fail(SPLITKV_ERR_INVALID_ARG, "splitkv_plan: num_cus=%d", num_cus);
  if (a.d_qk < 1 || a.d_v < 1 || (a.kv_dtype != SPLITKV_KV_BF16 && a.kv_dtype != SPLITKV_KV_E4M3))
    return fail(SPLITKV_ERR_INVALID_ARG, "splitkv_plan: d_qk=%d d_v=%d kv_dtype=%d", a.d_qk, a.d_v,
                a.kv_dtype);
  for (int32_t b = 0; b < a.B; ++b)
    if (seq_lens[b] < 0)
      return fail(SPLITKV_ERR_INVALID_ARG, "splitkv_plan: seq_lens[%d]=%d < 0", b, seq_lens[b]);
  if (a.requested_splits == 0)
    auto_splits(a, num_cus, seq_lens, num_splits);
  else
    for (int32_t b = 0; b < a.B; ++b)
      num_splits[b] = clamp_request(seq_lens[b], a.requested_splits, a.max_splits);
  int64_t off = 0;
  slot_offset[0] = 0;
  for (int32_t b = 0; b < a.B; ++b) {
    off += num_splits[b];
    if (off > INT32_MAX) return fail(SPLITKV_ERR_INVALID_ARG, "splitkv_plan: too many slots");
    slot_offset[b + 1] = static_cast<int32_t>(off);
  }
  *total_slots = static_cast<int32_t>(off);
  if (slot_info) {
    if (off > slot_info_capacity)
      return fail(SPLITKV_ERR_INVALID_ARG,
                  "splitkv_plan: slot_info capacity %d < %lld slots", slot_info_capacity,
                  static_cast<long long>(off));
    for (int32_t b = 0; b < a.B; ++b)
      for (int32_t i = 0; i < num_splits[b]; ++i) {
        int64_t s, e;
        split_range(seq_lens[b], num_splits[b], i, &s, &e);
        int32_t* r = slot_info + 4 * int64_t(slot_offset[b] + i);
        r[0] = b;
        r[1] = (num_splits[b] << 16) | i;
        r[2] = static_cast<int32_t>(s);
        r[3] = static_cast<int32_t>(e);
      }
  }
  return SPLITKV_OK;
}

}  // namespace splitkv

using namespace splitkv;

extern "C" {

const char* splitkv_last_error(void) { return g_last_error.c_str(); }

splitkv_status splitkv_split_range(int32_t L, int32_t n, int32_t i, int32_t* s, int32_t* e) {
  if (!s || !e) return fail(SPLITKV_ERR_INVALID_ARG, "splitkv_split_range: null output");
  if (L < 0 || n < 1 || i < 0 || i >= n)
    return fail(SPLITKV_ERR_INVALID_ARG, "splitkv_split_range: L=%d n=%d i=%d", L, n, i);
  int64_t s64, e64;
  split_range(L, n, i, &s64, &e64);
  *s = static_cast<int32_t>(s64);
  *e = static_cast<int32_t>(e64);
  return SPLITKV_OK;
}

size_t splitkv_workspace_bytes(int32_t total_slots, int32_t T, int32_t Hq, int32_t d_v) {
  if (total_slots < 0 || T < 0 || Hq < 0 || d_v < 0) return 0;
  const size_t rows = size_t(total_slots) * size_t(T) * size_t(Hq);
  size_t ml = 2 * rows * sizeof(float);
  ml = (ml + 255) / 256 * 256;
  return ml + rows * size_t(d_v) * sizeof(float);
}

splitkv_status splitkv_validate_block_table(const int32_t* bt, const int32_t* seq_lens, int32_t B,
                                            int64_t bt_stride, int32_t page_size,
                                            int32_t num_pages) {
  if (!bt || !seq_lens || B < 0 || page_size < 1 || num_pages < 0)
    return fail(SPLITKV_ERR_INVALID_ARG, "splitkv_validate_block_table: bad arguments");
  for (int32_t b = 0; b < B; ++b) {
    if (seq_lens[b] < 0)
      return fail(SPLITKV_ERR_INVALID_ARG, "seq_lens[%d]=%d < 0", b, seq_lens[b]);
    const int64_t pages = ceil_div(seq_lens[b], page_size);
    if (pages > bt_stride)
      return fail(SPLITKV_ERR_INVALID_ARG,
                  "sequence %d needs %lld pages but the block-table row holds %lld", b,
                  static_cast<long long>(pages), static_cast<long long>(bt_stride));
    for (int64_t p = 0; p < pages; ++p) {
      const int32_t v = bt[b * bt_stride + p];
      if (v < 0 || v >= num_pages)
        return fail(SPLITKV_ERR_INVALID_ARG, "block_table[%d][%lld]=%d outside [0, %d)", b,
                    static_cast<long long>(p), v, num_pages);
    }
  }
  return SPLITKV_OK;
}

size_t splitkv_args_size(void) { return sizeof(splitkv_args); }
size_t splitkv_plan_args_size(void) { return sizeof(splitkv_plan_args); }

}  // extern "C"
