// Host-side split planner and the host entry points that touch no device.
//
// The count the caller asks for is the count the kernels use: the partition
// is computed from the runtime value only, never from a stored default (the
// defect analysed in "vLLM 0.30.0 FA4 SplitKV Bug: H100 Decode Can Be 48%
// Slower", section "The actual bug is one missing constructor argument").
// Auto mode aims at SPLITKV_AUTO_WG_PER_CU workgroups per compute unit with a
// floor of SPLITKV_AUTO_MIN_TOKENS tokens per split, since every extra split
// adds merge work ("Shipped: 484.5 tok/s on one GB300 ...", section "Why 8
// splits lost").
#include <cstdio>
#include <cstring>
#include <string>

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
  int64_t sum_len = 0;
  for (int32_t b = 0; b < a.B; ++b) {
    if (seq_lens[b] < 0)
      return fail(SPLITKV_ERR_INVALID_ARG, "splitkv_plan: seq_lens[%d]=%d < 0", b, seq_lens[b]);
    sum_len += seq_lens[b];
  }
  int64_t chunk = 0;
  if (a.requested_splits == 0) {
    const int64_t rows_per_wg =
        a.kernel == SPLITKV_KERNEL_MLA ? SPLITKV_ROWS_PER_WG_MLA : SPLITKV_ROWS_PER_WG_GQA;
    const int64_t g = a.Hq / a.Hkv;
    const int64_t units = int64_t(a.Hkv) * ceil_div(g * a.T, rows_per_wg);
    // an MLA workgroup fills a compute unit; grouped-query workgroups fit two
    const int64_t per_cu =
        a.kernel == SPLITKV_KERNEL_MLA ? SPLITKV_AUTO_WG_PER_CU_MLA : SPLITKV_AUTO_WG_PER_CU;
    const int64_t target = per_cu * num_cus;
    chunk = ceil_div(sum_len * units, target);
    if (chunk < SPLITKV_AUTO_MIN_TOKENS) chunk = SPLITKV_AUTO_MIN_TOKENS;
  }
  int64_t off = 0;
  slot_offset[0] = 0;
  for (int32_t b = 0; b < a.B; ++b) {
    const int64_t L = seq_lens[b];
    // auto: floor, so the plan never asks for more than the target workgroups
    const int64_t want = a.requested_splits > 0 ? a.requested_splits : L / chunk;
    num_splits[b] = clamp_request(L, want, a.max_splits);
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
