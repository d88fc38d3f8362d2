// Internal declarations shared by the library's host translation units.
#pragma once

#include <cstdarg>
#include <cstdint>

#include "splitkv.h"

namespace splitkv {

// Records a thread-local message for splitkv_last_error() and returns `code`.
splitkv_status fail(splitkv_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Number of 16-token granules of a sequence of L tokens.
inline int64_t num_granules(int64_t L) { return ceil_div(L, SPLITKV_GRANULE); }

// Split i of n over L tokens: [s, e).  Every range is non-empty when n <= ceil(L/16).
inline void split_range(int64_t L, int64_t n, int64_t i, int64_t* s, int64_t* e) {
  const int64_t nblk = num_granules(L);
  *s = SPLITKV_GRANULE * ((i * nblk) / n);
  const int64_t hi = SPLITKV_GRANULE * (((i + 1) * nblk) / n);
  *e = hi < L ? hi : L;
}

// Pure host planner (no device queries).
splitkv_status plan_host(const splitkv_plan_args& a, int32_t num_cus, const int32_t* seq_lens,
                         int32_t* num_splits, int32_t* slot_offset, int32_t* slot_info,
                         int32_t slot_info_capacity, int32_t* total_slots);

}  // namespace splitkv
