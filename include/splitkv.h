/*
 * splitkv.h -- C ABI of the MI355X (gfx950) split-KV decode-attention library.
 *
 * The operation: a few query tokens per sequence attend over a long, paged KV
 * cache.  Each sequence's KV range is cut into num_splits ranges; every range
 * yields a partial result (running max m, weight sum l, unnormalised output
 * o) and a log-sum-exp combine merges the partials into the exact softmax
 * output and its log-sum-exp.  Splitting exists to spread few-KV-head,
 * long-context decode over many compute units ("vLLM 0.30.0 FA4 SplitKV Bug:
 * H100 Decode Can Be 48% Slower", sections "What SplitKV is trying to do" and
 * "Gemma 4 exposes the failure clearly"); extra splits never change the
 * result, empty ones contribute zero weight (same page, "Why the result is
 * still correct").
 *
 * Conventions for every entry point:
 *   - Pointers marked (host) are host memory; every other pointer is device
 *     memory on the current HIP device.  The library never allocates device
 *     memory and keeps no per-call state: the caller owns every buffer,
 *     including the workspace (per-call buffer allocation inside attention
 *     backends was flagged as a memory hazard in "Xqa decode kernels",
 *     review comments).  The one exception is splitkv_decode_noalloc, whose
 *     partials live in a fixed module-scope device array that is loaded with
 *     the library, never allocated per call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Launches are asynchronous; device faults surface at the caller's next
 *     synchronisation.
 *   - Every call validates its arguments on the host and returns a status.
 *     Nothing asserts or aborts across the ABI; splitkv_last_error() returns
 *     a thread-local message for the last non-OK status.  Unsupported
 *     devices and shapes fail cleanly with SPLITKV_ERR_UNSUPPORTED (an
 *     unsupported-architecture path that crashed engine start-up is one of
 *     the failures recorded in "Xqa decode kernels", commit timeline).
 *   - Element strides are in elements of the tensor's own type; the last
 *     (feature) dimension is always contiguous.  Queries need not be
 *     contiguous otherwise ("Xqa decode kernels", timeline: a contiguity
 *     assertion on the query crashed Hopper and was relaxed).
 *
 * Shapes and layouts:
 *   q            bf16 [B][T][Hq][d_qk], strides q_stride_b/_t/_h.
 *   k_cache      [num_pages][Hkv][page_size][d_qk] via strides
 *                k_stride_page/_head/_tok (HND layout by default, any order
 *                of the three outer dimensions through the strides).
 *   v_cache      same with d_v; ignored for MLA, where V = K[..., :d_v].
 *   block_table  int32 [B][bt_stride]; entry p of row b is the physical page
 *                holding logical tokens [p*page_size, (p+1)*page_size).
 *                Entries past ceil(L_b / page_size) are never read.
 *   seq_lens     int32 [B]; L_b counts every cached token of sequence b,
 *                including its own T query tokens.  Query token t sits at
 *                position L_b - T + t and sees keys j <= L_b - T + t.
 *   head map     query head h reads KV head h / (Hq / Hkv).
 *   out          [B][T][Hq][d_v], bf16 or fp32 (out_dtype), contiguous.
 *   lse          fp32 [B][T][Hq] natural-log log-sum-exp of the scaled
 *                scores; may be NULL.
 *   workspace    the split partials; layout (S = total_slots, R = T*Hq):
 *                  part_m [S][R]   fp32 max of scale*q.k over the split
 *                                  (natural log units; -inf if the row sees
 *                                  nothing)
 *                  part_l [S][R]   fp32 sum of exp(s - m)
 *                  part_o [S][R][d_v]  fp32 sum of exp(s - m) * v (v
 *                                  dequantised), from the first 256-byte
 *                                  boundary after part_l
 *                For d_v = 512 (the MLA kernels) part_o is compact instead:
 *                  part_s [S][R][2]  fp32 scale of each 256-feature half of
 *                                  the row, right after part_l
 *                  part_q [S][R][512]  int16 codes from the first 256-byte
 *                                  boundary after part_s: o = code * scale
 *                                  of its half, the scale being the half's
 *                                  largest |o| / 32767 (codes within half a
 *                                  step of o, i.e. 2^-16 of that largest
 *                                  magnitude).
 *                splitkv_workspace_bytes() gives a size that holds either.
 *   debug        optional int32 [S][Hkv][row_blocks][8] records
 *                (b, i, hk, s, e, groups, xor_phys, sum_phys mod 2^31) over
 *                the 16-token groups of the split's range; row_blocks =
 *                ceil(g*T / rows_per_wg).  NULL disables it.
 */
#ifndef SPLITKV_H
#define SPLITKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t splitkv_status;
#define SPLITKV_OK 0
#define SPLITKV_ERR_INVALID_ARG (-1)   /* null pointer, bad size, inconsistent shape */
#define SPLITKV_ERR_UNSUPPORTED (-2)   /* device is not gfx950, or shape not built */
#define SPLITKV_ERR_WORKSPACE (-3)     /* workspace smaller than splitkv_workspace_bytes() */
#define SPLITKV_ERR_LAUNCH (-4)        /* a kernel launch returned an error */
#define SPLITKV_ERR_DEVICE (-5)        /* a HIP runtime query failed */

/* Split-range contract (see splitkv_plan). */
#define SPLITKV_GRANULE 16             /* tokens; split ranges start on multiples of it */
#define SPLITKV_AUTO_SPLIT_MIN_BYTES 196608  /* auto: no split unless a sequence has this many KV bytes per workgroup */
#define SPLITKV_AUTO_LAT_NUM 3                /* auto: latency floor isqrt(L_max * NUM / DEN) tokens per split */
#define SPLITKV_AUTO_LAT_DEN 2
#define SPLITKV_AUTO_BALANCE 4                /* auto: workgroups per compute unit of the balanced candidate */
#define SPLITKV_AUTO_WG_OVERHEAD_BYTES 32768  /* auto: fixed cost of one workgroup, in bytes of streaming */
#define SPLITKV_MAX_SPLITS_LIMIT 256   /* upper bound of max_splits */
#define SPLITKV_ROWS_PER_WG_GQA 16     /* query rows (g*T) one GQA workgroup covers */
#define SPLITKV_ROWS_PER_WG_MLA 128    /* query rows (T*Hq) one MLA workgroup covers */
#define SPLITKV_DEBUG_INTS 8
#define SPLITKV_NOALLOC_SCRATCH_BYTES 67108864  /* library-owned partials of splitkv_decode_noalloc, per device */
#define SPLITKV_SINGLE_LAUNCH_MAX_WORKGROUPS 64  /* splitkv_decode: one launch for grids up to this */

enum { SPLITKV_KV_BF16 = 0, SPLITKV_KV_E4M3 = 1 };
enum { SPLITKV_KERNEL_GQA = 0, SPLITKV_KERNEL_MLA = 1 };
enum { SPLITKV_OUT_BF16 = 0, SPLITKV_OUT_F32 = 1 };
enum { SPLITKV_Q_BF16 = 0, SPLITKV_Q_E4M3 = 1 };

typedef struct {
  int32_t B, T, Hq, Hkv;
  int32_t kernel;            /* SPLITKV_KERNEL_GQA or SPLITKV_KERNEL_MLA (rows per workgroup) */
  int32_t requested_splits;  /* > 0: honoured exactly when <= min(max_splits, nblk); 0: auto */
  int32_t max_splits;        /* 1 .. SPLITKV_MAX_SPLITS_LIMIT */
  int32_t num_cus;           /* > 0: compute units to plan for; 0: query the current device */
  int32_t d_qk, d_v;         /* head dimensions (auto mode sizes splits in bytes) */
  int32_t kv_dtype;          /* SPLITKV_KV_BF16 or SPLITKV_KV_E4M3 */
} splitkv_plan_args;

/*
 * splitkv_plan -- host-only split planner.
 *
 * The runtime count decides the ranges: a request n > 0 yields exactly
 * min(n, max_splits, nblk) non-empty splits, nblk = ceil(L / 16) (the
 * regression in "vLLM 0.30.0 FA4 SplitKV Bug ...", section "The actual bug is
 * one missing constructor argument", read a stored count of one and gave
 * every other split an empty range).
 *
 * n == 0 sizes splits for the machine, weighing the merge, which has a cost
 * that can eat the gain of more splits ("Shipped: 484.5 tok/s on one GB300
 * ...", section "Why 8 splits lost").  With cap_b = min(max_splits,
 * max(nblk_b, 1)), units = Hkv * ceil(g*T / rows_per_wg) workgroups per split,
 * tb = bytes one workgroup streams per token ((d_qk + d_v) * elem for GQA,
 * elem = 2 for bf16, 1 for e4m3; d_qk * 2 for MLA whatever the cache dtype:
 * V is the first d_v features of the same row, and a token costs the matrix
 * work on bf16 operands) and L_max the longest sequence:
 *   1. if L_max * tb < SPLITKV_AUTO_SPLIT_MIN_BYTES no sequence is split
 *      (the merge launch would cost more than it saves);
 *   2. c_lat = max(16, isqrt(L_max * SPLITKV_AUTO_LAT_NUM / SPLITKV_AUTO_LAT_DEN)),
 *      the tokens per split below which the merge of more partials costs
 *      more than the shorter split saves;  W = units * sum_b L_b;
 *   3. candidate A, one round: c1 = max(c_lat, ceil(W / num_cus)),
 *      n_b = clamp(floor(L_b / c1), 1, cap_b) -- at most one workgroup per
 *      compute unit when the batch allows it;
 *      candidate B, balanced: c = max(c_lat, ceil(W / (SPLITKV_AUTO_BALANCE *
 *      num_cus))), n_b = clamp(ceil(L_b / c), 1, cap_b) -- no workgroup
 *      longer than c, for batches of unequal lengths;
 *      candidates C and D, fewer splits: as A with c = ceil(4 * c1 / 3) and
 *      with c = 2 * c1;
 *   4. each candidate's step is estimated by list scheduling its workgroups,
 *      in launch order (slot by slot, the units of a slot consecutively),
 *      onto num_cus identical compute units, a workgroup costing
 *      ceil(SPLITKV_AUTO_WG_OVERHEAD_BYTES / tb) + (end - start) tokens, plus
 *      the merge: ceil(Pb / (num_cus * tb)) tokens, Pb = 2 * sum over the
 *      sequences with n_b > 1 of n_b * T * Hq * row_bytes, the partials
 *      written and read back, spread over every compute unit, row_bytes =
 *      (d_v + 2) * 4, or 2 * d_v + 16 for MLA (the compact layout of the
 *      workspace); the lowest estimate wins, the earlier of A, B, C, D on a
 *      tie.
 *
 * Split i of n covers [16*floor(i*nblk/n), min(L, 16*floor((i+1)*nblk/n))).
 * L == 0 gives one empty split.
 *
 * Outputs (all host): num_splits[B]; slot_offset[B+1] (exclusive prefix
 * sum); slot_info[S][4], the work record of slot s = slot_offset[b] + i:
 *   { b, (num_splits[b] << 16) | i, start, end }
 * so a workgroup learns its sequence, split and token range [start, end)
 * with one load.  slot_info is written only if slot_info_host is not NULL and
 * S <= slot_info_capacity (in slots; else SPLITKV_ERR_INVALID_ARG);
 * *total_slots = S.  B * max_splits always bounds S.
 */
splitkv_status splitkv_plan(const splitkv_plan_args* args, const int32_t* seq_lens_host,
                            int32_t* num_splits_host, int32_t* slot_offset_host,
                            int32_t* slot_info_host, int32_t slot_info_capacity,
                            int32_t* total_slots);

/* Token range [*s, *e) of split i of n for a sequence of L tokens (host; same formula as the kernels). */
splitkv_status splitkv_split_range(int32_t L, int32_t n, int32_t i, int32_t* s, int32_t* e);

/* Bytes of fp32 workspace the partials of S slots need. */
size_t splitkv_workspace_bytes(int32_t total_slots, int32_t T, int32_t Hq, int32_t d_v);

/* Arguments of the decode entry points. */
typedef struct {
  const void* q;                   /* bf16 */
  int64_t q_stride_b, q_stride_t, q_stride_h;
  const void* k_cache;             /* bf16 or e4m3 codes */
  const void* v_cache;             /* same dtype; ignored (may be NULL) for MLA */
  int64_t k_stride_page, k_stride_head, k_stride_tok;
  int64_t v_stride_page, v_stride_head, v_stride_tok;
  const int32_t* block_table;
  int64_t bt_stride;
  const int32_t* seq_lens;         /* [B] */
  const int32_t* num_splits;       /* [B]   from splitkv_plan, on the device */
  const int32_t* slot_offset;      /* [B+1] */
  const int32_t* slot_info;        /* [S][4] */
  int32_t total_slots;             /* S, the host value splitkv_plan returned */
  int32_t B, T, Hq, Hkv, d_qk, d_v, page_size, num_pages;
  int32_t kv_dtype;                /* SPLITKV_KV_BF16 or SPLITKV_KV_E4M3 */
  float scale;                     /* softmax scale applied to q.k */
  float k_scale, v_scale;          /* dequant scales of an e4m3 cache (1 for bf16) */
  float* workspace;
  size_t workspace_bytes;
  void* out;
  int32_t out_dtype;               /* SPLITKV_OUT_BF16 or SPLITKV_OUT_F32 */
  float* lse;                      /* may be NULL */
  int32_t* debug;                  /* may be NULL */
  int32_t uniform_splits;          /* > 0: every sequence has exactly this many splits (then
                                      slot_offset[b] = b * uniform_splits and total_slots =
                                      B * uniform_splits, checked); the merge then takes its plan
                                      from this value instead of reading num_splits/slot_offset.
                                      0: no such promise */
  int32_t q_dtype;                 /* SPLITKV_Q_BF16 (0: q used as given) or SPLITKV_Q_E4M3 (MLA
                                      over an e4m3 cache only: q quantised to e4m3 codes of
                                      q / q_scale inside the kernel) */
  float q_scale;                   /* per-tensor query scale for SPLITKV_Q_E4M3 (ignored for bf16) */
  int32_t max_seq_splits;          /* > 0: the largest num_splits[b] of the plan, which sizes the
                                      merge's launch (a smaller value than the truth is slower,
                                      never wrong); 0: not given */
  int32_t max_range_tokens;        /* > 0: no split range of the plan holds more tokens (a hint:
                                      MLA steps whose ranges are all short and whose 64-row
                                      workgroups fit on the compute units at once run the
                                      short-range kernel, which is correct for ranges of any
                                      length, so a wrong hint is slower, never wrong); 0: not
                                      given */
  int32_t* tickets;                /* splitkv_decode_single_launch only: int32 [B][Hkv][row_blocks]
                                      arrival counters (row_blocks = ceil(g*T / 16)), all zero
                                      before the first call; every completed call leaves them
                                      zero.  Ignored (may be NULL) elsewhere */
} splitkv_args;

/*
 * splitkv_decode_partial -- GQA partial kernel over a bf16 cache.
 * One workgroup per (slot, KV head, block of 16 query rows) writes the
 * partial (m, l, o) of its split ("vLLM 0.30.0 FA4 SplitKV Bug ...", section
 * "What SplitKV is trying to do": each split computes a partial attention
 * result).  Requires kv_dtype == BF16, d_qk == d_v in {64, 128, 256},
 * page_size % 16 == 0, 16-byte aligned q / caches / strides.
 */
splitkv_status splitkv_decode_partial(const splitkv_args* args, void* stream);

/*
 * splitkv_decode_partial_fp8 -- the same over an e4m3 cache with bf16
 * queries ("Xqa decode kernels", section "Purpose": BF16/FP16 queries with an
 * FP8 KV cache).  Codes widen exactly to bf16; k_scale multiplies the scores,
 * v_scale the output.  The query is never quantised and takes no scale of its
 * own (same page, timeline: no q_scale for model-dtype queries over an FP8
 * cache).  Requires kv_dtype == E4M3, d_qk == d_v in {64, 128, 256}.
 */
splitkv_status splitkv_decode_partial_fp8(const splitkv_args* args, void* stream);

/*
 * splitkv_mla_decode_partial -- MLA partial kernel: one latent KV head
 * (Hkv == 1) of width d_qk == 576 serves as key, its first d_v == 512
 * columns as value; one workgroup per (slot, block of 128 query rows in
 * (t, h) order, SPLITKV_ROWS_PER_WG_MLA).  Causal within the T query tokens ("Shipped: 484.5 tok/s on
 * one GB300 ...", table "What shipped": split-KV MLA decode of one request
 * at six tokens).  The latent cache is bf16 or e4m3 (kv_dtype); e4m3 codes
 * widen exactly to bf16 and k_scale / v_scale (the same value for a latent
 * cache whose values are its keys' first columns) scale the scores and the
 * output; the query stays bf16 ("Xqa decode kernels", section "Purpose":
 * bf16 queries over an FP8 KV cache).
 *
 * With q_dtype == SPLITKV_Q_E4M3 (e4m3 cache only) the queries go FP8 as well
 * ("Xqa decode kernels", timeline: FP8-Q, used only where the cache is FP8):
 * each bf16 query value is quantised to the e4m3 code of q / q_scale (the
 * correctly rounded fp32 quotient, saturated to +-448, nearest code, ties to
 * even -- the encoding of splitkv_append_kv) and the scores run on the FP8
 * matrix path over the codes; P V runs on bf16 operands as in the other
 * modes.  The result approximates attention over the dequantised queries,
 * keys and values.  q_scale must be positive and finite.
 */
splitkv_status splitkv_mla_decode_partial(const splitkv_args* args, void* stream);

/*
 * splitkv_mla_short_range -- 1 if an MLA step with these arguments runs the
 * short-range partial kernel (64 query rows and eight waves a workgroup:
 * chosen when args->max_range_tokens is 1 .. 256 and the plan's 64-row
 * workgroups, total_slots * ceil(T*Hq / 64), fit on the device's compute
 * units at once, or forced by SPLITKV_MLA_KERNEL=short in the environment),
 * 0 if it runs the 128-row kernel (also for a null args).  Host only; the
 * device is the current one.
 */
int32_t splitkv_mla_short_range(const splitkv_args* args);

/*
 * splitkv_combine -- log-sum-exp merge of the partials of every sequence into
 * out and lse: M = max_i m_i, w_i = exp(m_i - M) (0 for an empty split),
 * out = sum_i w_i o_i / sum_i w_i l_i, lse = M + ln(sum_i w_i l_i); a row
 * with no visible key gives out = 0, lse = -inf ("vLLM 0.30.0 FA4 SplitKV
 * Bug ...", section "Why the result is still correct": empty splits
 * contribute zero weight).
 */
splitkv_status splitkv_combine(const splitkv_args* args, void* stream);

/*
 * splitkv_decode -- the whole decode step: the partial kernel that kv_dtype
 * and `kernel` select, then the combine.  Sequences with a single split
 * write out/lse directly from the partial kernel and are skipped by the
 * combine; when every sequence has one split the combine is not launched.
 * `kernel` is SPLITKV_KERNEL_GQA or SPLITKV_KERNEL_MLA.  A grouped-query step
 * whose args carry tickets runs as one launch (see
 * splitkv_decode_single_launch) when 1 < max_seq_splits <= 8, a row block's
 * min(16, g*T) rows hold at most 256 float4 columns (rows x d_v / 4), and
 * the partial kernel's grid has at most SPLITKV_SINGLE_LAUNCH_MAX_WORKGROUPS
 * workgroups: there the last arriver merges in one round of loads and the
 * step measured faster than two kernels.
 */
splitkv_status splitkv_decode(const splitkv_args* args, int32_t kernel, void* stream);

/*
 * splitkv_decode_single_launch -- the whole grouped-query decode step in one
 * kernel: the workgroups of one (sequence, KV head, row block) take a ticket
 * in args->tickets when their partial is stored, and the last to arrive
 * merges the sequence's partials into out/lse (the same log-sum-exp merge as
 * splitkv_combine), so the merge costs no second launch ("Shipped: 484.5
 * tok/s on one GB300 ...", section "Why 8 splits lost": the merge can eat the
 * gain of more splits).  The partials still go through args->workspace.
 * `kernel` must be SPLITKV_KERNEL_GQA (else SPLITKV_ERR_UNSUPPORTED); the
 * tickets array must be given when any sequence has several splits.  Calls
 * that share a tickets array must not overlap.
 */
splitkv_status splitkv_decode_single_launch(const splitkv_args* args, int32_t kernel, void* stream);

/*
 * splitkv_decode_noalloc -- splitkv_decode for callers that cannot allocate
 * device memory or hand in a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  The same kernels run; the
 * partials go to a buffer the library owns (SPLITKV_NOALLOC_SCRATCH_BYTES =
 * 64 MiB, one copy per device, held until the process ends) instead of
 * args->workspace, which is ignored together with args->workspace_bytes.
 * A plan whose partials need more (splitkv_workspace_bytes(total_slots, T,
 * Hq, d_v) > SPLITKV_NOALLOC_SCRATCH_BYTES) fails with SPLITKV_ERR_WORKSPACE
 * before anything is launched.  Nothing in the buffer has to start at zero:
 * every partial the combine reads is written by the partial kernel of the
 * same call.  Every call on one device shares that device's buffer, so calls
 * that overlap on one device (streams without an ordering between them)
 * race; calls ordered on one stream do not.  The call itself allocates
 * nothing (no hipMalloc, no allocating library routine).
 */
splitkv_status splitkv_decode_noalloc(const splitkv_args* args, int32_t kernel, void* stream);

/* Arguments of splitkv_append_kv. */
typedef struct {
  const void* k_new;               /* bf16 [B][T][Hkv][d_k], strides k_new_stride_b/_t/_h */
  const void* v_new;               /* bf16 [B][T][Hkv][d_v]; NULL exactly when v_cache is NULL */
  int64_t k_new_stride_b, k_new_stride_t, k_new_stride_h;
  int64_t v_new_stride_b, v_new_stride_t, v_new_stride_h;
  void* k_cache;                   /* bf16 or e4m3 codes, [num_pages][Hkv][page_size][d_k] via strides */
  void* v_cache;                   /* same dtype with d_v; NULL for a latent cache (MLA: V = K[..., :d_v]) */
  int64_t k_stride_page, k_stride_head, k_stride_tok;
  int64_t v_stride_page, v_stride_head, v_stride_tok;
  const int32_t* block_table;      /* [B][bt_stride] */
  int64_t bt_stride;
  const int32_t* positions;        /* [B] logical position of sequence b's first new token */
  int32_t B, T, Hkv, d_k, d_v, page_size, num_pages;
  int32_t kv_dtype;                /* SPLITKV_KV_BF16 or SPLITKV_KV_E4M3 */
  float k_scale, v_scale;          /* e4m3 cache: the per-tensor scales the decode reads it with */
} splitkv_append_args;

/*
 * splitkv_append_kv -- the step before decode: new token t of sequence b is
 * written to logical position positions[b] + t, i.e. to page
 * block_table[b][pos / page_size], slot pos % page_size, for every KV head.
 * A bf16 cache stores the bf16 codes unchanged.  An e4m3 cache, which the
 * decode reads as code x scale ("Xqa decode kernels", section "Purpose":
 * bf16 queries over an FP8 KV cache; "Test Plan": the fp8 cache dtype),
 * stores the inverse: the e4m3 code nearest to x / scale (an fp32
 * division), saturated to +-448, ties to the even code; NaN stays NaN.
 * Device data is not trusted: a token whose position is negative or past
 * the block-table row (bt_stride entries), or whose page is outside
 * [0, num_pages), is skipped and nothing of it is written.  Requires d_k and
 * d_v multiples of 8, 16-byte aligned new rows and caches (bases and
 * strides).  Rows of one call must not overlap (two new tokens mapped to the
 * same slot race).
 */
splitkv_status splitkv_append_kv(const splitkv_append_args* args, void* stream);

/*
 * splitkv_validate_block_table -- host-side check that every block-table
 * entry a sequence reads (the first ceil(L_b / page_size)) lies in
 * [0, num_pages).  All pointers are host memory.
 */
splitkv_status splitkv_validate_block_table(const int32_t* block_table_host,
                                            const int32_t* seq_lens_host, int32_t B,
                                            int64_t bt_stride, int32_t page_size,
                                            int32_t num_pages);

/*
 * splitkv_e4m3_to_bf16 -- widen n e4m3 codes to bf16 codes on the device with
 * the conversion the FP8 kernels use (exposed so that tests can check every
 * code).
 */
splitkv_status splitkv_e4m3_to_bf16(const uint8_t* in, uint16_t* out, int64_t n, void* stream);

/*
 * Measurement helpers (the benchmark's floors).  What a decode kernel reaches
 * is judged against what a plain read-only kernel of the same grid reaches
 * and against the cost of a kernel that does nothing ("vLLM 0.30.0 FA4 SplitKV
 * Bug ...", section "The kernel profile isolates one operation": the same
 * grid, thread count and shared memory separate launch and occupancy effects
 * from useful work).
 *
 * splitkv_calib_empty -- launch one empty kernel (one wave) on `stream`.
 *
 * splitkv_calib_stream_read -- read `bytes` (a multiple of 16) of device
 * memory at `src` (16-byte aligned) with `workgroups` workgroups of 256
 * threads, each reading one contiguous share with 16-byte loads, thirty-two
 * in flight per thread (non-temporal loads when `workgroups` is at least the
 * device's compute-unit count, as the grouped-query kernel chooses them);
 * workgroup w stores the XOR of what it read to sink[w]
 * (`sink` holds `workgroups` uint32 values).  Bad arguments give
 * SPLITKV_ERR_INVALID_ARG.
 *
 * The compute-bound kernels (MLA) are judged against what their two inner
 * resources deliver on this GPU, measured the same way:
 *
 * splitkv_calib_mfma -- `workgroups` workgroups of four waves; every wave
 * runs `iters` (1 .. 2^24) rounds of four independent
 * v_mfma_f32_32x32x16_bf16 chains on register operands (131,072 FLOPs a
 * round).  Wave w of workgroup g writes sink[2 (4 g + w)] (a checksum of its
 * results) and sink[2 (4 g + w) + 1] (the core-clock cycles of its loop, from
 * s_memtime); `sink` holds 8 * workgroups uint32 values.
 *
 * splitkv_calib_lds_read -- `workgroups` workgroups of four waves, each
 * filling 64 KiB of LDS; every wave then runs `iters` (1 .. 2^24) rounds of
 * sixteen conflict-free reads of 1 KiB a wave -- `mode` 0: ds_read_b128 (16
 * bytes a lane), 1: ds_read_b64_tr_b16 (8 bytes a lane, 512 bytes a wave).
 * sink as for splitkv_calib_mfma (a checksum, then the read loop's cycles).
 *
 * Both give SPLITKV_ERR_INVALID_ARG for a null or misaligned sink or counts
 * out of range; the caller owns `sink` (device memory).
 */
splitkv_status splitkv_calib_empty(void* stream);
splitkv_status splitkv_calib_stream_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink,
                                         void* stream);
splitkv_status splitkv_calib_mfma(int32_t workgroups, int32_t iters, uint32_t* sink, void* stream);
splitkv_status splitkv_calib_lds_read(int32_t workgroups, int32_t iters, int32_t mode, uint32_t* sink,
                                      void* stream);

const char* splitkv_last_error(void);   /* thread-local message of the last failure */
const char* splitkv_version(void);      /* source revision the library was built from */
size_t splitkv_args_size(void);         /* sizeof(splitkv_args), for binding checks */
size_t splitkv_plan_args_size(void);    /* sizeof(splitkv_plan_args) */
size_t splitkv_append_args_size(void);  /* sizeof(splitkv_append_args) */

#ifdef __cplusplus
}
#endif
#endif /* SPLITKV_H */
