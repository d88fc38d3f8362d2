// C ABI of the split-KV decode library: argument checks, the gfx950 gate and
// dispatch to the kernels.  Every entry point returns a status and records a
// message instead of asserting; the library allocates nothing.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "device.h"
#include "internal.h"

#ifndef SPLITKV_REVISION
#define SPLITKV_REVISION "unknown"
#endif

namespace splitkv {

hipError_t launch_gqa_partial(const PartialParams& p, int D, bool fp8, bool fused, hipStream_t stream);
hipError_t launch_mla_partial(const PartialParams& p, int kind, hipStream_t stream);
hipError_t launch_mla_short_partial(const PartialParams& p, bool fp8, hipStream_t stream);
hipError_t launch_mla_short_q8_partial(const PartialParams& p, hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);
hipError_t launch_e4m3_to_bf16(const uint8_t* in, uint16_t* out, int64_t n, hipStream_t stream);

hipError_t launch_append(const AppendParams& p, int rows, int kinds, hipStream_t stream);

namespace {

struct DeviceInfo {
  bool checked = false;
  bool gfx950 = false;
  int cus = 0;
  char arch[64] = {0};
};

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
DeviceInfo g_dev[kMaxDevices];

// The kernels are written for gfx950 only; anything else is refused cleanly.
splitkv_status check_device(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(SPLITKV_ERR_DEVICE, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.checked) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(SPLITKV_ERR_DEVICE, "hipGetDeviceProperties(%d) failed", dev);
    strncpy(d.arch, prop.gcnArchName, sizeof(d.arch) - 1);
    d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.checked = true;
  }
  if (!d.gfx950)
    return fail(SPLITKV_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950 only",
                dev, d.arch);
  if (cus) *cus = d.cus;
  return SPLITKV_OK;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

enum class Kind { GqaBf16, GqaFp8, Mla };

struct Layout {
  float* m;
  float* l;
  float* o;       // fp32 o (d_v < 512)
  float* s;       // d_v = 512: two scales per row
  int16_t* q;     // d_v = 512: int16 codes of o
};

// The partials' layout in the workspace (documented in splitkv.h): m, l,
// then fp32 o at the next 256-byte boundary; for d_v = 512 (the MLA kernel)
// m, l, two scales per row, then int16 codes at the next 256-byte boundary
// (smaller than the fp32 layout that splitkv_workspace_bytes sizes).
Layout workspace_layout(const splitkv_args& a) {
  const size_t rows = size_t(a.total_slots) * size_t(a.T) * size_t(a.Hq);
  Layout w = {nullptr, nullptr, nullptr, nullptr, nullptr};
  if (!a.workspace) return w;
  char* base = reinterpret_cast<char*>(a.workspace);
  w.m = a.workspace;
  w.l = a.workspace + rows;
  if (a.d_v == 512) {
    w.s = a.workspace + 2 * rows;
    w.q = reinterpret_cast<int16_t*>(base + (4 * rows * sizeof(float) + 255) / 256 * 256);
  } else {
    w.o = reinterpret_cast<float*>(base + (2 * rows * sizeof(float) + 255) / 256 * 256);
  }
  return w;
}

splitkv_status check_common(const splitkv_args* a, const char* fn) {
  if (!a) return fail(SPLITKV_ERR_INVALID_ARG, "%s: null args", fn);
  if (!a->seq_lens || !a->num_splits || !a->slot_offset)
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: null plan pointer", fn);
  if (a->B < 1 || a->T < 1 || a->Hq < 1 || a->Hkv < 1 || a->Hq % a->Hkv != 0)
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: bad shape B=%d T=%d Hq=%d Hkv=%d", fn, a->B, a->T,
                a->Hq, a->Hkv);
  if (a->total_slots < a->B)
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: total_slots=%d < B=%d", fn, a->total_slots, a->B);
  if (a->out_dtype != SPLITKV_OUT_BF16 && a->out_dtype != SPLITKV_OUT_F32)
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: out_dtype=%d", fn, a->out_dtype);
  if (a->lse && !aligned(a->lse, 4)) return fail(SPLITKV_ERR_INVALID_ARG, "%s: lse misaligned", fn);
  return SPLITKV_OK;
}

splitkv_status check_partial(const splitkv_args* a, Kind kind, bool need_ws, const char* fn,
                             int* row_blocks) {
  splitkv_status st = check_common(a, fn);
  if (st != SPLITKV_OK) return st;
  if (!a->q || !a->k_cache || !a->block_table || !a->slot_info)
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: null q, k_cache, block_table or slot_info", fn);
  if (!aligned(a->slot_info, 16)) return fail(SPLITKV_ERR_INVALID_ARG, "%s: slot_info misaligned", fn);
  if (kind != Kind::Mla && !a->v_cache) return fail(SPLITKV_ERR_INVALID_ARG, "%s: null v_cache", fn);
  if (a->page_size < 16 || a->page_size % SPLITKV_GRANULE != 0)
    return fail(SPLITKV_ERR_UNSUPPORTED, "%s: page_size=%d must be a positive multiple of 16", fn,
                a->page_size);
  if (a->num_pages < 1) return fail(SPLITKV_ERR_INVALID_ARG, "%s: num_pages=%d", fn, a->num_pages);
  if (a->bt_stride < 1) return fail(SPLITKV_ERR_INVALID_ARG, "%s: bt_stride < 1", fn);
  const int want_kv = kind == Kind::GqaFp8 ? SPLITKV_KV_E4M3 : SPLITKV_KV_BF16;
  // the MLA kernel reads a bf16 or an e4m3 latent cache
  if (a->kv_dtype != want_kv && !(kind == Kind::Mla && a->kv_dtype == SPLITKV_KV_E4M3))
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: kv_dtype=%d, this entry point takes %d", fn,
                a->kv_dtype, want_kv);
  if (kind == Kind::Mla) {
    if (a->Hkv != 1 || a->d_qk != 576 || a->d_v != 512)
      return fail(SPLITKV_ERR_UNSUPPORTED, "%s: MLA needs Hkv=1, d_qk=576, d_v=512 (got %d, %d, %d)",
                  fn, a->Hkv, a->d_qk, a->d_v);
    if ((a->page_size & (a->page_size - 1)) != 0)
      return fail(SPLITKV_ERR_UNSUPPORTED, "%s: MLA needs a power-of-two page size (got %d)", fn,
                  a->page_size);
    if (a->k_stride_page * 2 > INT32_MAX || a->k_stride_tok * 2 > INT32_MAX)
      return fail(SPLITKV_ERR_UNSUPPORTED, "%s: MLA cache strides must fit 31 bits", fn);
  } else if (a->d_qk != a->d_v || (a->d_qk != 64 && a->d_qk != 128 && a->d_qk != 256)) {
    return fail(SPLITKV_ERR_UNSUPPORTED, "%s: head dims d_qk=%d d_v=%d; built for 64, 128 and 256", fn,
                a->d_qk, a->d_v);
  }
  if (!(a->scale > 0.f) || !(a->k_scale > 0.f) || !(a->v_scale > 0.f))
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: scales must be positive", fn);
  if (a->q_dtype != SPLITKV_Q_BF16 && a->q_dtype != SPLITKV_Q_E4M3)
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: q_dtype=%d", fn, a->q_dtype);
  if (a->q_dtype == SPLITKV_Q_E4M3) {
    // e4m3 queries run only where the cache is e4m3 too, on the MLA kernel
    if (kind != Kind::Mla || a->kv_dtype != SPLITKV_KV_E4M3)
      return fail(SPLITKV_ERR_UNSUPPORTED, "%s: e4m3 queries need the MLA kernel over an e4m3 cache", fn);
    if (!(a->q_scale > 0.f) || !(a->q_scale < INFINITY))
      return fail(SPLITKV_ERR_INVALID_ARG, "%s: q_scale must be positive and finite", fn);
  }
  // 16-byte vector loads of q rows and cache rows
  const int64_t elem = a->kv_dtype == SPLITKV_KV_E4M3 ? 1 : 2;
  if (!aligned(a->q, 16) || (a->q_stride_b * 2) % 16 || (a->q_stride_t * 2) % 16 ||
      (a->q_stride_h * 2) % 16)
    return fail(SPLITKV_ERR_UNSUPPORTED, "%s: q or its strides not 16-byte aligned", fn);
  if (!aligned(a->k_cache, 16) || (a->k_stride_page * elem) % 16 ||
      (a->k_stride_head * elem) % 16 || (a->k_stride_tok * elem) % 16)
    return fail(SPLITKV_ERR_UNSUPPORTED, "%s: k_cache or its strides not 16-byte aligned", fn);
  if (kind != Kind::Mla &&
      (!aligned(a->v_cache, 16) || (a->v_stride_page * elem) % 16 ||
       (a->v_stride_head * elem) % 16 || (a->v_stride_tok * elem) % 16))
    return fail(SPLITKV_ERR_UNSUPPORTED, "%s: v_cache or its strides not 16-byte aligned", fn);
  if (!a->out || !aligned(a->out, 16)) return fail(SPLITKV_ERR_INVALID_ARG, "%s: out null or misaligned", fn);
  if (need_ws) {
    const size_t need = splitkv_workspace_bytes(a->total_slots, a->T, a->Hq, a->d_v);
    if (!a->workspace || !aligned(a->workspace, 16) || a->workspace_bytes < need)
      return fail(SPLITKV_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu (16-byte aligned)", fn,
                  a->workspace_bytes, need);
  }
  const int64_t rows = kind == Kind::Mla ? int64_t(a->T) * a->Hq : int64_t(a->Hq / a->Hkv) * a->T;
  const int64_t rpw = kind == Kind::Mla ? SPLITKV_ROWS_PER_WG_MLA : SPLITKV_ROWS_PER_WG_GQA;
  *row_blocks = int(ceil_div(rows, rpw));
  const int64_t wgs = int64_t(a->total_slots) * a->Hkv * *row_blocks;
  if (wgs > (int64_t(1) << 30)) return fail(SPLITKV_ERR_INVALID_ARG, "%s: grid too large", fn);
  if (kind != Kind::Mla) {
    // the grouped-query kernels take 32-bit strides and a packed launch geometry
    const int64_t st[] = {a->q_stride_b, a->q_stride_t, a->q_stride_h, a->k_stride_page * elem,
                          a->k_stride_head * elem, a->k_stride_tok * elem, a->v_stride_page * elem,
                          a->v_stride_head * elem, a->v_stride_tok * elem, a->bt_stride};
    for (int64_t x : st)
      if (x < 0 || x > INT32_MAX)
        return fail(SPLITKV_ERR_UNSUPPORTED, "%s: a stride of %lld does not fit 31 bits", fn,
                    static_cast<long long>(x));
    // buffer offsets inside one 16-token group are 32-bit
    if (16 * (a->k_stride_tok * elem) + a->d_qk * elem > INT32_MAX ||
        16 * (a->v_stride_tok * elem) + a->d_v * elem > INT32_MAX)
      return fail(SPLITKV_ERR_UNSUPPORTED, "%s: token strides too large", fn);
    if (a->Hkv > 0xffff || *row_blocks > 0xff)
      return fail(SPLITKV_ERR_UNSUPPORTED, "%s: Hkv=%d or %d row blocks too large", fn, a->Hkv,
                  *row_blocks);
  }
  return SPLITKV_OK;
}

PartialParams make_partial_params(const splitkv_args& a, Kind kind, int row_blocks, bool direct) {
  const int64_t elem = a.kv_dtype == SPLITKV_KV_E4M3 ? 1 : 2;
  PartialParams p;
  memset(&p, 0, sizeof(p));
  p.q = static_cast<const uint16_t*>(a.q);
  p.qsb = a.q_stride_b;
  p.qst = a.q_stride_t;
  p.qsh = a.q_stride_h;
  // rows (t, h) of a sequence evenly spaced: the MLA kernel reads them with
  // 32-bit byte offsets from the sequence's query
  p.q_rows_linear = kind == Kind::Mla && a.q_stride_h >= 0 && a.q_stride_t == int64_t(a.Hq) * a.q_stride_h &&
                    (int64_t(a.T) * a.Hq - 1) * a.q_stride_h * 2 + 2 * 576 < (int64_t(1) << 31);
  p.k = static_cast<const uint8_t*>(a.k_cache);
  p.v = kind == Kind::Mla ? p.k : static_cast<const uint8_t*>(a.v_cache);
  p.ksp = a.k_stride_page * elem;
  p.ksh = a.k_stride_head * elem;
  p.kst = a.k_stride_tok * elem;
  p.vsp = kind == Kind::Mla ? p.ksp : a.v_stride_page * elem;
  p.vsh = kind == Kind::Mla ? p.ksh : a.v_stride_head * elem;
  p.vst = kind == Kind::Mla ? p.kst : a.v_stride_tok * elem;
  p.bt = a.block_table;
  p.bt_stride = a.bt_stride;
  p.seq_lens = a.seq_lens;
  p.num_splits = a.num_splits;
  p.slot_offset = a.slot_offset;
  p.slot_info = a.slot_info;
  p.T = a.T;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.g = a.Hq / a.Hkv;
  p.page_size = a.page_size;
  p.rows = kind == Kind::Mla ? a.T * a.Hq : p.g * a.T;
  p.row_blocks = row_blocks;
  p.total_wg = a.total_slots * a.Hkv * row_blocks;
  p.page_shift = (a.page_size & (a.page_size - 1)) == 0 ? __builtin_ctz(unsigned(a.page_size)) : -1;
  const bool q8 = a.q_dtype == SPLITKV_Q_E4M3;
  p.q_scale = q8 ? a.q_scale : 1.f;
  p.q_rcp = p.q_scale >= 0x1p-64f && p.q_scale <= 0x1p64f ? 1.f / p.q_scale : 0.f;
  p.scale_log2 = a.scale * a.k_scale * p.q_scale * kLog2e;
  p.v_scale = a.v_scale;
  const Layout w = workspace_layout(a);
  p.part_m = w.m;
  p.part_l = w.l;
  p.part_o = w.o;
  p.part_s = w.s;
  p.part_q = w.q;
  p.out = a.out;
  p.out_f32 = a.out_dtype == SPLITKV_OUT_F32;
  p.lse = a.lse;
  p.debug = a.debug;
  p.tickets = a.tickets;
  p.direct = direct ? 1 : 0;
  return p;
}

// Compute units of the current device, queried once per device (0 if unknown).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev] = n;
  }
  return cus[dev];
}

// The MLA kernel of a step: the short-range one (64 rows, eight waves a
// workgroup) when the caller says every split range is at most eight 32-token
// tiles and its 64-row workgroups all fit on the compute units at once; the
// 128-row one otherwise.  SPLITKV_MLA_KERNEL=short or =long in the
// environment forces either (for tests and measurements).
bool use_short_mla(const splitkv_args& a) {
  if (const char* env = getenv("SPLITKV_MLA_KERNEL")) {
    if (!strcmp(env, "short")) return true;
    if (!strcmp(env, "long")) return false;
  }
  const int64_t wgs = int64_t(a.total_slots) * ceil_div(int64_t(a.T) * a.Hq, int64_t(64));
  return a.max_range_tokens > 0 && a.max_range_tokens <= 8 * 32 && wgs <= device_cus();
}

splitkv_status run_partial(const splitkv_args* a, Kind kind, bool direct, void* stream,
                           const char* fn, bool fused = false) {
  int row_blocks = 0;
  // Direct mode only needs the workspace when some sequence has several splits.
  const bool need_ws = !direct || (a && a->total_slots > a->B);
  splitkv_status st = check_partial(a, kind, need_ws, fn, &row_blocks);
  if (st != SPLITKV_OK) return st;
  if (fused && need_ws && (!a->tickets || !aligned(a->tickets, 4)))
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: the single launch needs the tickets array", fn);
  st = check_device(nullptr);
  if (st != SPLITKV_OK) return st;
  const PartialParams p = make_partial_params(*a, kind, row_blocks, direct);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (kind != Kind::Mla)
    err = launch_gqa_partial(p, a->d_qk, kind == Kind::GqaFp8, fused, s);
  else if (!use_short_mla(*a))
    err = launch_mla_partial(p, a->q_dtype == SPLITKV_Q_E4M3 ? 2 : a->kv_dtype == SPLITKV_KV_E4M3 ? 1 : 0, s);
  else {
    // the same plan in 64-row blocks (two to a plan row block)
    const PartialParams ps =
        make_partial_params(*a, kind, int(ceil_div(int64_t(a->T) * a->Hq, int64_t(64))), direct);
    err = a->q_dtype == SPLITKV_Q_E4M3 ? launch_mla_short_q8_partial(ps, s)
                                       : launch_mla_short_partial(ps, a->kv_dtype == SPLITKV_KV_E4M3, s);
  }
  if (err != hipSuccess) return fail(SPLITKV_ERR_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(err));
  return SPLITKV_OK;
}

splitkv_status run_combine(const splitkv_args* a, bool skip_single, void* stream, const char* fn) {
  splitkv_status st = check_common(a, fn);
  if (st != SPLITKV_OK) return st;
  if (a->d_v != 64 && a->d_v != 128 && a->d_v != 256 && a->d_v != 512)
    return fail(SPLITKV_ERR_UNSUPPORTED, "%s: d_v=%d; built for 64, 128, 256, 512", fn, a->d_v);
  if (!a->out || !aligned(a->out, 16)) return fail(SPLITKV_ERR_INVALID_ARG, "%s: out null or misaligned", fn);
  const size_t need = splitkv_workspace_bytes(a->total_slots, a->T, a->Hq, a->d_v);
  if (!a->workspace || !aligned(a->workspace, 16) || a->workspace_bytes < need)
    return fail(SPLITKV_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, a->workspace_bytes,
                need);
  if (a->uniform_splits < 0 || a->uniform_splits > SPLITKV_MAX_SPLITS_LIMIT ||
      (a->uniform_splits > 0 && int64_t(a->uniform_splits) * a->B != a->total_slots))
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: uniform_splits=%d inconsistent with B=%d, total_slots=%d",
                fn, a->uniform_splits, a->B, a->total_slots);
  if (a->max_seq_splits < 0 || a->max_seq_splits > SPLITKV_MAX_SPLITS_LIMIT)
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: max_seq_splits=%d outside [0, %d]", fn, a->max_seq_splits,
                SPLITKV_MAX_SPLITS_LIMIT);
  st = check_device(nullptr);
  if (st != SPLITKV_OK) return st;
  const Layout w = workspace_layout(*a);
  CombineParams p;
  p.num_splits = a->num_splits;
  p.slot_offset = a->slot_offset;
  p.part_m = w.m;
  p.part_l = w.l;
  p.part_o = w.o;
  p.out = a->out;
  p.out_f32 = a->out_dtype == SPLITKV_OUT_F32;
  p.lse = a->lse;
  p.B = a->B;
  p.R = a->T * a->Hq;
  p.d_v = a->d_v;
  p.skip_single = skip_single ? 1 : 0;
  p.uniform_splits = a->uniform_splits;
  p.max_seq_splits = a->max_seq_splits;
  const hipError_t err = launch_combine(p, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(SPLITKV_ERR_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(err));
  return SPLITKV_OK;
}

// Partials buffer of splitkv_decode_noalloc: a module-scope device array, one
// copy per device, held until the process ends.  In host code its name only
// stands in for the symbol; the device address comes from hipGetSymbolAddress,
// once per device with that device current, and only that address is handed
// to the kernels.
static __device__ __align__(256) uint8_t scratch[SPLITKV_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

splitkv_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(SPLITKV_ERR_DEVICE, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !p)
      return fail(SPLITKV_ERR_DEVICE, "hipGetSymbolAddress of the partials buffer failed on device %d: %s",
                  dev, hipGetErrorString(err));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SPLITKV_OK;
}

}  // namespace
}  // namespace splitkv

using namespace splitkv;

extern "C" {

splitkv_status splitkv_plan(const splitkv_plan_args* args, const int32_t* seq_lens_host,
                            int32_t* num_splits_host, int32_t* slot_offset_host,
                            int32_t* slot_info_host, int32_t slot_info_capacity,
                            int32_t* total_slots) {
  if (!args) return fail(SPLITKV_ERR_INVALID_ARG, "splitkv_plan: null args");
  int cus = args->num_cus;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return fail(SPLITKV_ERR_DEVICE, "splitkv_plan: cannot query the compute-unit count");
  }
  return plan_host(*args, cus, seq_lens_host, num_splits_host, slot_offset_host, slot_info_host,
                   slot_info_capacity, total_slots);
}

splitkv_status splitkv_decode_partial(const splitkv_args* args, void* stream) {
  return run_partial(args, Kind::GqaBf16, false, stream, "splitkv_decode_partial");
}

splitkv_status splitkv_decode_partial_fp8(const splitkv_args* args, void* stream) {
  return run_partial(args, Kind::GqaFp8, false, stream, "splitkv_decode_partial_fp8");
}

int32_t splitkv_mla_short_range(const splitkv_args* args) {
  return args && use_short_mla(*args) ? 1 : 0;
}

splitkv_status splitkv_mla_decode_partial(const splitkv_args* args, void* stream) {
  return run_partial(args, Kind::Mla, false, stream, "splitkv_mla_decode_partial");
}

splitkv_status splitkv_combine(const splitkv_args* args, void* stream) {
  return run_combine(args, false, stream, "splitkv_combine");
}

splitkv_status splitkv_decode(const splitkv_args* args, int32_t kernel, void* stream) {
  if (!args) return fail(SPLITKV_ERR_INVALID_ARG, "splitkv_decode: null args");
  Kind kind;
  if (kernel == SPLITKV_KERNEL_MLA) kind = Kind::Mla;
  else if (kernel == SPLITKV_KERNEL_GQA) kind = args->kv_dtype == SPLITKV_KV_E4M3 ? Kind::GqaFp8 : Kind::GqaBf16;
  else return fail(SPLITKV_ERR_INVALID_ARG, "splitkv_decode: unknown kernel %d", kernel);
  // The single launch (ticketed last-arriver merge) replaces the merge kernel
  // for small steps: a grid of a few workgroups whose groups the last arriver
  // merges in one round of loads (one float4 column of one row per thread,
  // at most eight splits).  It measured faster than two kernels only there: a
  // larger group is merged by one workgroup far more slowly than by the merge
  // kernel's whole grid, and on a full grid every workgroup's device-scope
  // release costs more than the second launch saves.
  if (kind != Kind::Mla && args->tickets && args->max_seq_splits > 1 && args->Hkv > 0 && args->T > 0 &&
      args->total_slots > args->B && args->max_seq_splits <= 8) {
    const int64_t rw = std::min<int64_t>(SPLITKV_ROWS_PER_WG_GQA, int64_t(args->Hq / args->Hkv) * args->T);
    const int64_t wgs = int64_t(args->total_slots) * args->Hkv *
                        ceil_div(int64_t(args->Hq / args->Hkv) * args->T, SPLITKV_ROWS_PER_WG_GQA);
    if (rw * (args->d_v / 4) <= 256 && wgs <= SPLITKV_SINGLE_LAUNCH_MAX_WORKGROUPS)
      return run_partial(args, kind, true, stream, "splitkv_decode", true);
  }
  splitkv_status st = run_partial(args, kind, true, stream, "splitkv_decode");
  if (st != SPLITKV_OK || args->total_slots == args->B) return st;
  return run_combine(args, true, stream, "splitkv_decode");
}

splitkv_status splitkv_decode_single_launch(const splitkv_args* args, int32_t kernel, void* stream) {
  const char* fn = "splitkv_decode_single_launch";
  if (!args) return fail(SPLITKV_ERR_INVALID_ARG, "%s: null args", fn);
  if (kernel != SPLITKV_KERNEL_GQA)
    return fail(SPLITKV_ERR_UNSUPPORTED, "%s: built for the grouped-query kernels only", fn);
  const Kind kind = args->kv_dtype == SPLITKV_KV_E4M3 ? Kind::GqaFp8 : Kind::GqaBf16;
  return run_partial(args, kind, true, stream, fn, true);
}

splitkv_status splitkv_decode_noalloc(const splitkv_args* args, int32_t kernel, void* stream) {
  const char* fn = "splitkv_decode_noalloc";
  if (!args) return fail(SPLITKV_ERR_INVALID_ARG, "%s: null args", fn);
  // size check first: a plan that does not fit is refused before any device call
  const size_t need = splitkv_workspace_bytes(args->total_slots, args->T, args->Hq, args->d_v);
  if (need > size_t(SPLITKV_NOALLOC_SCRATCH_BYTES))
    return fail(SPLITKV_ERR_WORKSPACE,
                "%s: the plan's partials need %zu bytes; the library buffer holds %d "
                "(use fewer splits, or splitkv_decode with a workspace)",
                fn, need, SPLITKV_NOALLOC_SCRATCH_BYTES);
  splitkv_status st = check_device(nullptr);
  if (st != SPLITKV_OK) return st;
  void* buf = nullptr;
  st = scratch_address(&buf);
  if (st != SPLITKV_OK) return st;
  splitkv_args a = *args;
  a.workspace = static_cast<float*>(buf);
  a.workspace_bytes = size_t(SPLITKV_NOALLOC_SCRATCH_BYTES);
  return splitkv_decode(&a, kernel, stream);
}

splitkv_status splitkv_e4m3_to_bf16(const uint8_t* in, uint16_t* out, int64_t n, void* stream) {
  if (!in || !out || n < 0 || !aligned(in, 4) || !aligned(out, 2))
    return fail(SPLITKV_ERR_INVALID_ARG, "splitkv_e4m3_to_bf16: bad arguments");
  if (n == 0) return SPLITKV_OK;
  splitkv_status st = check_device(nullptr);
  if (st != SPLITKV_OK) return st;
  const hipError_t err = launch_e4m3_to_bf16(in, out, n, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(SPLITKV_ERR_LAUNCH, "splitkv_e4m3_to_bf16: %s", hipGetErrorString(err));
  return SPLITKV_OK;
}

splitkv_status splitkv_append_kv(const splitkv_append_args* a, void* stream) {
  const char* fn = "splitkv_append_kv";
  if (!a) return fail(SPLITKV_ERR_INVALID_ARG, "%s: null args", fn);
  if (!a->k_new || !a->k_cache || !a->block_table || !a->positions)
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: null k_new, k_cache, block_table or positions", fn);
  if ((a->v_new == nullptr) != (a->v_cache == nullptr))
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: v_new and v_cache must both be given or both be NULL", fn);
  if (a->B < 1 || a->T < 1 || a->Hkv < 1 || a->page_size < 1 || a->num_pages < 1 || a->bt_stride < 1)
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: bad shape B=%d T=%d Hkv=%d page_size=%d num_pages=%d", fn,
                a->B, a->T, a->Hkv, a->page_size, a->num_pages);
  const bool has_v = a->v_cache != nullptr;
  if (a->d_k < 8 || a->d_k % 8 || (has_v && (a->d_v < 8 || a->d_v % 8)))
    return fail(SPLITKV_ERR_UNSUPPORTED, "%s: d_k=%d d_v=%d must be positive multiples of 8", fn, a->d_k,
                a->d_v);
  if (a->kv_dtype != SPLITKV_KV_BF16 && a->kv_dtype != SPLITKV_KV_E4M3)
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: kv_dtype=%d", fn, a->kv_dtype);
  const bool fp8 = a->kv_dtype == SPLITKV_KV_E4M3;
  if (fp8 && (!(a->k_scale > 0.f) || !(a->k_scale < INFINITY) ||
              (has_v && (!(a->v_scale > 0.f) || !(a->v_scale < INFINITY)))))
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: e4m3 scales must be positive and finite", fn);
  const int64_t elem = fp8 ? 1 : 2;
  auto rows_ok = [&](const void* base, int64_t sb, int64_t st, int64_t sh) {
    return aligned(base, 16) && (sb * 2) % 16 == 0 && (st * 2) % 16 == 0 && (sh * 2) % 16 == 0;
  };
  auto cache_ok = [&](const void* base, int64_t sp, int64_t sh, int64_t sk) {
    return aligned(base, 16) && (sp * elem) % 16 == 0 && (sh * elem) % 16 == 0 && (sk * elem) % 16 == 0;
  };
  if (!rows_ok(a->k_new, a->k_new_stride_b, a->k_new_stride_t, a->k_new_stride_h) ||
      (has_v && !rows_ok(a->v_new, a->v_new_stride_b, a->v_new_stride_t, a->v_new_stride_h)))
    return fail(SPLITKV_ERR_UNSUPPORTED, "%s: new rows or their strides not 16-byte aligned", fn);
  if (!cache_ok(a->k_cache, a->k_stride_page, a->k_stride_head, a->k_stride_tok) ||
      (has_v && !cache_ok(a->v_cache, a->v_stride_page, a->v_stride_head, a->v_stride_tok)))
    return fail(SPLITKV_ERR_UNSUPPORTED, "%s: caches or their strides not 16-byte aligned", fn);
  if (!aligned(a->block_table, 4) || !aligned(a->positions, 4))
    return fail(SPLITKV_ERR_INVALID_ARG, "%s: block_table or positions misaligned", fn);
  const int64_t rows = int64_t(a->B) * a->T * a->Hkv;
  if (rows > INT32_MAX) return fail(SPLITKV_ERR_INVALID_ARG, "%s: grid too large", fn);
  splitkv_status st = check_device(nullptr);
  if (st != SPLITKV_OK) return st;
  AppendParams p;
  memset(&p, 0, sizeof(p));
  p.src[0] = static_cast<const uint16_t*>(a->k_new);
  p.ssb[0] = a->k_new_stride_b;
  p.sst[0] = a->k_new_stride_t;
  p.ssh[0] = a->k_new_stride_h;
  p.dst[0] = static_cast<uint8_t*>(a->k_cache);
  p.dsp[0] = a->k_stride_page * elem;
  p.dsh[0] = a->k_stride_head * elem;
  p.dsk[0] = a->k_stride_tok * elem;
  p.d[0] = a->d_k;
  p.scale[0] = a->k_scale;
  if (has_v) {
    p.src[1] = static_cast<const uint16_t*>(a->v_new);
    p.ssb[1] = a->v_new_stride_b;
    p.sst[1] = a->v_new_stride_t;
    p.ssh[1] = a->v_new_stride_h;
    p.dst[1] = static_cast<uint8_t*>(a->v_cache);
    p.dsp[1] = a->v_stride_page * elem;
    p.dsh[1] = a->v_stride_head * elem;
    p.dsk[1] = a->v_stride_tok * elem;
    p.d[1] = a->d_v;
    p.scale[1] = a->v_scale;
  }
  p.bt = a->block_table;
  p.bt_stride = a->bt_stride;
  p.positions = a->positions;
  p.T = a->T;
  p.Hkv = a->Hkv;
  p.page_size = a->page_size;
  p.num_pages = a->num_pages;
  p.fp8 = fp8 ? 1 : 0;
  const hipError_t err = launch_append(p, int(rows), has_v ? 2 : 1, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(SPLITKV_ERR_LAUNCH, "%s: %s", fn, hipGetErrorString(err));
  return SPLITKV_OK;
}

size_t splitkv_append_args_size(void) { return sizeof(splitkv_append_args); }

const char* splitkv_version(void) { return SPLITKV_REVISION; }

}  // extern "C"
