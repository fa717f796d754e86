// C ABI of the sink-attention library: argument validation, the decode
// split planner, and dispatch to the gfx950 kernels.  Declarations and the
// contract of every entry point are in include/sink_attn.h.
#include "sink_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

sink_attn_status fail(sink_attn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

sink_attn_status ok() {
  g_last_error[0] = '\0';
  return SINK_ATTN_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kHeadDim = 64;
constexpr int kPageSize = 16;

sink_attn_status check_heads(int32_t hq, int32_t hkv) {
  if (hq <= 0 || hkv <= 0) return fail(SINK_ATTN_ERR_BAD_SHAPE, "head counts must be positive (Hq=%d, Hkv=%d)", hq, hkv);
  if (hq % hkv) return fail(SINK_ATTN_ERR_BAD_SHAPE, "Hq=%d is not a multiple of Hkv=%d", hq, hkv);
  const int G = hq / hkv;
  if (!(G == 1 || G == 2 || G == 4 || G == 8 || G == 16))
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "group size Hq/Hkv=%d is not built (1, 2, 4, 8, 16)", G);
  return ok();
}

// Compute units of the current device, queried once per device.  The
// automatic plans size their grids to the machine (one workgroup per CU for
// the balanced decode, a few per CU elsewhere), so a device that exposes
// fewer CUs (a partitioned GPU) gets a grid that still divides evenly.
// Without a usable device (host-only planning, no GPU) the full MI355X's 256.
constexpr int kDefaultCUs = 256;
constexpr int kMaxDevices = 64;
std::once_flag g_cu_once[kMaxDevices];
int g_cu_count[kMaxDevices];

int device_cus() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();  // leave no sticky error for the next launch check
    return kDefaultCUs;
  }
  std::call_once(g_cu_once[dev], [dev]() {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0) {
      (void)hipGetLastError();
      n = kDefaultCUs;
    }
    g_cu_count[dev] = n;
  });
  return g_cu_count[dev];
}

sink_attn_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SINK_ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Keys per split are rounded to whole pages.  The automatic plan aims at
// eight workgroups (32 waves) per compute unit while keeping each split at
// least 16 pages long, so that a workgroup amortises its merge.
int32_t plan_splits(int32_t batch, int32_t hkv, int32_t max_kv_len, int32_t requested) {
  const int32_t pages = (max_kv_len + kPageSize - 1) / kPageSize;
  if (requested > 0) {
    int32_t s = requested;
    if (pages > 0 && s > pages) s = pages;  // never more splits than pages
    return s < 1 ? 1 : s;
  }
  if (pages <= 16) return 1;
  const int64_t units = (int64_t)batch * hkv;
  const int64_t target_wgs = 8 * (int64_t)device_cus();
  int64_t s = (target_wgs + units - 1) / units;
  const int64_t max_by_len = (pages + 15) / 16;  // >= 16 pages per split
  if (s > max_by_len) s = max_by_len;
  if (s < 1) s = 1;
  if (s > 256) s = 256;
  return (int32_t)s;
}

// Load-balanced plan: the batch's pages are cut, per KV head, into n_ranges
// equal ranges (a multiple of 4: one workgroup holds four ranges, one per
// wave).  Every range carries the same work, so the grid must spread evenly
// over the compute units: the automatic plan launches at most one workgroup
// per CU (the device's CU count), i.e. one streaming wave per SIMD, which
// keeps two K/V steps in flight per wave -- enough to saturate HBM -- and
// makes the ranges as long as possible, so the start-up of a wave and the
// merge of a request's partials stay small against its streaming.  Ranges
// shorter than kMinRangePages pages are not worth a wave.  An explicit request
// takes exactly that many ranges (rounded up to a multiple of 4) and allows
// ranges down to one page.
constexpr int32_t kMinRangePages = 8;
constexpr int32_t kMaxRanges = 1 << 20;

struct RangePlan {
  int32_t n_ranges;
  int32_t min_pages;
};

RangePlan plan_ranges(int32_t batch, int32_t hkv, int32_t max_kv_len, int32_t requested) {
  int64_t r;
  int32_t min_pages;
  if (requested > 0) {
    r = (requested + 3) / 4 * 4;
    min_pages = 1;
  } else {
    const int64_t pages_ub = (int64_t)batch * ((max_kv_len + kPageSize - 1) / kPageSize);
    const int64_t wgs_per_head = device_cus() / hkv;
    r = 4 * (wgs_per_head > 1 ? wgs_per_head : 1);
    const int64_t by_len = (pages_ub + kMinRangePages - 1) / kMinRangePages;
    if (r > by_len) r = (by_len + 3) / 4 * 4;
    min_pages = kMinRangePages;
  }
  if (r > kMaxRanges) r = kMaxRanges;
  if (r < 4) r = 4;
  return RangePlan{(int32_t)r, min_pages};
}

size_t balanced_slots(int32_t batch, int32_t n_ranges) { return (size_t)n_ranges + batch - 1; }

size_t align_up(size_t n, size_t a) { return (n + a - 1) / a * a; }

// sink_attn_decode's automatic plan: requests longer than 16 pages go to the
// load-balanced plan; shorter ones fit one chunk, written by one kernel.
bool auto_uses_balanced(int32_t max_kv_len, int32_t num_splits) {
  return num_splits == 0 && (max_kv_len + kPageSize - 1) / kPageSize > 16;
}

int32_t chunk_pages_for(int32_t max_kv_len, int32_t splits) {
  const int32_t pages = (max_kv_len + kPageSize - 1) / kPageSize;
  int32_t cp = (pages + splits - 1) / splits;
  return cp < 1 ? 1 : cp;
}

}  // namespace

namespace sa {
// Records the failure of an entry point defined in another source file, as
// the calling thread's last error.
sink_attn_status api_fail(sink_attn_status s, const char* detail) { return fail(s, "%s", detail); }
}  // namespace sa

extern "C" {

const char* sink_attn_status_string(sink_attn_status s) {
  switch (s) {
    case SINK_ATTN_OK: return "ok";
    case SINK_ATTN_ERR_NULL_ARG: return "a required pointer is NULL";
    case SINK_ATTN_ERR_BAD_SHAPE: return "bad or inconsistent sizes";
    case SINK_ATTN_ERR_UNSUPPORTED: return "configuration not supported";
    case SINK_ATTN_ERR_MISALIGNED: return "misaligned pointer";
    case SINK_ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case SINK_ATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* sink_attn_last_error(void) { return g_last_error; }

const char* sink_attn_version(void) { return "sink_attn 0.1 gfx950"; }

int32_t sink_attn_decode_num_splits(int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                                    int32_t max_kv_len, int32_t num_splits) {
  (void)num_qo_heads;
  if (batch <= 0 || num_kv_heads <= 0 || max_kv_len < 0) return 1;
  return plan_splits(batch, num_kv_heads, max_kv_len, num_splits);
}

size_t sink_attn_decode_workspace_size(int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_kv_len, int32_t num_splits) {
  if (batch <= 0 || num_qo_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_kv_len < 0 ||
      num_splits < 0)
    return 0;
  if (auto_uses_balanced(max_kv_len, num_splits))
    return sink_attn_decode_balanced_workspace_size(batch, num_qo_heads, num_kv_heads, head_dim,
                                                    max_kv_len, 0);
  const int32_t s = plan_splits(batch, num_kv_heads, max_kv_len, num_splits);
  if (s <= 1) return 0;
  const size_t rows = (size_t)batch * num_qo_heads * s;
  const size_t o_bytes = rows * head_dim * sizeof(float);
  const size_t l_bytes = rows * sizeof(float);
  return o_bytes + ((l_bytes + 255) / 256) * 256;
}

int32_t sink_attn_decode_num_ranges(int32_t batch, int32_t num_kv_heads, int32_t max_kv_len,
                                    int32_t num_ranges) {
  if (batch <= 0 || num_kv_heads <= 0 || max_kv_len < 0 || num_ranges < 0) return 4;
  return plan_ranges(batch, num_kv_heads, max_kv_len, num_ranges).n_ranges;
}

size_t sink_attn_decode_balanced_workspace_size(int32_t batch, int32_t num_qo_heads,
                                                int32_t num_kv_heads, int32_t head_dim,
                                                int32_t max_kv_len, int32_t num_ranges) {
  if (batch <= 0 || num_qo_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_kv_len < 0 ||
      num_ranges < 0)
    return 0;
  const RangePlan plan = plan_ranges(batch, num_kv_heads, max_kv_len, num_ranges);
  const size_t rows = balanced_slots(batch, plan.n_ranges) * num_qo_heads;
  const size_t o_bytes = rows * head_dim * sizeof(float);
  const size_t l_bytes = rows * sizeof(float);
  return o_bytes + ((l_bytes + 255) / 256) * 256;
}

}  // extern "C"

namespace {

// The queries of a prefill step: projection rows, bias, rotary table.
struct PrefillStepInputs {
  const void* qkv;
  const void* bias;
  const float* table;
  int32_t max_pos;
  int32_t interleaved;
};

// Host checks and launch arguments of a prefill (step == nullptr) or of a
// prefill step's attention; nothing is launched.  *empty: no query rows.
sink_attn_status prefill_check(const void* q, const int32_t* qo_indptr, const void* k,
                               const void* v, const int32_t* kv_indptr,
                               const int32_t* page_indices, const int32_t* kv_len,
                               const float* sinks, int32_t batch, int32_t num_qo_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                               int32_t total_q, int32_t max_qlen, int32_t max_kv_len,
                               float sm_scale, int32_t causal, void* out,
                               sink_attn_dtype out_dtype, float* lse,
                               const PrefillStepInputs* step, sa::PrefillArgs* a, bool* empty) {
  const char* who = step ? "prefill_step" : "prefill";
  const void* queries = step ? step->qkv : q;
  if (!queries || !qo_indptr || !k || !v || !kv_indptr || !out)
    return fail(SINK_ATTN_ERR_NULL_ARG, "%s: %s, qo_indptr, k, v, kv_indptr and out are required",
                who, step ? "qkv" : "q");
  if (page_indices && !kv_len)
    return fail(SINK_ATTN_ERR_NULL_ARG, "%s: kv_len is required with a paged cache", who);
  if (batch <= 0 || total_q < 0 || max_qlen < 0 || max_kv_len < 0)
    return fail(SINK_ATTN_ERR_BAD_SHAPE, "%s: batch=%d total_q=%d max_qlen=%d max_kv_len=%d", who,
                batch, total_q, max_qlen, max_kv_len);
  if (max_qlen > total_q)
    return fail(SINK_ATTN_ERR_BAD_SHAPE, "%s: max_qlen=%d exceeds total_q=%d", who, max_qlen,
                total_q);
  if (causal && max_qlen > 0 && max_kv_len <= 0)
    return fail(SINK_ATTN_ERR_BAD_SHAPE, "%s: causal queries need keys (max_kv_len=%d)", who,
                max_kv_len);
  sink_attn_status st = check_heads(num_qo_heads, num_kv_heads);
  if (st != SINK_ATTN_OK) return st;
  if (head_dim != kHeadDim)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "%s: head_dim=%d (only 64 is built)", who, head_dim);
  if (page_indices && page_size != kPageSize)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "%s: page_size=%d (only 16 is built)", who, page_size);
  if (out_dtype != SINK_ATTN_BF16 && out_dtype != SINK_ATTN_F32)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "%s: unknown out_dtype %d", who, (int)out_dtype);
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale))
    return fail(SINK_ATTN_ERR_BAD_SHAPE, "%s: sm_scale must be positive and finite", who);
  if (!aligned(queries, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(SINK_ATTN_ERR_MISALIGNED, "%s: %s, k, v and out must be 16-byte aligned", who,
                step ? "qkv" : "q");
  if (!aligned(qo_indptr, 4) || !aligned(kv_indptr, 4) || (page_indices && !aligned(page_indices, 4)) ||
      (kv_len && !aligned(kv_len, 4)) || (sinks && !aligned(sinks, 4)) || (lse && !aligned(lse, 4)))
    return fail(SINK_ATTN_ERR_MISALIGNED, "%s: index, sink and lse arrays must be 4-byte aligned",
                who);
  *empty = total_q == 0 || max_qlen == 0;
  if (*empty) return ok();
  {
    // one workgroup per (256 / G query tokens, KV head, request): a flat grid
    const int64_t tokens_per_wg = 256 / (num_qo_heads / num_kv_heads);
    const int64_t wgs = (max_qlen + tokens_per_wg - 1) / tokens_per_wg * num_kv_heads * (int64_t)batch;
    if (wgs > 0x7fffffff)
      return fail(SINK_ATTN_ERR_BAD_SHAPE, "%s: %lld workgroups exceed the grid limit", who,
                  (long long)wgs);
  }
  a->q = static_cast<const uint16_t*>(q);
  a->qo_indptr = qo_indptr;
  a->k = static_cast<const uint16_t*>(k);
  a->v = static_cast<const uint16_t*>(v);
  a->kv_indptr = kv_indptr;
  a->page_indices = page_indices;
  a->kv_len = kv_len;
  a->sinks = sinks;
  a->batch = batch;
  a->hq = num_qo_heads;
  a->hkv = num_kv_heads;
  a->max_qlen = max_qlen;
  a->causal = causal ? 1 : 0;
  a->scale_log2 = sm_scale * 1.4426950408889634f;
  a->out = out;
  a->out_f32 = out_dtype == SINK_ATTN_F32;
  a->lse = lse;
  a->qkv = step ? static_cast<const uint16_t*>(step->qkv) : nullptr;
  a->bias = step ? static_cast<const uint16_t*>(step->bias) : nullptr;
  a->table = step ? step->table : nullptr;
  a->max_pos = step ? step->max_pos : 0;
  a->interleaved = step ? step->interleaved : 0;
  a->longest_first = batch <= sa::kPrefillLongestFirstMaxBatch;
  return ok();
}

}  // namespace

extern "C" {

sink_attn_status sink_attn_prefill(const void* q, const int32_t* qo_indptr, const void* k,
                                   const void* v, const int32_t* kv_indptr,
                                   const int32_t* page_indices, const int32_t* kv_len,
                                   const float* sinks, int32_t batch, int32_t num_qo_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                   int32_t total_q, int32_t max_qlen, int32_t max_kv_len,
                                   float sm_scale, int32_t causal, void* out,
                                   sink_attn_dtype out_dtype, float* lse, void* stream) {
  sa::PrefillArgs a;
  bool empty = false;
  sink_attn_status st = prefill_check(q, qo_indptr, k, v, kv_indptr, page_indices, kv_len, sinks,
                                      batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                                      total_q, max_qlen, max_kv_len, sm_scale, causal, out,
                                      out_dtype, lse, nullptr, &a, &empty);
  if (st != SINK_ATTN_OK || empty) return st;
  return hip_status(sa::launch_prefill(a, num_qo_heads / num_kv_heads,
                                       static_cast<hipStream_t>(stream)),
                    "prefill launch");
}

sink_attn_status sink_attn_merge(const float* o_parts, const float* lse_parts, int32_t num_rows,
                                 int32_t num_heads, int32_t num_splits, int32_t head_dim,
                                 void* out, sink_attn_dtype out_dtype, float* lse_out,
                                 void* stream) {
  if (!o_parts || !lse_parts || !out)
    return fail(SINK_ATTN_ERR_NULL_ARG, "merge: o_parts, lse_parts and out are required");
  if (num_rows < 0 || num_heads <= 0 || num_splits <= 0)
    return fail(SINK_ATTN_ERR_BAD_SHAPE, "merge: rows=%d heads=%d splits=%d", num_rows, num_heads,
                num_splits);
  if (head_dim != kHeadDim)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "merge: head_dim=%d (only 64 is built)", head_dim);
  if (out_dtype != SINK_ATTN_BF16 && out_dtype != SINK_ATTN_F32)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "merge: unknown out_dtype %d", (int)out_dtype);
  if (!aligned(o_parts, 16) || !aligned(out, 16))
    return fail(SINK_ATTN_ERR_MISALIGNED, "merge: o_parts and out must be 16-byte aligned");
  if (!aligned(lse_parts, 4) || (lse_out && !aligned(lse_out, 4)))
    return fail(SINK_ATTN_ERR_MISALIGNED, "merge: lse arrays must be 4-byte aligned");
  if (num_rows == 0) return ok();
  sa::MergeArgs a;
  a.o_parts = o_parts;
  a.lse_parts = lse_parts;
  a.rows = num_rows;
  a.heads = num_heads;
  a.splits = num_splits;
  a.out = out;
  a.out_f32 = out_dtype == SINK_ATTN_F32;
  a.lse = lse_out;
  return hip_status(sa::launch_merge(a, static_cast<hipStream_t>(stream)), "merge launch");
}

namespace {

sink_attn_status check_decode_common(const void* q, const void* k_pages, const void* v_pages,
                                     const int32_t* page_indptr, const int32_t* page_indices,
                                     const int32_t* kv_len, const float* sinks, int32_t batch,
                                     int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t page_size, int32_t max_kv_len, int32_t num_splits,
                                     float sm_scale) {
  if (!q || !k_pages || !v_pages || !page_indptr || !page_indices || !kv_len)
    return fail(SINK_ATTN_ERR_NULL_ARG,
                "decode: q, k_pages, v_pages, page_indptr, page_indices and kv_len are required");
  if (batch <= 0 || max_kv_len < 0 || num_splits < 0)
    return fail(SINK_ATTN_ERR_BAD_SHAPE, "decode: batch=%d max_kv_len=%d num_splits=%d", batch,
                max_kv_len, num_splits);
  sink_attn_status st = check_heads(num_qo_heads, num_kv_heads);
  if (st != SINK_ATTN_OK) return st;
  if (head_dim != kHeadDim)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "decode: head_dim=%d (only 64 is built)", head_dim);
  if (page_size != kPageSize)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "decode: page_size=%d (only 16 is built)", page_size);
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale))
    return fail(SINK_ATTN_ERR_BAD_SHAPE, "decode: sm_scale must be positive and finite");
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16))
    return fail(SINK_ATTN_ERR_MISALIGNED, "decode: q, k_pages and v_pages must be 16-byte aligned");
  if (!aligned(page_indptr, 4) || !aligned(page_indices, 4) || !aligned(kv_len, 4) ||
      (sinks && !aligned(sinks, 4)))
    return fail(SINK_ATTN_ERR_MISALIGNED, "decode: index and sink arrays must be 4-byte aligned");
  return ok();
}

sa::DecodeArgs decode_args(const void* q, const void* k_pages, const void* v_pages,
                           const int32_t* page_indptr, const int32_t* page_indices,
                           const int32_t* kv_len, const float* sinks, int32_t batch,
                           int32_t num_qo_heads, int32_t num_kv_heads, int32_t max_kv_len,
                           int32_t S, float sm_scale) {
  sa::DecodeArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_pages);
  a.v = static_cast<const uint16_t*>(v_pages);
  a.page_indptr = page_indptr;
  a.page_indices = page_indices;
  a.kv_len = kv_len;
  a.sinks = sinks;
  a.batch = batch;
  a.hq = num_qo_heads;
  a.hkv = num_kv_heads;
  a.num_splits = S;
  a.chunk_pages = chunk_pages_for(max_kv_len, S);
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.out = nullptr;
  a.out_f32 = 0;
  a.lse = nullptr;
  a.o_part = nullptr;
  a.lse_part = nullptr;
  a.write_partials = 0;
  return a;
}

}  // namespace

sink_attn_status sink_attn_decode_partial(const void* q, const void* k_pages, const void* v_pages,
                                          const int32_t* page_indptr, const int32_t* page_indices,
                                          const int32_t* kv_len, const float* sinks, int32_t batch,
                                          int32_t num_qo_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t page_size, int32_t max_kv_len,
                                          int32_t num_splits, float sm_scale, float* o_parts,
                                          float* lse_parts, void* stream) {
  sink_attn_status st = check_decode_common(q, k_pages, v_pages, page_indptr, page_indices, kv_len,
                                            sinks, batch, num_qo_heads, num_kv_heads, head_dim,
                                            page_size, max_kv_len, num_splits, sm_scale);
  if (st != SINK_ATTN_OK) return st;
  if (!o_parts || !lse_parts)
    return fail(SINK_ATTN_ERR_NULL_ARG, "decode_partial: o_parts and lse_parts are required");
  if (!aligned(o_parts, 16) || !aligned(lse_parts, 4))
    return fail(SINK_ATTN_ERR_MISALIGNED,
                "decode_partial: o_parts must be 16-byte and lse_parts 4-byte aligned");
  const int32_t S = plan_splits(batch, num_kv_heads, max_kv_len, num_splits);
  sa::DecodeArgs a = decode_args(q, k_pages, v_pages, page_indptr, page_indices, kv_len, sinks,
                                 batch, num_qo_heads, num_kv_heads, max_kv_len, S, sm_scale);
  a.o_part = o_parts;
  a.lse_part = lse_parts;
  a.write_partials = 1;
  return hip_status(sa::launch_decode(a, num_qo_heads / num_kv_heads,
                                      static_cast<hipStream_t>(stream)),
                    "decode_partial launch");
}

}  // extern "C"

namespace sa {
// Every host check of sink_attn_decode except the workspace's.
sink_attn_status decode_arguments_ok(const void* q, const void* k_pages, const void* v_pages,
                                     const int32_t* page_indptr, const int32_t* page_indices,
                                     const int32_t* kv_len, const float* sinks, int32_t batch,
                                     int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t page_size, int32_t max_kv_len, int32_t num_splits,
                                     float sm_scale, const void* out, sink_attn_dtype out_dtype,
                                     const float* lse) {
  sink_attn_status st = check_decode_common(q, k_pages, v_pages, page_indptr, page_indices, kv_len,
                                            sinks, batch, num_qo_heads, num_kv_heads, head_dim,
                                            page_size, max_kv_len, num_splits, sm_scale);
  if (st != SINK_ATTN_OK) return st;
  if (!out) return fail(SINK_ATTN_ERR_NULL_ARG, "decode: out is required");
  if (out_dtype != SINK_ATTN_BF16 && out_dtype != SINK_ATTN_F32)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "decode: unknown out_dtype %d", (int)out_dtype);
  if (!aligned(out, 16) || (lse && !aligned(lse, 4)))
    return fail(SINK_ATTN_ERR_MISALIGNED, "decode: out must be 16-byte and lse 4-byte aligned");
  return ok();
}
}  // namespace sa

extern "C" {

sink_attn_status sink_attn_decode(const void* q, const void* k_pages, const void* v_pages,
                                  const int32_t* page_indptr, const int32_t* page_indices,
                                  const int32_t* kv_len, const float* sinks, int32_t batch,
                                  int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t page_size, int32_t max_kv_len, int32_t num_splits,
                                  float sm_scale, void* out, sink_attn_dtype out_dtype, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  sink_attn_status st = sa::decode_arguments_ok(
      q, k_pages, v_pages, page_indptr, page_indices, kv_len, sinks, batch, num_qo_heads,
      num_kv_heads, head_dim, page_size, max_kv_len, num_splits, sm_scale, out, out_dtype, lse);
  if (st != SINK_ATTN_OK) return st;

  if (auto_uses_balanced(max_kv_len, num_splits))
    return sink_attn_decode_balanced(q, k_pages, v_pages, page_indptr, page_indices, kv_len, sinks,
                                     batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                                     max_kv_len, 0, sm_scale, out, out_dtype, lse, workspace,
                                     workspace_bytes, stream);
  const int32_t S = plan_splits(batch, num_kv_heads, max_kv_len, num_splits);
  const size_t need = sink_attn_decode_workspace_size(batch, num_qo_heads, num_kv_heads, head_dim,
                                                      max_kv_len, num_splits);
  if (need > 0) {
    if (!workspace)
      return fail(SINK_ATTN_ERR_WORKSPACE, "decode: %d splits need a %zu-byte workspace", S, need);
    if (workspace_bytes < need)
      return fail(SINK_ATTN_ERR_WORKSPACE, "decode: workspace of %zu bytes < %zu needed",
                  workspace_bytes, need);
    if (!aligned(workspace, 16))
      return fail(SINK_ATTN_ERR_MISALIGNED, "decode: workspace must be 16-byte aligned");
  }

  sa::DecodeArgs a = decode_args(q, k_pages, v_pages, page_indptr, page_indices, kv_len, sinks,
                                 batch, num_qo_heads, num_kv_heads, max_kv_len, S, sm_scale);
  a.out = out;
  a.out_f32 = out_dtype == SINK_ATTN_F32;
  a.lse = lse;
  if (S > 1) {
    a.o_part = static_cast<float*>(workspace);
    a.lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          (size_t)batch * num_qo_heads * S * head_dim * sizeof(float));
    a.write_partials = 1;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(sa::launch_decode(a, num_qo_heads / num_kv_heads, s), "decode launch");
  if (st != SINK_ATTN_OK || S == 1) return st;

  sa::MergeArgs m;
  m.o_parts = a.o_part;
  m.lse_parts = a.lse_part;
  m.rows = batch;
  m.heads = num_qo_heads;
  m.splits = S;
  m.out = out;
  m.out_f32 = a.out_f32;
  m.lse = lse;
  return hip_status(sa::launch_merge(m, s), "decode merge launch");
}

namespace {

// Validation and argument set-up shared by the three balanced entry points.
// `stage`: 1 = partial pass, 2 = finish, 3 = both.
sink_attn_status balanced_setup(const void* q, const void* k_pages, const void* v_pages,
                                const int32_t* page_indptr, const int32_t* page_indices,
                                const int32_t* kv_len, const float* sinks, int32_t batch,
                                int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t page_size, int32_t max_kv_len, int32_t num_ranges,
                                float sm_scale, void* out, sink_attn_dtype out_dtype, float* lse,
                                void* workspace, size_t workspace_bytes, int stage,
                                sa::BalancedDecodeArgs* a) {
  const char* who = stage == 1 ? "decode_balanced_partial"
                    : stage == 2 ? "decode_balanced_finish" : "decode_balanced";
  if (stage & 1) {
    sink_attn_status st = check_decode_common(q, k_pages, v_pages, page_indptr, page_indices,
                                              kv_len, sinks, batch, num_qo_heads, num_kv_heads,
                                              head_dim, page_size, max_kv_len, 0, sm_scale);
    if (st != SINK_ATTN_OK) return st;
  } else {
    if (!page_indptr) return fail(SINK_ATTN_ERR_NULL_ARG, "%s: page_indptr is required", who);
    if (batch <= 0 || max_kv_len < 0)
      return fail(SINK_ATTN_ERR_BAD_SHAPE, "%s: batch=%d max_kv_len=%d", who, batch, max_kv_len);
    sink_attn_status st = check_heads(num_qo_heads, num_kv_heads);
    if (st != SINK_ATTN_OK) return st;
    if (head_dim != kHeadDim)
      return fail(SINK_ATTN_ERR_UNSUPPORTED, "%s: head_dim=%d (only 64 is built)", who, head_dim);
    if (!aligned(page_indptr, 4) || (sinks && !aligned(sinks, 4)))
      return fail(SINK_ATTN_ERR_MISALIGNED, "%s: index and sink arrays must be 4-byte aligned",
                  who);
  }
  if (num_ranges < 0)
    return fail(SINK_ATTN_ERR_BAD_SHAPE, "%s: num_ranges=%d", who, num_ranges);
  if (!out) return fail(SINK_ATTN_ERR_NULL_ARG, "%s: out is required", who);
  if (out_dtype != SINK_ATTN_BF16 && out_dtype != SINK_ATTN_F32)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "%s: unknown out_dtype %d", who, (int)out_dtype);
  if (!aligned(out, 16) || (lse && !aligned(lse, 4)))
    return fail(SINK_ATTN_ERR_MISALIGNED, "%s: out must be 16-byte and lse 4-byte aligned", who);
  const size_t need = sink_attn_decode_balanced_workspace_size(batch, num_qo_heads, num_kv_heads,
                                                               head_dim, max_kv_len, num_ranges);
  if (!workspace)
    return fail(SINK_ATTN_ERR_WORKSPACE, "%s: needs a %zu-byte workspace", who, need);
  if (workspace_bytes < need)
    return fail(SINK_ATTN_ERR_WORKSPACE, "%s: workspace of %zu bytes < %zu needed", who,
                workspace_bytes, need);
  if (!aligned(workspace, 16))
    return fail(SINK_ATTN_ERR_MISALIGNED, "%s: workspace must be 16-byte aligned", who);

  const RangePlan plan = plan_ranges(batch, num_kv_heads, max_kv_len, num_ranges);
  a->q = static_cast<const uint16_t*>(q);
  a->k = static_cast<const uint16_t*>(k_pages);
  a->v = static_cast<const uint16_t*>(v_pages);
  a->page_indptr = page_indptr;
  a->page_indices = page_indices;
  a->kv_len = kv_len;
  a->sinks = sinks;
  a->batch = batch;
  a->hq = num_qo_heads;
  a->hkv = num_kv_heads;
  a->n_ranges = plan.n_ranges;
  a->min_range_pages = plan.min_pages;
  a->scale_log2 = sm_scale * 1.4426950408889634f;
  a->out = out;
  a->out_f32 = out_dtype == SINK_ATTN_F32;
  a->lse = lse;
  a->o_part = static_cast<float*>(workspace);
  a->lse_part = reinterpret_cast<float*>(
      static_cast<char*>(workspace) +
      balanced_slots(batch, plan.n_ranges) * num_qo_heads * head_dim * sizeof(float));
  a->qkv = nullptr;   // a plain decode; the decode step sets these
  a->bias = nullptr;
  a->table = nullptr;
  a->max_pos = 0;
  a->interleaved = 0;
  a->k_new = nullptr;
  a->v_new = nullptr;
  a->q_new = nullptr;
  return ok();
}

}  // namespace

sink_attn_status sink_attn_decode_balanced_partial(
    const void* q, const void* k_pages, const void* v_pages, const int32_t* page_indptr,
    const int32_t* page_indices, const int32_t* kv_len, const float* sinks, int32_t batch,
    int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
    int32_t max_kv_len, int32_t num_ranges, float sm_scale, void* out, sink_attn_dtype out_dtype,
    float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  sa::BalancedDecodeArgs a;
  sink_attn_status st = balanced_setup(q, k_pages, v_pages, page_indptr, page_indices, kv_len,
                                       sinks, batch, num_qo_heads, num_kv_heads, head_dim,
                                       page_size, max_kv_len, num_ranges, sm_scale, out, out_dtype,
                                       lse, workspace, workspace_bytes, 1, &a);
  if (st != SINK_ATTN_OK) return st;
  return hip_status(sa::launch_decode_balanced(a, num_qo_heads / num_kv_heads,
                                               static_cast<hipStream_t>(stream)),
                    "decode_balanced_partial launch");
}

sink_attn_status sink_attn_decode_balanced_finish(
    const int32_t* page_indptr, const float* sinks, int32_t batch, int32_t num_qo_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t max_kv_len, int32_t num_ranges, void* out,
    sink_attn_dtype out_dtype, float* lse, void* workspace, size_t workspace_bytes,
    void* stream) {
  sa::BalancedDecodeArgs a;
  sink_attn_status st = balanced_setup(nullptr, nullptr, nullptr, page_indptr, nullptr, nullptr,
                                       sinks, batch, num_qo_heads, num_kv_heads, head_dim,
                                       kPageSize, max_kv_len, num_ranges, 1.f, out, out_dtype,
                                       lse, workspace, workspace_bytes, 2, &a);
  if (st != SINK_ATTN_OK) return st;
  return hip_status(sa::launch_decode_finish(a, static_cast<hipStream_t>(stream)),
                    "decode_balanced_finish launch");
}

sink_attn_status sink_attn_decode_balanced(
    const void* q, const void* k_pages, const void* v_pages, const int32_t* page_indptr,
    const int32_t* page_indices, const int32_t* kv_len, const float* sinks, int32_t batch,
    int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
    int32_t max_kv_len, int32_t num_ranges, float sm_scale, void* out, sink_attn_dtype out_dtype,
    float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  sa::BalancedDecodeArgs a;
  sink_attn_status st = balanced_setup(q, k_pages, v_pages, page_indptr, page_indices, kv_len,
                                       sinks, batch, num_qo_heads, num_kv_heads, head_dim,
                                       page_size, max_kv_len, num_ranges, sm_scale, out, out_dtype,
                                       lse, workspace, workspace_bytes, 3, &a);
  if (st != SINK_ATTN_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(sa::launch_decode_balanced(a, num_qo_heads / num_kv_heads, s),
                  "decode_balanced launch");
  if (st != SINK_ATTN_OK) return st;
  return hip_status(sa::launch_decode_finish(a, s), "decode_balanced finish launch");
}

size_t sink_attn_decode_step_workspace_size(int32_t batch, int32_t num_qo_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t max_kv_len) {
  const size_t partials = sink_attn_decode_balanced_workspace_size(batch, num_qo_heads,
                                                                   num_kv_heads, head_dim,
                                                                   max_kv_len, 0);
  if (batch <= 0 || num_qo_heads <= 0 || head_dim != kHeadDim) return partials;
  return align_up(partials, 256) + (size_t)batch * num_qo_heads * head_dim * sizeof(uint16_t);
}

sink_attn_status sink_attn_decode_step(
    const void* qkv, const void* bias, const float* rope_table, int32_t max_pos,
    int32_t interleaved, void* k_pages, void* v_pages, const int32_t* page_indptr,
    const int32_t* page_indices, const int32_t* kv_len, const float* sinks, int32_t batch,
    int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
    int32_t max_kv_len, float sm_scale, void* out, sink_attn_dtype out_dtype, float* lse,
    void* workspace, size_t workspace_bytes, void* stream) {
  if (!qkv || !rope_table)
    return fail(SINK_ATTN_ERR_NULL_ARG, "decode_step: qkv and rope_table are required");
  if (max_pos < 1) return fail(SINK_ATTN_ERR_BAD_SHAPE, "decode_step: max_pos=%d", max_pos);
  if (interleaved != 0 && interleaved != 1)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "decode_step: interleaved must be 0 or 1");
  if ((bias && !aligned(bias, 16)) || !aligned(rope_table, 16))
    return fail(SINK_ATTN_ERR_MISALIGNED, "decode_step: bias and rope_table must be 16-byte aligned");
  // qkv stands in for q in the decode's checks (non-NULL, 16-byte aligned)
  sa::BalancedDecodeArgs a;
  sink_attn_status st = balanced_setup(qkv, k_pages, v_pages, page_indptr, page_indices, kv_len,
                                       sinks, batch, num_qo_heads, num_kv_heads, head_dim,
                                       page_size, max_kv_len, 0, sm_scale, out, out_dtype, lse,
                                       workspace, workspace_bytes, 3, &a);
  if (st != SINK_ATTN_OK) return st;
  const size_t need = sink_attn_decode_step_workspace_size(batch, num_qo_heads, num_kv_heads,
                                                           head_dim, max_kv_len);
  if (workspace_bytes < need)
    return fail(SINK_ATTN_ERR_WORKSPACE, "decode_step: workspace of %zu bytes < %zu needed",
                workspace_bytes, need);
  a.q_new = reinterpret_cast<uint16_t*>(
      static_cast<char*>(workspace) +
      align_up(sink_attn_decode_balanced_workspace_size(batch, num_qo_heads, num_kv_heads,
                                                        head_dim, max_kv_len, 0), 256));
  a.q = a.q_new;
  a.qkv = static_cast<const uint16_t*>(qkv);
  a.bias = static_cast<const uint16_t*>(bias);
  a.table = rope_table;
  a.max_pos = max_pos;
  a.interleaved = interleaved;
  a.k_new = static_cast<uint16_t*>(k_pages);
  a.v_new = static_cast<uint16_t*>(v_pages);
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(sa::launch_decode_balanced(a, num_qo_heads / num_kv_heads, s),
                  "decode_step launch");
  if (st != SINK_ATTN_OK) return st;
  return hip_status(sa::launch_decode_finish(a, s), "decode_step finish launch");
}

namespace {

// Largest draft per request the verification kernel packs: qlen x G
// (token, head) rows in at most four 16-column blocks.
constexpr int32_t kVerifyMaxTokens = 64;   // drafted tokens per request (one mask word)

// Column blocks of 16 (token, head) pairs per workgroup, 1 or 2: two blocks
// keep the kernel at two waves per SIMD, and wider drafts run more column
// groups, whose repeated page reads hit the XCD's L2 (measured faster than
// four blocks at one wave per SIMD for every draft width).
int verify_column_blocks(int32_t columns) {
  return columns <= 16 ? 1 : 2;
}

int32_t verify_column_groups(int32_t columns) {
  const int32_t w = 16 * verify_column_blocks(columns);
  return (columns + w - 1) / w;
}

// Split plan of the verification kernel.  Each chunk of a request re-reads
// its queries, merges its four waves and writes partials that a second
// kernel merges, so splitting only pays when the grid would not fill the
// GPU: one chunk while batch x Hkv x column groups reaches one workgroup
// per CU, else enough chunks for two workgroups per CU, each of at least 16
// pages.  An explicit request is taken as sink_attn_decode takes it.
int64_t verify_target_workgroups() { return 2 * (int64_t)device_cus(); }

// Wide drafts, more than kVerifyTileMinColumns (token, head) pairs per KV
// head, run the tile kernel (verify_tile.hip): 128-row tiles on 32x32 MFMAs
// with each K/V tile staged in LDS once per workgroup, where column groups
// on 16x16 MFMAs would read every page once per group.  Group sizes the
// tile kernel is built for only.
constexpr int32_t kVerifyTileMinColumns = 64;
constexpr int32_t kVerifyTileRows = 128;
constexpr int32_t kVerifyTileKeys = 64;
constexpr int32_t kVerifyTileMaxChunks = 64;
// Automatic chunking of the tile kernel: enough chunks of at least 8 tiles
// (512 keys) for about four (request, KV head, chunk) items per CU
// if every request had max_kv_len keys; each item runs one workgroup
// per 128-row tile.  One item per (request, KV head) lets the longest
// requests bound a ragged batch; chunks cut them at the price of partial
// writes and a merge pass.  Measured on 64 requests (L <= 4,096, 512
// (request, KV head) pairs): 16-token drafts 0.089 ms in one chunk, 0.077
// in two, 0.080 in three; 32-token trees (two row tiles) 0.144, 0.136 and
// 0.139 -- two chunks in both, whatever the row tiles.
int64_t verify_tile_target_items() { return 4 * (int64_t)device_cus(); }
constexpr int32_t kVerifyTileMinChunkTiles = 8;

bool verify_uses_tiles(int32_t group, int32_t columns) {
  return columns > kVerifyTileMinColumns &&
         (group == 1 || group == 2 || group == 4 || group == 8 || group == 16);
}

struct TilePlan {
  int32_t row_tiles, chunk_tiles, chunks;
};

TilePlan verify_tile_plan(int32_t batch, int32_t hkv, int32_t columns, int32_t max_kv_len,
                          int32_t requested) {
  TilePlan tp;
  tp.row_tiles = (columns + kVerifyTileRows - 1) / kVerifyTileRows;
  const int32_t tiles = max_kv_len > 0 ? (max_kv_len + kVerifyTileKeys - 1) / kVerifyTileKeys : 1;
  int64_t want;   // chunks per request of max_kv_len keys
  if (requested > 0) {
    want = requested;
  } else {
    const int64_t pairs = (int64_t)batch * hkv;
    const int64_t target = verify_tile_target_items();
    want = pairs > 0 ? (target + pairs - 1) / pairs : 1;
    const int64_t by_len = tiles / kVerifyTileMinChunkTiles;
    if (want > by_len) want = by_len;
  }
  if (want < 1) want = 1;
  if (want > tiles) want = tiles;
  int32_t ct = (int32_t)((tiles + want - 1) / want);
  const int32_t min_ct = (tiles + kVerifyTileMaxChunks - 1) / kVerifyTileMaxChunks;
  if (ct < min_ct) ct = min_ct;
  tp.chunk_tiles = ct;
  tp.chunks = (tiles + ct - 1) / ct;
  return tp;
}

int32_t verify_plan_splits(int32_t batch, int32_t hkv, int32_t columns, int32_t max_kv_len,
                           int32_t requested, int32_t group) {
  if (verify_uses_tiles(group, columns))
    return verify_tile_plan(batch, hkv, columns, max_kv_len, requested).chunks;
  if (requested > 0) return plan_splits(batch, hkv, max_kv_len, requested);
  const int32_t pages = (max_kv_len + kPageSize - 1) / kPageSize;
  const int64_t units = (int64_t)batch * hkv * verify_column_groups(columns);
  const int64_t target = verify_target_workgroups();
  if (units <= 0 || units * 2 >= target || pages <= 16) return 1;
  int64_t s = (target + units - 1) / units;
  const int64_t max_by_len = (pages + 15) / 16;
  if (s > max_by_len) s = max_by_len;
  if (s > 256) s = 256;
  return s < 1 ? 1 : (int32_t)s;
}

size_t verify_workspace(int32_t total_q, int32_t num_qo_heads, int32_t head_dim, int32_t splits) {
  if (splits <= 1 || total_q <= 0) return 0;
  const size_t rows = (size_t)total_q * num_qo_heads * splits;
  return rows * head_dim * sizeof(float) + ((rows * sizeof(float) + 255) / 256) * 256;
}

}  // namespace

int32_t sink_attn_verify_num_splits(int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                                    int32_t max_qlen, int32_t max_kv_len, int32_t num_splits) {
  if (batch <= 0 || num_qo_heads <= 0 || num_kv_heads <= 0 || num_qo_heads % num_kv_heads ||
      max_qlen < 0 || max_kv_len < 0 || num_splits < 0)
    return 1;
  const int32_t G = num_qo_heads / num_kv_heads;
  return verify_plan_splits(batch, num_kv_heads, max_qlen * G, max_kv_len, num_splits, G);
}

size_t sink_attn_verify_workspace_size(int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t total_q, int32_t max_qlen,
                                       int32_t max_kv_len, int32_t num_splits) {
  if (batch <= 0 || num_qo_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || total_q < 0 ||
      max_qlen < 0 || max_kv_len < 0 || num_splits < 0 || num_qo_heads % num_kv_heads)
    return 0;
  return verify_workspace(total_q, num_qo_heads, head_dim,
                          sink_attn_verify_num_splits(batch, num_qo_heads, num_kv_heads, max_qlen,
                                                      max_kv_len, num_splits));
}

namespace {

sink_attn_status verify_impl(const void* q, const int32_t* qo_indptr, const void* k_pages,
                             const void* v_pages, const int32_t* page_indptr,
                             const int32_t* page_indices, const int32_t* kv_len,
                             const float* sinks, const uint64_t* draft_mask, int32_t batch,
                             int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t page_size, int32_t total_q, int32_t max_qlen,
                             int32_t max_kv_len, int32_t num_splits, float sm_scale, void* out,
                             sink_attn_dtype out_dtype, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  sink_attn_status st = check_decode_common(q, k_pages, v_pages, page_indptr, page_indices, kv_len,
                                            sinks, batch, num_qo_heads, num_kv_heads, head_dim,
                                            page_size, max_kv_len, num_splits, sm_scale);
  if (st != SINK_ATTN_OK) return st;
  if (!qo_indptr || !out)
    return fail(SINK_ATTN_ERR_NULL_ARG, "verify: qo_indptr and out are required");
  if (total_q < 0 || max_qlen < 0 || max_qlen > total_q)
    return fail(SINK_ATTN_ERR_BAD_SHAPE, "verify: total_q=%d max_qlen=%d", total_q, max_qlen);
  const int32_t G = num_qo_heads / num_kv_heads;
  if (max_qlen > kVerifyMaxTokens)
    return fail(SINK_ATTN_ERR_UNSUPPORTED,
                "verify: max_qlen %d exceeds %d drafted tokens (use sink_attn_prefill)", max_qlen,
                kVerifyMaxTokens);
  if (draft_mask && !aligned(draft_mask, 8))
    return fail(SINK_ATTN_ERR_MISALIGNED, "verify: draft_mask must be 8-byte aligned");
  if (out_dtype != SINK_ATTN_BF16 && out_dtype != SINK_ATTN_F32)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "verify: unknown out_dtype %d", (int)out_dtype);
  if (!aligned(out, 16) || (lse && !aligned(lse, 4)) || !aligned(qo_indptr, 4))
    return fail(SINK_ATTN_ERR_MISALIGNED,
                "verify: out must be 16-byte, lse and qo_indptr 4-byte aligned");
  const int32_t S = verify_plan_splits(batch, num_kv_heads, max_qlen * G, max_kv_len, num_splits, G);
  const size_t need = verify_workspace(total_q, num_qo_heads, head_dim, S);
  if (need > 0) {
    if (!workspace)
      return fail(SINK_ATTN_ERR_WORKSPACE, "verify: %d splits need a %zu-byte workspace", S, need);
    if (workspace_bytes < need)
      return fail(SINK_ATTN_ERR_WORKSPACE, "verify: workspace of %zu bytes < %zu needed",
                  workspace_bytes, need);
    if (!aligned(workspace, 16))
      return fail(SINK_ATTN_ERR_MISALIGNED, "verify: workspace must be 16-byte aligned");
  }
  if (total_q == 0 || max_qlen == 0) return ok();

  if (verify_uses_tiles(G, max_qlen * G)) {
    const TilePlan tp = verify_tile_plan(batch, num_kv_heads, max_qlen * G, max_kv_len, num_splits);
    sa::VerifyTileArgs ta;
    ta.q = static_cast<const uint16_t*>(q);
    ta.qo_indptr = qo_indptr;
    ta.k = static_cast<const uint16_t*>(k_pages);
    ta.v = static_cast<const uint16_t*>(v_pages);
    ta.page_indptr = page_indptr;
    ta.page_indices = page_indices;
    ta.kv_len = kv_len;
    ta.sinks = sinks;
    ta.draft_mask = draft_mask;
    ta.batch = batch;
    ta.hq = num_qo_heads;
    ta.hkv = num_kv_heads;
    ta.max_qlen = max_qlen;
    ta.row_tiles = tp.row_tiles;
    ta.chunk_tiles = tp.chunk_tiles;
    ta.max_chunks = tp.chunks;
    ta.scale_log2 = sm_scale * 1.4426950408889634f;
    ta.out = out;
    ta.out_f32 = out_dtype == SINK_ATTN_F32;
    ta.lse = lse;
    ta.o_part = nullptr;
    ta.lse_part = nullptr;
    ta.longest_first = batch <= sa::kLongestFirstMaxBatch;
    if (tp.chunks > 1) {
      ta.o_part = static_cast<float*>(workspace);
      ta.lse_part = reinterpret_cast<float*>(
          static_cast<char*>(workspace) +
          (size_t)total_q * num_qo_heads * tp.chunks * head_dim * sizeof(float));
    }
    return hip_status(sa::launch_verify_tile(ta, G, static_cast<hipStream_t>(stream)),
                      "verify (tiles) launch");
  }

  sa::VerifyArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.qo_indptr = qo_indptr;
  a.k = static_cast<const uint16_t*>(k_pages);
  a.v = static_cast<const uint16_t*>(v_pages);
  a.page_indptr = page_indptr;
  a.page_indices = page_indices;
  a.kv_len = kv_len;
  a.sinks = sinks;
  a.batch = batch;
  a.hq = num_qo_heads;
  a.hkv = num_kv_heads;
  a.num_splits = S;
  a.chunk_pages = chunk_pages_for(max_kv_len, S);
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.out = out;
  a.out_f32 = out_dtype == SINK_ATTN_F32;
  a.lse = lse;
  a.o_part = nullptr;
  a.lse_part = nullptr;
  a.write_partials = 0;
  a.draft_mask = draft_mask;
  const int column_blocks = verify_column_blocks(max_qlen * G);
  a.col_groups = verify_column_groups(max_qlen * G);
  if (S > 1) {
    a.o_part = static_cast<float*>(workspace);
    a.lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          (size_t)total_q * num_qo_heads * S * head_dim * sizeof(float));
    a.write_partials = 1;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(sa::launch_verify(a, G, column_blocks, s), "verify launch");
  if (st != SINK_ATTN_OK || S == 1) return st;
  sa::MergeArgs mg;
  mg.o_parts = a.o_part;
  mg.lse_parts = a.lse_part;
  mg.rows = total_q;
  mg.heads = num_qo_heads;
  mg.splits = S;
  mg.out = out;
  mg.out_f32 = a.out_f32;
  mg.lse = lse;
  return hip_status(sa::launch_merge(mg, s), "verify merge launch");
}

}  // namespace

sink_attn_status sink_attn_verify(const void* q, const int32_t* qo_indptr, const void* k_pages,
                                  const void* v_pages, const int32_t* page_indptr,
                                  const int32_t* page_indices, const int32_t* kv_len,
                                  const float* sinks, int32_t batch, int32_t num_qo_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                  int32_t total_q, int32_t max_qlen, int32_t max_kv_len,
                                  int32_t num_splits, float sm_scale, void* out,
                                  sink_attn_dtype out_dtype, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return verify_impl(q, qo_indptr, k_pages, v_pages, page_indptr, page_indices, kv_len, sinks,
                     nullptr, batch, num_qo_heads, num_kv_heads, head_dim, page_size, total_q,
                     max_qlen, max_kv_len, num_splits, sm_scale, out, out_dtype, lse, workspace,
                     workspace_bytes, stream);
}

sink_attn_status sink_attn_verify_tree(const void* q, const int32_t* qo_indptr,
                                       const uint64_t* draft_mask, const void* k_pages,
                                       const void* v_pages, const int32_t* page_indptr,
                                       const int32_t* page_indices, const int32_t* kv_len,
                                       const float* sinks, int32_t batch, int32_t num_qo_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                       int32_t total_q, int32_t max_qlen, int32_t max_kv_len,
                                       int32_t num_splits, float sm_scale, void* out,
                                       sink_attn_dtype out_dtype, float* lse, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  if (!draft_mask) return fail(SINK_ATTN_ERR_NULL_ARG, "verify_tree: draft_mask is required");
  return verify_impl(q, qo_indptr, k_pages, v_pages, page_indptr, page_indices, kv_len, sinks,
                     draft_mask, batch, num_qo_heads, num_kv_heads, head_dim, page_size, total_q,
                     max_qlen, max_kv_len, num_splits, sm_scale, out, out_dtype, lse, workspace,
                     workspace_bytes, stream);
}

sink_attn_status sink_attn_rope_table(float* table, int32_t max_pos, int32_t head_dim,
                                      double rope_theta, double factor,
                                      int32_t original_max_pos, double beta_fast,
                                      double beta_slow, double attn_factor,
                                      sink_attn_yarn_ramp yarn_ramp, void* stream) {
  if (!table) return fail(SINK_ATTN_ERR_NULL_ARG, "rope_table: table is required");
  if (max_pos < 1) return fail(SINK_ATTN_ERR_BAD_SHAPE, "rope_table: max_pos=%d", max_pos);
  if (head_dim != kHeadDim)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "rope_table: head_dim %d (only 64)", head_dim);
  if (!(rope_theta > 1.0) || !(factor > 0.0) || !(attn_factor >= 0.0) ||
      !std::isfinite(rope_theta) || !std::isfinite(factor) || !std::isfinite(attn_factor))
    return fail(SINK_ATTN_ERR_BAD_SHAPE, "rope_table: theta=%g factor=%g attn_factor=%g",
                rope_theta, factor, attn_factor);
  if (factor > 1.0 && (original_max_pos < 1 || !(beta_slow > 0.0) || !(beta_fast > beta_slow) ||
                       !std::isfinite(beta_fast)))
    return fail(SINK_ATTN_ERR_BAD_SHAPE,
                "rope_table: YaRN needs original_max_pos >= 1 and 0 < beta_slow < beta_fast "
                "(got %d, %g, %g)", original_max_pos, beta_slow, beta_fast);
  if (yarn_ramp != SINK_ATTN_YARN_RAMP_TURNS && yarn_ramp != SINK_ATTN_YARN_RAMP_PAIRS)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "rope_table: unknown yarn_ramp %d", (int)yarn_ramp);
  if (!aligned(table, 16)) return fail(SINK_ATTN_ERR_MISALIGNED, "rope_table: table must be 16-byte aligned");
  sa::RopeTableArgs a;
  a.table = table;
  a.max_pos = max_pos;
  a.original_max_pos = original_max_pos;
  a.base = rope_theta;
  a.factor = factor;
  a.beta_fast = beta_fast;
  a.beta_slow = beta_slow;
  a.temperature = attn_factor > 0.0 ? attn_factor : (factor > 1.0 ? 0.1 * std::log(factor) + 1.0 : 1.0);
  a.pair_ramp = yarn_ramp == SINK_ATTN_YARN_RAMP_PAIRS ? 1 : 0;
  if (a.pair_ramp && factor > 1.0) {
    // the rounded pairs that turn beta_fast and beta_slow times in L
    auto pair_of = [&](double turns) {
      return kHeadDim * std::log(original_max_pos / (6.283185307179586 * turns)) /
             (2.0 * std::log(rope_theta));
    };
    a.ramp_low = std::max(std::floor(pair_of(beta_fast)), 0.0);
    a.ramp_high = std::min(std::ceil(pair_of(beta_slow)), kHeadDim / 2 - 1.0);
  } else {
    a.ramp_low = a.ramp_high = 0.0;
  }
  return hip_status(sa::launch_rope_table(a, static_cast<hipStream_t>(stream)), "rope_table launch");
}

}  // extern "C"

namespace {

// Host checks and launch arguments of the append (kv_only: the key and
// value heads only, q_out unused); nothing is launched.
sink_attn_status append_check(const void* qkv, const void* bias, const float* rope_table,
                              int32_t max_pos, const int32_t* qo_indptr, const int32_t* kv_len,
                              const int32_t* page_indptr, const int32_t* page_indices,
                              int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t page_size, int32_t total_q,
                              int32_t interleaved, void* q_out, void* k_pages, void* v_pages,
                              int32_t kv_only, sa::RopeAppendArgs* a) {
  const char* who = kv_only ? "prefill_step" : "qkv_rope_append";
  if (!qkv || !rope_table || !qo_indptr || !kv_len || !page_indptr || !page_indices ||
      (!q_out && !kv_only) || !k_pages || !v_pages)
    return fail(SINK_ATTN_ERR_NULL_ARG, "%s: only bias may be NULL", who);
  if (batch < 1 || num_qo_heads < 1 || num_kv_heads < 1 || total_q < 0 || max_pos < 1)
    return fail(SINK_ATTN_ERR_BAD_SHAPE, "%s: batch=%d Hq=%d Hkv=%d total_q=%d max_pos=%d", who,
                batch, num_qo_heads, num_kv_heads, total_q, max_pos);
  if (head_dim != kHeadDim || page_size != kPageSize)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "%s: head_dim %d, page_size %d (only 64, 16)", who,
                head_dim, page_size);
  if (interleaved != 0 && interleaved != 1)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "%s: interleaved must be 0 or 1", who);
  if ((int64_t)total_q * 256 > 0xFFFFFFFFll || num_qo_heads + 2 * num_kv_heads > 65535 * 32)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "%s: grid too large", who);
  if (!aligned(qkv, 16) || (bias && !aligned(bias, 16)) || !aligned(rope_table, 16) ||
      (q_out && !aligned(q_out, 16)) || !aligned(k_pages, 16) || !aligned(v_pages, 16) ||
      !aligned(qo_indptr, 4) || !aligned(kv_len, 4) || !aligned(page_indptr, 4) ||
      !aligned(page_indices, 4))
    return fail(SINK_ATTN_ERR_MISALIGNED,
                "%s: tensors must be 16-byte, index arrays 4-byte aligned", who);
  a->qkv = static_cast<const uint16_t*>(qkv);
  a->bias = static_cast<const uint16_t*>(bias);
  a->table = rope_table;
  a->max_pos = max_pos;
  a->qo_indptr = qo_indptr;
  a->kv_len = kv_len;
  a->page_indptr = page_indptr;
  a->page_indices = page_indices;
  a->batch = batch;
  a->hq = num_qo_heads;
  a->hkv = num_kv_heads;
  a->total_q = total_q;
  a->interleaved = interleaved;
  a->kv_only = kv_only;
  a->q_out = static_cast<uint16_t*>(q_out);
  a->k_pages = static_cast<uint16_t*>(k_pages);
  a->v_pages = static_cast<uint16_t*>(v_pages);
  return ok();
}

}  // namespace

extern "C" {

sink_attn_status sink_attn_qkv_rope_append(const void* qkv, const void* bias,
                                           const float* rope_table, int32_t max_pos,
                                           const int32_t* qo_indptr, const int32_t* kv_len,
                                           const int32_t* page_indptr,
                                           const int32_t* page_indices, int32_t batch,
                                           int32_t num_qo_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t page_size, int32_t total_q,
                                           int32_t interleaved, void* q_out, void* k_pages,
                                           void* v_pages, void* stream) {
  sa::RopeAppendArgs a;
  sink_attn_status st = append_check(qkv, bias, rope_table, max_pos, qo_indptr, kv_len,
                                     page_indptr, page_indices, batch, num_qo_heads,
                                     num_kv_heads, head_dim, page_size, total_q, interleaved,
                                     q_out, k_pages, v_pages, 0, &a);
  if (st != SINK_ATTN_OK || total_q == 0) return st;
  return hip_status(sa::launch_rope_append(a, static_cast<hipStream_t>(stream)),
                    "qkv_rope_append launch");
}

sink_attn_status sink_attn_prefill_step(
    const void* qkv, const void* bias, const float* rope_table, int32_t max_pos,
    int32_t interleaved, const int32_t* qo_indptr, void* k_pages, void* v_pages,
    const int32_t* page_indptr, const int32_t* page_indices, const int32_t* kv_len,
    const float* sinks, int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t page_size, int32_t total_q, int32_t max_qlen, int32_t max_kv_len,
    float sm_scale, int32_t causal, void* out, sink_attn_dtype out_dtype, float* lse,
    void* stream) {
  // every check of both kernels before either is launched
  sa::RopeAppendArgs ap;
  sink_attn_status st = append_check(qkv, bias, rope_table, max_pos, qo_indptr, kv_len,
                                     page_indptr, page_indices, batch, num_qo_heads,
                                     num_kv_heads, head_dim, page_size, total_q, interleaved,
                                     nullptr, k_pages, v_pages, 1, &ap);
  if (st != SINK_ATTN_OK) return st;
  const PrefillStepInputs step = {qkv, bias, rope_table, max_pos, interleaved};
  sa::PrefillArgs a;
  bool empty = false;
  st = prefill_check(nullptr, qo_indptr, k_pages, v_pages, page_indptr, page_indices, kv_len,
                     sinks, batch, num_qo_heads, num_kv_heads, head_dim, page_size, total_q,
                     max_qlen, max_kv_len, sm_scale, causal, out, out_dtype, lse, &step, &a,
                     &empty);
  if (st != SINK_ATTN_OK || total_q == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(sa::launch_rope_append(ap, s), "prefill_step append launch");
  if (st != SINK_ATTN_OK || empty) return st;
  return hip_status(sa::launch_prefill(a, num_qo_heads / num_kv_heads, s),
                    "prefill_step launch");
}

}  // extern "C"
