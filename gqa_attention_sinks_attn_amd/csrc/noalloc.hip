// sink_attn_decode for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the same
// call with the workspace taken from a fixed device array of this library
// instead of a caller's buffer.  Nothing here allocates: the array is a
// file-scope __device__ object that each GPU holds from the library's
// loading until the process ends.
#include "sink_attn.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

namespace sa {
sink_attn_status api_fail(sink_attn_status s, const char* detail);
sink_attn_status decode_arguments_ok(const void* q, const void* k_pages, const void* v_pages,
                                     const int32_t* page_indptr, const int32_t* page_indices,
                                     const int32_t* kv_len, const float* sinks, int32_t batch,
                                     int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t page_size, int32_t max_kv_len, int32_t num_splits,
                                     float sm_scale, const void* out, sink_attn_dtype out_dtype,
                                     const float* lse);
}

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;   // 16 MiB per GPU
constexpr int kMaxDevices = 64;

// The scratch array.  In host code its name stands for a host-side shadow,
// not a device address: only the pointer obtained from hipGetSymbolAddress
// below is ever passed to a kernel.
__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];

// Device address of this GPU's copy of the array, looked up once per device
// on the first call made with that device current.
hipError_t scratch_of(int dev, void** ptr) {
  std::call_once(g_once[dev], [dev]() {
    void* p = nullptr;
    g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_status[dev] == hipSuccess ? p : nullptr;
    if (g_status[dev] != hipSuccess) (void)hipGetLastError();
  });
  *ptr = g_scratch[dev];
  return g_status[dev];
}

}  // namespace

extern "C" sink_attn_status sink_attn_decode_noalloc(
    const void* q, const void* k_pages, const void* v_pages, const int32_t* page_indptr,
    const int32_t* page_indices, const int32_t* kv_len, const float* sinks, int32_t batch,
    int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
    int32_t max_kv_len, int32_t num_splits, float sm_scale, void* out, sink_attn_dtype out_dtype,
    float* lse, void* stream) {
  char msg[256];
  const sink_attn_status st = sa::decode_arguments_ok(
      q, k_pages, v_pages, page_indptr, page_indices, kv_len, sinks, batch, num_qo_heads,
      num_kv_heads, head_dim, page_size, max_kv_len, num_splits, sm_scale, out, out_dtype, lse);
  if (st != SINK_ATTN_OK) return st;
  const size_t need = sink_attn_decode_workspace_size(batch, num_qo_heads, num_kv_heads, head_dim,
                                                      max_kv_len, num_splits);
  if (need > kScratchBytes) {
    snprintf(msg, sizeof msg,
             "decode_noalloc: these sizes need a %zu-byte workspace; the static scratch holds "
             "%zu bytes (use sink_attn_decode with a workspace)",
             need, kScratchBytes);
    return sa::api_fail(SINK_ATTN_ERR_WORKSPACE, msg);
  }
  void* ws = nullptr;
  if (need > 0) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
      (void)hipGetLastError();
      snprintf(msg, sizeof msg, "decode_noalloc: no usable current device (%s)",
               hipGetErrorString(e));
      return sa::api_fail(SINK_ATTN_ERR_HIP, msg);
    }
    e = scratch_of(dev, &ws);
    if (e != hipSuccess || ws == nullptr) {
      snprintf(msg, sizeof msg, "decode_noalloc: hipGetSymbolAddress of the scratch array: %s",
               hipGetErrorString(e));
      return sa::api_fail(SINK_ATTN_ERR_HIP, msg);
    }
  }
  return sink_attn_decode(q, k_pages, v_pages, page_indptr, page_indices, kv_len, sinks, batch,
                          num_qo_heads, num_kv_heads, head_dim, page_size, max_kv_len, num_splits,
                          sm_scale, out, out_dtype, lse, ws, need > 0 ? kScratchBytes : 0, stream);
}
