/* A plain C99 program that runs the library on the GPU with no Python in
 * the process (built and run by tests/test_gpu_c_consumer.py): device
 * memory and copies through the HIP runtime's C API, a causal paged prefill
 * (sink_attn_prefill) and a paged decode (sink_attn_decode, automatic plan)
 * over the same cache, each compared with the fp64 oracle (the test
 * infrastructure's C library, oracle/sink_attn_oracle.c) at the parity bar:
 * max-abs <= 1e-2 and relative L2 <= 5e-3 on fp32 outputs, LSE within 5e-3.
 *
 * The inputs are bf16 values of a fixed linear congruential sequence
 * (uniform in [-2, 2)), pages permuted by a fixed stride, and N(0,1)-sized
 * sinks of the same sequence.  Exit status 0 when both calls pass. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sink_attn.h"

/* the oracle's entry point (oracle/sink_attn_oracle.c) */
int sa_oracle_attend(const uint16_t* q, const int32_t* qo_indptr, const uint16_t* k,
                     const uint16_t* v, const int32_t* kv_indptr, const int32_t* page_indices,
                     const int32_t* kv_len, const float* sinks, int batch, int hq, int hkv, int d,
                     int page_size, double sm_scale, int causal, const uint64_t* draft_mask,
                     double* out, double* lse, int nthreads);

enum { B = 3, HQ = 16, HKV = 2, D = 64, PS = 16 };

static uint32_t lcg_state = 12345u;
static float next_uniform(void) {   /* [-2, 2) */
  lcg_state = lcg_state * 1664525u + 1013904223u;
  return (float)(lcg_state >> 8) * (4.0f / 16777216.0f) - 2.0f;
}

static uint16_t to_bf16(float x) {   /* round to nearest, ties to even */
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

#define HIP_CHECK(call)                                                            \
  do {                                                                             \
    hipError_t e_ = (call);                                                        \
    if (e_ != hipSuccess) {                                                        \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));           \
      return 2;                                                                    \
    }                                                                              \
  } while (0)

static void* upload(const void* host, size_t bytes) {
  void* dev = NULL;
  if (hipMalloc(&dev, bytes > 0 ? bytes : 16) != hipSuccess) return NULL;
  if (bytes > 0 && hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return dev;
}

/* max-abs and relative L2 of got (fp32) against ref (fp64); LSE error */
static int compare(const char* name, const float* got, const double* ref, size_t n,
                   const float* got_lse, const double* ref_lse, size_t n_lse) {
  double max_abs = 0.0, num = 0.0, den = 0.0, lse_err = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double e = fabs((double)got[i] - ref[i]);
    if (!(e <= max_abs)) max_abs = e;   /* also catches NaN */
    num += e * e;
    den += ref[i] * ref[i];
  }
  for (size_t i = 0; i < n_lse; ++i) {
    const double e = fabs((double)got_lse[i] - ref_lse[i]);
    if (!(e <= lse_err)) lse_err = e;
  }
  const double rel = den > 0.0 ? sqrt(num / den) : sqrt(num);
  printf("[c consumer] %s: %zu values, max_abs=%.3e rel_l2=%.3e lse_err=%.3e\n", name, n, max_abs,
         rel, lse_err);
  return max_abs <= 1e-2 && rel <= 5e-3 && lse_err <= 5e-3 ? 0 : 1;
}

int main(void) {
  const int32_t qlens[B] = {37, 1, 130};
  const int32_t kv_len[B] = {100, 1, 300};
  int32_t qo_indptr[B + 1] = {0}, page_indptr[B + 1] = {0};
  for (int b = 0; b < B; ++b) {
    qo_indptr[b + 1] = qo_indptr[b] + qlens[b];
    page_indptr[b + 1] = page_indptr[b] + (kv_len[b] + PS - 1) / PS;
  }
  const int total_q = qo_indptr[B], n_pages = page_indptr[B];
  int32_t* page_indices = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_pages);
  for (int i = 0; i < n_pages; ++i) page_indices[i] = (i * 7 + 3) % n_pages;   /* 7 is coprime to 27 */

  const size_t q_elems = (size_t)total_q * HQ * D, kv_elems = (size_t)n_pages * HKV * PS * D;
  uint16_t* q = (uint16_t*)malloc(q_elems * 2);
  uint16_t* k = (uint16_t*)malloc(kv_elems * 2);
  uint16_t* v = (uint16_t*)malloc(kv_elems * 2);
  float sinks[HQ];
  for (size_t i = 0; i < q_elems; ++i) q[i] = to_bf16(next_uniform());
  for (size_t i = 0; i < kv_elems; ++i) k[i] = to_bf16(next_uniform());
  for (size_t i = 0; i < kv_elems; ++i) v[i] = to_bf16(next_uniform());
  for (int h = 0; h < HQ; ++h) sinks[h] = next_uniform();

  int n_dev = 0;
  HIP_CHECK(hipGetDeviceCount(&n_dev));
  if (n_dev < 1) {
    fprintf(stderr, "no GPU\n");
    return 2;
  }
  void* d_q = upload(q, q_elems * 2);
  void* d_k = upload(k, kv_elems * 2);
  void* d_v = upload(v, kv_elems * 2);
  void* d_qo = upload(qo_indptr, sizeof qo_indptr);
  void* d_pi = upload(page_indptr, sizeof page_indptr);
  void* d_idx = upload(page_indices, sizeof(int32_t) * (size_t)n_pages);
  void* d_len = upload(kv_len, sizeof kv_len);
  void* d_sinks = upload(sinks, sizeof sinks);
  void *d_out = NULL, *d_lse = NULL;
  HIP_CHECK(hipMalloc(&d_out, q_elems * sizeof(float)));
  HIP_CHECK(hipMalloc(&d_lse, (size_t)total_q * HQ * sizeof(float)));
  if (!d_q || !d_k || !d_v || !d_qo || !d_pi || !d_idx || !d_len || !d_sinks) {
    fprintf(stderr, "device upload failed\n");
    return 2;
  }
  const float scale = 0.125f;
  float* out = (float*)malloc(q_elems * sizeof(float));
  float* lse = (float*)malloc((size_t)total_q * HQ * sizeof(float));
  double* ref = (double*)malloc(q_elems * sizeof(double));
  double* ref_lse = (double*)malloc((size_t)total_q * HQ * sizeof(double));
  int failed = 0;

  /* 1. causal paged prefill of every request's new tokens */
  sink_attn_status st = sink_attn_prefill(d_q, (const int32_t*)d_qo, d_k, d_v,
                                          (const int32_t*)d_pi, (const int32_t*)d_idx,
                                          (const int32_t*)d_len, (const float*)d_sinks, B, HQ, HKV,
                                          D, PS, total_q, 130, 300, scale, 1, d_out, SINK_ATTN_F32,
                                          (float*)d_lse, NULL);
  if (st != SINK_ATTN_OK) {
    fprintf(stderr, "prefill: %s (%s)\n", sink_attn_status_string(st), sink_attn_last_error());
    return 2;
  }
  HIP_CHECK(hipDeviceSynchronize());
  HIP_CHECK(hipMemcpy(out, d_out, q_elems * sizeof(float), hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(lse, d_lse, (size_t)total_q * HQ * sizeof(float), hipMemcpyDeviceToHost));
  if (sa_oracle_attend(q, qo_indptr, k, v, page_indptr, page_indices, kv_len, sinks, B, HQ, HKV, D,
                       PS, scale, 1, NULL, ref, ref_lse, 0) != 0) {
    fprintf(stderr, "oracle failed\n");
    return 2;
  }
  failed |= compare("paged causal prefill", out, ref, q_elems, lse, ref_lse, (size_t)total_q * HQ);

  /* 2. decode of each request's last token over the same cache */
  int32_t dq_indptr[B + 1];
  for (int b = 0; b <= B; ++b) dq_indptr[b] = b;
  uint16_t* dq = (uint16_t*)malloc((size_t)B * HQ * D * 2);
  for (int b = 0; b < B; ++b)
    memcpy(dq + (size_t)b * HQ * D, q + (size_t)(qo_indptr[b + 1] - 1) * HQ * D, HQ * D * 2);
  void* d_dq = upload(dq, (size_t)B * HQ * D * 2);
  const size_t ws_bytes = sink_attn_decode_workspace_size(B, HQ, HKV, D, 300, 0);
  void* d_ws = NULL;
  if (ws_bytes > 0) HIP_CHECK(hipMalloc(&d_ws, ws_bytes));
  st = sink_attn_decode(d_dq, d_k, d_v, (const int32_t*)d_pi, (const int32_t*)d_idx,
                        (const int32_t*)d_len, (const float*)d_sinks, B, HQ, HKV, D, PS, 300, 0,
                        scale, d_out, SINK_ATTN_F32, (float*)d_lse, d_ws, ws_bytes, NULL);
  if (st != SINK_ATTN_OK) {
    fprintf(stderr, "decode: %s (%s)\n", sink_attn_status_string(st), sink_attn_last_error());
    return 2;
  }
  HIP_CHECK(hipDeviceSynchronize());
  HIP_CHECK(hipMemcpy(out, d_out, (size_t)B * HQ * D * sizeof(float), hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(lse, d_lse, (size_t)B * HQ * sizeof(float), hipMemcpyDeviceToHost));
  if (sa_oracle_attend(dq, dq_indptr, k, v, page_indptr, page_indices, kv_len, sinks, B, HQ, HKV, D,
                       PS, scale, 1, NULL, ref, ref_lse, 0) != 0) {
    fprintf(stderr, "oracle failed\n");
    return 2;
  }
  failed |= compare("paged decode", out, ref, (size_t)B * HQ * D, lse, ref_lse, (size_t)B * HQ);

  hipFree(d_q); hipFree(d_k); hipFree(d_v); hipFree(d_qo); hipFree(d_pi); hipFree(d_idx);
  hipFree(d_len); hipFree(d_sinks); hipFree(d_out); hipFree(d_lse); hipFree(d_dq);
  if (d_ws) hipFree(d_ws);
  free(q); free(k); free(v); free(dq); free(out); free(lse); free(ref); free(ref_lse);
  free(page_indices);
  printf("[c consumer] %s\n", failed ? "FAILED" : "ok");
  return failed;
}
