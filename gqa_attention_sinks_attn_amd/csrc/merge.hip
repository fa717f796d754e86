// Log-sum-exp merge of split-KV partials (gfx950).
//
// GPT-OSS on Day 0 (Perplexity), "Sink attention" under "Kernels for
// GPT-OSS": attention is split into chunks along the KV length and the sink
// sits in the first chunk only, so recombining the chunks is the plain
// weighted merge of normalised partials: L = max lse_c, w_c = e^(lse_c - L),
// o = sum w_c o_c / sum w_c, lse = L + ln sum w_c.  No sink is added here.
//
// One wave per (row, head); lane = output dim (head_dim 64).  The S
// log-sum-exps are read once per wave, the partial outputs as one coalesced
// 256-byte row per chunk.
#include "common.hpp"
#include "launch.hpp"

namespace sa {
namespace {

constexpr int kD = 64;

__global__ __launch_bounds__(256) void merge_kernel(MergeArgs p) {
  const int lane = thread_x() & 63;
  const int64_t pair = (int64_t)block_x() * 4 + (thread_x() >> 6);
  const int64_t n_pairs = (int64_t)p.rows * p.heads;
  if (pair >= n_pairs) return;
  const int S = p.splits;
  const float* ls = p.lse_parts + pair * S;
  const float* os = p.o_parts + pair * S * kD + lane;

  float L = -INFINITY;
  for (int c = 0; c < S; ++c) L = fmaxf(L, ls[c]);

  float den = 0.f, acc = 0.f;
  if (L != -INFINITY) {
    for (int c = 0; c < S; ++c) {
      const float lc = ls[c];
      float w;
      if (L == INFINITY) w = (lc == INFINITY) ? 1.f : 0.f;
      else w = __expf(lc - L);
      den += w;
      acc += (w != 0.f) ? w * os[(int64_t)c * kD] : 0.f;
    }
  }
  const float o = den > 0.f ? acc / den : 0.f;
  float lse;
  if (L == -INFINITY) lse = -INFINITY;
  else if (L == INFINITY) lse = INFINITY;
  else lse = L + __logf(den);

  const int64_t dst = pair * kD + lane;
  if (p.out_f32) reinterpret_cast<float*>(p.out)[dst] = o;
  else reinterpret_cast<uint16_t*>(p.out)[dst] = float_to_bf16_bits(o);
  if (p.lse != nullptr && lane == 0) p.lse[pair] = lse;
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const int64_t pairs = (int64_t)a.rows * a.heads;
  if (pairs == 0) return hipSuccess;
  dim3 grid((unsigned)((pairs + 3) / 4));
  hipLaunchKernelGGL(merge_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sa
