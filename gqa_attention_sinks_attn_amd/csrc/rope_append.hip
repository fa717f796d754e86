// The step that feeds the attention path: QKV projection bias, YaRN rotary
// position encoding, and the append of the new tokens' keys and values to
// the paged cache (gfx950).
//
// GPT-OSS on Day 0 (Perplexity), "Attention: GQA with attention sinks": the
// model's QKV projections carry a bias and its positions are encoded with
// YaRN.  The page gives no formula; YaRN is taken as published (Peng et al.
// 2023): per pair d the base frequency base^(-2d/D) is kept when the pair
// turns more than beta_fast times within the original context length L,
// divided by the scale factor s when it turns fewer than beta_slow times, and
// blended linearly between the two, in the turn count (the paper's formula)
// or in the pair index between the rounded bounds (DeepSeek-V3's code, which
// the page names); q and k are both multiplied by the temperature
// 0.1 ln s + 1.  "Accelerating Sonar Through
// Speculation" (Perplexity), "Inference with Speculative Decoding": the
// scheduler reserves room for the next tokens in the paged cache before the
// step runs; token t of a request with qlen new tokens and kv_len keys
// (counting the new ones) sits at position kv_len - qlen + t.
//
// rope_table_kernel: one thread per (position, pair); frequency, angle and
// sin/cos in fp64 (positions reach 10^5 and more, where an fp32 angle would
// be off by ~1e-2 rad), stored as fp32 times the temperature.
//
// rope_append_kernel: HBM-bound elementwise work.  One workgroup = four
// consecutive tokens x 32 heads, eight lanes per head; each lane moves 16
// bytes of the head per token (half pairing: dims 4j..4j+3 and
// 32+4j..32+4j+3; interleaved: 8j..8j+7), and issues the loads of all four
// tokens before the first store, so enough bytes are in flight to cover HBM
// latency.  It adds the bias, rotates query and key heads with the token's
// cos/sin row, rounds to bf16 and stores: queries to q_out, keys and values
// to their page slot.  Tokens whose position lies outside the table or the
// request's reserved pages are skipped whole.
#include "common.hpp"
#include "launch.hpp"

namespace sa {
namespace {

constexpr int kD = 64;
constexpr int kHalf = 32;
constexpr int kPage = 16;
constexpr int kHeadsPerBlock = 32;
constexpr int kRowsPerBlock = 4;       // tokens per workgroup, loads issued together
constexpr double kTwoPi = 6.283185307179586;

__global__ __launch_bounds__(256) void rope_table_kernel(RopeTableArgs a) {
  const int64_t i = (int64_t)block_x() * 256 + thread_x();
  if (i >= (int64_t)a.max_pos * kHalf) return;
  const int p = (int)(i / kHalf);
  const int d = (int)(i % kHalf);
  const double theta = pow(a.base, -2.0 * d / kD);
  double f = theta;
  if (a.factor > 1.0) {
    double keep;   // 1: keep theta, 0: theta / factor
    if (a.pair_ramp) {
      // linear in the pair index between the rounded correction pairs
      if (a.ramp_high <= a.ramp_low) keep = d <= a.ramp_low ? 1.0 : 0.0;
      else keep = fmin(fmax(1.0 - (d - a.ramp_low) / (a.ramp_high - a.ramp_low), 0.0), 1.0);
    } else {
      const double turns = a.original_max_pos * theta / kTwoPi;   // L / wavelength
      if (turns < a.beta_slow) keep = 0.0;
      else if (turns > a.beta_fast) keep = 1.0;
      else keep = (turns - a.beta_slow) / (a.beta_fast - a.beta_slow);
    }
    f = (1.0 - keep) * theta / a.factor + keep * theta;
  }
  const double angle = (double)p * f;
  const double s = sin(angle), c = cos(angle);
  a.table[(int64_t)p * kD + d] = (float)(a.temperature * c);
  a.table[(int64_t)p * kD + kHalf + d] = (float)(a.temperature * s);
}

__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

// Per-token values every lane of the workgroup shares.
struct TokenSlot {
  int row;       // token row, or -1 when the token is skipped
  int pos;       // position in the request
  int page;      // cache page of that position (first page id when not needed)
};

__global__ __launch_bounds__(256) void rope_append_kernel(RopeAppendArgs a) {
  const int row0 = block_x() * kRowsPerBlock;
  // request of the first row: last b with qo_indptr[b] <= row0 (uniform)
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(a.qo_indptr[mid]) <= row0) lo = mid; else hi = mid - 1;
  }
  int b = lo;

  TokenSlot tok[kRowsPerBlock];
#pragma unroll
  for (int r = 0; r < kRowsPerBlock; ++r) {
    const int row = row0 + r;
    tok[r].row = -1;
    tok[r].pos = 0;
    tok[r].page = 0;
    if (row >= a.total_q) continue;
    while (b + 1 < a.batch && __builtin_amdgcn_readfirstlane(a.qo_indptr[b + 1]) <= row) ++b;
    const int q0 = __builtin_amdgcn_readfirstlane(a.qo_indptr[b]);
    const int qlen = __builtin_amdgcn_readfirstlane(a.qo_indptr[b + 1]) - q0;
    const int pos = __builtin_amdgcn_readfirstlane(a.kv_len[b]) - qlen + (row - q0);
    const int pg0 = __builtin_amdgcn_readfirstlane(a.page_indptr[b]);
    const int n_pages = __builtin_amdgcn_readfirstlane(a.page_indptr[b + 1]) - pg0;
    if (pos < 0 || pos >= a.max_pos || pos / kPage >= n_pages) continue;   // caller error: skip
    tok[r].row = row;
    tok[r].pos = pos;
    tok[r].page = __builtin_amdgcn_readfirstlane(a.page_indices[pg0 + pos / kPage]);
  }

  const int H = a.hq + 2 * a.hkv;
  const int h = (a.kv_only ? a.hq : 0) + block_y() * kHeadsPerBlock + (thread_x() >> 3);
  if (h >= H) return;
  const int j = thread_x() & 7;
  const bool rotated = h < a.hq + a.hkv;
  const bool is_q = h < a.hq;
  const bool is_k = !is_q && rotated;
  const int g = is_q ? 0 : (is_k ? h - a.hq : h - a.hq - a.hkv);
  uint16_t* cache = is_k ? a.k_pages : a.v_pages;
  // this lane's two 8-byte pieces: (off0, off1) within the head
  const int off0 = a.interleaved ? 8 * j : 4 * j;
  const int off1 = a.interleaved ? 8 * j + 4 : kHalf + 4 * j;

  float bl[4] = {0.f, 0.f, 0.f, 0.f}, bh[4] = {0.f, 0.f, 0.f, 0.f};
  if (a.bias != nullptr) {
    const uint16_t* bsrc = a.bias + (int64_t)h * kD;
    const u32x2 w0 = ld8(bsrc + off0), w1 = ld8(bsrc + off1);
    bl[0] = lo_bf16(w0[0]); bl[1] = hi_bf16(w0[0]); bl[2] = lo_bf16(w0[1]); bl[3] = hi_bf16(w0[1]);
    bh[0] = lo_bf16(w1[0]); bh[1] = hi_bf16(w1[0]); bh[2] = lo_bf16(w1[1]); bh[3] = hi_bf16(w1[1]);
  }

  // every load of the workgroup's tokens first, then the arithmetic and stores
  u32x2 x0[kRowsPerBlock], x1[kRowsPerBlock];
  f32x4 cv[kRowsPerBlock], sv[kRowsPerBlock];
#pragma unroll
  for (int r = 0; r < kRowsPerBlock; ++r) {
    if (tok[r].row < 0) continue;
    const uint16_t* src = a.qkv + ((int64_t)tok[r].row * H + h) * kD;
    x0[r] = ld8(src + off0);
    x1[r] = ld8(src + off1);
    if (rotated) {
      const float* cs = a.table + (int64_t)tok[r].pos * kD + 4 * j;
      cv[r] = *reinterpret_cast<const f32x4*>(cs);
      sv[r] = *reinterpret_cast<const f32x4*>(cs + kHalf);
    }
  }
#pragma unroll
  for (int r = 0; r < kRowsPerBlock; ++r) {
    if (tok[r].row < 0) continue;
    // (u[i], v[i]) is rotated pair i of the lane: interleaved pairs are
    // adjacent dims, half pairs are dims 4j+i and 32+4j+i
    float u[4], v[4];
    {
      const float p0[4] = {lo_bf16(x0[r][0]) + bl[0], hi_bf16(x0[r][0]) + bl[1],
                           lo_bf16(x0[r][1]) + bl[2], hi_bf16(x0[r][1]) + bl[3]};
      const float p1[4] = {lo_bf16(x1[r][0]) + bh[0], hi_bf16(x1[r][0]) + bh[1],
                           lo_bf16(x1[r][1]) + bh[2], hi_bf16(x1[r][1]) + bh[3]};
      if (a.interleaved) {
        u[0] = p0[0]; v[0] = p0[1]; u[1] = p0[2]; v[1] = p0[3];
        u[2] = p1[0]; v[2] = p1[1]; u[3] = p1[2]; v[3] = p1[3];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) { u[i] = p0[i]; v[i] = p1[i]; }
      }
    }
    if (rotated) {
#pragma unroll
      for (int i = 0; i < 4; ++i) rotate_pair(u[i], v[i], cv[r][i], sv[r][i]);
    }
    u32x2 o0, o1;
    if (a.interleaved) {
      o0[0] = pack_bf16x2(u[0], v[0]); o0[1] = pack_bf16x2(u[1], v[1]);
      o1[0] = pack_bf16x2(u[2], v[2]); o1[1] = pack_bf16x2(u[3], v[3]);
    } else {
      o0[0] = pack_bf16x2(u[0], u[1]); o0[1] = pack_bf16x2(u[2], u[3]);
      o1[0] = pack_bf16x2(v[0], v[1]); o1[1] = pack_bf16x2(v[2], v[3]);
    }
    uint16_t* dst = is_q ? a.q_out + ((int64_t)tok[r].row * a.hq + h) * kD
                         : cache + (((int64_t)tok[r].page * a.hkv + g) * kPage + tok[r].pos % kPage) * kD;
    *reinterpret_cast<u32x2*>(dst + off0) = o0;
    *reinterpret_cast<u32x2*>(dst + off1) = o1;
  }
}

}  // namespace

hipError_t launch_rope_table(const RopeTableArgs& a, hipStream_t stream) {
  const int64_t threads = (int64_t)a.max_pos * kHalf;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks < 1 || blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_rope_append(const RopeAppendArgs& a, hipStream_t stream) {
  const int H = a.kv_only ? 2 * a.hkv : a.hq + 2 * a.hkv;
  dim3 grid((unsigned)((a.total_q + kRowsPerBlock - 1) / kRowsPerBlock),
            (unsigned)((H + kHeadsPerBlock - 1) / kHeadsPerBlock));
  hipLaunchKernelGGL(rope_append_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sa
