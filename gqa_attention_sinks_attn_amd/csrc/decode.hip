// Paged split-KV decode with a per-head sink (gfx950).
//
// GPT-OSS on Day 0 (Perplexity), "Sink attention" under "Kernels for
// GPT-OSS": the softmax runs online with a running maximum m and scale d;
// starting m at the head's sink with d = 1 puts the sink into the
// denominator once, and when the KV sequence is split into chunks only the
// first chunk may carry it.  Work is parallel over heads and along the KV
// length (same passage).
//
// One workgroup = (request b, KV head g, chunk c); the grid lists every
// chunk-0 workgroup first.  Its four waves take the chunk's pages two at a
// time, round robin, each keeping its own online state for the G query heads
// of KV head g; the four states are merged in LDS at the end.  Per two-page
// step a wave:
//   * takes the two page ids from a register that holds its next 32 steps'
//     ids (one vector load per 32 steps, outside the step loop, read back
//     with readlane) and has issued the step's K and V loads one step
//     earlier (software pipeline, two register sets in flight per wave; the
//     issue is unconditional -- past the end it repeats the last step's
//     pages, which the cache serves -- so the compiler only waits for the
//     step being processed),
//   * computes S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (16 keys x 16 head
//     columns; columns >= G are padding) with K straight from registers,
//   * updates m, d and O in the exp2 domain, and
//   * accumulates O^T += V^T P^T on the same MFMA.  P^T comes straight from
//     the score registers; V is staged in a wave-private LDS slice in its
//     natural [key][dim] layout and read back transposed with
//     ds_read_b64_tr_b16 in the key order the score layout produces.
#include "common.hpp"
#include "launch.hpp"

namespace sa {
namespace {

constexpr int kWaves = 4;
constexpr int kPage = 16;
constexpr int kD = 64;
constexpr int kVPitch = 80;                      // LDS row pitch in bf16 (160 B)
constexpr int kWaveLds = 2 * kPage * kVPitch;    // bf16 elements per wave slice

struct alignas(16) CombineSlot {
  float m[16];
  float d[16];
  float o[16][kD];
};

constexpr int kLdsBytes =
    (kWaves * kWaveLds * 2) > (kWaves * (int)sizeof(CombineSlot))
        ? (kWaves * kWaveLds * 2)
        : (kWaves * (int)sizeof(CombineSlot));

// Complete the loads feeding `x` here (an empty asm reading the register).
template <class T>
__device__ __forceinline__ void settle(const T& x) {
  asm volatile("" ::"v"(x));
}

struct StepRegs {
  u32x4 k00, k01, k10, k11;   // K: page 0/1, dims 8 grp + {0, 32}
  u32x4 v00, v01, v10, v11;   // V: page 0/1, 32 contiguous bytes each
};

template <int G>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[kLdsBytes];
  uint16_t* lds_v = reinterpret_cast<uint16_t*>(lds_raw);

  const int unit = block_x();          // b * Hkv + g
  const int c = block_y();             // chunk
  const int g = unit % p.hkv;
  const int b = unit / p.hkv;
  const int lane = thread_x() & 63;
  // wave index in an SGPR: everything derived from it (page ranges, page-id
  // addresses) stays scalar, so page ids come through scalar loads
  const int wave = __builtin_amdgcn_readfirstlane(thread_x() >> 6);
  const int col = lane & 15;     // head column of the MFMA tile
  const int grp = lane >> 4;     // lane group 0..3
  const bool live_col = col < G;
  const int h = g * G + (live_col ? col : 0);

  const int L = __builtin_amdgcn_readfirstlane(p.kv_len[b]);
  const int n_pages = (L + kPage - 1) / kPage;
  const int pg0 = c * p.chunk_pages;
  const int pg1 = min(n_pages, pg0 + p.chunk_pages);
  const int32_t* pages = p.page_indices + __builtin_amdgcn_readfirstlane(p.page_indptr[b]);

  // Q^T operand: column `col` = head h, k-step s covers dims 32 s + 8 grp .. +7.
  bf16x8 bq0, bq1;
  {
    const uint16_t* qh = p.q + ((int64_t)b * p.hq + h) * kD + 8 * grp;
    const u32x4 z = {0u, 0u, 0u, 0u};
    bq0 = as_bf16x8(live_col ? ld16(qh) : z);
    bq1 = as_bf16x8(live_col ? ld16(qh + 32) : z);
  }

  // Online state in log2 units.  The sink-carrying state (wave 0 of chunk
  // 0) starts at m = sigma * log2(e), d = 1; every other state starts empty.
  float m = -INFINITY;
  float d = 0.f;   // lane-partial denominator (summed over groups at the end)
  if (c == 0 && wave == 0 && p.sinks != nullptr) {
    const float s = p.sinks[h];
    m = s * kLog2e;
    d = (grp == 0 && s != -INFINITY) ? 1.f : 0.f;
  }
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0, o2 = o0, o3 = o0;

  uint16_t* my_v = lds_v + wave * kWaveLds;
  const int64_t head_stride = (int64_t)kPage * kD;           // one page x head block
  const int64_t page_stride = (int64_t)p.hkv * head_stride;
  const int koff = col * kD + 8 * grp;                       // K operand offset
  const int voff = (lane >> 2) * kD + 16 * (lane & 3);       // V: 32 B per lane

  // Page ids: one vector load per block of 32 steps (lane l holds the id of
  // page l % 2 of step l / 2), placed outside the step loop and completed
  // there, then read with readlane.  Step `st` covers pages first + 8 st and
  // first + 8 st + 1 of the request.
  const int first = pg0 + 2 * wave;
  const int n_steps = pg1 > first ? (pg1 - first + 7) / 8 : 0;
  struct Pids { int a, b; };
  int ids = 0;
  auto pids = [&](int st) -> Pids {   // st: step index inside the current block
    return Pids{__builtin_amdgcn_readlane(ids, 2 * st), __builtin_amdgcn_readlane(ids, 2 * st + 1)};
  };

  auto issue = [&](StepRegs& r, Pids ids) {
    const uint16_t* kb0 = p.k + ids.a * page_stride + g * head_stride;
    const uint16_t* vb0 = p.v + ids.a * page_stride + g * head_stride;
    const uint16_t* kb1 = p.k + ids.b * page_stride + g * head_stride;
    const uint16_t* vb1 = p.v + ids.b * page_stride + g * head_stride;
    r.k00 = ld16(kb0 + koff);
    r.k01 = ld16(kb0 + koff + 32);
    r.k10 = ld16(kb1 + koff);
    r.k11 = ld16(kb1 + koff + 32);
    r.v00 = ld16(vb0 + voff);
    r.v01 = ld16(vb0 + voff + 8);
    r.v10 = ld16(vb1 + voff);
    r.v11 = ld16(vb1 + voff + 8);
  };

  auto process = [&](StepRegs& r, int step) {
    const int pp = first + 8 * step;
    const bool two = (pp + 1) < pg1;
    // Rows past the request's last key (the tail of its last page, or a
    // missing second page) are zeroed: their probabilities are 0, and 0
    // times whatever an unwritten cache slot holds must stay 0 in the MFMA.
    {
      const int vkey = pp * kPage + (lane >> 2);
      const u32x4 z = {0u, 0u, 0u, 0u};
      if (vkey >= L) { r.v00 = z; r.v01 = z; }
      if (!two || vkey + kPage >= L) { r.v10 = z; r.v11 = z; }
      uint16_t* r0 = my_v + (lane >> 2) * kVPitch + 16 * (lane & 3);
      uint16_t* r1 = r0 + kPage * kVPitch;
      *reinterpret_cast<u32x4*>(r0) = r.v00;
      *reinterpret_cast<u32x4*>(r0 + 8) = r.v01;
      *reinterpret_cast<u32x4*>(r1) = r.v10;
      *reinterpret_cast<u32x4*>(r1 + 8) = r.v11;
    }

    // S^T = K Q^T for both pages: lane holds head col, keys 4 grp + i
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
    s0 = mfma16(as_bf16x8(r.k00), bq0, s0);
    s1 = mfma16(as_bf16x8(r.k10), bq0, s1);
    s0 = mfma16(as_bf16x8(r.k01), bq1, s0);
    s1 = mfma16(as_bf16x8(r.k11), bq1, s1);

    float sc[8];
    const int key_base = pp * kPage + 4 * grp;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = (key_base + i < L) ? s0[i] * p.scale_log2 : -INFINITY;
      sc[4 + i] = (two && key_base + kPage + i < L) ? s1[i] * p.scale_log2 : -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                     fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    mx = fmaxf(mx, xor_lane(mx, 16));
    mx = fmaxf(mx, xor_lane(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float alpha = (m == m_new) ? 1.f : fast_exp2(m - m_new);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    float pr[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pr[i] = fast_exp2(sc[i] - m_use);
      psum += pr[i];
    }
    d = d * alpha + psum;
    m = m_new;
    o0 *= alpha; o1 *= alpha; o2 *= alpha; o3 *= alpha;

    // P^T operand: slot j <-> key (j < 4 ? 4 grp + j : 16 + 4 grp + j - 4)
    const u32x4 pw = {pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                      pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
    const bf16x8 pb = as_bf16x8(pw);

    // V^T operand per 16-dim block: row = dim 16 db + col, same key slots.
    // Source lane s of group grp points at key 4 grp + s / 4, dims
    // 16 db + 4 (s % 4); lane j then holds V[4 grp + e][16 db + j], e = 0..3.
    const uint16_t* src = my_v + (4 * grp + (col >> 2)) * kVPitch + 4 * (col & 3);
    o0 = mfma16(as_bf16x8(lds_tr16_pair(src, src + kPage * kVPitch)), pb, o0);
    o1 = mfma16(as_bf16x8(lds_tr16_pair(src + 16, src + kPage * kVPitch + 16)), pb, o1);
    o2 = mfma16(as_bf16x8(lds_tr16_pair(src + 32, src + kPage * kVPitch + 32)), pb, o2);
    o3 = mfma16(as_bf16x8(lds_tr16_pair(src + 48, src + kPage * kVPitch + 48)), pb, o3);
  };

  // Software pipeline: loads for step st + 1 are issued before step st is
  // processed, unconditionally (past the block's last step they repeat it;
  // the cache serves the repeat), so the compiler waits only for the step
  // being processed.  sched_barrier pins the issue/process order.
  for (int blk = 0; blk < n_steps; blk += 32) {
    const int nb = min(32, n_steps - blk);
    {
      const int st = blk + min(lane >> 1, nb - 1);
      const int pp = first + 8 * st;
      ids = pages[min(pp + (lane & 1), pg1 - 1)];
      settle(ids);
    }
    StepRegs ra, rb;
    issue(ra, pids(0));
    for (int i = 0; i < nb; i += 2) {
      issue(rb, pids(min(i + 1, nb - 1)));
      __builtin_amdgcn_sched_barrier(0);
      process(ra, blk + i);
      __builtin_amdgcn_sched_barrier(0);
      issue(ra, pids(min(i + 2, nb - 1)));
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < nb) process(rb, blk + i + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // finish the wave: total denominator per head column
  d += xor_lane(d, 16);
  d += xor_lane(d, 32);

  __syncthreads();  // all waves are done with their V slices
  CombineSlot* slots = reinterpret_cast<CombineSlot*>(lds_raw);
  CombineSlot& mine = slots[wave];
  if (grp == 0) {
    mine.m[col] = m;
    mine.d[col] = d;
  }
  *reinterpret_cast<f32x4*>(&mine.o[col][0 + 4 * grp]) = o0;
  *reinterpret_cast<f32x4*>(&mine.o[col][16 + 4 * grp]) = o1;
  *reinterpret_cast<f32x4*>(&mine.o[col][32 + 4 * grp]) = o2;
  *reinterpret_cast<f32x4*>(&mine.o[col][48 + 4 * grp]) = o3;
  __syncthreads();

  // 256 threads: column t / 16, dims 4 (t % 16) .. +3
  const int t = thread_x();
  const int oc = t >> 4;
  const int d0 = 4 * (t & 15);
  if (oc >= G) return;
  float M = slots[0].m[oc];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, slots[w].m[oc]);
  float den = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float mw = slots[w].m[oc];
    const float e = (mw == M) ? 1.f : fast_exp2(mw - M);
    den += e * slots[w].d[oc];
    acc += e * *reinterpret_cast<const f32x4*>(&slots[w].o[oc][d0]);
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  acc *= inv;
  // natural-log LSE of this state; -inf when it holds nothing
  const float lse = den > 0.f ? (M + __builtin_amdgcn_logf(den)) * kLn2 : -INFINITY;
  const int hh = g * G + oc;

  if (!p.write_partials) {
    const int64_t base = ((int64_t)b * p.hq + hh) * kD + d0;
    if (p.out_f32) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + base) = acc;
    } else {
      uint32_t* dst = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(p.out) + base);
      dst[0] = pack_bf16x2(acc[0], acc[1]);
      dst[1] = pack_bf16x2(acc[2], acc[3]);
    }
    if (p.lse != nullptr && d0 == 0) p.lse[(int64_t)b * p.hq + hh] = lse;
  } else {
    const int64_t row = ((int64_t)b * p.hq + hh) * p.num_splits + c;
    *reinterpret_cast<f32x4*>(p.o_part + row * kD + d0) = acc;
    if (d0 == 0) p.lse_part[row] = lse;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int group, hipStream_t stream) {
  dim3 grid(a.batch * a.hkv, a.num_splits);
  dim3 block(256);
  switch (group) {
    case 1: hipLaunchKernelGGL(decode_kernel<1>, grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(decode_kernel<2>, grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(decode_kernel<4>, grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL(decode_kernel<8>, grid, block, 0, stream, a); break;
    case 16: hipLaunchKernelGGL(decode_kernel<16>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sa
