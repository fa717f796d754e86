// Paged split-KV decode with a per-head sink (gfx950).
//
// GPT-OSS on Day 0 (Perplexity), "Sink attention" under "Kernels for
// GPT-OSS": the softmax runs online with a running maximum m and scale d;
// starting m at the head's sink with d = 1 puts the sink into the
// denominator once, and when the KV sequence is split into chunks only the
// first chunk may carry it.  Work is parallel over heads and along the KV
// length (same passage).
//
// One workgroup = (request b, KV head g, chunk c).  Its four waves take the
// chunk's pages two at a time, round robin, each wave keeping its own online
// state for the G query heads of KV head g; the four states are merged in
// LDS at the end.  Per two-page step a wave:
//   * gathers the two page ids (scalar loads) and loads K straight into
//     MFMA operand registers (16 B per lane per load),
//   * stages V (2 x 2 KiB) in a wave-private LDS slice,
//   * computes S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (16 keys x 16 head
//     columns; columns >= G are padding),
//   * updates m, d and O in the exp2 domain, and
//   * accumulates O^T += V^T P^T on the same MFMA, with P^T taken straight
//     from the score registers (the key order inside the contraction is the
//     one the score layout gives, and V^T is read from LDS to match).
#include "common.hpp"
#include "launch.hpp"

namespace sa {
namespace {

constexpr int kWaves = 4;
constexpr int kPage = 16;
constexpr int kD = 64;
constexpr int kRowElems = 68;            // LDS row stride in bf16 (136 B)
constexpr int kStepRows = 2 * kPage;     // rows of V staged per wave-step
constexpr int kWaveLds = kStepRows * kRowElems;   // bf16 elements per wave

struct alignas(16) CombineSlot {
  float m[16];
  float d[16];
  float o[16][kD];
};

constexpr int kLdsBytes =
    (kWaves * kWaveLds * 2) > (kWaves * (int)sizeof(CombineSlot))
        ? (kWaves * kWaveLds * 2)
        : (kWaves * (int)sizeof(CombineSlot));

template <int G>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[kLdsBytes];
  uint16_t* lds_v = reinterpret_cast<uint16_t*>(lds_raw);

  const int c = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;     // head column of the MFMA tile
  const int grp = lane >> 4;     // lane group 0..3
  const bool live_col = col < G;
  const int h = g * G + (live_col ? col : 0);

  const int L = p.kv_len[b];
  const int n_pages = (L + kPage - 1) / kPage;
  const int pg0 = c * p.chunk_pages;
  const int pg1 = min(n_pages, pg0 + p.chunk_pages);
  const int32_t* pages = p.page_indices + p.page_indptr[b];

  // Q^T operand: column `col` = head h, k-step s covers dims 32 s + 8 grp .. +7.
  bf16x8 bq[2];
  {
    const uint16_t* qh = p.q + ((int64_t)b * p.hq + h) * kD + 8 * grp;
    u32x4 z = {0u, 0u, 0u, 0u};
    bq[0] = as_bf16x8(live_col ? ld16(qh) : z);
    bq[1] = as_bf16x8(live_col ? ld16(qh + 32) : z);
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
  f32x4 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint16_t* my_v = lds_v + wave * kWaveLds;
  const int64_t head_stride = (int64_t)kPage * kD;           // one page x head block
  const int64_t page_stride = (int64_t)p.hkv * head_stride;

  for (int pp = pg0 + 2 * wave; pp < pg1; pp += 2 * kWaves) {
    const bool two = (pp + 1) < pg1;
    const int pid0 = pages[pp];
    const int pid1 = two ? pages[pp + 1] : pid0;
    const uint16_t* kb0 = p.k + pid0 * page_stride + g * head_stride;
    const uint16_t* kb1 = p.k + pid1 * page_stride + g * head_stride;
    const uint16_t* vb0 = p.v + pid0 * page_stride + g * head_stride;
    const uint16_t* vb1 = p.v + pid1 * page_stride + g * head_stride;

    // K operand: row = key (lane % 16), dims 32 s + 8 grp .. +7
    const int koff = col * kD + 8 * grp;
    u32x4 k00 = ld16(kb0 + koff), k01 = ld16(kb0 + koff + 32);
    u32x4 k10 = ld16(kb1 + koff), k11 = ld16(kb1 + koff + 32);
    // V rows: lane reads 32 contiguous bytes, key lane/4, dims 16 (lane%4) ..
    const int voff = (lane >> 2) * kD + 16 * (lane & 3);
    u32x4 v00 = ld16(vb0 + voff), v01 = ld16(vb0 + voff + 8);
    u32x4 v10 = ld16(vb1 + voff), v11 = ld16(vb1 + voff + 8);

    // Rows past the request's last key (the tail of its last page, or a
    // missing second page) are zeroed: their probabilities are 0, and 0 times
    // whatever an unwritten cache slot holds must stay 0 in the MFMA.
    {
      const int vkey = pp * kPage + (lane >> 2);
      const u32x4 z = {0u, 0u, 0u, 0u};
      if (vkey >= L) { v00 = z; v01 = z; }
      if (!two || vkey + kPage >= L) { v10 = z; v11 = z; }
    }
    // stage V in LDS, rows [page*16 + key], 136-byte stride
    {
      uint16_t* r0 = my_v + (lane >> 2) * kRowElems + 16 * (lane & 3);
      uint16_t* r1 = r0 + kPage * kRowElems;
      u32x2* w0 = reinterpret_cast<u32x2*>(r0);
      u32x2* w1 = reinterpret_cast<u32x2*>(r1);
      w0[0] = u32x2{v00[0], v00[1]}; w0[1] = u32x2{v00[2], v00[3]};
      w0[2] = u32x2{v01[0], v01[1]}; w0[3] = u32x2{v01[2], v01[3]};
      w1[0] = u32x2{v10[0], v10[1]}; w1[1] = u32x2{v10[2], v10[3]};
      w1[2] = u32x2{v11[0], v11[1]}; w1[3] = u32x2{v11[2], v11[3]};
    }

    // S^T = K Q^T for both pages: lane holds head col, keys 4 grp + i
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    s0 = mfma16(as_bf16x8(k00), bq[0], s0);
    s0 = mfma16(as_bf16x8(k01), bq[1], s0);
    s1 = mfma16(as_bf16x8(k10), bq[0], s1);
    s1 = mfma16(as_bf16x8(k11), bq[1], s1);

    float sc[8];
    const int key_base = pp * kPage + 4 * grp;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = (key_base + i < L) ? s0[i] * p.scale_log2 : -INFINITY;
      sc[4 + i] = (two && key_base + kPage + i < L) ? s1[i] * p.scale_log2 : -INFINITY;
    }
    float mx = sc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
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
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] *= alpha;

    // P^T operand: slot j <-> key (j < 4 ? 4 grp + j : 16 + 4 grp + j - 4)
    u32x4 pw = {pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
    const bf16x8 pb = as_bf16x8(pw);

    // V^T operand per 16-dim block: row = dim 16 db + col, same key slots
    const uint16_t* rA = my_v + (4 * grp) * kRowElems + col;
    const uint16_t* rB = rA + kPage * kRowElems;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int dc = 16 * db;
      u32x4 vw;
      vw[0] = (uint32_t)rA[0 * kRowElems + dc] | ((uint32_t)rA[1 * kRowElems + dc] << 16);
      vw[1] = (uint32_t)rA[2 * kRowElems + dc] | ((uint32_t)rA[3 * kRowElems + dc] << 16);
      vw[2] = (uint32_t)rB[0 * kRowElems + dc] | ((uint32_t)rB[1 * kRowElems + dc] << 16);
      vw[3] = (uint32_t)rB[2 * kRowElems + dc] | ((uint32_t)rB[3 * kRowElems + dc] << 16);
      o[db] = mfma16(as_bf16x8(vw), pb, o[db]);
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
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    float* dst = &mine.o[col][16 * db + 4 * grp];
    *reinterpret_cast<f32x4*>(dst) = o[db];
  }
  __syncthreads();

  // 256 threads: column t / 16, dims 4 (t % 16) .. +3
  const int t = threadIdx.x;
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
  dim3 grid(a.num_splits, a.hkv, a.batch);
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
