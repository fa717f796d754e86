// Multi-token verification attention with a per-head sink (gfx950): a few
// drafted tokens per request against a paged KV cache, causal within the
// draft.
//
// GPT-OSS on Day 0 (Perplexity), "Sink attention" under "Kernels for
// GPT-OSS": the sink is an extra logit per head, folded into the online
// softmax by starting the running maximum at the sink with d = 1; work is
// parallel over heads and along the KV length, and when the KV sequence is
// split only the first chunk carries the sink.  "Accelerating Sonar Through
// Speculation" (Perplexity), "Speculative Decoding" (its acceptance stage)
// and "MTP": the target model runs once over each request's drafted tokens
// to score every one of them.  This kernel is the decode kernel with those
// tokens packed into the matrix columns.
//
// One workgroup = (request b, KV head g, chunk c, column group z), four
// waves taking the chunk's pages two at a time, round robin (as the split-KV
// decode).  The rows of (b, g) are the qlen_b drafted tokens x G query
// heads; column c' = 16 (NB z + blk) + (lane % 16) is token t = c' / G, head
// g G + c' % G; columns past the draft are padding.  Token t sits at
// position P + t, P = kv_len - qlen, and sees keys 0 .. P + t (bottom-right
// causal alignment), or, with a draft mask (same page, "EAGLE": tree drafts
// are verified under custom attention masks), every prefix key plus drafted
// key P + i when bit i of its mask word is set.  The mask is tested only on
// the steps that reach the drafted keys.
//
// The Z column groups of one (request, KV head, chunk) read the same pages.
// Workgroups are dealt to the 8 XCDs round robin, so the flat index puts
// those Z groups on one XCD back to back, where the later reads hit its L2.
//
// Per two-page step and column block:
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16, K straight from registers
//     (one load serves every column block);
//   * on the steps that reach the drafted keys, the per-column limit (or
//     the draft mask) masks keys;
//   * softmax in exp2 against a per-column reference maximum, raised (with
//     the rescale of d and O) only when a step would push a lane's partial
//     sum past 2^15, so most steps skip the maximum and the rescale;
//   * O^T += V^T P^T on the same MFMA, V^T from a wave-private LDS slice
//     read transposed with ds_read_b64_tr_b16 (read once per step, shared
//     by the column blocks).
// The four waves are merged in LDS; chunk c writes the final rows (one
// chunk) or its normalised partial and log-sum-exp.
#include "common.hpp"
#include "launch.hpp"

namespace sa {
namespace {

constexpr int kWaves = 4;
constexpr int kPage = 16;
constexpr int kD = 64;
constexpr int kVPitch = 80;                      // LDS row pitch in bf16 (160 B)
constexpr int kWaveLds = 2 * kPage * kVPitch;    // bf16 elements per wave slice
constexpr float kFastLimit = 32768.f;            // lane-partial step sum that forces a rescale

// acc + lo(w) + hi(w) for a packed bf16 pair, accumulated in fp32
__device__ __forceinline__ float dot2_sum(uint32_t w, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

template <class T>
__device__ __forceinline__ void settle(const T& x) {
  asm volatile("" ::"v"(x));
}

struct StepRegs {
  u32x4 k00, k01, k10, k11;   // K: page 0/1, dims 8 grp + {0, 32}
  u32x4 v00, v01, v10, v11;   // V: page 0/1, 32 contiguous bytes each
};

template <int NB>
struct alignas(16) VerifySlot {
  float m[16 * NB];
  float d[16 * NB];
  float o[16 * NB][kD];
};

template <int G, int NB, bool TREE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void verify_kernel(VerifyArgs p) {
  constexpr int kSlotBytes = (int)sizeof(VerifySlot<NB>);
  constexpr int kLdsBytes = (kWaves * kWaveLds * 2) > (kWaves * kSlotBytes)
                                ? (kWaves * kWaveLds * 2) : (kWaves * kSlotBytes);
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[kLdsBytes];
  uint16_t* lds_v = reinterpret_cast<uint16_t*>(lds_raw);

  // flat index -> (work item = c * B * Hkv + unit, column group zg)
  const int n_work = p.batch * p.hkv * p.num_splits;
  const int xcd = block_x() & 7;
  const int rest = block_x() >> 3;
  const int zg = rest % p.col_groups;
  const int item = (rest / p.col_groups) * 8 + xcd;
  if (item >= n_work) return;
  const int unit = item % (p.batch * p.hkv);   // b * Hkv + g
  const int c = item / (p.batch * p.hkv);      // chunk
  const int cb = 16 * NB * zg;                 // first column of the group
  const int g = unit % p.hkv;
  const int b = unit / p.hkv;
  const int lane = thread_x() & 63;
  const int wave = __builtin_amdgcn_readfirstlane(thread_x() >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;

  const int q0 = __builtin_amdgcn_readfirstlane(p.qo_indptr[b]);
  const int qlen = __builtin_amdgcn_readfirstlane(p.qo_indptr[b + 1]) - q0;
  if (qlen * G <= cb) return;   // no rows in this group (q0 may be past the last row)
  const int L = __builtin_amdgcn_readfirstlane(p.kv_len[b]);
  const int n_pages = (L + kPage - 1) / kPage;
  const int pg0 = c * p.chunk_pages;
  const int pg1 = min(n_pages, pg0 + p.chunk_pages);
  const int32_t* pages = p.page_indices + __builtin_amdgcn_readfirstlane(p.page_indptr[b]);

  // This lane's column in each block: token, head, key limit (keys <= lim
  // are allowed; padding columns allow none), drafted-key bits, Q^T operand.
  const int P = L - qlen;
  int head[NB], lim[NB];
  bool live[NB];
  uint32_t mlo[NB], mhi[NB];
  bf16x8 bq0[NB], bq1[NB];
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    const int cc = cb + 16 * blk + col;
    const int t = cc / G;
    live[blk] = t < qlen;
    head[blk] = g * G + cc % G;
    lim[blk] = live[blk] ? (TREE ? P - 1 : P + t) : -1;
    mlo[blk] = mhi[blk] = 0u;
    if (TREE && live[blk]) {
      const uint64_t bits = p.draft_mask[q0 + t];
      mlo[blk] = (uint32_t)bits;
      mhi[blk] = (uint32_t)(bits >> 32);
    }
    const uint16_t* qh = p.q + ((int64_t)(q0 + (live[blk] ? t : 0)) * p.hq + head[blk]) * kD + 8 * grp;
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 a = ld16(qh), e = ld16(qh + 32);
    bq0[blk] = as_bf16x8(live[blk] ? a : z);
    bq1[blk] = as_bf16x8(live[blk] ? e : z);
  }

  // Online state per column block, log2 units; the sink-carrying state
  // (wave 0 of chunk 0) starts at m = sigma log2(e), d = 1.
  float m[NB], d[NB];
  f32x4 o[NB][4];
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    // padding columns get a finite reference: they never force the slow
    // path, and their sums (of exp2(0)) are never written
    m[blk] = live[blk] ? -INFINITY : 0.f;
    d[blk] = 0.f;
    if (c == 0 && wave == 0 && p.sinks != nullptr && live[blk]) {
      const float s = p.sinks[head[blk]];
      m[blk] = s * kLog2e;
      d[blk] = (grp == 0 && s != -INFINITY) ? 1.f : 0.f;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) o[blk][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  uint16_t* my_v = lds_v + wave * kWaveLds;
  const int64_t head_stride = (int64_t)kPage * kD;
  const int64_t page_stride = (int64_t)p.hkv * head_stride;
  const int koff = col * kD + 8 * grp;
  const int voff = (lane >> 2) * kD + 16 * (lane & 3);

  const int first = pg0 + 2 * wave;
  const int n_steps = pg1 > first ? (pg1 - first + 7) / 8 : 0;
  struct Pids { int a, b; };
  int ids = 0;
  auto pids = [&](int st) -> Pids {
    return Pids{__builtin_amdgcn_readlane(ids, 2 * st), __builtin_amdgcn_readlane(ids, 2 * st + 1)};
  };
  auto issue = [&](StepRegs& r, Pids q) {
    const uint16_t* kb0 = p.k + q.a * page_stride + g * head_stride;
    const uint16_t* vb0 = p.v + q.a * page_stride + g * head_stride;
    const uint16_t* kb1 = p.k + q.b * page_stride + g * head_stride;
    const uint16_t* vb1 = p.v + q.b * page_stride + g * head_stride;
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
    // V rows past the request's last key (tail of its last page, or a
    // missing second page) are zeroed: 0 x an unwritten slot must stay 0.
    // Only a step that reaches the end of the cache (or misses its second
    // page) needs the selects: a wave-uniform branch.
    {
      uint16_t* r0 = my_v + (lane >> 2) * kVPitch + 16 * (lane & 3);
      uint16_t* r1 = r0 + kPage * kVPitch;
      if (two && pp * kPage + 2 * kPage <= L) {
        *reinterpret_cast<u32x4*>(r0) = r.v00;
        *reinterpret_cast<u32x4*>(r0 + 8) = r.v01;
        *reinterpret_cast<u32x4*>(r1) = r.v10;
        *reinterpret_cast<u32x4*>(r1 + 8) = r.v11;
      } else {
        const int vkey = pp * kPage + (lane >> 2);
        const u32x4 z = {0u, 0u, 0u, 0u};
        const bool d0 = vkey >= L;
        const bool d1 = !two || vkey + kPage >= L;
        *reinterpret_cast<u32x4*>(r0) = d0 ? z : r.v00;
        *reinterpret_cast<u32x4*>(r0 + 8) = d0 ? z : r.v01;
        *reinterpret_cast<u32x4*>(r1) = d1 ? z : r.v10;
        *reinterpret_cast<u32x4*>(r1 + 8) = d1 ? z : r.v11;
      }
    }
    // V^T operands of the step, one per 16-dim block, shared by every
    // column block: source lane s of group grp points at key 4 grp + s / 4,
    // dims 16 db + 4 (s % 4).
    const uint16_t* src = my_v + (4 * grp + (col >> 2)) * kVPitch + 4 * (col & 3);
    bf16x8 vt[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
      vt[db] = as_bf16x8(lds_tr16_pair(src + 16 * db, src + kPage * kVPitch + 16 * db));

    const int key_base = pp * kPage + 4 * grp;
    const int lim2 = two ? L : pp * kPage + kPage;   // keys of a missing second page
    // Masks are needed only on steps that reach the drafted keys (causal or
    // tree visibility, the end of the cache) or miss their second page.
    const bool edge = pp * kPage + 2 * kPage > P || !two;
    const bool draft = TREE && edge;
    // The step runs in phases over all column blocks at once (scores,
    // masks, exponentials, one slow-path test, P.V), so the matrix core and
    // the vector unit always have independent work from the other block
    // and a step has one mask branch and one slow-path branch.
    // (1) S^T = K Q^T per block, K straight from registers; raw scores (the
    //     scale is applied inside the exponent's FMA).
    float sc[NB][8];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
      s0 = mfma16(as_bf16x8(r.k00), bq0[blk], s0);
      s1 = mfma16(as_bf16x8(r.k10), bq0[blk], s1);
      s0 = mfma16(as_bf16x8(r.k01), bq1[blk], s0);
      s1 = mfma16(as_bf16x8(r.k11), bq1[blk], s1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[blk][i] = s0[i];
        sc[blk][4 + i] = s1[i];
      }
    }
    // (2) Masks.
    if (draft) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        // drafted key P + j is visible when bit j is set (j < qlen, so the
        // key also lies below kv_len)
        auto seen = [&](int key) -> bool {
          const int j = key - P;
          const uint32_t word = j < 32 ? mlo[blk] : mhi[blk];
          return key <= lim[blk] || ((unsigned)j < (unsigned)qlen && ((word >> (j & 31)) & 1u));
        };
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k0 = key_base + i, k1 = key_base + kPage + i;
          if (!seen(k0)) sc[blk][i] = -INFINITY;
          if (!(seen(k1) && k1 < lim2)) sc[blk][4 + i] = -INFINITY;
        }
      }
    } else if (edge) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k0 = key_base + i, k1 = key_base + kPage + i;
          if (!(k0 <= lim[blk])) sc[blk][i] = -INFINITY;
          if (!(k1 <= lim[blk] && k1 < lim2)) sc[blk][4 + i] = -INFINITY;
        }
    }
    // (3) Exponentiate against each column's reference maximum m:
    //     exp2(s * scale - m), one FMA per score (a masked score gives 0).
    //     The fast path holds while every lane's partial sum stays below
    //     kFastLimit and the column has a reference; otherwise take the true
    //     maximum of the step, rescale d and O, and exponentiate again.
    //     Either way the result is the online softmax's.
    uint32_t pw[NB][4];
    float psum[NB];
    const float sl2 = p.scale_log2;
    auto expo = [&](int blk, float m_use) {
      psum[blk] = 0.f;
      const float nm = -m_use;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pw[blk][i] = pack_bf16x2(fast_exp2(__builtin_fmaf(sc[blk][2 * i], sl2, nm)),
                                 fast_exp2(__builtin_fmaf(sc[blk][2 * i + 1], sl2, nm)));
        psum[blk] = dot2_sum(pw[blk][i], psum[blk]);
      }
    };
    bool slow = false;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      expo(blk, m[blk] == -INFINITY ? 0.f : m[blk]);
      slow = slow || !(psum[blk] <= kFastLimit) || m[blk] == -INFINITY;
    }
    // (4) The slow path (rare; wave-uniform): the rescale of d and O
    //     happens only here, so the fast path never touches the
    //     accumulators outside the MFMA.
    if (__any(slow)) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        const float* x = sc[blk];
        float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                         fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        mx = fmaxf(mx, xor_lane(mx, 16));
        mx = fmaxf(mx, xor_lane(mx, 32));
        const float m_new = fmaxf(m[blk], mx * sl2);
        const float alpha = (m[blk] == m_new) ? 1.f : fast_exp2(m[blk] - m_new);
        m[blk] = m_new;
        d[blk] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[blk][db] *= alpha;
        expo(blk, m_new == -INFINITY ? 0.f : m_new);
      }
    }
    // (5) O^T += V^T P^T; P^T slot j <-> key (j < 4 ? 4 grp + j : 16 + 4 grp + j - 4)
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      d[blk] += psum[blk];
      const bf16x8 pb = as_bf16x8(u32x4{pw[blk][0], pw[blk][1], pw[blk][2], pw[blk][3]});
#pragma unroll
      for (int db = 0; db < 4; ++db) o[blk][db] = mfma16(vt[db], pb, o[blk][db]);
    }
  };

  for (int blk0 = 0; blk0 < n_steps; blk0 += 32) {
    const int nb = min(32, n_steps - blk0);
    {
      const int st = blk0 + min(lane >> 1, nb - 1);
      const int pp = first + 8 * st;
      ids = pages[min(pp + (lane & 1), pg1 - 1)];
      settle(ids);
    }
    // three register sets: the loads of step i + 2 are in flight while
    // step i is processed
    StepRegs ra, rb, rc;
    issue(ra, pids(0));
    issue(rb, pids(min(1, nb - 1)));
    for (int i = 0; i < nb; i += 3) {
      issue(rc, pids(min(i + 2, nb - 1)));
      __builtin_amdgcn_sched_barrier(0);
      process(ra, blk0 + i);
      __builtin_amdgcn_sched_barrier(0);
      issue(ra, pids(min(i + 3, nb - 1)));
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < nb) process(rb, blk0 + i + 1);
      __builtin_amdgcn_sched_barrier(0);
      issue(rb, pids(min(i + 4, nb - 1)));
      __builtin_amdgcn_sched_barrier(0);
      if (i + 2 < nb) process(rc, blk0 + i + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    d[blk] += xor_lane(d[blk], 16);
    d[blk] += xor_lane(d[blk], 32);
  }

  __syncthreads();  // all waves are done with their V slices
  VerifySlot<NB>* slots = reinterpret_cast<VerifySlot<NB>*>(lds_raw);
  VerifySlot<NB>& mine = slots[wave];
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    const int cc = 16 * blk + col;   // column within the group
    if (grp == 0) {
      mine.m[cc] = m[blk];
      mine.d[cc] = d[blk];
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
      *reinterpret_cast<f32x4*>(&mine.o[cc][16 * db + 4 * grp]) = o[blk][db];
  }
  __syncthreads();

  // 256 threads: column (t / 16) + 16 k, dims 4 (t % 16) .. +3
  const int tt = thread_x();
  const int d0 = 4 * (tt & 15);
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int cc = (tt >> 4) + 16 * k;   // column within the group
    const int t = (cb + cc) / G;
    if (t >= qlen) continue;
    float M = slots[0].m[cc];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, slots[w].m[cc]);
    float den = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = slots[w].m[cc];
      const float e = (mw == M) ? 1.f : fast_exp2(mw - M);
      den += e * slots[w].d[cc];
      acc += e * *reinterpret_cast<const f32x4*>(&slots[w].o[cc][d0]);
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    acc *= inv;
    const float lse = den > 0.f ? (M + __builtin_amdgcn_logf(den)) * kLn2 : -INFINITY;
    const int hh = g * G + (cb + cc) % G;
    const int64_t row = (int64_t)(q0 + t) * p.hq + hh;
    if (!p.write_partials) {
      const int64_t base = row * kD + d0;
      if (p.out_f32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + base) = acc;
      } else {
        uint32_t* dst = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(p.out) + base);
        dst[0] = pack_bf16x2(acc[0], acc[1]);
        dst[1] = pack_bf16x2(acc[2], acc[3]);
      }
      if (p.lse != nullptr && d0 == 0) p.lse[row] = lse;
    } else {
      const int64_t prow = row * p.num_splits + c;
      *reinterpret_cast<f32x4*>(p.o_part + prow * kD + d0) = acc;
      if (d0 == 0) p.lse_part[prow] = lse;
    }
  }
}

template <int G, bool TREE>
hipError_t launch_g(const VerifyArgs& a, int nb, hipStream_t stream) {
  const int64_t work = (int64_t)a.batch * a.hkv * a.num_splits;
  const int64_t blocks = (work + 7) / 8 * 8 * a.col_groups;
  if (a.col_groups < 1 || blocks > INT32_MAX) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks);
  dim3 block(256);
  if (nb == 1) { hipLaunchKernelGGL((verify_kernel<G, 1, TREE>), grid, block, 0, stream, a); return hipGetLastError(); }
  if (nb == 2) { hipLaunchKernelGGL((verify_kernel<G, 2, TREE>), grid, block, 0, stream, a); return hipGetLastError(); }
  return hipErrorInvalidValue;
}

template <int G>
hipError_t launch_mode(const VerifyArgs& a, int nb, hipStream_t stream) {
  return a.draft_mask != nullptr ? launch_g<G, true>(a, nb, stream) : launch_g<G, false>(a, nb, stream);
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, int group, int column_blocks, hipStream_t stream) {
  switch (group) {
    case 1: return launch_mode<1>(a, column_blocks, stream);
    case 2: return launch_mode<2>(a, column_blocks, stream);
    case 4: return launch_mode<4>(a, column_blocks, stream);
    case 8: return launch_mode<8>(a, column_blocks, stream);
    case 16: return launch_mode<16>(a, column_blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sa
