// Load-balanced paged decode with a per-head sink (gfx950): two kernels.
//
// GPT-OSS on Day 0 (Perplexity), "Sink attention" under "Kernels for
// GPT-OSS": attention is parallelised across heads and along the KV length;
// the online softmax keeps a running maximum m and scale d, and starting m at
// the head's sink with d = 1 puts the sink into the denominator once -- so
// when a sequence is split, only the piece that holds its first key may
// carry the sink.
//
// Stage 1 (decode_balanced_kernel).  The batch's page table is one array
// (page_indices, offsets page_indptr), so its pages form one global list of
// nnz = page_indptr[B] pages.  For each KV head the list is cut into
// n_ranges equal ranges of Rw = ceil(nnz / n_ranges) pages, one per wave:
// every wave streams the same number of pages whatever the length mix, and
// the grid is sized to the machine rather than to the longest request.  A
// wave walks its range two pages per step (the step's K and V loads issued
// one step ahead, unconditionally -- past the range they repeat its last
// pages, which the cache serves -- so the compiler waits only for the step
// being processed).  Per step:
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (16 keys x 16 head columns per
//     page; columns >= G are padding), K straight from registers;
//   * masking: keys past kv_len and pages outside the current request;
//   * online softmax in the exp2 domain;
//   * O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 over the step's 32 keys,
//     P^T straight from the score registers, V staged in a wave-private LDS
//     slice and read back transposed with ds_read_b64_tr_b16.
// A step whose two pages straddle a request boundary is processed twice from
// the same registers, once per side.  When a request ends inside the range
// (or the range ends) the wave closes its segment: a request that lies
// inside one range is written straight to the output; otherwise the
// normalised partial (o, lse) goes to slot (range + request) of the
// workspace -- unique, since a range holds one segment per request.
//
// Stage 2 (decode_finish_kernel), one wave per (request, query head): merges
// the partials of requests that span several ranges by log-sum-exp, and
// writes requests without pages (o = 0, lse = sink).
//
// The decode step (STEP): stage 1 also does the step that precedes the
// attention for each request's one new token ("Accelerating Sonar Through
// Speculation", "Inference with Speculative Decoding": the new token's slot
// is reserved in the paged cache before the step; "GPT-OSS on Day 0",
// "Attention: GQA with attention sinks": QKV bias and YaRN rotary encoding).
// Before it streams its range, a wave writes the new keys and values whose
// cache slot lies in its own pages (for its KV head): it is the only reader
// of those slots, so its later loads see them.  Each wave rotates the query
// of every request it visits when it opens the segment (in the operand
// layout a lane holds both members of each rotated pair).  The arithmetic is
// the append kernel's, so the result equals the append followed by the
// decode bit for bit.
#include "common.hpp"
#include "launch.hpp"

namespace sa {
namespace {

constexpr int kPage = 16;
constexpr int kD = 64;
constexpr int kWaves = 4;
constexpr int kVPitch = 80;                    // LDS row pitch in bf16 (160 B)
constexpr int kWaveLds = 2 * kPage * kVPitch;  // two pages of V per wave

template <class T>
__device__ __forceinline__ void settle(const T& x) {
  asm volatile("" ::"v"(x));
}

struct StepRegs {
  u32x4 k00, k01, k10, k11;   // K: page 0/1, dims 8 grp + {0, 32}
  u32x4 v00, v01, v10, v11;   // V: page 0/1, 32 contiguous bytes each
};

// One 16-byte piece of a new token's head, as the append kernel handles
// it: dims off0 .. off0 + 3 and off1 .. off1 + 3 of lane j (off = 4 j and
// 32 + 4 j in the rotate-half pairing, 8 j and 8 j + 4 interleaved), i.e.
// rotary pairs 4 j .. 4 j + 3 in both; the bias added in fp32, the key and
// query heads rotated by the token's table row (cos at 4 j, sin 32 floats
// further), rounded to bf16 once.
__device__ __forceinline__ void new_piece(u32x2 x0, u32x2 x1, u32x2 b0, u32x2 b1, bool rotate,
                                          f32x4 c, f32x4 s, int interleaved, uint16_t* dst,
                                          int off0, int off1) {
  float lo[4] = {lo_bf16(x0[0]) + lo_bf16(b0[0]), hi_bf16(x0[0]) + hi_bf16(b0[0]),
                 lo_bf16(x0[1]) + lo_bf16(b0[1]), hi_bf16(x0[1]) + hi_bf16(b0[1])};
  float hi[4] = {lo_bf16(x1[0]) + lo_bf16(b1[0]), hi_bf16(x1[0]) + hi_bf16(b1[0]),
                 lo_bf16(x1[1]) + lo_bf16(b1[1]), hi_bf16(x1[1]) + hi_bf16(b1[1])};
  if (rotate) {
    float u[4], v[4];
    if (interleaved) {
      u[0] = lo[0]; v[0] = lo[1]; u[1] = lo[2]; v[1] = lo[3];
      u[2] = hi[0]; v[2] = hi[1]; u[3] = hi[2]; v[3] = hi[3];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) { u[i] = lo[i]; v[i] = hi[i]; }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) rotate_pair(u[i], v[i], c[i], s[i]);
    if (interleaved) {
      lo[0] = u[0]; lo[1] = v[0]; lo[2] = u[1]; lo[3] = v[1];
      hi[0] = u[2]; hi[1] = v[2]; hi[2] = u[3]; hi[3] = v[3];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) { lo[i] = u[i]; hi[i] = v[i]; }
    }
  }
  *reinterpret_cast<u32x2*>(dst + off0) = u32x2{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3])};
  *reinterpret_cast<u32x2*>(dst + off1) = u32x2{pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
}

__device__ __forceinline__ u32x2 ld8(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }

// Largest request b < B with indptr[b] <= pg (indptr non-decreasing,
// indptr[0] = 0 <= pg): a 64-way sampled search, then a 64-way search inside
// the sampled block.  Wave-uniform result.
__device__ __forceinline__ int find_request(const int32_t* indptr, int B, int pg, int lane) {
  const int stride = (B + 63) >> 6;
  const int idx = lane * stride;
  const bool in = idx < B;
  const int v = in ? indptr[idx] : 0x7fffffff;
  const uint64_t m = __ballot(in && v <= pg);
  // m != 0 when indptr[0] = 0 <= pg; the clamp only guards malformed input
  const int base = m ? (63 - __clzll((long long)m)) * stride : 0;
  if (stride == 1) return __builtin_amdgcn_readfirstlane(base);
  int best = base;
  for (int off = 0; off < stride; off += 64) {
    const int i2 = base + off + lane;
    const bool in2 = (off + lane < stride) && i2 < B;
    const int v2 = in2 ? indptr[i2] : 0x7fffffff;
    const uint64_t m2 = __ballot(in2 && v2 <= pg);
    const uint64_t live = __ballot(in2);
    if (m2) best = base + off + 63 - __clzll((long long)m2);
    if (m2 != live) break;
  }
  return __builtin_amdgcn_readfirstlane(best);
}

// Pages per range: nnz split over n_ranges, at least min_pages.
__device__ __forceinline__ int range_width(int nnz, int n_ranges, int min_pages) {
  return max(min_pages, (nnz + n_ranges - 1) / n_ranges);
}

template <int G, bool STEP>
__global__ __launch_bounds__(256) void decode_balanced_kernel(BalancedDecodeArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[kWaves * kWaveLds];

  const int lane = thread_x() & 63;
  const int wave = __builtin_amdgcn_readfirstlane(thread_x() >> 6);
  const int g = block_y();
  const int u = block_x() * kWaves + wave;   // this wave's range
  const int col = lane & 15;
  const int grp = lane >> 4;
  const bool live_col = col < G;
  const int h = g * G + (live_col ? col : 0);
  const int B = p.batch;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  const int nnz = __builtin_amdgcn_readfirstlane(p.page_indptr[B]);
  const int Rw = __builtin_amdgcn_readfirstlane(range_width(nnz, p.n_ranges, p.min_range_pages));
  const int p0 = __builtin_amdgcn_readfirstlane(u * Rw);
  const int p1 = __builtin_amdgcn_readfirstlane(min(nnz, p0 + Rw));
  if (p0 >= p1) return;
  const int n_steps = (p1 - p0 + 1) >> 1;

  // (Every lambda of this kernel is forced inline: with the decode step's
  // extra call sites the inliner would otherwise outline some of them, and
  // an outlined helper works through the stack and generic pointers.)

  // Start-up.  Loads that need only the range go out first: the first 32
  // steps' page ids (lane l: page p0 + l, i.e. step l / 2, page l % 2), the
  // first level of the request lookup, and the head's sink.  The first
  // step's K/V loads follow as soon as the ids arrive, before the lookup
  // resolves, so the stream starts one round trip after the ids.
  auto load_ids = [&](int first_step) __attribute__((always_inline)) {
    return p.page_indices[min(p0 + 2 * first_step + lane, p1 - 1)];
  };
  int ids = load_ids(0);
  int ids_next = load_ids(32);
  const int stride = (B + 63) >> 6;
  const int sval = p.page_indptr[min(lane * stride, B)];
  const float sink = p.sinks != nullptr ? p.sinks[h] : -INFINITY;

  const int64_t head_stride = (int64_t)kPage * kD;
  const int64_t page_stride = (int64_t)p.hkv * head_stride;
  const int koff = col * kD + 8 * grp;
  const int voff = (lane >> 2) * kD + 16 * (lane & 3);
  auto issue = [&](StepRegs& r, int pid_a, int pid_b) __attribute__((always_inline)) {
    const uint16_t* kb0 = p.k + pid_a * page_stride + g * head_stride;
    const uint16_t* vb0 = p.v + pid_a * page_stride + g * head_stride;
    const uint16_t* kb1 = p.k + pid_b * page_stride + g * head_stride;
    const uint16_t* vb1 = p.v + pid_b * page_stride + g * head_stride;
    r.k00 = ld16(kb0 + koff);
    r.k01 = ld16(kb0 + koff + 32);
    r.k10 = ld16(kb1 + koff);
    r.k11 = ld16(kb1 + koff + 32);
    r.v00 = ld16(vb0 + voff);
    r.v01 = ld16(vb0 + voff + 8);
    r.v10 = ld16(vb1 + voff);
    r.v11 = ld16(vb1 + voff + 8);
  };
  // Page ids of step st (clamped to the last step): `ids` holds the 32
  // steps from `base`, `ids_next` the 32 after them.  Each id block is
  // loaded before the K/V loads that precede its first use, so reading it
  // never waits for K/V data.
  int base = 0;
  auto issue_step = [&](StepRegs& r, int st) __attribute__((always_inline)) {
    const int j = min(st, n_steps - 1) - base;
    const int src = j < 32 ? ids : ids_next;
    const int jj = j & 31;
    issue(r, __builtin_amdgcn_readlane(src, 2 * jj), __builtin_amdgcn_readlane(src, 2 * jj + 1));
  };
  StepRegs ra, rb;
  issue_step(ra, 0);
  __builtin_amdgcn_sched_barrier(0);

  // The request that owns page p0: the first level's ballot, then (for more
  // than 64 requests) the search inside the chosen block of `stride`.
  const uint64_t m1 = __ballot(sval <= p0);
  int b = m1 ? (63 - __clzll((long long)m1)) * stride : 0;
  if (stride > 1) b = find_request(p.page_indptr, B, p0, lane);
  b = __builtin_amdgcn_readfirstlane(b);
  int seg_start, seg_end, Lb;
  // decode step: requests b .. b + 3 (lanes 16 r ..): page range and length,
  // for the append below, in the same round trip (request b's from lane 0)
  int g0_s0 = 0, g0_s1 = 0, g0_L = 0;
  if constexpr (STEP) {
    const int bb = b + (lane >> 4);
    g0_s0 = bb < B ? p.page_indptr[bb] : p1;
    g0_s1 = bb < B ? p.page_indptr[bb + 1] : p1;
    g0_L = bb < B ? p.kv_len[bb] : 0;
    seg_start = __builtin_amdgcn_readfirstlane(g0_s0);
    seg_end = __builtin_amdgcn_readfirstlane(g0_s1);
    Lb = __builtin_amdgcn_readfirstlane(g0_L);
  } else {
    seg_start = __builtin_amdgcn_readfirstlane(p.page_indptr[b]);
    seg_end = __builtin_amdgcn_readfirstlane(p.page_indptr[b + 1]);
    Lb = __builtin_amdgcn_readfirstlane(p.kv_len[b]);
  }

  // Q^T operand of request bb (column `col` = head h; padding columns read
  // head g*G and are zeroed at use).
  auto q_of = [&](int bb, u32x4& a, u32x4& c) __attribute__((always_inline)) {
    const uint16_t* qh = p.q + ((int64_t)bb * p.hq + h) * kD + 8 * grp;
    a = ld16(qh);
    c = ld16(qh + 32);
  };

  // Decode step.  Before it streams its range, the wave (1) appends the new
  // keys and values whose cache slot lies in its pages -- it is the only
  // reader of those slots -- and (2) rotates the query of every request its
  // range holds into the query buffer (p.q) the decode reads; waves whose
  // ranges share a request write the same values.  Requests go in groups of
  // four.  Queries: lane (hs, j) = lane (lane / 8, lane % 8) takes piece j
  // of query head g G + 8 hp + hs, for head passes hp; keys and values:
  // sixteen lanes per request, eight for the key head and eight for the
  // value head.  All of a group's loads go out before its arithmetic.  The
  // stores complete (and are visible to this work-group's loads) before
  // the queries are read and before any later step's loads are issued; the
  // first step's, already in flight, are issued again when one of its two
  // pages holds a new slot.
  auto append_step = [&]() __attribute__((always_inline)) {
    constexpr int kPasses = (G + 7) / 8;
    const int j = lane & 7;
    const int hs = lane >> 3;
    const int off0 = p.interleaved ? 8 * j : 4 * j;
    const int off1 = p.interleaved ? 8 * j + 4 : 32 + 4 * j;
    const int64_t row_elems = (int64_t)(p.hq + 2 * p.hkv) * kD;
    const u32x2 zero2 = {0u, 0u};
    u32x2 qb0[kPasses], qb1[kPasses];   // query bias pieces (the same for every request)
#pragma unroll
    for (int hp = 0; hp < kPasses; ++hp) {
      const int head = g * G + min(8 * hp + hs, G - 1);
      qb0[hp] = p.bias != nullptr ? ld8(p.bias + (int64_t)head * kD + off0) : zero2;
      qb1[hp] = p.bias != nullptr ? ld8(p.bias + (int64_t)head * kD + off1) : zero2;
    }
    const int rr = lane >> 4;           // key / value lanes: request bs + rr
    const int role = (lane >> 3) & 1;   // 0: key head, 1: value head
    const int kvhead = p.hq + role * p.hkv + g;
    int first = p1;   // the first page of the range that receives a token
    for (int bs = b; bs < B; bs += 4) {
      const int bb = bs + rr;
      const bool in = bb < B;
      int s0 = g0_s0, s1 = g0_s1, L = g0_L;   // the first group's came with the lookup
      if (bs != b) {
        s0 = in ? p.page_indptr[bb] : p1;
        s1 = in ? p.page_indptr[bb + 1] : p1;
        L = in ? p.kv_len[bb] : 0;
      }
      if (__builtin_amdgcn_readfirstlane(s0) >= p1) break;   // request bs starts past the range
      // queries: the group's requests that have pages in the range and a
      // table row for their new token
      bool qok[4];
      int qpos[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rs0 = __builtin_amdgcn_readlane(s0, 16 * r);
        const int rs1 = __builtin_amdgcn_readlane(s1, 16 * r);
        const int rL = __builtin_amdgcn_readlane(L, 16 * r);
        qok[r] = bs + r < B && rs0 < p1 && rs1 > p0 && rs1 > rs0 && rL >= 1 && rL <= p.max_pos;
        qpos[r] = qok[r] ? rL - 1 : 0;
      }
      u32x2 qx0[4][kPasses], qx1[4][kPasses];
      f32x4 qc[4], qs[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!qok[r]) continue;
        const float* cs = p.table + (int64_t)qpos[r] * kD + 4 * j;
        qc[r] = *reinterpret_cast<const f32x4*>(cs);
        qs[r] = *reinterpret_cast<const f32x4*>(cs + 32);
#pragma unroll
        for (int hp = 0; hp < kPasses; ++hp) {
          const int head = g * G + min(8 * hp + hs, G - 1);
          const uint16_t* src = p.qkv + (int64_t)(bs + r) * row_elems + (int64_t)head * kD;
          qx0[r][hp] = ld8(src + off0);
          qx1[r][hp] = ld8(src + off1);
        }
      }
      // keys and values: lanes of request bb whose new slot is in the range
      const int pos = L - 1;
      const int pi = s0 + (pos >> 4);
      const bool mine = in && L >= 1 && L <= p.max_pos && pi < s1 && pi >= p0 && pi < p1;
      const uint64_t owners = __ballot(mine);
      u32x2 kx0 = zero2, kx1 = zero2, kb0 = zero2, kb1 = zero2;
      f32x4 kc = {0.f, 0.f, 0.f, 0.f}, ks = kc;
      uint32_t page = 0;
      if (mine) {
        const uint16_t* src = p.qkv + (int64_t)bb * row_elems + (int64_t)kvhead * kD;
        kx0 = ld8(src + off0);
        kx1 = ld8(src + off1);
        if (p.bias != nullptr) {
          kb0 = ld8(p.bias + (int64_t)kvhead * kD + off0);
          kb1 = ld8(p.bias + (int64_t)kvhead * kD + off1);
        }
        if (role == 0) {
          const float* cs = p.table + (int64_t)pos * kD + 4 * j;
          kc = *reinterpret_cast<const f32x4*>(cs);
          ks = *reinterpret_cast<const f32x4*>(cs + 32);
        }
        page = (uint32_t)p.page_indices[pi];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!qok[r]) continue;
#pragma unroll
        for (int hp = 0; hp < kPasses; ++hp) {
          if (8 * hp + hs >= G) continue;
          const int head = g * G + 8 * hp + hs;
          new_piece(qx0[r][hp], qx1[r][hp], qb0[hp], qb1[hp], true, qc[r], qs[r], p.interleaved,
                    p.q_new + ((int64_t)(bs + r) * p.hq + head) * kD, off0, off1);
        }
      }
      if (owners != 0) {
        // requests are in page order: the group's first owner has the lowest page
        first = min(first, __builtin_amdgcn_readlane(pi, __builtin_ctzll(owners)));
        if (mine)
          new_piece(kx0, kx1, kb0, kb1, role == 0, kc, ks, p.interleaved,
                    (role == 0 ? p.k_new : p.v_new) +
                        (((int64_t)page * p.hkv + g) * kPage + (pos & (kPage - 1))) * kD,
                    off0, off1);
      }
    }
    wait_vmem<0>();
    asm volatile("" ::: "memory");
    first = __builtin_amdgcn_readfirstlane(first);
    if (first < p0 + 2) issue_step(ra, 0);
  };

  u32x4 qa, qc;
  if constexpr (STEP) {
    // the first step's loads are in flight while the new tokens are
    // appended and the queries rotated (into the buffer q_of reads)
    append_step();
    __builtin_amdgcn_sched_barrier(0);
  }
  q_of(b, qa, qc);
  settle(qa);
  settle(qc);
  // The next request's end, length and query, fetched at every segment
  // start and used when the segment ends: crossing into a request that has
  // pages costs no round trip.
  int nx_end, nx_L;
  u32x4 nqa, nqc;
  auto prefetch_next = [&]() __attribute__((always_inline)) {
    const int bn = min(b + 1, B - 1);
    nx_end = p.page_indptr[min(b + 2, B)];
    nx_L = p.kv_len[bn];
    q_of(bn, nqa, nqc);
  };
  prefetch_next();

  float m, d;
  f32x4 o0, o1, o2, o3;
  // Online state in log2 units; a segment that holds its request's first
  // page starts at the sink (m = sigma log2 e, d = 1 on one lane group).
  auto reset = [&](bool with_sink) __attribute__((always_inline)) {
    m = with_sink ? sink * kLog2e : -INFINITY;
    d = (with_sink && grp == 0 && sink != -INFINITY) ? 1.f : 0.f;
    o0 = f32x4{0.f, 0.f, 0.f, 0.f};
    o1 = o0; o2 = o0; o3 = o0;
  };
  reset(p0 == seg_start);

  uint16_t* my_v = lds_v + wave * kWaveLds;

  // Close the current segment (request b over this range's pages).
  auto flush = [&]() __attribute__((always_inline)) {
    float dt = d + xor_lane(d, 16);
    dt += xor_lane(dt, 32);
    const float inv = dt > 0.f ? 1.f / dt : 0.f;
    const float lse2 = dt > 0.f ? m + __builtin_amdgcn_logf(dt) : -INFINITY;
    const bool whole = (seg_start / Rw == (seg_end - 1) / Rw);   // one range holds it
    if (!live_col) return;
    const f32x4 r0 = o0 * inv, r1 = o1 * inv, r2 = o2 * inv, r3 = o3 * inv;
    if (whole) {
      const int64_t ob_off = ((int64_t)b * p.hq + h) * kD + 4 * grp;
      if (p.out_f32) {
        float* ob = reinterpret_cast<float*>(p.out) + ob_off;
        *reinterpret_cast<f32x4*>(ob) = r0;
        *reinterpret_cast<f32x4*>(ob + 16) = r1;
        *reinterpret_cast<f32x4*>(ob + 32) = r2;
        *reinterpret_cast<f32x4*>(ob + 48) = r3;
      } else {
        uint16_t* ob = reinterpret_cast<uint16_t*>(p.out) + ob_off;
        *reinterpret_cast<u32x2*>(ob) = u32x2{pack_bf16x2(r0[0], r0[1]), pack_bf16x2(r0[2], r0[3])};
        *reinterpret_cast<u32x2*>(ob + 16) = u32x2{pack_bf16x2(r1[0], r1[1]), pack_bf16x2(r1[2], r1[3])};
        *reinterpret_cast<u32x2*>(ob + 32) = u32x2{pack_bf16x2(r2[0], r2[1]), pack_bf16x2(r2[2], r2[3])};
        *reinterpret_cast<u32x2*>(ob + 48) = u32x2{pack_bf16x2(r3[0], r3[1]), pack_bf16x2(r3[2], r3[3])};
      }
      if (p.lse != nullptr && grp == 0) p.lse[(int64_t)b * p.hq + h] = lse2 * kLn2;
    } else {
      const int64_t slot = (int64_t)u + b;
      float* ob = p.o_part + (slot * p.hq + h) * kD + 4 * grp;
      *reinterpret_cast<f32x4*>(ob) = r0;
      *reinterpret_cast<f32x4*>(ob + 16) = r1;
      *reinterpret_cast<f32x4*>(ob + 32) = r2;
      *reinterpret_cast<f32x4*>(ob + 48) = r3;
      if (grp == 0) p.lse_part[slot * p.hq + h] = lse2 * kLn2;
    }
  };

  // Move to the request that owns page pg = seg_end, the current request's
  // end, and start a segment there (it holds that request's first page, so
  // it carries the sink).  Usually request b + 1, whose end, length and
  // query were prefetched (`use_prefetch`); after requests without pages, or
  // when the prefetch was issued within the same step, a lookup.  Either
  // branch leaves no load pending except the new prefetch, so the waits of
  // the step code never depend on which branch ran.
  auto advance = [&](int pg, bool use_prefetch) __attribute__((always_inline)) {
    const int ne = use_prefetch ? __builtin_amdgcn_readfirstlane(nx_end) : 0;
    if (use_prefetch && ne > seg_end) {
      b = b + 1;
      seg_start = seg_end;
      seg_end = ne;
      Lb = __builtin_amdgcn_readfirstlane(nx_L);
      qa = nqa;
      qc = nqc;
    } else {
      b = find_request(p.page_indptr, B, pg, lane);
      seg_start = __builtin_amdgcn_readfirstlane(p.page_indptr[b]);
      seg_end = __builtin_amdgcn_readfirstlane(p.page_indptr[b + 1]);
      Lb = __builtin_amdgcn_readfirstlane(p.kv_len[b]);
      q_of(b, qa, qc);
      settle(qa);
      settle(qc);
    }
    reset(true);
    prefetch_next();
  };

  // One pass over a step's two pages (global pages pa, pa + 1) for the
  // current request; use_a / use_b select the pages that belong to it.
  // na / nb: keys of page a / b that exist (the rest, and every key of a
  // page that is not used, are masked and their V rows zeroed).
  auto process = [&](const StepRegs& r, int pa, bool use_a,
                     bool use_b) __attribute__((always_inline)) {
    const int key_a = (pa - seg_start) * kPage;   // request position of page a's key 0
    const int na = use_a ? Lb - key_a : 0;
    const int nb = use_b ? Lb - key_a - kPage : 0;
    {
      const int row = lane >> 2;
      const bool da = row >= na;
      const bool db = row >= nb;
      uint16_t* r0 = my_v + row * kVPitch + 16 * (lane & 3);
      uint16_t* r1 = r0 + kPage * kVPitch;
      *reinterpret_cast<u32x4*>(r0) = da ? zero4 : r.v00;
      *reinterpret_cast<u32x4*>(r0 + 8) = da ? zero4 : r.v01;
      *reinterpret_cast<u32x4*>(r1) = db ? zero4 : r.v10;
      *reinterpret_cast<u32x4*>(r1 + 8) = db ? zero4 : r.v11;
    }
    const bf16x8 bq0 = as_bf16x8(live_col ? qa : zero4);
    const bf16x8 bq1 = as_bf16x8(live_col ? qc : zero4);
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
    s0 = mfma16(as_bf16x8(r.k00), bq0, s0);
    s1 = mfma16(as_bf16x8(r.k10), bq0, s1);
    s0 = mfma16(as_bf16x8(r.k01), bq1, s0);
    s1 = mfma16(as_bf16x8(r.k11), bq1, s1);
    float sc[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = (4 * grp + i < na) ? s0[i] * p.scale_log2 : -INFINITY;
      sc[4 + i] = (4 * grp + i < nb) ? s1[i] * p.scale_log2 : -INFINITY;
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
    // V^T operand per 16-dim block: source lane s of group grp points at key
    // 4 grp + s / 4 of each page, dims 16 db + 4 (s % 4)
    const uint16_t* src = my_v + (4 * grp + (col >> 2)) * kVPitch + 4 * (col & 3);
    o0 = mfma16(as_bf16x8(lds_tr16_pair(src, src + kPage * kVPitch)), pb, o0);
    o1 = mfma16(as_bf16x8(lds_tr16_pair(src + 16, src + kPage * kVPitch + 16)), pb, o1);
    o2 = mfma16(as_bf16x8(lds_tr16_pair(src + 32, src + kPage * kVPitch + 32)), pb, o2);
    o3 = mfma16(as_bf16x8(lds_tr16_pair(src + 48, src + kPage * kVPitch + 48)), pb, o3);
  };

  // A step: pages pa and pa + 1 (the second may lie past the range).  A
  // request may end exactly before the step (its end was the previous
  // step's last page) and/or between the step's two pages (the step
  // straddles): each case is its own path, and only the first segment
  // change of a step uses the prefetch.
  auto step_body = [&](const StepRegs& r, int pa) __attribute__((always_inline)) {
    // The next-request prefetch went out before the K/V loads of the other
    // register set, so completing it here waits for nothing this step's
    // own data does not already wait for.
    settle(nx_end);
    settle(nx_L);
    settle(nqa);
    settle(nqc);
    const bool has_b = pa + 1 < p1;
    if (pa >= seg_end) {
      flush();
      advance(pa, true);
      if (has_b && pa + 1 >= seg_end) {   // a one-page request
        process(r, pa, true, false);
        flush();
        advance(pa + 1, false);
        process(r, pa, false, true);
      } else {
        process(r, pa, true, has_b);
      }
    } else if (has_b && pa + 1 >= seg_end) {   // straddles a request boundary
      process(r, pa, true, false);
      flush();
      advance(pa + 1, true);
      // the new segment starts at page pa + 1: keys of page "a" precede it
      process(r, pa, false, true);
    } else {
      process(r, pa, true, has_b);
    }
  };

  // Two register sets in flight: step s + 1 is issued before step s is
  // processed, step s + 2 before step s + 1.  Every issue is unconditional
  // (clamped to the last step), so the waits stay exact.
  for (int s = 0; s < n_steps; s += 2) {
    issue_step(rb, s + 1);
    __builtin_amdgcn_sched_barrier(0);
    step_body(ra, p0 + 2 * s);
    __builtin_amdgcn_sched_barrier(0);
    const bool rotate = s + 2 - base == 32;   // step s + 2 opens the next block
    int ids_new = 0;
    if (rotate) ids_new = load_ids(base + 64);
    issue_step(ra, s + 2);
    if (rotate) {
      base += 32;
      ids = ids_next;
      ids_next = ids_new;
    }
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < n_steps) step_body(rb, p0 + 2 * (s + 1));
    __builtin_amdgcn_sched_barrier(0);
  }
  flush();
}

// One wave per (request, query head): lane = dim.  Merges the partials of a
// request that spans several ranges: L = max lse_c, w_c = exp(lse_c - L),
// o = sum w_c o_c / sum w_c, lse = L + ln sum w_c; writes requests without
// pages.  All loads of one (request, head) go out together: the lse values
// lane-parallel, the first eight partial rows unconditionally.
__global__ __launch_bounds__(256) void decode_finish_kernel(BalancedDecodeArgs p) {
  const int lane = thread_x() & 63;
  const int64_t pair = (int64_t)block_x() * 4 + __builtin_amdgcn_readfirstlane(thread_x() >> 6);
  if (pair >= (int64_t)p.batch * p.hq) return;
  const int b = (int)(pair / p.hq);
  const int h = (int)(pair % p.hq);
  const int nnz = __builtin_amdgcn_readfirstlane(p.page_indptr[p.batch]);
  const int s0 = __builtin_amdgcn_readfirstlane(p.page_indptr[b]);
  const int s1 = __builtin_amdgcn_readfirstlane(p.page_indptr[b + 1]);
  const int Rw = range_width(nnz, p.n_ranges, p.min_range_pages);
  const int64_t obase = pair * kD + lane;
  if (s1 <= s0) {   // no pages: no keys
    if (p.out_f32) reinterpret_cast<float*>(p.out)[obase] = 0.f;
    else reinterpret_cast<uint16_t*>(p.out)[obase] = 0;
    if (p.lse != nullptr && lane == 0) p.lse[pair] = p.sinks ? p.sinks[h] : -INFINITY;
    return;
  }
  const int u0 = s0 / Rw, u1 = (s1 - 1) / Rw;
  if (u0 == u1) return;   // written by the first pass
  const int n = u1 - u0 + 1;
  const int64_t row0 = ((int64_t)u0 + b) * p.hq + h;   // slot u0 + b + c -> row0 + c * hq
  constexpr int kPre = 8;
  float ov[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) ov[j] = p.o_part[(row0 + (int64_t)min(j, n - 1) * p.hq) * kD + lane];
  if (n <= kPre) {
    // the usual case: every lane loads the n log-sum-exps itself (the same
    // addresses in every lane) and merges its dimension with no exchange
    float lv[kPre];
#pragma unroll
    for (int j = 0; j < kPre; ++j) lv[j] = p.lse_part[row0 + (int64_t)min(j, n - 1) * p.hq];
    float Lm = -INFINITY;
#pragma unroll
    for (int j = 0; j < kPre; ++j) Lm = j < n ? fmaxf(Lm, lv[j]) : Lm;
    float den = 0.f, acc = 0.f;
    if (Lm != -INFINITY) {
#pragma unroll
      for (int j = 0; j < kPre; ++j) {
        float w = (Lm == INFINITY) ? (lv[j] == INFINITY ? 1.f : 0.f) : __expf(lv[j] - Lm);
        w = j < n ? w : 0.f;
        den += w;
        acc += w != 0.f ? w * ov[j] : 0.f;
      }
    }
    const float o = den > 0.f ? acc / den : 0.f;
    if (p.out_f32) reinterpret_cast<float*>(p.out)[obase] = o;
    else reinterpret_cast<uint16_t*>(p.out)[obase] = float_to_bf16_bits(o);
    if (p.lse != nullptr && lane == 0) {
      float l;
      if (Lm == -INFINITY) l = -INFINITY;
      else if (Lm == INFINITY) l = INFINITY;
      else l = Lm + __logf(den);
      p.lse[pair] = l;
    }
    return;
  }
  // more partials: log-sum-exp over them 64 at a time across lanes
  float L = -INFINITY;
  for (int cb = 0; cb < n; cb += 64) {
    const int c = min(cb + lane, n - 1);
    L = fmaxf(L, p.lse_part[row0 + (int64_t)c * p.hq]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) L = fmaxf(L, xor_lane(L, off));
  float den = 0.f, acc = 0.f;
  if (L != -INFINITY) {
    for (int cb = 0; cb < n; cb += 64) {
      const int c = cb + lane;
      const float lc = p.lse_part[row0 + (int64_t)min(c, n - 1) * p.hq];
      float w = (L == INFINITY) ? (lc == INFINITY ? 1.f : 0.f) : __expf(lc - L);
      w = c < n ? w : 0.f;
      float ws = w;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) ws += xor_lane(ws, off);
      den += ws;
      const int cn = min(64, n - cb);
      int j = 0;
      if (cb == 0) {
#pragma unroll
        for (; j < kPre; ++j) {
          const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                         __builtin_bit_cast(int, w), j));
          acc += (j < cn && wj != 0.f) ? wj * ov[j] : 0.f;
        }
      }
      for (; j < cn; j += 8) {   // eight rows in flight (clamped; extras weigh 0)
        float oj[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
          oj[t] = p.o_part[(row0 + (int64_t)(cb + min(j + t, cn - 1)) * p.hq) * kD + lane];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                         __builtin_bit_cast(int, w), min(j + t, 63)));
          acc += (j + t < cn && wj != 0.f) ? wj * oj[t] : 0.f;
        }
      }
    }
  }
  const float o = den > 0.f ? acc / den : 0.f;
  if (p.out_f32) reinterpret_cast<float*>(p.out)[obase] = o;
  else reinterpret_cast<uint16_t*>(p.out)[obase] = float_to_bf16_bits(o);
  if (p.lse != nullptr && lane == 0) {
    float l;
    if (L == -INFINITY) l = -INFINITY;
    else if (L == INFINITY) l = INFINITY;
    else l = L + __logf(den);
    p.lse[pair] = l;
  }
}

}  // namespace

namespace {
template <bool STEP>
hipError_t launch_first_pass(const BalancedDecodeArgs& a, int group, hipStream_t stream) {
  dim3 grid(a.n_ranges / kWaves, a.hkv);
  dim3 block(256);
  switch (group) {
    case 1: hipLaunchKernelGGL((decode_balanced_kernel<1, STEP>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_balanced_kernel<2, STEP>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_balanced_kernel<4, STEP>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((decode_balanced_kernel<8, STEP>), grid, block, 0, stream, a); break;
    case 16: hipLaunchKernelGGL((decode_balanced_kernel<16, STEP>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_balanced(const BalancedDecodeArgs& a, int group, hipStream_t stream) {
  return a.qkv != nullptr ? launch_first_pass<true>(a, group, stream)
                          : launch_first_pass<false>(a, group, stream);
}

hipError_t launch_decode_finish(const BalancedDecodeArgs& a, hipStream_t stream) {
  const int64_t pairs = (int64_t)a.batch * a.hq;
  if (pairs == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_finish_kernel, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace sa
