// Wide drafted-token verification with a per-head sink (gfx950): the
// drafted tokens x query heads of a request form up to 128-row tiles that
// stream its paged KV cache through LDS, split along the KV length.
//
// GPT-OSS on Day 0 (Perplexity), "Sink attention" under "Kernels for
// GPT-OSS": the sink is an extra logit per head, folded into the online
// softmax by starting the running maximum at the sink with d = 1; work is
// parallel over heads and along the KV length, and when the KV sequence is
// split only the first chunk carries the sink.  "Accelerating Sonar Through
// Speculation" (Perplexity), "Speculative Decoding" and "MTP": the target
// model runs once over each request's drafted tokens; "EAGLE": tree drafts
// are checked under custom attention masks.
//
// One workgroup = (request b, KV head g, KV chunk c, row tile rt), four
// waves.  Row rho = 128 rt + 32 w + (lane % 32) of wave w is drafted token
// t = rho / G with query head g G + rho % G; rows past qlen_b G are padding.
// Token t sits at position P + t, P = kv_len - qlen, and sees keys 0 .. P + t
// (bottom-right causal alignment), or, with a draft mask, every key below P
// plus drafted key P + i when bit i of its word is set.
//
// Chunk c covers the 64-key tiles c Ct .. c Ct + Ct - 1 of the request.  The
// workgroup loads each tile's K and V straight into LDS (three buffers, the
// next two tiles in flight while one is computed), and every wave computes
// on it:
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 for the tile's two 32-key
//     halves, so a lane holds 16 scores of one row per half;
//   * the halves are interleaved: the scores of half 1 are computed while
//     half 0 is exponentiated, and O^T += V^T P^T of half 0 runs while half
//     1 is exponentiated (V^T read transposed with ds_read_b64_tr_b16 in
//     the key order of the score layout, P^T straight from registers);
//   * softmax against a per-row reference maximum: exp2(s scale - m) with
//     one FMA; only when a lane's partial sum of a half passes 2^15, or the
//     row has no reference yet, does a wave-uniform slow path take the true
//     maximum and rescale d and O;
//   * masks run only on tiles that reach the drafted keys or the end of
//     the cache.
// A request that fits in one chunk writes its rows; a longer one writes a
// normalised partial (o, lse) per chunk, which verify_tile_finish merges.
#include "common.hpp"
#include "launch.hpp"

namespace sa {
namespace {

constexpr int kD = 64;
constexpr int kTile = 64;             // keys per tile
constexpr int kRows = 128;            // rows per workgroup (4 waves x 32)
constexpr int kTileBytes = kTile * kD * 2;  // one K or V tile in LDS, rows unpadded
constexpr int kBufs = 3;                    // LDS tile buffers
constexpr float kFastLimit = 32768.f; // lane-partial half-tile sum that forces a rescale

// acc + lo(w) + hi(w) for a packed bf16 pair, accumulated in fp32.
__device__ __forceinline__ float dot2_sum(uint32_t w, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

__device__ __forceinline__ int n_chunks_of(int L, int chunk_tiles) {
  const int tiles = (L + kTile - 1) / kTile;
  return (tiles + chunk_tiles - 1) / chunk_tiles;
}

typedef __attribute__((address_space(3))) int lds_int;

// Inclusive prefix sum over the 64 lanes on the vector unit (wave-uniform
// control flow): shifts by 1, 2, 4 and 8 lanes inside each 16-lane row, then
// lane 15 of each row added into the next row and lane 31 into the upper two
// rows (the row_shr and row_bcast forms of DPP); lanes without a source add
// 0.  No LDS round trips, unlike a ds_bpermute ladder.
__device__ __forceinline__ int wave_prefix_sum(int v, int) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}

// Longest-first order of the work items (request b, KV head g, chunk c).
// An item's length is its chunk's tile count: every chunk but a request's
// last is full (chunk_tiles tiles); the last holds the rest.  The order:
// all full chunks, then the last chunks by decreasing length (quantised to
// 64 levels of chunk_tiles), each group in (request, chunk, KV head) order;
// items of requests without drafted tokens are left out.  Workgroups are
// dispatched in index order, so the long items start first and the short
// ones fill the tail (list scheduling, longest first).  Every wave of the
// workgroup computes the same item from the request lengths, with no
// exchange; hist is this wave's 64-entry LDS histogram.  Returns false
// when rank i is past the last item.
__device__ __forceinline__ bool longest_first_item(const VerifyTileArgs& p, int i, int lane,
                                                   lds_int* hist, int& item) {
  const int B = p.batch;
  const int ct = p.chunk_tiles;
  const int nb = (B + 63) >> 6;
  int q0[4], q1[4], len[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = 64 * k + lane;
    const bool in = k < nb && r < B;
    q0[k] = in ? p.qo_indptr[r] : 0;
    q1[k] = in ? p.qo_indptr[r + 1] : 0;
    len[k] = in ? p.kv_len[r] : 0;
  }
  // per request (lane, block k): full chunks nf, the last chunk's level lv
  // (-1 if the request has no partial chunk) and w = items per chunk
  int nf[4], lv[4], w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int tiles = (len[k] + kTile - 1) / kTile;
    nf[k] = tiles / ct;
    const int part = tiles - nf[k] * ct;
    lv[k] = part > 0 ? (part * 64 - 1) / ct : -1;
    w[k] = q1[k] > q0[k] ? p.hkv : 0;
  }
  int idx = i;
  bool found = false, full = false;
  int r_sel = 0, off = 0, w_sel = 1, nf_sel = 0;
  // full chunks
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (k < nb && !found) {
      const int c = nf[k] * w[k];
      const int incl = wave_prefix_sum(c, lane);
      const int tot = __builtin_amdgcn_readlane(incl, 63);
      if (idx < tot) {
        const int ln = __builtin_ctzll(__ballot(incl > idx));
        off = idx - __builtin_amdgcn_readlane(incl - c, ln);
        r_sel = 64 * k + ln;
        w_sel = __builtin_amdgcn_readlane(w[k], ln);
        nf_sel = __builtin_amdgcn_readlane(nf[k], ln);
        full = true;
        found = true;
      } else {
        idx -= tot;
      }
    }
  }
  if (!found) {
    // last chunks: a histogram of jobs by level, levels taken from the top
    hist[lane] = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (lv[k] >= 0 && w[k] > 0)
        __hip_atomic_fetch_add(hist + lv[k], w[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const int h = hist[lane];
    const int pre = wave_prefix_sum(h, lane);
    const int total = __builtin_amdgcn_readlane(pre, 63);
    if (idx >= total) return false;
    const int above = total - pre;   // jobs on higher levels
    const int jb = __builtin_ctzll(__ballot(h > 0 && above <= idx && idx < above + h));
    idx -= __builtin_amdgcn_readlane(above, jb);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k < nb && !found) {
        const int c = lv[k] == jb ? w[k] : 0;
        const int incl = wave_prefix_sum(c, lane);
        const int tot = __builtin_amdgcn_readlane(incl, 63);
        if (idx < tot) {
          const int ln = __builtin_ctzll(__ballot(incl > idx));
          off = idx - __builtin_amdgcn_readlane(incl - c, ln);
          r_sel = 64 * k + ln;
          w_sel = __builtin_amdgcn_readlane(w[k], ln);
          nf_sel = __builtin_amdgcn_readlane(nf[k], ln);
          found = true;
        } else {
          idx -= tot;
        }
      }
    }
    if (!found) return false;
  }
  const int chunk = full ? off / w_sel : nf_sel;
  const int g = off - (off / w_sel) * w_sel;
  item = chunk * (p.batch * p.hkv) + r_sel * p.hkv + g;
  return true;
}

template <int G, bool TREE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void verify_tile_kernel(VerifyTileArgs p) {
  __shared__ __attribute__((aligned(1024))) char lds_k[kBufs * kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v[kBufs * kTileBytes];
  __shared__ int lds_hist[4][64];

  // flat index -> (item slot, row tile rt): the row tiles of one slot go to
  // the same XCD (workgroups are dealt to the 8 XCDs round robin), back to
  // back, so their reads of the same pages meet in that XCD's L2.  Slot ->
  // work item (c * B * Hkv + unit): longest first for batches of up to 256
  // requests (longest_first_item), else the slot itself.
  const int n_units = p.batch * p.hkv;
  const int xcd = block_x() & 7;
  const int rest = block_x() >> 3;
  const int rt = rest % p.row_tiles;
  const int slot = (rest / p.row_tiles) * 8 + xcd;
  int item = slot;
  if (p.longest_first) {
    const int ln = thread_x() & 63;
    lds_int* hist = (lds_int*)lds_hist[thread_x() >> 6];
    if (!longest_first_item(p, slot, ln, hist, item)) return;
  }
  if (item >= n_units * p.max_chunks) return;
  const int unit = item % n_units;
  const int c = item / n_units;
  const int g = unit % p.hkv;
  const int b = unit / p.hkv;

  const int q0 = p.qo_indptr[b];
  const int qlen = p.qo_indptr[b + 1] - q0;
  const int n_rows = qlen * G;
  if (kRows * rt >= n_rows) return;
  const int L = p.kv_len[b];
  const int n_chunks = n_chunks_of(L, p.chunk_tiles);
  if (c >= n_chunks) return;
  const int n_tiles_all = (L + kTile - 1) / kTile;
  const int tile0 = c * p.chunk_tiles;
  const int n_tiles = min(n_tiles_all - tile0, p.chunk_tiles);
  const int P = L - qlen;          // keys below P: the cached prefix
  const int kv_start = p.page_indptr[b];

  const int tid = thread_x();
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 31;
  const int hh = lane >> 5;

  // ---- this lane's row ----
  const int rho = kRows * rt + 32 * wave + r;
  const bool valid = rho < n_rows;
  const int t = valid ? rho / G : 0;
  const int head = g * G + rho % G;
  bf16x8 bq[4];
  {
    const uint16_t* qrow = p.q + ((int64_t)(q0 + t) * p.hq + head) * kD + 8 * hh;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int s = 0; s < 4; ++s) bq[s] = as_bf16x8(valid ? ld16(qrow + 16 * s) : z);
  }
  uint32_t mlo = 0u, mhi = 0u;
  if (TREE && valid) {
    const uint64_t w = p.draft_mask[q0 + t];
    mlo = (uint32_t)w;
    mhi = (uint32_t)(w >> 32);
  }
  // causal limit of the row: keys <= lim are visible
  const int lim = P + t;

  // ---- online state (log2 units); chunk 0 starts at the sink.  Padding
  // rows get a finite reference, so they never take the slow path. ----
  float m = valid ? -INFINITY : 0.f;
  float d = 0.f;
  if (valid && c == 0 && p.sinks != nullptr) {
    const float sg = p.sinks[head];
    m = sg * kLog2e;
    d = (hh == 0 && sg != -INFINITY) ? 1.f : 0.f;
  }
  f32x16 o[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[db][j] = 0.f;

  // ---- tile loader.  A tile's K and V go straight from global memory
  // into LDS, 1 KiB blocks of eight key rows (key row r in block r / 8).
  // Wave w loads page w of every tile: K and V rows 16 w .. 16 w + 15, two
  // blocks each, one page id (wave-uniform, a scalar load) and a fixed
  // offset per lane inside the page.  The lane -> (row, 16-byte chunk) map
  // of a block lays it out as the operand reads want it (chunk c of row
  // r' = r % 8, e = (r / 8) % 2):
  //   K: slot 16 (c / 2) + ((2 r' + c % 2 + e) mod 16), so the 16 rows of
  //      one K-operand read fall in 16 different bank groups and k-step s
  //      is a constant offset;
  //   V: slot 16 (c / 4 + 2 (r' / 4)) + 4 (r' % 4) + c % 4, so the four
  //      rows x four chunks of one transposed read fall in 16 different
  //      bank groups and every V^T operand is a constant offset.
  // Rows past the last key read the first row of their page (a page past
  // the request's end is replaced by its first page), a key of the request
  // and so finite: their scores are masked, so P is 0 for them. ----
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t page_bytes = (uint32_t)p.hkv * 16 * kD * 2;   // one page, every KV head
  const char* kbytes = reinterpret_cast<const char*>(p.k);
  const char* vbytes = reinterpret_cast<const char*>(p.v);
  const int32_t* pages = p.page_indices + kv_start;
  uint32_t koff[2], voff[2], kzero[2], vzero[2];
  int krow[2], vrow[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int x = ((lane & 15) - e) & 15;
    const int kc = 2 * (lane >> 4) + (x & 1);
    krow[e] = 8 * e + (x >> 1);
    koff[e] = (uint32_t)g * 16 * kD * 2 + krow[e] * kD * 2 + 16 * kc;
    kzero[e] = (uint32_t)g * 16 * kD * 2 + 16 * kc;
    const int vc = 4 * ((lane >> 4) & 1) + (lane & 3);
    vrow[e] = 8 * e + 4 * (lane >> 5) + ((lane & 15) >> 2);
    voff[e] = (uint32_t)g * 16 * kD * 2 + vrow[e] * kD * 2 + 16 * vc;
    vzero[e] = (uint32_t)g * 16 * kD * 2 + 16 * vc;
  }
  auto tile_key0 = [&](int kt) { return (tile0 + kt) * kTile; };
  // Page ids of this wave's page in tiles first .. first + 63, one per lane,
  // loaded together and read out with v_readlane (a wave-uniform value);
  // the assembly use makes the compiler wait for them right here.
  auto load_ids = [&](int first) {
    const int kt = first + lane;
    int id = 0;
    if (kt < n_tiles) {
      const int key0 = tile_key0(kt);
      id = pages[key0 + 16 * wave_u < L ? (key0 >> 4) + wave_u : 0];
    }
    asm volatile("" ::"v"(id));
    return id;
  };
  auto issue = [&](int kt, int bf, int id) {
    const int key0 = tile_key0(kt);
    const char* kp = kbytes + (uint64_t)(uint32_t)id * page_bytes;
    const char* vp = vbytes + (uint64_t)(uint32_t)id * page_bytes;
    const uint32_t kd = lds_offset(lds_k) + bf * kTileBytes + wave_u * 2048;
    const uint32_t vd = lds_offset(lds_v) + bf * kTileBytes + wave_u * 2048;
    const bool tail = key0 + kTile > L;   // wave-uniform: only the last tile
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      uint32_t ko = koff[e], vo = voff[e];
      if (tail) {
        const int row0 = key0 + 16 * wave_u;
        ko = row0 + krow[e] < L ? ko : kzero[e];
        vo = row0 + vrow[e] < L ? vo : vzero[e];
      }
      load_lds16(kp, ko, kd + 1024 * e);
      load_lds16(vp, vo, vd + 1024 * e);
    }
  };

  // the prologue's own global loads complete here, not inside the loop
  asm volatile("" ::"v"(bq[0]), "v"(bq[1]), "v"(bq[2]), "v"(bq[3]));
  int ids = load_ids(0);
  issue(0, 0, __builtin_amdgcn_readlane(ids, 0));
  if (n_tiles > 1) issue(1, 1, __builtin_amdgcn_readlane(ids, 1));

  const float sl2 = p.scale_log2;
  // Operand reads, byte offsets inside a tile buffer.  K operand of k-step
  // s, half kb: key 32 kb + r, dims 16 s + 8 hh (chunk 2 s + hh) at
  // kread + 4096 kb + 256 s.  V^T operand: the transposed read of 16-lane
  // group q = lane / 16 covers dims 16 (q % 2) + 4 (lane % 4) .. of a 32-dim
  // block db (chunk 2 (q % 2) + (lane % 4) / 2 + 4 db) and key row
  // 4 hh + (lane % 16) / 4 (+ 8 for the upper four values) of the 16-key
  // slice hf of half kb, at vread + 4096 kb + 2048 hf + 256 db (+ 1024).
  const int kread = ((lane & 31) >> 3) * 1024 + 16 * ((2 * (lane & 7) + hh + ((lane >> 3) & 1)) & 15);
  const int vread = 512 * hh + 64 * ((lane & 15) >> 2) + 16 * (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) +
                    8 * (lane & 1);

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt % kBufs;
    // this wave's part of tile kt has landed (tile kt + 1 may be in
    // flight); the barrier makes every part visible and frees the buffer of
    // tile kt - 1 for tile kt + 2
    if (kt + 1 < n_tiles) wait_vmem<4>();
    else wait_vmem<0>();
    barrier_only();
    if (kt + 2 < n_tiles) {
      if (((kt + 2) & 63) == 0) ids = load_ids(kt + 2);
      issue(kt + 2, (kt + 2) % kBufs, __builtin_amdgcn_readlane(ids, (kt + 2) & 63));
    }
    const int key0 = (tile0 + kt) * kTile;
    const char* kbuf = lds_k + buf * kTileBytes;
    // V^T reads from one LDS address per tile, hidden from loop strength
    // reduction, so that each read's constant part becomes its offset
    uint32_t vaddr = lds_offset(lds_v) + buf * kTileBytes + vread;
    asm volatile("" : "+v"(vaddr));
    const __attribute__((address_space(3))) char* vbuf =
        (const __attribute__((address_space(3))) char*)(uintptr_t)vaddr;
    // tiles that reach the drafted keys (from P) or the end of the cache
    const bool edge = key0 + kTile > P;
    const f32x16 zero16 = {};

    // K operand (A of S^T) for k-step s, half kb: keys 32 kb + r, dims
    // 16 s + 8 hh.  V^T operand (A of O^T) for half kb, k-step hf, dim
    // block db: dims 32 db + .., keys 32 kb + 16 hf + {4 hh .., 8 + 4 hh ..}.
    auto kop = [&](int s, int kb) {
      return as_bf16x8(*reinterpret_cast<const u32x4*>(kbuf + kread + 4096 * kb + 256 * s));
    };
    auto vop = [&](int kb, int hf, int db) {
      const auto* src = vbuf + 4096 * kb + 2048 * hf + 256 * db;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src + 1024));
      const u32x2 a = __builtin_bit_cast(u32x2, lo), b2 = __builtin_bit_cast(u32x2, hi);
      return as_bf16x8(u32x4{a[0], a[1], b2[0], b2[1]});
    };
    // S^T[kb]: keys 32 kb + 8 (j / 4) + 4 hh + j % 4, column = this row
    f32x16 sacc[2];
    uint32_t pk[2][2][4];   // [kb][hf][pair]
    auto mask = [&](int kb) {
      if (TREE) {
        // draft index of the key at offset 32 kb + 8 (j / 4) + j % 4 +
        // 4 hh: below 0 a prefix key (seen), from qlen on past the cache
        int base = key0 + 32 * kb + 4 * hh - P;
        asm volatile("" : "+v"(base));
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int jj = base + 8 * (j >> 2) + (j & 3);
          const uint32_t w = jj < 32 ? mlo : mhi;
          const bool seen = jj < 0 || (jj < qlen && ((w >> (jj & 31)) & 1u));
          if (!seen) sacc[kb][j] = -INFINITY;
        }
        return;
      }
      int rel = lim - key0 - 32 * kb - 4 * hh;
      // defined here, so the compares cannot be hoisted out of the (rare)
      // edge branch into every tile
      asm volatile("" : "+v"(rel));
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (8 * (j >> 2) + (j & 3) > rel) sacc[kb][j] = -INFINITY;
    };
    // exp2(s * scale - m) of scores j = 8 hf + 2 q, + 1 of half kb, packed;
    // the row sum adds the rounded values the MFMA consumes.
    auto expo2 = [&](float neg_m, int kb, int hf, int q, float& acc) {
      const int j = 8 * hf + 2 * q;
      const float e0 = fast_exp2(__builtin_fmaf(sacc[kb][j], sl2, neg_m));
      const float e1 = fast_exp2(__builtin_fmaf(sacc[kb][j + 1], sl2, neg_m));
      const uint32_t w = pack_bf16x2(e0, e1);
      pk[kb][hf][q] = w;
      acc = dot2_sum(w, acc);
    };
    auto neg_ref = [&]() { return (m == -INFINITY) ? 0.f : -m; };
    // Fast path: half kb was exponentiated against the reference m.  It is
    // valid while every partial sum stays below 2^15 and the row has a
    // reference; otherwise take the half's true maximum, rescale O, d and
    // m, and exponentiate again.
    auto settle = [&](int kb, float ds) {
      if (__any(!(ds <= kFastLimit) || m == -INFINITY)) {
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 16; j += 2) mx = fmaxf(fmaxf(mx, sacc[kb][j]), sacc[kb][j + 1]);
        mx = fmaxf(mx, xor_lane(mx, 32));
        const float m_new = fmaxf(m, mx * sl2);
        const float alpha = (m == m_new) ? 1.f : fast_exp2(m - m_new);
        d *= alpha;
        o[0] *= alpha;
        o[1] *= alpha;
        m = m_new;
        float a0 = 0.f, a1 = 0.f;
        const float nm = neg_ref();
#pragma unroll
        for (int i = 0; i < 8; ++i) expo2(nm, kb, i >> 2, i & 3, (i & 1) ? a1 : a0);
        ds = a0 + a1;
      }
      d += ds;
    };
    auto pb_of = [&](int kb, int hf) {
      return as_bf16x8(u32x4{pk[kb][hf][0], pk[kb][hf][1], pk[kb][hf][2], pk[kb][hf][3]});
    };

    // (1) S^T of half 0; the K operands of both halves are read once.
    bf16x8 ko[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) ko[s][kb] = kop(s, kb);
#pragma unroll
    for (int s = 0; s < 4; ++s) sacc[0] = mfma32(ko[s][0], bq[s], s == 0 ? zero16 : sacc[0]);
    if (edge) mask(0);
    // (2) S^T of half 1 on the matrix core while half 0 is exponentiated.
    {
      float a0 = 0.f, a1 = 0.f;
      const float nm = neg_ref();
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if ((i & 1) == 0) sacc[1] = mfma32(ko[i >> 1][1], bq[i >> 1], i == 0 ? zero16 : sacc[1]);
        expo2(nm, 0, i >> 2, i & 3, (i & 1) ? a1 : a0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);  // VALU
      }
      settle(0, a0 + a1);
    }
    if (edge) mask(1);
    // (3) O^T += V^T P^T of half 0 while half 1 is exponentiated.  The V^T
    //     operands of the tile are read once, at the start.
    bf16x8 vo[2][2][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) vo[i >> 2][(i >> 1) & 1][i & 1] = vop(i >> 2, (i >> 1) & 1, i & 1);
    {
      float a0 = 0.f, a1 = 0.f;
      const float nm = neg_ref();
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if ((i & 1) == 0) {
          const int hf = i >> 2, db = (i >> 1) & 1;
          o[db] = mfma32(vo[0][hf][db], pb_of(0, hf), o[db]);
        }
        expo2(nm, 1, i >> 2, i & 3, (i & 1) ? a1 : a0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);    // DS read: all of V^T
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);     // VALU
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // VALU
      }
      settle(1, a0 + a1);
    }
    // (4) O^T += V^T P^T of half 1.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hf = i >> 1, db = i & 1;
      o[db] = mfma32(vo[1][hf][db], pb_of(1, hf), o[db]);
    }
  }

  // ---- epilogue: o = O / d, lse = m + log2 d (natural log at the boundary) ----
  const float dt = d + xor_lane(d, 32);
  if (!valid) return;
  const float inv = dt > 0.f ? 1.f / dt : 0.f;
  const float lse2 = dt > 0.f ? m + __builtin_amdgcn_logf(dt) : -INFINITY;
  const int64_t pair = (int64_t)(q0 + t) * p.hq + head;
  if (n_chunks == 1) {
    const int64_t orow = pair * kD;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int dim = 32 * db + 8 * a + 4 * hh;
        const float x0 = o[db][4 * a + 0] * inv, x1 = o[db][4 * a + 1] * inv;
        const float x2 = o[db][4 * a + 2] * inv, x3 = o[db][4 * a + 3] * inv;
        if (p.out_f32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + orow + dim) =
              f32x4{x0, x1, x2, x3};
        } else {
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + orow + dim) =
              u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
        }
      }
    if (p.lse != nullptr && hh == 0) p.lse[pair] = lse2 * kLn2;
  } else {
    const int64_t slot = pair * p.max_chunks + c;
    float* op = p.o_part + slot * kD;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int dim = 32 * db + 8 * a + 4 * hh;
        *reinterpret_cast<f32x4*>(op + dim) =
            f32x4{o[db][4 * a] * inv, o[db][4 * a + 1] * inv, o[db][4 * a + 2] * inv,
                  o[db][4 * a + 3] * inv};
      }
    if (hh == 0) p.lse_part[slot] = lse2 * kLn2;
  }
}

// One workgroup per (request, drafted token).  Wave w merges head groups
// w, w + 4, ... of four query heads each; lane l takes head 4 grp + l / 16
// and dims 4 (l % 16) .. + 3 of the group.  Merges the n > 1 chunk
// partials of a request that spans several chunks by log-sum-exp (L = max
// lse_c, w_c = e^(lse_c - L), o = sum w_c o_c / sum w_c, lse = L + ln sum
// w_c); requests in one chunk were written by the first pass.  The
// log-sum-exps and 16-byte row pieces of four head groups and up to four
// chunks are loaded in one batch, all in flight together: one round trip
// after the request's lengths, and no cross-lane traffic.
__global__ __launch_bounds__(256) void verify_tile_finish_kernel(VerifyTileArgs p) {
  constexpr int kBatch = 4;   // chunks per batch of loads
  constexpr int kGroups = 4;  // head groups per wave and batch
  const int lane = thread_x() & 63;
  const int wave = __builtin_amdgcn_readfirstlane(thread_x() >> 6);
  const int b = block_x() / p.max_qlen;
  const int t = block_x() % p.max_qlen;
  const int q0 = __builtin_amdgcn_readfirstlane(p.qo_indptr[b]);
  const int qlen = __builtin_amdgcn_readfirstlane(p.qo_indptr[b + 1]) - q0;
  if (t >= qlen) return;
  const int n = n_chunks_of(__builtin_amdgcn_readfirstlane(p.kv_len[b]), p.chunk_tiles);
  if (n <= 1) return;
  const int groups = (p.hq + 3) / 4;
  const int q4 = lane & 15;
  for (int g0 = wave; g0 < groups; g0 += 4 * kGroups) {
    int64_t pair[kGroups];
    bool live[kGroups];
    float lv[kGroups][kBatch];
    f32x4 ov[kGroups][kBatch];
#pragma unroll
    for (int i = 0; i < kGroups; ++i) {
      const int h = 4 * (g0 + 4 * i) + (lane >> 4);
      live[i] = g0 + 4 * i < groups && h < p.hq;
      pair[i] = (int64_t)(q0 + t) * p.hq + (live[i] ? h : 0);
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int64_t slot = pair[i] * p.max_chunks + min(j, n - 1);
        lv[i][j] = p.lse_part[slot];
        ov[i][j] = *reinterpret_cast<const f32x4*>(p.o_part + slot * kD + 4 * q4);
      }
    }
#pragma unroll
    for (int i = 0; i < kGroups; ++i) {
      if (!live[i]) continue;
      const float* ls = p.lse_part + pair[i] * p.max_chunks;
      const float* os = p.o_part + pair[i] * p.max_chunks * kD + 4 * q4;
      float Lm = -INFINITY;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) Lm = fmaxf(Lm, lv[i][j]);
      for (int c0 = kBatch; c0 < n; c0 += kBatch)
#pragma unroll
        for (int j = 0; j < kBatch; ++j) Lm = fmaxf(Lm, ls[min(c0 + j, n - 1)]);
      auto weight = [&](float lc) {
        if (Lm == -INFINITY) return 0.f;
        if (Lm == INFINITY) return lc == INFINITY ? 1.f : 0.f;
        return __expf(lc - Lm);
      };
      float den = 0.f;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const float w = j < n ? weight(lv[i][j]) : 0.f;
        den += w;
        if (w != 0.f) acc += w * ov[i][j];
      }
      for (int c0 = kBatch; c0 < n; c0 += kBatch) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int cj = min(c0 + j, n - 1);
          const float w = c0 + j < n ? weight(ls[cj]) : 0.f;
          den += w;
          if (w != 0.f) acc += w * *reinterpret_cast<const f32x4*>(os + (int64_t)cj * kD);
        }
      }
      const float inv = den > 0.f ? 1.f / den : 0.f;
      const int64_t dst = pair[i] * kD + 4 * q4;
      if (p.out_f32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + dst) = acc * inv;
      } else {
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + dst) =
            u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
      }
      if (p.lse != nullptr && q4 == 0) {
        float l;
        if (Lm == -INFINITY) l = -INFINITY;
        else if (Lm == INFINITY) l = INFINITY;
        else l = Lm + __logf(den);
        p.lse[pair[i]] = l;
      }
    }
  }
}

template <int G>
hipError_t launch_g(const VerifyTileArgs& a, hipStream_t stream) {
  const int64_t items = (int64_t)a.batch * a.hkv * a.max_chunks;
  const int64_t wgs = ((items + 7) / 8) * 8 * a.row_tiles;
  if (wgs == 0) return hipSuccess;
  if (wgs > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (a.draft_mask != nullptr)
    hipLaunchKernelGGL((verify_tile_kernel<G, true>), dim3((unsigned)wgs), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((verify_tile_kernel<G, false>), dim3((unsigned)wgs), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_chunks == 1) return e;
  const int64_t rows = (int64_t)a.batch * a.max_qlen;   // (request, token) slots
  if (rows == 0) return hipSuccess;
  if (rows > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(verify_tile_finish_kernel, dim3((unsigned)rows), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_verify_tile(const VerifyTileArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_g<1>(a, stream);
    case 2: return launch_g<2>(a, stream);
    case 4: return launch_g<4>(a, stream);
    case 8: return launch_g<8>(a, stream);
    case 16: return launch_g<16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sa
