// Causal ragged prefill with a per-head sink (gfx950).
//
// GPT-OSS on Day 0 (Perplexity), "Sink attention" under "Kernels for
// GPT-OSS": the sink is an extra logit accumulated next to the Q.K products
// before the softmax; the softmax runs online with a running maximum m and
// scale d, and starting m at the head's sink with d = 1 folds the sink into
// the denominator once.  The same template serves prefill and decode.
//
// Work decomposition (one workgroup = 4 waves = 256 packed query rows):
//   * rows are (token, query head) pairs of ONE KV head g: 32-row column
//     blocks, each one head x 32 consecutive tokens (two heads x 16 tokens
//     when G = 16); eight blocks per workgroup, so a workgroup covers
//     256 / G tokens x G heads and every K/V tile it stages in LDS is reused
//     by all 256 rows (GQA packing);
//   * keys are walked in tiles of 64 up to the causal edge of the
//     workgroup's last token; K and V tiles go straight from global memory
//     into LDS (three buffers: the next two tiles are in flight while one
//     is computed), laid out for conflict-free operand reads;
//   * each wave computes S^T = K Q^T for its 2 x 32 rows on
//     v_mfma_f32_32x32x16_bf16, so a lane holds 32 scores of one query row
//     and the row maximum needs one cross-lane exchange;
//   * the running maximum is a reference value m: scores are exponentiated
//     as exp2(s * scale - m) with one FMA and no per-tile maximum; only when
//     a row's tile sum would exceed 2^16 (a new, much larger maximum) or the
//     row has no reference yet does the tile take the slow path that finds
//     the true maximum and rescales m, d and O -- the same quantity as the
//     textbook update, with the max reduction and the rescale of O skipped
//     on almost every tile;
//   * P is rounded to bf16 in registers and fed directly as the B operand of
//     O^T += V^T P^T; the row sums of the same rounded values are taken on
//     the matrix core too (v_mfma_f32_16x16x32_bf16 with a 0/1 A operand),
//     so the weights of every row sum to one and the vector unit, the
//     loop's bottleneck, only exponentiates and packs; V stays in its
//     natural layout in LDS and is read transposed with ds_read_b64_tr_b16
//     in the key order of the score layout;
//   * masking (causal edge, ragged tail) is applied only on tiles that
//     straddle an edge, comparing key offsets inside the tile (constants)
//     against one per-row limit;
//   * the grid is flat, its slowest index counting query tiles from the end
//     of each request, so the tile that sees the most keys of every
//     (request, KV head) pair starts first (with or without a cached
//     prefix) and the short ones fill the tail.
#include <climits>

#include "common.hpp"
#include "launch.hpp"

namespace sa {
namespace {

constexpr int kD = 64;
constexpr int kTile = 64;            // keys per tile
constexpr int kTileBytes = kTile * kD * 2;  // one K or V tile in LDS, rows unpadded
constexpr int kBufs = 3;                    // LDS tile buffers
constexpr float kFastLimit = 65536.f; // row tile sum that forces a rescale
constexpr int kOrderLevels = 8;       // length levels of the workgroup order (<= 64)

// Inclusive scans over the 64 lanes on the vector unit (wave-uniform control
// flow): shifts by 1, 2, 4 and 8 lanes inside each 16-lane row, then lane 15
// of each row added into the next row and lane 31 into the upper two rows
// (the row_shr and row_bcast forms of DPP).  Lanes without a source add the
// identity.  No LDS round trips, unlike a ds_bpermute ladder.
template <class Op>
__device__ __forceinline__ int wave_scan(int v, Op op, int identity) {
  v = op(v, __builtin_amdgcn_update_dpp(identity, v, 0x111, 0xf, 0xf, false));   // row_shr:1
  v = op(v, __builtin_amdgcn_update_dpp(identity, v, 0x112, 0xf, 0xf, false));   // row_shr:2
  v = op(v, __builtin_amdgcn_update_dpp(identity, v, 0x114, 0xf, 0xf, false));   // row_shr:4
  v = op(v, __builtin_amdgcn_update_dpp(identity, v, 0x118, 0xf, 0xf, false));   // row_shr:8
  v = op(v, __builtin_amdgcn_update_dpp(identity, v, 0x142, 0xa, 0xf, false));   // row_bcast:15
  v = op(v, __builtin_amdgcn_update_dpp(identity, v, 0x143, 0xc, 0xf, false));   // row_bcast:31
  return v;
}

__device__ __forceinline__ int wave_prefix_sum(int v, int) {
  return wave_scan(v, [](int a, int b) { return a + b; }, 0);
}

// Maximum over the wave, wave-uniform.
__device__ __forceinline__ int wave_max(int v) {
  return __builtin_amdgcn_readlane(wave_scan(v, [](int a, int b) { return max(a, b); }, INT_MIN), 63);
}

// Query tiles of a request whose key-tile count reaches level v or more,
// i.e. whose key count exceeds x (the level's bound): tile j from the end
// (j = 0 is the last) sees min(L, L + e - j T) keys when causal, where e
// pads the first tile (qlen + e = n_tiles T), and all L keys otherwise.
template <int T>
__device__ __forceinline__ int tiles_at_or_above(int v, int x, int L, int e, int n_tiles,
                                                 bool causal) {
  if (v == 0) return n_tiles;
  if (L <= x) return 0;
  if (!causal) return n_tiles;
  const int jmax = (L + e - x - 1) / T;   // last j >= 1 that still exceeds x
  return 1 + min(max(jmax, 0), n_tiles - 1);
}

// Longest-first order of the workgroups (request b, query tile j from the
// end, KV head g).  A workgroup's length is the number of 64-key tiles it
// walks.  The order: by that length in kOrderLevels levels of the longest
// request's tile count, from the top; within a level by request, then j,
// then g, so that consecutive workgroups share a request's keys (and, KV
// heads being the fastest index, every XCD keeps meeting the same KV heads
// in its L2).  Eight levels rather than finer ones: coarser levels keep
// more consecutive workgroups on one request (2-3% on equal requests) and
// still sort a ragged batch's tiles well enough.
// Workgroups are dispatched in index order, so long ones start first and
// short ones fill the tail.  Every wave computes the same answer from the
// request lengths, with no exchange: each lane holds two requests and counts
// their tiles at or above every level, a butterfly sums all the levels over
// the wave at once, and the workgroup's level and request follow from
// prefix sums, so the cost does not grow with the request count.  Returns
// false past the last workgroup; otherwise also the chosen request's
// offsets and lengths, read out of the lanes that loaded them (no second
// round trip to memory).
struct RequestSpan {
  int q_begin, qlen, kv_start, L;
};

template <int T>
__device__ __forceinline__ bool longest_first_tile(const PrefillArgs& p, int i, int lane, int& b,
                                                   int& j, int& g, RequestSpan& rq) {
  const int B = p.batch;
  int L[2], e[2], nt[2], qb[2], ks[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int r = 64 * k + lane;
    const bool in = r < B;
    const int q0 = in ? p.qo_indptr[r] : 0;
    const int q1 = in ? p.qo_indptr[r + 1] : 0;
    const int k0 = in ? p.kv_indptr[r] : 0;
    int len = 0;
    if (in) len = p.kv_len != nullptr ? p.kv_len[r] : p.kv_indptr[r + 1] - k0;
    L[k] = len;
    qb[k] = q0;
    ks[k] = k0;
    nt[k] = (q1 - q0 + T - 1) / T;
    e[k] = nt[k] * T - (q1 - q0);
  }
  const bool causal = p.causal != 0;
  const int lmax = __builtin_amdgcn_readfirstlane(
      max(1, wave_max(max((L[0] + kTile - 1) / kTile, (L[1] + kTile - 1) / kTile))));
  // Key counts above bound(v) reach level v.
  auto bound = [&](int v) {
    if (v >= kOrderLevels) return 0x7fffffff;
    // fewest key tiles at level v: level(l) = (kOrderLevels l - 1) / lmax
    const int64_t lo = ((int64_t)v * lmax + kOrderLevels) / kOrderLevels;
    return (int)(kTile * (lo - 1));
  };
  // A[v]: query tiles of the batch at level v or above (A[0] all of them),
  // each lane counting its two requests, all levels at once, then summed
  // over the wave.  Level v holds workgroups A[v + 1] hkv .. A[v] hkv - 1.
  int A[kOrderLevels + 1];
#pragma unroll
  for (int v = 0; v < kOrderLevels; ++v) {
    const int x = bound(v);
    A[v] = tiles_at_or_above<T>(v, x, L[0], e[0], nt[0], causal);
    if (B > 64) A[v] += tiles_at_or_above<T>(v, x, L[1], e[1], nt[1], causal);
  }
  // summed over the lanes, the levels side by side
#pragma unroll
  for (int v = 0; v < kOrderLevels; ++v) A[v] = __builtin_amdgcn_readlane(wave_prefix_sum(A[v], lane), 63);
  A[kOrderLevels] = 0;
  if (i >= A[0] * p.hkv) return false;
  int v = 0;     // the highest level that starts at or before workgroup i
#pragma unroll
  for (int u = kOrderLevels - 1; u > 0; --u)
    if (v == 0 && A[u] * p.hkv > i) v = u;
  int above = 0;
#pragma unroll
  for (int u = 1; u <= kOrderLevels; ++u)
    if (u == v + 1) above = A[u] * p.hkv;   // workgroups on higher levels
  int idx = i - above;
  const int xv_lo = bound(v);
  const int xv_hi = bound(v + 1);
  // the requests with workgroups at level v, in order
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (64 * k < B) {
      const int first = tiles_at_or_above<T>(v + 1, xv_hi, L[k], e[k], nt[k], causal);
      const int c = (tiles_at_or_above<T>(v, xv_lo, L[k], e[k], nt[k], causal) - first) * p.hkv;
      const int incl = wave_prefix_sum(c, lane);
      const int tot = __builtin_amdgcn_readlane(incl, 63);
      if (idx < tot) {
        const int ln = __builtin_ctzll(__ballot(incl > idx));
        const int off = idx - __builtin_amdgcn_readlane(incl - c, ln);
        b = 64 * k + ln;
        j = __builtin_amdgcn_readlane(first, ln) + off / p.hkv;
        g = off % p.hkv;
        rq.q_begin = __builtin_amdgcn_readlane(qb[k], ln);
        rq.qlen = __builtin_amdgcn_readlane(nt[k] * T - e[k], ln);
        rq.kv_start = __builtin_amdgcn_readlane(ks[k], ln);
        rq.L = __builtin_amdgcn_readlane(L[k], ln);
        return true;
      }
      idx -= tot;
    }
  }
  return false;
}

template <int G, bool PAGED, bool STEP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(PrefillArgs p) {
  constexpr int T = 256 / G;  // tokens per workgroup
  __shared__ __attribute__((aligned(1024))) char lds_k[kBufs * kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v[kBufs * kTileBytes];

  // Heaviest first.  Batches of up to 128 requests: longest_first_tile.
  // Larger ones: the grid is flat with the round j as its slowest index, and
  // round j takes the j-th query tile from the end of every request.  A
  // request's last tile sees all of its keys, so round 0 holds the largest
  // workgroup of every request (whatever its cached prefix), and work falls
  // with j.
  int j, g, b;
  RequestSpan rq;
  if (p.longest_first) {
    if (!longest_first_tile<T>(p, block_x(), thread_x() & 63, b, j, g, rq)) return;
  } else {
    const int units = p.hkv * p.batch;
    const int wg = block_x();
    j = wg / units;
    g = (wg % units) % p.hkv;
    b = (wg % units) / p.hkv;
    rq.q_begin = p.qo_indptr[b];
    rq.qlen = p.qo_indptr[b + 1] - rq.q_begin;
    rq.kv_start = p.kv_indptr[b];
    rq.L = p.kv_len != nullptr ? p.kv_len[b] : p.kv_indptr[b + 1] - rq.kv_start;
  }
  const int q_begin = rq.q_begin;
  const int qlen = rq.qlen;
  const int qt = (qlen + T - 1) / T - 1 - j;
  if (qt < 0) return;
  const int t0 = qt * T;
  const int kv_start = rq.kv_start;
  const int L = rq.L;
  const int pos_base = L - qlen;  // absolute position of token 0

  const int tid = thread_x();
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 31;
  const int hh = lane >> 5;

  // ---- this lane's two query rows (one per column block) ----
  int head[2], tok[2], pos[2];
  bool valid[2];
  bf16x8 bq[2][4];
  int wave_pos_max = -1;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int cbi = 2 * wave + cb;
    // Row map of column block cbi: with 32 or more tokens per workgroup
    // (G <= 8) a block is 32 consecutive tokens of one head; with 16 (G = 16)
    // it is two heads x 16 tokens (workgroup row 32 cbi + r is head
    // (32 cbi + r) / 16, token r % 16).
    int hl, tl, tl_last;
    if constexpr (T >= 32) {
      hl = cbi % G;
      tl = 32 * (cbi / G) + r;
      tl_last = 32 * (cbi / G) + 31;
    } else {
      hl = (32 * cbi + r) / T;
      tl = r % T;
      tl_last = T - 1;
    }
    head[cb] = g * G + hl;
    tok[cb] = t0 + tl;
    valid[cb] = tok[cb] < qlen;
    pos[cb] = valid[cb] ? pos_base + tok[cb] : -1;
    const int last_tok = min(t0 + tl_last, qlen - 1);
    wave_pos_max = max(wave_pos_max, pos_base + last_tok);
    const u32x4 z = {0u, 0u, 0u, 0u};
    if constexpr (STEP) {
      // The query from its projection row: bias added in fp32, rotated by
      // the token's table row with the append kernel's arithmetic, rounded
      // to bf16 once.  The lane holds dims 8 hh + 16 s .. + 7 (s = 0..3),
      // so both members of every rotated pair: dims d and d + 32 (chunks s
      // and s + 2) in the rotate-half pairing, 2 i and 2 i + 1 (inside a
      // chunk) interleaved.  A position outside the table is read clamped
      // (the append writes nothing for it; the row's result is unspecified).
      const int row = q_begin + (valid[cb] ? tok[cb] : 0);
      const uint16_t* xrow = p.qkv + ((int64_t)row * (p.hq + 2 * p.hkv) + head[cb]) * kD + 8 * hh;
      const float* trow = p.table + (int64_t)min(max(pos[cb], 0), p.max_pos - 1) * kD;
      float x[4][8];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 w = ld16(xrow + 16 * s);
        const u32x4 bw = p.bias != nullptr ? ld16(p.bias + (int64_t)head[cb] * kD + 8 * hh + 16 * s) : z;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[s][2 * i] = lo_bf16(w[i]) + lo_bf16(bw[i]);
          x[s][2 * i + 1] = hi_bf16(w[i]) + hi_bf16(bw[i]);
        }
      }
      if (p.interleaved) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const f32x4 c = *reinterpret_cast<const f32x4*>(trow + 8 * s + 4 * hh);
          const f32x4 sn = *reinterpret_cast<const f32x4*>(trow + 32 + 8 * s + 4 * hh);
#pragma unroll
          for (int k = 0; k < 4; ++k) rotate_pair(x[s][2 * k], x[s][2 * k + 1], c[k], sn[k]);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const float* cs = trow + 16 * s + 8 * hh;
          const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs);
          const f32x4 c1 = *reinterpret_cast<const f32x4*>(cs + 4);
          const f32x4 s0 = *reinterpret_cast<const f32x4*>(cs + 32);
          const f32x4 s1 = *reinterpret_cast<const f32x4*>(cs + 36);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            rotate_pair(x[s][i], x[s + 2][i], i < 4 ? c0[i] : c1[i - 4], i < 4 ? s0[i] : s1[i - 4]);
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 y = {pack_bf16x2(x[s][0], x[s][1]), pack_bf16x2(x[s][2], x[s][3]),
                         pack_bf16x2(x[s][4], x[s][5]), pack_bf16x2(x[s][6], x[s][7])};
        bq[cb][s] = as_bf16x8(valid[cb] ? y : z);
      }
    } else {
      const uint16_t* qrow =
          p.q + ((int64_t)(q_begin + (valid[cb] ? tok[cb] : 0)) * p.hq + head[cb]) * kD + 8 * hh;
#pragma unroll
      for (int s = 0; s < 4; ++s) bq[cb][s] = as_bf16x8(valid[cb] ? ld16(qrow + 16 * s) : z);
    }
  }

  // ---- key range of the workgroup ----
  const int last_tok_wg = min(t0 + T, qlen) - 1;
  const int pos_min_wg = pos_base + t0;
  const int pos_max_wg = pos_base + last_tok_wg;
  const int kv_hi = p.causal ? min(L, pos_max_wg + 1) : L;
  const int n_tiles = (kv_hi + kTile - 1) / kTile;

  // ---- online state (log2 units); the sink starts every row.  d holds the
  // sink's term of the denominator (lanes hh = 0); the keys' terms are summed
  // on the matrix core into dk: in every lane l, element 0 (and 2) holds row
  // l % 16 of the column block and element 1 (and 3) row 16 + l % 16, so a
  // lane's own row r = l % 32 is element r / 16 of its own dk. ----
  // (The sinks are read once the first tile is in flight, below.)
  float m[2] = {-INFINITY, -INFINITY}, d[2] = {0.f, 0.f};
  f32x4 dk[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  f32x16 o[2][2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[cb][db][j] = 0.f;

  // ---- tile loader.  A tile's K and V go straight from global memory
  // into LDS (load_lds16), 1 KiB blocks of eight key rows (key row r in
  // block r / 8).  Wave w loads K and V rows 16 w .. 16 w + 15 of every
  // tile, two blocks each: on a paged cache one page (one wave-uniform page
  // id, read with v_readlane from a vector of 64 tiles' ids loaded at
  // once), on a contiguous one from a wave-uniform row base; each lane's
  // offset from that base is fixed.  The lane -> (row, 16-byte chunk) map
  // of a block lays it out as the operand reads want it (chunk c of row
  // r' = r % 8, e = (r / 8) % 2):
  //   K: slot 16 (c / 2) + ((2 r' + c % 2 + e) mod 16), so the 16 rows of
  //      one K-operand read fall in 16 different bank groups and k-step s
  //      is a constant offset;
  //   V: slot 16 (c / 4 + 2 (r' / 4)) + 4 (r' % 4) + c % 4, so the four
  //      rows x four chunks of one transposed read fall in 16 different
  //      bank groups and every V^T operand is a constant offset.
  // Rows past the last key read a key of the request, so their V rows are
  // finite: the first row of their page (a page past the end is replaced by
  // the request's first page) or, on a contiguous cache, the tile's first
  // key.  Their scores are masked (every tile holding such rows is an edge
  // tile), so P is 0 for them. ----
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t stride_bytes = PAGED ? (uint32_t)p.hkv * 16 * kD * 2   // one page
                                      : (uint32_t)p.hkv * kD * 2;       // one key
  const char* kbytes = reinterpret_cast<const char*>(p.k);
  const char* vbytes = reinterpret_cast<const char*>(p.v);
  uint32_t koff[2], voff[2], kzero[2], vzero[2];
  int krow[2], vrow[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int x = ((lane & 15) - e) & 15;
    const int kc = 2 * (lane >> 4) + (x & 1);
    const int vc = 4 * ((lane >> 4) & 1) + (lane & 3);
    krow[e] = 8 * e + (x >> 1);
    vrow[e] = 8 * e + 4 * (lane >> 5) + ((lane & 15) >> 2);
    if constexpr (PAGED) {
      koff[e] = (uint32_t)g * 16 * kD * 2 + krow[e] * kD * 2 + 16 * kc;
      voff[e] = (uint32_t)g * 16 * kD * 2 + vrow[e] * kD * 2 + 16 * vc;
      kzero[e] = (uint32_t)g * 16 * kD * 2 + 16 * kc;
      vzero[e] = (uint32_t)g * 16 * kD * 2 + 16 * vc;
    } else {
      koff[e] = (16 * wave_u + krow[e]) * stride_bytes + 16 * kc;
      voff[e] = (16 * wave_u + vrow[e]) * stride_bytes + 16 * vc;
      kzero[e] = 16 * kc;
      vzero[e] = 16 * vc;
    }
  }
  // Paged caches: page ids of this wave's page in tiles first .. first + 63,
  // one per lane; the assembly use makes the compiler wait for them here.
  auto load_ids = [&](int first) {
    const int kt = first + lane;
    int id = 0;
    if (kt < n_tiles) {
      const int key0 = kt * kTile;
      id = p.page_indices[kv_start + (key0 + 16 * wave_u < L ? (key0 >> 4) + wave_u : 0)];
    }
    asm volatile("" ::"v"(id));
    return id;
  };
  auto issue = [&](int kt, int bf, int id) {
    const int key0 = kt * kTile;
    const char* kp;
    const char* vp;
    if constexpr (PAGED) {
      kp = kbytes + (uint64_t)(uint32_t)id * stride_bytes;
      vp = vbytes + (uint64_t)(uint32_t)id * stride_bytes;
    } else {
      (void)id;
      const uint64_t t = ((uint64_t)(uint32_t)(kv_start + key0) * p.hkv + g) * (kD * 2);
      kp = kbytes + t;
      vp = vbytes + t;
    }
    const uint32_t kd = lds_offset(lds_k) + bf * kTileBytes + wave_u * 2048;
    const uint32_t vd = lds_offset(lds_v) + bf * kTileBytes + wave_u * 2048;
    const bool tail = key0 + kTile > L;   // wave-uniform
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

  int ids = 0;
  if constexpr (PAGED) ids = load_ids(0);
  if (n_tiles > 0) issue(0, 0, __builtin_amdgcn_readlane(ids, 0));
  if (p.sinks != nullptr) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const float sg = p.sinks[head[cb]];
      m[cb] = sg * kLog2e;
      d[cb] = (hh == 0 && sg != -INFINITY) ? 1.f : 0.f;
    }
  }
  // The prologue's own global loads (queries, sinks) complete here, not
  // inside the loop.  The first tile is already in flight, so its latency
  // overlaps theirs; the compiler, which does not count the tile loads,
  // waits for everything issued so far, then the second tile goes out.
  asm volatile("" ::"v"(bq[0][0]), "v"(bq[0][1]), "v"(bq[0][2]), "v"(bq[0][3]), "v"(bq[1][0]),
               "v"(bq[1][1]), "v"(bq[1][2]), "v"(bq[1][3]), "v"(m[0]), "v"(m[1]));
  // The negated reference the fast path subtracts (0 for a row without one,
  // whose tile then takes the slow path anyway), refreshed where m changes.
  float nm[2];
  auto refresh_ref = [&](int cb) { nm[cb] = (m[cb] == -INFINITY) ? 0.f : -m[cb]; };
  refresh_ref(0);
  refresh_ref(1);
  if (n_tiles > 1) issue(1, 1, __builtin_amdgcn_readlane(ids, 1));

  const float sl2 = p.scale_log2;
  // Operand reads, byte offsets inside a tile buffer.  K operand of k-step
  // s, key block kb: key 32 kb + r, dims 16 s + 8 hh (chunk 2 s + hh) at
  // kread + 4096 kb + 256 s.  V^T operand: the transposed read of 16-lane
  // group q = lane / 16 covers dims 16 (q % 2) + 4 (lane % 4) .. of a 32-dim
  // block db (chunk 2 (q % 2) + (lane % 4) / 2 + 4 db) and key row
  // 4 hh + (lane % 16) / 4 (+ 8 for the upper four values) of the 16-key
  // slice hf of key block kb, at vread + 4096 kb + 2048 hf + 256 db (+ 1024).
  // Row sums of P on the matrix core: D(16x16) += A(16x32) B(32x16) with B =
  // a P^T operand of the O^T product as it stands in registers.  Read as a
  // 16x16x32 operand, lane l's eight keys are k-group l / 16 of column l % 16,
  // and they belong to row l % 32 of the column block: k-groups 0 and 2 of
  // column n are row n, k-groups 1 and 3 row 16 + n.  So the even rows of A
  // are ones on k-groups 0 and 2 and the odd rows ones on 1 and 3: D[m][n]
  // is the slice's sum of row n (m even) or row 16 + n (m odd), and lane l,
  // which holds D rows 4 (l / 16) .. + 3 of column l % 16, gets both.  The
  // sums add the bf16-rounded weights the O^T product consumes (exact
  // products, fp32 accumulation), so every row stays an exact convex
  // combination of V.
  bf16x8 ones_sel;
  {
    const bool one = (((lane & 15) + (lane >> 4)) & 1) == 0;
    const uint32_t w = one ? 0x3F803F80u : 0u;   // two bf16 1.0 or two zeros
    ones_sel = as_bf16x8(u32x4{w, w, w, w});
  }
  const int kread = ((lane & 31) >> 3) * 1024 + 16 * ((2 * (lane & 7) + hh + ((lane >> 3) & 1)) & 15);
  const int vread = 512 * hh + 64 * ((lane & 15) >> 2) + 16 * (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) +
                    8 * (lane & 1);

  // Every scalar load of the prologue completes here.  Left pending, it
  // would make the compiler count the loop's LDS reads as if they could
  // return out of order, and wait for all eight K reads of a tile before its
  // first product (s_waitcnt lgkmcnt(0) in every tile).
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), no vector-memory wait
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt % kBufs;
    // this wave's part of tile kt has landed (tile kt + 1 may be in
    // flight); the barrier makes every part visible and frees the buffer of
    // tile kt - 1 for tile kt + 2
    if (kt + 1 < n_tiles) wait_vmem<4>();
    else wait_vmem<0>();
    barrier_only();
    if (kt + 2 < n_tiles) {
      if constexpr (PAGED) {
        if (((kt + 2) & 63) == 0) ids = load_ids(kt + 2);
      }
      issue(kt + 2, (kt + 2) % kBufs, __builtin_amdgcn_readlane(ids, (kt + 2) & 63));
    }
    const int key0 = kt * kTile;
    const bool wave_live = !p.causal || key0 <= wave_pos_max;
    if (wave_live) {
      const char* kbuf = lds_k + buf * kTileBytes;
      // V^T reads from one LDS address per tile, hidden from loop strength
      // reduction, so that each read's constant part becomes its offset
      uint32_t vaddr = lds_offset(lds_v) + buf * kTileBytes + vread;
      asm volatile("" : "+v"(vaddr));
      const __attribute__((address_space(3))) char* vbuf =
          (const __attribute__((address_space(3))) char*)(uintptr_t)vaddr;
      const bool edge = (p.causal && key0 + kTile - 1 > pos_min_wg) || (key0 + kTile > L);
      const f32x16 zero16 = {};
      // K operand (A of S^T) for k-step s, key block kb: keys 32 kb + r,
      // dims 16 s + 8 hh.  V^T operand (A of O^T) for key block kb, half hf,
      // dim block db: dims 32 db + .., keys 32 kb + 16 hf + {4 hh .., 8 + 4 hh ..}.
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
      // S^T[kb][cb]: keys 32 kb + 8 (j/4) + 4 hh + j%4, column = row r of cb
      f32x16 sacc[2][2];
      uint32_t pk[2][2][2][4];  // [cb][kb][hf][pair]
      auto mask = [&](int cb) {
        const int lim = p.causal ? min(pos[cb], L - 1) : L - 1;
        int rel = lim - key0 - 4 * hh;
        // defined here, so the compares below cannot be hoisted out of the
        // (rare) edge branch into every tile
        asm volatile("" : "+v"(rel));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (32 * kb + 8 * (j >> 2) + (j & 3) > rel) sacc[kb][cb][j] = -INFINITY;
      };
      // exp2(s * scale - m) of the scores j = 8 hf + 2 q, +1 (q = 2 qp, 2 qp + 1)
      // of key block kb, packed to bf16 (the P^T operand of O^T and of the
      // row sums).
      auto expo4 = [&](int cb, float neg_m, int kb, int hf, int qp) {
#pragma unroll
        for (int q = 2 * qp; q < 2 * qp + 2; ++q) {
          const int j = 8 * hf + 2 * q;
          const float e0 = fast_exp2(__builtin_fmaf(sacc[kb][cb][j], sl2, neg_m));
          const float e1 = fast_exp2(__builtin_fmaf(sacc[kb][cb][j + 1], sl2, neg_m));
          pk[cb][kb][hf][q] = pack_bf16x2(e0, e1);
        }
      };
      auto pb_of = [&](int cb, int kb, int hf) {
        return as_bf16x8(u32x4{pk[cb][kb][hf][0], pk[cb][kb][hf][1], pk[cb][kb][hf][2], pk[cb][kb][hf][3]});
      };
      // Row sums of block cb's tile (layout of dk) from its four P^T operands.
      auto row_sums = [&](int cb) {
        f32x4 rs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) rs = mfma16(ones_sel, pb_of(cb, i >> 1, i & 1), rs);
        return rs;
      };
      // Fast path: the tile was exponentiated against the current reference
      // m.  It is valid while every row's tile sum stays below 2^16 and the
      // row has a reference; otherwise (rare: a new maximum, or the row's
      // first live tile without a sink) take the true row maximum, rescale O,
      // d, the key sums and m, and exponentiate again.
      // The sums are compared as unsigned bit patterns: an overflowed weight
      // makes them inf, or NaN where a 0 of the selector meets it inside the
      // product, and both patterns exceed the limit's (a float compare would
      // not see the NaN: device code is built without NaN semantics).
      auto settle_row = [&](int cb, f32x4 rs) {
        constexpr uint32_t kLimitBits = 0x47800000u;   // 65536.f
        static_assert(__builtin_bit_cast(uint32_t, kFastLimit) == kLimitBits, "limit bits");
        if (__any(__builtin_bit_cast(uint32_t, rs[0]) > kLimitBits ||
                  __builtin_bit_cast(uint32_t, rs[1]) > kLimitBits || m[cb] == -INFINITY)) {
          float mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; j += 2)
              mx = fmaxf(fmaxf(mx, sacc[kb][cb][j]), sacc[kb][cb][j + 1]);
          mx = fmaxf(mx, xor_lane(mx, 32));
          const float m_new = fmaxf(m[cb], mx * sl2);
          const float alpha = (m[cb] == m_new) ? 1.f : fast_exp2(m[cb] - m_new);
          // the key sums of rows l % 16 and 16 + l % 16: one is this lane's
          // row, the other's factor lives in lane l ^ 16
          const float alpha_x = xor_lane(alpha, 16);
          const bool lo_row = r < 16;
          d[cb] *= alpha;
          dk[cb][0] *= lo_row ? alpha : alpha_x;
          dk[cb][1] *= lo_row ? alpha_x : alpha;
          o[cb][0] *= alpha;
          o[cb][1] *= alpha;
          m[cb] = m_new;
          refresh_ref(cb);
#pragma unroll
          for (int i = 0; i < 8; ++i) expo4(cb, nm[cb], i >> 2, (i >> 1) & 1, i & 1);
          rs = row_sums(cb);
        }
        dk[cb][0] += rs[0];
        dk[cb][1] += rs[1];
      };

      // (1) S^T of column block 0.  The tile's K operands are read once and
      //     serve both blocks.
      bf16x8 ko[4][2];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) ko[s][kb] = kop(s, kb);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          sacc[kb][0] = mfma32(ko[s][kb], bq[0][s], s == 0 ? zero16 : sacc[kb][0]);
      // the reads go out a few ahead of the products that consume them, so
      // each product waits for its own operand only
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // DS read
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // DS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);   // MFMA
      if (edge) mask(0);
      // (2) S^T of column block 1 on the matrix core while the vector unit
      //     exponentiates block 0; block 0's row sums go to the matrix core
      //     as each 16-key slice of P is packed.
      {
        const float nmr = nm[0];
        f32x4 rs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int s = i >> 1, kb = i & 1;
          sacc[kb][1] = mfma32(ko[s][kb], bq[1][s], s == 0 ? zero16 : sacc[kb][1]);
          expo4(0, nmr, i >> 2, (i >> 1) & 1, i & 1);
          if (i & 1) rs = mfma16(ones_sel, pb_of(0, i >> 2, (i >> 1) & 1), rs);
        }
#pragma unroll
        for (int i = 0; i < 12; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);   // VALU
        }
        settle_row(0, rs);
      }
      if (edge) mask(1);
      // (3) O^T of block 0 += V^T P^T on the matrix core while block 1 is
      //     exponentiated (its row sums follow each packed slice).  The
      //     tile's V^T operands are read once, all at the start (the first
      //     exponentials cover their latency), and serve both blocks.
      bf16x8 vo[2][2][2];
      {
        const float nmr = nm[1];
        f32x4 rs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 8; ++i) vo[i >> 2][(i >> 1) & 1][i & 1] = vop(i >> 2, (i >> 1) & 1, i & 1);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int kb = i >> 2, hf = (i >> 1) & 1, db = i & 1;
          o[0][db] = mfma32(vo[kb][hf][db], pb_of(0, kb, hf), o[0][db]);
          expo4(1, nmr, i >> 2, (i >> 1) & 1, i & 1);
          if (i & 1) rs = mfma16(ones_sel, pb_of(1, i >> 2, (i >> 1) & 1), rs);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);    // DS read: all of V^T
        __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);    // VALU
#pragma unroll
        for (int i = 0; i < 12; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU
        }
        settle_row(1, rs);
      }
      // (4) O^T of block 1.
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kb = i >> 2, hf = (i >> 1) & 1, db = i & 1;
        o[1][db] = mfma32(vo[kb][hf][db], pb_of(1, kb, hf), o[1][db]);
      }
    }
  }

  // ---- epilogue: o = O / d, lse = m + log2 d (natural log at the boundary) ----
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    // this lane's row r = lane % 32: the sink's term from lanes r and r + 32,
    // the keys' terms from element r / 16 of its own key sums
    const float dt = d[cb] + xor_lane(d[cb], 32) + (r < 16 ? dk[cb][0] : dk[cb][1]);
    if (!valid[cb]) continue;
    const float inv = dt > 0.f ? 1.f / dt : 0.f;
    const int64_t orow = ((int64_t)(q_begin + tok[cb]) * p.hq + head[cb]) * kD;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int dim = 32 * db + 8 * a + 4 * hh;
        const float x0 = o[cb][db][4 * a + 0] * inv, x1 = o[cb][db][4 * a + 1] * inv;
        const float x2 = o[cb][db][4 * a + 2] * inv, x3 = o[cb][db][4 * a + 3] * inv;
        if (p.out_f32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + orow + dim) =
              f32x4{x0, x1, x2, x3};
        } else {
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + orow + dim) =
              u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
        }
      }
    if (p.lse != nullptr && hh == 0) {
      p.lse[(int64_t)(q_begin + tok[cb]) * p.hq + head[cb]] =
          dt > 0.f ? (m[cb] + __builtin_amdgcn_logf(dt)) * kLn2 : -INFINITY;
    }
  }
}

template <int G>
hipError_t launch_g(const PrefillArgs& a, hipStream_t stream) {
  constexpr int T = 256 / G;
  const int q_tiles = (a.max_qlen + T - 1) / T;
  if (q_tiles == 0 || a.batch == 0) return hipSuccess;
  const int64_t wgs = (int64_t)q_tiles * a.hkv * a.batch;
  if (wgs > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)wgs);
  if (a.qkv != nullptr)   // the prefill step: a paged cache
    hipLaunchKernelGGL((prefill_kernel<G, true, true>), grid, dim3(256), 0, stream, a);
  else if (a.page_indices != nullptr)
    hipLaunchKernelGGL((prefill_kernel<G, true, false>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<G, false, false>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int group, hipStream_t stream) {
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
