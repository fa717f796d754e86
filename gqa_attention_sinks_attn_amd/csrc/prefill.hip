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
//     blocks, each one head x 32 consecutive tokens; eight blocks per
//     workgroup, so a workgroup covers 256 / G tokens x G heads and every
//     K/V tile it stages in LDS is reused by all 256 rows (GQA packing);
//   * keys are walked in tiles of 64 up to the causal edge of the
//     workgroup's last token; K and V tiles are double-buffered in LDS and
//     the next tile's global loads are in flight while this one computes;
//   * each wave computes S^T = K Q^T for its 2 x 32 rows on
//     v_mfma_f32_32x32x16_bf16, so a lane holds 32 scores of one query row
//     and the row maximum needs one cross-lane exchange;
//   * P is rounded to bf16 in registers and fed directly as the B operand
//     of O^T += V^T P^T; V is stored transposed in LDS in the key order the
//     score layout produces;
//   * masking (causal edge, ragged tail) is applied only on tiles that
//     straddle an edge; late query tiles are launched first.
#include "common.hpp"
#include "launch.hpp"

namespace sa {
namespace {

constexpr int kD = 64;
constexpr int kTile = 64;          // keys per tile
constexpr int kKRow = 72;          // K tile row stride in bf16 (144 B)
constexpr int kVRow = 68;          // V^T tile row stride in bf16 (136 B)
constexpr int kKBuf = kTile * kKRow;   // bf16 elements per K buffer
constexpr int kVBuf = kD * kVRow;      // bf16 elements per V^T buffer

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

template <bool PAGED>
__device__ __forceinline__ const uint16_t* kv_row(const PrefillArgs& p, const uint16_t* base,
                                                  int b, int g, int key, int kv_start) {
  if constexpr (PAGED) {
    const int page = p.page_indices[kv_start + (key >> 4)];
    return base + (((int64_t)page * p.hkv + g) * 16 + (key & 15)) * kD;
  } else {
    return base + ((int64_t)(kv_start + key) * p.hkv + g) * kD;
  }
}

template <int G, bool PAGED>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs p) {
  constexpr int T = 256 / G;  // tokens per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2 * kKBuf];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2 * kVBuf];

  const int qt = (int)gridDim.x - 1 - (int)blockIdx.x;  // late (long) tiles first
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int q_begin = p.qo_indptr[b];
  const int qlen = p.qo_indptr[b + 1] - q_begin;
  const int t0 = qt * T;
  if (t0 >= qlen) return;
  const int kv_start = p.kv_indptr[b];
  int L;
  if (p.kv_len != nullptr) L = p.kv_len[b];
  else L = p.kv_indptr[b + 1] - kv_start;
  const int pos_base = L - qlen;  // absolute position of token 0

  const int tid = threadIdx.x;
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
    head[cb] = g * G + (cbi % G);
    tok[cb] = t0 + 32 * (cbi / G) + r;
    valid[cb] = tok[cb] < qlen;
    pos[cb] = valid[cb] ? pos_base + tok[cb] : -1;
    const int last_tok = min(t0 + 32 * (cbi / G) + 31, qlen - 1);
    wave_pos_max = max(wave_pos_max, pos_base + last_tok);
    const uint16_t* qrow =
        p.q + ((int64_t)(q_begin + (valid[cb] ? tok[cb] : 0)) * p.hq + head[cb]) * kD + 8 * hh;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int s = 0; s < 4; ++s) bq[cb][s] = as_bf16x8(valid[cb] ? ld16(qrow + 16 * s) : z);
  }

  // ---- key range of the workgroup ----
  const int last_tok_wg = min(t0 + T, qlen) - 1;
  const int pos_min_wg = pos_base + t0;
  const int pos_max_wg = pos_base + last_tok_wg;
  const int kv_hi = p.causal ? min(L, pos_max_wg + 1) : L;
  const int n_tiles = (kv_hi + kTile - 1) / kTile;

  // ---- online state (log2 units); the sink starts every row ----
  float m[2], d[2];
  f32x16 o[2][2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    m[cb] = -INFINITY;
    d[cb] = 0.f;
    if (p.sinks != nullptr) {
      const float sg = p.sinks[head[cb]];
      m[cb] = sg * kLog2e;
      d[cb] = (hh == 0 && sg != -INFINITY) ? 1.f : 0.f;
    }
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[cb][db][j] = 0.f;
  }

  // ---- tile loader: thread -> two K rows (16 B chunk) and a V key pair ----
  const int ld_row = tid >> 3;   // 0..31
  const int ld_chunk = tid & 7;  // 16-byte chunk within a 128-byte row
  u32x4 rk0, rk1, rv0, rv1;
  auto load_tile = [&](int kt) {
    const int key0 = kt * kTile;
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int ka = key0 + ld_row, kb2 = key0 + 32 + ld_row;
    const int va = key0 + 2 * ld_row, vb = va + 1;
    rk0 = ka < L ? ld16(kv_row<PAGED>(p, p.k, b, g, ka, kv_start) + 8 * ld_chunk) : z;
    rk1 = kb2 < L ? ld16(kv_row<PAGED>(p, p.k, b, g, kb2, kv_start) + 8 * ld_chunk) : z;
    rv0 = va < L ? ld16(kv_row<PAGED>(p, p.v, b, g, va, kv_start) + 8 * ld_chunk) : z;
    rv1 = vb < L ? ld16(kv_row<PAGED>(p, p.v, b, g, vb, kv_start) + 8 * ld_chunk) : z;
  };
  auto store_tile = [&](int buf) {
    uint16_t* kd = lds_k + buf * kKBuf;
    *reinterpret_cast<u32x4*>(kd + ld_row * kKRow + 8 * ld_chunk) = rk0;
    *reinterpret_cast<u32x4*>(kd + (32 + ld_row) * kKRow + 8 * ld_chunk) = rk1;
    // V^T: row = dim, column = key; pack the key pair per dim
    uint32_t* vd = reinterpret_cast<uint32_t*>(lds_v + buf * kVBuf + (8 * ld_chunk) * kVRow +
                                               2 * ld_row);
    constexpr int kVRowW = kVRow / 2;  // row stride in 32-bit words
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      vd[(2 * w) * kVRowW] = lo_pair(rv0[w], rv1[w]);
      vd[(2 * w + 1) * kVRowW] = hi_pair(rv0[w], rv1[w]);
    }
  };

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  const float sl2 = p.scale_log2;
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_tiles) load_tile(kt + 1);
    const int key0 = kt * kTile;
    const bool wave_live = !p.causal || key0 <= wave_pos_max;
    if (wave_live) {
      const uint16_t* kbuf = lds_k + buf * kKBuf;
      const uint16_t* vbuf = lds_v + buf * kVBuf;
      // S^T[kb][cb]: keys 32 kb + 8 (j/4) + 4 hh + j%4, column = row r of cb
      f32x16 sacc[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int j = 0; j < 16; ++j) sacc[kb][cb][j] = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 a = as_bf16x8(
              *reinterpret_cast<const u32x4*>(kbuf + (32 * kb + r) * kKRow + 16 * s + 8 * hh));
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) sacc[kb][cb] = mfma32(a, bq[cb][s], sacc[kb][cb]);
        }
      }

      const bool edge = (p.causal && key0 + kTile - 1 > pos_min_wg) || (key0 + kTile > L);
      bf16x8 pb[2][2][2];  // [kb][half][cb]
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        float sv[32];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) sv[16 * kb + j] = sacc[kb][cb][j] * sl2;
        if (edge) {
          const int lim = p.causal ? min(pos[cb], L - 1) : L - 1;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int key = key0 + 32 * kb + 8 * (j >> 2) + 4 * hh + (j & 3);
              if (key > lim) sv[16 * kb + j] = -INFINITY;
            }
        }
        float mx = sv[0];
#pragma unroll
        for (int i = 1; i < 32; ++i) mx = fmaxf(mx, sv[i]);
        mx = fmaxf(mx, xor_lane(mx, 32));
        const float m_new = fmaxf(m[cb], mx);
        const float alpha = (m[cb] == m_new) ? 1.f : fast_exp2(m[cb] - m_new);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          sv[i] = fast_exp2(sv[i] - m_use);
          ps += sv[i];
        }
        d[cb] = d[cb] * alpha + ps;
        m[cb] = m_new;
#pragma unroll
        for (int db = 0; db < 2; ++db) o[cb][db] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const float* x = sv + 16 * kb + 8 * hf;
            u32x4 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                       pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
            pb[kb][hf][cb] = as_bf16x8(w);
          }
      }

      // O^T[cb][db] += V^T[dims 32 db.., keys] P^T
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            const uint16_t* vr = vbuf + (32 * db + r) * kVRow + 32 * kb + 16 * hf + 4 * hh;
            const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 8);
            const u32x4 vw = {lo[0], lo[1], hi[0], hi[1]};
            const bf16x8 a = as_bf16x8(vw);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) o[cb][db] = mfma32(a, pb[kb][hf][cb], o[cb][db]);
          }
    }
    if (kt + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: o = O / d, lse = m + log2 d (natural log at the boundary) ----
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float dt = d[cb] + xor_lane(d[cb], 32);
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
  dim3 grid(q_tiles, a.hkv, a.batch);
  if (a.page_indices != nullptr)
    hipLaunchKernelGGL((prefill_kernel<G, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<G, false>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_g<1>(a, stream);
    case 2: return launch_g<2>(a, stream);
    case 4: return launch_g<4>(a, stream);
    case 8: return launch_g<8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sa
