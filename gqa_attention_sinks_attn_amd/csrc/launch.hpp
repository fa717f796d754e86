// Internal launch interface between the C ABI layer (api.cpp) and the
// kernels.  Host code only; every pointer here has been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

struct DecodeArgs {
  const uint16_t* q;            // bf16 [B, Hq, 64]
  const uint16_t* k;            // bf16 [num_pages, Hkv, 16, 64]
  const uint16_t* v;
  const int32_t* page_indptr;   // [B+1]
  const int32_t* page_indices;  // [nnz]
  const int32_t* kv_len;        // [B]
  const float* sinks;           // [Hq] or nullptr
  int32_t batch, hq, hkv;
  int32_t num_splits;           // S >= 1
  int32_t chunk_pages;          // pages per split
  float scale_log2;             // sm_scale * log2(e)
  void* out;                    // final output (S == 1)
  int32_t out_f32;
  float* lse;                   // final lse or nullptr (S == 1)
  float* o_part;                // [B, Hq, S, 64] (S > 1)
  float* lse_part;              // [B, Hq, S]
  int32_t write_partials;       // 1: write o_part/lse_part, 0: write out/lse
};

struct BalancedDecodeArgs {
  const uint16_t* q;            // bf16 [B, Hq, 64]
  const uint16_t* k;            // bf16 [num_pages, Hkv, 16, 64]
  const uint16_t* v;
  const int32_t* page_indptr;   // [B+1]
  const int32_t* page_indices;  // [nnz]
  const int32_t* kv_len;        // [B]
  const float* sinks;           // [Hq] or nullptr
  int32_t batch, hq, hkv;
  int32_t n_ranges;             // page ranges per KV head, a multiple of 4
  int32_t min_range_pages;      // lower bound of the range width
  float scale_log2;             // sm_scale * log2(e)
  void* out;                    // [B, Hq, 64]
  int32_t out_f32;
  float* lse;                   // [B, Hq] or nullptr
  float* o_part;                // [n_ranges + B - 1, Hq, 64]
  float* lse_part;              // [n_ranges + B - 1, Hq]
  // Decode step (qkv != nullptr): the first pass also does the new token's
  // bias, rotation and append; q then points at q_new.
  const uint16_t* qkv;          // bf16 [B, Hq + 2 Hkv, 64], one new token per request
  const uint16_t* bias;         // bf16 [(Hq + 2 Hkv) 64] or nullptr
  const float* table;           // [max_pos, 64]: temperature x cos | temperature x sin
  int32_t max_pos;
  int32_t interleaved;          // 0: dim i pairs with i + 32; 1: 2i with 2i + 1
  uint16_t* k_new;              // the K/V cache (k, v), written at each new token's slot
  uint16_t* v_new;
  uint16_t* q_new;              // bf16 [B, Hq, 64]: the rotated queries, written, then read as q
};

struct VerifyArgs {
  const uint16_t* q;            // bf16 [total_q, Hq, 64]
  const int32_t* qo_indptr;     // [B+1]
  const uint16_t* k;            // bf16 [num_pages, Hkv, 16, 64]
  const uint16_t* v;
  const int32_t* page_indptr;   // [B+1]
  const int32_t* page_indices;  // [nnz]
  const int32_t* kv_len;        // [B]
  const float* sinks;           // [Hq] or nullptr
  int32_t batch, hq, hkv;
  int32_t num_splits;           // S >= 1
  int32_t chunk_pages;          // pages per split
  float scale_log2;             // sm_scale * log2(e)
  void* out;                    // [total_q, Hq, 64] (S == 1)
  int32_t out_f32;
  float* lse;                   // [total_q, Hq] or nullptr (S == 1)
  float* o_part;                // [total_q, Hq, S, 64] (S > 1)
  float* lse_part;              // [total_q, Hq, S]
  int32_t write_partials;
  const uint64_t* draft_mask;   // [total_q] drafted-token visibility, or nullptr (causal)
  int32_t col_groups;           // Z: groups of 64 (token, head) columns per (request, KV head)
};

// Largest batch whose verification jobs the tile kernel orders longest first
// (four requests per lane of a wave).
constexpr int32_t kLongestFirstMaxBatch = 256;

struct VerifyTileArgs {
  const uint16_t* q;            // bf16 [total_q, Hq, 64]
  const int32_t* qo_indptr;     // [B+1]
  const uint16_t* k;            // bf16 [num_pages, Hkv, 16, 64]
  const uint16_t* v;
  const int32_t* page_indptr;   // [B+1]
  const int32_t* page_indices;  // [nnz]
  const int32_t* kv_len;        // [B]
  const float* sinks;           // [Hq] or nullptr
  const uint64_t* draft_mask;   // [total_q] drafted-token visibility, or nullptr (causal)
  int32_t batch, hq, hkv;
  int32_t max_qlen;             // upper bound of qlen_b (finish grid)
  int32_t row_tiles;            // 128-row tiles per (request, KV head)
  int32_t chunk_tiles;          // 64-key tiles per KV chunk
  int32_t max_chunks;           // chunks of the longest request (<= 64)
  float scale_log2;             // sm_scale * log2(e)
  void* out;                    // [total_q, Hq, 64]
  int32_t out_f32;
  float* lse;                   // [total_q, Hq] or nullptr
  float* o_part;                // [total_q, Hq, max_chunks, 64] (max_chunks > 1)
  float* lse_part;              // [total_q, Hq, max_chunks]
  int32_t longest_first;        // 1: workgroup i takes the i-th longest job (batch <= kLongestFirstMaxBatch)
};

struct MergeArgs {
  const float* o_parts;         // [N, H, S, 64]
  const float* lse_parts;       // [N, H, S] natural log
  int32_t rows, heads, splits;
  void* out;
  int32_t out_f32;
  float* lse;                   // nullable
};

struct PrefillArgs {
  const uint16_t* q;            // bf16 [total_q, Hq, 64]
  const int32_t* qo_indptr;     // [B+1]
  const uint16_t* k;            // contiguous [total_kv, Hkv, 64] or paged
  const uint16_t* v;
  const int32_t* kv_indptr;     // token offsets or page offsets
  const int32_t* page_indices;  // nullptr = contiguous
  const int32_t* kv_len;        // nullptr = kv_indptr gaps (contiguous only)
  const float* sinks;
  int32_t batch, hq, hkv;
  int32_t max_qlen;
  int32_t causal;
  float scale_log2;
  void* out;
  int32_t out_f32;
  float* lse;
  // Prefill step (qkv != nullptr, paged cache): the queries are read from
  // the projection rows and biased and rotated at load; q is unused.
  const uint16_t* qkv;          // bf16 [total_q, Hq + 2 Hkv, 64]
  const uint16_t* bias;         // bf16 [(Hq + 2 Hkv) 64] or nullptr
  const float* table;           // [max_pos, 64]
  int32_t max_pos;
  int32_t interleaved;
  int32_t longest_first;        // 1: workgroup i takes the i-th longest query tile (batch <= 128)
};

// Largest batch whose prefill query tiles the kernel orders longest first
// (two requests per lane of a wave).
constexpr int32_t kPrefillLongestFirstMaxBatch = 128;

hipError_t launch_decode(const DecodeArgs& a, int group, hipStream_t stream);
hipError_t launch_decode_balanced(const BalancedDecodeArgs& a, int group, hipStream_t stream);
hipError_t launch_decode_finish(const BalancedDecodeArgs& a, hipStream_t stream);
struct RopeTableArgs {
  float* table;                 // [max_pos, 64]: temperature x cos | temperature x sin
  int32_t max_pos;
  int32_t original_max_pos;
  double base, factor, beta_fast, beta_slow, temperature;
  int32_t pair_ramp;            // 0: blend linear in the turn count; 1: in the pair index
  double ramp_low, ramp_high;   // pair-index ramp: the rounded bounds
};

struct RopeAppendArgs {
  const uint16_t* qkv;          // bf16 [total_q, Hq + 2 Hkv, 64]
  const uint16_t* bias;         // bf16 [(Hq + 2 Hkv) 64] or nullptr
  const float* table;           // [max_pos, 64]
  int32_t max_pos;
  const int32_t* qo_indptr;     // [B+1]
  const int32_t* kv_len;        // [B], the new tokens included
  const int32_t* page_indptr;   // [B+1]
  const int32_t* page_indices;
  int32_t batch, hq, hkv, total_q, interleaved;
  int32_t kv_only;              // 1: the key and value heads only (q_out unused)
  uint16_t* q_out;              // bf16 [total_q, Hq, 64]
  uint16_t* k_pages;            // bf16 [num_pages, Hkv, 16, 64]
  uint16_t* v_pages;
};

hipError_t launch_verify(const VerifyArgs& a, int group, int column_blocks, hipStream_t stream);
hipError_t launch_verify_tile(const VerifyTileArgs& a, int group, hipStream_t stream);
hipError_t launch_rope_table(const RopeTableArgs& a, hipStream_t stream);
hipError_t launch_rope_append(const RopeAppendArgs& a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, int group, hipStream_t stream);

}  // namespace sa
