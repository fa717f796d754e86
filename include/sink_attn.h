/*
 * sink_attn.h — C ABI of the MI355X (gfx950) sink-attention library.
 *
 * The operation (GPT-OSS on Day 0, Perplexity: "Attention: GQA with
 * attention sinks", and "Sink attention" under "Kernels for GPT-OSS"):
 * grouped-query attention in which every query head h owns one pretrained
 * scalar sink sigma_h that takes part in that head's softmax as one extra
 * logit with no value vector.  For a query row with allowed keys J:
 *
 *     M   = max({tau * q.k_j : j in J} U {sigma_h})
 *     Z   = exp(sigma_h - M) + sum_{j in J} exp(tau * q.k_j - M)
 *     o   = sum_{j in J} exp(tau * q.k_j - M) / Z * v_j
 *     lse = M + ln Z                                   (natural log)
 *
 * The page computes this online: a running maximum m started at the head's
 * sink and a running scale d started at 1, so the sink enters the
 * denominator exactly once; when the key sequence is split into chunks the
 * sink belongs to the first chunk only (same section).  Query head h reads
 * KV head h / (Hq / Hkv).
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless stated; `stream` is a hipStream_t
 *     passed as void* (NULL = the null stream).  Work is enqueued on it and
 *     the call returns without synchronising.  The caller owns every buffer
 *     and keeps inputs alive until the stream's work completes.
 *   - The library allocates no device memory, keeps no pointer after
 *     returning and holds no state other than a thread-local error string
 *     and the per-device compute-unit count (written once, under
 *     std::call_once), so calls from several host threads are safe.
 *   - bf16 tensors are raw bfloat16 bit patterns; all of q, k, v, out and a
 *     workspace must be 16-byte aligned; int32 index arrays 4-byte aligned.
 *   - head_dim must be 64 and page_size 16 (SINK_ATTN_ERR_UNSUPPORTED
 *     otherwise).  Hq must be a multiple of Hkv, with Hq / Hkv in
 *     {1, 2, 4, 8, 16} for every entry point.
 *   - Automatic plans size their grids from the current device's compute
 *     unit count, queried once per device (256, a whole MI355X, when no
 *     device can be queried); the host-only planning queries below use the
 *     same count, so they agree with the launches on the same device.
 *   - sinks: fp32 [Hq] in logit units (not multiplied by sm_scale); NULL
 *     means no sink (sigma = -inf), i.e. standard attention.  A sink of
 *     +inf gives o = 0, lse = +inf.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     error return means nothing was launched or written.  Device index
 *     data (indptr, page ids, lengths) cannot be validated without a
 *     device->host copy and must be consistent with the host scalars
 *     (max_qlen, max_kv_len, num_pages) passed alongside.  A launch failure
 *     reported by the HIP runtime returns SINK_ATTN_ERR_HIP; a fault inside
 *     a kernel surfaces at the caller's next synchronisation.
 *   - Empty rows (no allowed key): o = 0, lse = sigma (or -inf).
 *   - NaN or Inf in q, k or v propagate; nothing scans the inputs.
 */
#ifndef SINK_ATTN_H_
#define SINK_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SINK_ATTN_OK = 0,
  SINK_ATTN_ERR_NULL_ARG = 1,     /* a required pointer is NULL              */
  SINK_ATTN_ERR_BAD_SHAPE = 2,    /* non-positive or inconsistent sizes      */
  SINK_ATTN_ERR_UNSUPPORTED = 3,  /* valid but not built (head_dim, ...)     */
  SINK_ATTN_ERR_MISALIGNED = 4,   /* a pointer breaks its alignment rule     */
  SINK_ATTN_ERR_WORKSPACE = 5,    /* workspace missing or too small          */
  SINK_ATTN_ERR_HIP = 6           /* the HIP runtime reported an error       */
} sink_attn_status;

typedef enum {
  SINK_ATTN_BF16 = 0,
  SINK_ATTN_F32 = 1
} sink_attn_dtype;

/*
 * Causal (or full) attention over a ragged batch of query chunks.
 * Prefill half of the sink-aware attention template (same section: one
 * template serves prefill and decode).
 *
 *   q            bf16 [total_q, Hq, 64]; request b owns query rows
 *                qo_indptr[b] .. qo_indptr[b+1]-1.
 *   qo_indptr    int32 [batch+1], non-decreasing, qo_indptr[0] = 0,
 *                qo_indptr[batch] = total_q.
 *   k, v         page_indices == NULL: contiguous bf16 [total_kv, Hkv, 64],
 *                request b owns tokens kv_indptr[b] .. kv_indptr[b+1]-1.
 *                page_indices != NULL: paged bf16 [num_pages, Hkv, 16, 64]
 *                (one 2 KiB block per page and KV head); token j of request
 *                b is slot j % 16 of page page_indices[kv_indptr[b] + j/16].
 *   kv_indptr    int32 [batch+1]: token offsets (contiguous) or offsets into
 *                page_indices (paged).
 *   page_indices int32 [nnz] page ids, or NULL for the contiguous layout.
 *   kv_len       int32 [batch] keys per request; required when paged, may
 *                be NULL when contiguous (then kv_indptr[b+1]-kv_indptr[b]).
 *                Query t of request b sits at absolute position
 *                kv_len[b] - qlen_b + t (the new tokens are the last qlen_b
 *                keys) and, when causal, sees keys 0 .. that position.
 *                Requires qlen_b <= kv_len[b] when causal.
 *   sinks        fp32 [Hq] or NULL.
 *   max_qlen     host upper bound of qlen_b (sizes the grid, no device read).
 *   max_kv_len   host upper bound of kv_len[b].
 *   sm_scale     tau, multiplies q.k (e.g. 1/sqrt(64)).
 *   causal       1 = causal, 0 = every query sees all kv_len[b] keys.
 *   out          [total_q, Hq, 64] in out_dtype (bf16 rounded to nearest
 *                even, or fp32).
 *   lse          fp32 [total_q, Hq] natural-log denominators, or NULL.
 */
sink_attn_status sink_attn_prefill(
    const void* q, const int32_t* qo_indptr,
    const void* k, const void* v, const int32_t* kv_indptr,
    const int32_t* page_indices, const int32_t* kv_len,
    const float* sinks,
    int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t page_size,
    int32_t total_q, int32_t max_qlen, int32_t max_kv_len,
    float sm_scale, int32_t causal,
    void* out, sink_attn_dtype out_dtype, float* lse,
    void* stream);

/*
 * Number of KV chunks per request of the split-KV plan for these sizes
 * (num_splits = 0: the planner's choice, as sink_attn_decode_partial uses
 * it; always >= 1).  Host-only: no launch, no copy.
 */
int32_t sink_attn_decode_num_splits(int32_t batch, int32_t num_qo_heads,
                                    int32_t num_kv_heads, int32_t max_kv_len,
                                    int32_t num_splits);

/*
 * Workspace bytes that sink_attn_decode needs for these sizes and
 * num_splits.  Takes num_kv_heads and max_kv_len besides the batch, head
 * and split counts because the automatic plan picks the load-balanced
 * workspace (sized by its page ranges per KV head) from them.  num_splits = 0 (the automatic plan): when max_kv_len exceeds
 * 16 pages the call runs the load-balanced plan and needs
 * sink_attn_decode_balanced_workspace_size(..., num_ranges = 0) bytes;
 * otherwise one chunk per request and 0 bytes.  num_splits = S > 0: 0 when
 * S = 1 (the kernel writes the output directly), else fp32 partial outputs
 * [batch, Hq, S, 64] followed by fp32 partial log-sum-exps [batch, Hq, S].
 */
size_t sink_attn_decode_workspace_size(int32_t batch, int32_t num_qo_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t max_kv_len, int32_t num_splits);

/*
 * One query token per request against a paged KV cache, split along the
 * KV length (same section: work parallelised across heads and along the
 * KV sequence; the sink enters the first chunk only).
 *
 *   q            bf16 [batch, Hq, 64]; the query of request b sits at
 *                position kv_len[b]-1 and sees all kv_len[b] keys (its own
 *                key/value are already in the cache).
 *   k_pages, v_pages, page_indptr, page_indices, kv_len: paged layout as in
 *                sink_attn_prefill (page_indptr = kv_indptr).
 *   max_kv_len   host upper bound of kv_len[b].
 *   num_splits   S >= 1 chunks of ceil(max_kv_len/S) keys rounded up to a
 *                multiple of 16.  Chunk 0 (keys 0 ..) carries the sink; a
 *                chunk past a request's keys is empty.  S > 1 writes
 *                partials to the workspace, then merges them on the same
 *                stream.  0 = the automatic plan: requests of up to 16 pages
 *                take one chunk; longer batches run sink_attn_decode_balanced
 *                with its automatic range count (same result, work split by
 *                pages across the whole batch).
 *   out          [batch, Hq, 64] in out_dtype;  lse fp32 [batch, Hq] or NULL.
 *   workspace    device buffer of at least sink_attn_decode_workspace_size()
 *                bytes (may be NULL when that size is 0).
 */
sink_attn_status sink_attn_decode(
    const void* q,
    const void* k_pages, const void* v_pages,
    const int32_t* page_indptr, const int32_t* page_indices,
    const int32_t* kv_len,
    const float* sinks,
    int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t page_size,
    int32_t max_kv_len, int32_t num_splits,
    float sm_scale,
    void* out, sink_attn_dtype out_dtype, float* lse,
    void* workspace, size_t workspace_bytes,
    void* stream);

/*
 * sink_attn_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same call and result as sink_attn_decode with the same arguments, minus
 * the workspace, which is taken from a fixed 16 MiB device array of this
 * library (one per GPU, held from library load until the process ends; its
 * device address is looked up once per device, on the first call made with
 * that device current).  Nothing is allocated or freed.
 *
 *   Limit: sink_attn_decode_workspace_size() for these arguments must be at
 *   most 16 MiB (16,777,216 bytes), else SINK_ATTN_ERR_WORKSPACE with nothing
 *   enqueued (for 64 query heads and the automatic plan, about 880 requests
 *   of up to 4,096 keys).  Sizes that need no workspace never touch the array.
 *   Every call on one GPU shares that GPU's array, which keeps the previous
 *   call's contents; nothing in it needs clearing between calls.  Calls that
 *   overlap in time on one GPU (other streams, other host threads) race on
 *   the array: serialise them.
 */
sink_attn_status sink_attn_decode_noalloc(
    const void* q,
    const void* k_pages, const void* v_pages,
    const int32_t* page_indptr, const int32_t* page_indices,
    const int32_t* kv_len,
    const float* sinks,
    int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t page_size,
    int32_t max_kv_len, int32_t num_splits,
    float sm_scale,
    void* out, sink_attn_dtype out_dtype, float* lse,
    void* stream);

/*
 * The first half of sink_attn_decode on its own: the split-KV partial pass,
 * without the merge.  Same arguments and planning as sink_attn_decode
 * (num_splits = 0 -> automatic plan; the plan's S is
 * sink_attn_decode_num_splits()).  Writes every chunk's partial, also when
 * S = 1, so that sink_attn_merge(o_parts, lse_parts, batch, Hq, S, ...)
 * completes the decode:
 *   o_parts      fp32 [batch, Hq, S, 64]  (each normalised by its own
 *                denominator; 0 for an empty chunk)
 *   lse_parts    fp32 [batch, Hq, S]      natural log; -inf for an empty
 *                chunk, sigma_h for an empty chunk 0 that holds the sink.
 */
sink_attn_status sink_attn_decode_partial(
    const void* q,
    const void* k_pages, const void* v_pages,
    const int32_t* page_indptr, const int32_t* page_indices,
    const int32_t* kv_len,
    const float* sinks,
    int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t page_size,
    int32_t max_kv_len, int32_t num_splits,
    float sm_scale,
    float* o_parts, float* lse_parts,
    void* stream);

/*
 * Merge of split-KV partials by log-sum-exp: L = max_c lse_c,
 * w_c = exp(lse_c - L), o = sum w_c o_c / sum w_c, lse = L + ln sum w_c.
 * Takes no sink: the sink already sits inside chunk 0's partial.
 *
 *   o_parts      fp32 [num_rows, num_heads, num_splits, 64], each partial
 *                normalised by its own denominator.
 *   lse_parts    fp32 [num_rows, num_heads, num_splits], natural log;
 *                -inf marks an empty chunk.
 *   out          [num_rows, num_heads, 64] in out_dtype; lse_out fp32
 *                [num_rows, num_heads] or NULL.  All chunks empty gives
 *                o = 0, lse = -inf.
 */
sink_attn_status sink_attn_merge(
    const float* o_parts, const float* lse_parts,
    int32_t num_rows, int32_t num_heads, int32_t num_splits, int32_t head_dim,
    void* out, sink_attn_dtype out_dtype, float* lse_out,
    void* stream);

/*
 * Load-balanced decode: the same result as sink_attn_decode, with the work
 * cut by pages instead of by request (same section: work parallelised
 * across heads and along the KV sequence, the sink entering once per
 * sequence).  Per KV head the batch's pages, page_indices[0 ..
 * page_indptr[batch]-1], are split into num_ranges equal ranges of
 * consecutive entries, one per wave, so every wave streams the same number
 * of pages whatever the mix of lengths.  A request that lies inside one
 * range is finished there; the partials of a request that spans several
 * ranges are merged by log-sum-exp in a second pass, the sink entering
 * only the partial that holds the request's first page.
 *
 * Arguments as in sink_attn_decode, except:
 *   page_indptr  rows of the page table must be non-decreasing with
 *                page_indptr[0] = 0; a request's row may hold more pages
 *                than ceil(kv_len[b]/16) (the extra keys are masked, but
 *                their pages are read) and must hold at least that many.
 *   num_ranges   ranges per KV head, rounded up to a multiple of 4, or 0 for
 *                the automatic plan (sink_attn_decode_num_ranges()).
 *   workspace    required: at least sink_attn_decode_balanced_workspace_size()
 *                bytes, 16-byte aligned.  Layout: fp32 partial outputs
 *                [num_ranges + batch - 1, Hq, 64], then fp32 partial
 *                log-sum-exps [num_ranges + batch - 1, Hq] at the next
 *                256-byte boundary.  Nothing needs clearing between calls;
 *                calls that share one workspace must not overlap in time.
 */
int32_t sink_attn_decode_num_ranges(int32_t batch, int32_t num_kv_heads, int32_t max_kv_len,
                                    int32_t num_ranges);

size_t sink_attn_decode_balanced_workspace_size(int32_t batch, int32_t num_qo_heads,
                                                int32_t num_kv_heads, int32_t head_dim,
                                                int32_t max_kv_len, int32_t num_ranges);

/* Both passes, enqueued on `stream`. */
sink_attn_status sink_attn_decode_balanced(
    const void* q,
    const void* k_pages, const void* v_pages,
    const int32_t* page_indptr, const int32_t* page_indices,
    const int32_t* kv_len,
    const float* sinks,
    int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t page_size,
    int32_t max_kv_len, int32_t num_ranges,
    float sm_scale,
    void* out, sink_attn_dtype out_dtype, float* lse,
    void* workspace, size_t workspace_bytes,
    void* stream);

/*
 * The first pass alone: streams the pages, writes out/lse of every request
 * that lies inside one range and the partials of the others into the
 * workspace.  sink_attn_decode_balanced_finish with the same sizes,
 * num_ranges, out, lse and workspace completes the call.
 */
sink_attn_status sink_attn_decode_balanced_partial(
    const void* q,
    const void* k_pages, const void* v_pages,
    const int32_t* page_indptr, const int32_t* page_indices,
    const int32_t* kv_len,
    const float* sinks,
    int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t page_size,
    int32_t max_kv_len, int32_t num_ranges,
    float sm_scale,
    void* out, sink_attn_dtype out_dtype, float* lse,
    void* workspace, size_t workspace_bytes,
    void* stream);

/*
 * The second pass alone: merges the partials of every request that spans
 * several ranges and writes requests without pages (o = 0, lse = sigma or
 * -inf).  Reads page_indptr and the workspace the first pass wrote.
 */
sink_attn_status sink_attn_decode_balanced_finish(
    const int32_t* page_indptr, const float* sinks,
    int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t max_kv_len, int32_t num_ranges,
    void* out, sink_attn_dtype out_dtype, float* lse,
    void* workspace, size_t workspace_bytes,
    void* stream);

/*
 * Multi-token verification: a few new tokens per request (the drafted tokens
 * of speculative decoding, checked in one pass) against a paged KV cache.
 * The same operation as sink_attn_prefill on a paged cache with causal = 1,
 * built like the split-KV decode: work parallel over heads and along the KV
 * length, the sink in chunk 0 only (same section as sink_attn_decode), and
 * the drafted tokens x G query heads of a request packed into the matrix
 * columns, so a short draft streams the cache at decode speed.
 *
 *   q, qo_indptr     bf16 [total_q, Hq, 64]; request b owns rows
 *                    qo_indptr[b] .. qo_indptr[b+1]-1 (its qlen_b drafted
 *                    tokens, in order).
 *   k_pages ... kv_len, sinks: as sink_attn_decode.  Token t of request b sits
 *                    at position kv_len[b] - qlen_b + t (the drafted tokens
 *                    are the last qlen_b keys of the cache) and sees keys 0 ..
 *                    that position.  Requires 1 <= qlen_b <= kv_len[b] for
 *                    every request with rows.
 *   total_q, max_qlen host scalars: rows, and an upper bound of qlen_b.
 *                    max_qlen must be <= 64 (SINK_ATTN_ERR_UNSUPPORTED
 *                    otherwise: use sink_attn_prefill).  A (request, KV
 *                    head) has C = max_qlen x Hq / Hkv (token, head) pairs.
 *                    C <= 64: each chunk runs one workgroup when C <= 16,
 *                    else ceil(C / 32) workgroups of 32 pairs.  C > 64 (with
 *                    Hq / Hkv in {1, 2, 4, 8, 16}): each chunk runs
 *                    ceil(C / 128) workgroups of 128 pairs that stage the
 *                    request's K/V tiles in LDS, and chunks are whole
 *                    64-key tiles.
 *   num_splits       0: automatic plan (sink_attn_verify_num_splits).  C <=
 *                    64: one chunk per request when the grid already holds
 *                    >= 256 workgroups, else enough chunks of >= 16 pages
 *                    for about 512.  C > 64: chunks of >= 512 keys towards
 *                    1,024 (request, KV head, chunk) items (each one
 *                    workgroup per 128-pair group), at most 64 chunks.
 *                    S > 0: S chunks per request of ceil(max_kv_len / S)
 *                    keys, rounded up to a multiple of 16 (C <= 64) or of
 *                    64 (C > 64; at most 64 chunks); a chunk past a
 *                    request's keys is empty.
 *   out, lse         [total_q, Hq, 64] in out_dtype; fp32 [total_q, Hq] or
 *                    NULL (natural log).
 *   workspace        sink_attn_verify_workspace_size() bytes (0 with one
 *                    split): fp32 partials [total_q, Hq, S, 64], then fp32
 *                    [total_q, Hq, S] at the next 256-byte boundary.
 */
size_t sink_attn_verify_workspace_size(int32_t batch, int32_t num_qo_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t total_q, int32_t max_qlen,
                                       int32_t max_kv_len, int32_t num_splits);

/*
 * The chunk count S that sink_attn_verify and sink_attn_verify_tree use for
 * these sizes (num_splits = 0: the automatic plan above).  Host-only (no
 * launch, no copy); 1 for invalid sizes.
 */
int32_t sink_attn_verify_num_splits(int32_t batch, int32_t num_qo_heads,
                                    int32_t num_kv_heads, int32_t max_qlen,
                                    int32_t max_kv_len, int32_t num_splits);

sink_attn_status sink_attn_verify(
    const void* q, const int32_t* qo_indptr,
    const void* k_pages, const void* v_pages,
    const int32_t* page_indptr, const int32_t* page_indices,
    const int32_t* kv_len,
    const float* sinks,
    int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t page_size,
    int32_t total_q, int32_t max_qlen, int32_t max_kv_len, int32_t num_splits,
    float sm_scale,
    void* out, sink_attn_dtype out_dtype, float* lse,
    void* workspace, size_t workspace_bytes,
    void* stream);

/*
 * Verification of a tree of drafted tokens ("Accelerating Sonar Through
 * Speculation", Perplexity, section "EAGLE": tree-shaped drafts are checked in
 * one target pass under custom attention masks; the page notes that dense
 * full-sequence masks slowed attention by up to half).  The mask here is one
 * 64-bit word per drafted token: the prefix is always visible, and the mask
 * replaces causality among the drafted tokens only.
 *
 *   draft_mask       uint64 [total_q], 8-byte aligned, device memory.  Row r
 *                    = qo_indptr[b] + t (drafted token t of request b) sees
 *                    every key j < P = kv_len[b] - qlen_b, and drafted key
 *                    P + i (i < qlen_b) exactly when bit i of draft_mask[r]
 *                    is set.  Bits at or above qlen_b are ignored.  A token
 *                    normally sees itself and its ancestors; a row that sees
 *                    no key at all gets o = 0, lse = sigma.
 *   everything else  as sink_attn_verify (same limits, same workspace size:
 *                    sink_attn_verify_workspace_size).
 *
 * SINK_ATTN_ERR_NULL_ARG without a mask; SINK_ATTN_ERR_MISALIGNED if it is
 * not 8-byte aligned.
 */
sink_attn_status sink_attn_verify_tree(
    const void* q, const int32_t* qo_indptr, const uint64_t* draft_mask,
    const void* k_pages, const void* v_pages,
    const int32_t* page_indptr, const int32_t* page_indices,
    const int32_t* kv_len,
    const float* sinks,
    int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t page_size,
    int32_t total_q, int32_t max_qlen, int32_t max_kv_len, int32_t num_splits,
    float sm_scale,
    void* out, sink_attn_dtype out_dtype, float* lse,
    void* workspace, size_t workspace_bytes,
    void* stream);

/*
 * The step before attention: the QKV projection's bias, YaRN rotary position
 * encoding and the append of the new keys and values to the paged cache.
 * "GPT-OSS on Day 0" (Perplexity), "Attention: GQA with attention sinks":
 * YaRN positions and QKV bias are listed as model changes, with no formula;
 * YaRN is read as published (Peng et al. 2023, "NTK-by-parts" frequencies
 * plus the attention temperature 0.1 ln s + 1 on q and k).  "Accelerating
 * Sonar Through Speculation" (Perplexity), "Inference with Speculative
 * Decoding": room for the next tokens is reserved in the paged cache before
 * the step runs.
 *
 * sink_attn_rope_table fills the cos/sin table once (at model load):
 *   table            fp32 [max_pos, 64], 16-byte aligned, device memory;
 *                    column d < 32 = T cos(p f_d), column 32 + d = T sin(p f_d)
 *                    for position p and pair d, T the temperature.
 *   rope_theta       base of the frequencies f_d = theta^(-2d/64) (> 1).
 *   factor           YaRN scale s; s <= 1 gives plain rotary frequencies.
 *   original_max_pos, beta_fast, beta_slow
 *                    YaRN's L, beta and alpha (used when s > 1): pair d keeps
 *                    f_d when it turns more than beta_fast times in L tokens,
 *                    gets f_d / s when it turns fewer than beta_slow times,
 *                    and a blend of the two between.
 *   attn_factor      T; 0 selects 0.1 ln s + 1 (1 when s <= 1).
 *   yarn_ramp        the blend between the two bounds:
 *                    SINK_ATTN_YARN_RAMP_TURNS (0): linear in the turn count
 *                    r_d = L f_d / (2 pi), as the YaRN paper writes it;
 *                    SINK_ATTN_YARN_RAMP_PAIRS (1): linear in the pair index
 *                    between low = floor(d(beta_fast)) and high =
 *                    ceil(d(beta_slow)), d(r) = 64 ln(L / (2 pi r)) /
 *                    (2 ln theta) the pair that turns r times (clamped to
 *                    0 .. 31; a step at low when high <= low), as DeepSeek-V3,
 *                    which the page names, and the YaRN authors' code do.
 *                    The two agree on which pairs keep, blend or divide by
 *                    s.  Other values: SINK_ATTN_ERR_UNSUPPORTED.
 * Angles and sin/cos are evaluated in fp64.  SINK_ATTN_ERR_BAD_SHAPE for
 * max_pos < 1, theta <= 1, factor <= 0, attn_factor < 0, or (s > 1)
 * original_max_pos < 1 or not 0 < beta_slow < beta_fast.
 */
typedef enum {
  SINK_ATTN_YARN_RAMP_TURNS = 0,
  SINK_ATTN_YARN_RAMP_PAIRS = 1
} sink_attn_yarn_ramp;

sink_attn_status sink_attn_rope_table(float* table, int32_t max_pos, int32_t head_dim,
                                      double rope_theta, double factor,
                                      int32_t original_max_pos, double beta_fast,
                                      double beta_slow, double attn_factor,
                                      sink_attn_yarn_ramp yarn_ramp, void* stream);

/*
 * sink_attn_qkv_rope_append: for every new token, add the bias to its fused
 * QKV projection row, rotate the query and key heads by the token's position,
 * write the queries to q_out and the keys and values into the token's cache
 * slot.  Nothing else of the cache is written.
 *
 *   qkv              bf16 [total_q, Hq + 2 Hkv, 64]: the Hq query heads, then
 *                    the Hkv key heads, then the Hkv value heads of each token.
 *   bias             bf16 [(Hq + 2 Hkv) x 64] in the same head order, or NULL.
 *                    Added before the rotation; value heads get the bias only.
 *   rope_table, max_pos  the table above.
 *   qo_indptr        [batch + 1]: request b's new tokens are rows
 *                    qo_indptr[b] .. qo_indptr[b+1]-1.
 *   kv_len           [batch]: keys of request b counting the new ones; token t
 *                    of request b sits at position p = kv_len[b] - qlen_b + t.
 *   page_indptr, page_indices  request b's pages (reserved for every
 *                    position < kv_len[b]); the token's key and value go to slot
 *                    p % 16 of page page_indices[page_indptr[b] + p / 16],
 *                    layout [num_pages, Hkv, 16, 64] as everywhere in this
 *                    library.
 *   interleaved      0: dimension i pairs with i + 32 (rotate-half layout);
 *                    1: dimension 2i pairs with 2i + 1.
 *   q_out            bf16 [total_q, Hq, 64], ready for sink_attn_prefill,
 *                    sink_attn_decode or sink_attn_verify.
 * Results are rounded to bf16 (round to nearest even) once, after the fp32
 * bias add and rotation.  A token whose position is outside [0, max_pos) or
 * past its request's pages is skipped (nothing of it is written); device
 * data is not otherwise checked.  Host checks as the other entry points
 * (NULL, shapes, 16-byte alignment of tensors, 4-byte of index arrays).
 */
sink_attn_status sink_attn_qkv_rope_append(
    const void* qkv, const void* bias, const float* rope_table, int32_t max_pos,
    const int32_t* qo_indptr, const int32_t* kv_len,
    const int32_t* page_indptr, const int32_t* page_indices,
    int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t page_size, int32_t total_q, int32_t interleaved,
    void* q_out, void* k_pages, void* v_pages, void* stream);

/*
 * sink_attn_prefill_step: one prefill (or chunked-prefill, or verification)
 * step in one call -- the new tokens' QKV bias and rotary encoding, the
 * append of their keys and values to the paged cache, and the causal (or
 * full) attention of their queries over the cache.  The result (out, lse
 * and the cache) equals, bit for bit,
 *     sink_attn_qkv_rope_append(qkv, bias, rope_table, max_pos, qo_indptr,
 *         kv_len, page_indptr, page_indices, batch, Hq, Hkv, 64, 16,
 *         total_q, interleaved, q, k, v)
 *     sink_attn_prefill(q, qo_indptr, k, v, page_indptr, page_indices,
 *         kv_len, sinks, batch, Hq, Hkv, 64, 16, total_q, max_qlen,
 *         max_kv_len, sm_scale, causal, out, out_dtype, lse)
 * but the rotated queries are never written out: the append writes the key
 * and value heads only, and the attention kernel reads each query from its
 * projection row, adding the bias and rotating it as it loads it.  GPT-OSS
 * on Day 0, "Attention: GQA with attention sinks" (bias, YaRN) and "Sink
 * attention"; Accelerating Sonar Through Speculation, "Inference with
 * Speculative Decoding" (the new tokens' cache slots are reserved before
 * the step).
 *
 *   qkv, bias, rope_table, max_pos, interleaved  as sink_attn_qkv_rope_append.
 *   qo_indptr, kv_len, page_indptr, page_indices  as both calls above (a
 *                    paged cache; kv_len counts the new tokens).
 *   k_pages, v_pages the cache, written at the new tokens' slots and read.
 *   the rest         as sink_attn_prefill.
 * A token whose position is not in [0, max_pos) is not appended and its
 * row's result is unspecified.  Host checks: those of both calls, before
 * either kernel is launched.
 */
sink_attn_status sink_attn_prefill_step(
    const void* qkv, const void* bias, const float* rope_table, int32_t max_pos,
    int32_t interleaved, const int32_t* qo_indptr, void* k_pages, void* v_pages,
    const int32_t* page_indptr, const int32_t* page_indices, const int32_t* kv_len,
    const float* sinks, int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t page_size, int32_t total_q, int32_t max_qlen,
    int32_t max_kv_len, float sm_scale, int32_t causal,
    void* out, sink_attn_dtype out_dtype, float* lse, void* stream);

/*
 * sink_attn_decode_step: one decode step in one call -- each request's one
 * new token gets its QKV bias and rotary encoding and is appended to the
 * paged cache, and the decode then attends over the cache including it.
 * The result (out, lse and the cache) equals, bit for bit,
 *     sink_attn_qkv_rope_append(qkv, bias, rope_table, max_pos,
 *         qo_indptr = 0, 1, .., batch, kv_len, page_indptr, page_indices,
 *         batch, Hq, Hkv, 64, 16, total_q = batch, interleaved, q, k, v)
 *     sink_attn_decode_balanced(q, k, v, page_indptr, page_indices, kv_len,
 *         sinks, batch, Hq, Hkv, 64, 16, max_kv_len, num_ranges = 0, ...)
 * but runs as two kernels instead of three: before it streams its pages,
 * each wave of the decode's first pass appends the new keys and values of
 * its own pages and rotates the queries of the requests it reads (into the
 * workspace).
 * GPT-OSS on Day 0, "Attention: GQA with attention sinks" (bias, YaRN) and
 * "Sink attention"; Accelerating Sonar Through Speculation, "Inference with
 * Speculative Decoding" (the new token's cache slot is reserved before the
 * step).
 *
 *   qkv, bias        as sink_attn_qkv_rope_append, one row per request:
 *                    bf16 [batch, Hq + 2 Hkv, 64]; bias may be NULL.
 *   rope_table, max_pos, interleaved  as sink_attn_qkv_rope_append.
 *   k_pages, v_pages the cache, read by the decode and written at each
 *                    request's new slot: position p = kv_len[b] - 1, slot
 *                    p % 16 of page page_indices[page_indptr[b] + p / 16].
 *   kv_len           [batch]: keys of each request counting the new token.
 *   the rest         as sink_attn_decode_balanced with num_ranges = 0.
 *   workspace        sink_attn_decode_step_workspace_size() bytes: the
 *                    balanced decode's partials, then the rotated queries
 *                    (bf16 [batch, Hq, 64]).
 * A request whose new position is not in [0, max_pos) is not written to the
 * cache and its output is unspecified (its table row is read clamped);
 * requests with kv_len = 0 get o = 0, lse = sink as in the decode.  Host
 * checks as sink_attn_decode_balanced plus rope_table (non-NULL, 16-byte
 * aligned), bias (16-byte aligned), max_pos >= 1, interleaved in {0, 1}
 * and the workspace size.
 */
size_t sink_attn_decode_step_workspace_size(int32_t batch, int32_t num_qo_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t max_kv_len);
sink_attn_status sink_attn_decode_step(
    const void* qkv, const void* bias, const float* rope_table, int32_t max_pos,
    int32_t interleaved, void* k_pages, void* v_pages,
    const int32_t* page_indptr, const int32_t* page_indices, const int32_t* kv_len,
    const float* sinks, int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t page_size, int32_t max_kv_len, float sm_scale,
    void* out, sink_attn_dtype out_dtype, float* lse,
    void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* sink_attn_status_string(sink_attn_status s);

/* Detail of the calling thread's last failed call ("" if none). */
const char* sink_attn_last_error(void);

/* Library version string. */
const char* sink_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SINK_ATTN_H_ */
