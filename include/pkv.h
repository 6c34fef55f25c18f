/*
 * pkv.h -- paged, variable-length attention over a page-table-indexed KV cache,
 * for AMD Instinct MI355X (gfx950). C ABI of libpkv.so.
 *
 * Passages cited below are from these pages (title; section = function/class):
 *   [DCA] "sglang 0.4.10.post2 -> 0.5.0rc0: sglang/srt/layers/attention/
 *          dual_chunk_flashattention_backend.py"
 *   [FA]  "sgl-project--sglang/python/sglang/srt/layers/attention/
 *          flashattention_backend.py"
 *   [NSA] "sglang/srt/layers/attention/nsa_backend.py"
 *
 * Conventions shared by every entry point
 *   - Every array argument is a caller-owned DEVICE pointer (hipMalloc'd or a
 *     torch tensor's data_ptr()), dense and row-major in the layout given.
 *     The library allocates nothing, keeps no state between calls and is
 *     reentrant; the one exception is sparse_topk_decode_noalloc, whose
 *     per-GPU static device array holds its split workspace (see there).
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued on
 *     it and the call returns without synchronising.
 *   - Return value is a pkv_status_t. Argument errors that the host can see
 *     (NULL required pointers, bad sizes, unsupported head dims or dtypes) are
 *     reported synchronously before anything is enqueued; PKV_ELAUNCH reports a
 *     failed kernel launch. pkv_last_error() gives a human-readable detail for
 *     the calling thread.
 *   - Device-data preconditions (index ranges, lengths that fit the tables) are
 *     not validated; kernels clamp every index they dereference to the array
 *     sizes passed in, so a violated precondition gives wrong numbers, never an
 *     out-of-bounds access.
 *   - bf16 is IEEE binary16-brain (1-8-7), stored as 16-bit words; results in
 *     bf16 are rounded to nearest even. Arithmetic is fp32. LSE is the natural
 *     log of the softmax denominator (scale included); an empty key set gives
 *     O = 0 and LSE = -inf ([DCA] _dual_chunk_flash_attn_decoding_with_exp_sums).
 *   - LSE arrays are token-major [tokens, heads] ([FA] forward_extend passes
 *     softmax_lse.T.contiguous() to merge_state_v2).
 *   - softmax_scale must be finite and > 0 (the pages pass 1/sqrt(head dim));
 *     every attention entry point returns PKV_EINVAL otherwise.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = 1,       /* bad argument (NULL, negative size, inconsistent sizes) */
  PKV_EUNSUPPORTED = 2, /* well-formed but not instantiated (head dim, dtype, group) */
  PKV_ELAUNCH = 3       /* the HIP runtime rejected a launch */
} pkv_status_t;

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype_t;

/*
 * Workspaces (paged_attn_varlen_prefill[_append], paged_attn_cascade,
 * paged_attn_decode_merged, sparse_topk_decode). A workspace starts with
 * PKV_WORKSPACE_COUNTER_BYTES bytes of completion counters at a fixed place
 * that does not depend on the call's shape; the per-split partial results
 * follow them. Hence one buffer, at least as large as the size function
 * returns for each shape, serves calls of any shape in any order. Before its
 * first use the counter region must be zero (any fill on the stream:
 * hipMemsetAsync, torch.zero_); every launch that runs to completion leaves it
 * zero again. A call rejected by its argument checks has enqueued nothing and
 * has left it as it was. Calls that share a workspace must be ordered (one
 * stream, or synchronised).
 */
#define PKV_WORKSPACE_COUNTER_BYTES 65536

/* Static string naming a status code. */
const char* pkv_status_string(int status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* pkv_last_error(void);

/*
 * build_page_table -- integer metadata for one forward pass.
 *
 * Strided mode (prefill_lens == NULL), [FA] init_forward_metadata (decode and
 * extend branches, token slots reduced to page ids); [DCA] init_forward_metadata:
 *   page_table[b, p] = req_to_token[r, p * page_size] / page_size
 *       for p < ceil(L_b / page_size), else 0,   r = req_pool_indices[b],
 *   kv_lens[b] = L_b = seq_lens[b].
 * Prefill-aware sliding-window mode (prefill_lens != NULL, page_size must be 1),
 * [FA] _build_pa_page_table_kernel / _build_pa_page_table:
 *   pf = prefill_lens[r]  (pool-sized array, indexed by the pool row),
 *   decode_start = max(pf, seq_lens[b] - window),
 *   gap = decode_start > pf ? decode_start - pf : 0,
 *   kv_lens[b] = seq_lens[b] - gap,
 *   page_table[b, j] = req_to_token[r, j < pf ? j : j + gap] for j < kv_lens[b],
 *   else 0.
 * Both modes, when cu_seqlens_k != NULL: cu_seqlens_k = [0, cumsum(kv_lens)].
 *
 * req_to_token  [req_to_token_rows, req_to_token_stride] int32 token slot ids
 * req_pool_indices [batch] int32 rows of req_to_token
 * seq_lens      [batch] int32
 * prefill_lens  [req_to_token_rows] int32, or NULL
 * page_table    [batch, width] int32 (out; every element written)
 * kv_lens       [batch] int32 (out)
 * cu_seqlens_k  [batch + 1] int32 (out) or NULL
 * Errors: PKV_EINVAL for NULL required pointers, batch < 0, width < 0,
 * page_size < 1, rows/stride < 1 with batch > 0, window < 0 or page_size != 1
 * in sliding-window mode. batch == 0 is a no-op apart from cu_seqlens_k[0] = 0.
 */
pkv_status_t build_page_table(const int32_t* req_to_token, int64_t req_to_token_rows,
                              int64_t req_to_token_stride, const int32_t* req_pool_indices,
                              const int32_t* seq_lens, const int32_t* prefill_lens,
                              int32_t window, int32_t batch, int32_t page_size, int32_t width,
                              int32_t* page_table, int32_t* kv_lens, int32_t* cu_seqlens_k,
                              void* stream);

/*
 * paged_attn_varlen_prefill -- causal extend over a paged cache.
 * [FA] forward_extend (flash_attn_with_kvcache with cache_seqlens = prefix + new,
 * cu_seqlens_q over the new tokens, causal=True). Request b owns q rows
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]) = M_b rows; its L_b = kv_lens[b] keys
 * are read through page_table row b (key t at k_cache[page_table[b, t / P], t % P]).
 * New row j sits at position L_b - M_b + j and, when causal, sees keys
 * [0, L_b - M_b + j] (bottom-right alignment, [NSA] _cal_indexer_k_start_end);
 * otherwise all L_b keys. q head h reads kv head h / (Hq / Hkv).
 * Masks on top of causal ([FA] forward_extend window_size and
 * make_local_attention_virtual_batches); at most one of the two is set:
 *   window_left = W >= 0: sliding window (W, 0), the row at position p sees
 *          keys [max(0, p - W), p] (W + 1 keys); -1 turns it off.
 *   attn_chunk = C > 0: chunked local attention, the row at position p sees
 *          keys [floor(p / C) * C, p], the same as splitting each request into
 *          C-aligned virtual requests; 0 turns it off.
 *
 * q        [total_q, num_q_heads, head_dim]         dtype
 * k_cache, v_cache [num_pages, page_size, num_kv_heads, head_dim] dtype
 * page_table [batch, pt_stride] int32 page ids; cu_seqlens_q [batch + 1];
 * kv_lens [batch] int32 (requires L_b <= pt_stride * page_size, and M_b <= L_b when causal)
 * max_seqlen_q >= every M_b and max_seqlen_k >= every L_b: launch bounds, as
 *          in flash_attn_varlen_func; they size the grid and the key splits.
 *          (A max_seqlen_k below some L_b is still correct, only slower.)
 * workspace caller-owned device memory of at least
 *          paged_attn_varlen_prefill_workspace_size(...) bytes (0 when no q
 *          tile is split: NULL allowed); layout and zeroing rule as stated at
 *          PKV_WORKSPACE_COUNTER_BYTES.
 * out      [total_q, num_q_heads, head_dim] dtype (out); lse [total_q, num_q_heads]
 *          fp32 (out) or NULL.
 * Supported: dtype PKV_BF16, head_dim 64 or 128, Hq % Hkv == 0,
 * Hq / Hkv <= 16, causal 0 or 1, num_pages * page_size < 2^31.
 * Errors: PKV_EINVAL for bad sizes, NULL pointers, a short workspace,
 * window_left < -1, attn_chunk < 0, both masks set, or a mask with causal 0;
 * PKV_EUNSUPPORTED outside the supported set.
 */
size_t paged_attn_varlen_prefill_workspace_size(int32_t batch, int32_t total_q,
                                                int32_t max_seqlen_q, int32_t max_seqlen_k,
                                                int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t head_dim);
pkv_status_t paged_attn_varlen_prefill(const void* q, int32_t dtype, const void* k_cache,
                                       const void* v_cache, int64_t num_pages,
                                       const int32_t* page_table, int32_t pt_stride,
                                       const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                                       int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                                       int32_t max_seqlen_k, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                       float softmax_scale, int32_t causal, int32_t window_left,
                                       int32_t attn_chunk, void* workspace,
                                       size_t workspace_bytes, void* out, float* lse,
                                       void* stream);

/*
 * paged_kv_append -- write new tokens' keys and values into the cache.
 * [FA] forward_extend / forward_decode: before attending, the layer's new k and
 * v are stored with set_kv_buffer at out_cache_loc:
 *   k_cache[out_cache_loc[i]] = k_new[i],  v_cache[out_cache_loc[i]] = v_new[i]
 * where a slot indexes the cache viewed as [num_slots, Hkv, D]
 * (num_slots = num_pages * page_size; slot s is page s / P, position s % P).
 *
 * k_new, v_new   [n_tokens, num_kv_heads, head_dim], dtype (PKV_BF16 or PKV_F32)
 * out_cache_loc  [n_tokens] int32, distinct slots (a slot outside [0, num_slots)
 *                is skipped; repeated slots leave an unspecified one of the rows)
 * k_cache, v_cache  the cache, same dtype, written in place.
 * Errors: PKV_EINVAL for NULL pointers (n_tokens > 0) or bad sizes;
 * PKV_EUNSUPPORTED for another dtype or head_dim * element size not a multiple
 * of 16 bytes. n_tokens == 0 enqueues nothing.
 */
pkv_status_t paged_kv_append(const void* k_new, const void* v_new, int32_t dtype,
                             const int32_t* out_cache_loc, int32_t n_tokens, int32_t num_kv_heads,
                             int32_t head_dim, void* k_cache, void* v_cache, int64_t num_slots,
                             void* stream);

/*
 * paged_attn_varlen_prefill_append -- the extend step with its cache write:
 * [FA] forward_extend with save_kv_cache, i.e. paged_kv_append of the new
 * tokens (k_new / v_new [total_q, Hkv, D], one row per new token in
 * cu_seqlens_q order, slots out_cache_loc [total_q]) followed by
 * paged_attn_varlen_prefill over the updated cache. Arguments as for those
 * two calls (the caches are written, hence not const). The caller's page
 * table maps position kv_lens[b] - M_b + j of request b to slot
 * out_cache_loc[cu_seqlens_q[b] + j], as the pages' req_to_token does, and no
 * request's cached prefix uses those slots. Every argument is checked before
 * anything is enqueued; then two kernels run on the stream (the scatter, then
 * the attention).
 */
pkv_status_t paged_attn_varlen_prefill_append(
    const void* q, int32_t dtype, void* k_cache, void* v_cache, int64_t num_pages,
    const int32_t* page_table, int32_t pt_stride, const int32_t* cu_seqlens_q,
    const int32_t* kv_lens, int32_t batch, int32_t total_q, int32_t max_seqlen_q,
    int32_t max_seqlen_k, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t page_size, float softmax_scale, int32_t causal, int32_t window_left,
    int32_t attn_chunk, const void* k_new, const void* v_new, const int32_t* out_cache_loc,
    void* workspace, size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * paged_attn_decode_splitkv -- one query token per request, key axis split.
 * [FA] forward_decode (flash_attn_with_kvcache, num_splits); [DCA]
 * _dual_chunk_flash_attn_decoding (partial decodes over disjoint key ranges
 * returning LSE, empty ranges forced to (0, -inf)).
 * Split s of request b covers keys [s * kv_chunk, min((s + 1) * kv_chunk, L_b));
 * it yields the attention output normalised over that range alone, O_s, and
 * LSE_s; an empty range yields (0, -inf). kv_chunk == 0 means one split.
 * The query sits at position L_b - 1. window_left = W >= 0 keeps only keys
 * [max(0, L_b - 1 - W), L_b - 1] and attn_chunk = C > 0 only keys
 * [floor((L_b - 1) / C) * C, L_b - 1] ([FA] forward_decode window_size, local
 * attention); splits outside the kept range are empty. -1 / 0 turn them off;
 * at most one may be set (PKV_EINVAL otherwise, or for W < -1 or C < 0).
 *
 * q        [batch, num_q_heads, head_dim] dtype
 * k_cache, v_cache [num_pages, page_size, num_kv_heads, head_dim] dtype
 * page_table [batch, pt_stride] int32; kv_lens [batch] int32
 *          (requires L_b <= pt_stride * page_size and L_b <= num_splits * kv_chunk)
 * num_splits == 1: writes out [batch, num_q_heads, head_dim] (dtype) and, if
 *          non-NULL, lse [batch, num_q_heads]; o_partial/lse_partial unused.
 * num_splits > 1: writes o_partial [num_splits, batch, num_q_heads, head_dim]
 *          fp32 and lse_partial [num_splits, batch, num_q_heads] fp32 (combine
 *          them with merge_state); out/lse unused.
 * Supported: dtype PKV_F32 or PKV_BF16, head_dim 64 or 128, Hq % Hkv == 0,
 * Hq / Hkv <= 16. kv_chunk must be a multiple of page_size ([DCA]
 * _dual_chunk_flash_attn_prefill_func rejects chunks not divisible by the
 * block size) and of 32.
 */
pkv_status_t paged_attn_decode_splitkv(const void* q, int32_t dtype, const void* k_cache,
                                       const void* v_cache, int64_t num_pages,
                                       const int32_t* page_table, int32_t pt_stride,
                                       const int32_t* kv_lens, int32_t batch,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t page_size, float softmax_scale,
                                       int32_t window_left, int32_t attn_chunk,
                                       int32_t kv_chunk, int32_t num_splits, float* o_partial,
                                       float* lse_partial, void* out, float* lse, void* stream);

/*
 * paged_attn_decode_merged -- paged_attn_decode_splitkv and merge_state over
 * its num_splits parts in one call ([FA] forward_decode runs the split decode
 * and its combine back to back; [DCA] _dual_chunk_flash_attn_decoding merges
 * the partial decodes it has just produced). Arguments as for
 * paged_attn_decode_splitkv, except:
 * kv_chunk, num_splits: as for paged_attn_decode_splitkv, or both 0 for
 *          balanced ranges: the visible keys of all requests, laid end to end
 *          in 16-key tiles, are cut into equal ranges, one per workgroup of a
 *          single round on a 256-CU device (256 workgroups in all, one per
 *          CU), each of at least 8 tiles; a range may end one request and start the next. A
 *          request covered by one range is written directly; otherwise each
 *          range's part is handed over and the last of them to finish merges
 *          them in range order (so the result does not depend on timing).
 *          Needs at most 2^24 keys per request (pt_stride * page_size); where
 *          this or the group kernel (below) does not apply, the library picks
 *          fixed splits of at most 8 per request instead.
 * workspace: device scratch of at least
 *          paged_attn_decode_merged_workspace_size(...) bytes (may be NULL when
 *          that size is 0, i.e. num_splits == 1): completion counters (one per
 *          request and group of 256 / head_dim kv heads, in the counter
 *          region), then the partials o [parts, num_q_heads, head_dim] fp32 and
 *          lse [parts, num_q_heads] fp32, each 256-byte aligned, with parts =
 *          num_splits * batch (fixed splits, split-major) or 256 + 8 * batch
 *          (balanced ranges); layout and zeroing rule as stated at
 *          PKV_WORKSPACE_COUNTER_BYTES.
 * out      [batch, num_q_heads, head_dim] dtype (out); lse [batch, num_q_heads]
 *          fp32 (out) or NULL.
 * With fixed splits the result is bit-identical to paged_attn_decode_splitkv
 * followed by merge_state on the same arguments; with balanced ranges it is
 * the same attention over other part boundaries (equal within rounding). On the
 * bf16 kv-head-group kernel (bf16, 256 / head_dim kv heads whose query heads
 * fit 16 columns) this is one launch; otherwise the decode and merge_state
 * kernels run back to back. A request with no visible key gets (0, -inf).
 * Errors as for paged_attn_decode_splitkv, plus PKV_EINVAL for a NULL out or a
 * workspace smaller than the size function returns.
 */
size_t paged_attn_decode_merged_workspace_size(int32_t batch, int32_t num_q_heads,
                                               int32_t head_dim, int32_t num_splits);

pkv_status_t paged_attn_decode_merged(const void* q, int32_t dtype, const void* k_cache,
                                      const void* v_cache, int64_t num_pages,
                                      const int32_t* page_table, int32_t pt_stride,
                                      const int32_t* kv_lens, int32_t batch, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                      float softmax_scale, int32_t window_left, int32_t attn_chunk,
                                      int32_t kv_chunk, int32_t num_splits, void* workspace,
                                      size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * merge_state -- combine partial attention states over disjoint key sets.
 * [DCA] _merge_attn_outputs and the merge closing _dual_chunk_flash_attn_decoding;
 * [FA] forward_extend / forward_decode call merge_state_v2(o_a, lse_a, o_b, lse_b)
 * (this is its S-way form):
 *   m = max_s lse[s], w_s = exp(lse[s] - m),
 *   out = sum_s w_s o[s] / sum_s w_s, lse_out = m + ln(sum_s w_s);
 *   m == -inf gives (0, -inf). A part with lse -inf (an empty split) adds
 *   nothing, whatever its o holds (NaN included).
 * o_parts [num_parts, n_tokens, num_heads, head_dim_v] fp32;
 * lse_parts [num_parts, n_tokens, num_heads] fp32;
 * out [n_tokens, num_heads, head_dim_v] of out_dtype (out);
 * lse_out [n_tokens, num_heads] fp32 (out) or NULL.
 * Errors: PKV_EINVAL for NULL, num_parts < 1, negative sizes.
 */
pkv_status_t merge_state(const float* o_parts, const float* lse_parts, int32_t num_parts,
                         int32_t n_tokens, int32_t num_heads, int32_t head_dim_v, void* out,
                         int32_t out_dtype, float* lse_out, void* stream);

/*
 * sparse_topk_decode -- top-k index-gathered MLA decode over one latent KV head.
 * [NSA] forward_decode: logical top-k indices map to cache slots through the
 * request's token table (transform_index_page_table_decode, page size 1);
 * entries equal to -1 are padding and are skipped (_pad_topk_indices,
 * _forward_aiter). [NSA] _forward_fa3: the cache row is
 * [c_kv (head_dim_v) | k_rope (head_dim_qk - head_dim_v)]; the score is the dot
 * product of q = [q_nope | q_rope] with the whole row; the value is c_kv.
 *   slot_j = req_to_token[req_pool_indices[b], topk_idx[b, j]] (topk_idx != -1)
 *   s_j = softmax_scale * <q[b, h], kv_cache[slot_j]>
 *   out[b, h] = sum_j softmax(s)_j * kv_cache[slot_j, :head_dim_v]
 *
 * q        [batch, num_q_heads, head_dim_qk] bf16
 * kv_cache [num_slots, head_dim_qk] bf16
 * req_to_token [req_to_token_rows, req_to_token_stride] int32
 * topk_idx [batch, topk] int32 logical indices in [0, stride) or -1
 * workspace: device scratch of at least sparse_topk_decode_workspace_size(...)
 *          bytes (may be NULL when that size is 0): one completion counter
 *          per (request, head block) in the counter region, then per-split
 *          partial results; layout and zeroing rule as stated at
 *          PKV_WORKSPACE_COUNTER_BYTES.
 * out      [batch, num_q_heads, head_dim_v] bf16 (out); lse [batch, num_q_heads]
 *          fp32 (out) or NULL.
 * Supported: head_dim_qk 576, head_dim_v 512, num_q_heads a multiple of 32,
 * topk <= 131072 (PKV_EUNSUPPORTED above).
 */
size_t sparse_topk_decode_workspace_size(int32_t batch, int32_t topk, int32_t num_q_heads,
                                         int32_t head_dim_v);

pkv_status_t sparse_topk_decode(const void* q, const void* kv_cache, int64_t num_slots,
                                const int32_t* req_to_token, int64_t req_to_token_rows,
                                int64_t req_to_token_stride, const int32_t* req_pool_indices,
                                const int32_t* topk_idx, int32_t topk, int32_t batch,
                                int32_t num_q_heads, int32_t head_dim_qk, int32_t head_dim_v,
                                float softmax_scale, void* workspace, size_t workspace_bytes,
                                void* out, float* lse, void* stream);

/*
 * sparse_topk_decode_noalloc -- sparse_topk_decode that allocates nothing and
 * takes no workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops or harnesses that forbid it). Its
 * split partials and counters live in a library-owned device array of
 * PKV_SPARSE_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held from the
 * library's load until the process ends; the first call on each GPU looks up
 * that GPU's copy and clears its counters with a kernel on `stream`. Calls on
 * one GPU share the array: calls that overlap in time on one GPU race (order
 * them on one stream). Arguments, results and errors as for
 * sparse_topk_decode, plus PKV_EUNSUPPORTED when the shape needs more than
 * PKV_SPARSE_NOALLOC_SCRATCH_BYTES of workspace
 * (sparse_topk_decode_workspace_size).
 */
#define PKV_SPARSE_NOALLOC_SCRATCH_BYTES (32u << 20)
pkv_status_t sparse_topk_decode_noalloc(const void* q, const void* kv_cache, int64_t num_slots,
                                        const int32_t* req_to_token, int64_t req_to_token_rows,
                                        int64_t req_to_token_stride,
                                        const int32_t* req_pool_indices, const int32_t* topk_idx,
                                        int32_t topk, int32_t batch, int32_t num_q_heads,
                                        int32_t head_dim_qk, int32_t head_dim_v,
                                        float softmax_scale, void* out, float* lse, void* stream);

/*
 * build_dca_decode_tables -- per-request metadata of dual chunk attention
 * decode. [DCA] init_forward_metadata (decode): chunk_len = chunk_size -
 * local_size, c = (L - 1) / chunk_len for L = seq_lens[b] (the cached length
 * including the query token, L >= 1; L = 0 is read as c = 0):
 *   lens_intra = L - c * chunk_len, table_intra row = block_tables row from
 *     page c * chunk_len / page_size;
 *   lens_succ = chunk_len if c >= 1 else 0, table_succ row from page
 *     (c - 1) * chunk_len / page_size (all 0 when c = 0);
 *   lens_inter = max(c - 1, 0) * chunk_len (read through the request's own row);
 *   scaling_factor = max(0.1 * ln(L / original_max_position_embeddings) + 1, 1)
 *     when original_max_position_embeddings > 0, else 1.
 * Table rows hold chunk_len / page_size entries (the widest the pages' tables
 * can be): the pages that hold their stage's keys, in order, then 0.
 *
 * block_tables [batch, bt_stride] int32 page ids (the strided page table)
 * table_intra, table_succ [batch, chunk_len / page_size] int32 (out; table_succ
 *   may be NULL); lens_intra, lens_succ, lens_inter [batch] int32 (out);
 * scaling_factor [batch] fp32 (out) or NULL.
 * Errors: PKV_EINVAL for chunk_len not a multiple of page_size ([DCA]
 * _dual_chunk_flash_attn_decoding rejects it), bad sizes or NULL pointers.
 */
pkv_status_t build_dca_decode_tables(const int32_t* block_tables, int32_t bt_stride,
                                     const int32_t* seq_lens, int32_t batch, int32_t chunk_len,
                                     int32_t page_size, int32_t original_max_position_embeddings,
                                     int32_t* table_intra, int32_t* lens_intra,
                                     int32_t* table_succ, int32_t* lens_succ,
                                     int32_t* lens_inter, float* scaling_factor, void* stream);

/*
 * paged_attn_dca_decode -- dual chunk attention decode as one split-KV pass.
 * [DCA] _dual_chunk_flash_attn_decoding runs three decodes -- q over the
 * query's own chunk (intra), q_succ over the chunk before it (succ), q_inter
 * over all earlier keys (inter) -- and merges them by LSE. Here the key axis
 * is cut into kv_chunk splits as in paged_attn_decode_splitkv (kv_chunk
 * divides chunk_len, so a split lies inside one chunk) and each split scores
 * its keys with the query of the stage its chunk belongs to; merge_state of
 * the partials gives the three-stage result. With q_scale non-NULL the
 * queries of request b are multiplied by q_scale[b] and rounded back to the
 * query dtype first (the pages' scaling_factor; see build_dca_decode_tables).
 *
 * q, q_succ, q_inter [batch, num_q_heads, head_dim] dtype; other arguments,
 * outputs, dtypes and errors as for paged_attn_decode_splitkv, plus
 * PKV_EINVAL for chunk_len < 1 or not a multiple of kv_chunk (kv_chunk > 0).
 */
pkv_status_t paged_attn_dca_decode(const void* q, const void* q_succ, const void* q_inter,
                                   int32_t dtype, const void* k_cache, const void* v_cache,
                                   int64_t num_pages, const int32_t* page_table,
                                   int32_t pt_stride, const int32_t* kv_lens, int32_t batch,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t page_size, float softmax_scale, int32_t chunk_len,
                                   const float* q_scale, int32_t kv_chunk, int32_t num_splits,
                                   float* o_partial, float* lse_partial, void* out, float* lse,
                                   void* stream);

/*
 * build_cascade_expand_table -- key lists of cascade attention's expand pass.
 * [FA] init_forward_metadata, target verify with topk > 1 ("create expand page
 * table"). Request b has L_b = seq_lens[b] committed tokens and n = num_draft
 * draft tokens at positions L_b .. L_b + n - 1 of its req_to_token row
 * r = req_pool_indices[b]. custom_mask is flat, one byte per entry (0 = hidden):
 * request blocks in order, each n rows of L_b + n entries; row i says which
 * positions draft i may see. Row b*n + i of the output lists the slots
 * req_to_token[r, L_b + j] of the drafts j that row i sees, in increasing j,
 * then the hidden ones, also in increasing j; expand_lens[b*n + i] is the
 * count seen, cu_expand_lens (if non-NULL) its zero-led prefix sum.
 *
 * custom_mask    [mask_len] uint8, mask_len = sum_b n * (L_b + n)
 * req_to_token   [req_to_token_rows, req_to_token_stride] int32 (L_b + n <= stride)
 * expand_table   [batch * n, n] int32 (out); expand_lens [batch * n] int32 (out);
 * cu_expand_lens [batch * n + 1] int32 (out) or NULL.
 * Supported: 1 <= num_draft <= 256. Errors: PKV_EINVAL for NULL pointers
 * (batch > 0) or bad sizes; batch == 0 enqueues nothing. Indices read from
 * device memory are clamped into their arrays.
 */
pkv_status_t build_cascade_expand_table(const uint8_t* custom_mask, int64_t mask_len,
                                        const int32_t* req_to_token, int64_t req_to_token_rows,
                                        int64_t req_to_token_stride,
                                        const int32_t* req_pool_indices, const int32_t* seq_lens,
                                        int32_t batch, int32_t num_draft, int32_t* expand_table,
                                        int32_t* expand_lens, int32_t* cu_expand_lens,
                                        void* stream);

/*
 * paged_attn_expand_merge -- cascade attention's expand pass and merge.
 * [FA] forward_extend / forward_decode with use_cascade_attn: every q row is
 * its own one-token request whose keys are the slots
 * expand_table[row, :expand_lens[row]] of the cache viewed with page size 1
 * (non-causal), and its (O, LSE) is merged into the prefix pass's state with
 * merge_state_v2's combine:
 *   m = max(LSE_a, LSE_b); w = exp(LSE - m);
 *   O = (w_a O_a + w_b O_b) / (w_a + w_b); LSE = m + ln(w_a + w_b)
 * (both -inf: O = 0, LSE = -inf; a row with no keys leaves the state as is).
 *
 * q        [n_rows, num_q_heads, head_dim] bf16
 * k_cache, v_cache  the cache as [num_slots, num_kv_heads, head_dim] bf16
 * expand_table [n_rows, expand_stride] int32 slots; expand_lens [n_rows] int32
 * out      [n_rows, num_q_heads, head_dim] bf16, in: prefix-pass O, out: merged O
 * lse      [n_rows, num_q_heads] fp32, in: prefix-pass LSE, out: merged LSE
 * Supported: head_dim 64 or 128, Hq % Hkv == 0, Hq / Hkv <= 16.
 */
pkv_status_t paged_attn_expand_merge(const void* q, int32_t dtype, const void* k_cache,
                                     const void* v_cache, int64_t num_slots,
                                     const int32_t* expand_table, int32_t expand_stride,
                                     const int32_t* expand_lens, int32_t n_rows,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     float softmax_scale, void* out, float* lse, void* stream);

/*
 * paged_attn_cascade -- cascade attention in one call: the prefix pass, then
 * the expand pass with its merge ([FA] forward_extend / forward_decode with
 * use_cascade_attn). The prefix pass computes what paged_attn_varlen_prefill
 * with causal = 0 does: the rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) of
 * request b see all kv_lens[b] committed keys through page_table (for
 * draft-tree verification, cu_seqlens_q steps by n and kv_lens are the
 * committed lengths); then the expand pass over the total_q rows merges each
 * row's expand keys (slots in expand_table, the cache viewed with page size
 * 1) into its result, as paged_attn_expand_merge does. When
 * (num_q_heads / num_kv_heads) * max_seqlen_q <= 32 (bf16, head_dim 64 or
 * 128) the prefix pass packs each kv head's (head, draft) rows into one
 * 32-row tile and splits the keys itself, its splits' partials going through
 * the workspace and a short merge launch (split order) into out / lse;
 * otherwise it is the prefill kernel. Arguments as for those two calls,
 * except: workspace of at least paged_attn_cascade_workspace_size(...) bytes
 * (0: NULL allowed; layout and zeroing rule as stated at
 * PKV_WORKSPACE_COUNTER_BYTES); max_seqlen_k sizes the key splits (a smaller
 * one than some kv_lens[b] is still correct, only slower); lse is required.
 * Every argument is checked before anything is enqueued; then two kernels (three
 * with a split packed prefix pass) run on the stream.
 */
size_t paged_attn_cascade_workspace_size(int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                                         int32_t max_seqlen_k, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim);
pkv_status_t paged_attn_cascade(const void* q, int32_t dtype, const void* k_cache,
                                const void* v_cache, int64_t num_pages, const int32_t* page_table,
                                int32_t pt_stride, const int32_t* cu_seqlens_q,
                                const int32_t* kv_lens, int32_t batch, int32_t total_q,
                                int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                float softmax_scale, const int32_t* expand_table,
                                int32_t expand_stride, const int32_t* expand_lens,
                                void* workspace, size_t workspace_bytes, void* out, float* lse,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
