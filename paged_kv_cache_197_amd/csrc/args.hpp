// Kernel argument blocks shared by the launchers and the C ABI (plain data).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pkv {

struct PageTableArgs {
  const int32_t* r2t;
  int64_t rows, stride;
  const int32_t* rpi;
  const int32_t* seq_lens;
  const int32_t* prefill_lens;  // nullptr: strided mode
  int32_t window, batch, page_size, width;
  int32_t* page_table;
  int32_t* kv_lens;
  int32_t* cu_seqlens_k;        // may be nullptr
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* pt;
  int32_t pt_stride;
  const int32_t* kv_lens;
  int32_t batch, hq, hkv, page_size;
  int64_t num_pages;
  float scale_log2;   // softmax_scale * log2(e)
  int32_t chunk;      // tokens per split (> 0)
  int32_t num_splits;
  float* o_part;      // [S, B, Hq, D] (num_splits > 1)
  float* lse_part;    // [S, B, Hq]
  void* out;          // [B, Hq, D] dtype (num_splits == 1)
  float* lse;         // [B, Hq] or nullptr
  int32_t window_left;   // >= 0: sliding window (W, 0); else none
  int32_t attn_chunk;    // > 0: chunked local attention; else none
  // dual chunk attention: with dca_chunk > 0 the keys of the query's own
  // chunk ((L - 1) / dca_chunk) are scored with q, the chunk before it with
  // q_succ, earlier ones with q_inter (a split lies inside one chunk)
  const void* q_succ;
  const void* q_inter;
  int32_t dca_chunk;
  const float* q_scale;   // [B] factors applied to the queries (rounded back), or null
  // merged decode (num_splits > 1): completion counters, one per (request,
  // kv-head group), in a zeroed workspace; the last non-empty split of each
  // merges o_part / lse_part into out / lse. Null: partials only.
  int* counters;
  // > 0 (merged decode, bf16 kv-head groups): the visible keys of the batch
  // are cut into this many equal ranges per group instead of fixed splits;
  // partial rows [units + batch, Hq] in o_part / lse_part
  int32_t units;
};

// Query a split scores its keys with: q, or under dual chunk attention the
// query of the stage its chunk belongs to. L >= 1 (the split is not empty).
__device__ inline const void* split_query(const DecodeArgs& a, int split_start, int L) {
  if (a.dca_chunk <= 0) return a.q;
  const int c = (L - 1) / a.dca_chunk;
  const int ci = split_start / a.dca_chunk;
  return ci >= c ? a.q : (ci == c - 1 ? a.q_succ : a.q_inter);
}

// First key a query at absolute position pos may see: pos - W for a sliding
// window (W, 0) (inclusive on both sides), the start of pos's aligned block
// for chunked local attention, else 0. The last key is pos (causal).
__host__ __device__ inline int key_lower_bound(int pos, int window_left, int attn_chunk) {
  if (window_left >= 0) return pos - window_left > 0 ? pos - window_left : 0;
  if (attn_chunk > 0) return pos / attn_chunk * attn_chunk;
  return 0;
}

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* pt;
  int32_t pt_stride;
  const int32_t* cu_q;
  const int32_t* kv_lens;
  int32_t batch, total_q, max_seqlen_q, hq, hkv, page_size;
  int32_t page_shift;   // log2(page_size) when it is a power of two, else -1
  int64_t num_pages;
  float scale_log2;
  int32_t causal;
  int32_t split_tiles;  // 32-key tiles per key split
  int32_t max_splits;   // splits per q tile (grid extent)
  int32_t qtile_slots;  // >= the q tiles of all requests: ceil(total_q / 32) + batch, capped
  int32_t groups;       // groups of four waves per workgroup (1 or 2)
  void* ws_o;           // [max_splits, qtile_slots, Hq] blocks of 32 rows x D bf16 partial outputs
  float* ws_lse;        // [max_splits, qtile_slots, Hq, 32] partial LSEs (max_splits > 1)
  int32_t* counters;    // [qtile_slots, Hkv, ceil(G / 4)] in the workspace's counter region
  void* out;
  float* lse;
  int32_t window_left;  // >= 0: sliding window (W, 0); else none (causal only)
  int32_t attn_chunk;   // > 0: chunked local attention; else none (causal only)
};

// Prefix pass of draft-tree (cascade) verification on packed query rows:
// request b's M_b = cu_q[b+1] - cu_q[b] rows (G * M_b <= 32) see all kv_lens[b]
// committed keys. The split fields of `d` (chunk, num_splits) and its page
// table and lengths drive the split order; d.q, d.k, d.v are the tensors.
struct DraftPrefixArgs {
  DecodeArgs d;
  const int32_t* cu_q;   // [batch + 1]
  int32_t total_q;
  void* part_o;          // [num_splits, total_q, Hq, D] bf16 (num_splits > 1)
  float* part_lse;       // [num_splits, total_q, Hq]
};

struct SparseArgs {
  const void* q;
  const void* kv;
  int64_t num_slots;
  const int32_t* r2t;
  int64_t r2t_rows, r2t_stride;
  const int32_t* rpi;
  const int32_t* topk_idx;
  int32_t topk, batch, hq, dqk, dv;
  float scale_log2;
  void* workspace;
  size_t workspace_bytes;
  void* out;
  float* lse;
};

// Metadata of dual chunk attention decode (per request).
struct DcaTableArgs {
  const int32_t* block_tables;   // [batch, bt_stride] page ids
  int32_t bt_stride;
  const int32_t* seq_lens;
  int32_t batch, chunk_len, page_size, width;   // width = chunk_len / page_size
  int32_t original_max_position_embeddings;
  int32_t* table_intra;   // [batch, width]
  int32_t* table_succ;    // [batch, width] or null
  int32_t* lens_intra;
  int32_t* lens_succ;
  int32_t* lens_inter;
  float* scaling_factor;  // [batch] or null
};

// Expand-pass key lists of cascade attention (one row per draft token).
struct CascadeExpandArgs {
  const uint8_t* mask;   // flat custom mask: per request n rows of L_b + n entries
  int64_t mask_len;
  const int32_t* req_to_token;
  int64_t r2t_rows, r2t_stride;
  const int32_t* req_pool_indices;
  const int32_t* seq_lens;   // committed tokens L_b
  int32_t batch, num_draft;
  int32_t* table;            // [batch * n, n] slots
  int32_t* lens;             // [batch * n]
  int32_t* cu;               // [batch * n + 1] or null
};

// Expand pass + merge: each q row over its listed slots, merged into out / lse.
struct ExpandMergeArgs {
  const void* q;   // [rows, hq, D] bf16
  const void* k;   // cache viewed as [num_slots, hkv, D] bf16
  const void* v;
  int64_t num_slots;
  const int32_t* table;   // [rows, stride] slots
  const int32_t* lens;    // [rows]
  int32_t stride, rows, hq, hkv;
  float scale_log2;
  void* out;    // [rows, hq, D] bf16, in: prefix-pass O, out: merged O
  float* lse;   // [rows, hq], in: prefix-pass LSE, out: merged LSE
};

}  // namespace pkv
