// Internal launchers (one per kernel family), called by the C ABI in api.cpp
// after argument validation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {
struct PageTableArgs;
struct DecodeArgs;
struct PrefillArgs;
struct SparseArgs;
struct CascadeExpandArgs;
struct ExpandMergeArgs;
struct DraftPrefixArgs;
struct DcaTableArgs;
}  // namespace pkv

namespace pkv_launch {
hipError_t page_table(const pkv::PageTableArgs& a, hipStream_t stream);
hipError_t merge_state(const float* o_parts, const float* lse_parts, int num_parts, int64_t rows,
                       int dv, void* out, int out_dtype, float* lse_out, hipStream_t stream);
hipError_t decode_splitkv(const pkv::DecodeArgs& a, int dtype, int head_dim, hipStream_t stream);
// kv-head groups per request when the decode runs the bf16 group kernel (the
// one that can merge its splits itself), else 0
int decode_groups(const pkv::DecodeArgs& a, int dtype, int head_dim);
hipError_t prefill(const pkv::PrefillArgs& a, int head_dim, hipStream_t stream);
hipError_t kv_append(const void* k_new, const void* v_new, const int32_t* loc, int32_t n,
                     int64_t row_bytes, void* k_cache, void* v_cache, int64_t num_slots,
                     hipStream_t stream);
size_t sparse_workspace_bytes(int batch, int topk, int num_q_heads, int head_dim_v);
// completion counters a split sparse launch uses (0 when it does not split)
int64_t sparse_counters(int batch, int topk, int num_q_heads);
hipError_t sparse_topk(const pkv::SparseArgs& a, hipStream_t stream);
// sparse_topk on the library's per-device scratch array instead of a caller
// workspace (when `split`, i.e. the shape needs one); allocates nothing
hipError_t sparse_topk_noalloc(const pkv::SparseArgs& a, bool split, hipStream_t stream);
hipError_t cascade_expand(const pkv::CascadeExpandArgs& a, hipStream_t stream);
hipError_t expand_merge(const pkv::ExpandMergeArgs& a, int head_dim, hipStream_t stream);
// kv heads per workgroup of the packed draft prefix pass (4, 2 or 1), or 0
// where it does not apply (then the prefill kernel runs the prefix pass)
int draft_prefix_heads(int dtype, int head_dim, int num_q_heads, int num_kv_heads,
                       int max_seqlen_q);
hipError_t draft_prefix(const pkv::DraftPrefixArgs& a, int head_dim, hipStream_t stream);
hipError_t dca_tables(const pkv::DcaTableArgs& a, hipStream_t stream);
}  // namespace pkv_launch
