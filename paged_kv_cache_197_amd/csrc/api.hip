// C ABI of libpkv.so (declared in include/pkv.h): host-side argument checks,
// then one launcher call per entry point. No allocation, no synchronisation.
#include <math.h>

#include <algorithm>
#include <stdarg.h>
#include <stdio.h>

#include "args.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace pkv_host {

static thread_local char g_last_error[512] = "";

pkv_status_t fail(pkv_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

static pkv_status_t ok() {
  g_last_error[0] = '\0';
  return PKV_OK;
}

static pkv_status_t from_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PKV_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// log2(v) when v is a power of two, else -1
static int32_t log2_if_pow2(int32_t v) {
  if (v <= 0 || (v & (v - 1)) != 0) return -1;
  int32_t k = 0;
  while ((1 << k) != v) ++k;
  return k;
}

// softmax_scale must be finite and positive: the kernels keep their running
// maxima in raw score units and apply the scale inside the exponent, which
// orders scores correctly only for a positive scale
static bool scale_ok(float softmax_scale) {
  return softmax_scale > 0.f && softmax_scale <= 3.402823466e38f;
}

static float scale_log2(float softmax_scale) {
  return static_cast<float>(static_cast<double>(softmax_scale) * 1.4426950408889634);
}

// Key-split plan of paged_attn_varlen_prefill. A workgroup handles
// one (q tile, kv head); when there are fewer such units than half the CUs,
// the 32-key tiles a q tile sees are cut into splits of split_tiles tiles so
// that about kPrefillWorkgroups workgroups run, never below kMinSplitTiles
// tiles per split. The workspace holds the split counters (in its fixed
// counter region, zero between calls), then the partial LSEs and outputs.
// Largest draft count per request of the cascade expand table (a wave holds a
// request's draft columns, four per lane).
constexpr int32_t kMaxDraft = 256;

constexpr int64_t kPrefillWorkgroups = 256;
constexpr int64_t kMinSplitTiles = 4;
// (q tile, kv head) units from which workgroups of one group of four waves
// (two per CU) are used: at least two rounds of the 512 workgroup slots, so
// that the longer per-workgroup chains (no key halving inside) are hidden by
// the second workgroup per CU; below it two groups per workgroup halve them.
constexpr int64_t kOneGroupUnits = 1024;

struct PrefillPlan {
  int32_t split_tiles, max_splits, qtile_slots, groups;
  int64_t counters;
  size_t counter_bytes, lse_bytes, o_bytes, bytes;
};

static size_t round_up256(size_t v) { return (v + 255) / 256 * 256; }

static PrefillPlan prefill_plan(int64_t batch, int64_t total_q, int64_t max_seqlen_q,
                                int64_t max_seqlen_k, int64_t hq, int64_t hkv, int64_t head_dim) {
  PrefillPlan p;
  const int64_t n_kt = max_seqlen_k > 0 ? (max_seqlen_k + 31) / 32 : 1;
  // q tiles of all requests: at most ceil(total_q / 32) + batch (and at most
  // batch * ceil(max_seqlen_q / 32) when max_seqlen_q bounds every request)
  const int64_t qtiles =
      std::min<int64_t>((total_q + 31) / 32 + batch, batch * ((max_seqlen_q + 31) / 32));
  p.qtile_slots = static_cast<int32_t>(std::min<int64_t>((total_q + 31) / 32 + batch, 1 << 30));
  const int64_t units = std::max<int64_t>(1, qtiles * hkv);
  const int64_t want = (2 * units >= kPrefillWorkgroups)
                           ? 1
                           : std::min<int64_t>(16, kPrefillWorkgroups / units);
  const int64_t tiles = std::max<int64_t>(kMinSplitTiles, (n_kt + want - 1) / want);
  p.split_tiles = static_cast<int32_t>(std::min<int64_t>(tiles, 1 << 30));
  p.max_splits = static_cast<int32_t>((n_kt + p.split_tiles - 1) / p.split_tiles);
  p.counter_bytes = p.lse_bytes = p.o_bytes = p.bytes = 0;
  p.counters = 0;
  p.groups = 2;
  if (p.max_splits <= 1) {
    p.max_splits = 1;
    if (units >= kOneGroupUnits) p.groups = 1;
    return p;
  }
  const int64_t n_hb = (hq / hkv + 3) / 4;
  // counters: one per (q-tile slot, kv head, head block), in the fixed region
  // at the start of the workspace. Splits are planned only below
  // kPrefillWorkgroups / 2 units, which keeps them far below its capacity
  // (at most 2 * 127 slot-heads x 4 head blocks); prefill_prepare checks it.
  p.counters = p.qtile_slots * hkv * n_hb;
  p.counter_bytes = PKV_WORKSPACE_COUNTER_BYTES;
  // one block of 32 rows per (split, q-tile slot, head)
  const size_t blocks = static_cast<size_t>(p.max_splits) * p.qtile_slots * hq;
  p.lse_bytes = round_up256(blocks * 32 * 4);
  p.o_bytes = blocks * 32 * head_dim * 2;   // bf16
  p.bytes = p.counter_bytes + p.lse_bytes + p.o_bytes;
  return p;
}

// Packed draft prefix pass (cascade): key splits of `chunk` keys (a multiple
// of 32, at least kDraftMinChunk) so that the (kv-head group, request, split)
// workgroups number about kDraftWorkgroups (two per CU) when every request
// is max_seqlen_k long; the last split also takes any keys past
// splits * chunk. On the tree-verification batch (64 requests, two kv-head
// groups, lengths up to 16384) a sweep of 256..2048 put 512 first (4 splits:
// 0.70 of HBM for the whole cascade step, 0.66 at 384 and 768, 0.65 at
// 2048): more splits add partials and workgroup start-up, fewer leave CUs
// idle. With more than one split the workspace holds the splits' partials
// after its counter region: o [splits, total_q, Hq, D] bf16, then lse
// [splits, total_q, Hq] fp32, each 256-byte aligned.
constexpr int64_t kDraftWorkgroups = 512;
constexpr int64_t kDraftMinChunk = 256;

struct DraftPlan {
  int32_t chunk, splits;
  size_t o_bytes, bytes;
};

static DraftPlan draft_plan(int64_t batch, int64_t total_q, int64_t max_seqlen_k, int64_t hq,
                            int64_t hkv, int64_t head_dim, int64_t heads_per_wg) {
  DraftPlan p{};
  const int64_t lmax = std::max<int64_t>(max_seqlen_k, 1);
  const int64_t per_split = std::max<int64_t>(1, batch * (hkv / heads_per_wg));
  const int64_t want = std::max<int64_t>(1, (kDraftWorkgroups + per_split - 1) / per_split);
  int64_t chunk = (lmax + want - 1) / want;
  chunk = std::max<int64_t>(kDraftMinChunk, (chunk + 31) / 32 * 32);
  p.chunk = static_cast<int32_t>(std::min<int64_t>(chunk, int64_t{1} << 30));
  p.splits = static_cast<int32_t>((lmax + p.chunk - 1) / p.chunk);
  if (p.splits > 1) {
    const size_t rows = static_cast<size_t>(p.splits) * total_q * hq;
    p.o_bytes = round_up256(rows * head_dim * 2);
    p.bytes = PKV_WORKSPACE_COUNTER_BYTES + p.o_bytes + round_up256(rows * 4);
  }
  return p;
}

}  // namespace pkv_host

using pkv_host::fail;

#define PKV_REQUIRE(cond, code, ...) \
  do {                               \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

// Balanced merged decode: ranges per kv-head group so that groups x ranges
// is one workgroup per CU of a 256-CU device (measured faster than two per CU
// on both the long-context and the windowed batch: fewer partial rows to
// merge, and one workgroup's four-tile loads already cover its CU's share of
// HBM bandwidth), and the most partial rows (ranges + batch, or 8 fixed splits
// x batch where the group kernel does not run) its workspace must hold.
constexpr int kBalancedSlots = 256;
constexpr int kBalancedMaxSplits = 8;
constexpr int64_t kBalancedMaxKeys = int64_t{1} << 24;

// merged decode workspace: counters, then o [parts, Hq, D] fp32, then lse
// [parts, Hq] fp32 with parts = S x B (fixed splits) or 256 + 8 B (balanced,
// num_splits == 0)
static size_t decode_merged_ws_bytes(int64_t batch, int64_t num_q_heads, int64_t head_dim,
                                     int64_t num_splits) {
  if (num_splits == 1 || num_splits < 0 || batch <= 0 || num_q_heads <= 0 || head_dim <= 0)
    return 0;
  const int64_t parts = num_splits == 0 ? kBalancedSlots + kBalancedMaxSplits * batch
                                        : num_splits * batch;
  const size_t rows = static_cast<size_t>(parts * num_q_heads);
  return PKV_WORKSPACE_COUNTER_BYTES + pkv_host::round_up256(rows * head_dim * 4) +
         pkv_host::round_up256(rows * 4);
}

static pkv_status_t decode_impl(const void* q, const void* q_succ, const void* q_inter,
                                int32_t dca_chunk, const float* q_scale, int32_t dtype,
                                const void* k_cache, const void* v_cache, int64_t num_pages,
                                const int32_t* page_table, int32_t pt_stride,
                                const int32_t* kv_lens, int32_t batch, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                float softmax_scale, int32_t window_left, int32_t attn_chunk,
                                int32_t kv_chunk, int32_t num_splits, float* o_partial,
                                float* lse_partial, void* out, float* lse, void* stream,
                                bool merged = false, void* workspace = nullptr,
                                size_t workspace_bytes = 0) {
  PKV_REQUIRE(dtype == PKV_F32 || dtype == PKV_BF16, PKV_EUNSUPPORTED,
              "decode: dtype %d not supported", dtype);
  PKV_REQUIRE(head_dim == 64 || head_dim == 128, PKV_EUNSUPPORTED,
              "decode: head_dim %d not supported (64, 128)", head_dim);
  PKV_REQUIRE(batch >= 0 && num_q_heads >= 1 && num_kv_heads >= 1, PKV_EINVAL,
              "decode: bad sizes batch %d Hq %d Hkv %d", batch, num_q_heads, num_kv_heads);
  PKV_REQUIRE(num_q_heads % num_kv_heads == 0, PKV_EINVAL,
              "decode: num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads,
              num_kv_heads);
  PKV_REQUIRE(num_q_heads / num_kv_heads <= 16, PKV_EUNSUPPORTED,
              "decode: GQA group %d > 16", num_q_heads / num_kv_heads);
  PKV_REQUIRE(page_size >= 1 && pt_stride >= 1 && num_pages >= 1, PKV_EINVAL,
              "decode: page_size %d pt_stride %d num_pages %lld", page_size, pt_stride,
              (long long)num_pages);
  PKV_REQUIRE(window_left >= -1 && attn_chunk >= 0 && !(window_left >= 0 && attn_chunk > 0),
              PKV_EINVAL, "decode: window_left %d / attn_chunk %d (at most one of them)",
              window_left, attn_chunk);
  PKV_REQUIRE(pkv_host::scale_ok(softmax_scale), PKV_EINVAL,
              "decode: softmax_scale %g is not finite and positive", softmax_scale);
  PKV_REQUIRE(kv_chunk >= 0, PKV_EINVAL, "decode: kv_chunk %d < 0", kv_chunk);
  PKV_REQUIRE(kv_chunk % page_size == 0, PKV_EINVAL,
              "decode: kv_chunk %d is not a multiple of page_size %d", kv_chunk, page_size);
  PKV_REQUIRE(kv_chunk % 32 == 0, PKV_EINVAL, "decode: kv_chunk %d is not a multiple of 32",
              kv_chunk);
  // merged decode: kv_chunk 0 with num_splits 0 asks for balanced ranges
  const bool balanced = merged && kv_chunk == 0 && num_splits == 0;
  PKV_REQUIRE(num_splits >= 1 || balanced, PKV_EINVAL, "decode: num_splits %d < 1", num_splits);
  PKV_REQUIRE(kv_chunk > 0 || num_splits <= 1, PKV_EINVAL,
              "decode: kv_chunk 0 (one split) needs num_splits 1, got %d", num_splits);
  PKV_REQUIRE(dca_chunk >= 0, PKV_EINVAL, "decode: chunk_len %d < 0", dca_chunk);
  if (dca_chunk > 0) {
    PKV_REQUIRE(kv_chunk > 0 && dca_chunk % kv_chunk == 0, PKV_EINVAL,
                "decode: chunk_len %d is not a multiple of kv_chunk %d", dca_chunk, kv_chunk);
    PKV_REQUIRE(window_left < 0 && attn_chunk == 0, PKV_EINVAL,
                "decode: dual chunk attention takes no window or local chunks");
  }
  if (batch == 0) return pkv_host::ok();
  PKV_REQUIRE(q && k_cache && v_cache && page_table && kv_lens, PKV_EINVAL,
              "decode: NULL required pointer");
  PKV_REQUIRE(dca_chunk == 0 || (q_succ && q_inter), PKV_EINVAL,
              "decode: dual chunk attention needs q_succ and q_inter");
  if (num_splits == 1 || merged) {
    PKV_REQUIRE(out != nullptr, PKV_EINVAL, "decode: out is NULL");
  } else {
    PKV_REQUIRE(o_partial && lse_partial, PKV_EINVAL,
                "decode: num_splits %d needs o_partial and lse_partial", num_splits);
  }
  const size_t ws_need = decode_merged_ws_bytes(batch, num_q_heads, head_dim, num_splits);
  if (merged && ws_need > 0) {
    PKV_REQUIRE(workspace != nullptr && workspace_bytes >= ws_need, PKV_EINVAL,
                "decode: workspace of %zu bytes given, %zu needed", workspace_bytes, ws_need);
  }
  const int64_t grid = static_cast<int64_t>(num_kv_heads) * batch * max(num_splits, 1);
  PKV_REQUIRE(grid <= 0x7fffffff, PKV_EUNSUPPORTED, "decode: grid too large");
  const int64_t cap = static_cast<int64_t>(pt_stride) * page_size;
  pkv::DecodeArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.pt = page_table;
  a.pt_stride = pt_stride;
  a.kv_lens = kv_lens;
  a.batch = batch;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.page_size = page_size;
  a.num_pages = num_pages;
  a.scale_log2 = pkv_host::scale_log2(softmax_scale);
  // one split: a chunk that covers every representable key position
  a.chunk = kv_chunk > 0 ? kv_chunk
                         : static_cast<int32_t>(((cap < 0x40000000LL ? cap : 0x40000000LL) + 31) /
                                                32 * 32);
  a.num_splits = num_splits;
  a.units = 0;
  a.window_left = window_left;
  a.attn_chunk = attn_chunk;
  a.q_succ = q_succ;
  a.q_inter = q_inter;
  a.dca_chunk = dca_chunk;
  a.q_scale = q_scale;
  a.o_part = o_partial;
  a.lse_part = lse_partial;
  a.out = out;
  a.lse = lse;
  a.counters = nullptr;
  bool merge_after = false;
  if (merged && num_splits != 1) {
    // partials in the workspace after its counter region; the group kernel
    // merges them itself when its counters fit, else merge_state follows
    char* ws = static_cast<char*>(workspace);
    const int64_t parts = balanced ? kBalancedSlots + kBalancedMaxSplits * int64_t{batch}
                                   : int64_t{num_splits} * batch;
    const int64_t rows = parts * num_q_heads;
    a.o_part = reinterpret_cast<float*>(ws + PKV_WORKSPACE_COUNTER_BYTES);
    a.lse_part = reinterpret_cast<float*>(ws + PKV_WORKSPACE_COUNTER_BYTES +
                                          pkv_host::round_up256(static_cast<size_t>(rows) * head_dim * 4));
    const int groups = pkv_launch::decode_groups(a, dtype, head_dim);
    const bool counters_fit = static_cast<int64_t>(batch) * groups * 4 <= PKV_WORKSPACE_COUNTER_BYTES;
    if (balanced && groups > 0 && counters_fit && cap <= kBalancedMaxKeys) {
      a.units = (kBalancedSlots + groups - 1) / groups;
      a.num_splits = 2;   // (not read in this mode; anything but one split)
      a.counters = reinterpret_cast<int*>(ws);
    } else {
      if (balanced) {
        // fixed splits instead: at most eight, on whole pages and tiles
        int64_t unit = page_size;
        while (unit % 32 != 0) unit += page_size;
        const int64_t per = (cap + kBalancedMaxSplits - 1) / kBalancedMaxSplits;
        const int64_t chunk = (per + unit - 1) / unit * unit;
        PKV_REQUIRE(chunk <= 0x7fffffff, PKV_EUNSUPPORTED, "decode: key capacity too large");
        a.chunk = static_cast<int32_t>(chunk);
        a.num_splits = static_cast<int32_t>((cap + chunk - 1) / chunk);
        num_splits = a.num_splits;
      }
      if (a.num_splits == 1) {
        a.out = out;   // one split: written directly
      } else if (groups > 0 && counters_fit) {
        a.counters = reinterpret_cast<int*>(ws);
      } else {
        merge_after = true;
      }
    }
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const pkv_status_t r =
      pkv_host::from_hip(pkv_launch::decode_splitkv(a, dtype, head_dim, st), "decode launch");
  if (r != PKV_OK || !merge_after) return r;
  return pkv_host::from_hip(
      pkv_launch::merge_state(a.o_part, a.lse_part, num_splits,
                              static_cast<int64_t>(batch) * num_q_heads, head_dim, out, dtype,
                              lse, st),
      "merge_state launch");
}

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_EINVAL: return "PKV_EINVAL";
    case PKV_EUNSUPPORTED: return "PKV_EUNSUPPORTED";
    case PKV_ELAUNCH: return "PKV_ELAUNCH";
    default: return "PKV_UNKNOWN";
  }
}

const char* pkv_last_error(void) { return pkv_host::g_last_error; }

pkv_status_t build_page_table(const int32_t* req_to_token, int64_t req_to_token_rows,
                              int64_t req_to_token_stride, const int32_t* req_pool_indices,
                              const int32_t* seq_lens, const int32_t* prefill_lens,
                              int32_t window, int32_t batch, int32_t page_size, int32_t width,
                              int32_t* page_table, int32_t* kv_lens, int32_t* cu_seqlens_k,
                              void* stream) {
  PKV_REQUIRE(batch >= 0, PKV_EINVAL, "build_page_table: batch %d < 0", batch);
  PKV_REQUIRE(width >= 0, PKV_EINVAL, "build_page_table: width %d < 0", width);
  PKV_REQUIRE(page_size >= 1, PKV_EINVAL, "build_page_table: page_size %d < 1", page_size);
  PKV_REQUIRE(width <= 65535 * 256, PKV_EUNSUPPORTED, "build_page_table: width %d too large",
              width);
  if (prefill_lens != nullptr) {
    PKV_REQUIRE(page_size == 1, PKV_EINVAL,
                "build_page_table: the sliding-window table is token-level (page_size 1), got %d",
                page_size);
    PKV_REQUIRE(window >= 0, PKV_EINVAL, "build_page_table: window %d < 0", window);
  }
  if (batch > 0) {
    PKV_REQUIRE(req_to_token && req_pool_indices && seq_lens && page_table && kv_lens,
                PKV_EINVAL, "build_page_table: NULL required pointer");
    PKV_REQUIRE(req_to_token_rows >= 1 && req_to_token_stride >= 1, PKV_EINVAL,
                "build_page_table: req_to_token is %lld x %lld", (long long)req_to_token_rows,
                (long long)req_to_token_stride);
  }
  pkv::PageTableArgs a;
  a.r2t = req_to_token;
  a.rows = req_to_token_rows;
  a.stride = req_to_token_stride;
  a.rpi = req_pool_indices;
  a.seq_lens = seq_lens;
  a.prefill_lens = prefill_lens;
  a.window = window;
  a.batch = batch;
  a.page_size = page_size;
  a.width = width;
  a.page_table = page_table;
  a.kv_lens = kv_lens;
  a.cu_seqlens_k = cu_seqlens_k;
  if (batch == 0 && cu_seqlens_k == nullptr) return pkv_host::ok();
  return pkv_host::from_hip(pkv_launch::page_table(a, static_cast<hipStream_t>(stream)),
                            "build_page_table launch");
}

pkv_status_t merge_state(const float* o_parts, const float* lse_parts, int32_t num_parts,
                         int32_t n_tokens, int32_t num_heads, int32_t head_dim_v, void* out,
                         int32_t out_dtype, float* lse_out, void* stream) {
  PKV_REQUIRE(num_parts >= 1, PKV_EINVAL, "merge_state: num_parts %d < 1", num_parts);
  PKV_REQUIRE(n_tokens >= 0 && num_heads >= 0 && head_dim_v >= 1, PKV_EINVAL,
              "merge_state: bad sizes n_tokens %d num_heads %d head_dim_v %d", n_tokens,
              num_heads, head_dim_v);
  PKV_REQUIRE(out_dtype == PKV_F32 || out_dtype == PKV_BF16, PKV_EUNSUPPORTED,
              "merge_state: out_dtype %d", out_dtype);
  const int64_t rows = static_cast<int64_t>(n_tokens) * num_heads;
  if (rows == 0) return pkv_host::ok();
  PKV_REQUIRE(o_parts && lse_parts && out, PKV_EINVAL, "merge_state: NULL required pointer");
  return pkv_host::from_hip(
      pkv_launch::merge_state(o_parts, lse_parts, num_parts, rows, head_dim_v, out, out_dtype,
                              lse_out, static_cast<hipStream_t>(stream)),
      "merge_state launch");
}

pkv_status_t paged_attn_decode_splitkv(const void* q, int32_t dtype, const void* k_cache,
                                       const void* v_cache, int64_t num_pages,
                                       const int32_t* page_table, int32_t pt_stride,
                                       const int32_t* kv_lens, int32_t batch,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t page_size, float softmax_scale,
                                       int32_t window_left, int32_t attn_chunk,
                                       int32_t kv_chunk, int32_t num_splits, float* o_partial,
                                       float* lse_partial, void* out, float* lse, void* stream) {
  return decode_impl(q, nullptr, nullptr, 0, nullptr, dtype, k_cache, v_cache, num_pages,
                     page_table, pt_stride, kv_lens, batch, num_q_heads, num_kv_heads, head_dim,
                     page_size, softmax_scale, window_left, attn_chunk, kv_chunk, num_splits,
                     o_partial, lse_partial, out, lse, stream);
}

size_t paged_attn_decode_merged_workspace_size(int32_t batch, int32_t num_q_heads,
                                               int32_t head_dim, int32_t num_splits) {
  return decode_merged_ws_bytes(batch, num_q_heads, head_dim, num_splits);
}

pkv_status_t paged_attn_decode_merged(const void* q, int32_t dtype, const void* k_cache,
                                      const void* v_cache, int64_t num_pages,
                                      const int32_t* page_table, int32_t pt_stride,
                                      const int32_t* kv_lens, int32_t batch, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                      float softmax_scale, int32_t window_left, int32_t attn_chunk,
                                      int32_t kv_chunk, int32_t num_splits, void* workspace,
                                      size_t workspace_bytes, void* out, float* lse,
                                      void* stream) {
  return decode_impl(q, nullptr, nullptr, 0, nullptr, dtype, k_cache, v_cache, num_pages,
                     page_table, pt_stride, kv_lens, batch, num_q_heads, num_kv_heads, head_dim,
                     page_size, softmax_scale, window_left, attn_chunk, kv_chunk, num_splits,
                     nullptr, nullptr, out, lse, stream, true, workspace, workspace_bytes);
}

pkv_status_t paged_attn_dca_decode(const void* q, const void* q_succ, const void* q_inter,
                                   int32_t dtype, const void* k_cache, const void* v_cache,
                                   int64_t num_pages, const int32_t* page_table,
                                   int32_t pt_stride, const int32_t* kv_lens, int32_t batch,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t page_size, float softmax_scale, int32_t chunk_len,
                                   const float* q_scale, int32_t kv_chunk, int32_t num_splits,
                                   float* o_partial, float* lse_partial, void* out, float* lse,
                                   void* stream) {
  PKV_REQUIRE(chunk_len >= 1, PKV_EINVAL, "paged_attn_dca_decode: chunk_len %d < 1", chunk_len);
  return decode_impl(q, q_succ, q_inter, chunk_len, q_scale, dtype, k_cache, v_cache, num_pages,
                     page_table, pt_stride, kv_lens, batch, num_q_heads, num_kv_heads, head_dim,
                     page_size, softmax_scale, -1, 0, kv_chunk, num_splits, o_partial,
                     lse_partial, out, lse, stream);
}

size_t paged_attn_varlen_prefill_workspace_size(int32_t batch, int32_t total_q,
                                                int32_t max_seqlen_q, int32_t max_seqlen_k,
                                                int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t head_dim) {
  if (batch <= 0 || total_q <= 0 || max_seqlen_q <= 0 || max_seqlen_k < 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || head_dim <= 0)
    return 0;
  return pkv_host::prefill_plan(batch, total_q, max_seqlen_q, max_seqlen_k, num_q_heads,
                                num_kv_heads, head_dim)
      .bytes;
}

}  // extern "C"

// Validation and argument packing shared by the prefill entry points; sets
// *nothing when there is no work (nothing to launch).
static pkv_status_t prefill_prepare(const void* q, int32_t dtype, const void* k_cache,
                                    const void* v_cache, int64_t num_pages,
                                    const int32_t* page_table, int32_t pt_stride,
                                    const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                                    int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                                    int32_t max_seqlen_k, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                    float softmax_scale, int32_t causal, int32_t window_left,
                                    int32_t attn_chunk, void* workspace,
                                    size_t workspace_bytes, void* out, float* lse,
                                    pkv::PrefillArgs& a, bool* nothing,
                                    bool plan_workspace = true) {
  *nothing = false;
  PKV_REQUIRE(dtype == PKV_BF16, PKV_EUNSUPPORTED, "prefill: dtype %d not supported (bf16)",
              dtype);
  PKV_REQUIRE(head_dim == 64 || head_dim == 128, PKV_EUNSUPPORTED,
              "prefill: head_dim %d not supported (64, 128)", head_dim);
  PKV_REQUIRE(batch >= 0 && total_q >= 0 && max_seqlen_q >= 0 && max_seqlen_k >= 0 &&
                  num_q_heads >= 1 && num_kv_heads >= 1,
              PKV_EINVAL, "prefill: bad sizes");
  PKV_REQUIRE(num_q_heads % num_kv_heads == 0, PKV_EINVAL,
              "prefill: num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads,
              num_kv_heads);
  PKV_REQUIRE(num_q_heads / num_kv_heads <= 16, PKV_EUNSUPPORTED, "prefill: GQA group %d > 16",
              num_q_heads / num_kv_heads);
  PKV_REQUIRE(page_size >= 1 && pt_stride >= 1 && num_pages >= 1, PKV_EINVAL,
              "prefill: page_size %d pt_stride %d num_pages %lld", page_size, pt_stride,
              (long long)num_pages);
  PKV_REQUIRE(num_pages * page_size <= 0x7fffffffLL, PKV_EUNSUPPORTED,
              "prefill: a cache of %lld slots (more than 2^31)",
              (long long)(num_pages * page_size));
  PKV_REQUIRE(causal == 0 || causal == 1, PKV_EINVAL, "prefill: causal %d", causal);
  PKV_REQUIRE(window_left >= -1 && attn_chunk >= 0 && !(window_left >= 0 && attn_chunk > 0),
              PKV_EINVAL, "prefill: window_left %d / attn_chunk %d (at most one of them)",
              window_left, attn_chunk);
  PKV_REQUIRE(causal == 1 || (window_left < 0 && attn_chunk == 0), PKV_EINVAL,
              "prefill: a sliding window or local chunks need causal rows");
  PKV_REQUIRE(max_seqlen_q <= total_q, PKV_EINVAL, "prefill: max_seqlen_q %d > total_q %d",
              max_seqlen_q, total_q);
  PKV_REQUIRE(pkv_host::scale_ok(softmax_scale), PKV_EINVAL,
              "prefill: softmax_scale %g is not finite and positive", softmax_scale);
  if (batch == 0 || total_q == 0 || max_seqlen_q == 0) {
    *nothing = true;
    return pkv_host::ok();
  }
  PKV_REQUIRE(q && k_cache && v_cache && page_table && cu_seqlens_q && kv_lens && out,
              PKV_EINVAL, "prefill: NULL required pointer");
  const pkv_host::PrefillPlan plan =
      plan_workspace ? pkv_host::prefill_plan(batch, total_q, max_seqlen_q, max_seqlen_k,
                                              num_q_heads, num_kv_heads, head_dim)
                     : pkv_host::PrefillPlan{};
  PKV_REQUIRE(plan.counters * 4 <= PKV_WORKSPACE_COUNTER_BYTES, PKV_EUNSUPPORTED,
              "prefill: %lld split counters exceed the workspace's counter region",
              (long long)plan.counters);
  PKV_REQUIRE(plan.bytes == 0 || (workspace != nullptr && workspace_bytes >= plan.bytes),
              PKV_EINVAL, "prefill: workspace of %zu bytes, need %zu", workspace_bytes,
              plan.bytes);
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.pt = page_table;
  a.pt_stride = pt_stride;
  a.cu_q = cu_seqlens_q;
  a.kv_lens = kv_lens;
  a.batch = batch;
  a.total_q = total_q;
  a.max_seqlen_q = max_seqlen_q;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.page_size = page_size;
  a.page_shift = pkv_host::log2_if_pow2(page_size);
  a.num_pages = num_pages;
  a.scale_log2 = pkv_host::scale_log2(softmax_scale);
  a.causal = causal;
  a.split_tiles = plan.split_tiles;
  a.max_splits = plan.max_splits;
  a.qtile_slots = plan.qtile_slots;
  a.groups = plan.groups;
  char* ws = static_cast<char*>(workspace);
  a.counters = plan.bytes ? reinterpret_cast<int32_t*>(ws) : nullptr;
  a.ws_lse = plan.bytes ? reinterpret_cast<float*>(ws + plan.counter_bytes) : nullptr;
  a.ws_o = plan.bytes ? static_cast<void*>(ws + plan.counter_bytes + plan.lse_bytes)
                      : nullptr;
  a.out = out;
  a.lse = lse;
  a.window_left = window_left;
  a.attn_chunk = attn_chunk;
  return pkv_host::ok();
}

extern "C" {

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
                                       void* stream) {
  pkv::PrefillArgs a;
  bool nothing = false;
  const pkv_status_t st = prefill_prepare(
      q, dtype, k_cache, v_cache, num_pages, page_table, pt_stride, cu_seqlens_q, kv_lens, batch,
      total_q, max_seqlen_q, max_seqlen_k, num_q_heads, num_kv_heads, head_dim, page_size,
      softmax_scale, causal, window_left, attn_chunk, workspace, workspace_bytes, out, lse, a,
      &nothing);
  if (st != PKV_OK || nothing) return st;
  return pkv_host::from_hip(pkv_launch::prefill(a, head_dim, static_cast<hipStream_t>(stream)),
                            "prefill launch");
}

// checks shared by the append entry points; row_bytes = Hkv * D * element size
static pkv_status_t append_check(const char* who, const void* k_new, const void* v_new,
                                 int32_t dtype, const int32_t* out_cache_loc, int32_t n_tokens,
                                 int32_t num_kv_heads, int32_t head_dim, void* k_cache,
                                 void* v_cache, int64_t num_slots, int64_t* row_bytes) {
  PKV_REQUIRE(dtype == PKV_BF16 || dtype == PKV_F32, PKV_EUNSUPPORTED, "%s: dtype %d", who,
              dtype);
  PKV_REQUIRE(n_tokens >= 0 && num_kv_heads >= 1 && head_dim >= 1 && num_slots >= 1,
              PKV_EINVAL, "%s: bad sizes", who);
  const int64_t es = dtype == PKV_BF16 ? 2 : 4;
  *row_bytes = static_cast<int64_t>(num_kv_heads) * head_dim * es;
  PKV_REQUIRE((static_cast<int64_t>(head_dim) * es) % 16 == 0, PKV_EUNSUPPORTED,
              "%s: head_dim %d x %lld bytes not a multiple of 16", who, head_dim, (long long)es);
  PKV_REQUIRE(n_tokens == 0 || (k_new && v_new && out_cache_loc && k_cache && v_cache),
              PKV_EINVAL, "%s: NULL required pointer", who);
  return pkv_host::ok();
}

pkv_status_t paged_kv_append(const void* k_new, const void* v_new, int32_t dtype,
                             const int32_t* out_cache_loc, int32_t n_tokens, int32_t num_kv_heads,
                             int32_t head_dim, void* k_cache, void* v_cache, int64_t num_slots,
                             void* stream) {
  int64_t row_bytes = 0;
  const pkv_status_t st = append_check("paged_kv_append", k_new, v_new, dtype, out_cache_loc,
                                       n_tokens, num_kv_heads, head_dim, k_cache, v_cache,
                                       num_slots, &row_bytes);
  if (st != PKV_OK || n_tokens == 0) return st;
  return pkv_host::from_hip(pkv_launch::kv_append(k_new, v_new, out_cache_loc, n_tokens, row_bytes,
                                                  k_cache, v_cache, num_slots,
                                                  static_cast<hipStream_t>(stream)),
                            "paged_kv_append launch");
}

pkv_status_t paged_attn_varlen_prefill_append(
    const void* q, int32_t dtype, void* k_cache, void* v_cache, int64_t num_pages,
    const int32_t* page_table, int32_t pt_stride, const int32_t* cu_seqlens_q,
    const int32_t* kv_lens, int32_t batch, int32_t total_q, int32_t max_seqlen_q,
    int32_t max_seqlen_k, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t page_size, float softmax_scale, int32_t causal, int32_t window_left,
    int32_t attn_chunk, const void* k_new, const void* v_new, const int32_t* out_cache_loc,
    void* workspace, size_t workspace_bytes, void* out, float* lse, void* stream) {
  // every check before anything is enqueued: the cache is written only when
  // the attention will run too
  pkv::PrefillArgs a;
  bool nothing = false;
  pkv_status_t st = prefill_prepare(
      q, dtype, k_cache, v_cache, num_pages, page_table, pt_stride, cu_seqlens_q, kv_lens, batch,
      total_q, max_seqlen_q, max_seqlen_k, num_q_heads, num_kv_heads, head_dim, page_size,
      softmax_scale, causal, window_left, attn_chunk, workspace, workspace_bytes, out, lse, a,
      &nothing);
  if (st != PKV_OK) return st;
  int64_t row_bytes = 0;
  st = append_check("paged_attn_varlen_prefill_append", k_new, v_new, dtype, out_cache_loc,
                    total_q, num_kv_heads, head_dim, k_cache, v_cache, num_pages * page_size,
                    &row_bytes);
  if (st != PKV_OK || total_q == 0) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = pkv_host::from_hip(pkv_launch::kv_append(k_new, v_new, out_cache_loc, total_q, row_bytes,
                                                k_cache, v_cache, num_pages * page_size, s),
                          "paged_attn_varlen_prefill_append: append launch");
  if (st != PKV_OK || nothing) return st;
  return pkv_host::from_hip(pkv_launch::prefill(a, head_dim, s),
                            "paged_attn_varlen_prefill_append: prefill launch");
}

size_t sparse_topk_decode_workspace_size(int32_t batch, int32_t topk, int32_t num_q_heads,
                                         int32_t head_dim_v) {
  if (batch <= 0 || topk <= 0 || num_q_heads <= 0 || head_dim_v <= 0) return 0;
  return pkv_launch::sparse_workspace_bytes(batch, topk, num_q_heads, head_dim_v);
}

}  // extern "C"

// Checks and argument packing shared by the sparse entry points (workspace
// fields left for the caller); sets *nothing when there is no work.
static pkv_status_t sparse_prepare(const char* who, const void* q, const void* kv_cache,
                                   int64_t num_slots, const int32_t* req_to_token,
                                   int64_t req_to_token_rows, int64_t req_to_token_stride,
                                   const int32_t* req_pool_indices, const int32_t* topk_idx,
                                   int32_t topk, int32_t batch, int32_t num_q_heads,
                                   int32_t head_dim_qk, int32_t head_dim_v, float softmax_scale,
                                   void* out, float* lse, pkv::SparseArgs& a, bool* nothing) {
  *nothing = false;
  PKV_REQUIRE(head_dim_qk == 576 && head_dim_v == 512, PKV_EUNSUPPORTED,
              "%s: head dims %d/%d not supported (576/512)", who, head_dim_qk, head_dim_v);
  PKV_REQUIRE(batch >= 0 && topk >= 0 && num_q_heads >= 1, PKV_EINVAL,
              "%s: bad sizes batch %d topk %d heads %d", who, batch, topk, num_q_heads);
  PKV_REQUIRE(num_q_heads % 32 == 0, PKV_EUNSUPPORTED,
              "%s: num_q_heads %d not a multiple of 32", who, num_q_heads);
  PKV_REQUIRE(topk <= 131072, PKV_EUNSUPPORTED,
              "%s: topk %d above 131072 (64 key splits of 2048)", who, topk);
  PKV_REQUIRE(pkv_host::scale_ok(softmax_scale), PKV_EINVAL,
              "%s: softmax_scale %g is not finite and positive", who, softmax_scale);
  if (batch == 0) {
    *nothing = true;
    return pkv_host::ok();
  }
  PKV_REQUIRE(q && kv_cache && req_to_token && req_pool_indices && out, PKV_EINVAL,
              "%s: NULL required pointer", who);
  PKV_REQUIRE(topk == 0 || topk_idx != nullptr, PKV_EINVAL, "%s: NULL topk_idx", who);
  PKV_REQUIRE(num_slots >= 1 && req_to_token_rows >= 1 && req_to_token_stride >= 1, PKV_EINVAL,
              "%s: empty cache or token table", who);
  PKV_REQUIRE(pkv_launch::sparse_counters(batch, topk, num_q_heads) * 4 <=
                  PKV_WORKSPACE_COUNTER_BYTES,
              PKV_EUNSUPPORTED,
              "%s: batch %d needs more split counters than the workspace's counter region holds",
              who, batch);
  a.q = q;
  a.kv = kv_cache;
  a.num_slots = num_slots;
  a.r2t = req_to_token;
  a.r2t_rows = req_to_token_rows;
  a.r2t_stride = req_to_token_stride;
  a.rpi = req_pool_indices;
  a.topk_idx = topk_idx;
  a.topk = topk;
  a.batch = batch;
  a.hq = num_q_heads;
  a.dqk = head_dim_qk;
  a.dv = head_dim_v;
  a.scale_log2 = pkv_host::scale_log2(softmax_scale);
  a.workspace = nullptr;
  a.workspace_bytes = 0;
  a.out = out;
  a.lse = lse;
  return pkv_host::ok();
}

extern "C" {

pkv_status_t sparse_topk_decode(const void* q, const void* kv_cache, int64_t num_slots,
                                const int32_t* req_to_token, int64_t req_to_token_rows,
                                int64_t req_to_token_stride, const int32_t* req_pool_indices,
                                const int32_t* topk_idx, int32_t topk, int32_t batch,
                                int32_t num_q_heads, int32_t head_dim_qk, int32_t head_dim_v,
                                float softmax_scale, void* workspace, size_t workspace_bytes,
                                void* out, float* lse, void* stream) {
  pkv::SparseArgs a;
  bool nothing = false;
  const pkv_status_t st = sparse_prepare(
      "sparse_topk_decode", q, kv_cache, num_slots, req_to_token, req_to_token_rows,
      req_to_token_stride, req_pool_indices, topk_idx, topk, batch, num_q_heads, head_dim_qk,
      head_dim_v, softmax_scale, out, lse, a, &nothing);
  if (st != PKV_OK || nothing) return st;
  const size_t need = sparse_topk_decode_workspace_size(batch, topk, num_q_heads, head_dim_v);
  PKV_REQUIRE(workspace_bytes >= need && (need == 0 || workspace != nullptr), PKV_EINVAL,
              "sparse_topk_decode: workspace of %zu bytes, need %zu", workspace_bytes, need);
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  return pkv_host::from_hip(pkv_launch::sparse_topk(a, static_cast<hipStream_t>(stream)),
                            "sparse_topk_decode launch");
}

pkv_status_t sparse_topk_decode_noalloc(const void* q, const void* kv_cache, int64_t num_slots,
                                        const int32_t* req_to_token, int64_t req_to_token_rows,
                                        int64_t req_to_token_stride,
                                        const int32_t* req_pool_indices, const int32_t* topk_idx,
                                        int32_t topk, int32_t batch, int32_t num_q_heads,
                                        int32_t head_dim_qk, int32_t head_dim_v,
                                        float softmax_scale, void* out, float* lse, void* stream) {
  pkv::SparseArgs a;
  bool nothing = false;
  const pkv_status_t st = sparse_prepare(
      "sparse_topk_decode_noalloc", q, kv_cache, num_slots, req_to_token, req_to_token_rows,
      req_to_token_stride, req_pool_indices, topk_idx, topk, batch, num_q_heads, head_dim_qk,
      head_dim_v, softmax_scale, out, lse, a, &nothing);
  if (st != PKV_OK || nothing) return st;
  const size_t need = sparse_topk_decode_workspace_size(batch, topk, num_q_heads, head_dim_v);
  PKV_REQUIRE(need <= PKV_SPARSE_NOALLOC_SCRATCH_BYTES, PKV_EUNSUPPORTED,
              "sparse_topk_decode_noalloc: this shape needs %zu bytes of scratch, the library "
              "holds %zu per GPU (use sparse_topk_decode with a workspace)",
              need, (size_t)PKV_SPARSE_NOALLOC_SCRATCH_BYTES);
  return pkv_host::from_hip(
      pkv_launch::sparse_topk_noalloc(a, need > 0, static_cast<hipStream_t>(stream)),
      "sparse_topk_decode_noalloc launch");
}

pkv_status_t build_dca_decode_tables(const int32_t* block_tables, int32_t bt_stride,
                                     const int32_t* seq_lens, int32_t batch, int32_t chunk_len,
                                     int32_t page_size, int32_t original_max_position_embeddings,
                                     int32_t* table_intra, int32_t* lens_intra,
                                     int32_t* table_succ, int32_t* lens_succ,
                                     int32_t* lens_inter, float* scaling_factor, void* stream) {
  PKV_REQUIRE(batch >= 0 && bt_stride >= 1 && page_size >= 1 && chunk_len >= 1, PKV_EINVAL,
              "build_dca_decode_tables: bad sizes");
  PKV_REQUIRE(chunk_len % page_size == 0, PKV_EINVAL,
              "build_dca_decode_tables: chunk_len %d is not a multiple of page_size %d",
              chunk_len, page_size);
  PKV_REQUIRE(original_max_position_embeddings >= 0, PKV_EINVAL,
              "build_dca_decode_tables: original_max_position_embeddings %d < 0",
              original_max_position_embeddings);
  if (batch == 0) return pkv_host::ok();
  PKV_REQUIRE(block_tables && seq_lens && table_intra && lens_intra && lens_succ && lens_inter,
              PKV_EINVAL, "build_dca_decode_tables: NULL required pointer");
  pkv::DcaTableArgs a;
  a.block_tables = block_tables;
  a.bt_stride = bt_stride;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.chunk_len = chunk_len;
  a.page_size = page_size;
  a.width = chunk_len / page_size;
  a.original_max_position_embeddings = original_max_position_embeddings;
  a.table_intra = table_intra;
  a.table_succ = table_succ;
  a.lens_intra = lens_intra;
  a.lens_succ = lens_succ;
  a.lens_inter = lens_inter;
  a.scaling_factor = scaling_factor;
  return pkv_host::from_hip(pkv_launch::dca_tables(a, static_cast<hipStream_t>(stream)),
                            "build_dca_decode_tables launch");
}

pkv_status_t build_cascade_expand_table(const uint8_t* custom_mask, int64_t mask_len,
                                        const int32_t* req_to_token, int64_t req_to_token_rows,
                                        int64_t req_to_token_stride,
                                        const int32_t* req_pool_indices, const int32_t* seq_lens,
                                        int32_t batch, int32_t num_draft, int32_t* expand_table,
                                        int32_t* expand_lens, int32_t* cu_expand_lens,
                                        void* stream) {
  PKV_REQUIRE(batch >= 0 && mask_len >= 0, PKV_EINVAL,
              "build_cascade_expand_table: batch %d, mask_len %lld", batch, (long long)mask_len);
  PKV_REQUIRE(num_draft >= 1, PKV_EINVAL, "build_cascade_expand_table: num_draft %d < 1",
              num_draft);
  PKV_REQUIRE(num_draft <= pkv_host::kMaxDraft, PKV_EUNSUPPORTED,
              "build_cascade_expand_table: num_draft %d > %d", num_draft, pkv_host::kMaxDraft);
  if (batch == 0) return pkv_host::ok();
  PKV_REQUIRE(custom_mask && req_to_token && req_pool_indices && seq_lens && expand_table &&
                  expand_lens,
              PKV_EINVAL, "build_cascade_expand_table: NULL required pointer");
  PKV_REQUIRE(req_to_token_rows >= 1 && req_to_token_stride >= 1, PKV_EINVAL,
              "build_cascade_expand_table: empty token table");
  pkv::CascadeExpandArgs a;
  a.mask = custom_mask;
  a.mask_len = mask_len;
  a.req_to_token = req_to_token;
  a.r2t_rows = req_to_token_rows;
  a.r2t_stride = req_to_token_stride;
  a.req_pool_indices = req_pool_indices;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.num_draft = num_draft;
  a.table = expand_table;
  a.lens = expand_lens;
  a.cu = cu_expand_lens;
  return pkv_host::from_hip(pkv_launch::cascade_expand(a, static_cast<hipStream_t>(stream)),
                            "build_cascade_expand_table launch");
}

static pkv_status_t expand_merge_prepare(const char* who, const void* q, int32_t dtype,
                                         const void* k_cache, const void* v_cache,
                                         int64_t num_slots, const int32_t* expand_table,
                                         int32_t expand_stride, const int32_t* expand_lens,
                                         int32_t n_rows, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         float softmax_scale, void* out, float* lse,
                                         pkv::ExpandMergeArgs& a) {
  PKV_REQUIRE(dtype == PKV_BF16, PKV_EUNSUPPORTED, "%s: dtype %d not supported (bf16)", who,
              dtype);
  PKV_REQUIRE(head_dim == 64 || head_dim == 128, PKV_EUNSUPPORTED,
              "%s: head_dim %d not supported (64, 128)", who, head_dim);
  PKV_REQUIRE(n_rows >= 0 && num_q_heads >= 1 && num_kv_heads >= 1 && expand_stride >= 1,
              PKV_EINVAL, "%s: bad sizes", who);
  PKV_REQUIRE(num_q_heads % num_kv_heads == 0, PKV_EINVAL,
              "%s: num_q_heads %d not a multiple of num_kv_heads %d", who, num_q_heads,
              num_kv_heads);
  PKV_REQUIRE(num_q_heads / num_kv_heads <= 16, PKV_EUNSUPPORTED, "%s: GQA group %d > 16", who,
              num_q_heads / num_kv_heads);
  PKV_REQUIRE(n_rows == 0 || (q && k_cache && v_cache && expand_table && expand_lens && out &&
                              lse),
              PKV_EINVAL, "%s: NULL required pointer (out and lse are both needed)", who);
  PKV_REQUIRE(n_rows == 0 || num_slots >= 1, PKV_EINVAL, "%s: empty cache", who);
  PKV_REQUIRE(pkv_host::scale_ok(softmax_scale), PKV_EINVAL,
              "%s: softmax_scale %g is not finite and positive", who, softmax_scale);
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.num_slots = num_slots;
  a.table = expand_table;
  a.lens = expand_lens;
  a.stride = expand_stride;
  a.rows = n_rows;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.scale_log2 = pkv_host::scale_log2(softmax_scale);
  a.out = out;
  a.lse = lse;
  return pkv_host::ok();
}

pkv_status_t paged_attn_expand_merge(const void* q, int32_t dtype, const void* k_cache,
                                     const void* v_cache, int64_t num_slots,
                                     const int32_t* expand_table, int32_t expand_stride,
                                     const int32_t* expand_lens, int32_t n_rows,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     float softmax_scale, void* out, float* lse, void* stream) {
  pkv::ExpandMergeArgs a;
  const pkv_status_t st = expand_merge_prepare(
      "paged_attn_expand_merge", q, dtype, k_cache, v_cache, num_slots, expand_table,
      expand_stride, expand_lens, n_rows, num_q_heads, num_kv_heads, head_dim, softmax_scale,
      out, lse, a);
  if (st != PKV_OK || n_rows == 0) return st;
  return pkv_host::from_hip(pkv_launch::expand_merge(a, head_dim, static_cast<hipStream_t>(stream)),
                            "paged_attn_expand_merge launch");
}

size_t paged_attn_cascade_workspace_size(int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                                         int32_t max_seqlen_k, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim) {
  if (batch <= 0 || total_q <= 0 || max_seqlen_q <= 0 || max_seqlen_k < 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || head_dim <= 0)
    return 0;
  const int w = pkv_launch::draft_prefix_heads(PKV_BF16, head_dim, num_q_heads, num_kv_heads,
                                               max_seqlen_q);
  if (w > 0)
    return pkv_host::draft_plan(batch, total_q, max_seqlen_k, num_q_heads, num_kv_heads,
                                head_dim, w)
        .bytes;
  return pkv_host::prefill_plan(batch, total_q, max_seqlen_q, max_seqlen_k, num_q_heads,
                                num_kv_heads, head_dim)
      .bytes;
}

pkv_status_t paged_attn_cascade(const void* q, int32_t dtype, const void* k_cache,
                                const void* v_cache, int64_t num_pages, const int32_t* page_table,
                                int32_t pt_stride, const int32_t* cu_seqlens_q,
                                const int32_t* kv_lens, int32_t batch, int32_t total_q,
                                int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                float softmax_scale, const int32_t* expand_table,
                                int32_t expand_stride, const int32_t* expand_lens,
                                void* workspace, size_t workspace_bytes, void* out, float* lse,
                                void* stream) {
  // every check before anything is enqueued; the prefix pass packs each kv
  // head's (head, draft) rows into one MFMA tile when they fit (w > 0), else
  // it is the prefill kernel with causal = 0
  const int w = pkv_launch::draft_prefix_heads(dtype, head_dim, num_q_heads, num_kv_heads,
                                               max_seqlen_q);
  pkv::PrefillArgs pa;
  bool nothing = false;
  pkv_status_t st = prefill_prepare(
      q, dtype, k_cache, v_cache, num_pages, page_table, pt_stride, cu_seqlens_q, kv_lens, batch,
      total_q, max_seqlen_q, max_seqlen_k, num_q_heads, num_kv_heads, head_dim, page_size,
      softmax_scale, 0, -1, 0, workspace, workspace_bytes, out, lse, pa, &nothing, w == 0);
  if (st != PKV_OK) return st;
  pkv::ExpandMergeArgs ea;
  st = expand_merge_prepare("paged_attn_cascade", q, dtype, k_cache, v_cache,
                            num_pages * page_size, expand_table, expand_stride, expand_lens,
                            total_q, num_q_heads, num_kv_heads, head_dim, softmax_scale, out, lse,
                            ea);
  if (st != PKV_OK || nothing) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (w == 0) {
    st = pkv_host::from_hip(pkv_launch::prefill(pa, head_dim, s),
                            "paged_attn_cascade: prefix pass launch");
  } else {
    const pkv_host::DraftPlan plan = pkv_host::draft_plan(
        batch, total_q, max_seqlen_k, num_q_heads, num_kv_heads, head_dim, w);
    PKV_REQUIRE(plan.bytes == 0 || (workspace != nullptr && workspace_bytes >= plan.bytes),
                PKV_EINVAL, "paged_attn_cascade: workspace of %zu bytes, need %zu",
                workspace_bytes, plan.bytes);
    pkv::DraftPrefixArgs da{};
    pkv::DecodeArgs& d = da.d;
    d.q = q;
    d.k = k_cache;
    d.v = v_cache;
    d.pt = page_table;
    d.pt_stride = pt_stride;
    d.kv_lens = kv_lens;
    d.batch = batch;
    d.hq = num_q_heads;
    d.hkv = num_kv_heads;
    d.page_size = page_size;
    d.num_pages = num_pages;
    d.scale_log2 = pkv_host::scale_log2(softmax_scale);
    d.chunk = plan.chunk;
    d.num_splits = plan.splits;
    d.out = out;
    d.lse = lse;
    d.window_left = -1;
    d.attn_chunk = 0;
    da.cu_q = cu_seqlens_q;
    da.total_q = total_q;
    if (plan.splits > 1) {
      char* ws = static_cast<char*>(workspace);
      da.part_o = ws + PKV_WORKSPACE_COUNTER_BYTES;
      da.part_lse = reinterpret_cast<float*>(ws + PKV_WORKSPACE_COUNTER_BYTES + plan.o_bytes);
    }
    st = pkv_host::from_hip(pkv_launch::draft_prefix(da, head_dim, s),
                            "paged_attn_cascade: prefix pass launch");
  }
  if (st != PKV_OK) return st;
  return pkv_host::from_hip(pkv_launch::expand_merge(ea, head_dim, s),
                            "paged_attn_cascade: expand pass launch");
}

}  // extern "C"
