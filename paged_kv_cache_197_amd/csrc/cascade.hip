// Cascade attention for draft-tree verification ([FA] init_forward_metadata,
// target verify with topk > 1, and the use_cascade_attn branches of
// forward_extend / forward_decode).
//
// Request b has L_b committed tokens and n draft tokens at positions
// L_b .. L_b+n-1. Draft row (b, i) attends over every committed token (the
// prefix pass: the prefill kernel, non-causal, n rows per request) and over
// the drafts its custom-mask row allows (the expand pass); the two partial
// states are merged by their LSEs.
//
// cascade_expand_kernel builds the expand pass's key lists: row (b, i) lists
// the slots of the visible drafts in position order, then the hidden ones, and
// its length is the visible count; expand_cu_kernel adds the lengths' prefix
// sum when asked for.
//
// expand_merge_kernel runs the expand pass and the merge in one pass: one
// wave per (draft row, kv head) holds the G query heads of that kv head with
// D/64 dims per lane, streams the row's listed keys (a few, one coalesced
// row read each for K and V), keeps an online softmax per head (scores
// summed across the wave with DPP and permlane swaps), then merges with the prefix pass's (O, LSE) that
// the caller's out / lse hold, and writes the result over them.
#include "args.hpp"
#include "common.hpp"
#include "lanes.hpp"
#include "launch.hpp"

namespace pkv {

// One wave per request. Its mask block starts after the blocks of the
// requests before it: n * (sum of their L) + b * n * n entries, summed by the
// wave from seq_lens. Lane j holds draft column j (and j + 64, ... for n > 64):
// its slot, and per row its mask byte; a ballot gives each visible column its
// place among the visible ones and each hidden column its place after them.
constexpr int kExpandChunks = 4;   // columns per lane: n <= 256

__global__ __launch_bounds__(256) void cascade_expand_kernel(CascadeExpandArgs a) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= a.batch) return;   // wave-uniform
  const int n = a.num_draft;
  const uint8_t* __restrict__ mask = a.mask;
  int32_t* __restrict__ table = a.table;

  int64_t before = 0;   // committed tokens of the requests before b
  for (int t = lane; t < b; t += 64) before += max(a.seq_lens[t], 0);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) before += __shfl_xor(before, m);
  const int L = max(a.seq_lens[b], 0);
  const int64_t start = static_cast<int64_t>(n) * before + static_cast<int64_t>(b) * n * n;

  const int64_t row = clamp_index(a.req_pool_indices[b], a.r2t_rows);
  const int32_t* r2t = a.req_to_token + row * a.r2t_stride;
  const int64_t last_col = a.r2t_stride - 1;
  int32_t slot[kExpandChunks];
#pragma unroll
  for (int c = 0; c < kExpandChunks; ++c) {
    const int j = 64 * c + lane;
    slot[c] = j < n ? r2t[min(static_cast<int64_t>(L) + j, last_col)] : 0;
  }
  const uint64_t below = (1ull << lane) - 1;   // lanes before this one
  for (int i = 0; i < n; ++i) {
    const int64_t m0 = start + static_cast<int64_t>(i) * (L + n) + L;
    uint64_t vis[kExpandChunks];
    int total = 0;
#pragma unroll
    for (int c = 0; c < kExpandChunks; ++c) {
      const int j = 64 * c + lane;
      const int64_t mi = m0 + j;
      const bool v = j < n && mi < a.mask_len && mask[mi] != 0;
      vis[c] = __ballot(v);
      total += __popcll(vis[c]);
    }
    int32_t* out = table + (static_cast<int64_t>(b) * n + i) * n;
    int vis_before = 0;   // visible columns in earlier chunks
#pragma unroll
    for (int c = 0; c < kExpandChunks; ++c) {
      const int j = 64 * c + lane;
      if (j < n) {
        const bool v = (vis[c] >> lane) & 1;
        const int vb = vis_before + __popcll(vis[c] & below);   // visible columns before j
        out[v ? vb : total + (j - vb)] = slot[c];
      }
      vis_before += __popcll(vis[c]);
    }
    if (lane == 0) a.lens[static_cast<int64_t>(b) * n + i] = total;
  }
}

// Zero-led prefix sum of the expand lengths (rows = batch * n), one workgroup
// of 1024 threads scanning 1024 rows at a time.
__global__ __launch_bounds__(1024) void expand_cu_kernel(const int32_t* __restrict__ lens,
                                                         int64_t rows, int32_t* __restrict__ cu) {
  __shared__ int32_t s[1024];
  const int tid = threadIdx.x;
  int32_t carry = 0;
  if (tid == 0) cu[0] = 0;
  for (int64_t r0 = 0; r0 < rows; r0 += 1024) {
    const int64_t r = r0 + tid;
    const int32_t v = r < rows ? lens[r] : 0;
    s[tid] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int32_t u = tid >= off ? s[tid - off] : 0;
      __syncthreads();
      s[tid] += u;
      __syncthreads();
    }
    if (r < rows) cu[r + 1] = carry + s[tid];
    carry += s[1023];
    __syncthreads();   // the next chunk reuses s
  }
}

// GMAX >= the GQA group (4, 8 or 16): the per-head arrays are sized by it, so
// small groups keep few registers and many waves per SIMD.
template <int D, int GMAX>
__global__ __launch_bounds__(256) void expand_merge_kernel(ExpandMergeArgs a) {
  constexpr int DPL = D / 64;   // dims per lane
  constexpr int KB = 4;         // keys whose rows are requested together
  const int lane = threadIdx.x & 63;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (item >= static_cast<int64_t>(a.rows) * a.hkv) return;   // wave-uniform
  const int r = static_cast<int>(item / a.hkv);
  const int kvh = static_cast<int>(item - static_cast<int64_t>(r) * a.hkv);
  const int G = a.hq / a.hkv;

  // Everything that does not depend on the key list is requested up front,
  // together with the list itself (lane t holds entry t): the row's query
  // heads, and the prefix pass's output and LSE that the merge reads.
  const int32_t* row_keys = a.table + static_cast<int64_t>(r) * a.stride;
  const int cnt = min(max(a.lens[r], 0), a.stride);
  const int32_t lane_slot = lane < a.stride ? row_keys[lane] : 0;
  const int64_t row0 = static_cast<int64_t>(r) * a.hq + static_cast<int64_t>(kvh) * G;
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + row0 * D + lane * DPL;
  uint16_t* ob = static_cast<uint16_t*>(a.out) + row0 * D + lane * DPL;
  float qf[GMAX][DPL], o1[GMAX][DPL], lse1[GMAX];
  float m[GMAX], l[GMAX], acc[GMAX][DPL];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    m[g] = neg_inf();
    l[g] = 0.f;
    lse1[g] = g < G ? a.lse[row0 + g] : neg_inf();
#pragma unroll
    for (int d = 0; d < DPL; ++d) {
      acc[g][d] = 0.f;
      qf[g][d] = g < G ? bf16_to_f32(qb[g * D + d]) : 0.f;
      o1[g][d] = g < G ? bf16_to_f32(ob[g * D + d]) : 0.f;
    }
  }

  const uint16_t* kb = static_cast<const uint16_t*>(a.k);
  const uint16_t* vb = static_cast<const uint16_t*>(a.v);
  for (int t0 = 0; t0 < cnt; t0 += KB) {
    float kf[KB][DPL], vf[KB][DPL];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int t = min(t0 + u, cnt - 1);
      const int32_t raw = t < 64 ? __builtin_amdgcn_readlane(lane_slot, t) : row_keys[t];
      const int64_t slot = clamp_index(raw, a.num_slots);
      const int64_t off = (slot * a.hkv + kvh) * D + lane * DPL;
#pragma unroll
      for (int d = 0; d < DPL; ++d) {
        kf[u][d] = bf16_to_f32(kb[off + d]);
        vf[u][d] = bf16_to_f32(vb[off + d]);
      }
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (t0 + u < cnt) {
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
          if (g < G) {
            float part = 0.f;
#pragma unroll
            for (int d = 0; d < DPL; ++d) part = __builtin_fmaf(qf[g][d], kf[u][d], part);
            const float sc = wave_sum64(part) * a.scale_log2;
            const float m_new = fmaxf(m[g], sc);
            const float alpha = fast_exp2(m[g] - m_new);   // 0 while m is -inf
            const float p = fast_exp2(sc - m_new);
            l[g] = __builtin_fmaf(l[g], alpha, p);
#pragma unroll
            for (int d = 0; d < DPL; ++d)
              acc[g][d] = __builtin_fmaf(acc[g][d], alpha, p * vf[u][d]);
            m[g] = m_new;
          }
        }
      }
    }
  }

  // merge with the prefix pass's state and write over it
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g < G) {
      const float lse2 = cnt > 0 ? (m[g] + fast_log2(l[g])) * kLn2 : neg_inf();
      const float mx = fmaxf(lse1[g], lse2);
      float w1 = 0.f, w2 = 0.f;
      if (mx != neg_inf()) {
        w1 = fast_exp2((lse1[g] - mx) * kLog2e);
        w2 = fast_exp2((lse2 - mx) * kLog2e);
      }
      const float total = w1 + w2;
      const float inv = total > 0.f ? 1.f / total : 0.f;
      const float inv_l = cnt > 0 ? 1.f / l[g] : 0.f;
      float res[DPL];
#pragma unroll
      for (int d = 0; d < DPL; ++d) res[d] = (w1 * o1[g][d] + w2 * (acc[g][d] * inv_l)) * inv;
      uint16_t* dst = ob + g * D;
      if constexpr (DPL == 2) {
        *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(res[0], res[1]);
      } else {
        dst[0] = f32_to_bf16(res[0]);
      }
      if (lane == 0) a.lse[row0 + g] = mx == neg_inf() ? neg_inf() : mx + fast_log2(total) * kLn2;
    }
  }
}

}  // namespace pkv

namespace pkv_launch {

hipError_t cascade_expand(const pkv::CascadeExpandArgs& a, hipStream_t stream) {
  if (a.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(pkv::cascade_expand_kernel, dim3((a.batch + 3) / 4), dim3(256), 0, stream, a);
  if (a.cu != nullptr)
    hipLaunchKernelGGL(pkv::expand_cu_kernel, dim3(1), dim3(1024), 0, stream, a.lens,
                       static_cast<int64_t>(a.batch) * a.num_draft, a.cu);
  return hipGetLastError();
}

template <int D>
static void launch_expand_merge(const pkv::ExpandMergeArgs& a, dim3 grid, hipStream_t stream) {
  const int G = a.hq / a.hkv;
  if (G <= 4)
    hipLaunchKernelGGL((pkv::expand_merge_kernel<D, 4>), grid, dim3(256), 0, stream, a);
  else if (G <= 8)
    hipLaunchKernelGGL((pkv::expand_merge_kernel<D, 8>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((pkv::expand_merge_kernel<D, 16>), grid, dim3(256), 0, stream, a);
}

hipError_t expand_merge(const pkv::ExpandMergeArgs& a, int head_dim, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(a.rows) * a.hkv;
  const dim3 grid(static_cast<unsigned>((items + 3) / 4));
  if (head_dim == 128) launch_expand_merge<128>(a, grid, stream);
  else launch_expand_merge<64>(a, grid, stream);
  return hipGetLastError();
}

}  // namespace pkv_launch
