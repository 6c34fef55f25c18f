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
// its length is the visible count (plus the lengths' prefix sum). One
// workgroup walks the requests 256 at a time; a block scan gives each
// request's offset into the flat mask (request blocks of n rows of L_b + n
// entries) and into the prefix sum.
//
// expand_merge_kernel runs the expand pass and the merge in one pass: one
// wave per (draft row, kv head) holds the G query heads of that kv head with
// D/64 dims per lane, streams the row's listed keys (a few, one coalesced
// row read each for K and V), keeps an online softmax per head (scores
// summed across the wave), then merges with the prefix pass's (O, LSE) that
// the caller's out / lse hold, and writes the result over them.
#include "args.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace pkv {

__global__ __launch_bounds__(256) void cascade_expand_kernel(CascadeExpandArgs a) {
  __shared__ int64_t s_off[256];
  __shared__ int32_t s_cnt[256];
  const int tid = threadIdx.x;
  const int n = a.num_draft;
  int64_t mask_base = 0;   // mask entries of the requests before this chunk
  int32_t cu_base = 0;     // listed keys of the requests before this chunk
  if (tid == 0 && a.cu != nullptr) a.cu[0] = 0;
  for (int b0 = 0; b0 < a.batch; b0 += 256) {
    const int b = b0 + tid;
    const bool live = b < a.batch;
    const int L = live ? max(a.seq_lens[b], 0) : 0;
    const int64_t blk = live ? static_cast<int64_t>(n) * (L + n) : 0;

    // inclusive scan of the requests' mask block sizes
    s_off[tid] = blk;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int64_t v = tid >= off ? s_off[tid - off] : 0;
      __syncthreads();
      s_off[tid] += v;
      __syncthreads();
    }
    const int64_t start = mask_base + s_off[tid] - blk;

    int32_t listed = 0;
    if (live) {
      const int64_t row = clamp_index(a.req_pool_indices[b], a.r2t_rows);
      const int32_t* r2t = a.req_to_token + row * a.r2t_stride;
      const int64_t last_col = a.r2t_stride - 1;
      for (int i = 0; i < n; ++i) {
        const int64_t m0 = start + static_cast<int64_t>(i) * (L + n) + L;
        int32_t* out = a.table + (static_cast<int64_t>(b) * n + i) * n;
        int k = 0;
        for (int pass = 0; pass < 2; ++pass) {   // visible drafts, then hidden ones
          for (int j = 0; j < n; ++j) {
            const int64_t mi = m0 + j;
            const bool vis = mi < a.mask_len && a.mask[mi] != 0;
            if (vis == (pass == 0)) {
              const int64_t col = min(static_cast<int64_t>(L) + j, last_col);
              out[k++] = r2t[col];
            }
          }
          if (pass == 0) {
            a.lens[static_cast<int64_t>(b) * n + i] = k;
            listed += k;
          }
        }
      }
    }

    // exclusive scan of the requests' listed keys for the prefix sum
    s_cnt[tid] = listed;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int32_t v = tid >= off ? s_cnt[tid - off] : 0;
      __syncthreads();
      s_cnt[tid] += v;
      __syncthreads();
    }
    if (live && a.cu != nullptr) {
      int32_t run = cu_base + s_cnt[tid] - listed;
      for (int i = 0; i < n; ++i) {
        const int64_t r = static_cast<int64_t>(b) * n + i;
        run += a.lens[r];   // written above by this thread
        a.cu[r + 1] = run;
      }
    }
    mask_base += s_off[255];
    cu_base += s_cnt[255];
    __syncthreads();   // the next chunk reuses the scan arrays
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void expand_merge_kernel(ExpandMergeArgs a) {
  constexpr int DPL = D / 64;   // dims per lane
  constexpr int GMAX = 16;
  const int lane = threadIdx.x & 63;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (item >= static_cast<int64_t>(a.rows) * a.hkv) return;   // wave-uniform
  const int r = static_cast<int>(item / a.hkv);
  const int kvh = static_cast<int>(item - static_cast<int64_t>(r) * a.hkv);
  const int G = a.hq / a.hkv;
  const int cnt = min(max(a.lens[r], 0), a.stride);

  const uint16_t* qb = static_cast<const uint16_t*>(a.q) +
                       (static_cast<int64_t>(r) * a.hq + static_cast<int64_t>(kvh) * G) * D +
                       lane * DPL;
  float qf[GMAX][DPL];
  float m[GMAX], l[GMAX], acc[GMAX][DPL];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    m[g] = neg_inf();
    l[g] = 0.f;
#pragma unroll
    for (int d = 0; d < DPL; ++d) {
      acc[g][d] = 0.f;
      qf[g][d] = g < G ? bf16_to_f32(qb[g * D + d]) : 0.f;
    }
  }

  const uint16_t* kb = static_cast<const uint16_t*>(a.k);
  const uint16_t* vb = static_cast<const uint16_t*>(a.v);
  const int32_t* row_keys = a.table + static_cast<int64_t>(r) * a.stride;
  for (int t = 0; t < cnt; ++t) {
    const int64_t slot = clamp_index(row_keys[t], a.num_slots);
    const int64_t off = (slot * a.hkv + kvh) * D + lane * DPL;
    float kf[DPL], vf[DPL];
#pragma unroll
    for (int d = 0; d < DPL; ++d) {
      kf[d] = bf16_to_f32(kb[off + d]);
      vf[d] = bf16_to_f32(vb[off + d]);
    }
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if (g < G) {
        float part = 0.f;
#pragma unroll
        for (int d = 0; d < DPL; ++d) part = __builtin_fmaf(qf[g][d], kf[d], part);
        const float s = wave_sum(part) * a.scale_log2;
        const float m_new = fmaxf(m[g], s);
        const float alpha = fast_exp2(m[g] - m_new);   // 0 while m is -inf
        const float p = fast_exp2(s - m_new);
        l[g] = __builtin_fmaf(l[g], alpha, p);
#pragma unroll
        for (int d = 0; d < DPL; ++d) acc[g][d] = __builtin_fmaf(acc[g][d], alpha, p * vf[d]);
        m[g] = m_new;
      }
    }
  }

  // merge with the prefix pass's state held in out / lse
  uint16_t* ob = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g < G) {
      const int64_t row = static_cast<int64_t>(r) * a.hq + static_cast<int64_t>(kvh) * G + g;
      const float lse1 = a.lse[row];
      const float lse2 = cnt > 0 ? (m[g] + fast_log2(l[g])) * kLn2 : neg_inf();
      const float mx = fmaxf(lse1, lse2);
      float w1 = 0.f, w2 = 0.f;
      if (mx != neg_inf()) {
        w1 = fast_exp2((lse1 - mx) * kLog2e);
        w2 = fast_exp2((lse2 - mx) * kLog2e);
      }
      const float total = w1 + w2;
      const float inv = total > 0.f ? 1.f / total : 0.f;
      const float inv_l = cnt > 0 ? 1.f / l[g] : 0.f;
      uint16_t* dst = ob + row * D + lane * DPL;
      float res[DPL];
#pragma unroll
      for (int d = 0; d < DPL; ++d) {
        const float o1 = bf16_to_f32(dst[d]);
        const float o2 = acc[g][d] * inv_l;
        res[d] = (w1 * o1 + w2 * o2) * inv;
      }
      if constexpr (DPL == 2) {
        *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(res[0], res[1]);
      } else {
        dst[0] = f32_to_bf16(res[0]);
      }
      if (lane == 0) a.lse[row] = mx == neg_inf() ? neg_inf() : mx + fast_log2(total) * kLn2;
    }
  }
}

}  // namespace pkv

namespace pkv_launch {

hipError_t cascade_expand(const pkv::CascadeExpandArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(pkv::cascade_expand_kernel, dim3(1), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t expand_merge(const pkv::ExpandMergeArgs& a, int head_dim, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(a.rows) * a.hkv;
  const dim3 grid(static_cast<unsigned>((items + 3) / 4));
  if (head_dim == 128)
    hipLaunchKernelGGL(pkv::expand_merge_kernel<128>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(pkv::expand_merge_kernel<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv_launch
