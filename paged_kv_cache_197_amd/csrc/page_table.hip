// build_page_table: req_to_token rows -> per-request page table, kv_lens and
// cu_seqlens_k, in one launch. Strided mode reduces each request's token
// slots to the ids of its pages ([FA] init_forward_metadata); the
// prefill-aware sliding-window mode keeps the prompt and the newest window of
// decoded positions ([FA] _build_pa_page_table_kernel).
//
// Grid: x = request, y = column blocks of 256 over `width`. Every element of
// page_table is written (zero past the request's length). Block (0, 0)
// additionally recomputes every kv_len and writes the prefix sum.
#include "args.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace pkv {

struct ReqGeom {
  int64_t row_base;  // r * stride, or -1 for an out-of-range pool row
  int32_t kv_len;
  int32_t pf;        // prefill length (sliding-window mode)
  int32_t gap;       // tokens skipped between prefill and window
};

__device__ __forceinline__ ReqGeom request_geometry(const PageTableArgs& a, int b) {
  ReqGeom g;
  const int64_t r = a.rpi[b];
  const bool row_ok = r >= 0 && r < a.rows;
  g.row_base = row_ok ? r * a.stride : -1;
  const int32_t sl = max(a.seq_lens[b], 0);
  if (a.prefill_lens != nullptr) {
    const int32_t pf = row_ok ? a.prefill_lens[r] : 0;
    const int32_t decode_start = max(pf, sl - a.window);
    g.gap = decode_start > pf ? decode_start - pf : 0;
    g.pf = pf;
    g.kv_len = sl - g.gap;
  } else {
    g.gap = 0;
    g.pf = 0;
    g.kv_len = sl;
  }
  return g;
}

__global__ __launch_bounds__(256) void page_table_kernel(PageTableArgs a) {
  const int b = blockIdx.x;
  const int col = blockIdx.y * 256 + threadIdx.x;
  const ReqGeom g = request_geometry(a, b);

  if (col < a.width) {
    int32_t val = 0;
    if (a.prefill_lens != nullptr) {
      if (col < g.kv_len && g.row_base >= 0) {
        const int64_t pos = col < g.pf ? col : static_cast<int64_t>(col) + g.gap;
        val = pos < a.stride ? a.r2t[g.row_base + pos] : 0;
      }
    } else {
      const int64_t n_pages = (static_cast<int64_t>(g.kv_len) + a.page_size - 1) / a.page_size;
      if (col < n_pages && g.row_base >= 0) {
        const int64_t pos = static_cast<int64_t>(col) * a.page_size;
        val = pos < a.stride ? a.r2t[g.row_base + pos] / a.page_size : 0;
      }
    }
    a.page_table[static_cast<int64_t>(b) * a.width + col] = val;
  }
  if (col == 0) a.kv_lens[b] = g.kv_len;

  // prefix sum of kv_lens over the whole batch, by block (0, 0)
  if (a.cu_seqlens_k != nullptr && blockIdx.x == 0 && blockIdx.y == 0) {
    __shared__ int32_t wave_sums[4];
    __shared__ int32_t carry_s;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (threadIdx.x == 0) {
      a.cu_seqlens_k[0] = 0;
      carry_s = 0;
    }
    __syncthreads();
    for (int base = 0; base < a.batch; base += 256) {
      const int i = base + threadIdx.x;
      int32_t v = i < a.batch ? request_geometry(a, i).kv_len : 0;
      // inclusive scan within the wave
      for (int off = 1; off < 64; off <<= 1) {
        const int32_t t = __shfl_up(v, off);
        if (lane >= off) v += t;
      }
      if (lane == 63) wave_sums[wave] = v;
      __syncthreads();
      int32_t before = carry_s;
      for (int w = 0; w < wave; ++w) before += wave_sums[w];
      if (i < a.batch) a.cu_seqlens_k[i + 1] = before + v;
      __syncthreads();
      if (threadIdx.x == 255) carry_s = before + v;
      __syncthreads();
    }
  }
}

__global__ void write_zero_kernel(int32_t* p) { *p = 0; }

}  // namespace pkv

namespace pkv_launch {

hipError_t page_table(const pkv::PageTableArgs& a, hipStream_t stream) {
  if (a.batch == 0) {
    if (a.cu_seqlens_k != nullptr) {
      hipLaunchKernelGGL(pkv::write_zero_kernel, dim3(1), dim3(1), 0, stream, a.cu_seqlens_k);
    }
    return hipGetLastError();
  }
  const int col_blocks = a.width > 0 ? (a.width + 255) / 256 : 1;
  hipLaunchKernelGGL(pkv::page_table_kernel, dim3(a.batch, col_blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv_launch
