// build_dca_decode_tables: the per-request metadata of dual chunk attention
// decode ([DCA] init_forward_metadata, decode branch). With chunk_len C and
// the query's chunk c = (L - 1) / C:
//   intra: keys [cC, L), table = the request's page-table row from page cC / P
//   succ:  keys [(c - 1)C, cC) (none when c = 0), table from page (c - 1) C / P
//   inter: max(c - 1, 0) C keys from key 0 (the request's own row)
// and, when original_max_position_embeddings > 0, the query scaling factor
// max(0.1 ln(L / original_max_position_embeddings) + 1, 1). Table rows are
// C / P columns wide and list the pages of their stage's keys, then 0.
//
// Integer gather, one thread per (request, column) for both tables.
#include "args.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace pkv {

__global__ __launch_bounds__(256) void dca_tables_kernel(DcaTableArgs a) {
  const int b = blockIdx.x;
  const int col = blockIdx.y * 256 + threadIdx.x;
  const int L = max(a.seq_lens[b], 0);
  const int C = a.chunk_len;
  const int c = L > 0 ? (L - 1) / C : 0;
  const int64_t last_page = L > 0 ? (L - 1) / a.page_size + 1 : 0;   // pages the request holds
  const int32_t* row = a.block_tables + static_cast<int64_t>(b) * a.bt_stride;
  const int64_t last_col = a.bt_stride - 1;
  if (col < a.width) {
    const int64_t out = static_cast<int64_t>(b) * a.width + col;
    const int64_t i_intra = static_cast<int64_t>(c) * C / a.page_size + col;
    a.table_intra[out] = i_intra < last_page ? row[min(i_intra, last_col)] : 0;
    if (a.table_succ != nullptr) {
      // c >= 1: the C / P pages of the chunk before the query's, all held
      const int64_t i_succ = static_cast<int64_t>(c - 1) * C / a.page_size + col;
      a.table_succ[out] = (c >= 1 && i_succ < last_page) ? row[min(i_succ, last_col)] : 0;
    }
  }
  if (blockIdx.y == 0 && threadIdx.x == 0) {
    a.lens_intra[b] = L - c * C;
    a.lens_succ[b] = c >= 1 ? C : 0;
    a.lens_inter[b] = max(c - 1, 0) * C;
    if (a.scaling_factor != nullptr) {
      float f = 1.f;
      if (a.original_max_position_embeddings > 0)
        f = fmaxf(0.1f * logf(static_cast<float>(L) /
                              static_cast<float>(a.original_max_position_embeddings)) + 1.f,
                  1.f);
      a.scaling_factor[b] = f;
    }
  }
}

}  // namespace pkv

namespace pkv_launch {

hipError_t dca_tables(const pkv::DcaTableArgs& a, hipStream_t stream) {
  if (a.batch <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(a.batch), static_cast<unsigned>((a.width + 255) / 256));
  hipLaunchKernelGGL(pkv::dca_tables_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv_launch
