// paged_kv_append: write the new tokens' keys and values into the cache
// ([FA] forward_extend / forward_decode: set_kv_buffer at out_cache_loc before
// attending). Row i of k_new / v_new ([n, Hkv, D], one token) goes to token
// slot out_cache_loc[i] of the cache viewed as [num_slots, Hkv, D].
//
// HBM-bound scatter: each row is copied in 16-byte pieces, consecutive
// threads taking consecutive pieces of one row, so reads and writes are
// contiguous runs of the row's Hkv * D elements. A slot outside [0, num_slots)
// is skipped (a violated precondition writes nothing).
#include "args.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace pkv {

__global__ __launch_bounds__(256) void kv_append_kernel(const char* __restrict__ k_new,
                                                        const char* __restrict__ v_new,
                                                        const int32_t* __restrict__ loc,
                                                        int32_t n, int32_t pieces_per_row,
                                                        char* k_cache, char* v_cache,
                                                        int64_t num_slots) {
  const int64_t total = static_cast<int64_t>(n) * pieces_per_row;
  const int64_t row_bytes = static_cast<int64_t>(pieces_per_row) * 16;
  for (int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; p < total;
       p += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t i = p / pieces_per_row;
    const int64_t c = p - i * pieces_per_row;
    const int64_t slot = loc[i];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t src = i * row_bytes + c * 16;
    const int64_t dst = slot * row_bytes + c * 16;
    *reinterpret_cast<u32x4*>(k_cache + dst) = *reinterpret_cast<const u32x4*>(k_new + src);
    *reinterpret_cast<u32x4*>(v_cache + dst) = *reinterpret_cast<const u32x4*>(v_new + src);
  }
}

}  // namespace pkv

namespace pkv_launch {

hipError_t kv_append(const void* k_new, const void* v_new, const int32_t* loc, int32_t n,
                     int64_t row_bytes, void* k_cache, void* v_cache, int64_t num_slots,
                     hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int32_t pieces = static_cast<int32_t>(row_bytes / 16);
  const int64_t total = static_cast<int64_t>(n) * pieces;
  // enough workgroups to fill the chip several times over, each thread a few pieces
  const int64_t want = (total + 255) / 256;
  const unsigned blocks = static_cast<unsigned>(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(pkv::kv_append_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const char*>(k_new), static_cast<const char*>(v_new), loc, n,
                     pieces, static_cast<char*>(k_cache), static_cast<char*>(v_cache), num_slots);
  return hipGetLastError();
}

}  // namespace pkv_launch
