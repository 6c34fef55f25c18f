// merge_state: S-way LSE-weighted combine of partial attention states
// ([DCA] _merge_attn_outputs; [FA] merge_state_v2 call sites).
//
// Memory-bound: each thread owns VEC consecutive output elements of one
// (token, head) row, reads the row's S LSE values (L1/L2 hits after the
// first lane) and S x VEC partial values with vector loads, and writes VEC
// outputs. Traffic per row: S * (Dv * 4 + 4) bytes read, Dv * sizeof(out) +
// 4 bytes written.
#include "common.hpp"
#include "launch.hpp"

namespace pkv {

template <typename TO>
__device__ __forceinline__ void store_vec4(TO* dst, float4 v);

template <>
__device__ __forceinline__ void store_vec4<float>(float* dst, float4 v) {
  *reinterpret_cast<float4*>(dst) = v;
}
template <>
__device__ __forceinline__ void store_vec4<bf16_t>(bf16_t* dst, float4 v) {
  u32x2 w;
  w.x = pack_bf16x2(v.x, v.y);
  w.y = pack_bf16x2(v.z, v.w);
  *reinterpret_cast<u32x2*>(dst) = w;
}

__device__ __forceinline__ void store_one(float* dst, float v) { *dst = v; }
__device__ __forceinline__ void store_one(bf16_t* dst, float v) { dst->bits = f32_to_bf16(v); }

template <typename TO, int VEC>
__global__ __launch_bounds__(256) void merge_state_kernel(const float* __restrict__ o_parts,
                                                          const float* __restrict__ lse_parts,
                                                          int num_parts, int64_t rows, int dv,
                                                          TO* __restrict__ out,
                                                          float* __restrict__ lse_out) {
  const int vecs_per_row = dv / VEC;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= rows * vecs_per_row) return;
  const int64_t row = idx / vecs_per_row;
  const int col = static_cast<int>(idx - row * vecs_per_row) * VEC;

  // The parts' pieces are requested eight at a time, all in flight before
  // the first is used, and the first eight go out before the LSEs, so that
  // both arrive in one round trip. A part of zero weight (an empty split, or
  // one far below the max) adds nothing, whatever its output holds.
  constexpr int BATCH = 8;
  float v[BATCH][VEC];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int s = min(s0 + k, num_parts - 1);
      const float* src = o_parts + (s * rows + row) * dv + col;
      if (VEC == 4) {
        const float4 q = *reinterpret_cast<const float4*>(src);
        v[k][0] = q.x;
        v[k][1 % VEC] = q.y;
        v[k][2 % VEC] = q.z;
        v[k][3 % VEC] = q.w;
      } else {
        v[k][0] = src[0];
      }
    }
  };
  load_batch(0);
  float m = neg_inf();
  for (int s = 0; s < num_parts; ++s) m = fmaxf(m, lse_parts[s * rows + row]);

  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
  float total = 0.f;
  if (m != neg_inf()) {
    for (int s0 = 0; s0 < num_parts; s0 += BATCH) {
      if (s0 > 0) load_batch(s0);
#pragma unroll
      for (int k = 0; k < BATCH; ++k) {
        const int s = min(s0 + k, num_parts - 1);
        const float w = (s0 + k < num_parts) ? merge_weight(lse_parts[s * rows + row], m) : 0.f;
        if (w == 0.f) continue;
        merge_add(w, v[k], acc, total);
      }
    }
  }
  const float inv = merge_norm(total);
  TO* dst = out + row * dv + col;
  if (VEC == 4) {
    store_vec4<TO>(dst, make_float4(acc[0] * inv, acc[1 % VEC] * inv, acc[2 % VEC] * inv,
                                    acc[3 % VEC] * inv));
  } else {
    store_one(dst, acc[0] * inv);
  }
  if (lse_out != nullptr && col == 0) {
    lse_out[row] = merge_lse(m, total);
  }
}

}  // namespace pkv

namespace pkv_launch {

hipError_t merge_state(const float* o_parts, const float* lse_parts, int num_parts, int64_t rows,
                       int dv, void* out, int out_dtype, float* lse_out, hipStream_t stream) {
  const int vec = (dv % 4 == 0) ? 4 : 1;
  const int64_t threads = rows * (dv / vec);
  if (threads == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  if (out_dtype == PKV_F32) {
    if (vec == 4)
      hipLaunchKernelGGL((pkv::merge_state_kernel<float, 4>), grid, dim3(256), 0, stream, o_parts,
                         lse_parts, num_parts, rows, dv, static_cast<float*>(out), lse_out);
    else
      hipLaunchKernelGGL((pkv::merge_state_kernel<float, 1>), grid, dim3(256), 0, stream, o_parts,
                         lse_parts, num_parts, rows, dv, static_cast<float*>(out), lse_out);
  } else {
    if (vec == 4)
      hipLaunchKernelGGL((pkv::merge_state_kernel<pkv::bf16_t, 4>), grid, dim3(256), 0, stream,
                         o_parts, lse_parts, num_parts, rows, dv, static_cast<pkv::bf16_t*>(out),
                         lse_out);
    else
      hipLaunchKernelGGL((pkv::merge_state_kernel<pkv::bf16_t, 1>), grid, dim3(256), 0, stream,
                         o_parts, lse_parts, num_parts, rows, dv, static_cast<pkv::bf16_t*>(out),
                         lse_out);
  }
  return hipGetLastError();
}

}  // namespace pkv_launch
