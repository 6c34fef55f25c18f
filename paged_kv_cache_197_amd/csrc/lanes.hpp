// Cross-lane maxima and sums that stay in the VALU (no LDS round trip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// max(v, v of lane l ^ 8): a DPP rotation by eight inside each 16-lane row
// (row_ror:8) pairs lane i of the row with lane i ^ 8.
__device__ __forceinline__ float max_xor8(float v) {
  const int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false);
  return fmaxf(v, __int_as_float(o));
}

// max(v, v of lane l ^ 16): v_permlane16_swap exchanges the odd 16-lane rows
// of one operand with the even rows of the other; with both operands v, each
// lane sees its own value and its partner's.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum over all 64 lanes, in every lane, without LDS: DPP within each quad
// (lane ^ 1, lane ^ 2), DPP rotations by 4 and 8 inside each 16-lane row (the
// four quad sums of the row), then the row pairs l ^ 16 and l ^ 32 through
// the permlane swaps.
template <int CTRL>
__device__ __forceinline__ float add_dpp_t(float v) {
  const int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false);
  return v + __int_as_float(o);
}
__device__ __forceinline__ float wave_sum64(float v) {
  v = add_dpp_t<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v = add_dpp_t<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v = add_dpp_t<0x124>(v);   // row_ror:4
  v = add_dpp_t<0x128>(v);   // row_ror:8
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
  v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

}  // namespace pkv
