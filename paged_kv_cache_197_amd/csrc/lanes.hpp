// Cross-lane maxima that stay in the VALU (no LDS round trip).
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

}  // namespace pkv
