// Shared device helpers for the gfx950 kernels: bf16 packing, MFMA operand
// types, wavefront reductions and the launch-status plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Storage type for bf16 elements (raw 16-bit words).
struct bf16_t {
  uint16_t bits;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// low / high half of a packed pair
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}
// Two fp32 -> packed bf16 pair (lo in bits 0-15), one v_cvt_pk_bf16_f32, RNE.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Pair the low halves / high halves of two packed words: (a.lo, b.lo), (a.hi, b.hi).
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Reductions across lanes l, l^16, l^32, l^48 (the four 16-lane groups),
// in the VALU: v_permlane16_swap pairs each 16-lane row with its neighbour
// (l ^ 16) and v_permlane32_swap each half of the wave with the other
// (l ^ 32); with both operands v each lane sees its own value and its
// partner's.
__device__ __forceinline__ float max_over_groups16(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_groups16(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// max(v, v of lane l ^ 32) without an LDS round trip: v_permlane32_swap hands
// each half of the wave the other half's values.
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Make the load that produced `v` complete here: an empty asm statement that
// reads the register, so the waitcnt inserted for it lands before a loop
// instead of inside it.
__device__ __forceinline__ void retire(uint32_t v) { asm volatile("" ::"v"(v)); }

// Data handed from one workgroup to another within a launch (split partials,
// then a counter). Every handed-over word is stored and loaded at device scope
// (cache-policy bit sc1): the AMDGPU memory model of the gfx942 generation,
// which gfx950 follows, encodes relaxed agent-scope atomic stores and loads
// this way, i.e. they are coherent across the per-XCD L2 caches. Ordering: each
// producer wave waits until its stores have completed (vmcnt(0)), the
// workgroup barrier follows, then one lane adds to the agent-scope counter;
// the workgroup that sees the final count loads only after that add has
// returned. This is a release / acquire pair without their cache maintenance
// (write-back and invalidate of the whole XCD L2), which is not needed because
// no handed-over word goes through an ordinary access; that maintenance would
// also drop data other workgroups reuse from the L2.
// Buffer resources need a wave-uniform base; the byte offsets are per lane.
constexpr int kScopeDevice = 16;   // sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, kScopeDevice);
}
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x2_t v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, kScopeDevice);
}
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kScopeDevice);
}
__device__ __forceinline__ float load_coherent1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kScopeDevice));
}
__device__ __forceinline__ f32x2_t load_coherent2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kScopeDevice));
}
__device__ __forceinline__ f32x4 load_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kScopeDevice));
}
// all of this wave's memory operations have completed
__device__ __forceinline__ void wait_all_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// agent-scope counter, relaxed: the ordering comes from wait_all_vmem, the
// barrier around the add, and the device-scope accesses of the data
__device__ __forceinline__ int counter_add(int* c, int v) {
  return __hip_atomic_fetch_add(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void counter_reset(int* c) {
  __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LSE-weighted combine of partial states, one part at a time in split order:
// m = max of the parts' LSEs, w = exp(lse - m), acc += w * o, total += w,
// out = acc / total, lse_out = m + ln(total). Parts of weight 0 (empty
// splits: lse = -inf) are skipped. merge_state and the merged decode both go
// through these, so the two give the same bits.
__device__ __forceinline__ float merge_weight(float lse_part, float m) {
  return fast_exp2((lse_part - m) * kLog2e);
}
template <int N>
__device__ __forceinline__ void merge_add(float w, const float (&v)[N], float (&acc)[N],
                                          float& total) {
  total += w;
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = __builtin_fmaf(w, v[i], acc[i]);
}
__device__ __forceinline__ float merge_norm(float total) { return total > 0.f ? 1.f / total : 0.f; }
__device__ __forceinline__ float merge_lse(float m, float total) {
  return m == neg_inf() ? neg_inf() : __builtin_fmaf(fast_log2(total), kLn2, m);
}

// Clamp an index read from device memory into [0, n): a violated precondition
// turns into a wrong (but in-bounds) access instead of a fault.
__device__ __forceinline__ int64_t clamp_index(int64_t i, int64_t n) {
  return (static_cast<uint64_t>(i) < static_cast<uint64_t>(n)) ? i : 0;
}

}  // namespace pkv
