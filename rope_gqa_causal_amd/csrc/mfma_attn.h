// mfma_attn.h -- gfx950 helpers shared by the matrix-core attention kernels
// (causal prefill and differential attention).
#pragma once

#include "common.h"

namespace rgc {

constexpr float kAttnLog2e = 1.4426950408889634f;
constexpr float kAttnLn2 = 0.6931471805599453f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// c + a.lo * b.lo + a.hi * b.hi over packed bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// One v_mfma_f32_32x32x16_bf16: c += A(32x16) * B(16x32), fp32 accumulate.
__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// max / sum of x[lane] and x[lane ^ 32] with one v_permlane32_swap: the swap
// hands each half the other half's value in one of its two results.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// V^T fragment from a row-major V tile in LDS (rows of ROW_BYTES): two
// transposed 8-byte reads.  In each 16-lane group (h = lane/32 picks the key
// half, (lane/16)%2 the 16-row half of the d block) lane x supplies the
// address of 4 consecutive d of key 16kk + 4h + x/4 (+8 for the second
// read); lane j then holds those 4 keys' values at d = 32db + lane%32 -- the
// MFMA A-operand layout.
template <int ROW_BYTES>
__device__ __forceinline__ u32x4 vt_frag(const char* a) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 8 * ROW_BYTES));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

}  // namespace rgc
