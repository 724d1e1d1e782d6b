// decode_lanes.h -- lane-level helpers shared by the decode kernels
// (decode.hip, decode_stream.hip): DPP and shuffle reductions over the
// lanes of a wave, the packed bf16 dot product, and the length check.
#pragma once

#include "common.h"
#include "launch.h"

namespace rgc {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the lanes that differ in the bits of [lo, 64): xor partners lo,
// 2lo, ..., 32.  Within a 16-lane row quad swizzles and row rotations (DPP)
// are used; across rows, LDS-free lane shuffles.
template <int LO>
__device__ __forceinline__ float sum_above(float x) {
  if (LO <= 1) x += dpp<0xB1>(x);          // quad_perm [1,0,3,2]
  if (LO <= 2) x += dpp<0x4E>(x);          // quad_perm [2,3,0,1]
  if (LO <= 4) x += dpp<0x124>(x);         // row_ror:4
  if (LO <= 8) x += dpp<0x128>(x);         // row_ror:8
  if (LO <= 16) x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}
template <int LO>
__device__ __forceinline__ float max_above(float x) {
  if (LO <= 1) x = fmaxf(x, dpp<0xB1>(x));
  if (LO <= 2) x = fmaxf(x, dpp<0x4E>(x));
  if (LO <= 4) x = fmaxf(x, dpp<0x124>(x));
  if (LO <= 8) x = fmaxf(x, dpp<0x128>(x));
  if (LO <= 16) x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}
// Sum over the lanes of one LPK-lane key group (xor 1 [, 2]).
template <int LPK>
__device__ __forceinline__ float sum_within(float x) {
  if (LPK >= 2) x += dpp<0xB1>(x);
  if (LPK >= 4) x += dpp<0x4E>(x);
  return x;
}

// Sum over the LPR lanes of one row group (lanes that differ in the bits
// below LPR: xor 1, 2, 4, 8 within a 16-lane row, xor 16, 32 across).
template <int LPR>
__device__ __forceinline__ float sum_within_row(float x) {
  if (LPR >= 2) x += dpp<0xB1>(x);                // quad_perm [1,0,3,2]
  if (LPR >= 4) x += dpp<0x4E>(x);                // quad_perm [2,3,0,1]
  if (LPR >= 8) x += dpp<0x141>(x);               // row_half_mirror
  if (LPR >= 16) x += dpp<0x140>(x);              // row_mirror
  if (LPR >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ bool len_ok(const AttnParams& p, int L) {
  const int lim = p.max_len < p.S_max ? p.max_len : p.S_max;
  return L >= 1 && L <= lim;
}

}  // namespace
}  // namespace rgc
