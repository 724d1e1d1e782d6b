// rope_math.h -- the angle and the rotation of one RoPE pair, shared by the
// RoPE kernels and by the decode that rotates its new token itself, so both
// paths round identically.
//
// Operation (page "750美元从零训练3个LLM：一位开发者的实战复盘", section V1;
// page "从零手训LLaMa：125M模型11小时训练全记录", core-architecture section):
// pair i of a head vector at position p turns by the angle p * theta_i,
// theta_i = base^(-2i/D).
#pragma once
#include <hip/hip_runtime.h>

namespace rgc {

// sin and cos of a (possibly large) angle in radians.  The product
// position * theta and the reduction to [-pi, pi] run in fp64 with 2*pi
// split into a double and its rounding error, so the reduced angle is good
// to ~1e-16 absolute for any int32 position; fp32 sincosf then adds ~1 ulp.
__device__ __forceinline__ void angle_sincos(double ang, float* s, float* c) {
  const double kInv2Pi = 0.15915494309189535;
  const double k2PiHi = 6.283185307179586;          // nearest double to 2*pi
  const double k2PiLo = 2.4492935982947064e-16;     // 2*pi - k2PiHi
  double n = rint(ang * kInv2Pi);
  double r = fma(-n, k2PiHi, ang);
  r = fma(-n, k2PiLo, r);
  sincosf((float)r, s, c);
}

// The pair (a, b) turned by the angle whose sine and cosine are sn, cs.
__device__ __forceinline__ void rope_rotate_pair(float a, float b, float sn, float cs, float& ra, float& rb) {
  ra = fmaf(a, cs, -b * sn);
  rb = fmaf(a, sn, b * cs);
}

}  // namespace rgc
