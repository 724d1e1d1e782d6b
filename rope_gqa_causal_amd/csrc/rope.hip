// rope.hip -- rotary position embedding, in place, on q or k rows.
//
// Operation (page "750美元从零训练3个LLM：一位开发者的实战复盘", section V1;
// page "从零手训LLaMa：125M模型11小时训练全记录", core-architecture section):
// each pair of a head vector turns by position * theta_i.
//
// HBM-bound: every element is read once and written once.  A thread owns one
// token and a run of pairs, forms their angles once (fp64 product and
// reduction modulo 2*pi, fp32 sin/cos), and reuses them for all H heads of
// the token, so the transcendental work is amortised over the heads and the
// inner loop is two 16-byte loads, E rotations and two 16-byte stores.
#include "common.h"
#include "launch.h"

namespace rgc {
namespace {

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

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ float get(const u32x4& v, int e) {
    return __uint_as_float(v[e]);
  }
  static __device__ __forceinline__ void put(u32x4& v, const float* x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(x[e]);
  }
  static __device__ __forceinline__ float load1(const float* p) { return *p; }
  static __device__ __forceinline__ void store1(float* p, float x) { *p = x; }
};
template <>
struct Elem<bf16_t> {
  static __device__ __forceinline__ float get(const u32x4& v, int e) {
    return (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
  }
  static __device__ __forceinline__ void put(u32x4& v, const float* x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
  }
  static __device__ __forceinline__ float load1(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store1(bf16_t* p, float x) { *p = f32_to_bf16(x); }
};

// Vector path: a thread owns token (b, s) and pairs [c*E, c*E + E).
// Half style: the pairs' first members are x[c*E .. c*E+E) and the second
// members x[D/2 + c*E ..], one 16-byte load each.  Interleaved style: the
// pairs are the 2E contiguous elements x[2cE .. 2cE + 2E), two 16-byte loads.
template <typename T, int STYLE>
__global__ void __launch_bounds__(256) rope_vec_kernel(RopeParams p) {
  constexpr int E = 16 / sizeof(T);
  const int cpt = p.D / (2 * E);
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t ntok = (int64_t)p.B * p.S;
  if (gid >= ntok * cpt) return;
  const int c = (int)(gid % cpt);
  const int64_t tok = gid / cpt;
  const int s = (int)(tok % p.S);
  const int b = (int)(tok / p.S);
  const double pos = (double)((p.pos0 ? p.pos0[b] : 0) + s);

  float sn[E], cs[E];
#pragma unroll
  for (int e = 0; e < E; ++e) angle_sincos(pos * p.theta[c * E + e], &sn[e], &cs[e]);

  T* base = reinterpret_cast<T*>(p.x) + (int64_t)b * p.sb + (int64_t)s * p.ss;
  const int off0 = (STYLE == ROPE_HALF) ? c * E : 2 * c * E;
  const int off1 = (STYLE == ROPE_HALF) ? p.D / 2 + c * E : 2 * c * E + E;
  for (int h = 0; h < p.H; ++h) {
    T* row = base + (int64_t)h * p.sh;
    u32x4 v0 = ld16(row + off0);
    u32x4 v1 = ld16(row + off1);
    float a[E], bb[E], ra[E], rb[E];
    if (STYLE == ROPE_HALF) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        a[e] = Elem<T>::get(v0, e);
        bb[e] = Elem<T>::get(v1, e);
      }
    } else {
#pragma unroll
      for (int e = 0; e < E / 2; ++e) {
        a[e] = Elem<T>::get(v0, 2 * e);
        bb[e] = Elem<T>::get(v0, 2 * e + 1);
        a[E / 2 + e] = Elem<T>::get(v1, 2 * e);
        bb[E / 2 + e] = Elem<T>::get(v1, 2 * e + 1);
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      ra[e] = fmaf(a[e], cs[e], -bb[e] * sn[e]);
      rb[e] = fmaf(a[e], sn[e], bb[e] * cs[e]);
    }
    float w0[E], w1[E];
    if (STYLE == ROPE_HALF) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        w0[e] = ra[e];
        w1[e] = rb[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < E / 2; ++e) {
        w0[2 * e] = ra[e];
        w0[2 * e + 1] = rb[e];
        w1[2 * e] = ra[E / 2 + e];
        w1[2 * e + 1] = rb[E / 2 + e];
      }
    }
    Elem<T>::put(v0, w0);
    Elem<T>::put(v1, w1);
    st16(row + off0, v0);
    st16(row + off1, v1);
  }
}

// Scalar path for any even D and any element-aligned layout: a thread owns
// one pair of one token and walks the heads.
template <typename T, int STYLE>
__global__ void __launch_bounds__(256) rope_scalar_kernel(RopeParams p) {
  const int half = p.D / 2;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t ntok = (int64_t)p.B * p.S;
  if (gid >= ntok * half) return;
  const int i = (int)(gid % half);
  const int64_t tok = gid / half;
  const int s = (int)(tok % p.S);
  const int b = (int)(tok / p.S);
  const double pos = (double)((p.pos0 ? p.pos0[b] : 0) + s);
  float sn, cs;
  angle_sincos(pos * p.theta[i], &sn, &cs);
  const int ia = (STYLE == ROPE_HALF) ? i : 2 * i;
  const int ib = (STYLE == ROPE_HALF) ? i + half : 2 * i + 1;
  T* base = reinterpret_cast<T*>(p.x) + (int64_t)b * p.sb + (int64_t)s * p.ss;
  for (int h = 0; h < p.H; ++h) {
    T* row = base + (int64_t)h * p.sh;
    float a = Elem<T>::load1(row + ia), bb = Elem<T>::load1(row + ib);
    Elem<T>::store1(row + ia, fmaf(a, cs, -bb * sn));
    Elem<T>::store1(row + ib, fmaf(a, sn, bb * cs));
  }
}

template <typename T, int STYLE>
hipError_t launch_typed(const RopeParams& p, hipStream_t stream) {
  constexpr int E = 16 / sizeof(T);
  const int64_t ntok = (int64_t)p.B * p.S;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(p.x);
  const bool vec = (p.D % (2 * E) == 0) && (addr % 16 == 0) && (p.sb % E == 0) &&
                   (p.ss % E == 0) && (p.sh % E == 0);
  const int block = 256;
  if (vec) {
    const int64_t n = ntok * (p.D / (2 * E));
    hipLaunchKernelGGL((rope_vec_kernel<T, STYLE>), dim3((unsigned)((n + block - 1) / block)),
                       dim3(block), 0, stream, p);
  } else {
    const int64_t n = ntok * (p.D / 2);
    hipLaunchKernelGGL((rope_scalar_kernel<T, STYLE>), dim3((unsigned)((n + block - 1) / block)),
                       dim3(block), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(const RopeParams& p, int dtype, int style, hipStream_t stream) {
  if (dtype == DT_F32)
    return style == ROPE_HALF ? launch_typed<float, ROPE_HALF>(p, stream)
                              : launch_typed<float, ROPE_INTERLEAVED>(p, stream);
  return style == ROPE_HALF ? launch_typed<bf16_t, ROPE_HALF>(p, stream)
                            : launch_typed<bf16_t, ROPE_INTERLEAVED>(p, stream);
}

}  // namespace rgc
