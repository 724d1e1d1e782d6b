// rope.hip -- rotary position embedding on q or k rows, and the fused decode
// prologue (RoPE on q and k, then the cache append of k and v).
//
// Operation (page "750美元从零训练3个LLM：一位开发者的实战复盘", section V1;
// page "从零手训LLaMa：125M模型11小时训练全记录", core-architecture section):
// each pair of a head vector turns by position * theta_i.  The fused form
// follows the cached-generation step of the first page's section V3: the new
// token's q and k are rotated at its position, and its k and v join the cache.
//
// HBM-bound: every element is read once and written once.  A workgroup owns
// a few whole tokens: its threads first form the sin and cos of every pair
// of those tokens once (fp64 product and reduction modulo 2*pi, fp32
// sin/cos) into LDS, then walk (token, head, 16-byte chunk) units, so the
// transcendentals are shared by all heads and a decode step of few tokens
// still spreads over many threads.
#include "common.h"
#include "launch.h"
#include "rope_math.h"

namespace rgc {
namespace {

constexpr int kBlock = 256;
constexpr int kTableFloats = 1024;  // sin (and cos) entries per workgroup

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

// The E pairs of chunk c: half style takes x[cE..cE+E) with x[D/2+cE..],
// interleaved style the 2E contiguous elements x[2cE..2cE+2E).  Both are two
// 16-byte vectors at element offsets off0 and off1 of the row.
template <typename T, int STYLE>
struct Chunk {
  static constexpr int E = 16 / sizeof(T);
  int off0, off1;
  __device__ __forceinline__ Chunk(int c, int D)
      : off0(STYLE == ROPE_HALF ? c * E : 2 * c * E), off1(STYLE == ROPE_HALF ? D / 2 + c * E : 2 * c * E + E) {}

  // dst[off0, off1] = rotation of src[off0, off1] by the chunk's angles.
  // With NORM the head vector is first divided by sqrt(mean of squares +
  // eps): the cpt lanes that hold one row (adjacent, a power of two, aligned)
  // add their sums of squares with xor shuffles.
  template <bool NORM = false>
  __device__ __forceinline__ void rotate(const T* src, T* dst, const float* sn, const float* cs, int cpt = 1,
                                         float inv_d = 0.f, float eps = 0.f) const {
    u32x4 v0 = ld16(src + off0);
    u32x4 v1 = ld16(src + off1);
    float a[E], bb[E];
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
    if (NORM) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) ss = fmaf(a[e], a[e], fmaf(bb[e], bb[e], ss));
      for (int m = 1; m < cpt; m <<= 1) ss += __shfl_xor(ss, m, 64);
      const float r = 1.f / sqrtf(fmaf(ss, inv_d, eps));
#pragma unroll
      for (int e = 0; e < E; ++e) {
        a[e] *= r;
        bb[e] *= r;
      }
    }
    float w0[E], w1[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float ra, rb;
      rope_rotate_pair(a[e], bb[e], sn[e], cs[e], ra, rb);
      if (STYLE == ROPE_HALF) {
        w0[e] = ra;
        w1[e] = rb;
      } else {
        float* w = e < E / 2 ? w0 : w1;
        const int k = e < E / 2 ? e : e - E / 2;
        w[2 * k] = ra;
        w[2 * k + 1] = rb;
      }
    }
    Elem<T>::put(v0, w0);
    Elem<T>::put(v1, w1);
    st16(dst + off0, v0);
    st16(dst + off1, v1);
  }
  __device__ __forceinline__ void copy(const T* src, T* dst) const {
    st16(dst + off0, ld16(src + off0));
    st16(dst + off1, ld16(src + off1));
  }
};

// Sin and cos of pair i of the workgroup's tokens, tl-major, into LDS.
// sin_sign -1 turns by minus the angle: the gradient through RoPE.
__device__ __forceinline__ void token_table(const double* theta, const int32_t* pos0, int64_t tok0, int tpb,
                                            int64_t ntok, int S, int half, float sin_sign, float* sn, float* cs) {
  for (int t = threadIdx.x; t < tpb * half; t += kBlock) {
    const int tl = t / half, i = t % half;
    const int64_t tok = tok0 + tl;
    if (tok >= ntok) break;
    const int b = (int)(tok / S), s = (int)(tok % S);
    angle_sincos((double)((pos0 ? pos0[b] : 0) + s) * theta[i], &sn[t], &cs[t]);
    sn[t] *= sin_sign;
  }
  __syncthreads();
}

// Vector path of rgc_rope_apply: units (token, head, chunk) of tpb tokens.
template <typename T, int STYLE>
__global__ void __launch_bounds__(kBlock) rope_vec_kernel(RopeParams p, int tpb) {
  constexpr int E = 16 / sizeof(T);
  __shared__ float sn_t[kTableFloats], cs_t[kTableFloats];
  const int half = p.D / 2, cpt = p.D / (2 * E);
  const int64_t ntok = (int64_t)p.B * p.S, tok0 = (int64_t)blockIdx.x * tpb;
  token_table(p.theta, p.pos0, tok0, tpb, ntok, p.S, half, p.sin_sign, sn_t, cs_t);
  const int U = p.H * cpt;
  for (int u = threadIdx.x; u < tpb * U; u += kBlock) {
    const int tl = u / U, h = (u % U) / cpt, c = u % cpt;
    const int64_t tok = tok0 + tl;
    if (tok >= ntok) break;
    float sn[E], cs[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      sn[e] = sn_t[tl * half + c * E + e];
      cs[e] = cs_t[tl * half + c * E + e];
    }
    const int b = (int)(tok / p.S), s = (int)(tok % p.S);
    T* row = reinterpret_cast<T*>(p.x) + (int64_t)b * p.sb + (int64_t)s * p.ss + (int64_t)h * p.sh;
    Chunk<T, STYLE>(c, p.D).rotate(row, row, sn, cs);
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
  sn *= p.sin_sign;
  const int ia = (STYLE == ROPE_HALF) ? i : 2 * i;
  const int ib = (STYLE == ROPE_HALF) ? i + half : 2 * i + 1;
  T* base = reinterpret_cast<T*>(p.x) + (int64_t)b * p.sb + (int64_t)s * p.ss;
  for (int h = 0; h < p.H; ++h) {
    T* row = base + (int64_t)h * p.sh;
    float a = Elem<T>::load1(row + ia), bb = Elem<T>::load1(row + ib), ra, rb;
    rope_rotate_pair(a, bb, sn, cs, ra, rb);
    Elem<T>::store1(row + ia, ra);
    Elem<T>::store1(row + ib, rb);
  }
}

// Fused prologue: head slots [0, Hq) rotate q in place, [Hq, Hq+Hkv) rotate
// the new k into its cache slot, [Hq+Hkv, Hq+2Hkv) copy the new v into its
// cache slot.  With NORM, q and k head vectors are RMS-normalised first (QK
// norm: page "训练3.8B LLM至0.384 CORE，成本998美元 – Hugo Vergnes", section
// 设置; RMSNorm: page "从零手训LLaMa：125M模型11小时训练全记录",
// core-architecture section).  A cache slot outside [0, S_max) is skipped and
// flagged; q is still rotated.
template <typename T, int STYLE, bool NORM>
__global__ void __launch_bounds__(kBlock) rope_append_kernel(RopeAppendParams p, int tpb) {
  constexpr int E = 16 / sizeof(T);
  __shared__ float sn_t[kTableFloats], cs_t[kTableFloats];
  const int half = p.D / 2, cpt = p.D / (2 * E);
  const int64_t ntok = (int64_t)p.B * p.S, tok0 = (int64_t)blockIdx.x * tpb;
  token_table(p.theta, p.pos0, tok0, tpb, ntok, p.S, half, 1.f, sn_t, cs_t);
  const int U = (p.Hq + 2 * p.Hkv) * cpt;
  for (int u = threadIdx.x; u < tpb * U; u += kBlock) {
    const int tl = u / U, h = (u % U) / cpt, c = u % cpt;
    const int64_t tok = tok0 + tl;
    if (tok >= ntok) break;
    const int b = (int)(tok / p.S), s = (int)(tok % p.S);
    const int64_t slot = (int64_t)(p.pos0 ? p.pos0[b] : 0) + s;
    const Chunk<T, STYLE> ch(c, p.D);
    if (h >= p.Hq && !(slot >= 0 && slot < p.S_max)) {
      if (p.err && h == p.Hq && c == 0) p.err[0] = 1;
      continue;
    }
    if (h >= p.Hq + p.Hkv) {
      const int vh = h - p.Hq - p.Hkv;
      ch.copy(reinterpret_cast<const T*>(p.v_new) + (int64_t)b * p.n_sb + (int64_t)s * p.n_ss + (int64_t)vh * p.n_sh,
              reinterpret_cast<T*>(p.v_cache) + (int64_t)b * p.c_sb + (int64_t)vh * p.c_sh + slot * p.c_ss);
      continue;
    }
    float sn[E], cs[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      sn[e] = sn_t[tl * half + c * E + e];
      cs[e] = cs_t[tl * half + c * E + e];
    }
    const float inv_d = 1.f / (float)p.D;
    if (h < p.Hq) {
      T* row = reinterpret_cast<T*>(p.q) + (int64_t)b * p.q_sb + (int64_t)s * p.q_ss + (int64_t)h * p.q_sh;
      ch.template rotate<NORM>(row, row, sn, cs, cpt, inv_d, p.eps);
    } else {
      const int kh = h - p.Hq;
      ch.template rotate<NORM>(
          reinterpret_cast<const T*>(p.k_new) + (int64_t)b * p.n_sb + (int64_t)s * p.n_ss + (int64_t)kh * p.n_sh,
          reinterpret_cast<T*>(p.k_cache) + (int64_t)b * p.c_sb + (int64_t)kh * p.c_sh + slot * p.c_ss, sn, cs, cpt,
          inv_d, p.eps);
    }
  }
}

// Tokens per workgroup: enough (token, head, chunk) units for the 256
// threads, within the LDS table.
int tokens_per_block(int units_per_token, int D) {
  int t = kBlock / (units_per_token > 0 ? units_per_token : 1);
  const int cap = kTableFloats / (D / 2);
  if (t > cap) t = cap;
  return t < 1 ? 1 : t;
}

template <typename T, int STYLE>
hipError_t launch_typed(const RopeParams& p, hipStream_t stream) {
  constexpr int E = 16 / sizeof(T);
  const int64_t ntok = (int64_t)p.B * p.S;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(p.x);
  const bool vec = (p.D % (2 * E) == 0) && (addr % 16 == 0) && (p.sb % E == 0) &&
                   (p.ss % E == 0) && (p.sh % E == 0);
  const int block = 256;
  KernelTimer kt_(vec ? "rope_vec_kernel" : "rope_scalar_kernel", stream);
  if (vec) {
    const int tpb = tokens_per_block(p.H * (p.D / (2 * E)), p.D);
    hipLaunchKernelGGL((rope_vec_kernel<T, STYLE>), dim3((unsigned)((ntok + tpb - 1) / tpb)), dim3(kBlock), 0,
                       stream, p, tpb);
  } else {
    const int64_t n = ntok * (p.D / 2);
    hipLaunchKernelGGL((rope_scalar_kernel<T, STYLE>), dim3((unsigned)((n + block - 1) / block)),
                       dim3(block), 0, stream, p);
  }
  return hipGetLastError();
}

template <typename T, int STYLE>
hipError_t launch_append_typed(const RopeAppendParams& p, bool norm, hipStream_t stream) {
  constexpr int E = 16 / sizeof(T);
  const int64_t ntok = (int64_t)p.B * p.S;
  const int tpb = tokens_per_block((p.Hq + 2 * p.Hkv) * (p.D / (2 * E)), p.D);
  const dim3 grid((unsigned)((ntok + tpb - 1) / tpb));
  KernelTimer kt_("rope_append_kernel", stream);
  if (norm)
    hipLaunchKernelGGL((rope_append_kernel<T, STYLE, true>), grid, dim3(kBlock), 0, stream, p, tpb);
  else
    hipLaunchKernelGGL((rope_append_kernel<T, STYLE, false>), grid, dim3(kBlock), 0, stream, p, tpb);
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

hipError_t launch_rope_append(const RopeAppendParams& p, int dtype, int style, bool norm, hipStream_t stream) {
  if (dtype == DT_F32)
    return style == ROPE_HALF ? launch_append_typed<float, ROPE_HALF>(p, norm, stream)
                              : launch_append_typed<float, ROPE_INTERLEAVED>(p, norm, stream);
  return style == ROPE_HALF ? launch_append_typed<bf16_t, ROPE_HALF>(p, norm, stream)
                            : launch_append_typed<bf16_t, ROPE_INTERLEAVED>(p, norm, stream);
}

}  // namespace rgc
