// rope.hip -- rotary position embedding on q or k rows, and the fused decode
// prologue (RoPE on q and k, then the cache append of k and v).
//
// Operation (page "750美元从零训练3个LLM：一位开发者的实战复盘", section V1;
// page "从零手训LLaMa：125M模型11小时训练全记录", core-architecture section):
// each pair of a head vector turns by position * theta_i.  The fused form
// follows the cached-generation step of the first page's section V3: the new
// token's q and k are rotated at its position, and its k and v join the cache.
//
// HBM-bound: every element is read once and written once.  A thread owns one
// token, a run of E pairs (one 16-byte vector per half-row) and a group of
// heads: it forms the E angles once (fp64 product and reduction modulo 2*pi,
// fp32 sin/cos) and reuses them for every head of its group.  The number of
// head groups is chosen per call so that a batch of few tokens (one decode
// step) still spreads over enough threads, while a long prefill keeps whole
// heads per thread and amortises the transcendentals over all of them.
#include "common.h"
#include "launch.h"

namespace rgc {
namespace {

constexpr int kTargetThreads = 1 << 16;

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
  __device__ __forceinline__ void rotate(const T* src, T* dst, const float* sn, const float* cs) const {
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
    float w0[E], w1[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float ra = fmaf(a[e], cs[e], -bb[e] * sn[e]);
      const float rb = fmaf(a[e], sn[e], bb[e] * cs[e]);
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

// Split a flat thread index into (token, chunk, head group).
struct Work {
  int b, s, c, g;
  __device__ __forceinline__ Work(int64_t gid, int S, int cpt, int ngroups) {
    g = (int)(gid % ngroups);
    const int64_t t = gid / ngroups;
    c = (int)(t % cpt);
    const int64_t tok = t / cpt;
    s = (int)(tok % S);
    b = (int)(tok / S);
  }
};

template <typename T, int STYLE>
__device__ __forceinline__ void chunk_angles(const double* theta, double pos, int c, float* sn, float* cs) {
  constexpr int E = 16 / sizeof(T);
#pragma unroll
  for (int e = 0; e < E; ++e) angle_sincos(pos * theta[c * E + e], &sn[e], &cs[e]);
}

// Vector path of rgc_rope_apply.
template <typename T, int STYLE>
__global__ void __launch_bounds__(256) rope_vec_kernel(RopeParams p, int ngroups) {
  constexpr int E = 16 / sizeof(T);
  const int cpt = p.D / (2 * E);
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)p.B * p.S * cpt * ngroups) return;
  const Work w(gid, p.S, cpt, ngroups);
  const int hpg = (p.H + ngroups - 1) / ngroups;
  const int h0 = w.g * hpg, h1 = min(p.H, h0 + hpg);
  if (h0 >= h1) return;
  float sn[E], cs[E];
  chunk_angles<T, STYLE>(p.theta, (double)((p.pos0 ? p.pos0[w.b] : 0) + w.s), w.c, sn, cs);
  const Chunk<T, STYLE> ch(w.c, p.D);
  T* base = reinterpret_cast<T*>(p.x) + (int64_t)w.b * p.sb + (int64_t)w.s * p.ss;
  for (int h = h0; h < h1; ++h) {
    T* row = base + (int64_t)h * p.sh;
    ch.rotate(row, row, sn, cs);
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

// Fused prologue: head slots [0, Hq) rotate q in place, [Hq, Hq+Hkv) rotate
// the new k into its cache slot, [Hq+Hkv, Hq+2Hkv) copy the new v into its
// cache slot.  A cache slot outside [0, S_max) is skipped and flagged; q is
// still rotated.
template <typename T, int STYLE>
__global__ void __launch_bounds__(256) rope_append_kernel(RopeAppendParams p, int ngroups) {
  constexpr int E = 16 / sizeof(T);
  const int cpt = p.D / (2 * E);
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)p.B * p.S * cpt * ngroups) return;
  const Work w(gid, p.S, cpt, ngroups);
  const int nslots = p.Hq + 2 * p.Hkv;
  const int hpg = (nslots + ngroups - 1) / ngroups;
  const int h0 = w.g * hpg, h1 = min(nslots, h0 + hpg);
  if (h0 >= h1) return;
  const int64_t slot = (int64_t)p.pos0[w.b] + w.s;
  const bool in_cache = slot >= 0 && slot < p.S_max;
  if (!in_cache && p.err && w.c == 0 && h1 > p.Hq) p.err[0] = 1;
  float sn[E], cs[E];
  chunk_angles<T, STYLE>(p.theta, (double)slot, w.c, sn, cs);
  const Chunk<T, STYLE> ch(w.c, p.D);
  T* qb = reinterpret_cast<T*>(p.q) + (int64_t)w.b * p.q_sb + (int64_t)w.s * p.q_ss;
  const T* kb = reinterpret_cast<const T*>(p.k_new) + (int64_t)w.b * p.n_sb + (int64_t)w.s * p.n_ss;
  const T* vb = reinterpret_cast<const T*>(p.v_new) + (int64_t)w.b * p.n_sb + (int64_t)w.s * p.n_ss;
  T* kc = reinterpret_cast<T*>(p.k_cache) + (int64_t)w.b * p.c_sb + slot * p.c_ss;
  T* vc = reinterpret_cast<T*>(p.v_cache) + (int64_t)w.b * p.c_sb + slot * p.c_ss;
  for (int h = h0; h < h1; ++h) {
    if (h < p.Hq) {
      T* row = qb + (int64_t)h * p.q_sh;
      ch.rotate(row, row, sn, cs);
    } else if (!in_cache) {
      break;
    } else if (h < p.Hq + p.Hkv) {
      const int kh = h - p.Hq;
      ch.rotate(kb + (int64_t)kh * p.n_sh, kc + (int64_t)kh * p.c_sh, sn, cs);
    } else {
      const int vh = h - p.Hq - p.Hkv;
      ch.copy(vb + (int64_t)vh * p.n_sh, vc + (int64_t)vh * p.c_sh);
    }
  }
}

// Head groups per (token, chunk): enough threads to fill the GPU, whole
// heads otherwise.
int head_groups(int64_t token_chunks, int heads) {
  int64_t g = (kTargetThreads + token_chunks - 1) / token_chunks;
  if (g > heads) g = heads;
  return g < 1 ? 1 : (int)g;
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
    const int64_t tc = ntok * (p.D / (2 * E));
    const int ng = head_groups(tc, p.H);
    const int64_t n = tc * ng;
    hipLaunchKernelGGL((rope_vec_kernel<T, STYLE>), dim3((unsigned)((n + block - 1) / block)),
                       dim3(block), 0, stream, p, ng);
  } else {
    const int64_t n = ntok * (p.D / 2);
    hipLaunchKernelGGL((rope_scalar_kernel<T, STYLE>), dim3((unsigned)((n + block - 1) / block)),
                       dim3(block), 0, stream, p);
  }
  return hipGetLastError();
}

template <typename T, int STYLE>
hipError_t launch_append_typed(const RopeAppendParams& p, hipStream_t stream) {
  constexpr int E = 16 / sizeof(T);
  const int64_t tc = (int64_t)p.B * p.S * (p.D / (2 * E));
  const int ng = head_groups(tc, p.Hq + 2 * p.Hkv);
  const int64_t n = tc * ng;
  const int block = 256;
  hipLaunchKernelGGL((rope_append_kernel<T, STYLE>), dim3((unsigned)((n + block - 1) / block)),
                     dim3(block), 0, stream, p, ng);
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

hipError_t launch_rope_append(const RopeAppendParams& p, int dtype, int style, hipStream_t stream) {
  if (dtype == DT_F32)
    return style == ROPE_HALF ? launch_append_typed<float, ROPE_HALF>(p, stream)
                              : launch_append_typed<float, ROPE_INTERLEAVED>(p, stream);
  return style == ROPE_HALF ? launch_append_typed<bf16_t, ROPE_HALF>(p, stream)
                            : launch_append_typed<bf16_t, ROPE_INTERLEAVED>(p, stream);
}

}  // namespace rgc
