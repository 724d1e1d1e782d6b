// decode.hip -- cached decode: one new query row per sequence against its
// bf16 KV cache.
//
// Operation (page "750美元从零训练3个LLM：一位开发者的实战复盘", sections V2
// and V3; page "从零手训LLaMa：125M模型11小时训练全记录", KV cache paragraph):
// the newest token's query attends over every cached key and value of its
// sequence, the query heads of a group sharing one KV head.
//
// HBM-bound (about 3 flop per cache byte).  Design:
//  * split-K over the cache length: a workgroup owns one (sequence, KV head,
//    head subgroup) and a chunk of 128 keys (256 at head dim 32), so a
//    ragged batch spreads over many workgroups of equal size; empty chunks of
//    short sequences exit at once;
//  * every K and V byte of the chunk is read exactly once, with 16-byte
//    loads that cover whole rows, and serves all the query heads of the
//    group (up to 4 per workgroup);
//  * all of a wave's loads are issued before any arithmetic;
//  * q.k uses packed bf16 dot products (v_dot2_f32_bf16) over a 4-lane key
//    layout that needs only two quad swizzles per key; the probabilities go
//    through LDS to a second layout in which each lane accumulates 8 output
//    elements of its keys, so p.V needs no per-key reduction;
//  * a chunk's partial (max, sum, unnormalised output) goes to the
//    workspace and a second, small kernel merges the chunks by max-rescaled
//    sums.  A sequence that fits in one chunk is finished by the first.
//    (Merging inside the first kernel, by the last chunk to arrive, would
//    need device-scope fences, and on gfx950 each of those writes back and
//    invalidates the XCD's L2: measured 16x slower than the second launch.)
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

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// Keys per wave and per workgroup (4 waves).  A wave covers at least one
// pass of the q.k layout (64 / (D / 32) keys).
template <int D>
struct Chunk {
  static constexpr int WAVE_KEYS = (64 / (D / 32)) > 32 ? (64 / (D / 32)) : 32;
  static constexpr int KEYS = 4 * WAVE_KEYS;
};
int chunk_keys(int D) { return D == 32 ? Chunk<32>::KEYS : D == 64 ? Chunk<64>::KEYS : Chunk<128>::KEYS; }

struct DecodeWs {
  float* part_o;    // [B][Hq][NS][D]  unnormalised partial outputs
  float* part_ml;   // [B][Hq][NS][2]  (max in log2 units, sum)
  int NS;
};

__device__ __forceinline__ bool len_ok(const AttnParams& p, int L) {
  const int lim = p.max_len < p.S_max ? p.max_len : p.S_max;
  return L >= 1 && L <= lim;
}

// D: head dim; GS: query heads per workgroup (all of them share KV head kvh).
template <int D, int GS>
__global__ void __launch_bounds__(256) decode_split_kernel(AttnParams p, DecodeWs ws, int nsub) {
  constexpr int WK = Chunk<D>::WAVE_KEYS;
  constexpr int LPK = D / 32;      // lanes per key in the q.k layout
  constexpr int KPP = 64 / LPK;    // keys per pass
  constexpr int PASSES = WK / KPP; // passes over the wave's keys
  constexpr int LPR = D / 8;       // lanes per row in the p.V layout
  constexpr int KPI = 64 / LPR;    // keys per load in the p.V layout
  constexpr int VLOADS = WK / KPI;

  __shared__ f32x4 p_lds[4][WK];
  __shared__ float o_lds[4][GS][D];
  __shared__ float ml_lds[4][GS][2];

  const int split = blockIdx.x;
  const int hs = blockIdx.y % nsub;
  const int kvh = blockIdx.y / nsub;
  const int b = blockIdx.z;
  const int group = p.Hq / p.Hkv;
  const int h0 = kvh * group + hs * GS;
  const int L = p.seq_lens[b];
  const int tid = threadIdx.x;

  if (!len_ok(p, L)) {
    if (split == 0) {
      for (int i = tid; i < GS * D; i += 256) {
        bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb + (int64_t)(h0 + i / D) * p.o_sh;
        orow[i % D] = 0x7FC0;  // NaN
      }
      if (tid < GS && p.lse) p.lse[(int64_t)b * p.Hq + h0 + tid] = __builtin_nanf("");
      if (tid == 0 && p.err) p.err[0] = 1;
    }
    return;
  }
  const int k0 = split * Chunk<D>::KEYS;
  if (k0 >= L) return;
  const int ns = (L + Chunk<D>::KEYS - 1) / Chunk<D>::KEYS;

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int kw = k0 + wave * WK;
  const float c = p.scale * kLog2e;

  const bf16_t* kbase = reinterpret_cast<const bf16_t*>(p.k) + (int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh;
  const bf16_t* vbase = reinterpret_cast<const bf16_t*>(p.v) + (int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh;

  float m_w[GS], l_w[GS], acc[GS][8];
#pragma unroll
  for (int g = 0; g < GS; ++g) {
    m_w[g] = -INFINITY;
    l_w[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }

  const bool active = kw < L;  // wave-uniform
  const int part = lane % LPK, key_sub = lane / LPK;
  const int dgrp = lane % LPR, kq = lane / LPR;
  if (active) {
    // ---- issue every load of the wave's keys ----
    u32x4 kf[PASSES][4], vf[VLOADS];
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int key = kw + ps * KPP + key_sub;
      const bf16_t* kr = kbase + (int64_t)key * p.kv_ss;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        kf[ps][i] = key < L ? ld16(kr + 8 * (part + LPK * i)) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int t = 0; t < VLOADS; ++t) {
      const int key = kw + t * KPI + kq;
      vf[t] = key < L ? ld16(vbase + (int64_t)key * p.kv_ss + 8 * dgrp) : u32x4{0, 0, 0, 0};
    }
    u32x4 qf[GS][4];
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      const bf16_t* qr = reinterpret_cast<const bf16_t*>(p.q) + (int64_t)b * p.q_sb + (int64_t)(h0 + g) * p.q_sh;
#pragma unroll
      for (int i = 0; i < 4; ++i) qf[g][i] = ld16(qr + 8 * (part + LPK * i));
    }

    // ---- scores: z = scale * log2(e) * q.k ----
    float z[GS][PASSES];
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const bool valid = kw + ps * KPP + key_sub < L;
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) d = dot2(qf[g][i][e], kf[ps][i][e], d);
        d = sum_within<LPK>(d);
        z[g][ps] = valid ? d * c : -INFINITY;
      }
    }
    // ---- softmax over the wave's keys (replicated across a key's lanes) ----
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      float mx = z[g][0];
#pragma unroll
      for (int ps = 1; ps < PASSES; ++ps) mx = fmaxf(mx, z[g][ps]);
      m_w[g] = max_above<LPK>(mx);
      float sm = 0.f;
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps) {
        z[g][ps] = exp2f(z[g][ps] - m_w[g]);
        sm += z[g][ps];
      }
      l_w[g] = sum_above<LPK>(sm);
    }
    if (part == 0) {
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps) {
        f32x4 pv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < GS; ++g) pv[g] = z[g][ps];
        p_lds[wave][ps * KPP + key_sub] = pv;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes landed
    __builtin_amdgcn_wave_barrier();
    // ---- p.V: lane owns d in [8*dgrp, 8*dgrp+8) for keys t*KPI + kq ----
#pragma unroll
    for (int t = 0; t < VLOADS; ++t) {
      const f32x4 pv = p_lds[wave][t * KPI + kq];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v0 = bf16_lo(vf[t][e]), v1 = bf16_hi(vf[t][e]);
#pragma unroll
        for (int g = 0; g < GS; ++g) {
          acc[g][2 * e] = fmaf(pv[g], v0, acc[g][2 * e]);
          acc[g][2 * e + 1] = fmaf(pv[g], v1, acc[g][2 * e + 1]);
        }
      }
    }
#pragma unroll
    for (int g = 0; g < GS; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = sum_above<LPR>(acc[g][e]);
  }
  // ---- merge the four waves ----
  if (lane < LPR) {
#pragma unroll
    for (int g = 0; g < GS; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) o_lds[wave][g][8 * lane + e] = acc[g][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      ml_lds[wave][g][0] = m_w[g];
      ml_lds[wave][g][1] = l_w[g];
    }
  }
  __syncthreads();
  for (int i = tid; i < GS * D; i += 256) {
    const int g = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, ml_lds[w][g][0]);
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = exp2f(ml_lds[w][g][0] - M);  // 0 for a wave without keys
      lsum = fmaf(ml_lds[w][g][1], f, lsum);
      o = fmaf(o_lds[w][g][d], f, o);
    }
    const int h = h0 + g;
    if (ns == 1) {
      bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh;
      orow[d] = f32_to_bf16(o / lsum);
      if (d == 0 && p.lse) p.lse[(int64_t)b * p.Hq + h] = (M + log2f(lsum)) * kLn2;
    } else {
      const int64_t slot = ((int64_t)b * p.Hq + h) * ws.NS + split;
      ws.part_o[slot * D + d] = o;
      if (d == 0) {
        ws.part_ml[slot * 2] = M;
        ws.part_ml[slot * 2 + 1] = lsum;
      }
    }
  }
}

// Merge the chunks of one (sequence, query head): max-rescaled sums.
template <int D>
__global__ void __launch_bounds__(D) decode_combine_kernel(AttnParams p, DecodeWs ws) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int L = p.seq_lens[b];
  if (!len_ok(p, L)) return;
  const int ns = (L + Chunk<D>::KEYS - 1) / Chunk<D>::KEYS;
  if (ns <= 1) return;
  const int64_t base = ((int64_t)b * p.Hq + h) * ws.NS;
  float M = -INFINITY;
  for (int c = 0; c < ns; ++c) M = fmaxf(M, ws.part_ml[(base + c) * 2]);
  float lsum = 0.f, o = 0.f;
  for (int c = 0; c < ns; ++c) {
    const float f = exp2f(ws.part_ml[(base + c) * 2] - M);
    lsum = fmaf(ws.part_ml[(base + c) * 2 + 1], f, lsum);
    o = fmaf(ws.part_o[(base + c) * D + d], f, o);
  }
  bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh;
  orow[d] = f32_to_bf16(o / lsum);
  if (d == 0 && p.lse) p.lse[(int64_t)b * p.Hq + h] = (M + log2f(lsum)) * kLn2;
}

int heads_per_wg(int group) {
  for (int gs = 4; gs >= 1; --gs)
    if (group % gs == 0) return gs;
  return 1;
}

template <int D>
hipError_t launch_d(const AttnParams& p, DecodeWs ws, hipStream_t stream) {
  const int group = p.Hq / p.Hkv;
  const int gs = heads_per_wg(group);
  const int nsub = group / gs;
  const dim3 grid(ws.NS, p.Hkv * nsub, p.B);
  switch (gs) {
    case 4: hipLaunchKernelGGL((decode_split_kernel<D, 4>), grid, dim3(256), 0, stream, p, ws, nsub); break;
    case 3: hipLaunchKernelGGL((decode_split_kernel<D, 3>), grid, dim3(256), 0, stream, p, ws, nsub); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<D, 2>), grid, dim3(256), 0, stream, p, ws, nsub); break;
    default: hipLaunchKernelGGL((decode_split_kernel<D, 1>), grid, dim3(256), 0, stream, p, ws, nsub); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ws.NS <= 1) return e;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(p.Hq, p.B), dim3(D), 0, stream, p, ws);
  return hipGetLastError();
}

}  // namespace

// Workspace: partial outputs, then partial (max, sum) pairs.
struct WsLayout {
  int NS;
  size_t o_bytes, ml_bytes;
};
WsLayout ws_layout(int B, int Hq, int D, int max_len) {
  WsLayout l;
  const int chunk = chunk_keys(D);
  l.NS = (max_len + chunk - 1) / chunk;
  const int64_t slots = (int64_t)B * Hq * l.NS;
  l.o_bytes = ((size_t)(slots * D * 4) + 255) & ~(size_t)255;
  l.ml_bytes = ((size_t)(slots * 2 * 4) + 255) & ~(size_t)255;
  return l;
}

size_t decode_workspace_bytes(int B, int Hq, int /*Hkv*/, int D, int max_len) {
  const WsLayout l = ws_layout(B, Hq, D, max_len);
  return l.o_bytes + l.ml_bytes;
}

hipError_t launch_decode_bf16(const AttnParams& p, void* workspace, hipStream_t stream) {
  const WsLayout l = ws_layout(p.B, p.Hq, p.D, p.max_len);
  DecodeWs ws;
  ws.NS = l.NS;
  char* base = reinterpret_cast<char*>(workspace);
  ws.part_o = reinterpret_cast<float*>(base);
  ws.part_ml = reinterpret_cast<float*>(base + l.o_bytes);
  switch (p.D) {
    case 32: return launch_d<32>(p, ws, stream);
    case 64: return launch_d<64>(p, ws, stream);
    default: return launch_d<128>(p, ws, stream);
  }
}

}  // namespace rgc
