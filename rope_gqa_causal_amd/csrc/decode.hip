// decode.hip -- cached decode: one new query row per sequence against its
// bf16 KV cache.
//
// Operation (page "750美元从零训练3个LLM：一位开发者的实战复盘", sections V2
// and V3; page "从零手训LLaMa：125M模型11小时训练全记录", KV cache paragraph):
// the newest token's query attends over every cached key and value of its
// sequence, the query heads of a group sharing one KV head.
//
// HBM-bound (about 3 flop per cache byte).  Design:
//  * split-K over the cache length: a workgroup of four waves owns one
//    (sequence, KV head, head subgroup) and a chunk of 4 x 64 keys (4 x 32
//    when the batch is too small to fill the chip that way), so a ragged
//    batch spreads over many workgroups of equal size; empty chunks of short
//    sequences exit at once;
//  * every K and V byte of the chunk is read exactly once, with 16-byte
//    loads, and serves all the query heads of the group (up to 4 per
//    workgroup);
//  * every load of a wave is unconditional: keys past the end re-read the
//    last row and are masked in the scores.  (A guarded load per key makes
//    the compiler wait for all earlier loads at each guard, which
//    serialises the wave's memory traffic.)  The K rows of all the wave's
//    keys go out before any arithmetic; the V rows of a q.k pass's keys go
//    out right after that pass's scores, into the registers its K rows
//    leave free, so K and V never hold separate register sets and three
//    workgroups fit a compute unit (two when all loads went out first:
//    6 % slower per call on the ragged batch);
//  * q.k uses packed bf16 dot products (v_dot2_f32_bf16) over a 4-lane key
//    layout that needs only two quad swizzles per key; the probabilities go
//    through LDS to a second layout in which each lane accumulates 8 output
//    elements of its keys; there two keys' values of one element are paired
//    by a byte permute and meet their two probabilities (rounded to bf16) in
//    one packed dot product.  The key lanes are summed in the LDS merge of
//    the four waves;
//  * a chunk's partial (max, sum, unnormalised output) goes to the
//    workspace and a second, small kernel merges the chunks by max-rescaled
//    sums.  A sequence that fits in one chunk is finished by the first;
//  * a grid too small to fill the chip this way (a few sequences, as in
//    batch-1 generation) takes a third kernel instead: one 12-wave
//    workgroup per (sequence, query head) walks the whole sequence in at
//    most two passes and writes the final row, so the step is one launch.
//    (Merging inside the first kernel, by the last chunk to arrive, would
//    need device-scope fences, and on gfx950 each of those writes back and
//    invalidates the XCD's L2: measured 16x slower than the second launch.)
#include <mutex>

#include "common.h"
#include "launch.h"
#include "rope_math.h"
#include "decode_lanes.h"

namespace rgc {
namespace {

// Keys per wave and per workgroup (4 waves).  A wave covers at least one
// pass of the q.k layout (64 / (D / 32) keys), times MUL.
constexpr int kWaves = 4;
template <int D, int MUL>
struct Chunk {
  static constexpr int WAVE_KEYS = ((64 / (D / 32)) > 32 ? (64 / (D / 32)) : 32) * MUL;
  static constexpr int KEYS = kWaves * WAVE_KEYS;
};
int chunk_keys(int D, int mul) {
  const int wave_keys = (D == 32 ? 64 : 32) * mul;
  return kWaves * wave_keys;
}

struct DecodeWs {
  float* part_o;    // [B][Hq][NS][D]  unnormalised partial outputs
  float* part_ml;   // [B][Hq][NS][2]  (max in log2 units, sum)
  int NS;           // chunks of the longest sequence
  int chunk;        // keys per chunk
};


// D: head dim; GS: query heads per workgroup (all of them share KV head kvh);
// MUL: keys per wave in units of one q.k pass.  ROPE: the new token's RoPE
// and append happen here (DecodeRope): every workgroup turns its q rows at
// position L - 1; the sequence's last chunk, the only one that holds slot
// L - 1, takes the new token's rotated k and its v from registers instead
// of the cache, and its first head subgroup writes them into the caches (no
// workgroup reads that slot from memory, so the write races with nothing).
template <int D, int GS, int MUL, bool ROPE>
__global__ void __launch_bounds__(64 * kWaves) decode_split_kernel(AttnParams p, DecodeWs ws, int nsub,
                                                                   DecodeRope r) {
  constexpr int WK = Chunk<D, MUL>::WAVE_KEYS;
  constexpr int LPK = D / 32;      // lanes per key in the q.k layout
  constexpr int KPP = 64 / LPK;    // keys per pass
  constexpr int PASSES = WK / KPP; // passes over the wave's keys
  constexpr int LPR = D / 8;       // lanes per row in the p.V layout
  constexpr int KPI = 64 / LPR;    // keys per load in the p.V layout
  constexpr int VLOADS = WK / KPI;

  __shared__ f32x4 p_lds[kWaves][WK];
  __shared__ float o_lds[kWaves][KPI][GS][D];
  __shared__ float ml_lds[kWaves][GS][2];

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
      for (int i = tid; i < GS * D; i += 64 * kWaves) {
        bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb + (int64_t)(h0 + i / D) * p.o_sh;
        orow[i % D] = 0x7FC0;  // NaN
      }
      if (tid < GS && p.lse) p.lse[(int64_t)b * p.Hq + h0 + tid] = __builtin_nanf("");
      if (tid == 0 && p.err) p.err[0] = 1;
    }
    return;
  }
  const int k0 = split * Chunk<D, MUL>::KEYS;
  if (k0 >= L) return;
  const int ns = (L + Chunk<D, MUL>::KEYS - 1) / Chunk<D, MUL>::KEYS;

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
  const bool last = split == ns - 1;  // the chunk that holds slot L - 1
  if (active) {
    // ---- issue every load of the wave's keys (q first: the scores need it
    // before the values).  Keys past the end re-read the last row, which
    // keeps every load unconditional and in bounds; their scores are masked
    // to -inf, so they weigh nothing.
    u32x4 qf[GS][4];
    // With ROPE, lane m < D/2 instead loads pair m (elements ia, ib) of each
    // q row and of the new k (and every lane its piece of the new v); it
    // turns them below and the rows reach the q.k layout through LDS.  These
    // loads, and the lane's theta, go out first and unconditionally (lanes
    // past D/2 read pair 0 and ignore it), and their values are only used
    // after the K and V loads are issued: a wait for them then never waits
    // for K or V.
    constexpr int HALF = D / 2;
    const int lm = lane < HALF ? lane : 0;
    const int ia = r.style == ROPE_HALF ? lm : 2 * lm, ib = r.style == ROPE_HALF ? lm + HALF : 2 * lm + 1;
    bf16_t qa[GS + 1], qb[GS + 1];
    double theta = 0.0;
    u32x4 kn[4] = {}, vn = {};  // the new token's rotated k and its v (last chunk)
    if constexpr (ROPE) {
      theta = r.theta[lm];
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        const bf16_t* qr = reinterpret_cast<const bf16_t*>(p.q) + (int64_t)b * p.q_sb + (int64_t)(h0 + g) * p.q_sh;
        qa[g] = qr[ia];
        qb[g] = qr[ib];
      }
      const bf16_t* knr = reinterpret_cast<const bf16_t*>(r.k_new) + (int64_t)b * r.n_sb + (int64_t)kvh * r.n_sh;
      qa[GS] = knr[ia];
      qb[GS] = knr[ib];
      vn = ld16(reinterpret_cast<const bf16_t*>(r.v_new) + (int64_t)b * r.n_sb + (int64_t)kvh * r.n_sh + 8 * dgrp);
    } else {
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        const bf16_t* qr = reinterpret_cast<const bf16_t*>(p.q) + (int64_t)b * p.q_sb + (int64_t)(h0 + g) * p.q_sh;
#pragma unroll
        for (int i = 0; i < 4; ++i) qf[g][i] = ld16(qr + 8 * (part + LPK * i));
      }
    }
    u32x4 kf[PASSES][4], vf[VLOADS];
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int key = min(kw + ps * KPP + key_sub, L - 1);
      const bf16_t* kr = kbase + (int64_t)key * p.kv_ss;
#pragma unroll
      for (int i = 0; i < 4; ++i) kf[ps][i] = ld16_nt(kr + 8 * (part + LPK * i));
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the K loads ahead of the arithmetic

    if constexpr (ROPE) {
      // Pair m = lane turns by (L - 1) theta_m (same angle, rotation and
      // rounding as the RoPE kernels); the rotated rows go through this
      // wave's LDS rows into the q.k layout.
      __shared__ __attribute__((aligned(16))) bf16_t rows[kWaves][GS + 1][D];
      if (lane < HALF) {
        float sn, cs;
        angle_sincos((double)(L - 1) * theta, &sn, &cs);
#pragma unroll
        for (int g = 0; g <= GS; ++g) {
          if (g == GS && !last) break;
          float ra, rb;
          rope_rotate_pair(bf16_to_f32(qa[g]), bf16_to_f32(qb[g]), sn, cs, ra, rb);
          rows[wave][g][ia] = f32_to_bf16(ra);
          rows[wave][g][ib] = f32_to_bf16(rb);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's rows landed
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int g = 0; g < GS; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) qf[g][i] = *reinterpret_cast<const u32x4*>(&rows[wave][g][8 * (part + LPK * i)]);
      if (last) {
#pragma unroll
        for (int i = 0; i < 4; ++i) kn[i] = *reinterpret_cast<const u32x4*>(&rows[wave][GS][8 * (part + LPK * i)]);
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps)
          if (min(kw + ps * KPP + key_sub, L - 1) == L - 1)
#pragma unroll
            for (int i = 0; i < 4; ++i) kf[ps][i] = kn[i];
        if (hs == 0) {
          bf16_t* kc = reinterpret_cast<bf16_t*>(r.k_cache) + (int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh +
                       (int64_t)(L - 1) * p.kv_ss;
          bf16_t* vc = reinterpret_cast<bf16_t*>(r.v_cache) + (int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh +
                       (int64_t)(L - 1) * p.kv_ss;
#pragma unroll
          for (int ps = 0; ps < PASSES; ++ps)
            if (kw + ps * KPP + key_sub == L - 1)
#pragma unroll
              for (int i = 0; i < 4; ++i) st16(kc + 8 * (part + LPK * i), kn[i]);
#pragma unroll
          for (int t = 0; t < VLOADS; ++t)
            if (kw + t * KPI + kq == L - 1) st16(vc + 8 * dgrp, vn);
        }
      }
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
      // This pass's keys' V rows, into the registers its K rows leave free
      // (so K and V never hold separate register sets: three workgroups
      // fit a compute unit).
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = ps * (VLOADS / PASSES); t < (ps + 1) * (VLOADS / PASSES); ++t) {
        const int key = min(kw + t * KPI + kq, L - 1);
        vf[t] = ld16_nt(vbase + (int64_t)key * p.kv_ss + 8 * dgrp);
      }
      __builtin_amdgcn_sched_barrier(0);
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
    // ---- p.V: lane owns d in [8*dgrp, 8*dgrp+8) for keys t*KPI + kq.
    // Two keys at a time: their values of one d side by side in a bf16
    // pair (one byte permute) meet the pair of their probabilities in one
    // packed dot product.
#pragma unroll
    for (int t = 0; t < VLOADS; t += 2) {
      const f32x4 pa = p_lds[wave][t * KPI + kq];
      const f32x4 pb = p_lds[wave][(t + 1) * KPI + kq];
      uint32_t pp[GS];
#pragma unroll
      for (int g = 0; g < GS; ++g) pp[g] = pack_bf16x2(pa[g], pb[g]);
      u32x4 va = vf[t], vb = vf[t + 1];
      if constexpr (ROPE) {
        if (last) {  // the new token's v for slot L - 1 (the cache slot is not written yet)
          if (min(kw + t * KPI + kq, L - 1) == L - 1) va = vn;
          if (min(kw + (t + 1) * KPI + kq, L - 1) == L - 1) vb = vn;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = __builtin_amdgcn_perm(vb[e], va[e], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(vb[e], va[e], 0x07060302u);
#pragma unroll
        for (int g = 0; g < GS; ++g) {
          acc[g][2 * e] = dot2(pp[g], lo, acc[g][2 * e]);
          acc[g][2 * e + 1] = dot2(pp[g], hi, acc[g][2 * e + 1]);
        }
      }
    }
  }
  // ---- merge the four waves and their KPI key lanes ----
#pragma unroll
  for (int g = 0; g < GS; ++g) {
    *reinterpret_cast<f32x4*>(&o_lds[wave][kq][g][8 * dgrp]) = f32x4{acc[g][0], acc[g][1], acc[g][2], acc[g][3]};
    *reinterpret_cast<f32x4*>(&o_lds[wave][kq][g][8 * dgrp + 4]) = f32x4{acc[g][4], acc[g][5], acc[g][6], acc[g][7]};
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      ml_lds[wave][g][0] = m_w[g];
      ml_lds[wave][g][1] = l_w[g];
    }
  }
  __syncthreads();
  for (int i = tid; i < GS * D; i += 64 * kWaves) {
    const int g = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ml_lds[w][g][0]);
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = exp2f(ml_lds[w][g][0] - M);  // 0 for a wave without keys
      lsum = fmaf(ml_lds[w][g][1], f, lsum);
      float ow = 0.f;
#pragma unroll
      for (int k = 0; k < KPI; ++k) ow += o_lds[w][k][g][d];
      o = fmaf(ow, f, o);
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

// Small grids: one workgroup of W waves per (sequence, KV head, head
// subgroup) covers W x WK keys per pass and walks the whole sequence.  q is
// loaded (with ROPE: loaded and turned) once; every wave carries its running
// max, sum and output across passes, rescaled when the max rises.  The W
// waves then merge in LDS and write the final row: no partials and no merge
// launch.  Used where the split kernel's chunks could not fill the chip
// anyway (a few sequences, as in batch-1 generation), so its second launch
// would dominate the step.  With 12 waves one pass covers 384, 768 or 1536
// keys at head dim 128, 64 or 32.
template <int D, int GS, int MUL, bool ROPE, int W>
__global__ void __launch_bounds__(64 * W) decode_loop_kernel(AttnParams p, int nsub, DecodeRope r) {
  constexpr int WK = Chunk<D, MUL>::WAVE_KEYS;
  constexpr int KEYS = W * WK;
  constexpr int LPK = D / 32;      // lanes per key in the q.k layout
  constexpr int KPP = 64 / LPK;    // keys per pass
  constexpr int PASSES = WK / KPP; // passes over the wave's keys
  constexpr int LPR = D / 8;       // lanes per row in the p.V layout
  constexpr int KPI = 64 / LPR;    // keys per load in the p.V layout
  constexpr int VLOADS = WK / KPI;
  constexpr int HALF = D / 2;

  __shared__ f32x4 p_lds[W][WK];
  __shared__ float o_lds[W][GS][D];
  __shared__ float ml_lds[W][GS][2];
  // With ROPE: each wave's turned q rows and the new token's turned k row.
  __shared__ __attribute__((aligned(16))) bf16_t rows[ROPE ? W : 1][GS + 1][D];

  const int hs = blockIdx.y % nsub;
  const int kvh = blockIdx.y / nsub;
  const int b = blockIdx.z;
  const int group = p.Hq / p.Hkv;
  const int h0 = kvh * group + hs * GS;
  const int L = p.seq_lens[b];
  const int tid = threadIdx.x;
  if (!len_ok(p, L)) {
    for (int i = tid; i < GS * D; i += 64 * W) {
      bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb + (int64_t)(h0 + i / D) * p.o_sh;
      orow[i % D] = 0x7FC0;  // NaN
    }
    if (tid < GS && p.lse) p.lse[(int64_t)b * p.Hq + h0 + tid] = __builtin_nanf("");
    if (tid == 0 && p.err) p.err[0] = 1;
    return;
  }
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const float c = p.scale * kLog2e;
  const bf16_t* kbase = reinterpret_cast<const bf16_t*>(p.k) + (int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh;
  const bf16_t* vbase = reinterpret_cast<const bf16_t*>(p.v) + (int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh;
  const int part = lane % LPK, key_sub = lane / LPK;
  const int dgrp = lane % LPR, kq = lane / LPR;

  float m_w[GS], l_w[GS], acc[GS][8];
#pragma unroll
  for (int g = 0; g < GS; ++g) {
    m_w[g] = -INFINITY;
    l_w[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }

  // Every load is unconditional: keys past the end re-read the last row and
  // are masked in the scores.  Plain (temporal) loads: this kernel serves
  // small batches, whose caches a generation reads again at every step and
  // which the L2 and the MALL hold between steps.
  auto load = [&](u32x4 (&kf)[PASSES][4], u32x4 (&vf)[VLOADS], int kw) {
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int key = min(kw + ps * KPP + key_sub, L - 1);
      const bf16_t* kr = kbase + (int64_t)key * p.kv_ss;
#pragma unroll
      for (int i = 0; i < 4; ++i) kf[ps][i] = ld16(kr + 8 * (part + LPK * i));
    }
#pragma unroll
    for (int t = 0; t < VLOADS; ++t) {
      const int key = min(kw + t * KPI + kq, L - 1);
      vf[t] = ld16(vbase + (int64_t)key * p.kv_ss + 8 * dgrp);
    }
  };
  // q (with ROPE: the lane's theta, the q and new-k pairs -- lanes past D/2
  // read pair 0 and ignore it -- and its piece of the new v) is loaded
  // first, then the first pass's K and V; the pairs are converted and turned
  // only after those loads are issued, so a wait for them never waits for K
  // or V, and the rotation (the RoPE kernels' angle, rotation and rounding,
  // through this wave's LDS rows) runs under the cache loads.
  u32x4 qf[GS][4];
  u32x4 vn = {};
  const int lm = lane < HALF ? lane : 0;
  const int ia = r.style == ROPE_HALF ? lm : 2 * lm, ib = r.style == ROPE_HALF ? lm + HALF : 2 * lm + 1;
  bf16_t qa[GS + 1], qb[GS + 1];
  double theta = 0.0;
  if constexpr (ROPE) {
    theta = r.theta[lm];
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      const bf16_t* qr = reinterpret_cast<const bf16_t*>(p.q) + (int64_t)b * p.q_sb + (int64_t)(h0 + g) * p.q_sh;
      qa[g] = qr[ia];
      qb[g] = qr[ib];
    }
    const bf16_t* knr = reinterpret_cast<const bf16_t*>(r.k_new) + (int64_t)b * r.n_sb + (int64_t)kvh * r.n_sh;
    qa[GS] = knr[ia];
    qb[GS] = knr[ib];
    vn = ld16(reinterpret_cast<const bf16_t*>(r.v_new) + (int64_t)b * r.n_sb + (int64_t)kvh * r.n_sh + 8 * dgrp);
  } else {
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      const bf16_t* qr = reinterpret_cast<const bf16_t*>(p.q) + (int64_t)b * p.q_sb + (int64_t)(h0 + g) * p.q_sh;
#pragma unroll
      for (int i = 0; i < 4; ++i) qf[g][i] = ld16(qr + 8 * (part + LPK * i));
    }
  }
  u32x4 kf[PASSES][4], vf[VLOADS];
  load(kf, vf, wave * WK);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (ROPE) {
    if (lane < HALF) {
      float sn, cs;
      angle_sincos((double)(L - 1) * theta, &sn, &cs);
#pragma unroll
      for (int g = 0; g <= GS; ++g) {
        float ra, rb;
        rope_rotate_pair(bf16_to_f32(qa[g]), bf16_to_f32(qb[g]), sn, cs, ra, rb);
        rows[wave][g][ia] = f32_to_bf16(ra);
        rows[wave][g][ib] = f32_to_bf16(rb);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's rows landed
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int g = 0; g < GS; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) qf[g][i] = *reinterpret_cast<const u32x4*>(&rows[wave][g][8 * (part + LPK * i)]);
  }

  auto compute = [&](u32x4 (&kf)[PASSES][4], u32x4 (&vf)[VLOADS], int kw) {
    if (kw >= L) return;  // wave-uniform: no key of this wave in the chunk
    if constexpr (ROPE) {
      // Slot L - 1 comes from the turned row in LDS and v_new (only the
      // pass holding it has a key index that clamps to L - 1); the first
      // head subgroup writes the new token's k and v into the caches.
      const u32x4* kn = reinterpret_cast<const u32x4*>(&rows[wave][GS][0]);
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps)
        if (min(kw + ps * KPP + key_sub, L - 1) == L - 1)
#pragma unroll
          for (int i = 0; i < 4; ++i) kf[ps][i] = kn[part + LPK * i];
#pragma unroll
      for (int t = 0; t < VLOADS; ++t)
        if (min(kw + t * KPI + kq, L - 1) == L - 1) vf[t] = vn;
      if (hs == 0) {
        bf16_t* kc = reinterpret_cast<bf16_t*>(r.k_cache) + (int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh +
                     (int64_t)(L - 1) * p.kv_ss;
        bf16_t* vc = reinterpret_cast<bf16_t*>(r.v_cache) + (int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh +
                     (int64_t)(L - 1) * p.kv_ss;
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps)
          if (kw + ps * KPP + key_sub == L - 1)
#pragma unroll
            for (int i = 0; i < 4; ++i) st16(kc + 8 * (part + LPK * i), kn[part + LPK * i]);
#pragma unroll
        for (int t = 0; t < VLOADS; ++t)
          if (kw + t * KPI + kq == L - 1) st16(vc + 8 * dgrp, vn);
      }
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
    // ---- running softmax: raise the max, rescale, add this chunk ----
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      float mx = z[g][0];
#pragma unroll
      for (int ps = 1; ps < PASSES; ++ps) mx = fmaxf(mx, z[g][ps]);
      const float m_new = fmaxf(m_w[g], max_above<LPK>(mx));
      const float a = exp2f(m_w[g] - m_new);  // 0 on the wave's first chunk
      l_w[g] *= a;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] *= a;
      m_w[g] = m_new;
      float sm = 0.f;
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps) {
        z[g][ps] = exp2f(z[g][ps] - m_new);
        sm += z[g][ps];
      }
      l_w[g] += sum_above<LPK>(sm);
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
    // ---- p.V, two keys' values of one d paired per packed dot product ----
#pragma unroll
    for (int t = 0; t < VLOADS; t += 2) {
      const f32x4 pa = p_lds[wave][t * KPI + kq];
      const f32x4 pb = p_lds[wave][(t + 1) * KPI + kq];
      uint32_t pp[GS];
#pragma unroll
      for (int g = 0; g < GS; ++g) pp[g] = pack_bf16x2(pa[g], pb[g]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = __builtin_amdgcn_perm(vf[t + 1][e], vf[t][e], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(vf[t + 1][e], vf[t][e], 0x07060302u);
#pragma unroll
        for (int g = 0; g < GS; ++g) {
          acc[g][2 * e] = dot2(pp[g], lo, acc[g][2 * e]);
          acc[g][2 * e + 1] = dot2(pp[g], hi, acc[g][2 * e + 1]);
        }
      }
    }
  };

  for (int kc = 0;;) {
    compute(kf, vf, kc + wave * WK);
    kc += KEYS;
    if (kc >= L) break;
    load(kf, vf, kc + wave * WK);
    __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the arithmetic
  }

  // ---- merge: the KPI key lanes of a wave by lane shuffles, then the W
  // waves in LDS; final rows ----
#pragma unroll
  for (int g = 0; g < GS; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = sum_above<LPR>(acc[g][e]);
  if (kq == 0) {
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      *reinterpret_cast<f32x4*>(&o_lds[wave][g][8 * dgrp]) = f32x4{acc[g][0], acc[g][1], acc[g][2], acc[g][3]};
      *reinterpret_cast<f32x4*>(&o_lds[wave][g][8 * dgrp + 4]) = f32x4{acc[g][4], acc[g][5], acc[g][6], acc[g][7]};
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      ml_lds[wave][g][0] = m_w[g];
      ml_lds[wave][g][1] = l_w[g];
    }
  }
  __syncthreads();
  for (int i = tid; i < GS * D; i += 64 * W) {
    const int g = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, ml_lds[w][g][0]);
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float f = exp2f(ml_lds[w][g][0] - M);  // 0 for a wave without keys
      lsum = fmaf(ml_lds[w][g][1], f, lsum);
      o = fmaf(o_lds[w][g][d], f, o);
    }
    const int h = h0 + g;
    bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh;
    orow[d] = f32_to_bf16(o / lsum);
    if (d == 0 && p.lse) p.lse[(int64_t)b * p.Hq + h] = (M + log2f(lsum)) * kLn2;
  }
}

// Merge the chunks of one (sequence, query head): max-rescaled sums.
template <int D>
__global__ void __launch_bounds__(256) decode_combine_kernel(AttnParams p, DecodeWs ws) {
  // One wave per (sequence, query head).  The partial rows of the first
  // kPre chunks and lane c's (max, sum) of chunk c are all loaded at once,
  // so the merge waits for one round of loads; the global max and the
  // rescaled sum are wave reductions, and each lane holds D / 64 outputs.
  constexpr int EPL = D >= 64 ? D / 64 : 1;  // output elements per lane
  constexpr int kPre = 16;
  const int lane = threadIdx.x & 63;
  // The (sequence, head) index is wave-uniform: through readfirstlane it
  // lives in a scalar register, so its length comes by a scalar load.
  const int bh = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (bh >= p.B * p.Hq) return;
  const int b = bh / p.Hq, h = bh % p.Hq;
  const int L = p.seq_lens[b];
  if (!len_ok(p, L)) return;
  const int ns = (L + ws.chunk - 1) / ws.chunk;
  if (ns <= 1) return;
  const int64_t base = (int64_t)bh * ws.NS;  // slot (b, h, c) = (b * Hq + h) * NS + c
  const bool act = lane * EPL < D;
  float v[kPre][EPL];
#pragma unroll
  for (int u = 0; u < kPre; ++u)
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      v[u][e] = (act && u < ns) ? ws.part_o[(base + u) * D + lane * EPL + e] : 0.f;
  const float m0 = lane < ns ? ws.part_ml[(base + lane) * 2] : -INFINITY;
  const float l0 = lane < ns ? ws.part_ml[(base + lane) * 2 + 1] : 0.f;
  float M = m0;
  for (int c = lane + 64; c < ns; c += 64) M = fmaxf(M, ws.part_ml[(base + c) * 2]);
  M = wave_max(M);
  const float f0 = lane < ns ? exp2f(m0 - M) : 0.f;
  float lsum = l0 * f0;
  for (int c = lane + 64; c < ns; c += 64)
    lsum = fmaf(ws.part_ml[(base + c) * 2 + 1], exp2f(ws.part_ml[(base + c) * 2] - M), lsum);
  lsum = wave_sum(lsum);

  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const float fu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f0), u));  // 0 past ns
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = fmaf(fu, v[u][e], o[e]);
  }
  for (int c = kPre; c < ns; ++c) {  // long sequences only
    const float f = exp2f(ws.part_ml[(base + c) * 2] - M);
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      if (act) o[e] = fmaf(f, ws.part_o[(base + c) * D + lane * EPL + e], o[e]);
  }
  if (act) {
    const float inv = 1.f / lsum;
    bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) orow[e] = f32_to_bf16(o[e] * inv);
  }
  if (lane == 0 && p.lse) p.lse[(int64_t)b * p.Hq + h] = (M + log2f(lsum)) * kLn2;
}

int heads_per_wg(int group) {
  for (int gs = 4; gs >= 1; --gs)
    if (group % gs == 0) return gs;
  return 1;
}

template <int D, int MUL, bool ROPE>
hipError_t launch_dm(const AttnParams& p, const DecodeRope& r, DecodeWs ws, int gs, int nsub, hipStream_t stream) {
  const dim3 grid(ws.NS, p.Hkv * nsub, p.B), block(64 * kWaves);
  KernelTimer kt_("decode_split_kernel", stream);
  switch (gs) {
    case 4: hipLaunchKernelGGL((decode_split_kernel<D, 4, MUL, ROPE>), grid, block, 0, stream, p, ws, nsub, r); break;
    case 3: hipLaunchKernelGGL((decode_split_kernel<D, 3, MUL, ROPE>), grid, block, 0, stream, p, ws, nsub, r); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<D, 2, MUL, ROPE>), grid, block, 0, stream, p, ws, nsub, r); break;
    default:
      hipLaunchKernelGGL((decode_split_kernel<D, 1, MUL, ROPE>), grid, block, 0, stream, p, ws, nsub, r);
      break;
  }
  return hipGetLastError();
}

// Longer chunks (two q.k passes per wave) halve the partials and the fixed
// cost per workgroup; they are used when the batch still gives at least
// four workgroups per compute unit.
int chunk_mul(int B, int Hkv, int nsub, int D, int max_len) {
  const int64_t wgs = (int64_t)B * Hkv * nsub * ((max_len + chunk_keys(D, 2) - 1) / chunk_keys(D, 2));
  return wgs >= 4 * 256 ? 2 : 1;
}

// The walking form: one query head per workgroup (so q and the output take
// few registers), 64 keys per wave (32 at head dim 128), 12 waves (three per
// SIMD, up to 168 registers each: the token's RoPE prologue does not spill).
// Both variants take the same shape, so the step with RoPE inside stays bit
// for bit the two-launch step.
template <bool ROPE>
constexpr int loop_waves() { return 12; }
template <int D>
constexpr int loop_mul() { return D == 128 ? 1 : 2; }
template <int D, bool ROPE>
constexpr int loop_keys() { return loop_waves<ROPE>() * Chunk<D, loop_mul<D>()>::WAVE_KEYS; }

template <int D, bool ROPE>
hipError_t launch_loop(const AttnParams& p, const DecodeRope& r, hipStream_t stream) {
  const int nsub = p.Hq / p.Hkv;  // one query head per workgroup
  const dim3 grid(1, p.Hkv * nsub, p.B), block(64 * loop_waves<ROPE>());
  KernelTimer kt_("decode_loop_kernel", stream);
  hipLaunchKernelGGL((decode_loop_kernel<D, 1, loop_mul<D>(), ROPE, loop_waves<ROPE>()>), grid, block, 0, stream,
                     p, nsub, r);
  return hipGetLastError();
}

// The walking form takes over when the split grid would not give every
// compute unit a workgroup and a sequence needs at most kLoopPasses passes
// of the walking workgroup (so its serial walk stays short).
constexpr int kLoopPasses = 2;
template <int D, bool ROPE>
bool use_loop(const AttnParams& p, int nsub, int mul) {
  const int64_t units = (int64_t)p.B * p.Hkv * nsub;
  const int64_t split_wgs = units * ((p.max_len + chunk_keys(D, mul) - 1) / chunk_keys(D, mul));
  const int passes = (p.max_len + loop_keys<D, ROPE>() - 1) / loop_keys<D, ROPE>();
  return split_wgs <= 256 && passes <= kLoopPasses;
}

template <int D, bool ROPE>
hipError_t launch_d(const AttnParams& p, const DecodeRope& r, DecodeWs ws, hipStream_t stream) {
  const int group = p.Hq / p.Hkv;
  const int gs = heads_per_wg(group);
  const int nsub = group / gs;
  const int mul = chunk_mul(p.B, p.Hkv, nsub, D, p.max_len);
  if (use_loop<D, ROPE>(p, nsub, mul)) return launch_loop<D, ROPE>(p, r, stream);
  ws.chunk = chunk_keys(D, mul);
  ws.NS = (p.max_len + ws.chunk - 1) / ws.chunk;
  hipError_t e = mul == 2 ? launch_dm<D, 2, ROPE>(p, r, ws, gs, nsub, stream)
                          : launch_dm<D, 1, ROPE>(p, r, ws, gs, nsub, stream);
  if (e != hipSuccess || ws.NS <= 1) return e;
  KernelTimer kt_("decode_combine_kernel", stream);
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3((p.B * p.Hq + 3) / 4), dim3(256), 0, stream, p, ws);
  return hipGetLastError();
}

}  // namespace

// Workspace: partial outputs, then partial (max, sum) pairs, sized for the
// shorter chunks (the most partials either chunk length can produce).
struct WsLayout {
  size_t o_bytes, ml_bytes;
};
WsLayout ws_layout(int B, int Hq, int D, int max_len) {
  WsLayout l;
  const int chunk = chunk_keys(D, 1);
  const int64_t slots = (int64_t)B * Hq * ((max_len + chunk - 1) / chunk);
  l.o_bytes = ((size_t)(slots * D * 4) + 255) & ~(size_t)255;
  l.ml_bytes = ((size_t)(slots * 2 * 4) + 255) & ~(size_t)255;
  return l;
}

size_t decode_workspace_bytes(int B, int Hq, int /*Hkv*/, int D, int max_len) {
  const WsLayout l = ws_layout(B, Hq, D, max_len);
  return l.o_bytes + l.ml_bytes;
}

namespace {

template <bool ROPE>
hipError_t launch_decode(const AttnParams& p, const DecodeRope& r, void* workspace, hipStream_t stream) {
  const WsLayout l = ws_layout(p.B, p.Hq, p.D, p.max_len);
  DecodeWs ws;
  ws.NS = 0;     // set with the chunk length at launch
  ws.chunk = 0;
  char* base = reinterpret_cast<char*>(workspace);
  ws.part_o = reinterpret_cast<float*>(base);
  ws.part_ml = reinterpret_cast<float*>(base + l.o_bytes);
  switch (p.D) {
    case 32: return launch_d<32, ROPE>(p, r, ws, stream);
    case 64: return launch_d<64, ROPE>(p, r, ws, stream);
    default: return launch_d<128, ROPE>(p, r, ws, stream);
  }
}

}  // namespace

// The decode's partials in a library-owned device array, for callers that
// cannot allocate a workspace.  Each GPU holds its own copy of `scratch`
// (device code objects are loaded per device); the host needs that copy's
// device address, which hipGetSymbolAddress gives once per device with the
// device current.  The array's name itself is a host-side stand-in and is
// never passed to a kernel.
namespace {
__device__ __align__(256) char scratch[kDecodeStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_static_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = a;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_bf16(const AttnParams& p, void* workspace, hipStream_t stream) {
  return launch_decode<false>(p, DecodeRope{}, workspace, stream);
}

hipError_t launch_decode_rope_bf16(const AttnParams& p, const DecodeRope& r, void* workspace, hipStream_t stream) {
  return launch_decode<true>(p, r, workspace, stream);
}

}  // namespace rgc
