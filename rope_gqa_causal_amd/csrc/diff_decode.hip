// diff_decode.hip -- cached decode of differential attention: one new query
// row per sequence against its k1, k2 and v caches.
//
// Operation (page "750美元从零训练3个LLM：一位开发者的实战复盘", section
// "V2：引入前沿技术": a second attention map, weighted by lambda, is
// subtracted from the first): for sequence b and query head h, with KV head
// h / (Hq/Hkv) and the L = seq_lens[b] cached slots,
//   o = softmax(scale q1 . K1[0..L-1]) V - lambda softmax(scale q2 . K2[0..L-1]) V.
//
// HBM-bound, as the plain decode: every byte of the three caches is read
// once per group of query heads.  Split-K over the cache length: a
// workgroup of four waves owns one (sequence, KV head, head subgroup of at
// most 2 query heads) and a chunk of 4 x 64 keys (4 x 32 at head dim 128);
// each wave issues every load of its keys (q1, q2, then K1, K2, V) before
// any arithmetic, keys past the end re-reading the last row and masked in
// the scores.  Each map keeps its own running max, sum and output; the two
// maps' probabilities share one LDS transposition and one set of V loads.
// A chunk's two partials go to the workspace and a second kernel merges
// each map by max-rescaled sums, then forms o1/l1 - lambda o2/l2 and rounds
// once.  A sequence that fits in one chunk is finished by the first kernel.
#include "common.h"
#include "decode_lanes.h"
#include "launch.h"

namespace rgc {
namespace {

constexpr int kDW = 4;  // waves per workgroup

// Row layout: a load instruction covers whole cache rows, LPR = D/8 lanes
// per row (one 16-byte piece each), KPI = 64/LPR rows.  Keys per wave: 64
// (32 at head dim 128, where K1, K2 and V rows of 64 keys would not fit the
// registers).
template <int D>
struct DChunk {
  static constexpr int LPR = D / 8;
  static constexpr int KPI = 64 / LPR;
  static constexpr int WK = D == 128 ? 32 : 64;            // keys per wave
  static constexpr int LOADS = WK / KPI;                   // row loads per matrix
  static constexpr int KEYS = kDW * WK;                    // keys per workgroup
};
int diff_chunk_keys(int D) { return kDW * (D == 128 ? 32 : 64); }

struct DiffWs {
  float* part_o;   // [B][Hq][NS][2][D]  unnormalised partial outputs of both maps
  float* part_ml;  // [B][Hq][NS][2][2]  (max in log2 units, sum) of both maps
  int NS;
};

__device__ __forceinline__ bool dlen_ok(const DiffParams& d, int L) {
  const int lim = d.a.max_len < d.a.S_max ? d.a.max_len : d.a.S_max;
  return L >= 1 && L <= lim;
}

// GS: query heads per workgroup (1 or 2; the two maps' probabilities of
// both heads share one f32x4 per key in LDS).
template <int D, int GS>
__global__ void __launch_bounds__(64 * kDW) diff_decode_kernel(DiffParams dp, DiffWs ws, int nsub) {
  const AttnParams& p = dp.a;
  using C = DChunk<D>;
  constexpr int LPR = C::LPR, KPI = C::KPI, WK = C::WK, LOADS = C::LOADS;

  __shared__ float o_lds[kDW][2][GS][D];
  __shared__ float ml_lds[kDW][2][GS][2];

  const int split = blockIdx.x;
  const int hs = blockIdx.y % nsub;
  const int kvh = blockIdx.y / nsub;
  const int b = blockIdx.z;
  const int group = p.Hq / p.Hkv;
  const int h0 = kvh * group + hs * GS;
  const int L = p.seq_lens[b];
  const int tid = threadIdx.x;

  if (!dlen_ok(dp, L)) {
    if (split == 0) {
      for (int i = tid; i < GS * D; i += 64 * kDW) {
        bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb + (int64_t)(h0 + i / D) * p.o_sh;
        orow[i % D] = 0x7FC0;  // NaN
      }
      if (tid == 0 && p.err) p.err[0] = 1;
    }
    return;
  }
  const int k0 = split * C::KEYS;
  if (k0 >= L) return;
  const int ns = (L + C::KEYS - 1) / C::KEYS;

  const int wave = tid >> 6, lane = tid & 63;
  const int kw = k0 + wave * WK;
  const float c = p.scale * kLog2e;
  const int64_t rowbase = (int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh;
  const bf16_t* kb1 = reinterpret_cast<const bf16_t*>(p.k) + rowbase;
  const bf16_t* kb2 = reinterpret_cast<const bf16_t*>(dp.k2) + rowbase;
  const bf16_t* vb = reinterpret_cast<const bf16_t*>(p.v) + rowbase;
  const int pc = lane % LPR, kr = lane / LPR;  // this lane's 16-byte piece and row of a load

  // [map][head]
  float m_w[2][GS], l_w[2][GS], acc[2][GS][8];
#pragma unroll
  for (int mp = 0; mp < 2; ++mp)
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      m_w[mp][g] = -INFINITY;
      l_w[mp][g] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[mp][g][e] = 0.f;
    }

  if (kw < L) {  // wave-uniform
    // ---- every load of the wave's keys, issued before any arithmetic:
    // q1 and q2 (this lane's piece of each head), then rows t KPI + kr of K1,
    // K2 and V (keys past the end re-read the last row and are masked) ----
    u32x4 qf[2][GS];
#pragma unroll
    for (int mp = 0; mp < 2; ++mp)
#pragma unroll
      for (int g = 0; g < GS; ++g)
        qf[mp][g] = ld16(reinterpret_cast<const bf16_t*>(mp ? dp.q2 : p.q) + (int64_t)b * p.q_sb +
                         (int64_t)(h0 + g) * p.q_sh + 8 * pc);
    u32x4 kf[2][LOADS], vf[LOADS];
#pragma unroll
    for (int t = 0; t < LOADS; ++t) {
      const int64_t off = (int64_t)min(kw + t * KPI + kr, L - 1) * p.kv_ss + 8 * pc;
      kf[0][t] = ld16_nt(kb1 + off);
      kf[1][t] = ld16_nt(kb2 + off);
      vf[t] = ld16_nt(vb + off);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the arithmetic

    // ---- scores of both maps (a row's LPR lanes add their pieces' dot
    // products), softmax over the wave's keys; every lane of a row then
    // holds that key's probabilities, the layout of its V row ----
    float z[2][GS][LOADS];
#pragma unroll
    for (int t = 0; t < LOADS; ++t) {
      const bool valid = kw + t * KPI + kr < L;
#pragma unroll
      for (int mp = 0; mp < 2; ++mp)
#pragma unroll
        for (int g = 0; g < GS; ++g) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) d = dot2(qf[mp][g][e], kf[mp][t][e], d);
          d = sum_within_row<LPR>(d);
          z[mp][g][t] = valid ? d * c : -INFINITY;
        }
    }
#pragma unroll
    for (int mp = 0; mp < 2; ++mp)
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        float mx = z[mp][g][0];
#pragma unroll
        for (int t = 1; t < LOADS; ++t) mx = fmaxf(mx, z[mp][g][t]);
        m_w[mp][g] = max_above<LPR>(mx);
        float sm = 0.f;
#pragma unroll
        for (int t = 0; t < LOADS; ++t) {
          z[mp][g][t] = exp2f(z[mp][g][t] - m_w[mp][g]);
          sm += z[mp][g][t];
        }
        l_w[mp][g] = sum_above<LPR>(sm);
      }
    // ---- p.V for both maps: two keys' values of one d paired per packed
    // dot product with the pair of their bf16 probabilities ----
#pragma unroll
    for (int t = 0; t < LOADS; t += 2) {
      uint32_t pp[2][GS];
#pragma unroll
      for (int mp = 0; mp < 2; ++mp)
#pragma unroll
        for (int g = 0; g < GS; ++g) pp[mp][g] = pack_bf16x2(z[mp][g][t], z[mp][g][t + 1]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = __builtin_amdgcn_perm(vf[t + 1][e], vf[t][e], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(vf[t + 1][e], vf[t][e], 0x07060302u);
#pragma unroll
        for (int mp = 0; mp < 2; ++mp)
#pragma unroll
          for (int g = 0; g < GS; ++g) {
            acc[mp][g][2 * e] = dot2(pp[mp][g], lo, acc[mp][g][2 * e]);
            acc[mp][g][2 * e + 1] = dot2(pp[mp][g], hi, acc[mp][g][2 * e + 1]);
          }
      }
    }
  }
  // ---- merge the rows of the wave (shuffles) and the four waves (LDS) ----
#pragma unroll
  for (int mp = 0; mp < 2; ++mp)
#pragma unroll
    for (int g = 0; g < GS; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[mp][g][e] = sum_above<LPR>(acc[mp][g][e]);
  if (kr == 0) {
#pragma unroll
    for (int mp = 0; mp < 2; ++mp)
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        *reinterpret_cast<f32x4*>(&o_lds[wave][mp][g][8 * pc]) =
            f32x4{acc[mp][g][0], acc[mp][g][1], acc[mp][g][2], acc[mp][g][3]};
        *reinterpret_cast<f32x4*>(&o_lds[wave][mp][g][8 * pc + 4]) =
            f32x4{acc[mp][g][4], acc[mp][g][5], acc[mp][g][6], acc[mp][g][7]};
      }
  }
  if (lane == 0) {
#pragma unroll
    for (int mp = 0; mp < 2; ++mp)
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        ml_lds[wave][mp][g][0] = m_w[mp][g];
        ml_lds[wave][mp][g][1] = l_w[mp][g];
      }
  }
  __syncthreads();
  for (int i = tid; i < GS * D; i += 64 * kDW) {
    const int g = i / D, d = i % D;
    float M[2], ls[2], o[2];
#pragma unroll
    for (int mp = 0; mp < 2; ++mp) {
      M[mp] = -INFINITY;
#pragma unroll
      for (int w = 0; w < kDW; ++w) M[mp] = fmaxf(M[mp], ml_lds[w][mp][g][0]);
      ls[mp] = 0.f;
      o[mp] = 0.f;
#pragma unroll
      for (int w = 0; w < kDW; ++w) {
        const float f = exp2f(ml_lds[w][mp][g][0] - M[mp]);  // 0 for a wave without keys
        ls[mp] = fmaf(ml_lds[w][mp][g][1], f, ls[mp]);
        o[mp] = fmaf(o_lds[w][mp][g][d], f, o[mp]);
      }
    }
    const int h = h0 + g;
    if (ns == 1) {
      bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh;
      orow[d] = f32_to_bf16(o[0] / ls[0] - dp.lambda * (o[1] / ls[1]));
    } else {
      const int64_t slot = ((int64_t)b * p.Hq + h) * ws.NS + split;
#pragma unroll
      for (int mp = 0; mp < 2; ++mp) {
        ws.part_o[(slot * 2 + mp) * D + d] = o[mp];
        if (d == 0) {
          ws.part_ml[(slot * 2 + mp) * 2] = M[mp];
          ws.part_ml[(slot * 2 + mp) * 2 + 1] = ls[mp];
        }
      }
    }
  }
}

// Merge the chunks of one (sequence, query head), each map by
// max-rescaled sums, then o1/l1 - lambda o2/l2.  One wave per (sequence,
// head); lane c holds chunk c's (max, sum), each lane D/64 outputs.  The
// partial rows of the first kPre chunks are loaded in one round, so the
// merge waits for one round of loads.
template <int D>
__global__ void __launch_bounds__(256) diff_combine_kernel(DiffParams dp, DiffWs ws, int chunk) {
  const AttnParams& p = dp.a;
  constexpr int EPL = D >= 64 ? D / 64 : 1;
  constexpr int kPre = 8;
  const int lane = threadIdx.x & 63;
  const int bh = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (bh >= p.B * p.Hq) return;
  const int b = bh / p.Hq, h = bh % p.Hq;
  const int L = p.seq_lens[b];
  if (!dlen_ok(dp, L)) return;
  const int ns = (L + chunk - 1) / chunk;
  if (ns <= 1) return;
  const int64_t base = (int64_t)bh * ws.NS;
  const bool act = lane * EPL < D;
  float v[2][kPre][EPL];
#pragma unroll
  for (int mp = 0; mp < 2; ++mp)
#pragma unroll
    for (int u = 0; u < kPre; ++u)
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        v[mp][u][e] = (act && u < ns) ? ws.part_o[((base + u) * 2 + mp) * D + lane * EPL + e] : 0.f;
  float m0[2], l0[2];
#pragma unroll
  for (int mp = 0; mp < 2; ++mp) {
    m0[mp] = lane < ns ? ws.part_ml[((base + lane) * 2 + mp) * 2] : -INFINITY;
    l0[mp] = lane < ns ? ws.part_ml[((base + lane) * 2 + mp) * 2 + 1] : 0.f;
  }
  float res[2][EPL], lsum[2];
#pragma unroll
  for (int mp = 0; mp < 2; ++mp) {
    float M = m0[mp];
    for (int cc = lane + 64; cc < ns; cc += 64) M = fmaxf(M, ws.part_ml[((base + cc) * 2 + mp) * 2]);
    M = wave_max(M);
    const float f0 = lane < ns ? exp2f(m0[mp] - M) : 0.f;
    float ls = l0[mp] * f0;
    for (int cc = lane + 64; cc < ns; cc += 64)
      ls = fmaf(ws.part_ml[((base + cc) * 2 + mp) * 2 + 1], exp2f(ws.part_ml[((base + cc) * 2 + mp) * 2] - M), ls);
    lsum[mp] = wave_sum(ls);
#pragma unroll
    for (int e = 0; e < EPL; ++e) res[mp][e] = 0.f;
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const float fu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f0), u));  // 0 past ns
#pragma unroll
      for (int e = 0; e < EPL; ++e) res[mp][e] = fmaf(fu, v[mp][u][e], res[mp][e]);
    }
    for (int cc = kPre; cc < ns; ++cc) {  // long sequences only
      const float f = exp2f(ws.part_ml[((base + cc) * 2 + mp) * 2] - M);
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        if (act) res[mp][e] = fmaf(f, ws.part_o[((base + cc) * 2 + mp) * D + lane * EPL + e], res[mp][e]);
    }
  }
  if (act) {
    bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) orow[e] = f32_to_bf16(res[0][e] / lsum[0] - dp.lambda * (res[1][e] / lsum[1]));
  }
}

template <int D>
hipError_t launch_dd(const DiffParams& dp, DiffWs ws, hipStream_t stream) {
  const AttnParams& p = dp.a;
  const int group = p.Hq / p.Hkv;
  const int gs = group % 2 == 0 ? 2 : 1;
  const int nsub = group / gs;
  const int chunk = diff_chunk_keys(D);
  ws.NS = (p.max_len + chunk - 1) / chunk;
  const dim3 grid(ws.NS, p.Hkv * nsub, p.B), block(64 * kDW);
  {
    KernelTimer kt_("diff_decode_kernel", stream);
    if (gs == 2)
      hipLaunchKernelGGL((diff_decode_kernel<D, 2>), grid, block, 0, stream, dp, ws, nsub);
    else
      hipLaunchKernelGGL((diff_decode_kernel<D, 1>), grid, block, 0, stream, dp, ws, nsub);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || ws.NS <= 1) return e;
  }
  KernelTimer kt_("diff_combine_kernel", stream);
  hipLaunchKernelGGL(diff_combine_kernel<D>, dim3((p.B * p.Hq + 3) / 4), dim3(256), 0, stream, dp, ws, chunk);
  return hipGetLastError();
}

}  // namespace

// Workspace: both maps' partial outputs, then their (max, sum) pairs.
size_t diff_decode_workspace_bytes(int B, int Hq, int D, int max_len) {
  const int chunk = diff_chunk_keys(D);
  const int64_t slots = (int64_t)B * Hq * ((max_len + chunk - 1) / chunk) * 2;
  const size_t o_bytes = ((size_t)(slots * D * 4) + 255) & ~(size_t)255;
  const size_t ml_bytes = ((size_t)(slots * 2 * 4) + 255) & ~(size_t)255;
  return o_bytes + ml_bytes;
}

hipError_t launch_diff_decode_bf16(const DiffParams& dp, void* workspace, hipStream_t stream) {
  const AttnParams& p = dp.a;
  const int chunk = diff_chunk_keys(p.D);
  const int64_t slots = (int64_t)p.B * p.Hq * ((p.max_len + chunk - 1) / chunk) * 2;
  DiffWs ws;
  ws.part_o = reinterpret_cast<float*>(workspace);
  ws.part_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                        ((((size_t)(slots * p.D * 4)) + 255) & ~(size_t)255));
  ws.NS = 0;
  switch (p.D) {
    case 32: return launch_dd<32>(dp, ws, stream);
    case 64: return launch_dd<64>(dp, ws, stream);
    default: return launch_dd<128>(dp, ws, stream);
  }
}

}  // namespace rgc
