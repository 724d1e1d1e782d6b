// prefill.hip -- causal GQA attention of a block of query rows over the bf16
// cache, on the gfx950 matrix cores.
//
// Operation (page "750美元从零训练3个LLM：一位开发者的实战复盘", section V2;
// page "训练3.8B LLM至0.384 CORE，成本998美元 – Hugo Vergnes", sections 设置
// and 无效的方法; the m.nxbn.cn build-an-LLM page, section 3.1): row s of
// sequence b at slot p attends to slots 0..p of its KV head.
//
// A dense contraction (QK^T then PV), so it runs on bf16 MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//  * a workgroup owns one (sequence, KV head, head subgroup) and 128 query
//    positions; each of its 4 waves owns 32 positions of every head in the
//    subgroup (NB heads), so one K/V tile staged in LDS feeds all of them;
//  * scores are computed transposed, S^T = K Q^T (keys in the MFMA M
//    dimension), which leaves each lane holding one query's column: the
//    online-softmax max and sum are in-lane except one swap with the lane
//    32 away, and the probabilities are already laid out as the B operand of
//    O^T = V^T P^T, so P never leaves registers;
//  * K tiles sit in LDS row-major with a 16-byte XOR swizzle (conflict-free
//    row reads); V tiles are transposed while being staged (two keys per
//    32-bit LDS word) so that V^T fragments are two 8-byte LDS reads;
//  * the next K/V tile is fetched from HBM into registers while the current
//    one is multiplied (LDS double buffer, one barrier per tile);
//  * tiles above the causal diagonal are skipped per wave, and workgroups
//    are issued heaviest q-tile first; the blockIdx -> (KV head, tile)
//    mapping keeps every tile of one KV head on one XCD (shared L2).
#include "common.h"
#include "launch.h"

namespace rgc {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;  // query positions per workgroup
constexpr int kKT = 32;           // keys per tile

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int D>
struct Tile {
  static constexpr int CH = D / 8;                 // 16-byte chunks per row
  static constexpr int K_UNITS = kKT * CH;         // chunks in a K tile
  static constexpr int V_UNITS = (kKT / 2) * CH;   // (key pair, chunk) units
  static constexpr int K_PER_T = (K_UNITS + 255) / 256;
  static constexpr int V_PER_T = (V_UNITS + 255) / 256;
  static constexpr int VT_STRIDE = kKT + 4;        // bf16 per V^T row (72 B)
  static constexpr int K_ELEMS = kKT * D;
  static constexpr int VT_ELEMS = D * VT_STRIDE;
};

template <int D>
struct Stage {
  u32x4 k[Tile<D>::K_PER_T];
  u32x4 v[Tile<D>::V_PER_T][2];
};

// Fetch tile [j0, j0+32) of K and V into registers; keys past kmax read as 0
// (never from memory), so no unwritten cache slot can reach the arithmetic.
template <int D>
__device__ __forceinline__ void fetch_tile(Stage<D>& st, const bf16_t* kb, const bf16_t* vb,
                                           int64_t kv_ss, int j0, int kmax, int tid) {
  using T = Tile<D>;
#pragma unroll
  for (int i = 0; i < T::K_PER_T; ++i) {
    const int u = tid + 256 * i;
    st.k[i] = u32x4{0, 0, 0, 0};
    if (u < T::K_UNITS) {
      const int key = j0 + u / T::CH, c = u % T::CH;
      if (key <= kmax) st.k[i] = ld16(kb + (int64_t)key * kv_ss + 8 * c);
    }
  }
#pragma unroll
  for (int i = 0; i < T::V_PER_T; ++i) {
    const int u = tid + 256 * i;
    st.v[i][0] = st.v[i][1] = u32x4{0, 0, 0, 0};
    if (u < T::V_UNITS) {
      const int key = j0 + 2 * (u / T::CH), c = u % T::CH;
      if (key <= kmax) st.v[i][0] = ld16(vb + (int64_t)key * kv_ss + 8 * c);
      if (key + 1 <= kmax) st.v[i][1] = ld16(vb + (int64_t)(key + 1) * kv_ss + 8 * c);
    }
  }
}

// Registers -> LDS: K row-major with chunk c of key r at chunk (c ^ (r % CH));
// V transposed, element (d, key) at vt[d * VT_STRIDE + key].
template <int D>
__device__ __forceinline__ void store_tile(const Stage<D>& st, bf16_t* ks, bf16_t* vt, int tid) {
  using T = Tile<D>;
#pragma unroll
  for (int i = 0; i < T::K_PER_T; ++i) {
    const int u = tid + 256 * i;
    if (u < T::K_UNITS) {
      const int r = u / T::CH, c = u % T::CH;
      *reinterpret_cast<u32x4*>(ks + r * D + 8 * (c ^ (r % T::CH))) = st.k[i];
    }
  }
#pragma unroll
  for (int i = 0; i < T::V_PER_T; ++i) {
    const int u = tid + 256 * i;
    if (u < T::V_UNITS) {
      const int kp = u / T::CH, c = u % T::CH;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a = st.v[i][0][e], bb = st.v[i][1][e];
        // (d = 8c+2e): keys (2kp, 2kp+1) -> low halves; (d = 8c+2e+1): high halves
        const uint32_t lo = (a & 0xFFFFu) | (bb << 16);
        const uint32_t hi = (a >> 16) | (bb & 0xFFFF0000u);
        *reinterpret_cast<uint32_t*>(vt + (8 * c + 2 * e) * T::VT_STRIDE + 2 * kp) = lo;
        *reinterpret_cast<uint32_t*>(vt + (8 * c + 2 * e + 1) * T::VT_STRIDE + 2 * kp) = hi;
      }
    }
  }
}

// D: head dim (64 or 128); NB: query heads per wave (the head subgroup).
template <int D, int NB>
__global__ void __launch_bounds__(256, 1) prefill_kernel(AttnParams p, int nsub, int nqt) {
  using T = Tile<D>;
  constexpr int KS = D / 16;   // k-steps of QK^T
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) bf16_t k_lds[2][T::K_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t vt_lds[2][T::VT_ELEMS];

  const int nunits = p.B * p.Hkv * nsub;
  const int unit = blockIdx.x % nunits;
  const int qt = nqt - 1 - (int)(blockIdx.x / nunits);  // heaviest tiles first
  const int hs = unit % nsub;
  const int kvh = (unit / nsub) % p.Hkv;
  const int b = unit / (nsub * p.Hkv);
  const int group = p.Hq / p.Hkv;
  const int h0 = kvh * group + hs * NB;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;

  const int first = p.q_start ? p.q_start[b] : 0;
  const int s_base = qt * kBM + wave * 32;  // this wave's first row
  if (first < 0 || (int64_t)first + p.Sq > p.S_max) {
    // Device-side capacity violation: NaN rows, flag, no memory access.
    if (s_base + col < p.Sq && half == 0) {
      for (int g = 0; g < NB; ++g) {
        bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb +
                       (int64_t)(s_base + col) * p.o_ss + (int64_t)(h0 + g) * p.o_sh;
        for (int d = 0; d < D; ++d) orow[d] = 0x7FC0;
        if (p.lse) p.lse[((int64_t)b * p.Hq + h0 + g) * p.Sq + s_base + col] = __builtin_nanf("");
      }
    }
    if (tid == 0 && p.err) p.err[0] = 1;
    return;
  }

  const int s_end_wg = min(p.Sq, (qt + 1) * kBM);           // rows [qt*kBM, s_end_wg)
  const int kmax = first + s_end_wg - 1;                      // last key the workgroup needs
  const int nkt = kmax / kKT + 1;
  const int wave_rows = min(32, p.Sq - s_base);               // may be <= 0 (ragged tail)
  const int wave_kmax = first + s_base + wave_rows - 1;       // last key this wave needs
  const float c = p.scale * kLog2e;

  const bf16_t* kb = reinterpret_cast<const bf16_t*>(p.k) + (int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh;
  const bf16_t* vb = reinterpret_cast<const bf16_t*>(p.v) + (int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh;

  // Q^T fragments (B operand): lane holds query `col`, d = 16*ks + 8*half .. +8.
  u32x4 qf[NB][KS];
  {
    const int s = s_base + col;
#pragma unroll
    for (int g = 0; g < NB; ++g) {
      const bf16_t* qr = reinterpret_cast<const bf16_t*>(p.q) + (int64_t)b * p.q_sb +
                         (int64_t)s * p.q_ss + (int64_t)(h0 + g) * p.q_sh;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[g][ks] = (s < p.Sq) ? ld16(qr + 16 * ks + 8 * half) : u32x4{0, 0, 0, 0};
    }
  }

  f32x16 acc_o[NB][DB];
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[g][db][r] = 0.f;
  }

  Stage<D> st;
  fetch_tile<D>(st, kb, vb, p.kv_ss, 0, kmax, tid);
  store_tile<D>(st, k_lds[0], vt_lds[0], tid);
  __syncthreads();

  const int qabs = first + s_base + col;  // this lane's query slot
  for (int jt = 0; jt < nkt; ++jt) {
    const int buf = jt & 1;
    const bool more = jt + 1 < nkt;
    if (more) fetch_tile<D>(st, kb, vb, p.kv_ss, (jt + 1) * kKT, kmax, tid);

    const int j0 = jt * kKT;
    if (wave_rows > 0 && j0 <= wave_kmax) {
      const bf16_t* ks_ = k_lds[buf];
      const bf16_t* vt_ = vt_lds[buf];
      // ---- S^T = K Q^T: lane gets keys 8*(r/4) + 4*half + r%4 of query col ----
      f32x16 sacc[NB];
#pragma unroll
      for (int g = 0; g < NB; ++g)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[g][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int cidx = 2 * ks + half;
        const u32x4 a = *reinterpret_cast<const u32x4*>(ks_ + col * D + 8 * (cidx ^ (col % T::CH)));
#pragma unroll
        for (int g = 0; g < NB; ++g) sacc[g] = mfma(a, qf[g][ks], sacc[g]);
      }
      // ---- online softmax (log2 domain) ----
      const bool diag = j0 + kKT - 1 > first + s_base;
      u32x4 pf[NB][2];
#pragma unroll
      for (int g = 0; g < NB; ++g) {
        if (diag) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (key > qabs) sacc[g][r] = -INFINITY;
          }
        }
        float tmax = sacc[g][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, sacc[g][r]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m_run[g], tmax * c);
        const float alpha = exp2f(m_run[g] - m_new);
        m_run[g] = m_new;
        float psum = 0.f;
        float pr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pr[r] = exp2f(fmaf(sacc[g][r], c, -m_new));
          psum += pr[r];
        }
        l_run[g] = fmaf(l_run[g], alpha, psum);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[g][db][r] *= alpha;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int e = 0; e < 4; ++e) pf[g][kk][e] = pack_bf16x2(pr[8 * kk + 2 * e], pr[8 * kk + 2 * e + 1]);
      }
      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16_t* vrow = vt_ + (32 * db + col) * T::VT_STRIDE + 16 * kk + 4 * half;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
          const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int g = 0; g < NB; ++g) acc_o[g][db] = mfma(a, pf[g][kk], acc_o[g][db]);
        }
      }
    }
    if (more) store_tile<D>(st, k_lds[buf ^ 1], vt_lds[buf ^ 1], tid);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, rounded to bf16 ----
  const int s = s_base + col;
  if (wave_rows > 0 && s < p.Sq) {
#pragma unroll
    for (int g = 0; g < NB; ++g) {
      const float lsum = l_run[g] + __shfl_xor(l_run[g], 32, 64);
      const float inv = 1.f / lsum;
      bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb + (int64_t)s * p.o_ss +
                     (int64_t)(h0 + g) * p.o_sh;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = 32 * db + 8 * q4 + 4 * half;
          u32x2 w;
          w[0] = pack_bf16x2(acc_o[g][db][4 * q4] * inv, acc_o[g][db][4 * q4 + 1] * inv);
          w[1] = pack_bf16x2(acc_o[g][db][4 * q4 + 2] * inv, acc_o[g][db][4 * q4 + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + d) = w;
        }
      if (p.lse && half == 0) p.lse[((int64_t)b * p.Hq + h0 + g) * p.Sq + s] = (m_run[g] + log2f(lsum)) * kLn2;
    }
  }
}

// Query heads per wave: as many of the group as the register file holds
// without spilling (the O^T and Q^T fragments grow with NB * D).
int heads_per_wave(int group, int D) {
  const int cap = D == 128 ? 2 : 4;
  for (int nb = cap; nb >= 1; --nb)
    if (group % nb == 0) return nb;
  return 1;
}

template <int D, int NB>
void launch_nb(const AttnParams& p, int nsub, int nqt, hipStream_t stream) {
  const dim3 grid((unsigned)(p.B * p.Hkv * nsub * nqt));
  hipLaunchKernelGGL((prefill_kernel<D, NB>), grid, dim3(256), 0, stream, p, nsub, nqt);
}

template <int D>
hipError_t launch_d(const AttnParams& p, hipStream_t stream) {
  const int group = p.Hq / p.Hkv;
  const int nb = heads_per_wave(group, D);
  const int nsub = group / nb;
  const int nqt = (p.Sq + kBM - 1) / kBM;
  if (D == 128) {
    if (nb == 2) launch_nb<D, 2>(p, nsub, nqt, stream);
    else launch_nb<D, 1>(p, nsub, nqt, stream);
  } else {
    switch (nb) {
      case 4: launch_nb<D, (D == 128 ? 1 : 4)>(p, nsub, nqt, stream); break;
      case 3: launch_nb<D, (D == 128 ? 1 : 3)>(p, nsub, nqt, stream); break;
      case 2: launch_nb<D, 2>(p, nsub, nqt, stream); break;
      default: launch_nb<D, 1>(p, nsub, nqt, stream); break;
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const AttnParams& p, hipStream_t stream) {
  switch (p.D) {
    case 32: return launch_d<32>(p, stream);
    case 64: return launch_d<64>(p, stream);
    default: return launch_d<128>(p, stream);
  }
}

}  // namespace rgc
