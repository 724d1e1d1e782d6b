// backward.hip -- gradients of causal GQA self-attention (bf16, MFMA).
//
// Operation: the training pass of the attention the pages run (the 24 q /
// 8 KV model of page "训练3.8B LLM至0.384 CORE，成本998美元 – Hugo Vergnes",
// section 设置, is trained end to end).  For row i of query head h with
// weights w_ij = softmax_j(scale q_i.k_j) over keys j <= i and output
// gradient dO_i:
//   dV_j += w_ij dO_i,  dP_ij = dO_i . v_j,  dS_ij = w_ij (dP_ij - Dlt_i),
//   dQ_i = scale sum_j dS_ij k_j,  dK_j += scale dS_ij q_i,
// where Dlt_i = sum_j w_ij dP_ij = dO_i . o_i, and dK, dV sum over the query
// heads of each KV head's group.
//
// Two kernels, no atomics:
//  * dkdv_kernel: a workgroup owns 128 keys of one (sequence, KV head) (32
//    per wave, K and V in LDS) and walks every query head of the group and
//    every query block of 64 rows at or after its keys (the next block's
//    rows fetched into registers a step ahead, two LDS slots, one barrier a
//    step): S = Q K^T and
//    dP = dO V^T with keys in the MFMA N dimension, so each lane holds one
//    key and P, dS are already the A operand of dV += P^T dO and
//    dK += dS^T Q; dO and Q enter those as transposed fragments
//    (ds_read_b64_tr_b16) of the row-major tiles;
//  * dq_kernel (backward_dq.hip), launched first: a workgroup owns 128
//    query rows of one (sequence, head), forms their Dlt_i = dO_i . o_i
//    (fp32) into the workspace, and walks the 64-key tiles at or before
//    them.
// The weights are recomputed from the forward pass's lse; P and dS are
// rounded to bf16 for the MFMAs, everything accumulates in fp32, and dq, dk,
// dv are rounded once to bf16.
#include "bwd_tiles.h"
#include "launch.h"

namespace rgc {
namespace {

using namespace bwd;

// Cooperative copy of `rows` rows (row stride `gstride` elements) from HBM
// into a swizzled LDS tile; rows at or past `valid` are filled with zeros.
template <int D>
__device__ __forceinline__ void stage_rows(char* tile, const bf16_t* g, int64_t gstride, int rows, int valid,
                                           int tid, int nthreads) {
  constexpr int CH = BTile<D>::CH;
  for (int i = tid; i < rows * CH; i += nthreads) {
    const int r = i / CH, c = i % CH;
    const u32x4 v = r < valid ? ld16(g + (int64_t)r * gstride + 8 * c) : u32x4{0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(tile + BTile<D>::phys(r, c)) = v;
  }
}


constexpr int kKeysPerWave = 32;
constexpr int kDkdvWaves = 4;
constexpr int kDkdvThreads = 64 * kDkdvWaves;
constexpr int kKeyBlock = kKeysPerWave * kDkdvWaves;  // 128 keys per workgroup
constexpr int kQB = 64;                                // query rows per step

// Two slots of (Q, dO, lse, Dlt) for the current and the next query step,
// then K and V of the workgroup's keys (read once, into registers).  The
// slots come first so that every per-step LDS address is a per-lane offset
// plus an immediate below 64 KiB.
template <int D>
struct DkdvLds {
  static constexpr int Q = 0;                              // slot-relative: [64][D]
  static constexpr int DO = Q + kQB * D * 2;               // [64][D]
  static constexpr int LSE = DO + kQB * D * 2;             // [64] fp32, log2 units
  static constexpr int DLT = LSE + kQB * 4;                // [64] fp32
  static constexpr int SLOT_BYTES = DLT + kQB * 4;
  static constexpr int K = 2 * SLOT_BYTES;                 // [128][D]
  static constexpr int V = K + kKeyBlock * D * 2;          // [128][D]
  static constexpr int BYTES = V + kKeyBlock * D * 2;
};

// The staged inputs of one query step: rows of Q and dO, lse and Dlt of its
// 64 queries, and how many of them exist.
template <int D>
struct StepRegs {
  TileRegs<D, kQB, kDkdvThreads> q, d_o;
  float lse, dlt;
  int valid;
};

template <int D>
__device__ __forceinline__ void fetch_step(StepRegs<D>& st, const BwdParams& p, const float* dlt, int b, int h,
                                           int q0, int tid) {
  st.valid = min(kQB, p.S - q0);
  const int64_t off = (int64_t)b * p.q_sb + (int64_t)h * p.q_sh + (int64_t)q0 * p.q_ss;
  const uint32_t row_bytes = (uint32_t)p.q_ss * 2u;
  st.q.fetch(reinterpret_cast<const char*>(reinterpret_cast<const bf16_t*>(p.q) + off), row_bytes, st.valid, tid);
  st.d_o.fetch(reinterpret_cast<const char*>(reinterpret_cast<const bf16_t*>(p.dO) + off), row_bytes, st.valid,
               tid);
  const int64_t row0 = ((int64_t)b * p.Hq + h) * p.S + q0;
  const uint32_t i = (uint32_t)min(tid & (kQB - 1), st.valid - 1);
  st.lse = p.lse[row0 + i];
  st.dlt = dlt[row0 + i];
}

template <int D>
__device__ __forceinline__ void store_step(const StepRegs<D>& st, char* slot, int tid) {
  using L = DkdvLds<D>;
  st.q.store(slot + L::Q, st.valid, tid);
  st.d_o.store(slot + L::DO, st.valid, tid);
  if (tid < kQB) {
    const bool ok = tid < st.valid;
    reinterpret_cast<float*>(slot + L::LSE)[tid] = ok ? st.lse * kAttnLog2e : 0.f;
    reinterpret_cast<float*>(slot + L::DLT)[tid] = ok ? st.dlt : 0.f;
  }
}

// The arithmetic of one step for one wave, in two 32-query halves qm:
// S = Q K^T and dP = dO V^T with the wave's 32 keys in the MFMA N dimension
// (lane holds key my_key; register r holds query q0 + 32qm + 8(r/4) + 4half
// + r%4), the weights P and dS = P (dP - Dlt) rounded to bf16 as A operands,
// then dV += P^T dO and dK += dS^T Q with transposed dO / Q fragments as B
// operands.
//
// One wave runs per SIMD, so the step is software-pipelined by hand as a
// fixed sequence of 4 x (2 KS) matrix-instruction slots: the first half's
// scores, the second half's scores, the first half's dV/dK, the second
// half's dV/dK.  Each slot's LDS operand is read kLookahead slots ahead, and
// the weights of one score value are formed in each slot from two slots
// after the half's scores end, so that the vector work runs under the
// matrix instructions.  Scheduling barriers keep the compiler to this order.
// MASK zeroes the pairs with query < key and rows past S; steps where every
// pair is live skip it.
constexpr int kLookahead = 3;

template <int D, bool MASK>
__device__ __forceinline__ void dkdv_step(const char* slot, int q0, int S, int my_key, float c, int lane,
                                          const u32x4* kf, const u32x4* vf, f32x16* acc_dv, f32x16* acc_dk) {
  using L = DkdvLds<D>;
  constexpr int KS = BTile<D>::KS, DB = BTile<D>::DB;
  constexpr int NS = 2 * KS;    // score slots per half: S and dP over KS k-steps
  constexpr int NA = 4 * DB;    // dV/dK slots per half: 2 k-blocks x DB column blocks x {dV, dK}
  static_assert(NS == NA, "the pipeline assumes as many score as dV/dK slots per half");
  constexpr int NSLOT = 4 * NS;
  constexpr int VPS = 64 / NSLOT;  // weights formed per slot (32 values over the middle half of the slots)
  constexpr int V0 = NS + 2;       // slot of the first weight: two slots after the first half's scores
  constexpr int NF = kLookahead + 1;
  // Each half's scores are complete before its weights start, and each
  // k-block of weights is packed before the first dV/dK slot that uses it.
  static_assert(V0 + 16 / VPS >= 2 * NS + 2, "second half's weights start before its scores end");
  static_assert(V0 + 7 / VPS < 2 * NS && V0 + 15 / VPS < 2 * NS + 2 * DB, "first half's weights are late");
  static_assert(V0 + 23 / VPS < 3 * NS && V0 + 31 / VPS < 3 * NS + 2 * DB, "second half's weights are late");
  const int col = lane & 31, half = lane >> 5;

  // The LDS operand of slot J: Q / dO row fragments for the scores, dO / Q
  // transposed fragments for dV / dK.
  auto operand = [&](auto jc) -> u32x4 {
    constexpr int J = decltype(jc)::value, PH = J / NS, I = J % NS;
    if constexpr (PH < 2) {
      return row_frag<D>(slot + ((I & 1) ? L::DO : L::Q), 32 * PH + col, 2 * (I >> 1) + half);
    } else {
      constexpr int QM = PH - 2, KK = I / (2 * DB), Q = (I >> 1) % DB;
      return tr_frag<D>(slot + ((I & 1) ? L::Q : L::DO), Q, 2 * QM + KK, lane);
    }
  };

  f32x16 sm[2], dp[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int r = 0; r < 16; ++r) sm[h][r] = dp[h][r] = 0.f;
  u32x4 pp[2][2], pds[2][2];
  // Per half: lse and Dlt of rows qa, qa + 8 for k-blocks 0 and 1.
  f32x4 lsd[2][4], dsd[2][4];
  float pv_lo = 0.f, dv_lo = 0.f;
  u32x4 fr[NF];
  static_for<0, kLookahead>([&](auto jc) { fr[decltype(jc)::value] = operand(jc); });
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int qa = 32 * h + 16 * kk + 4 * half;
      lsd[h][2 * kk] = *reinterpret_cast<const f32x4*>(slot + L::LSE + 4 * qa);
      lsd[h][2 * kk + 1] = *reinterpret_cast<const f32x4*>(slot + L::LSE + 4 * (qa + 8));
      dsd[h][2 * kk] = *reinterpret_cast<const f32x4*>(slot + L::DLT + 4 * qa);
      dsd[h][2 * kk + 1] = *reinterpret_cast<const f32x4*>(slot + L::DLT + 4 * (qa + 8));
    }
  __builtin_amdgcn_sched_barrier(0);

  static_for<0, NSLOT>([&](auto jc) {
    constexpr int J = decltype(jc)::value, PH = J / NS, I = J % NS;
    if constexpr (J + kLookahead < NSLOT)
      fr[(J + kLookahead) % NF] = operand(std::integral_constant<int, J + kLookahead>{});
    const u32x4 op = fr[J % NF];
    if constexpr (PH < 2) {
      if constexpr (I & 1) dp[PH] = mfma(op, vf[I >> 1], dp[PH]);
      else sm[PH] = mfma(op, kf[I >> 1], sm[PH]);
    } else {
      constexpr int QM = PH - 2, KK = I / (2 * DB), Q = (I >> 1) % DB;
      if constexpr (I & 1) acc_dk[Q] = mfma(pds[QM][KK], op, acc_dk[Q]);
      else acc_dv[Q] = mfma(pp[QM][KK], op, acc_dv[Q]);
    }
    // VPS weights: values (J - V0) VPS + u of the halves' 2 x 16 score registers.
    static_for<0, VPS>([&](auto uc) {
    constexpr int V = (J - V0) * VPS + decltype(uc)::value;
    if constexpr (V >= 0 && V < 32) {
      constexpr int H = V / 16, R = V % 16, KK = R / 8, E = (R % 8) / 2, T = R % 2;
      constexpr int SEL = 2 * KK + ((R >> 2) & 1);
      const float w = __builtin_amdgcn_exp2f(fmaf(sm[H][R], c, -lsd[H][SEL][R & 3]));
      float pw = w, dw = w * (dp[H][R] - dsd[H][SEL][R & 3]);
      if constexpr (MASK) {
        const int qrow = q0 + 32 * H + 8 * (R >> 2) + 4 * half + (R & 3);
        const bool live = qrow < S && my_key <= qrow;
        pw = live ? pw : 0.f;
        dw = live ? dw : 0.f;
      }
      if constexpr (T == 0) {
        pv_lo = pw;
        dv_lo = dw;
      } else {
        pp[H][KK][E] = pack_bf16x2(pv_lo, pw);
        pds[H][KK][E] = pack_bf16x2(dv_lo, dw);
      }
    }
    });
    __builtin_amdgcn_sched_barrier(0);
  });
}

template <int D>
__global__ void __launch_bounds__(kDkdvThreads, 1) dkdv_kernel(BwdParams p, const float* dlt) {
  using T = BTile<D>;
  using L = DkdvLds<D>;
  constexpr int KS = T::KS, DB = T::DB;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  // Key blocks in order of work, the first (which meets every query block)
  // first, so that the last workgroups to start are the short ones.
  const int kblk = blockIdx.x / (p.B * p.Hkv);
  const int kvh = blockIdx.x % p.Hkv;
  const int b = (blockIdx.x / p.Hkv) % p.B;
  const int group = p.Hq / p.Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int key_blk0 = kblk * kKeyBlock;
  const int key0 = key_blk0 + wave * kKeysPerWave;  // this wave's first key
  const int my_key = key0 + col;                      // the key this lane holds in S and dP
  const float c = p.scale * kAttnLog2e;

  const bf16_t* kg = reinterpret_cast<const bf16_t*>(p.k) + (int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh;
  const bf16_t* vg = reinterpret_cast<const bf16_t*>(p.v) + (int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh;
  const int nvalid = min(kKeyBlock, p.S - key_blk0);
  stage_rows<D>(lds + L::K, kg + (int64_t)key_blk0 * p.kv_ss, p.kv_ss, kKeyBlock, nvalid, tid, kDkdvThreads);
  stage_rows<D>(lds + L::V, vg + (int64_t)key_blk0 * p.kv_ss, p.kv_ss, kKeyBlock, nvalid, tid, kDkdvThreads);

  f32x16 acc_dv[DB], acc_dk[DB];
#pragma unroll
  for (int q = 0; q < DB; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_dv[q][r] = acc_dk[q][r] = 0.f;

  // Steps n = (query head hh, query block qb of 64 rows) over the blocks at
  // or after the workgroup's first key; each step's rows are fetched into
  // registers one step ahead and stored into the other LDS slot after the
  // arithmetic.  Steps alternate between the two slots, two per iteration,
  // so that slot addresses are compile-time offsets.
  const int nqb = (p.S + kQB - 1) / kQB;
  const int qb_first = key_blk0 / kQB;
  const int nsteps = group * (nqb - qb_first);
  int hh = 0, qb = qb_first;  // the step being computed
  StepRegs<D> st;
  fetch_step<D>(st, p, dlt, b, kvh * group, qb * kQB, tid);
  store_step<D>(st, lds, tid);
  __syncthreads();
  // This wave's K and V rows stay in registers as the B operands of S and dP.
  u32x4 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = row_frag<D>(lds + L::K, wave * kKeysPerWave + col, 2 * ks + half);
    vf[ks] = row_frag<D>(lds + L::V, wave * kKeysPerWave + col, 2 * ks + half);
  }
  auto step = [&](auto slot_tag, int n) {
    constexpr int SL = decltype(slot_tag)::value;
    const int q0 = qb * kQB;
    int nhh = hh, nqb_ = qb + 1;
    if (nqb_ == nqb) nqb_ = qb_first, ++nhh;
    const bool more = n + 1 < nsteps;
    if (more) fetch_step<D>(st, p, dlt, b, kvh * group + nhh, nqb_ * kQB, tid);
    const char* slot = lds + SL * L::SLOT_BYTES;
    if (q0 >= key0 + kKeysPerWave - 1 && q0 + kQB <= p.S)  // every pair of the step is live
      dkdv_step<D, false>(slot, q0, p.S, my_key, c, lane, kf, vf, acc_dv, acc_dk);
    else
      dkdv_step<D, true>(slot, q0, p.S, my_key, c, lane, kf, vf, acc_dv, acc_dk);
    if (more) store_step<D>(st, lds + (SL ^ 1) * L::SLOT_BYTES, tid);
    __syncthreads();
    hh = nhh;
    qb = nqb_;
  };
  for (int n = 0; n < nsteps; n += 2) {
    step(std::integral_constant<int, 0>{}, n);
    if (n + 1 < nsteps) step(std::integral_constant<int, 1>{}, n + 1);
  }
  // acc[q] register r holds key row key0 + 8(r/4) + 4half + r%4, column
  // d = 32q + col.
  bf16_t* dkg = reinterpret_cast<bf16_t*>(p.dk) + (int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh;
  bf16_t* dvg = reinterpret_cast<bf16_t*>(p.dv) + (int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh;
#pragma unroll
  for (int q = 0; q < DB; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (key < p.S) {
        dkg[(int64_t)key * p.kv_ss + 32 * q + col] = f32_to_bf16(acc_dk[q][r] * p.scale);
        dvg[(int64_t)key * p.kv_ss + 32 * q + col] = f32_to_bf16(acc_dv[q][r]);
      }
    }
}

template <int D>
hipError_t launch_d(const BwdParams& p, float* dlt, hipStream_t stream) {
  // dQ first: it forms Dlt, which dK/dV reads.
  hipError_t e = launch_dq_bf16(p, dlt, stream);
  if (e != hipSuccess) return e;
  const int nkb = (p.S + kKeyBlock - 1) / kKeyBlock;
  KernelTimer kt_("dkdv_kernel", stream);
  hipLaunchKernelGGL(dkdv_kernel<D>, dim3((unsigned)(p.B * p.Hkv * nkb)), dim3(kDkdvThreads),
                     (size_t)DkdvLds<D>::BYTES, stream, p, (const float*)dlt);
  return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(int B, int S, int Hq) {
  return (((size_t)B * Hq * S * sizeof(float)) + 255) & ~(size_t)255;
}

hipError_t launch_backward_bf16(const BwdParams& p, void* workspace, hipStream_t stream) {
  float* dlt = reinterpret_cast<float*>(workspace);
  switch (p.D) {
    case 32: return launch_d<32>(p, dlt, stream);
    case 64: return launch_d<64>(p, dlt, stream);
    default: return launch_d<128>(p, dlt, stream);
  }
}

}  // namespace rgc
