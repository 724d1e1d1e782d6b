// backward_dq.hip -- dQ of causal GQA self-attention (bf16, MFMA), the
// first of the training pass's two kernels (dK/dV is in backward.hip); it
// also forms Dlt_i = dO_i . o_i, which the dK/dV kernel reads.
//
// For row i of query head h, with weights w_ij = softmax_j(scale q_i.k_j)
// over keys j <= i, dP_ij = dO_i . v_j and Dlt_i = dO_i . o_i:
//   dQ_i = scale sum_j w_ij (dP_ij - Dlt_i) k_j.
// A workgroup owns 128 query rows of one (sequence, head) (32 per wave) and
// walks the 64-key tiles at or before them (three LDS slots, one barrier a
// step): S^T = K Q^T and dP^T = V dO^T with queries in the N dimension (Q
// and dO fragments in registers), so dS^T is the B operand of
// dQ^T += K^T dS^T with K^T read transposed from the K tile; a tile's second
// half updates dQ during the next tile's scores.  The weights are recomputed
// from the forward pass's lse; dS is rounded to bf16 for the MFMAs,
// everything accumulates in fp32, and dq is rounded once to bf16.
#include "bwd_tiles.h"
#include "launch.h"

namespace rgc {
namespace {

using namespace bwd;

// Operands are read this many matrix-instruction slots ahead of their use.
constexpr int kLookahead = 3;

constexpr int kDqWaves = 4;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqRows = 32 * kDqWaves;  // 128 query rows per workgroup
constexpr int kKT = 64;                 // keys per tile
constexpr int kDqSlots = 3;             // LDS slots: the previous, current and next key tile

// One LDS slot holds the (K, V) rows of a key tile.  A step reads the
// current tile and the previous one and stores the next, fetched into
// registers during the step, into the third slot.
template <int D>
struct DqLds {
  static constexpr int K = 0;                   // slot-relative: [64][D]
  static constexpr int V = K + kKT * D * 2;     // [64][D]
  static constexpr int SLOT_BYTES = V + kKT * D * 2;
  static constexpr int BYTES = kDqSlots * SLOT_BYTES;
};

template <int D>
struct KvRegs {
  TileRegs<D, kKT, kDqThreads> k, v;
  int valid;
};

// The dQ arithmetic of one wave.  A key tile is two 32-key halves H; for
// each: S^T = K Q^T and dP^T = V dO^T with the wave's 32 queries in the MFMA
// N dimension (lane holds query qi; register r holds key
// j0 + 32H + 8(r/4) + 4half + r%4), dS^T = P^T (dP^T - Dlt) rounded to bf16
// in the B-operand layout of dQ^T += K^T dS^T, with K^T read transposed from
// the K tile.
//
// One wave runs per SIMD, so the work is software-pipelined by hand across
// tiles.  Step t issues, as a fixed sequence of matrix-instruction slots,
// the scores of half 0 of tile t, the dQ update of half 1 of tile t - 1, the
// scores of half 1 of tile t and the dQ update of half 0 of tile t.  The
// weights of tile t - 1's half 1 are formed under the first group and those
// of tile t's half 0 under the second and third, so that the vector work
// runs under matrix instructions; each slot's LDS operand is read
// kLookahead slots ahead.  Scheduling barriers keep the compiler to this
// order.  PREV is false on a wave's first tile; MASK zeroes the pairs with
// key > query (and rows past S) in both tiles' weights.
template <int D>
struct DqSched {
  static constexpr int KS = BTile<D>::KS, DB = BTile<D>::DB;
  static constexpr int NS = 2 * KS;  // score slots per half: S and dP over KS k-steps
  static constexpr int NA = 2 * DB;  // dQ slots per half: 2 k-blocks x DB column blocks
  // First slots of the phases: previous tile's dQ (B), half 1's scores (C),
  // half 0's dQ (D); half 0's scores start at slot 0.
  static constexpr int PB = NS, PC = NS + NA, PD = 2 * NS + NA, NSLOT = 2 * NS + 2 * NA;
  // Slot of weight value r (0..15) of the previous tile's half 1 (w1) and of
  // the current tile's half 0 (w0, from two slots after its scores end).
  static constexpr int w1(int r) { return r * NS / 16; }
  static constexpr int w0(int r) { return PB + 2 + r * (NS + NA - 2) / 16; }
};

// One entry of dS^T: P^T (dP^T - Dlt) with P^T = exp2(c s - lse2); the dP^T
// accumulator starts at -Dlt, so d is already dP^T - Dlt.  With
// lim = qi - (j0 + 4half) for the current tile's j0 (very negative for a row
// past S), the key at offset off + 4half from j0 is live iff off <= lim.
template <bool MASK>
__device__ __forceinline__ float dq_weight(float s, float d, float lse2, float c, int off, int lim) {
  const float v = __builtin_amdgcn_exp2f(fmaf(s, c, -lse2)) * d;
  if constexpr (MASK) return off <= lim ? v : 0.f;
  return v;
}

// Per-lane LDS offsets, relative to a slot, of the fragments a step reads:
// the row fragment of row col at chunk 2ks + half (rows 32H + col share the
// swizzle of row col, which depends on the row modulo 16), and the low and
// high halves of the transposed fragment of column block q at k-block 0
// (k-block kk lies 16 kk rows further, again the same swizzle).
template <int D>
struct DqOffsets {
  uint32_t row[BTile<D>::KS];
  uint32_t tr[BTile<D>::DB][2];
  __device__ __forceinline__ void init(int lane) {
    using T = BTile<D>;
    const int col = lane & 31, half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) row[ks] = (uint32_t)T::phys(col, 2 * ks + half);
    const int x = lane & 15, beta = (lane >> 4) & 1, h = lane >> 5;
    const int c_lane = 2 * beta + ((x & 3) >> 1), r = 4 * h + (x >> 2);
#pragma unroll
    for (int q = 0; q < T::DB; ++q) {
      tr[q][0] = (uint32_t)(T::phys(r, 4 * q + c_lane) + 8 * (x & 1));
      tr[q][1] = (uint32_t)(T::phys(r + 8, 4 * q + c_lane) + 8 * (x & 1));
    }
  }
};

// io(slot) runs at the end of each slot: the caller's loads and stores of
// the next key tile ride in the schedule there (a no-op where the caller
// moves that tile itself).
struct NoIo {
  template <typename J>
  __device__ __forceinline__ void operator()(J) const {}
};

template <int D, bool PREV, bool MASK, typename IO>
__device__ __forceinline__ void dq_step(const char* cur, const char* prev, const DqOffsets<D>& of, int lim,
                                        float lse2, const f32x16& dpinit, float c, const u32x4* qf,
                                        const u32x4* dof, f32x16* acc, f32x16* sm, f32x16* dp, IO&& io) {
  using L = DqLds<D>;
  using Sc = DqSched<D>;
  constexpr int DB = Sc::DB, PB = Sc::PB, PC = Sc::PC, PD = Sc::PD, NSLOT = Sc::NSLOT;
  constexpr int NF = kLookahead + 1;
  // k-block kk of a half's weights is packed before the first dQ slot that uses it.
  static_assert(Sc::w1(7) < PB && Sc::w1(15) < PB + DB, "previous tile's weights are late");
  static_assert(Sc::w0(7) < PD && Sc::w0(15) < PD + DB, "current tile's weights are late");
  static_assert(Sc::w0(15) < NSLOT, "weight placed past the last slot");
  constexpr int RB = BTile<D>::ROW_BYTES;
  // Phase of slot J: scores of half 0 (A), dQ of the previous tile's half 1
  // (B), scores of half 1 (C), dQ of half 0 (D).  Addresses are formed where
  // the operand is read, kLookahead slots ahead, so their adds spread over
  // the slots.
  auto operand = [&](auto jc) -> u32x4 {
    constexpr int J = decltype(jc)::value;
    if constexpr (J < PB || (J >= PC && J < PD)) {
      constexpr int H = J < PB ? 0 : 1, I = J < PB ? J : J - PC;
      return *reinterpret_cast<const u32x4*>(cur + of.row[I >> 1] + ((I & 1) ? L::V : L::K) + 32 * H * RB);
    } else if constexpr (J < PC) {
      constexpr int I = J - PB, Q = I % DB, R0 = L::K + (2 + I / DB) * 16 * RB;
      return tr_frag_at(prev + of.tr[Q][0] + R0, prev + of.tr[Q][1] + R0);
    } else {
      constexpr int I = J - PD, Q = I % DB, R0 = L::K + (I / DB) * 16 * RB;
      return tr_frag_at(cur + of.tr[Q][0] + R0, cur + of.tr[Q][1] + R0);
    }
  };
  constexpr auto needed = [](int j) constexpr { return PREV || j < PB || j >= PC; };

  u32x4 pf[2][2];  // [half][k-block]: half 1 of the previous tile, half 0 of this one
  float lo[2] = {0.f, 0.f};
  u32x4 fr[NF];
  static_for<0, kLookahead>([&](auto jc) {
    constexpr int J = decltype(jc)::value;
    if constexpr (needed(J)) fr[J % NF] = operand(jc);
  });
  __builtin_amdgcn_sched_barrier(0);

  static_for<0, NSLOT>([&](auto jc) {
    constexpr int J = decltype(jc)::value;
    if constexpr (J + kLookahead < NSLOT && needed(J + kLookahead))
      fr[(J + kLookahead) % NF] = operand(std::integral_constant<int, J + kLookahead>{});
    if constexpr (J < PB || (J >= PC && J < PD)) {
      constexpr int H = J < PB ? 0 : 1, I = J < PB ? J : J - PC;
      const f32x16 z = {};
      if constexpr (I & 1) dp[H] = mfma(fr[J % NF], dof[I >> 1], I < 2 ? dpinit : dp[H]);
      else sm[H] = mfma(fr[J % NF], qf[I >> 1], I < 2 ? z : sm[H]);
    } else if constexpr (J < PC) {
      if constexpr (PREV) {
        constexpr int I = J - PB;
        acc[I % DB] = mfma(fr[J % NF], pf[1][I / DB], acc[I % DB]);
      }
    } else {
      constexpr int I = J - PD;
      acc[I % DB] = mfma(fr[J % NF], pf[0][I / DB], acc[I % DB]);
    }
    static_for<0, 16>([&](auto rc) {
      constexpr int R = decltype(rc)::value, KK = R / 8, E = (R % 8) / 2;
      constexpr int OFF = 8 * (R >> 2) + (R & 3);  // key offset within the half, less 4half
      if constexpr (PREV && Sc::w1(R) == J) {
        const float v = dq_weight<MASK>(sm[1][R], dp[1][R], lse2, c, 32 + OFF - kKT, lim);
        if constexpr (R % 2 == 0) lo[1] = v;
        else pf[1][KK][E] = pack_bf16x2(lo[1], v);
      }
      if constexpr (Sc::w0(R) == J) {
        const float v = dq_weight<MASK>(sm[0][R], dp[0][R], lse2, c, OFF, lim);
        if constexpr (R % 2 == 0) lo[0] = v;
        else pf[0][KK][E] = pack_bf16x2(lo[0], v);
      }
    });
    io(jc);
    __builtin_amdgcn_sched_barrier(0);
  });
}

// The last dQ update of a wave: half 1 of its last tile, whose K rows are in
// `prev` (lim as for the step after that tile).
template <int D, bool MASK>
__device__ __forceinline__ void dq_tail(const char* prev, const DqOffsets<D>& of, int lim, float lse2, float c,
                                        f32x16* acc, const f32x16* sm, const f32x16* dp) {
  using L = DqLds<D>;
  constexpr int DB = BTile<D>::DB;
  u32x4 pf[2];
  static_for<0, 8>([&](auto ec) {
    constexpr int E2 = decltype(ec)::value, KK = E2 / 4, E = E2 % 4;
    constexpr int R0 = 2 * E2, R1 = R0 + 1;
    const float v0 = dq_weight<MASK>(sm[1][R0], dp[1][R0], lse2, c, 32 + 8 * (R0 >> 2) + (R0 & 3) - kKT, lim);
    const float v1 = dq_weight<MASK>(sm[1][R1], dp[1][R1], lse2, c, 32 + 8 * (R1 >> 2) + (R1 & 3) - kKT, lim);
    pf[KK][E] = pack_bf16x2(v0, v1);
  });
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int q = 0; q < DB; ++q) {
      const int r0 = (2 + kk) * 16 * BTile<D>::ROW_BYTES;
      acc[q] = mfma(tr_frag_at(prev + L::K + of.tr[q][0] + r0, prev + L::K + of.tr[q][1] + r0), pf[kk], acc[q]);
    }
}

template <int D>
__global__ void __launch_bounds__(kDqThreads, 1) dq_kernel(BwdParams p, float* dlt) {
  using T = BTile<D>;
  using L = DqLds<D>;
  constexpr int KS = T::KS, DB = T::DB;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int nqt = (p.S + kDqRows - 1) / kDqRows;
  const int qt = nqt - 1 - (int)(blockIdx.x / (p.B * p.Hq));  // heaviest tiles first
  const int h = blockIdx.x % p.Hq;
  const int b = (blockIdx.x / p.Hq) % p.B;
  const int kvh = h / (p.Hq / p.Hkv);
  // The wave index passes through readfirstlane so that the compiler sees
  // it, and every per-wave loop bound below, as uniform.
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const float c = p.scale * kAttnLog2e;

  const int s_base = qt * kDqRows + wave * 32;
  const int qi = s_base + col;  // this lane's query row
  const bool qvalid = qi < p.S;
  const int64_t qoff = (int64_t)b * p.q_sb + (int64_t)qi * p.q_ss + (int64_t)h * p.q_sh;
  u32x4 qf[KS], dof[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = qvalid ? ld16(reinterpret_cast<const bf16_t*>(p.q) + qoff + 16 * ks + 8 * half) : u32x4{0, 0, 0, 0};
    dof[ks] = qvalid ? ld16(reinterpret_cast<const bf16_t*>(p.dO) + qoff + 16 * ks + 8 * half) : u32x4{0, 0, 0, 0};
  }
  const float lse2 = qvalid ? p.lse[((int64_t)b * p.Hq + h) * p.S + qi] * kAttnLog2e : 0.f;
  // Dlt_i = dO_i . o_i in fp32: lanes l and l ^ 32 each hold half of the
  // query's dO and o rows.  This kernel runs before the dK/dV kernel and
  // leaves Dlt in the workspace for it.
  float dl = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4 ov =
        qvalid ? ld16(reinterpret_cast<const bf16_t*>(p.o) + qoff + 16 * ks + 8 * half) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dl = fmaf(bf16_lo(dof[ks][e]), bf16_lo(ov[e]), dl);
      dl = fmaf(bf16_hi(dof[ks][e]), bf16_hi(ov[e]), dl);
    }
  }
  dl += __shfl_xor(dl, 32, 64);
  if (qvalid && half == 0) dlt[((int64_t)b * p.Hq + h) * p.S + qi] = dl;

  f32x16 acc[DB], sm[2], dp[2];
#pragma unroll
  for (int q = 0; q < DB; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[q][r] = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) sm[0][r] = sm[1][r] = dp[0][r] = dp[1][r] = 0.f;

  const int last_row = min(p.S, (qt + 1) * kDqRows) - 1;  // the workgroup's last query
  const int nkt = last_row / kKT + 1;
  const int wave_last = s_base < p.S ? min(s_base + 31, p.S - 1) : -1;
  const int my_last = wave_last >= 0 ? wave_last / kKT : -1;  // this wave's last key tile
  const bool rows_full = s_base + 31 < p.S;
  const char* kg = reinterpret_cast<const char*>(reinterpret_cast<const bf16_t*>(p.k) + (int64_t)b * p.kv_sb +
                                                 (int64_t)kvh * p.kv_sh);
  const char* vg = reinterpret_cast<const char*>(reinterpret_cast<const bf16_t*>(p.v) + (int64_t)b * p.kv_sb +
                                                 (int64_t)kvh * p.kv_sh);
  const uint32_t row_bytes = (uint32_t)p.kv_ss * 2u;
  KvRegs<D> st;
  using TR = TileRegs<D, kKT, kDqThreads>;
  const uint32_t voff = TR::full_voff(tid, row_bytes), soff = TR::full_soff(tid);
  auto fetch = [&](int j0) {
    st.valid = min(kKT, p.S - j0);
    const int64_t off = (int64_t)j0 * p.kv_ss * 2;
    if (st.valid == kKT) {
      st.k.fetch_full(kg + off, row_bytes, voff);
      st.v.fetch_full(vg + off, row_bytes, voff);
    } else {
      st.k.fetch(kg + off, row_bytes, st.valid, tid);
      st.v.fetch(vg + off, row_bytes, st.valid, tid);
    }
  };
  auto store = [&](char* slot) {
    if (st.valid == kKT) {
      st.k.store_full(slot + L::K, soff);
      st.v.store_full(slot + L::V, soff);
    } else {
      st.k.store(slot + L::K, st.valid, tid);
      st.v.store(slot + L::V, st.valid, tid);
    }
  };
  DqOffsets<D> of;
  of.init(lane);
  fetch(0);
  store(lds);
  __syncthreads();
  // Step t (t < nkt) works on tile t in slot t % 3 and tile t - 1 in slot
  // (t - 1) % 3, and stores tile t + 1 into slot (t + 1) % 3, which tile
  // t - 2 last held (read in step t - 1, before that step's barrier).  One
  // more pass, t = nkt, runs the last waves' tails.  Every wave passes one
  // barrier per step, whichever of the loops below it is in.
  //
  // Tiles t < nfull have every key before every row of the wave; the wave's
  // last tile (the diagonal one) and every tile of a wave with rows past S
  // are masked.  Steps t in [1, t_hot) run the unmasked step with the next
  // tile's loads and stores inside its schedule, which needs that tile to
  // exist and be full; the remaining steps (masked, or before a ragged last
  // tile) and the tails follow in a general loop.
  const int nfull = rows_full ? (s_base + 1) / kKT : 0;
  const int t_hot = min(nfull, min(nkt - 1, p.S / kKT - 1));
  // The slot offset passes through readfirstlane so that the compiler keeps
  // it as one scalar per step instead of strength-reducing every fragment
  // address of the step into its own induction variable.
  auto slot_of = [&](int t) {
    return lds + __builtin_amdgcn_readfirstlane((t % kDqSlots) * L::SLOT_BYTES);
  };
  auto lim_of = [&](int t) { return qvalid ? qi - (t * kKT + 4 * half) : -(1 << 20); };
  auto advance = [&](int t) {  // store tile t + 1, fetched during step t, and wait for every wave
    if (t + 1 < nkt) store(slot_of(t + 1));
    __syncthreads();
  };
  f32x16 dpinit;  // the dP^T accumulators start at -Dlt of the lane's query
#pragma unroll
  for (int r = 0; r < 16; ++r) dpinit[r] = -dl;
  if (1 < nkt) fetch(kKT);
  if (my_last >= 0) {
    if (nfull > 0) dq_step<D, false, false>(lds, lds, of, lim_of(0), lse2, dpinit, c, qf, dof, acc, sm, dp, NoIo{});
    else dq_step<D, false, true>(lds, lds, of, lim_of(0), lse2, dpinit, c, qf, dof, acc, sm, dp, NoIo{});
  }
  advance(0);
  int t = 1;
  for (; t < t_hot; ++t) {
    // Tile t + 1 (full): its 2N chunk loads go out one per slot from slot 1,
    // and its stores into slot (t + 1) % 3 one per slot of the last phase.
    const int64_t goff = (int64_t)(t + 1) * kKT * p.kv_ss * 2;
    const char* kn = kg + goff;
    const char* vn = vg + goff;
    char* nxt = slot_of(t + 1);
    auto io = [&](auto jc) {
      constexpr int J = decltype(jc)::value, N = TR::N;
      if constexpr (J >= 1 && J < 1 + N) st.k.template fetch_chunk<J - 1>(kn, row_bytes, voff);
      if constexpr (J >= 1 + N && J < 1 + 2 * N) st.v.template fetch_chunk<J - 1 - N>(vn, row_bytes, voff);
      constexpr int PD = DqSched<D>::PD;
      if constexpr (J >= PD && J < PD + N) st.k.template store_chunk<J - PD>(nxt + L::K, soff);
      if constexpr (J >= PD + N && J < PD + 2 * N) st.v.template store_chunk<J - PD - N>(nxt + L::V, soff);
    };
    static_assert(2 * TR::N <= DqSched<D>::NA && 1 + 2 * TR::N <= DqSched<D>::PD,
                  "the next tile's loads and stores fit their phases");
    dq_step<D, true, false>(slot_of(t), slot_of(t + kDqSlots - 1), of, lim_of(t), lse2, dpinit, c, qf, dof, acc, sm,
                            dp, io);
    __syncthreads();
  }
  for (; t <= nkt; ++t) {
    if (t + 1 < nkt) fetch((t + 1) * kKT);
    if (t <= my_last)
      dq_step<D, true, true>(slot_of(t), slot_of(t + kDqSlots - 1), of, lim_of(t), lse2, dpinit, c, qf, dof, acc,
                             sm, dp, NoIo{});
    else if (my_last >= 0 && t == my_last + 1)
      dq_tail<D, true>(slot_of(t + kDqSlots - 1), of, lim_of(t), lse2, c, acc, sm, dp);
    if (t == nkt) break;
    advance(t);
  }
  // acc[q] register r holds d = 32q + 8(r/4) + 4half + r%4 of query qi.
  if (qvalid) {
    bf16_t* dqr = reinterpret_cast<bf16_t*>(p.dq) + qoff;
#pragma unroll
    for (int q = 0; q < DB; ++q)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * q + 8 * q4 + 4 * half;
        u32x2 wv;
        wv[0] = pack_bf16x2(acc[q][4 * q4] * p.scale, acc[q][4 * q4 + 1] * p.scale);
        wv[1] = pack_bf16x2(acc[q][4 * q4 + 2] * p.scale, acc[q][4 * q4 + 3] * p.scale);
        *reinterpret_cast<u32x2*>(dqr + d) = wv;
      }
  }
}

}  // namespace

hipError_t launch_dq_bf16(const BwdParams& p, float* dlt, hipStream_t stream) {
  const int nqt = (p.S + kDqRows - 1) / kDqRows;
  const dim3 grid((unsigned)(p.B * p.Hq * nqt)), block(kDqThreads);
  KernelTimer kt_("dq_kernel", stream);
  switch (p.D) {
    case 32: hipLaunchKernelGGL(dq_kernel<32>, grid, block, (size_t)DqLds<32>::BYTES, stream, p, dlt); break;
    case 64: hipLaunchKernelGGL(dq_kernel<64>, grid, block, (size_t)DqLds<64>::BYTES, stream, p, dlt); break;
    default: hipLaunchKernelGGL(dq_kernel<128>, grid, block, (size_t)DqLds<128>::BYTES, stream, p, dlt); break;
  }
  return hipGetLastError();
}

}  // namespace rgc
