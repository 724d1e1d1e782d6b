// prefill.hip -- causal GQA attention of a block of query rows over the bf16
// cache, on the gfx950 matrix cores.
//
// Operation (page "750美元从零训练3个LLM：一位开发者的实战复盘", section V2;
// page "训练3.8B LLM至0.384 CORE，成本998美元 – Hugo Vergnes", sections 设置
// and 无效的方法; the m.nxbn.cn build-an-LLM page, section 3.1): row s of
// sequence b at slot p attends to slots 0..p of its KV head.
//
// A dense contraction (QK^T then PV) on bf16 MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//  * a workgroup owns one KV head of one sequence and 256 query rows drawn
//    from ALL the query heads of that KV head: rows are (position, head)
//    pairs in position-major order, so every K/V tile the workgroup stages
//    in LDS serves each query head of the group, and the 256 rows span only
//    256/g positions (g = query heads per KV head), which keeps the causal
//    extent of its eight waves within a tile of each other;
//  * eight waves of 32 rows; waves w and w+4 share a SIMD.  The waves run a
//    ping-pong schedule: every tile step is split into a matrix phase (the
//    previous tile's O^T += V^T P^T and this tile's S^T = K Q^T, 32 MFMAs)
//    and a vector phase (mask, online softmax, probabilities rounded to
//    bf16), and waves 0-3 run their matrix phase while waves 4-7 run their
//    vector phase and vice versa, with a workgroup barrier at every phase
//    change.  The softmax of one wave thus issues beside the other wave's
//    matrix instructions instead of between its own;
//  * scores are computed transposed, S^T = K Q^T (keys in the MFMA M
//    dimension): a lane holds one query's column, so the softmax max and sum
//    are in-lane except one v_permlane32_swap with the lane 32 away, and the
//    probabilities are already in the B-operand layout of O^T = V^T P^T --
//    P never leaves registers;
//  * 64-key K and V tiles go HBM -> LDS by direct copies
//    (global_load_lds_dwordx4, no registers) into a 5-slot ring, issued in
//    the vector phase three tiles ahead of their first use; each wave waits
//    only for its own copies of the tile the next phase needs, and the phase
//    barrier publishes it.
//    Both tiles stay row-major in LDS with a per-row XOR swizzle of their
//    16-byte chunks: K fragments (A operand of S^T) are conflict-free
//    16-byte reads, and V^T fragments (A operand of O^T) come straight from
//    the row-major V tile through ds_read_b64_tr_b16, the gfx950 transposing
//    LDS read;
//  * the row sums add the probabilities in fp32 before they are rounded to
//    bf16 for the PV product (each weight is then off by at most half a
//    bf16 ulp, unbiased); no matrix-pipeline instruction (such as the packed
//    bf16 dot) runs in the vector phase, where it would stall the other
//    wave's matrix instructions;
//  * the running max is only raised (and O rescaled) when a tile's max
//    exceeds it by more than 2^8, so the rescale is almost never taken; p is
//    then at most 256, exact in fp32 and within bf16 range.  The tile max
//    itself is only computed on a wave's first tile (where it becomes the
//    running max) and when some lane's tile sum of p passes 2^8 (a necessary
//    condition for a p past 2^8) -- the common tile does no max reduction;
//  * the causal mask is applied on diagonal tiles only; tiles past a wave's
//    last row are skipped (the wave still keeps the barriers);
//  * work order: (sequence, KV head) units stay on one XCD (shared L2),
//    heaviest row blocks first; a grid with more row blocks than compute
//    units runs one persistent workgroup per compute unit, each walking a
//    list of row blocks dealt in snake order;
//  * the output rows leave through LDS as whole rows (a store instruction
//    covers D/8 lanes per row).
#include <atomic>
#include <type_traits>

#include "common.h"

#include "launch.h"
#include "lds_ring.h"
#include "mfma_attn.h"

namespace rgc {
namespace {

constexpr float kLog2e = kAttnLog2e;
constexpr float kLn2 = kAttnLn2;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;  // (position, head) rows per workgroup
constexpr int kKT = 64;             // keys per tile
constexpr int kSlots = 5;           // LDS ring (K and V tile per slot)
constexpr int kXcds = 8;            // MI355X: workgroup i is dispatched to XCD i % 8
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr float kSumTrigger = 256.0f;      // 2^kRescaleThreshold

// LDS layout: kSlots K tiles, then kSlots V tiles, each row-major
// [64 keys][D] in 16-byte chunks; chunk c of row r sits at chunk c ^ swz(r).
//  K: swz = r % CH, so the 16 rows of one K-fragment read hit 16 chunks.
//  V: swz = 4 * tv(r), an XOR of the 32-row d-block index by tv(r) (the low
//     bits of r that vary inside a transposed read), which spreads the 4
//     rows x 4 chunks of a half-wave read over all 64 banks.
template <int D>
struct Tile {
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int KS = D / 16;                  // k-steps of QK^T
  static constexpr int DB = D / 32;                  // 32-row blocks of O^T
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int MAT_BYTES = kKT * ROW_BYTES;  // one K or V tile
  static constexpr int V_REGION = kSlots * MAT_BYTES;
  static constexpr int LDS_BYTES = 2 * kSlots * MAT_BYTES;
  static constexpr int PIECES = MAT_BYTES / 1024;    // 1 KB pieces per tile
  static constexpr int LOADS = 2 * PIECES / kWaves;  // 16-byte pieces per lane per tile
  static __device__ __forceinline__ int swz_k(int r) { return r % CH; }
  static __device__ __forceinline__ constexpr int tv(int r) {
    return D == 128 ? (r & 3) : D == 64 ? ((r >> 1) & 1) : 0;
  }
  // The lane's piece i: matrix (0 = K, 1 = V), row and logical chunk.
  static __device__ __forceinline__ void piece(int wave, int lane, int i, int& mat, int& r, int& c, int& P) {
    const int g = wave * LOADS + i;
    mat = g / PIECES;
    P = (g % PIECES) * 64 + lane;
    r = P / CH;
    const int pc = P % CH;
    c = pc ^ (mat == 0 ? swz_k(r) : 4 * tv(r));
  }
};

// Tile copy: wave w's i-th piece is 1 KB of a slot (lane l at byte 16 l);
// the lane fetches the logical chunk stored there.
template <int D>
struct Stager {
  uint32_t goff[Tile<D>::LOADS];  // byte offset in HBM from the tile's first row
  uint32_t lblk;                  // LDS byte offset of the wave's first 1 KB block in slot 0 (wave-uniform)
  bool v;                         // the wave copies V (else K) (wave-uniform)
};

// A wave's LOADS pieces are consecutive 1 KB blocks of one matrix (PIECES is
// a multiple of LOADS), so one base and constant steps address them.
template <int D>
__device__ __forceinline__ void make_stager(Stager<D>& sg, int64_t kv_ss, int wave, int lane) {
  using T = Tile<D>;
  static_assert(T::PIECES % T::LOADS == 0, "a wave's pieces stay in one matrix");
  static_assert(T::LOADS >= 1 && T::LOADS <= 4, "dma_tile issues up to four copies");
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i) {
    int mat, r, c, P;
    T::piece(wave, lane, i, mat, r, c, P);
    sg.goff[i] = (uint32_t)(r * kv_ss * 2 + 16 * c);
  }
  const int g = wave * T::LOADS;
  sg.v = g >= T::PIECES;
  sg.lblk = (uint32_t)((sg.v ? T::V_REGION : 0) + 1024 * (g % T::PIECES));
}

// Copy tile [j0, j0+64) into ring slot SLOT.  Rows past kmax (only in a
// workgroup's last tile) are clamped to kmax: their keys are masked and
// their probabilities are 0, so the clamped (finite, written) rows never
// reach a result and no unwritten cache slot is read.
template <int D, int SLOT>
__device__ __forceinline__ void dma_tile(const Stager<D>& sg, uint32_t lds0, const char* kb, const char* vb,
                                         int64_t kv_ss, int j0, int kmax, int wave, int lane) {
  using T = Tile<D>;
  const uint32_t lb = lds0 + sg.lblk;
  if (j0 + kKT - 1 <= kmax) {
    const char* base = (sg.v ? vb : kb) + (int64_t)j0 * kv_ss * 2;
    dma16<SLOT * T::MAT_BYTES>(base, sg.goff[0], lb);
    if constexpr (T::LOADS > 1) dma16<SLOT * T::MAT_BYTES + 1024>(base, sg.goff[1], lb);
    if constexpr (T::LOADS > 2) dma16<SLOT * T::MAT_BYTES + 2048>(base, sg.goff[2], lb);
    if constexpr (T::LOADS > 3) dma16<SLOT * T::MAT_BYTES + 3072>(base, sg.goff[3], lb);
  } else {
    int key[T::LOADS], c[T::LOADS];
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      int mat, r, P;
      T::piece(wave, lane, i, mat, r, c[i], P);
      key[i] = min(j0 + r, kmax);
    }
    const char* base = sg.v ? vb : kb;
    dma16_v<SLOT * T::MAT_BYTES>(base + (int64_t)key[0] * kv_ss * 2 + 16 * c[0], lb);
    if constexpr (T::LOADS > 1) dma16_v<SLOT * T::MAT_BYTES + 1024>(base + (int64_t)key[1] * kv_ss * 2 + 16 * c[1], lb);
    if constexpr (T::LOADS > 2) dma16_v<SLOT * T::MAT_BYTES + 2048>(base + (int64_t)key[2] * kv_ss * 2 + 16 * c[2], lb);
    if constexpr (T::LOADS > 3) dma16_v<SLOT * T::MAT_BYTES + 3072>(base + (int64_t)key[3] * kv_ss * 2 + 16 * c[3], lb);
  }
}

template <int D>
struct WaveCtx {
  u32x4 qf[D / 16];          // Q^T fragments (B operand)
  const char* kp[D / 16];    // K-fragment address in slot 0, per k-step
  const char* vp[D / 32];    // V^T-fragment address in slot 0, per d-block
  f32x16 acc_o[D / 32];
  f32x16 s[2];               // S^T of the tile between its matrix and vector phases
  u32x4 pf[4];               // P^T (bf16) of the tile between its vector and matrix phases
  float m_run, l_run;
  float c;                   // scale * log2(e)
  int mask_base;             // first + pos(column) - 4*half: key offset limit is mask_base - j0
};

// Matrix phase: O^T += V^T P^T for the tile in slot SV (if PV), then
// S^T = K Q^T for the tile in slot SK (if S).  S^T block kb holds keys
// 32kb + 8(r/4) + 4half + r%4 of register r.  The LDS fragments stream
// through a ring of eight registers: each MFMA's operand is read seven
// MFMAs ahead of it (about 220 cycles of matrix work, more than an LDS read
// takes while the other waves of its group read too).  The S MFMAs
// alternate the two key blocks so that neighbouring MFMAs are independent.
template <int D, int SK, int SV, bool PV, bool S>
__device__ __forceinline__ void mfma_phase(WaveCtx<D>& w) {
  using T = Tile<D>;
  constexpr int KS = T::KS, DB = T::DB;
  constexpr int NPV = PV ? 4 * DB : 0;       // PV: kk-major, DB fragments per 16-key step
  constexpr int N = NPV + (S ? 2 * KS : 0);  // S: per k-step, key blocks 0 and 1
  constexpr int F = 8;                       // fragments in registers: F - 1 loads ahead
  if (S) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) w.s[kb][r] = 0.f;
  }
  auto load = [&](int i) -> u32x4 {
    if (i < NPV) return vt_frag<T::ROW_BYTES>(w.vp[i % DB] + SV * T::MAT_BYTES + (i / DB) * 16 * T::ROW_BYTES);
    const int j = i - NPV;
    return *reinterpret_cast<const u32x4*>(w.kp[j >> 1] + SK * T::MAT_BYTES + (j & 1) * 32 * T::ROW_BYTES);
  };
  auto mma = [&](int i, u32x4 f) {
    if (i < NPV) {
      w.acc_o[i % DB] = mfma(f, w.pf[i / DB], w.acc_o[i % DB]);
    } else {
      const int j = i - NPV;
      w.s[j & 1] = mfma(f, w.qf[j >> 1], w.s[j & 1]);
    }
  };
  if (N == 0) return;
  u32x4 f[F];
#pragma unroll
  for (int i = 0; i < F - 1 && i < N; ++i) f[i] = load(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + F - 1 < N) f[(i + F - 1) % F] = load(i + F - 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(i, f[i % F]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Vector phase of the tile starting at key j0: mask (diagonal tiles),
// online softmax (log2 domain), P^T rounded to bf16 into w.pf.
template <int D, bool FIRST>
__device__ __forceinline__ void softmax_phase(WaveCtx<D>& w, int j0, bool mask) {
  constexpr int DB = Tile<D>::DB;
  if (mask) {  // wave-uniform: diagonal tiles only
    // Keep key offsets <= lim.  Each score is clamped from above by +inf
    // (kept) or -inf (masked): the bound's sign is the sign of lim - off.
    // Integer and min instructions only, so no per-element comparison
    // result occupies a scalar register pair.
    const int lim = w.mask_base - j0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = lim - (32 * kb + 8 * (r >> 2) + (r & 3));
        const float bound = __builtin_bit_cast(float, ((uint32_t)d & 0x80000000u) | 0x7F800000u);
        w.s[kb][r] = fminf(w.s[kb][r], bound);
      }
  }
  // p = 2^(s*c - m) with the running max m; the row sum adds p in fp32 and
  // the PV product takes p rounded to bf16.
  float ps;
  auto probs = [&]() {
    float ps0 = 0.f, ps1 = 0.f, ps2 = 0.f, ps3 = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(w.s[kk >> 1][8 * (kk & 1) + 2 * e], w.c, -w.m_run));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(w.s[kk >> 1][8 * (kk & 1) + 2 * e + 1], w.c, -w.m_run));
        w.pf[kk][e] = pack_bf16x2(p0, p1);
        if (e & 1) {
          ps2 += p0;
          ps3 += p1;
        } else {
          ps0 += p0;
          ps1 += p1;
        }
      }
    }
    ps = (ps0 + ps1) + (ps2 + ps3);
  };
  auto tile_max = [&]() {
    float m0 = fmaxf(fmaxf(w.s[0][0], w.s[0][1]), w.s[0][2]);
    float m1 = fmaxf(fmaxf(w.s[1][0], w.s[1][1]), w.s[1][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
      m0 = fmaxf(fmaxf(m0, w.s[0][r]), w.s[0][r + 1]);
      m1 = fmaxf(fmaxf(m1, w.s[1][r]), w.s[1][r + 1]);
    }
    m0 = fmaxf(fmaxf(m0, w.s[0][15]), m1);
    m0 = fmaxf(m0, w.s[1][15]);
    return max_halves(m0) * w.c;
  };
  if constexpr (FIRST) {
    // A wave's first tile (m = -inf, O = 0, l = 0): the tile max becomes the
    // running max, then the probabilities are formed once.  Key 0 is kept in
    // every column, so the max is finite.
    w.m_run = tile_max();
    probs();
    w.l_run = ps;
    return;
  }
  probs();
  // The running max is raised (and O rescaled) only when the tile's max
  // exceeds it by more than the threshold, i.e. only if some p > 2^8 -- and
  // then the lane's sum of p exceeds 2^8 as well.  So the tile max is taken
  // only on tiles where some lane's sum does (a wave's first tile, where
  // m = -inf gives p = inf; a new max past the threshold; overflow): a rare,
  // wave-uniform branch that raises m, rescales and recomputes p.
  if (__builtin_amdgcn_ballot_w64(!(ps <= kSumTrigger))) {
    const float tmax = tile_max();
    const float m_new = tmax > w.m_run + kRescaleThreshold ? tmax : w.m_run;
    float alpha = __builtin_amdgcn_exp2f(w.m_run - m_new);  // 0 on the first tile
    // alpha passes through an empty asm, so the multiplications below
    // cannot be hoisted out of this rare path.
    asm volatile("; rescale" : "+v"(alpha));
    w.m_run = m_new;
    w.l_run *= alpha;
#pragma unroll
    for (int q = 0; q < DB; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) w.acc_o[q][r] *= alpha;
    probs();
  }
  w.l_run += ps;
}

// Per-wave bounds of the tile loop (wave-uniform).
struct WaveTiles {
  int last;       // last tile with a key of this wave (-1: no rows)
  int diag_from;  // first tile that needs the causal mask
};

// The wave's program: for each tile k its matrix phase (tile k-1's PV and
// tile k's S) then its vector phase (tile k's softmax), with a barrier
// after each.  Both groups run this one program, group B (waves 4-7) one
// barrier behind group A (waves 0-3): between two barriers the A wave of a
// SIMD runs a matrix phase while its B wave runs a vector phase, and the
// other way round in the next interval.
//
// The ring: the vector phase of tile t starts the wave's copy of tile t+3
// into the slot tile t-2 used (its last readers, the matrix phases of tile
// t-1 in both groups, are behind a barrier); the copies issue there, beside
// the other group's matrix phase, because the matrix phase is the longer of
// the two (its LDS fragment reads).  The matrix phase of tile t ends by
// waiting for the wave's copy of tile t+1 (started two vector phases
// earlier); the barrier after it publishes tile t+1, whose first reader is
// the matrix phase of tile t+1 in group A, two barriers later.
// SLOT = k % kSlots.
template <int D, int SLOT>
__device__ __forceinline__ void matrix_step(WaveCtx<D>& w, const Stager<D>& sg, uint32_t lds0, const char* kb,
                                            const char* vb, int64_t kv_ss, int k, int nkt, int kmax,
                                            const WaveTiles& wt, int wave, int lane) {
  using T = Tile<D>;
  constexpr int SPREV = (SLOT + kSlots - 1) % kSlots;
  // k < nkt here.  A wave past its last tile still forms S (discarded: no
  // vector phase follows) in the step that adds its last PV, so the loop
  // carries one form of the phase.
  if (k == 0) {
    if (wt.last >= 0) mfma_phase<D, SLOT, SPREV, false, true>(w);
  } else if (k - 1 <= wt.last) {
    mfma_phase<D, SLOT, SPREV, true, true>(w);
  }
  // tile k+1 landed: the copy of tile k+2 may still be in flight
  if (k + 2 < nkt) tile_dma_wait<T::LOADS>();
  else tile_dma_wait<0>();
  phase_barrier();
}

template <int D, int SLOT, bool FIRST = false>
__device__ __forceinline__ void vector_step(WaveCtx<D>& w, const Stager<D>& sg, uint32_t lds0, const char* kb,
                                            const char* vb, int64_t kv_ss, int t, int nkt, int kmax,
                                            const WaveTiles& wt, int wave, int lane) {
  if (t + 3 < nkt) dma_tile<D, (SLOT + 3) % kSlots>(sg, lds0, kb, vb, kv_ss, (t + 3) * kKT, kmax, wave, lane);
  if (t <= wt.last) softmax_phase<D, FIRST>(w, t * kKT, t >= wt.diag_from);
  phase_barrier();
}

template <int D, int SLOT>
__device__ __forceinline__ void tile_step(WaveCtx<D>& w, const Stager<D>& sg, uint32_t lds0, const char* kb,
                                          const char* vb, int64_t kv_ss, int k, int nkt, int kmax,
                                          const WaveTiles& wt, int wave, int lane) {
  matrix_step<D, SLOT>(w, sg, lds0, kb, vb, kv_ss, k, nkt, kmax, wt, wave, lane);
  vector_step<D, SLOT>(w, sg, lds0, kb, vb, kv_ss, k, nkt, kmax, wt, wave, lane);
}

// One work item: row block rb of unit (sequence b, KV head kvh).  Every
// wave of the workgroup runs it and passes the same barriers, so items
// chain in a persistent workgroup; an item that needs no work (rows past a
// document's end, a capacity violation) is skipped by the whole workgroup.
// ADD: the epilogue adds p.out_add_scale times this pass's o to o (an
// instantiation of its own, so the plain prefill's code is untouched).
template <int D, bool ADD>
__device__ __forceinline__ void run_item(const AttnParams& p, char* lds, int group, int b, int kvh, int rb,
                                         int tid, int lane, int wave) {
  using T = Tile<D>;
  constexpr int KS = T::KS, DB = T::DB;
  const int col = lane & 31, half = lane >> 5;

  // Rows of this sequence.  Padded batch: row s of sequence b sits at slot
  // q_start[b] + s of cache row b.  Packed documents (cu_seqlens): document b
  // is tokens cu[b] .. cu[b+1]-1 of q, o and the packed k, v, and its row s
  // sees its own tokens 0..s only.
  int Sq = p.Sq, first = p.q_start ? p.q_start[b] : 0;  // packed: p.Sq bounds every document
  int64_t tok0 = 0;
  if (p.cu_seqlens) {
    tok0 = p.cu_seqlens[b];
    Sq = p.cu_seqlens[b + 1] - (int)tok0;
    first = 0;
    if (tok0 < 0 || Sq < 0 || Sq > p.Sq || tok0 + Sq > p.S_max) {  // malformed offsets: flag, touch nothing
      if (tid == 0 && p.err) p.err[0] = 1;
      return;
    }
  }
  const int nrows = Sq * group;                // (position, head) rows of this unit
  const int R0 = rb * kRows;
  if (R0 >= nrows) return;                     // past this document's rows (whole workgroup)
  // This lane's column: row R = pos * group + head.
  const int R = R0 + wave * 32 + col;
  const int pos = R / group, h = kvh * group + R % group;
  const bool col_ok = R < nrows;
  const int64_t lse_base = p.cu_seqlens ? (int64_t)h * p.S_max + tok0 : ((int64_t)b * p.Hq + h) * Sq;
  if (first < 0 || (int64_t)first + Sq > p.S_max) {
    // Device-side capacity violation: NaN rows, flag, no cache access.
    if (col_ok && half == 0) {
      bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb + (tok0 + pos) * p.o_ss +
                     (int64_t)h * p.o_sh;
      for (int d = 0; d < D; ++d) orow[d] = 0x7FC0;
      if (p.lse) p.lse[lse_base + pos] = __builtin_nanf("");
    }
    if (tid == 0 && p.err) p.err[0] = 1;
    return;
  }

  // Tiles of the workgroup and of this wave (wave-uniform).
  const int pos_hi_wg = min(Sq - 1, (min(nrows, R0 + kRows) - 1) / group);
  const int kmax = first + pos_hi_wg;  // last key the workgroup needs
  const int nkt = kmax / kKT + 1;
  WaveTiles wt;
  {
    const int wr0 = R0 + wave * 32;
    const int wr1 = min(nrows, wr0 + 32) - 1;  // < wr0: a wave past the rows
    wt.last = wr1 >= wr0 ? (first + wr1 / group) / kKT : -1;
    wt.diag_from = (first + wr0 / group) / kKT;
  }

  const int64_t kv_off = ((int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh + tok0 * p.kv_ss) * 2;
  const char* kb = reinterpret_cast<const char*>(p.k) + kv_off;
  const char* vb = reinterpret_cast<const char*>(p.v) + kv_off;

  // Prologue: tiles 0, 1 and 2 into ring slots 0, 1 and 2, then this
  // lane's Q, all in flight together; one wait covers them (the first use
  // of Q then waits for nothing, as the loads it counts have landed).
  Stager<D> sg;
  make_stager<D>(sg, p.kv_ss, wave, lane);
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;  // LDS byte address of the ring
  dma_tile<D, 0>(sg, lds0, kb, vb, p.kv_ss, 0, kmax, wave, lane);
  if (nkt > 1) dma_tile<D, 1>(sg, lds0, kb, vb, p.kv_ss, kKT, kmax, wave, lane);
  if (nkt > 2) dma_tile<D, 2>(sg, lds0, kb, vb, p.kv_ss, 2 * kKT, kmax, wave, lane);

  WaveCtx<D> w;
  w.c = p.scale * kLog2e;
  w.mask_base = first + pos - 4 * half;
  {
    // Q^T fragments: lane holds column `col`, d = 16*ks + 8*half .. +8.
    const bf16_t* qr = reinterpret_cast<const bf16_t*>(p.q) + (int64_t)b * p.q_sb + (tok0 + pos) * p.q_ss +
                       (int64_t)h * p.q_sh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) w.qf[ks] = col_ok ? ld16(qr + 16 * ks + 8 * half) : u32x4{0, 0, 0, 0};
    tile_dma_wait<0>();
  }
  // K fragment: row `col` (block 1 is 32 rows further) at logical chunk
  // 2ks + half.  V^T fragment for d-block q: rows 4half + x/4 (+16kk, +8),
  // logical chunk 4q + c_lane stored at physical chunk 4(q ^ tv(row)) +
  // c_lane, 8-byte half x & 1.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) w.kp[ks] = lds + col * T::ROW_BYTES + 16 * ((2 * ks + half) ^ T::swz_k(col));
  {
    const int x = lane & 15, beta = lane >> 4;
    const int c_lane = 2 * (beta & 1) + ((x & 3) >> 1);
    const int r0 = 4 * half + (x >> 2);
#pragma unroll
    for (int q = 0; q < DB; ++q)
      w.vp[q] = lds + T::V_REGION + r0 * T::ROW_BYTES + 16 * (4 * (q ^ T::tv(r0)) + c_lane) + 8 * (x & 1);
  }
#pragma unroll
  for (int q = 0; q < DB; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) w.acc_o[q][r] = 0.f;
  w.m_run = -INFINITY;
  w.l_run = 0.f;

  phase_barrier();

  // Group B starts one barrier late and group A ends with one more, so
  // every wave passes the same barriers.
  const bool group_b = wave >= kWaves / 2;
  if (group_b) phase_barrier();
  // tile 0: S only
  matrix_step<D, 0>(w, sg, lds0, kb, vb, p.kv_ss, 0, nkt, kmax, wt, wave, lane);
  vector_step<D, 0, true>(w, sg, lds0, kb, vb, p.kv_ss, 0, nkt, kmax, wt, wave, lane);
  for (int k = 1; k < nkt; k += kSlots) {
    tile_step<D, 1>(w, sg, lds0, kb, vb, p.kv_ss, k, nkt, kmax, wt, wave, lane);
    if (k + 1 >= nkt) break;
    tile_step<D, 2>(w, sg, lds0, kb, vb, p.kv_ss, k + 1, nkt, kmax, wt, wave, lane);
    if (k + 2 >= nkt) break;
    tile_step<D, 3>(w, sg, lds0, kb, vb, p.kv_ss, k + 2, nkt, kmax, wt, wave, lane);
    if (k + 3 >= nkt) break;
    tile_step<D, 4>(w, sg, lds0, kb, vb, p.kv_ss, k + 3, nkt, kmax, wt, wave, lane);
    if (k + 4 >= nkt) break;
    tile_step<D, 0>(w, sg, lds0, kb, vb, p.kv_ss, k + 4, nkt, kmax, wt, wave, lane);
  }
  // the last tile's PV (slot (nkt - 1) % kSlots)
  if (nkt - 1 <= wt.last) {
    switch ((nkt - 1) % kSlots) {
      case 0: mfma_phase<D, 0, 0, true, false>(w); break;
      case 1: mfma_phase<D, 0, 1, true, false>(w); break;
      case 2: mfma_phase<D, 0, 2, true, false>(w); break;
      case 3: mfma_phase<D, 0, 3, true, false>(w); break;
      default: mfma_phase<D, 0, 4, true, false>(w); break;
    }
  }
  phase_barrier();
  if (!group_b) phase_barrier();

  // ---- epilogue: O = O^T / l, rounded to bf16 ----
  // acc_o[q] register r holds d = 32q + 8(r/4) + 4half + r%4 of column col.
  // The rows go out through LDS: each wave writes its 32 rows into a block
  // of its own (ring slots 3 and 4, which the next item's prologue copies do
  // not touch; every wave has passed the final barriers, so no tile is read
  // there any more), row-major with 16-byte chunks XOR-swizzled by the row,
  // and reads them back as whole rows.  A store instruction then writes
  // D/8 lanes' 16 bytes per row (a position's g heads are adjacent rows and
  // adjacent in o) instead of 8 bytes of each of 32 rows.  The rows are
  // stored with the nontemporal hint: o is not read again here, and the L2
  // keeps the K/V tiles that later row blocks of the unit read (the q loads
  // keep the default: each q line serves four of a wave's loads).
  if (wt.last >= 0) {
    constexpr int CH = T::CH;
    const float lsum = sum_halves(w.l_run);
    const float inv = 1.f / lsum;
    char* stage = lds + (wave < kWaves / 2 ? 0 : T::V_REGION) + 3 * T::MAT_BYTES + (wave & 3) * 32 * T::ROW_BYTES;
#pragma unroll
    for (int q = 0; q < DB; ++q)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c = 4 * q + q4;  // 16-byte chunk of d = 32q + 8q4
        u32x2 wv;
        wv[0] = pack_bf16x2(w.acc_o[q][4 * q4] * inv, w.acc_o[q][4 * q4 + 1] * inv);
        wv[1] = pack_bf16x2(w.acc_o[q][4 * q4 + 2] * inv, w.acc_o[q][4 * q4 + 3] * inv);
        *reinterpret_cast<u32x2*>(stage + col * T::ROW_BYTES + 16 * (c ^ (col % CH)) + 8 * half) = wv;
      }
    // A wave's LDS accesses complete in order, so its reads see its writes.
    constexpr int RPI = 64 / CH;  // rows per read
    const int c = lane % CH;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + lane / CH;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * T::ROW_BYTES + 16 * (c ^ (r % CH)));
      const int Rr = R0 + wave * 32 + r;
      if (Rr < nrows) {
        const int pr = Rr / group, hr = kvh * group + Rr % group;
        bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb + (tok0 + pr) * p.o_ss +
                       (int64_t)hr * p.o_sh;
        if constexpr (ADD) {
          // o += scale * (this pass's o), in fp32, rounded once (the
          // second pass of a differential attention at head dims the fused
          // differential kernel does not take).
          const u32x4 old = ld16(orow + 8 * c);
          u32x4 sum;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sum[e] = pack_bf16x2(fmaf(p.out_add_scale, bf16_lo(v[e]), bf16_lo(old[e])),
                                 fmaf(p.out_add_scale, bf16_hi(v[e]), bf16_hi(old[e])));
          st16(orow + 8 * c, sum);
        } else {
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(orow + 8 * c));
        }
      }
    }
    if (col_ok && p.lse && half == 0) p.lse[lse_base + pos] = (w.m_run + log2f(lsum)) * kLn2;
  }
}

// D: head dim (32, 64 or 128).
//
// Work order, XCD-aware.  Workgroup i runs on XCD i % 8.  Units u =
// (sequence, KV head) stay on one XCD, so the row blocks of a unit share
// its K/V in that XCD's L2 (and the MALL behind it).
//  * One item per workgroup (persistent == 0): XCD x takes the units u = x
//    (mod 8) in groups of four and walks each group row block by row block,
//    heaviest (last) block first, so heavy blocks start early and light
//    ones fill the end.  Packed documents, whose lengths differ widely, use
//    one group (all their units) so the long documents' heavy blocks start
//    at once.
//  * Persistent (one workgroup per compute unit): XCD x's items, in the
//    same order, are dealt to its workgroups in snake order (0..n-1,
//    n-1..0, ...), which evens out the sums of their tile counts; the
//    workgroups never leave the compute unit, so no item waits for a
//    workgroup launch.
template <int D, bool ADD>
__global__ void __launch_bounds__(kThreads, 1) prefill_kernel(AttnParams p, int nrb, int persistent) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int group = p.Hq / p.Hkv;
  const int units = p.B * p.Hkv;
  const int x = (int)(blockIdx.x % kXcds), r = (int)(blockIdx.x / kXcds);
  const int cnt = x < units ? (units - x + kXcds - 1) / kXcds : 0;  // units u = x (mod 8)
  const int tid = threadIdx.x, lane = tid & 63;
  // The wave index is wave-uniform; through readfirstlane the compiler
  // knows it, so the group's branches around the barriers are scalar.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = (int)(gridDim.x / kXcds);
  const int G = p.cu_seqlens ? cnt : 4;  // units walked together, block by block
  for (int it = 0;; ++it) {
    // k: this workgroup's it-th item in its XCD's list
    const int k = persistent ? it * nw + ((it & 1) ? nw - 1 - r : r) : (it == 0 ? r : cnt * nrb);
    if (k >= cnt * nrb) break;
    const int gi = k / (G * nrb), g0 = gi * G, gn = min(G, cnt - g0);
    const int kk = k - gi * G * nrb;
    const int u = x + kXcds * (g0 + kk % gn);
    run_item<D, ADD>(p, lds, group, u / p.Hkv, u % p.Hkv, nrb - 1 - kk / gn, tid, lane, wave);
  }
}

// Compute units of the current device (cached per device).
int compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D>
hipError_t launch_d(const AttnParams& p, hipStream_t stream) {
  const int group = p.Hq / p.Hkv;
  const int nrb = (int)(((int64_t)p.Sq * group + kRows - 1) / kRows);
  // every XCD sized for the largest unit share
  const int64_t total = (int64_t)kXcds * ((p.B * p.Hkv + kXcds - 1) / kXcds) * nrb;
  // More items than compute units (one workgroup fits a compute unit): one
  // persistent workgroup per compute unit, a multiple of the XCD count so
  // every XCD holds as many.  Packed documents keep one item per workgroup
  // (their row counts are on the device only).
  const int cus = compute_units() / kXcds * kXcds;
  const bool persistent = !p.cu_seqlens && cus > 0 && total > cus;
  const unsigned grid = persistent ? (unsigned)cus : (unsigned)total;
  KernelTimer kt_("prefill_kernel", stream);
  if (p.out_add)
    hipLaunchKernelGGL((prefill_kernel<D, true>), dim3(grid), dim3(kThreads), (size_t)Tile<D>::LDS_BYTES, stream, p,
                       nrb, persistent ? 1 : 0);
  else
    hipLaunchKernelGGL((prefill_kernel<D, false>), dim3(grid), dim3(kThreads), (size_t)Tile<D>::LDS_BYTES, stream,
                       p, nrb, persistent ? 1 : 0);
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
