// diff.hip -- causal differential attention with grouped KV heads, on the
// gfx950 matrix cores.
//
// Operation (page "750美元从零训练3个LLM：一位开发者的实战复盘", section
// V2): two attention maps are formed from two query/key pairs and the second,
// weighted by lambda, is subtracted from the first before the values are
// mixed:  o = (softmax(s q1 K1^T) - lambda softmax(s q2 K2^T)) V, causal, with
// query head h reading KV head h / (Hq/Hkv) for k1, k2 and v alike.
//
// The causal prefill's schedule, carried to two maps over one value tile:
//  * a workgroup of 8 waves owns 128 query positions of one query head.
//    Waves w and w+4 (which share a SIMD) take the same 32 positions and
//    split every 64-key tile between them: waves 0-3 take its keys 0-31,
//    waves 4-7 its keys 32-63.  The two waves of a SIMD thus always hold
//    equal work, and each keeps its own running max, sum and O^T per map,
//    merged through LDS at the end (the usual combination of two partial
//    softmaxes over disjoint keys).  Each workgroup runs two such items in
//    turn, a head's heavier and lighter query tile (see diff_kernel), so
//    the causal work evens out over the workgroups without a split of any
//    row's keys, and the second item needs no workgroup launch;
//  * scores are computed transposed (S^T = K Q^T, keys in the MFMA M
//    dimension): a lane holds one query's column, each map's softmax is
//    in-lane plus one v_permlane32_swap, and the bf16 probabilities are
//    already the B operand of O^T = V^T P^T;
//  * 64-key tiles of K1, K2 and V go HBM -> LDS by direct copies
//    (global_load_lds_dwordx4, no registers) into a 5-slot ring, three tiles
//    ahead of their first use;
//  * every tile step has a matrix phase (both maps' O^T += V^T P^T for the
//    previous tile and S^T = K Q^T for this tile, 16 MFMAs) and a vector
//    phase (both maps' mask, online softmax and bf16 probabilities); waves
//    0-3 and 4-7 run them one barrier apart, so one wave's softmax issues
//    beside the other wave's matrix instructions;
//  * each map's running max is set by a wave's first tile and then raised
//    lazily (only when a tile's max passes it by 2^8; the tile max is only
//    taken when a lane's sum of probabilities passes 2^8); the row sums add
//    the probabilities in fp32 before they are rounded to bf16 for the PV
//    product;
//  * the epilogue forms o1 / l1 - lambda * o2 / l2, rounds once to bf16 and
//    writes whole rows through LDS.
#include "common.h"
#include "launch.h"
#include "lds_ring.h"
#include "mfma_attn.h"

namespace rgc {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kQT = 128;           // query positions per query tile (one wave group)
constexpr int kKT = 64;            // keys per tile
constexpr int kSlots = 5;          // LDS ring slots (K1, K2 and V tile each)
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr float kSumTrigger = 256.0f;      // 2^kRescaleThreshold
// Initial running max: finite, so that a wave whose key half holds no key
// of a row yet (its p are all 0) keeps finite arithmetic; any real score
// exceeds it, and 2^(kNoMax - m) is 0 for any real max m.
constexpr float kNoMax = -1.0e30f;

// LDS layout: the K1 region (kSlots tiles), the K2 region, the V region;
// each tile row-major [64 keys][D] in 16-byte chunks, chunk c of row r
// stored at chunk c ^ swz(r).  Key tiles: a 16-byte fragment read serves
// 16 lanes (16 rows) per LDS cycle across 64 four-byte banks (256 bytes),
// which hold 256 / ROW_BYTES rows side by side, so swz(r) = (r / (256 /
// ROW_BYTES)) % CH gives the 16 rows 16 distinct chunk positions.  Value
// tile: 4 * tv(r), an XOR of the 32-row d-block index by the row bit that
// varies inside a transposed read (conflict-free ds_read_b64_tr_b16).
template <int D>
struct DTile {
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int KS = D / 16;                  // k-steps of QK^T
  static constexpr int DB = D / 32;                  // 32-row blocks of O^T
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int MAT_BYTES = kKT * ROW_BYTES;  // one tile of one matrix
  static constexpr int REGION = kSlots * MAT_BYTES;  // all slots of one matrix
  static constexpr int LDS_BYTES = 3 * REGION;
  static constexpr int PIECES = MAT_BYTES / 1024;    // 1 KB pieces per matrix tile
  static constexpr int LOADS = 3 * PIECES / kWaves;  // copies per wave per tile
  static constexpr int RPL = ROW_BYTES >= 256 ? 1 : 256 / ROW_BYTES;  // rows per 64-bank line
  static_assert(LOADS * kWaves == 3 * PIECES, "tile pieces must split evenly over the waves");
  static_assert(LOADS >= 1 && LOADS <= 4, "dma_tile issues up to four copies");
  static_assert(LDS_BYTES <= 160 * 1024, "the ring must fit the compute unit's LDS");
  static __device__ __forceinline__ int swz_k(int r) { return (r / RPL) % CH; }
  static __device__ __forceinline__ constexpr int tv(int r) { return (r >> 1) & 1; }  // D = 64
  // Piece g (0 .. 3*PIECES-1): matrix (0 = K1, 1 = K2, 2 = V); lane's row and logical chunk.
  static __device__ __forceinline__ void piece(int g, int lane, int& mat, int& r, int& c) {
    mat = g / PIECES;
    const int P = (g % PIECES) * 64 + lane;
    r = P / CH;
    c = (P % CH) ^ (mat < 2 ? swz_k(r) : 4 * tv(r));
  }
};

// A wave's copies of a tile: piece g = LOADS * wave + i, 1 KB of one
// matrix (lane l at byte 16 l); the pieces of one wave may span two
// matrices, so each has its own (wave-uniform) HBM base and LDS block, both
// chosen once here: the copies of a tile then issue without a branch.
template <int D>
struct DStager {
  const char* gb[DTile<D>::LOADS];  // HBM base of the piece's matrix (wave-uniform)
  uint32_t goff[DTile<D>::LOADS];   // byte offset in HBM from the tile's first row (per lane)
  uint32_t lblk[DTile<D>::LOADS];   // LDS byte offset of the piece in slot 0 (wave-uniform)
};

template <int D>
__device__ __forceinline__ void make_stager(DStager<D>& sg, const char* k1b, const char* k2b, const char* vb,
                                            int64_t kv_ss, int wave, int lane) {
  using T = DTile<D>;
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i) {
    const int g = wave * T::LOADS + i;
    int mat, r, c;
    T::piece(g, lane, mat, r, c);
    sg.goff[i] = (uint32_t)(r * kv_ss * 2 + 16 * c);
    const int m = g / T::PIECES;  // wave-uniform
    // readfirstlane states the uniformity, so both stay in scalar registers.
    const uint64_t a = (uint64_t)(uintptr_t)(m == 0 ? k1b : (m == 1 ? k2b : vb));
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    sg.gb[i] = (const char*)(uintptr_t)(lo | (hi << 32));
    sg.lblk[i] = (uint32_t)__builtin_amdgcn_readfirstlane(m * T::REGION + 1024 * (g % T::PIECES));
  }
}

// Copy tile [j0, j0+64) of K1, K2 and V into ring slot SLOT.  Rows past
// kmax (only in a workgroup's last tile) are clamped to kmax: their keys are
// masked and their probabilities are 0, so the clamped rows never reach a
// result and no unwritten cache slot is read.
template <int D, int SLOT, int I>
__device__ __forceinline__ void dma_piece_clamped(const DStager<D>& sg, uint32_t lds0, int64_t kv_ss, int j0,
                                                  int kmax, int wave, int lane) {
  using T = DTile<D>;
  int mat, r, c;
  T::piece(wave * T::LOADS + I, lane, mat, r, c);
  const int key = min(j0 + r, kmax);
  dma16_v<SLOT * T::MAT_BYTES>(sg.gb[I] + (int64_t)key * kv_ss * 2 + 16 * c, lds0 + sg.lblk[I]);
}
template <int D, int SLOT>
__device__ __forceinline__ void dma_tile(const DStager<D>& sg, uint32_t lds0, int64_t kv_ss, int j0, int kmax,
                                         int wave, int lane) {
  using T = DTile<D>;
  static_assert(T::LOADS == 3, "three copies per wave per tile");
  if (j0 + kKT - 1 <= kmax) {
    const int64_t toff = (int64_t)j0 * kv_ss * 2;
    dma16<SLOT * T::MAT_BYTES>(sg.gb[0] + toff, sg.goff[0], lds0 + sg.lblk[0]);
    dma16<SLOT * T::MAT_BYTES>(sg.gb[1] + toff, sg.goff[1], lds0 + sg.lblk[1]);
    dma16<SLOT * T::MAT_BYTES>(sg.gb[2] + toff, sg.goff[2], lds0 + sg.lblk[2]);
  } else {
    dma_piece_clamped<D, SLOT, 0>(sg, lds0, kv_ss, j0, kmax, wave, lane);
    dma_piece_clamped<D, SLOT, 1>(sg, lds0, kv_ss, j0, kmax, wave, lane);
    dma_piece_clamped<D, SLOT, 2>(sg, lds0, kv_ss, j0, kmax, wave, lane);
  }
}

template <int D>
struct DiffWave {
  u32x4 qf[2][D / 16];       // Q^T fragments of both maps (B operand)
  const char* kp[D / 16];    // K1-fragment address (this wave's key half) in slot 0, per k-step (K2: + REGION)
  const char* vp[D / 32];    // V^T-fragment address (this wave's key half) in slot 0, per d-block
  f32x16 acc[2][D / 32];     // O^T of both maps over this wave's keys
  f32x16 s[2];               // both maps' S^T (this wave's 32 keys) between matrix and vector phases
  u32x4 pf[2][2];            // both maps' P^T (bf16) between vector and matrix phases
  float m_run[2], l_run[2];
  float c;                   // scale * log2(e)
  int mask_base;             // first + pos(column) - 4*half - 32*key half: key offset limit is mask_base - j0
};

// Matrix phase: both maps' O^T += V^T P^T for the tile in slot SV (if PV),
// then both maps' S^T = K Q^T for the tile in slot SK (if S), over this
// wave's 32 keys of the tile.  S^T register r holds key 8(r/4) + 4half +
// r%4 of the wave's half.  A V^T fragment serves both maps; the LDS
// fragments stream through a ring of F registers, each read F-1 steps ahead
// of its use, and the S MFMAs alternate the maps so that neighbouring MFMAs
// are independent.
template <int D, int SK, int SV, bool PV, bool S>
__device__ __forceinline__ void mfma_phase(DiffWave<D>& w) {
  using T = DTile<D>;
  constexpr int KS = T::KS, DB = T::DB;
  constexpr int NPV = PV ? 2 * DB : 0;       // PV: per 16-key step, DB fragments
  constexpr int N = NPV + (S ? 2 * KS : 0);  // S: per k-step, maps 0 and 1
  constexpr int F = 6;
  if (S) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) w.s[m][r] = 0.f;
  }
  auto load = [&](int i) -> u32x4 {
    if (i < NPV) return vt_frag<T::ROW_BYTES>(w.vp[i % DB] + SV * T::MAT_BYTES + (i / DB) * 16 * T::ROW_BYTES);
    const int j = i - NPV;
    return *reinterpret_cast<const u32x4*>(w.kp[j >> 1] + (j & 1) * T::REGION + SK * T::MAT_BYTES);
  };
  auto mma = [&](int i, u32x4 f) {
    if (i < NPV) {
      w.acc[0][i % DB] = mfma(f, w.pf[0][i / DB], w.acc[0][i % DB]);
      w.acc[1][i % DB] = mfma(f, w.pf[1][i / DB], w.acc[1][i % DB]);
    } else {
      const int j = i - NPV;
      w.s[j & 1] = mfma(f, w.qf[j & 1][j >> 1], w.s[j & 1]);
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

// Vector phase of map MAP for the tile starting at key j0: mask (diagonal
// tiles), online softmax (log2 domain), P^T rounded to bf16 into w.pf[MAP].
template <int D, int MAP, bool FIRST>
__device__ __forceinline__ void softmax_map(DiffWave<D>& w, int j0, bool mask) {
  constexpr int DB = DTile<D>::DB;
  f32x16& s = w.s[MAP];
  if (mask) {  // wave-uniform: diagonal tiles only
    // Keep key offsets <= lim: each score is clamped from above by +inf
    // (kept) or -inf (masked), the bound's sign being that of lim - off.
    const int lim = w.mask_base - j0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = lim - (8 * (r >> 2) + (r & 3));
      const float bound = __builtin_bit_cast(float, ((uint32_t)d & 0x80000000u) | 0x7F800000u);
      s[r] = fminf(s[r], bound);
    }
  }
  // p = 2^(s*c - m); the row sum adds p in fp32, the PV product takes p
  // rounded to bf16.
  float ps;
  auto probs = [&]() {
    float ps0 = 0.f, ps1 = 0.f, ps2 = 0.f, ps3 = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * kk + 2 * e], w.c, -w.m_run[MAP]));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * kk + 2 * e + 1], w.c, -w.m_run[MAP]));
        w.pf[MAP][kk][e] = pack_bf16x2(p0, p1);
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
    float m0 = fmaxf(fmaxf(s[0], s[1]), s[2]);
    float m1 = fmaxf(fmaxf(s[3], s[4]), s[5]);
#pragma unroll
    for (int r = 6; r < 16; r += 2) {
      m0 = fmaxf(m0, s[r]);
      m1 = fmaxf(m1, s[r + 1]);
    }
    return max_halves(fmaxf(m0, m1)) * w.c;
  };
  if constexpr (FIRST) {
    // The wave's first tile (m = kNoMax, O = 0, l = 0): the tile max becomes
    // the running max, then the probabilities are formed once.  A column with
    // no key in this wave's half of the tile keeps kNoMax (its p are 0).
    w.m_run[MAP] = fmaxf(tile_max(), kNoMax);
    probs();
    w.l_run[MAP] = ps;
    return;
  }
  probs();
  // A tile max past the running max by more than the threshold makes some
  // p > 2^8 and the lane's sum > 2^8 too; so the max is only taken when some
  // lane's sum passes 2^8 (a wave's first keys, against kNoMax, make it
  // infinite): a rare, wave-uniform branch that raises m, rescales O and l
  // and recomputes p.  Masked scores are -inf and give p = 0 throughout.
  if (__builtin_amdgcn_ballot_w64(!(ps <= kSumTrigger))) {
    const float tmax = tile_max();
    const float m_new = tmax > w.m_run[MAP] + kRescaleThreshold ? tmax : w.m_run[MAP];
    float alpha = __builtin_amdgcn_exp2f(w.m_run[MAP] - m_new);  // 0 when m_run was kNoMax
    // alpha passes through an empty asm, so the multiplications below stay
    // inside this rare path.
    asm volatile("; rescale" : "+v"(alpha));
    w.m_run[MAP] = m_new;
    w.l_run[MAP] *= alpha;
#pragma unroll
    for (int q = 0; q < DB; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) w.acc[MAP][q][r] *= alpha;
    probs();
  }
  w.l_run[MAP] += ps;
}

// Per-wave bounds of the tile loop (wave-uniform).
struct WaveTiles {
  int last;       // last tile with a key of this wave's rows (-1: no rows)
  int diag_from;  // first tile that needs the causal mask
};

// The wave's program: for each tile k its matrix phase (tile k-1's PV and
// tile k's S, both maps) then its vector phase (tile k's softmax, both
// maps), with a barrier after each.  Waves 4-7 run it one barrier behind
// waves 0-3, so between two barriers one wave of a SIMD runs a matrix phase
// while the other runs a vector phase.
//
// The ring: the matrix phase of tile k starts the wave's copy of tile k+3
// into the slot tile k-2 used (its last readers, the matrix phases of tile
// k-1 in both groups, are behind a barrier), and ends by waiting for its
// copy of tile k+1 (started two matrix phases earlier); the barrier after
// it publishes tile k+1, whose first reader is the matrix phase of tile k+1
// in waves 0-3, two barriers later.  SLOT = k % kSlots.
template <int D, int SLOT>
__device__ __forceinline__ void matrix_step(DiffWave<D>& w, const DStager<D>& sg, uint32_t lds0,
                                            int64_t kv_ss, int k, int nkt, int kmax,
                                            const WaveTiles& wt, int wave, int lane) {
  using T = DTile<D>;
  constexpr int SPREV = (SLOT + kSlots - 1) % kSlots;
  if (k + 3 < nkt) dma_tile<D, (SLOT + 3) % kSlots>(sg, lds0, kv_ss, (k + 3) * kKT, kmax, wave, lane);
  // k < nkt here.  A wave past its last tile still forms S (discarded: no
  // vector phase follows) in the step that adds its last PV, so the loop
  // carries one form of the phase.
  if (k == 0) {
    if (wt.last >= 0) mfma_phase<D, SLOT, SPREV, false, true>(w);
  } else if (k - 1 <= wt.last) {
    mfma_phase<D, SLOT, SPREV, true, true>(w);
  }
  // tile k+1 landed: the copies of tiles k+2 and k+3 may still be in flight
  if (k + 3 < nkt) tile_dma_wait<2 * T::LOADS>();
  else if (k + 2 < nkt) tile_dma_wait<T::LOADS>();
  else tile_dma_wait<0>();
  phase_barrier();
}

template <int D, bool FIRST = false>
__device__ __forceinline__ void vector_step(DiffWave<D>& w, int t, const WaveTiles& wt) {
  if (t <= wt.last) {
    const bool mask = t >= wt.diag_from;
    softmax_map<D, 0, FIRST>(w, t * kKT, mask);
    softmax_map<D, 1, FIRST>(w, t * kKT, mask);
  }
  phase_barrier();
}

template <int D, int SLOT>
__device__ __forceinline__ void tile_step(DiffWave<D>& w, const DStager<D>& sg, uint32_t lds0,
                                          int64_t kv_ss, int k, int nkt, int kmax, const WaveTiles& wt,
                                          int wave, int lane) {
  matrix_step<D, SLOT>(w, sg, lds0, kv_ss, k, nkt, kmax, wt, wave, lane);
  vector_step<D>(w, k, wt);
}

// One item: query tile qt (128 positions) of one head, both maps.
template <int D>
__device__ __forceinline__ void diff_item(const DiffParams& dp, char* lds, int qt, int head) {
  using T = DTile<D>;
  constexpr int KS = T::KS, DB = T::DB;
  const AttnParams& p = dp.a;
  const int b = head / p.Hq, h = head % p.Hq;
  const int kvh = h / (p.Hq / p.Hkv);
  const int tid = threadIdx.x, lane = tid & 63;
  // Wave-uniform through readfirstlane, so the branches around the barriers
  // and the copies' matrix choice are scalar.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int kh = wave >= kWaves / 2 ? 1 : 0;  // the wave's key half of every tile
  const int s_base = qt * kQT + (wave & 3) * 32;

  // This lane's q1 and q2 first (they do not depend on the cache offset),
  // then the offset, the tile bounds and the first three tiles' copies, all
  // in flight together; one wait covers them.
  DiffWave<D> w;
  {
    // Q^T fragments: lane holds column `col`, d = 16*ks + 8*half .. +8.
    const int s = s_base + col;
    const int64_t qoff = (int64_t)b * p.q_sb + (int64_t)s * p.q_ss + (int64_t)h * p.q_sh;
    const bf16_t* q1r = reinterpret_cast<const bf16_t*>(p.q) + qoff;
    const bf16_t* q2r = reinterpret_cast<const bf16_t*>(dp.q2) + qoff;
    const bool ok = s < p.Sq;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      w.qf[0][ks] = ok ? ld16(q1r + 16 * ks + 8 * half) : u32x4{0, 0, 0, 0};
      w.qf[1][ks] = ok ? ld16(q2r + 16 * ks + 8 * half) : u32x4{0, 0, 0, 0};
    }
  }

  const int first = p.q_start ? p.q_start[b] : 0;
  if (first < 0 || (int64_t)first + p.Sq > p.S_max) {
    // Device-side capacity violation: NaN rows, flag, no cache access (the
    // whole workgroup leaves: first is the same for all its waves).
    if (kh == 0 && s_base + col < p.Sq && half == 0) {
      bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb + (int64_t)(s_base + col) * p.o_ss +
                     (int64_t)h * p.o_sh;
      for (int d = 0; d < D; ++d) orow[d] = 0x7FC0;
    }
    if (tid == 0 && p.err) p.err[0] = 1;
    return;
  }

  const int s_end_wg = min(p.Sq, (qt + 1) * kQT);
  const int kmax = first + s_end_wg - 1;  // last key the workgroup needs
  const int nkt = kmax / kKT + 1;
  WaveTiles wt;
  {
    const int rows = min(32, p.Sq - s_base);
    wt.last = rows > 0 ? (first + s_base + rows - 1) / kKT : -1;
    wt.diag_from = (first + s_base) / kKT;
  }

  const int64_t kv_off = ((int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh) * 2;
  DStager<D> sg;
  make_stager<D>(sg, reinterpret_cast<const char*>(p.k) + kv_off, reinterpret_cast<const char*>(dp.k2) + kv_off,
                 reinterpret_cast<const char*>(p.v) + kv_off, p.kv_ss, wave, lane);
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;  // LDS byte address of the ring
  dma_tile<D, 0>(sg, lds0, p.kv_ss, 0, kmax, wave, lane);
  if (nkt > 1) dma_tile<D, 1>(sg, lds0, p.kv_ss, kKT, kmax, wave, lane);
  if (nkt > 2) dma_tile<D, 2>(sg, lds0, p.kv_ss, 2 * kKT, kmax, wave, lane);

  w.c = p.scale * kAttnLog2e;
  w.mask_base = first + s_base + col - 4 * half - 32 * kh;
  tile_dma_wait<0>();
  // K fragment: row 32kh + col at logical chunk 2ks + half.  V^T fragment
  // for d-block q: rows 32kh + 4half + x/4 (+16kk, +8), logical chunk
  // 4q + c_lane stored at physical chunk 4(q ^ tv(row)) + c_lane, 8-byte
  // half x & 1 (tv(row) does not depend on the 32kh and 16kk offsets).
  {
    const int kr = 32 * kh + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) w.kp[ks] = lds + kr * T::ROW_BYTES + 16 * ((2 * ks + half) ^ T::swz_k(kr));
    const int x = lane & 15, beta = lane >> 4;
    const int c_lane = 2 * (beta & 1) + ((x & 3) >> 1);
    const int r0 = 4 * half + (x >> 2);
#pragma unroll
    for (int q = 0; q < DB; ++q)
      w.vp[q] = lds + 2 * T::REGION + (32 * kh + r0) * T::ROW_BYTES + 16 * (4 * (q ^ T::tv(r0)) + c_lane) +
                8 * (x & 1);
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
#pragma unroll
    for (int q = 0; q < DB; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) w.acc[m][q][r] = 0.f;
    w.m_run[m] = kNoMax;
    w.l_run[m] = 0.f;
  }

  phase_barrier();

  // Waves 4-7 start one barrier late and waves 0-3 end with one more, so
  // every wave passes the same barriers.
  if (kh) phase_barrier();
  // tile 0: S only
  matrix_step<D, 0>(w, sg, lds0, p.kv_ss, 0, nkt, kmax, wt, wave, lane);
  vector_step<D, true>(w, 0, wt);
  for (int k = 1; k < nkt; k += kSlots) {
    tile_step<D, 1>(w, sg, lds0, p.kv_ss, k, nkt, kmax, wt, wave, lane);
    if (k + 1 >= nkt) break;
    tile_step<D, 2>(w, sg, lds0, p.kv_ss, k + 1, nkt, kmax, wt, wave, lane);
    if (k + 2 >= nkt) break;
    tile_step<D, 3>(w, sg, lds0, p.kv_ss, k + 2, nkt, kmax, wt, wave, lane);
    if (k + 3 >= nkt) break;
    tile_step<D, 4>(w, sg, lds0, p.kv_ss, k + 3, nkt, kmax, wt, wave, lane);
    if (k + 4 >= nkt) break;
    tile_step<D, 0>(w, sg, lds0, p.kv_ss, k + 4, nkt, kmax, wt, wave, lane);
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
  if (!kh) phase_barrier();

  // ---- merge of the two key halves, then o = O1 / l1 - lambda * O2 / l2 ----
  // Every tile has been read and no copy is in flight, so the ring is free:
  // waves 4-7 leave their partial results (O^T, m, l of both maps) in the
  // K1/K2 regions, laid out [value][lane] in 16-byte units so that a wave's
  // stores and its partner's loads are whole-row accesses; waves 0-3 stage
  // the output rows in the V region and store them with the nontemporal
  // hint (o is not read again here).
  constexpr int kPartUnits = 2 * DB * 4 + 1;  // 16-byte units per lane: O^T of both maps, then m, l
  static_assert(kWaves / 2 * kPartUnits * 64 * 16 <= 2 * T::REGION, "partials fit the K1 and K2 regions");
  char* part = lds + (wave & 3) * kPartUnits * 64 * 16 + 16 * lane;
  if (kh) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int q = 0; q < DB; ++q)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int u = (m * DB + q) * 4 + q4;
          *reinterpret_cast<f32x4*>(part + u * 64 * 16) =
              f32x4{w.acc[m][q][4 * q4], w.acc[m][q][4 * q4 + 1], w.acc[m][q][4 * q4 + 2], w.acc[m][q][4 * q4 + 3]};
        }
    *reinterpret_cast<f32x4*>(part + (kPartUnits - 1) * 64 * 16) =
        f32x4{w.m_run[0], w.l_run[0], w.m_run[1], w.l_run[1]};
  }
  phase_barrier();
  if (!kh && wt.last >= 0) {
    // Two partial softmaxes over disjoint keys: O = 2^(ma-M) Oa + 2^(mb-M) Ob
    // and l likewise, with M = max(ma, mb) (per lane; both halves of a
    // column share their m).
    const f32x4 ml = *reinterpret_cast<const f32x4*>(part + (kPartUnits - 1) * 64 * 16);
    float wa[2], wb[2], lsum[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float mb = ml[2 * m], lb = ml[2 * m + 1];
      const float M = fmaxf(w.m_run[m], mb);
      wa[m] = __builtin_amdgcn_exp2f(w.m_run[m] - M);
      wb[m] = __builtin_amdgcn_exp2f(mb - M);
      lsum[m] = sum_halves(wa[m] * w.l_run[m] + wb[m] * lb);
    }
    const float w1 = 1.f / lsum[0];
    const float w2 = -dp.lambda / lsum[1];
    constexpr int CH = T::CH;
    char* stage = lds + 2 * T::REGION + wave * 32 * T::ROW_BYTES;
#pragma unroll
    for (int q = 0; q < DB; ++q)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(part + ((0 * DB + q) * 4 + q4) * 64 * 16);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(part + ((1 * DB + q) * 4 + q4) * 64 * 16);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float o1 = fmaf(wb[0], b0[e], wa[0] * w.acc[0][q][4 * q4 + e]);
          const float o2 = fmaf(wb[1], b1[e], wa[1] * w.acc[1][q][4 * q4 + e]);
          v[e] = fmaf(o2, w2, o1 * w1);
        }
        const int c = 4 * q + q4;  // 16-byte chunk of d = 32q + 8q4
        u32x2 wv;
        wv[0] = pack_bf16x2(v[0], v[1]);
        wv[1] = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<u32x2*>(stage + col * T::ROW_BYTES + 16 * (c ^ (col % CH)) + 8 * half) = wv;
      }
    // A wave's LDS accesses complete in order, so its reads see its writes.
    constexpr int RPI = 64 / CH;  // rows per read
    const int c = lane % CH;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + lane / CH;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * T::ROW_BYTES + 16 * (c ^ (r % CH)));
      const int s = s_base + r;
      if (s < p.Sq) {
        bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb + (int64_t)s * p.o_ss +
                       (int64_t)h * p.o_sh;
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(orow + 8 * c));
      }
    }
  }
}

// Work order: workgroup g takes head g % (B * Hq) and, for pair index
// pr = g / (B * Hq), that head's query tiles nqt-1-pr (the heavier) and pr
// (the lighter), one after the other: every workgroup carries the same
// number of key tiles (at nqt = 8, sixteen and two, fourteen and four, ...),
// the heavy pairs start first, and the second item needs no workgroup
// launch.  Workgroup g runs on XCD g % 8, so (with B * Hq a multiple of 8)
// both items of a head stay on one XCD: the lighter item's K1, K2 and V are
// a prefix of what the heavier one read into that L2.
template <int D>
__global__ void __launch_bounds__(kThreads, 1) diff_kernel(DiffParams dp, int nqt) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int heads = dp.a.B * dp.a.Hq;
  const int head = (int)blockIdx.x % heads, pr = (int)blockIdx.x / heads;
  const int items = pr < nqt - 1 - pr ? 2 : 1;
#pragma clang loop unroll(disable)
  for (int it = 0; it < items; ++it) {
    if (it) phase_barrier();  // every wave is done with the ring, partials and staging
    diff_item<D>(dp, lds, it ? pr : nqt - 1 - pr, head);
  }
}

template <int D>
hipError_t launch_d(const DiffParams& dp, hipStream_t stream) {
  const AttnParams& p = dp.a;
  const int nqt = (p.Sq + kQT - 1) / kQT;
  const int64_t total = (int64_t)p.B * p.Hq * ((nqt + 1) / 2);
  KernelTimer kt_("diff_kernel", stream);
  hipLaunchKernelGGL(diff_kernel<D>, dim3((unsigned)total), dim3(kThreads), (size_t)DTile<D>::LDS_BYTES, stream,
                     dp, nqt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_diff_bf16(const DiffParams& dp, hipStream_t stream) { return launch_d<64>(dp, stream); }

}  // namespace rgc
