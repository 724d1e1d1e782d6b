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
//  * a workgroup of 8 waves owns one query head and 256 query positions;
//    each wave owns 32 positions.  Two waves share a SIMD (<= 256 registers
//    each), so one wave's softmax (VALU) runs under the other's MFMAs;
//  * scores are computed transposed, S^T = K Q^T (keys in the MFMA M
//    dimension): a lane holds one query's column, so the softmax max and sum
//    are in-lane except one v_permlane32_swap with the lane 32 away, and the
//    probabilities are already in the B-operand layout of O^T = V^T P^T --
//    P never leaves registers;
//  * 64-key K and V tiles are staged HBM -> registers -> LDS through a
//    4-slot ring (tile j read, j+1 ready, j+2 written, j-1 still being read
//    by slower waves), so one barrier per two tiles suffices; the global
//    loads of tile j+2 are in flight while tile j is multiplied;
//  * both tiles stay row-major in LDS with a per-row XOR swizzle of their
//    16-byte chunks: K fragments (A operand of S^T) are conflict-free 16-byte
//    reads, and V^T fragments (A operand of O^T) come straight from the
//    row-major V tile through ds_read_b64_tr_b16, the gfx950 transposing LDS
//    read -- V is never transposed in software;
//  * the loop is unrolled over the ring so every LDS address is a per-lane
//    base register plus an immediate offset, and tile loads use a scalar base
//    plus a per-lane 32-bit offset: the VALU does softmax work only.  The
//    causal mask is applied on diagonal tiles only;
//  * the running max is only raised (and O rescaled) when a tile's max
//    exceeds it by more than 2^8, so the rescale is almost never taken; p is
//    then at most 256, exact in fp32 and within bf16 range.  The tile max
//    itself is only computed when some lane's tile sum of p passes 2^8 (a
//    necessary condition for a p past 2^8): a row block's first tile and the
//    rare raise -- the common tile does no max reduction at all;
//  * tiles above a wave's causal diagonal are skipped, workgroups are
//    issued heaviest q-tile first.
#include "common.h"
#include "launch.h"
#include "mfma_attn.h"

namespace rgc {
namespace {

constexpr float kLog2e = kAttnLog2e;
constexpr float kLn2 = kAttnLn2;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;   // query positions per workgroup
constexpr int kKT = 64;            // keys per tile
constexpr int kSlots = 4;          // LDS ring: tile j read, j+1 ready, j+2 written, j-1 draining
constexpr int kXcds = 8;           // MI355X: workgroup i is dispatched to XCD i % 8
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

// Tile staging: wave w's i-th piece covers 1 KB of a slot contiguously (lane
// l at byte 16l); the lane fetches the logical chunk stored there.
template <int D>
struct Stager {
  uint32_t goff[Tile<D>::LOADS];   // byte offset in HBM from the tile's first row
  uint32_t loff[Tile<D>::LOADS];   // byte offset in LDS of the piece in slot 0
};

template <int D>
__device__ __forceinline__ void make_stager(Stager<D>& sg, int64_t kv_ss, int wave, int lane) {
  using T = Tile<D>;
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i) {
    int mat, r, c, P;
    T::piece(wave, lane, i, mat, r, c, P);
    sg.goff[i] = (uint32_t)(r * kv_ss * 2 + 16 * c);
    sg.loff[i] = (mat ? T::V_REGION : 0) + 16 * P;
  }
}

// HBM -> registers for tile [j0, j0+64).  Rows past kmax (only in a
// workgroup's last tile) are clamped to kmax: their keys are masked and their
// probabilities are 0, so the clamped (finite, written) rows never reach a
// result and no unwritten cache slot is read.
template <int D>
__device__ __forceinline__ void fetch_tile(u32x4 (&st)[Tile<D>::LOADS], const Stager<D>& sg, const char* kb,
                                           const char* vb, int64_t kv_ss, int j0, int kmax, int wave,
                                           int lane) {
  using T = Tile<D>;
  if (j0 + kKT - 1 <= kmax) {
    const char* kt = kb + (int64_t)j0 * kv_ss * 2;
    const char* vt = vb + (int64_t)j0 * kv_ss * 2;
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int mat = (wave * T::LOADS + i) / T::PIECES;
      st[i] = ld16((mat ? vt : kt) + sg.goff[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      int mat, r, c, P;
      T::piece(wave, lane, i, mat, r, c, P);
      const int key = min(j0 + r, kmax);
      st[i] = ld16((mat ? vb : kb) + (int64_t)key * kv_ss * 2 + 16 * c);
    }
  }
}

template <int D, int SLOT>
__device__ __forceinline__ void store_tile(const u32x4 (&st)[Tile<D>::LOADS], const Stager<D>& sg, char* lds) {
  using T = Tile<D>;
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i)
    *reinterpret_cast<u32x4*>(lds + sg.loff[i] + SLOT * T::MAT_BYTES) = st[i];
}

template <int D>
struct WaveCtx {
  u32x4 qf[D / 16];          // Q^T fragments (B operand)
  const char* kp[D / 16];    // K-fragment address in slot 0, per k-step
  const char* vp[D / 32];    // V^T-fragment address in slot 0, per d-block
  f32x16 acc_o[D / 32];
  float m_run, l_run;
  float c;                   // scale * log2(e)
  int mask_base;             // qabs - 4*half: key offset limit is mask_base - j0
};

// Scores, online softmax and O update for the tile in slot SLOT.
template <int D, int SLOT, bool MASK>
__device__ __forceinline__ void compute_tile(WaveCtx<D>& w, int j0) {
  using T = Tile<D>;
  constexpr int KS = T::KS, DB = T::DB;
  // ---- S^T = K Q^T: block kb holds keys 32kb + 8(r/4) + 4half + r%4 ----
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    u32x4 kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[ks] = *reinterpret_cast<const u32x4*>(w.kp[ks] + SLOT * T::MAT_BYTES + kb * 32 * T::ROW_BYTES);
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s[kb] = mfma(kf[ks], w.qf[ks], s[kb]);
  }
  // ---- causal mask (diagonal tiles only) ----
  if (MASK) {
    const int lim = w.mask_base - j0;  // keep key offsets <= lim
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = -INFINITY;
  }
  // ---- online softmax (log2 domain) ----
  // p = 2^(s*c - m) with the running max m, rounded to bf16 for the PV
  // product; the row sum adds the same rounded values (packed bf16 dot
  // products with 1.0), so the numerator and the denominator use identical
  // weights.
  u32x4 pf[4];
  float ps;
  constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 (1.0, 1.0)
  auto probs = [&]() {
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kk >> 1][8 * (kk & 1) + 2 * e], w.c, -w.m_run));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kk >> 1][8 * (kk & 1) + 2 * e + 1], w.c, -w.m_run));
        pf[kk][e] = pack_bf16x2(p0, p1);
        if (e & 1) ps1 = dot2_bf16(pf[kk][e], kOnes, ps1);
        else ps0 = dot2_bf16(pf[kk][e], kOnes, ps0);
      }
    }
    ps = ps0 + ps1;
  };
  probs();
  // The running max is raised (and O rescaled) only when the tile's max
  // exceeds it by more than the threshold, i.e. only if some p > 2^8 -- and
  // then the lane's sum of p exceeds 2^8 as well.  So the tile max is taken
  // only on tiles where some lane's sum does (a row block's first tile, where
  // m = -inf gives p = inf; a new max past the threshold; overflow): a rare,
  // wave-uniform branch that raises m, rescales and recomputes p.
  if (__builtin_amdgcn_ballot_w64(!(ps <= kSumTrigger))) {
    float m0 = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
    float m1 = fmaxf(fmaxf(s[1][0], s[1][1]), s[1][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
      m0 = fmaxf(fmaxf(m0, s[0][r]), s[0][r + 1]);
      m1 = fmaxf(fmaxf(m1, s[1][r]), s[1][r + 1]);
    }
    m0 = fmaxf(fmaxf(m0, s[0][15]), m1);
    m0 = fmaxf(m0, s[1][15]);
    const float tmax = max_halves(m0) * w.c;
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
  // ---- O^T += V^T P^T ----
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int q = 0; q < DB; ++q)
      w.acc_o[q] = mfma(vt_frag<T::ROW_BYTES>(w.vp[q] + SLOT * T::MAT_BYTES + kk * 16 * T::ROW_BYTES), pf[kk], w.acc_o[q]);
}

// One step of the ring for tile jt in slot SLOT: fetch tile jt+2, multiply
// tile jt, store tile jt+2 into the slot tile jt-2 used, and on odd steps
// wait for every wave.  A store into tile jt-2's slot follows the barrier of
// step jt-1 or jt-2, so every wave has finished that tile; a tile stored in
// step jt is read in step jt+2, after the barrier of step jt or jt+1.
template <int D, int SLOT>
__device__ __forceinline__ void ring_step(WaveCtx<D>& w, u32x4 (&st)[Tile<D>::LOADS], const Stager<D>& sg,
                                          char* lds, const char* kb, const char* vb, int64_t kv_ss, int jt,
                                          int nkt, int kmax, int wave_last, int diag_from, int wave, int lane) {
  const bool refill = jt + 2 < nkt;
  if (refill) fetch_tile<D>(st, sg, kb, vb, kv_ss, (jt + 2) * kKT, kmax, wave, lane);
  if (jt <= wave_last) {
    if (jt < diag_from) compute_tile<D, SLOT, false>(w, jt * kKT);
    else compute_tile<D, SLOT, true>(w, jt * kKT);
  }
  if (refill) store_tile<D, (SLOT + 2) % kSlots>(st, sg, lds);
  if (SLOT & 1) __syncthreads();
}

// D: head dim (32, 64 or 128).
template <int D>
__global__ void __launch_bounds__(kThreads, 1) prefill_kernel(AttnParams p, int nqt) {
  using T = Tile<D>;
  constexpr int KS = T::KS, DB = T::DB;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  // XCD-aware order.  Workgroup i runs on XCD i % 8.  Units u = (sequence,
  // KV head) stay on one XCD, so the query heads of a unit share its K/V in
  // that XCD's L2 (and the MALL behind it).  XCD x takes the units u = x
  // (mod 8) in groups of four and walks each group q-tile slab by slab,
  // heaviest slab first, so heavy tiles start early and light ones fill the
  // end.  Walking unit by unit (heaviest tile first within each unit) leaves
  // heavy tiles of the last units for the end: on the 3.8B-shaped batch the
  // busiest compute unit then carries 120 tile-steps against an average of
  // 108 (112 with groups of four).  Larger groups balance a little better
  // but spread a unit's q-tiles over more time, so its K/V tiles are
  // fetched again; packed documents, whose lengths differ widely, use one
  // group (all their units) so the long documents' heavy tiles start at once.
  const int group = p.Hq / p.Hkv;
  int qt, b, kvh, h;
  {
    const int units = p.B * p.Hkv;
    const int x = (int)(blockIdx.x % kXcds), r = (int)(blockIdx.x / kXcds);
    const int cnt = x < units ? (units - x + kXcds - 1) / kXcds : 0;  // units u = x (mod 8)
    if (r >= cnt * group * nqt) return;
    const int G = p.cu_seqlens ? cnt : 4;  // units walked together, slab by slab
    const int gi = r / (G * group * nqt), g0 = gi * G, gn = min(G, cnt - g0);
    const int rr = r - gi * G * group * nqt;
    const int per_slab = gn * group;
    const int within = rr % per_slab;
    qt = nqt - 1 - rr / per_slab;
    const int u = x + kXcds * (g0 + within / group);
    kvh = u % p.Hkv;
    b = u / p.Hkv;
    h = kvh * group + within % group;
  }
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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
    if (qt * kBM >= Sq) return;  // past this document's rows
  }
  const int s_base = qt * kBM + wave * 32;  // this wave's first row
  const int64_t q_row0 = (int64_t)b * p.q_sb + tok0 * p.q_ss + (int64_t)h * p.q_sh;
  const int64_t o_row0 = (int64_t)b * p.o_sb + tok0 * p.o_ss + (int64_t)h * p.o_sh;
  const int64_t lse_row0 = p.cu_seqlens ? (int64_t)h * p.S_max + tok0 : ((int64_t)b * p.Hq + h) * Sq;
  if (first < 0 || (int64_t)first + Sq > p.S_max) {
    // Device-side capacity violation: NaN rows, flag, no cache access.
    if (s_base + col < Sq && half == 0) {
      bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + o_row0 + (int64_t)(s_base + col) * p.o_ss;
      for (int d = 0; d < D; ++d) orow[d] = 0x7FC0;
      if (p.lse) p.lse[lse_row0 + s_base + col] = __builtin_nanf("");
    }
    if (tid == 0 && p.err) p.err[0] = 1;
    return;
  }

  const int s_end_wg = min(Sq, (qt + 1) * kBM);       // rows [qt*kBM, s_end_wg)
  const int kmax = first + s_end_wg - 1;                // last key the workgroup needs
  const int nkt = kmax / kKT + 1;
  const int wave_rows = min(32, Sq - s_base);           // <= 0: a wave past the ragged tail
  const int wave_last = wave_rows > 0 ? (first + s_base + wave_rows - 1) / kKT : -1;
  const int diag_from = (first + s_base) / kKT;         // first tile that needs the mask

  const int64_t kv_off = ((int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh + tok0 * p.kv_ss) * 2;
  const char* kb = reinterpret_cast<const char*>(p.k) + kv_off;
  const char* vb = reinterpret_cast<const char*>(p.v) + kv_off;

  WaveCtx<D> w;
  w.c = p.scale * kLog2e;
  w.mask_base = first + s_base + col - 4 * half;
  {
    // Q^T fragments: lane holds query `col`, d = 16*ks + 8*half .. +8.
    const int s = s_base + col;
    const bf16_t* qr = reinterpret_cast<const bf16_t*>(p.q) + q_row0 + (int64_t)s * p.q_ss;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      w.qf[ks] = (s < Sq) ? ld16(qr + 16 * ks + 8 * half) : u32x4{0, 0, 0, 0};
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

  Stager<D> sg;
  make_stager<D>(sg, p.kv_ss, wave, lane);

  // Prologue: tiles 0 and 1 into slots 0 and 1.
  u32x4 st[T::LOADS];
  fetch_tile<D>(st, sg, kb, vb, p.kv_ss, 0, kmax, wave, lane);
  store_tile<D, 0>(st, sg, lds);
  if (nkt > 1) {
    fetch_tile<D>(st, sg, kb, vb, p.kv_ss, kKT, kmax, wave, lane);
    store_tile<D, 1>(st, sg, lds);
  }
  __syncthreads();

  for (int jt = 0; jt < nkt; jt += kSlots) {
    ring_step<D, 0>(w, st, sg, lds, kb, vb, p.kv_ss, jt, nkt, kmax, wave_last, diag_from, wave, lane);
    if (jt + 1 >= nkt) break;
    ring_step<D, 1>(w, st, sg, lds, kb, vb, p.kv_ss, jt + 1, nkt, kmax, wave_last, diag_from, wave, lane);
    if (jt + 2 >= nkt) break;
    ring_step<D, 2>(w, st, sg, lds, kb, vb, p.kv_ss, jt + 2, nkt, kmax, wave_last, diag_from, wave, lane);
    if (jt + 3 >= nkt) break;
    ring_step<D, 3>(w, st, sg, lds, kb, vb, p.kv_ss, jt + 3, nkt, kmax, wave_last, diag_from, wave, lane);
  }

  // ---- epilogue: O = O^T / l, rounded to bf16 ----
  // acc_o[q] register r holds d = 32q + 8(r/4) + 4half + r%4 of query col.
  if (wave_last >= 0) {
    const float lsum = sum_halves(w.l_run);
    const int s = s_base + col;
    if (s < Sq) {
      const float inv = 1.f / lsum;
      bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + o_row0 + (int64_t)s * p.o_ss;
#pragma unroll
      for (int q = 0; q < DB; ++q)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = 32 * q + 8 * q4 + 4 * half;
          u32x2 wv;
          wv[0] = pack_bf16x2(w.acc_o[q][4 * q4] * inv, w.acc_o[q][4 * q4 + 1] * inv);
          wv[1] = pack_bf16x2(w.acc_o[q][4 * q4 + 2] * inv, w.acc_o[q][4 * q4 + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + d) = wv;
        }
      if (p.lse && half == 0) p.lse[lse_row0 + s] = (w.m_run + log2f(lsum)) * kLn2;
    }
  }
}

template <int D>
hipError_t launch_d(const AttnParams& p, hipStream_t stream) {
  const int nqt = (p.Sq + kBM - 1) / kBM;
  // every XCD sized for the largest unit share
  const int64_t total = (int64_t)kXcds * ((p.B * p.Hkv + kXcds - 1) / kXcds) * (p.Hq / p.Hkv) * nqt;
  const dim3 grid((unsigned)(((total + kXcds - 1) / kXcds) * kXcds));
  KernelTimer kt_("prefill_kernel", stream);
  hipLaunchKernelGGL(prefill_kernel<D>, grid, dim3(kThreads), (size_t)Tile<D>::LDS_BYTES, stream, p, nqt);
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
