// diff.hip -- causal differential attention with grouped KV heads, on the
// gfx950 matrix cores.
//
// Operation (page "750美元从零训练3个LLM：一位开发者的实战复盘", section
// V2): two attention maps are formed from two query/key pairs and the second,
// weighted by lambda, is subtracted from the first before the values are
// mixed:  o = (softmax(s q1 K1^T) - lambda softmax(s q2 K2^T)) V, causal, with
// query head h reading KV head h / (Hq/Hkv) for k1, k2 and v alike.
//
// Same tiling as the causal prefill kernel, with two score maps sharing one
// value tile:
//  * a workgroup of 8 waves owns one query head and 256 query positions,
//    32 per wave; scores are computed transposed (S^T = K Q^T) so a lane
//    holds one query's column and each map's softmax is in-lane plus one
//    v_permlane32_swap;
//  * 64-key tiles of K1, K2 and V are staged HBM -> registers -> LDS through
//    a 4-slot ring (tile j+2 is stored into tile j-2's slot), one barrier per
//    two tiles;
//  * the maps are processed one after the other inside a tile (scores,
//    softmax, O update), so only one map's scores and probabilities are live
//    at a time; both read the same staged value tile;
//  * each map keeps its own running max and sum (lazy rescale, threshold
//    2^8) and its own fp32 output accumulator; the epilogue forms
//    o1 / l1 - lambda * o2 / l2 and rounds once to bf16.
#include "common.h"
#include "launch.h"
#include "mfma_attn.h"

namespace rgc {
namespace {

// Waves per workgroup (two per SIMD).  Head dim 64 only: at 128 the two
// maps' query fragments and accumulators alone take 192 registers and the
// kernel no longer fits two waves per SIMD.
template <int D>
constexpr int waves_for() { return 8; }
constexpr int kKT = 64;            // keys per tile
constexpr int kSlots = 4;          // LDS ring: tile j read, j+1 ready, j+2 written, j-1 draining
constexpr int kXcds = 8;           // MI355X: workgroup i is dispatched to XCD i % 8
constexpr float kRescaleThreshold = 8.0f;  // log2 units

// LDS layout: kSlots K1 tiles, kSlots K2 tiles, kSlots V tiles, each
// row-major [64 keys][D] in 16-byte chunks; chunk c of row r sits at chunk
// c ^ swz(r): r % CH for the key tiles (conflict-free 16-byte fragment
// reads), 4 * tv(r) for the value tile (conflict-free transposed reads).
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
  static constexpr int WAVES = waves_for<D>();
  static constexpr int LOADS = 3 * PIECES / WAVES;   // 16-byte pieces per lane per tile
  static_assert(LOADS * WAVES == 3 * PIECES, "tile pieces must split evenly over the waves");
  static __device__ __forceinline__ int swz_k(int r) { return r % CH; }
  static __device__ __forceinline__ constexpr int tv(int r) { return (r >> 1) & 1; }  // D = 64
  // The lane's piece i: matrix (0 = K1, 1 = K2, 2 = V), row and logical chunk.
  static __device__ __forceinline__ void piece(int wave, int lane, int i, int& mat, int& r, int& c, int& P) {
    const int g = wave * LOADS + i;
    mat = g / PIECES;
    P = (g % PIECES) * 64 + lane;
    r = P / CH;
    const int pc = P % CH;
    c = pc ^ (mat < 2 ? swz_k(r) : 4 * tv(r));
  }
};

template <int D>
struct DStager {
  uint32_t goff[DTile<D>::LOADS];  // byte offset in HBM from the tile's first row
  uint32_t loff[DTile<D>::LOADS];  // byte offset in LDS of the piece in slot 0
};

template <int D>
__device__ __forceinline__ void make_stager(DStager<D>& sg, int64_t kv_ss, int wave, int lane) {
  using T = DTile<D>;
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i) {
    int mat, r, c, P;
    T::piece(wave, lane, i, mat, r, c, P);
    sg.goff[i] = (uint32_t)(r * kv_ss * 2 + 16 * c);
    sg.loff[i] = mat * T::REGION + 16 * P;
  }
}

// HBM -> registers for tile [j0, j0+64) of K1, K2 and V.  Rows past kmax
// (only in a workgroup's last tile) are clamped to kmax: their keys are
// masked, so the clamped rows never reach a result.
template <int D>
__device__ __forceinline__ void fetch_tile(u32x4 (&st)[DTile<D>::LOADS], const DStager<D>& sg,
                                           const char* const (&base)[3], int64_t kv_ss, int j0, int kmax,
                                           int wave, int lane) {
  using T = DTile<D>;
  if (j0 + kKT - 1 <= kmax) {
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int mat = (wave * T::LOADS + i) / T::PIECES;
      st[i] = ld16(base[mat] + (int64_t)j0 * kv_ss * 2 + sg.goff[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      int mat, r, c, P;
      T::piece(wave, lane, i, mat, r, c, P);
      const int key = min(j0 + r, kmax);
      st[i] = ld16(base[mat] + (int64_t)key * kv_ss * 2 + 16 * c);
    }
  }
}

template <int D, int SLOT>
__device__ __forceinline__ void store_tile(const u32x4 (&st)[DTile<D>::LOADS], const DStager<D>& sg, char* lds) {
  using T = DTile<D>;
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i)
    *reinterpret_cast<u32x4*>(lds + sg.loff[i] + SLOT * T::MAT_BYTES) = st[i];
}

// One map's running state.
template <int D>
struct MapState {
  u32x4 qf[D / 16];          // Q^T fragments (B operand)
  f32x16 acc[D / 32];        // O^T accumulators
  float m_run, l_run;
};

template <int D>
struct DiffCtx {
  MapState<D> map[2];
  const char* kp[2][D / 16];  // K-fragment addresses (slot 0) of K1 and K2, per k-step
  const char* vp[D / 32];     // V^T-fragment address (slot 0) per d-block
  float c;                    // scale * log2(e)
  int mask_base;              // key offset limit is mask_base - j0
};

// Scores of map MAP for the tile in slot SLOT, its online softmax, and the
// bf16 P^T fragments (B operand of O^T = V^T P^T).
template <int D, int SLOT, int MAP, bool MASK>
__device__ __forceinline__ void map_softmax(DiffCtx<D>& w, int j0, u32x4 (&pf)[4]) {
  using T = DTile<D>;
  constexpr int KS = T::KS, DB = T::DB;
  MapState<D>& ms = w.map[MAP];
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    u32x4 kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[ks] = *reinterpret_cast<const u32x4*>(w.kp[MAP][ks] + SLOT * T::MAT_BYTES + kb * 32 * T::ROW_BYTES);
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s[kb] = mfma(kf[ks], ms.qf[ks], s[kb]);
  }
  if (MASK) {
    const int lim = w.mask_base - j0;  // keep key offsets <= lim
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = -INFINITY;
  }
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
  const bool need = tmax > ms.m_run + kRescaleThreshold;
  if (__builtin_amdgcn_ballot_w64(need)) {
    asm volatile("; rescale" ::);  // keeps this rare path a real branch (no if-conversion)
    const float m_new = need ? tmax : ms.m_run;
    const float alpha = __builtin_amdgcn_exp2f(ms.m_run - m_new);  // 0 on the first tile
    ms.m_run = m_new;
    ms.l_run *= alpha;
#pragma unroll
    for (int q = 0; q < DB; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) ms.acc[q][r] *= alpha;
  }
  // p rounded to bf16 for the PV product; the row sum adds the same rounded
  // values, so numerator and denominator use identical weights.
  float ps0 = 0.f, ps1 = 0.f;
  constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 (1.0, 1.0)
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kk >> 1][8 * (kk & 1) + 2 * e], w.c, -ms.m_run));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kk >> 1][8 * (kk & 1) + 2 * e + 1], w.c, -ms.m_run));
      pf[kk][e] = pack_bf16x2(p0, p1);
      if (e & 1) ps1 = dot2_bf16(pf[kk][e], kOnes, ps1);
      else ps0 = dot2_bf16(pf[kk][e], kOnes, ps0);
    }
  }
  ms.l_run += ps0 + ps1;
}

// O^T += V^T P^T of map MAP for the tile in slot SLOT.
template <int D, int SLOT, int MAP>
__device__ __forceinline__ void map_pv(DiffCtx<D>& w, const u32x4 (&pf)[4]) {
  using T = DTile<D>;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int q = 0; q < T::DB; ++q)
      w.map[MAP].acc[q] = mfma(vt_frag<T::ROW_BYTES>(w.vp[q] + SLOT * T::MAT_BYTES + kk * 16 * T::ROW_BYTES),
                               pf[kk], w.map[MAP].acc[q]);
}

// The two maps one after the other: each map's probabilities are consumed
// before the next map's scores exist, which keeps one map's working set in
// registers at a time (the value tile is read from LDS once per map).
template <int D, int SLOT, bool MASK>
__device__ __forceinline__ void compute_tile(DiffCtx<D>& w, int j0) {
  u32x4 pf[4];
  map_softmax<D, SLOT, 0, MASK>(w, j0, pf);
  map_pv<D, SLOT, 0>(w, pf);
  map_softmax<D, SLOT, 1, MASK>(w, j0, pf);
  map_pv<D, SLOT, 1>(w, pf);
}

template <int D, int SLOT>
__device__ __forceinline__ void ring_step(DiffCtx<D>& w, u32x4 (&st)[DTile<D>::LOADS], const DStager<D>& sg,
                                          char* lds, const char* const (&base)[3], int64_t kv_ss, int jt,
                                          int nkt, int kmax, int wave_last, int diag_from, int wave, int lane) {
  const bool refill = jt + 2 < nkt;
  if (refill) fetch_tile<D>(st, sg, base, kv_ss, (jt + 2) * kKT, kmax, wave, lane);
  if (jt <= wave_last) {
    if (jt < diag_from) compute_tile<D, SLOT, false>(w, jt * kKT);
    else compute_tile<D, SLOT, true>(w, jt * kKT);
  }
  if (refill) store_tile<D, (SLOT + 2) % kSlots>(st, sg, lds);
  // A store into tile jt-2's slot follows the barrier of step jt-1 or jt-2;
  // a tile stored in step jt is read in step jt+2, after the barrier of step
  // jt or jt+1: odd steps alone wait for every wave.
  if (SLOT & 1) __syncthreads();
}

template <int D>
__global__ void __launch_bounds__(64 * waves_for<D>(), 1) diff_kernel(DiffParams dp, int nqt) {
  using T = DTile<D>;
  constexpr int kBM = 32 * T::WAVES;  // query positions per workgroup
  constexpr int KS = T::KS, DB = T::DB;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const AttnParams& p = dp.a;

  // XCD-aware order, as in the prefill kernel: each XCD walks a contiguous
  // range of (sequence, KV head) groups, all their query heads and q-tiles,
  // heaviest q-tile first, so one group's K1/K2/V stay in one L2.
  const int group = p.Hq / p.Hkv;
  const int per_group = group * nqt;
  const int total = p.B * p.Hkv * per_group;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int lid = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
  if (lid >= total) return;
  const int gidx = lid / per_group;
  const int widx = lid % per_group;
  const int qt = nqt - 1 - widx / group;
  const int kvh = gidx % p.Hkv;
  const int b = gidx / p.Hkv;
  const int h = kvh * group + widx % group;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;

  const int first = p.q_start ? p.q_start[b] : 0;
  const int s_base = qt * kBM + wave * 32;
  if (first < 0 || (int64_t)first + p.Sq > p.S_max) {
    // Device-side capacity violation: NaN rows, flag, no cache access.
    if (s_base + col < p.Sq && half == 0) {
      bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb + (int64_t)(s_base + col) * p.o_ss +
                     (int64_t)h * p.o_sh;
      for (int d = 0; d < D; ++d) orow[d] = 0x7FC0;
    }
    if (tid == 0 && p.err) p.err[0] = 1;
    return;
  }

  const int s_end_wg = min(p.Sq, (qt + 1) * kBM);
  const int kmax = first + s_end_wg - 1;
  const int nkt = kmax / kKT + 1;
  const int wave_rows = min(32, p.Sq - s_base);
  const int wave_last = wave_rows > 0 ? (first + s_base + wave_rows - 1) / kKT : -1;
  const int diag_from = (first + s_base) / kKT;

  const int64_t kv_off = ((int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh) * 2;
  const char* const base[3] = {reinterpret_cast<const char*>(p.k) + kv_off,
                               reinterpret_cast<const char*>(dp.k2) + kv_off,
                               reinterpret_cast<const char*>(p.v) + kv_off};

  DiffCtx<D> w;
  w.c = p.scale * kAttnLog2e;
  w.mask_base = first + s_base + col - 4 * half;
  {
    const int s = s_base + col;
    const int64_t qoff = (int64_t)b * p.q_sb + (int64_t)s * p.q_ss + (int64_t)h * p.q_sh;
    const bf16_t* q1r = reinterpret_cast<const bf16_t*>(p.q) + qoff;
    const bf16_t* q2r = reinterpret_cast<const bf16_t*>(dp.q2) + qoff;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      w.map[0].qf[ks] = (s < p.Sq) ? ld16(q1r + 16 * ks + 8 * half) : u32x4{0, 0, 0, 0};
      w.map[1].qf[ks] = (s < p.Sq) ? ld16(q2r + 16 * ks + 8 * half) : u32x4{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int off = col * T::ROW_BYTES + 16 * ((2 * ks + half) ^ T::swz_k(col));
    w.kp[0][ks] = lds + off;
    w.kp[1][ks] = lds + T::REGION + off;
  }
  {
    const int x = lane & 15, beta = lane >> 4;
    const int c_lane = 2 * (beta & 1) + ((x & 3) >> 1);
    const int r0 = 4 * half + (x >> 2);
#pragma unroll
    for (int q = 0; q < DB; ++q)
      w.vp[q] = lds + 2 * T::REGION + r0 * T::ROW_BYTES + 16 * (4 * (q ^ T::tv(r0)) + c_lane) + 8 * (x & 1);
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
#pragma unroll
    for (int q = 0; q < DB; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) w.map[m].acc[q][r] = 0.f;
    w.map[m].m_run = -INFINITY;
    w.map[m].l_run = 0.f;
  }

  DStager<D> sg;
  make_stager<D>(sg, p.kv_ss, wave, lane);

  u32x4 st[T::LOADS];
  fetch_tile<D>(st, sg, base, p.kv_ss, 0, kmax, wave, lane);
  store_tile<D, 0>(st, sg, lds);
  if (nkt > 1) {
    fetch_tile<D>(st, sg, base, p.kv_ss, kKT, kmax, wave, lane);
    store_tile<D, 1>(st, sg, lds);
  }
  __syncthreads();

  for (int jt = 0; jt < nkt; jt += kSlots) {
    ring_step<D, 0>(w, st, sg, lds, base, p.kv_ss, jt, nkt, kmax, wave_last, diag_from, wave, lane);
    if (jt + 1 >= nkt) break;
    ring_step<D, 1>(w, st, sg, lds, base, p.kv_ss, jt + 1, nkt, kmax, wave_last, diag_from, wave, lane);
    if (jt + 2 >= nkt) break;
    ring_step<D, 2>(w, st, sg, lds, base, p.kv_ss, jt + 2, nkt, kmax, wave_last, diag_from, wave, lane);
    if (jt + 3 >= nkt) break;
    ring_step<D, 3>(w, st, sg, lds, base, p.kv_ss, jt + 3, nkt, kmax, wave_last, diag_from, wave, lane);
  }

  // ---- epilogue: o = O1 / l1 - lambda * O2 / l2, rounded once to bf16 ----
  // acc[q] register r holds d = 32q + 8(r/4) + 4half + r%4 of query col.
  if (wave_last >= 0) {
    const int s = s_base + col;
    if (s < p.Sq) {
      const float w1 = 1.f / sum_halves(w.map[0].l_run);
      const float w2 = -dp.lambda / sum_halves(w.map[1].l_run);
      bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (int64_t)b * p.o_sb + (int64_t)s * p.o_ss +
                     (int64_t)h * p.o_sh;
#pragma unroll
      for (int q = 0; q < DB; ++q)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = 32 * q + 8 * q4 + 4 * half;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = fmaf(w.map[1].acc[q][4 * q4 + e], w2, w.map[0].acc[q][4 * q4 + e] * w1);
          u32x2 wv;
          wv[0] = pack_bf16x2(v[0], v[1]);
          wv[1] = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<u32x2*>(orow + d) = wv;
        }
    }
  }
}

template <int D>
hipError_t launch_d(const DiffParams& dp, hipStream_t stream) {
  const AttnParams& p = dp.a;
  constexpr int kBM = 32 * waves_for<D>();
  const int nqt = (p.Sq + kBM - 1) / kBM;
  const int total = p.B * p.Hq * nqt;
  const dim3 grid((unsigned)(((total + kXcds - 1) / kXcds) * kXcds));
  KernelTimer kt_("diff_kernel", stream);
  hipLaunchKernelGGL(diff_kernel<D>, grid, dim3(64 * waves_for<D>()), (size_t)DTile<D>::LDS_BYTES, stream, dp,
                     nqt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_diff_bf16(const DiffParams& dp, hipStream_t stream) { return launch_d<64>(dp, stream); }

}  // namespace rgc
