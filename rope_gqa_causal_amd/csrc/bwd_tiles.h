// bwd_tiles.h -- LDS tile layout and register staging shared by the
// attention backward kernels (bf16, MFMA).
#pragma once
#include <type_traits>

#include "common.h"
#include "mfma_attn.h"

namespace rgc {
namespace bwd {

// Row-major bf16 tiles in LDS with 16-byte chunk c of row r stored at chunk
// c ^ swz(r).  With 64 four-byte banks (256 bytes), a 16-byte row fragment
// read covers 16 consecutive rows at one chunk, and a transposed fragment
// read (8 bytes a lane, 32 lanes at a time) covers 4 consecutive rows at 4
// consecutive chunks of an aligned group of 4.  swz is a bijection of the
// row's position among the rows that share a 256-byte bank line (so the
// first read meets every bank once), and it sends the 4 rows of the second
// read to different 4-chunk groups when they share a line (D = 128: one row
// per line; D = 64: two).
template <int D>
struct BTile {
  static constexpr int CH = D / 8;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int ROW_BYTES = D * 2;
  static __device__ __forceinline__ int swz(int r) {
    if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    if (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    return (r >> 2) & 3;
  }
  static __device__ __forceinline__ int phys(int r, int c) { return r * ROW_BYTES + 16 * (c ^ swz(r)); }
};

// 16-byte row fragment: row r, logical chunk c.
template <int D>
__device__ __forceinline__ u32x4 row_frag(const char* tile, int r, int c) {
  return *reinterpret_cast<const u32x4*>(tile + BTile<D>::phys(r, c));
}

// Transposed fragment of rows 16kk .. 16kk+15 and columns 32q .. 32q+31 of a
// row-major tile: lane j gets, at column 32q + j%32, the values of rows
// 16kk + 4h + (0..3) and 16kk + 8 + 4h + (0..3), h = j/32 -- the MFMA operand
// layout whose k index runs over rows (see vt_frag).
template <int D>
__device__ __forceinline__ u32x4 tr_frag(const char* tile, int q, int kk, int lane) {
  const int x = lane & 15, beta = (lane >> 4) & 1, h = lane >> 5;
  const int c_lane = 2 * beta + ((x & 3) >> 1);  // 4-column group inside the 32-column block
  const int r = 16 * kk + 4 * h + (x >> 2);
  const int c = 4 * q + c_lane;                   // logical 8-byte-pair chunk
  const char* lo = tile + BTile<D>::phys(r, c) + 8 * (x & 1);
  const char* hi = tile + BTile<D>::phys(r + 8, c) + 8 * (x & 1);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lo);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)hi);
  const u32x2 a2 = __builtin_bit_cast(u32x2, a), b2 = __builtin_bit_cast(u32x2, b);
  return u32x4{a2[0], a2[1], b2[0], b2[1]};
}

// Transposed fragment from its two halves' addresses (see tr_frag).
__device__ __forceinline__ u32x4 tr_frag_at(const char* lo, const char* hi) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lo);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)hi);
  const u32x2 a2 = __builtin_bit_cast(u32x2, a), b2 = __builtin_bit_cast(u32x2, b);
  return u32x4{a2[0], a2[1], b2[0], b2[1]};
}

// Compile-time loop: f(std::integral_constant<int, J>) for J = B .. E - 1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------------------
// A thread's share of a rows x D tile, fetched into registers ahead of use
// and stored into a swizzled LDS tile after the current step's arithmetic.
// The loads are unconditional (rows past `valid` re-read row valid - 1) so
// that nothing waits for them before the store; the store writes zeros for
// those rows.  Row offsets are 32-bit byte offsets from a uniform base (the
// host keeps the row stride below 2^24 elements).
template <int D, int ROWS, int NT>
struct TileRegs {
  static constexpr int CHUNKS = ROWS * BTile<D>::CH;
  static constexpr int N = (CHUNKS + NT - 1) / NT;  // 16-byte chunks per thread
  static_assert(CHUNKS % NT == 0 || CHUNKS < NT, "tile chunks must split evenly over the threads");
  u32x4 r[N];
  __device__ __forceinline__ void fetch(const char* g, uint32_t row_bytes, int valid, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = min(tid + i * NT, CHUNKS - 1), c = idx % BTile<D>::CH;
      const uint32_t row = (uint32_t)min(idx / BTile<D>::CH, valid - 1);
      r[i] = ld16(g + (row * row_bytes + 16u * (uint32_t)c));
    }
  }
  // A full tile (every row exists): voff = full_voff(tid, row_bytes) and
  // soff = full_soff(tid), both loop-invariant; a thread's successive chunks
  // lie NT / CH rows apart, a multiple of 16 rows, which the swizzle leaves
  // in place, so the LDS stores take immediate offsets.
  static constexpr int RSTEP = NT / BTile<D>::CH;
  static __device__ __forceinline__ uint32_t full_voff(int tid, uint32_t row_bytes) {
    return (uint32_t)(tid / BTile<D>::CH) * row_bytes + 16u * (uint32_t)(tid % BTile<D>::CH);
  }
  static __device__ __forceinline__ uint32_t full_soff(int tid) {
    return (uint32_t)BTile<D>::phys(tid / BTile<D>::CH, tid % BTile<D>::CH);
  }
  template <int I>
  __device__ __forceinline__ void fetch_chunk(const char* g, uint32_t row_bytes, uint32_t voff) {
    static_assert(CHUNKS % NT == 0 && RSTEP % 16 == 0, "full-tile path needs whole 16-row steps per thread");
    r[I] = ld16(g + (uint64_t)(I * RSTEP) * row_bytes + voff);
  }
  template <int I>
  __device__ __forceinline__ void store_chunk(char* tile, uint32_t soff) const {
    *reinterpret_cast<u32x4*>(tile + soff + I * RSTEP * BTile<D>::ROW_BYTES) = r[I];
  }
  __device__ __forceinline__ void fetch_full(const char* g, uint32_t row_bytes, uint32_t voff) {
    static_for<0, N>([&](auto ic) { fetch_chunk<decltype(ic)::value>(g, row_bytes, voff); });
  }
  __device__ __forceinline__ void store_full(char* tile, uint32_t soff) const {
    static_for<0, N>([&](auto ic) { store_chunk<decltype(ic)::value>(tile, soff); });
  }
  __device__ __forceinline__ void store(char* tile, int valid, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + i * NT, row = idx / BTile<D>::CH, c = idx % BTile<D>::CH;
      const u32x4 z{0, 0, 0, 0};
      if (CHUNKS % NT == 0 || idx < CHUNKS)
        *reinterpret_cast<u32x4*>(tile + BTile<D>::phys(row, c)) = row < valid ? r[i] : z;
    }
  }
};

}  // namespace bwd
}  // namespace rgc
