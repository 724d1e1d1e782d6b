// lds_ring.h -- HBM -> LDS tile copies and the phase barrier shared by the
// matrix-core attention kernels that stage K/V tiles in an LDS ring (the
// causal prefill and the differential prefill).
#pragma once

#include "common.h"

namespace rgc {

// HBM -> LDS without registers: one global_load_lds_dwordx4 moves 16 bytes
// per lane into 1 KB of LDS at the wave-uniform byte address in M0 (lane l
// at +16 l).  It is written in asm so that the compiler, which cannot see
// which LDS bytes such a load writes, does not wait for every one of them
// before each LDS read; the kernel waits for them itself (tile_dma_wait)
// before the barrier that publishes the tile.  The load has no result
// register, and its address registers are read when it issues.
//
// dma16 addresses HBM as a scalar base plus a per-lane 32-bit offset and
// LDS as a scalar base plus the constant IMM, both sums formed inside the
// asm: the copy costs no vector instruction (which would queue behind the
// other wave's softmax) and the compiler keeps no per-copy address live.
template <int IMM>
__device__ __forceinline__ void dma16(const char* gbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase),
               "s"(lds_base), "i"(IMM)
               : "memory");
}
// The general form: a per-lane 64-bit address.
template <int IMM>
__device__ __forceinline__ void dma16_v(const void* g, uint32_t lds_base) {
  asm volatile("s_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_base),
               "i"(IMM)
               : "memory");
}
// Wait until at most N of this wave's tile copies are still in flight
// (vmcnt(N); the kernels have no other vector-memory loads in flight in
// their loops, and copies complete in issue order).
template <int N>
__device__ __forceinline__ void tile_dma_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);  // vmcnt(N), expcnt(7), lgkmcnt(15)
}

// A workgroup barrier that waits for this wave's LDS accesses only: the
// tile copies in flight cross it.  The empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace rgc
