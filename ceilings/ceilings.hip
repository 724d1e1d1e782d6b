// ceilings.hip -- two measurement kernels that set what this MI355X delivers
// to a hand-written kernel, beside the published peaks: a streaming read of
// device memory and a loop of bf16 matrix-core instructions.  Measurement
// only; the attention library does not use them.
//
//  * ceil_stream_read: a fixed grid of workgroups strides over the buffer
//    with 16-byte loads, four in flight per lane, and folds what it reads
//    into one word per thread (written out, so no load can be dropped).
//    bytes / time is the read bandwidth a streaming kernel can reach.
//  * ceil_mfma_bf16: every wave issues back-to-back
//    v_mfma_f32_32x32x16_bf16 on four independent accumulators (no memory
//    traffic in the loop).  flops / time is the matrix-core rate a kernel
//    can reach at the clock the chip holds under that load.
//  * ceil_lds_mfma: workgroups of 8 waves (two per SIMD) on a 64 KiB LDS
//    image.  mode 0 reads 16 bytes per lane per instruction and folds them
//    (LDS read bandwidth alone); mode 1 feeds every 32 x 32 x 16 matrix
//    instruction a B operand of 16 bytes per lane read from LDS just before
//    it, the operand traffic of a kernel whose waves each read a whole
//    shared K or V tile.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t fold(u32x4 a) { return a[0] ^ a[1] ^ a[2] ^ a[3]; }

// Grid-stride form: consecutive lanes of the whole grid read consecutive
// 16-byte pieces, four pieces in flight per lane.
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
  }
  for (; i < n16; i += stride) acc ^= fold(src[i]);
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Contiguous form: workgroup w owns the w-th slice of the buffer and walks
// it in blocks of 256 lanes x U pieces (U 16-byte loads in flight per lane,
// 4 KiB contiguous per load instruction of the workgroup).  NT: the loads
// carry the nontemporal hint.
template <int U, bool NT>
__global__ void __launch_bounds__(256) stream_read_chunk_kernel(const u32x4* __restrict__ src, size_t n16,
                                                                uint32_t* __restrict__ out) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  size_t i = lo + threadIdx.x;
  for (; i + (U - 1) * 256 < hi; i += U * 256) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(src + i + u * 256) : src[i + u * 256];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= fold(v[u]);
  }
  for (; i < hi; i += 256) acc ^= fold(src[i]);
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ void __launch_bounds__(256) mfma_bf16_kernel(float* __restrict__ out, int iters) {
  const uint32_t t = threadIdx.x;
  u32x4 av = {0x3F803F80u ^ t, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  u32x4 bv = {0x3C003C00u, 0x3C003C00u ^ t, 0x3C003C00u, 0x3C003C00u};
  const bf16x8 a = __builtin_bit_cast(bf16x8, av), b = __builtin_bit_cast(bf16x8, bv);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// One 16-byte piece per lane, consecutive lanes on consecutive pieces (no
// bank conflict), the wave's 1 KiB block moving by one block per read.
template <bool MFMA>
__global__ void __launch_bounds__(512) lds_mfma_kernel(float* __restrict__ out, int iters) {
  __shared__ u32x4 img[4096];
  const uint32_t t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (uint32_t i = t; i < 4096; i += 512) img[i] = u32x4{i, i * 3u + 1u, i ^ 0x3F80u, 0x3F803F80u};
  __syncthreads();
  u32x4 av = {0x3F803F80u ^ t, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const bf16x8 a = __builtin_bit_cast(bf16x8, av);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  uint32_t acc = 0;
  uint32_t blk = wave * 8;
  // Software-pipelined: the four operands of the next step are read while
  // this step's instructions run.
  u32x4 b0 = img[(blk & 63) * 64 + lane], b1 = img[((blk + 1) & 63) * 64 + lane];
  u32x4 b2 = img[((blk + 2) & 63) * 64 + lane], b3 = img[((blk + 3) & 63) * 64 + lane];
  for (int i = 0; i < iters; ++i) {
    blk += 4;
    const u32x4 n0 = img[(blk & 63) * 64 + lane], n1 = img[((blk + 1) & 63) * 64 + lane];
    const u32x4 n2 = img[((blk + 2) & 63) * 64 + lane], n3 = img[((blk + 3) & 63) * 64 + lane];
    if (MFMA) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, b0), c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, b1), c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, b2), c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, b3), c3, 0, 0, 0);
    } else {
      acc ^= fold(b0) ^ fold(b1) ^ fold(b2) ^ fold(b3);
    }
    b0 = n0; b1 = n1; b2 = n2; b3 = n3;
  }
  acc ^= fold(b0) ^ fold(b1) ^ fold(b2) ^ fold(b3);
  float s = (float)acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[(size_t)blockIdx.x * blockDim.x + t] = s;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from src with `wgs` workgroups of 256
// threads; out receives wgs * 256 words.  mode 0: grid-stride, 4 loads in
// flight per lane; 1, 2: contiguous slices with 8 or 16 loads in flight;
// 3: as 1 with nontemporal loads.  0, or -1 for a bad argument, or -9 when
// the launch is refused.
int ceil_stream_read(const void* src, size_t bytes, uint32_t* out, int wgs, int mode, void* stream) {
  if (!src || !out || wgs <= 0 || bytes % 16 != 0 || mode < 0 || mode > 3) return -1;
  const u32x4* s = (const u32x4*)src;
  const size_t n = bytes / 16;
  hipStream_t st = (hipStream_t)stream;
  switch (mode) {
    case 0: hipLaunchKernelGGL(stream_read_kernel, dim3(wgs), dim3(256), 0, st, s, n, out); break;
    case 1: hipLaunchKernelGGL((stream_read_chunk_kernel<8, false>), dim3(wgs), dim3(256), 0, st, s, n, out); break;
    case 2: hipLaunchKernelGGL((stream_read_chunk_kernel<16, false>), dim3(wgs), dim3(256), 0, st, s, n, out); break;
    default: hipLaunchKernelGGL((stream_read_chunk_kernel<8, true>), dim3(wgs), dim3(256), 0, st, s, n, out); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -9;
}

// `wgs` workgroups of 4 waves, each wave `iters` x 4 matrix instructions of
// 32 x 32 x 16 (32768 flops each); out receives wgs * 256 floats.
int ceil_mfma_bf16(float* out, int wgs, int iters, void* stream) {
  if (!out || wgs <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3(wgs), dim3(256), 0, (hipStream_t)stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -9;
}

// `wgs` workgroups of 8 waves, each wave `iters` x 4 LDS reads of 16 bytes
// per lane (1 KiB per wave per read), with (mode 1) or without (mode 0) a
// 32 x 32 x 16 matrix instruction consuming each; out receives wgs * 512
// floats.
int ceil_lds_mfma(float* out, int wgs, int iters, int mode, void* stream) {
  if (!out || wgs <= 0 || iters <= 0 || mode < 0 || mode > 1) return -1;
  if (mode) hipLaunchKernelGGL(lds_mfma_kernel<true>, dim3(wgs), dim3(512), 0, (hipStream_t)stream, out, iters);
  else hipLaunchKernelGGL(lds_mfma_kernel<false>, dim3(wgs), dim3(512), 0, (hipStream_t)stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -9;
}

}  // extern "C"
