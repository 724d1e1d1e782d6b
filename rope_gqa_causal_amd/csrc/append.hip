// append.hip -- copy new K and V rows into the per-layer caches.
//
// Operation (page "750美元从零训练3个LLM：一位开发者的实战复盘", section V3;
// page "从零手训LLaMa：125M模型11小时训练全记录", KV cache paragraph): each
// step's keys and values are kept, one cache row per token and KV head.
//
// A pure byte copy, HBM-bound: one thread moves one 16-byte chunk of a K row
// and the matching chunk of the V row.  Consecutive threads walk a row, so
// both the reads and the writes are full 64-byte-or-wider segments.  A slot
// outside [0, S_max) is never written; it raises the error flag instead.
#include "common.h"
#include "launch.h"

namespace rgc {
namespace {

template <int ESZ>
__global__ void __launch_bounds__(256) append_kernel(AppendParams p) {
  const int cpr = p.D * ESZ / 16;  // 16-byte chunks per row
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nrows = (int64_t)p.B * p.S_new * p.Hkv;
  if (gid >= nrows * cpr) return;
  const int c = (int)(gid % cpr);
  const int64_t row = gid / cpr;
  const int h = (int)(row % p.Hkv);
  const int s = (int)((row / p.Hkv) % p.S_new);
  const int b = (int)(row / ((int64_t)p.Hkv * p.S_new));
  const int64_t slot = (int64_t)p.pos0[b] + s;
  if (slot < 0 || slot >= p.S_max) {
    if (p.err && c == 0) p.err[0] = 1;
    return;
  }
  const int64_t src = ((int64_t)b * p.sb + (int64_t)s * p.ss + (int64_t)h * p.sh) * ESZ + c * 16;
  const int64_t dst = ((int64_t)b * p.c_sb + (int64_t)h * p.c_sh + slot * p.c_ss) * ESZ + c * 16;
  u32x4 kv = ld16(reinterpret_cast<const char*>(p.k_new) + src);
  u32x4 vv = ld16(reinterpret_cast<const char*>(p.v_new) + src);
  st16(reinterpret_cast<char*>(p.k_cache) + dst, kv);
  st16(reinterpret_cast<char*>(p.v_cache) + dst, vv);
}

}  // namespace

hipError_t launch_append(const AppendParams& p, int dtype, hipStream_t stream) {
  const int esz = dtype == DT_F32 ? 4 : 2;
  const int64_t n = (int64_t)p.B * p.S_new * p.Hkv * (p.D * esz / 16);
  const int block = 256;
  const dim3 grid((unsigned)((n + block - 1) / block));
  KernelTimer kt_("append_kernel", stream);
  if (esz == 4)
    hipLaunchKernelGGL(append_kernel<4>, grid, dim3(block), 0, stream, p);
  else
    hipLaunchKernelGGL(append_kernel<2>, grid, dim3(block), 0, stream, p);
  return hipGetLastError();
}

}  // namespace rgc
