// attn_f32.hip -- causal GQA attention for fp32 tensors (prefill and decode).
//
// Operation: o = softmax(scale * q K^T) V over the keys at or before the
// query's slot, query head h reading KV head h / (Hq/Hkv) (page
// "750美元从零训练3个LLM：一位开发者的实战复盘", sections V2 and V3; page
// "训练3.8B LLM至0.384 CORE，成本998美元 – Hugo Vergnes", section 无效的方法).
//
// fp32 inputs have no fp32 matrix-core path worth its precision trade here,
// so this is the full-precision VALU kernel: one wave per query row, each
// lane an online-softmax over the keys j = lane, lane + 64, ... (fp32 exp,
// fp32 accumulation), then a max-rescaled merge of the 64 lane partials.  The
// query row sits in LDS and is read as a broadcast.  It serves the fp32
// workloads, which are small; bf16 goes through the matrix-core kernels.
#include "common.h"
#include "launch.h"

namespace rgc {
namespace {

template <int D>
__global__ void __launch_bounds__(64) attn_f32_kernel(AttnParams p, int decode) {
  __shared__ float qs[D];
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;  // (b, s, h) with h fastest
  const int h = (int)(row % p.Hq);
  const int s = (int)((row / p.Hq) % p.Sq);
  const int b = (int)(row / ((int64_t)p.Hq * p.Sq));
  const int kvh = h / (p.Hq / p.Hkv);

  int pos;
  bool ok;
  if (decode) {
    const int L = p.seq_lens[b];
    const int lim = p.max_len < p.S_max ? p.max_len : p.S_max;
    pos = L - 1;
    ok = L >= 1 && L <= lim;
  } else {
    const int first = p.q_start ? p.q_start[b] : 0;
    pos = first + s;
    ok = first >= 0 && (int64_t)first + p.Sq <= p.S_max;
  }
  float* orow = reinterpret_cast<float*>(p.o) + (int64_t)b * p.o_sb + (int64_t)s * p.o_ss +
                (int64_t)h * p.o_sh;
  if (!ok) {
    for (int d = lane; d < D; d += 64) orow[d] = __builtin_nanf("");
    if (p.lse && lane == 0) p.lse[((int64_t)b * p.Hq + h) * p.Sq + s] = __builtin_nanf("");
    if (p.err && lane == 0) p.err[0] = 1;
    return;
  }

  const float* qrow = reinterpret_cast<const float*>(p.q) + (int64_t)b * p.q_sb +
                      (int64_t)s * p.q_ss + (int64_t)h * p.q_sh;
  for (int d = lane; d < D; d += 64) qs[d] = qrow[d];
  __syncthreads();

  const float* kb = reinterpret_cast<const float*>(p.k) + (int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh;
  const float* vb = reinterpret_cast<const float*>(p.v) + (int64_t)b * p.kv_sb + (int64_t)kvh * p.kv_sh;

  float m = -INFINITY, l = 0.f;
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  for (int j = lane; j <= pos; j += 64) {
    const float* kr = kb + (int64_t)j * p.kv_ss;
    float dot = 0.f;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      f32x4 kv = *reinterpret_cast<const f32x4*>(kr + d);
      dot = fmaf(qs[d], kv[0], dot);
      dot = fmaf(qs[d + 1], kv[1], dot);
      dot = fmaf(qs[d + 2], kv[2], dot);
      dot = fmaf(qs[d + 3], kv[3], dot);
    }
    const float z = dot * p.scale;
    const float mn = fmaxf(m, z);
    const float alpha = expf(m - mn);  // exp(-inf) = 0 on the first key
    const float w = expf(z - mn);
    l = l * alpha + w;
    const float* vr = vb + (int64_t)j * p.kv_ss;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      f32x4 vv = *reinterpret_cast<const f32x4*>(vr + d);
      acc[d] = fmaf(acc[d], alpha, w * vv[0]);
      acc[d + 1] = fmaf(acc[d + 1], alpha, w * vv[1]);
      acc[d + 2] = fmaf(acc[d + 2], alpha, w * vv[2]);
      acc[d + 3] = fmaf(acc[d + 3], alpha, w * vv[3]);
    }
    m = mn;
  }
  // Merge the lane partials: rescale each by exp(m_lane - m_row).
  const float mrow = wave_max(m);
  const float f = (m == -INFINITY) ? 0.f : expf(m - mrow);
  const float lrow = wave_sum(l * f);
  const float inv = 1.f / lrow;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const float t = wave_sum(acc[d] * f);
    if (lane == (d & 63)) orow[d] = t * inv;
  }
  if (p.lse && lane == 0) p.lse[((int64_t)b * p.Hq + h) * p.Sq + s] = mrow + logf(lrow);
}

}  // namespace

hipError_t launch_attn_f32(const AttnParams& p, bool decode, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.B * p.Sq * p.Hq));
  const int dec = decode ? 1 : 0;
  KernelTimer kt_("attn_f32_kernel", stream);
  switch (p.D) {
    case 32: hipLaunchKernelGGL(attn_f32_kernel<32>, grid, dim3(64), 0, stream, p, dec); break;
    case 64: hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, stream, p, dec); break;
    default: hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, stream, p, dec); break;
  }
  return hipGetLastError();
}

}  // namespace rgc
