// api.hip -- the C ABI declared in include/rgc.h: host-side argument checks,
// then one launch (two for a split decode) on the caller's stream.
//
// Nothing is allocated, freed or synchronised here and no state is kept, so
// the entry points are thread-safe.  Every check runs before the first HIP
// call; a negative status means nothing was enqueued.  The head-count check
// (Hq a multiple of Hkv) is the configuration assertion the page
// "750美元从零训练3个LLM：一位开发者的实战复盘" recommends (section
// 五条来之不易的工程教训, lesson 4).
#include <cmath>

#include "../../include/rgc.h"
#include "launch.h"

using namespace rgc;

namespace {

bool dtype_ok(int dt) { return dt == RGC_F32 || dt == RGC_BF16; }
int esize(int dt) { return dt == RGC_F32 ? 4 : 2; }
bool headdim_ok(int D) { return D == 32 || D == 64 || D == 128; }

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }
// Strides in elements must keep every row start on a 16-byte boundary.
bool stride_ok(int64_t s, int dt) { return (s * esize(dt)) % 16 == 0; }

// The bf16 matrix-core kernels stage a tile's rows at 32-bit byte offsets
// from the tile's first row (up to 63 token strides of 2 bytes): a token
// stride in [0, 2^24) elements keeps every such offset below 2^31.
bool token_stride_ok(int64_t s) { return s >= 0 && s < (int64_t(1) << 24); }

int hip_status(hipError_t e) { return e == hipSuccess ? RGC_OK : RGC_ERR_HIP; }

}  // namespace

extern "C" {

int rgc_abi_version(void) { return RGC_ABI_VERSION; }

const char* rgc_status_string(int status) {
  switch (status) {
    case RGC_OK: return "ok";
    case RGC_ERR_NULL: return "a required pointer is NULL";
    case RGC_ERR_SHAPE: return "a size is negative or inconsistent";
    case RGC_ERR_GROUP: return "Hq is not a multiple of Hkv";
    case RGC_ERR_DTYPE: return "unsupported dtype";
    case RGC_ERR_HEADDIM: return "unsupported head dimension";
    case RGC_ERR_LAYOUT: return "misaligned pointer or stride";
    case RGC_ERR_CAPACITY: return "a length exceeds the cache capacity";
    case RGC_ERR_WORKSPACE: return "workspace missing or too small";
    case RGC_ERR_HIP: return "the HIP runtime refused the launch";
    case RGC_ERR_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

namespace {

int rope_impl(void* x, int dtype, int B, int S, int H, int D, int64_t sb, int64_t ss, int64_t sh,
              const int32_t* pos0, double base, int style, float sin_sign, void* stream) {
  if (!dtype_ok(dtype)) return RGC_ERR_DTYPE;
  if (B < 0 || S < 0 || H < 0 || D < 0) return RGC_ERR_SHAPE;
  if (D < 2 || D > kMaxRopeDim || D % 2 != 0) return RGC_ERR_HEADDIM;
  if (style != RGC_ROPE_HALF && style != RGC_ROPE_INTERLEAVED) return RGC_ERR_ARG;
  if (!(base > 0.0) || !std::isfinite(base)) return RGC_ERR_ARG;
  if (B == 0 || S == 0 || H == 0) return RGC_OK;
  if (!x) return RGC_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(x) % esize(dtype) != 0) return RGC_ERR_LAYOUT;
  RopeParams p;
  p.x = x;
  p.B = B;
  p.S = S;
  p.H = H;
  p.D = D;
  p.sb = sb;
  p.ss = ss;
  p.sh = sh;
  p.pos0 = pos0;
  p.sin_sign = sin_sign;
  for (int i = 0; i < kMaxRopeDim / 2; ++i)
    p.theta[i] = i < D / 2 ? std::pow(base, -2.0 * (double)i / (double)D) : 0.0;
  return hip_status(launch_rope(p, dtype, style, reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

int rgc_rope_apply(void* x, int dtype, int B, int S, int H, int D, int64_t sb, int64_t ss,
                   int64_t sh, const int32_t* pos0, double base, int style, void* stream) {
  return rope_impl(x, dtype, B, S, H, D, sb, ss, sh, pos0, base, style, 1.f, stream);
}

int rgc_rope_backward(void* g, int dtype, int B, int S, int H, int D, int64_t sb, int64_t ss,
                      int64_t sh, const int32_t* pos0, double base, int style, void* stream) {
  return rope_impl(g, dtype, B, S, H, D, sb, ss, sh, pos0, base, style, -1.f, stream);
}

int rgc_kv_cache_append(void* k_cache, void* v_cache, int dtype, int B, int Hkv, int D, int S_max,
                        int64_t c_sb, int64_t c_sh, int64_t c_ss, const void* k_new,
                        const void* v_new, int S_new, int64_t sb, int64_t ss, int64_t sh,
                        const int32_t* pos0, int32_t* err_flag, void* stream) {
  if (!dtype_ok(dtype)) return RGC_ERR_DTYPE;
  if (B < 0 || Hkv < 0 || D < 0 || S_max < 0 || S_new < 0) return RGC_ERR_SHAPE;
  if (!headdim_ok(D)) return RGC_ERR_HEADDIM;
  if (B == 0 || S_new == 0 || Hkv == 0) return RGC_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !pos0) return RGC_ERR_NULL;
  if (S_new > S_max) return RGC_ERR_CAPACITY;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return RGC_ERR_LAYOUT;
  if (!stride_ok(c_sb, dtype) || !stride_ok(c_sh, dtype) || !stride_ok(c_ss, dtype) ||
      !stride_ok(sb, dtype) || !stride_ok(ss, dtype) || !stride_ok(sh, dtype))
    return RGC_ERR_LAYOUT;
  AppendParams p;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.k_new = k_new;
  p.v_new = v_new;
  p.B = B;
  p.Hkv = Hkv;
  p.D = D;
  p.S_max = S_max;
  p.S_new = S_new;
  p.c_sb = c_sb;
  p.c_sh = c_sh;
  p.c_ss = c_ss;
  p.sb = sb;
  p.ss = ss;
  p.sh = sh;
  p.pos0 = pos0;
  p.err = err_flag;
  return hip_status(launch_append(p, dtype, reinterpret_cast<hipStream_t>(stream)));
}

namespace {

int rope_append_impl(void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache, int dtype,
                     int B, int S, int Hq, int Hkv, int D, int S_max, int64_t q_sb, int64_t q_ss, int64_t q_sh,
                     int64_t sb, int64_t ss, int64_t sh, int64_t c_sb, int64_t c_sh, int64_t c_ss,
                     const int32_t* pos0, double base, int style, bool norm, float eps, int32_t* err_flag,
                     void* stream) {
  if (!dtype_ok(dtype)) return RGC_ERR_DTYPE;
  if (B < 0 || S < 0 || Hq < 0 || Hkv < 0 || D < 0 || S_max < 0) return RGC_ERR_SHAPE;
  if (!headdim_ok(D)) return RGC_ERR_HEADDIM;
  if (style != RGC_ROPE_HALF && style != RGC_ROPE_INTERLEAVED) return RGC_ERR_ARG;
  if (!(base > 0.0) || !std::isfinite(base)) return RGC_ERR_ARG;
  if (norm && !(eps >= 0.f && std::isfinite(eps))) return RGC_ERR_ARG;
  if (B == 0 || S == 0 || (Hq == 0 && Hkv == 0)) return RGC_OK;
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !pos0) return RGC_ERR_NULL;
  if (S > S_max) return RGC_ERR_CAPACITY;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return RGC_ERR_LAYOUT;
  if (!stride_ok(q_sb, dtype) || !stride_ok(q_ss, dtype) || !stride_ok(q_sh, dtype) || !stride_ok(sb, dtype) ||
      !stride_ok(ss, dtype) || !stride_ok(sh, dtype) || !stride_ok(c_sb, dtype) || !stride_ok(c_sh, dtype) ||
      !stride_ok(c_ss, dtype))
    return RGC_ERR_LAYOUT;
  RopeAppendParams p;
  p.q = q;
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.B = B;
  p.S = S;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  p.S_max = S_max;
  p.q_sb = q_sb;
  p.q_ss = q_ss;
  p.q_sh = q_sh;
  p.n_sb = sb;
  p.n_ss = ss;
  p.n_sh = sh;
  p.c_sb = c_sb;
  p.c_sh = c_sh;
  p.c_ss = c_ss;
  p.pos0 = pos0;
  p.err = err_flag;
  p.eps = eps;
  for (int i = 0; i < kMaxRopeDim / 2; ++i)
    p.theta[i] = i < D / 2 ? std::pow(base, -2.0 * (double)i / (double)D) : 0.0;
  return hip_status(launch_rope_append(p, dtype, style, norm, reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

int rgc_rope_append(void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache, int dtype,
                    int B, int S, int Hq, int Hkv, int D, int S_max, int64_t q_sb, int64_t q_ss, int64_t q_sh,
                    int64_t sb, int64_t ss, int64_t sh, int64_t c_sb, int64_t c_sh, int64_t c_ss,
                    const int32_t* pos0, double base, int style, int32_t* err_flag, void* stream) {
  return rope_append_impl(q, k_new, v_new, k_cache, v_cache, dtype, B, S, Hq, Hkv, D, S_max, q_sb, q_ss, q_sh, sb,
                          ss, sh, c_sb, c_sh, c_ss, pos0, base, style, false, 0.f, err_flag, stream);
}

int rgc_norm_rope_append(void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache, int dtype,
                         int B, int S, int Hq, int Hkv, int D, int S_max, int64_t q_sb, int64_t q_ss,
                         int64_t q_sh, int64_t sb, int64_t ss, int64_t sh, int64_t c_sb, int64_t c_sh,
                         int64_t c_ss, const int32_t* pos0, double base, int style, float eps,
                         int32_t* err_flag, void* stream) {
  return rope_append_impl(q, k_new, v_new, k_cache, v_cache, dtype, B, S, Hq, Hkv, D, S_max, q_sb, q_ss, q_sh, sb,
                          ss, sh, c_sb, c_sh, c_ss, pos0, base, style, true, eps, err_flag, stream);
}

namespace {

int check_attn_common(int dtype, int B, int Sq, int Hq, int Hkv, int D, int S_max) {
  if (!dtype_ok(dtype)) return RGC_ERR_DTYPE;
  if (B < 0 || Sq < 0 || Hq < 0 || Hkv < 0 || D < 0 || S_max < 0) return RGC_ERR_SHAPE;
  if (!headdim_ok(D)) return RGC_ERR_HEADDIM;
  if (Hq == 0 || Hkv == 0) return RGC_ERR_SHAPE;
  if (Hq % Hkv != 0) return RGC_ERR_GROUP;
  return RGC_OK;
}

}  // namespace

int rgc_gqa_attn_prefill(void* o, const void* q, const void* k_cache, const void* v_cache,
                         int dtype, int B, int Sq, int Hq, int Hkv, int D, int S_max, int64_t q_sb,
                         int64_t q_ss, int64_t q_sh, int64_t o_sb, int64_t o_ss, int64_t o_sh,
                         int64_t kv_sb, int64_t kv_sh, int64_t kv_ss, const int32_t* q_start,
                         float scale, float* lse, int32_t* err_flag, void* stream) {
  int st = check_attn_common(dtype, B, Sq, Hq, Hkv, D, S_max);
  if (st != RGC_OK) return st;
  if (B == 0 || Sq == 0) return RGC_OK;
  if (!o || !q || !k_cache || !v_cache) return RGC_ERR_NULL;
  if (Sq > S_max) return RGC_ERR_CAPACITY;
  if (!(scale > 0.f) || !std::isfinite(scale)) return RGC_ERR_ARG;
  if (!aligned16(o) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return RGC_ERR_LAYOUT;
  if (!stride_ok(q_sb, dtype) || !stride_ok(q_ss, dtype) || !stride_ok(q_sh, dtype) ||
      !stride_ok(o_sb, dtype) || !stride_ok(o_ss, dtype) || !stride_ok(o_sh, dtype) ||
      !stride_ok(kv_sb, dtype) || !stride_ok(kv_sh, dtype) || !stride_ok(kv_ss, dtype))
    return RGC_ERR_LAYOUT;
  if (dtype == RGC_BF16 && !token_stride_ok(kv_ss)) return RGC_ERR_LAYOUT;
  if ((int64_t)B * Sq * Hq > 0x7FFFFFFFLL) return RGC_ERR_SHAPE;
  AttnParams p = {};
  p.o = o;
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.B = B;
  p.Sq = Sq;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  p.S_max = S_max;
  p.q_sb = q_sb;
  p.q_ss = q_ss;
  p.q_sh = q_sh;
  p.o_sb = o_sb;
  p.o_ss = o_ss;
  p.o_sh = o_sh;
  p.kv_sb = kv_sb;
  p.kv_sh = kv_sh;
  p.kv_ss = kv_ss;
  p.q_start = q_start;
  p.seq_lens = nullptr;
  p.max_len = S_max;
  p.scale = scale;
  p.lse = lse;
  p.err = err_flag;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return hip_status(dtype == RGC_BF16 ? launch_prefill_bf16(p, s) : launch_attn_f32(p, false, s));
}

int rgc_gqa_attn_prefill_varlen(void* o, const void* q, const void* k, const void* v, int dtype, int n_docs,
                                const int32_t* cu_seqlens, int max_seqlen, int total_tokens, int Hq, int Hkv,
                                int D, int64_t q_ts, int64_t q_hs, int64_t o_ts, int64_t o_hs, int64_t kv_ts,
                                int64_t kv_hs, float scale, float* lse, int32_t* err_flag, void* stream) {
  int st = check_attn_common(dtype, n_docs, max_seqlen, Hq, Hkv, D, total_tokens);
  if (st != RGC_OK) return st;
  if (dtype != RGC_BF16) return RGC_ERR_DTYPE;
  if (n_docs == 0 || max_seqlen == 0 || total_tokens == 0) return RGC_OK;
  if (!o || !q || !k || !v || !cu_seqlens) return RGC_ERR_NULL;
  if (max_seqlen > total_tokens) return RGC_ERR_CAPACITY;
  if (!(scale > 0.f) || !std::isfinite(scale)) return RGC_ERR_ARG;
  if (!aligned16(o) || !aligned16(q) || !aligned16(k) || !aligned16(v)) return RGC_ERR_LAYOUT;
  if (!stride_ok(q_ts, dtype) || !stride_ok(q_hs, dtype) || !stride_ok(o_ts, dtype) || !stride_ok(o_hs, dtype) ||
      !stride_ok(kv_ts, dtype) || !stride_ok(kv_hs, dtype))
    return RGC_ERR_LAYOUT;
  if (!token_stride_ok(kv_ts)) return RGC_ERR_LAYOUT;
  if ((int64_t)n_docs * Hq * ((max_seqlen + 255) / 256) > 0x7FFFFFFFLL) return RGC_ERR_SHAPE;
  AttnParams p = {};
  p.o = o;
  p.q = q;
  p.k = k;
  p.v = v;
  p.B = n_docs;
  p.Sq = max_seqlen;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  p.S_max = total_tokens;
  p.q_sb = 0;
  p.q_ss = q_ts;
  p.q_sh = q_hs;
  p.o_sb = 0;
  p.o_ss = o_ts;
  p.o_sh = o_hs;
  p.kv_sb = 0;
  p.kv_sh = kv_hs;
  p.kv_ss = kv_ts;
  p.q_start = nullptr;
  p.cu_seqlens = cu_seqlens;
  p.seq_lens = nullptr;
  p.max_len = total_tokens;
  p.scale = scale;
  p.lse = lse;
  p.err = err_flag;
  return hip_status(launch_prefill_bf16(p, reinterpret_cast<hipStream_t>(stream)));
}

size_t rgc_gqa_attn_backward_workspace_size(int B, int S, int Hq) {
  if (B < 0 || S < 0 || Hq <= 0) return 0;
  return backward_workspace_bytes(B, S, Hq);
}

int rgc_gqa_attn_backward(void* dq, void* dk, void* dv, const void* q, const void* k, const void* v,
                          const void* o, const void* d_o, const float* lse, int dtype, int B, int S, int Hq,
                          int Hkv, int D, int64_t q_sb, int64_t q_ss, int64_t q_sh, int64_t kv_sb,
                          int64_t kv_ss, int64_t kv_sh, float scale, void* workspace, size_t ws_bytes,
                          void* stream) {
  int st = check_attn_common(dtype, B, S, Hq, Hkv, D, S);
  if (st != RGC_OK) return st;
  if (dtype != RGC_BF16) return RGC_ERR_DTYPE;
  if (B == 0 || S == 0) return RGC_OK;
  if (!dq || !dk || !dv || !q || !k || !v || !o || !d_o || !lse) return RGC_ERR_NULL;
  if (!(scale > 0.f) || !std::isfinite(scale)) return RGC_ERR_ARG;
  if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
      !aligned16(o) || !aligned16(d_o))
    return RGC_ERR_LAYOUT;
  if (!stride_ok(q_sb, dtype) || !stride_ok(q_ss, dtype) || !stride_ok(q_sh, dtype) ||
      !stride_ok(kv_sb, dtype) || !stride_ok(kv_ss, dtype) || !stride_ok(kv_sh, dtype))
    return RGC_ERR_LAYOUT;
  if ((int64_t)B * S * Hq > 0x7FFFFFFFLL) return RGC_ERR_SHAPE;
  if (q_ss < 0 || q_ss >= (int64_t(1) << 24) || kv_ss < 0 || kv_ss >= (int64_t(1) << 24))
    return RGC_ERR_LAYOUT;  // 32-bit row offsets in the kernels
  const size_t need = backward_workspace_bytes(B, S, Hq);
  if (!workspace || ws_bytes < need) return RGC_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return RGC_ERR_LAYOUT;
  BwdParams p = {};
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dO = d_o;
  p.lse = lse;
  p.B = B;
  p.S = S;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  p.q_sb = q_sb;
  p.q_ss = q_ss;
  p.q_sh = q_sh;
  p.kv_sb = kv_sb;
  p.kv_ss = kv_ss;
  p.kv_sh = kv_sh;
  p.scale = scale;
  return hip_status(launch_backward_bf16(p, workspace, reinterpret_cast<hipStream_t>(stream)));
}

int rgc_diff_attn_prefill(void* o, const void* q1, const void* q2, const void* k1_cache,
                          const void* k2_cache, const void* v_cache, int dtype, int B, int Sq, int Hq,
                          int Hkv, int D, int S_max, int64_t q_sb, int64_t q_ss, int64_t q_sh,
                          int64_t o_sb, int64_t o_ss, int64_t o_sh, int64_t kv_sb, int64_t kv_sh,
                          int64_t kv_ss, const int32_t* q_start, float lambda, float scale,
                          int32_t* err_flag, void* stream) {
  int st = check_attn_common(dtype, B, Sq, Hq, Hkv, D, S_max);
  if (st != RGC_OK) return st;
  if (dtype != RGC_BF16) return RGC_ERR_DTYPE;
  if (B == 0 || Sq == 0) return RGC_OK;
  if (!o || !q1 || !q2 || !k1_cache || !k2_cache || !v_cache) return RGC_ERR_NULL;
  if (Sq > S_max) return RGC_ERR_CAPACITY;
  if (!(scale > 0.f) || !std::isfinite(scale) || !std::isfinite(lambda)) return RGC_ERR_ARG;
  if (!aligned16(o) || !aligned16(q1) || !aligned16(q2) || !aligned16(k1_cache) || !aligned16(k2_cache) ||
      !aligned16(v_cache))
    return RGC_ERR_LAYOUT;
  if (!stride_ok(q_sb, dtype) || !stride_ok(q_ss, dtype) || !stride_ok(q_sh, dtype) ||
      !stride_ok(o_sb, dtype) || !stride_ok(o_ss, dtype) || !stride_ok(o_sh, dtype) ||
      !stride_ok(kv_sb, dtype) || !stride_ok(kv_sh, dtype) || !stride_ok(kv_ss, dtype))
    return RGC_ERR_LAYOUT;
  if (!token_stride_ok(kv_ss)) return RGC_ERR_LAYOUT;
  if ((int64_t)B * Sq * Hq > 0x7FFFFFFFLL) return RGC_ERR_SHAPE;
  DiffParams dp = {};
  AttnParams& p = dp.a;
  p.o = o;
  p.q = q1;
  p.k = k1_cache;
  p.v = v_cache;
  p.B = B;
  p.Sq = Sq;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  p.S_max = S_max;
  p.q_sb = q_sb;
  p.q_ss = q_ss;
  p.q_sh = q_sh;
  p.o_sb = o_sb;
  p.o_ss = o_ss;
  p.o_sh = o_sh;
  p.kv_sb = kv_sb;
  p.kv_sh = kv_sh;
  p.kv_ss = kv_ss;
  p.q_start = q_start;
  p.seq_lens = nullptr;
  p.max_len = S_max;
  p.scale = scale;
  p.lse = nullptr;
  p.err = err_flag;
  dp.q2 = q2;
  dp.k2 = k2_cache;
  dp.lambda = lambda;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (D == 64) return hip_status(launch_diff_bf16(dp, s));
  // Other head dims: the two maps' outputs are linear in V, so o is the
  // causal prefill of (q1, K1, V), then the prefill of (q2, K2, V) added
  // with weight -lambda in its epilogue (two launches on the stream).
  hipError_t e = launch_prefill_bf16(p, s);
  if (e != hipSuccess) return hip_status(e);
  AttnParams p2 = p;
  p2.q = q2;
  p2.k = k2_cache;
  p2.out_add = 1;
  p2.out_add_scale = -lambda;
  return hip_status(launch_prefill_bf16(p2, s));
}

size_t rgc_diff_attn_decode_workspace_size(int B, int Hq, int Hkv, int D, int max_len) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || !headdim_ok(D) || max_len < 1) return 0;
  return diff_decode_workspace_bytes(B, Hq, D, max_len);
}

int rgc_diff_attn_decode(void* o, const void* q1, const void* q2, const void* k1_cache, const void* k2_cache,
                         const void* v_cache, int dtype, int B, int Hq, int Hkv, int D, int S_max, int64_t q_sb,
                         int64_t q_sh, int64_t o_sb, int64_t o_sh, int64_t kv_sb, int64_t kv_sh, int64_t kv_ss,
                         const int32_t* seq_lens, int max_len, float lambda, float scale, void* workspace,
                         size_t ws_bytes, int32_t* err_flag, void* stream) {
  int st = check_attn_common(dtype, B, 1, Hq, Hkv, D, S_max);
  if (st != RGC_OK) return st;
  if (dtype != RGC_BF16) return RGC_ERR_DTYPE;
  if (B == 0) return RGC_OK;
  if (!o || !q1 || !q2 || !k1_cache || !k2_cache || !v_cache || !seq_lens) return RGC_ERR_NULL;
  if (max_len < 1 || max_len > S_max) return RGC_ERR_CAPACITY;
  if (!(scale > 0.f) || !std::isfinite(scale) || !std::isfinite(lambda)) return RGC_ERR_ARG;
  if (!aligned16(o) || !aligned16(q1) || !aligned16(q2) || !aligned16(k1_cache) || !aligned16(k2_cache) ||
      !aligned16(v_cache))
    return RGC_ERR_LAYOUT;
  if (!stride_ok(q_sb, dtype) || !stride_ok(q_sh, dtype) || !stride_ok(o_sb, dtype) || !stride_ok(o_sh, dtype) ||
      !stride_ok(kv_sb, dtype) || !stride_ok(kv_sh, dtype) || !stride_ok(kv_ss, dtype))
    return RGC_ERR_LAYOUT;
  const size_t need = diff_decode_workspace_bytes(B, Hq, D, max_len);
  if (!workspace || ws_bytes < need) return RGC_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return RGC_ERR_LAYOUT;
  DiffParams dp = {};
  AttnParams& p = dp.a;
  p.o = o;
  p.q = q1;
  p.k = k1_cache;
  p.v = v_cache;
  p.B = B;
  p.Sq = 1;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  p.S_max = S_max;
  p.q_sb = q_sb;
  p.q_sh = q_sh;
  p.o_sb = o_sb;
  p.o_sh = o_sh;
  p.kv_sb = kv_sb;
  p.kv_sh = kv_sh;
  p.kv_ss = kv_ss;
  p.seq_lens = seq_lens;
  p.max_len = max_len;
  p.scale = scale;
  p.err = err_flag;
  dp.q2 = q2;
  dp.k2 = k2_cache;
  dp.lambda = lambda;
  return hip_status(launch_diff_decode_bf16(dp, workspace, reinterpret_cast<hipStream_t>(stream)));
}

size_t rgc_gqa_attn_decode_workspace_size(int B, int Hq, int Hkv, int D, int max_len) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || !headdim_ok(D) || max_len < 1) return 0;
  return decode_workspace_bytes(B, Hq, Hkv, D, max_len);
}

int rgc_gqa_attn_decode(void* o, const void* q, const void* k_cache, const void* v_cache,
                        int dtype, int B, int Hq, int Hkv, int D, int S_max, int64_t q_sb,
                        int64_t q_sh, int64_t o_sb, int64_t o_sh, int64_t kv_sb, int64_t kv_sh,
                        int64_t kv_ss, const int32_t* seq_lens, int max_len, float scale,
                        void* workspace, size_t ws_bytes, float* lse, int32_t* err_flag,
                        void* stream) {
  int st = check_attn_common(dtype, B, 1, Hq, Hkv, D, S_max);
  if (st != RGC_OK) return st;
  if (B == 0) return RGC_OK;
  if (!o || !q || !k_cache || !v_cache || !seq_lens) return RGC_ERR_NULL;
  if (max_len < 1 || max_len > S_max) return RGC_ERR_CAPACITY;
  if (!(scale > 0.f) || !std::isfinite(scale)) return RGC_ERR_ARG;
  if (!aligned16(o) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return RGC_ERR_LAYOUT;
  if (!stride_ok(q_sb, dtype) || !stride_ok(q_sh, dtype) || !stride_ok(o_sb, dtype) ||
      !stride_ok(o_sh, dtype) || !stride_ok(kv_sb, dtype) || !stride_ok(kv_sh, dtype) ||
      !stride_ok(kv_ss, dtype))
    return RGC_ERR_LAYOUT;
  AttnParams p = {};
  p.o = o;
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.B = B;
  p.Sq = 1;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  p.S_max = S_max;
  p.q_sb = q_sb;
  p.q_ss = 0;
  p.q_sh = q_sh;
  p.o_sb = o_sb;
  p.o_ss = 0;
  p.o_sh = o_sh;
  p.kv_sb = kv_sb;
  p.kv_sh = kv_sh;
  p.kv_ss = kv_ss;
  p.q_start = nullptr;
  p.seq_lens = seq_lens;
  p.max_len = max_len;
  p.scale = scale;
  p.lse = lse;
  p.err = err_flag;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == RGC_F32) return hip_status(launch_attn_f32(p, true, s));
  const size_t need = decode_workspace_bytes(B, Hq, Hkv, D, max_len);
  if (!workspace || ws_bytes < need) return RGC_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return RGC_ERR_LAYOUT;
  return hip_status(launch_decode_bf16(p, workspace, s));
}

namespace {

// The one-launch step; with use_static the partials go to the library's own
// per-GPU array instead of a caller workspace (nothing is allocated).
int decode_rope_append_impl(void* o, const void* q, const void* k_new, const void* v_new, void* k_cache,
                            void* v_cache, int dtype, int B, int Hq, int Hkv, int D, int S_max, int64_t q_sb,
                            int64_t q_sh, int64_t n_sb, int64_t n_sh, int64_t o_sb, int64_t o_sh, int64_t kv_sb,
                            int64_t kv_sh, int64_t kv_ss, const int32_t* seq_lens, int max_len, double base,
                            int style, float scale, void* workspace, size_t ws_bytes, bool use_static, float* lse,
                            int32_t* err_flag, void* stream) {
  int st = check_attn_common(dtype, B, 1, Hq, Hkv, D, S_max);
  if (st != RGC_OK) return st;
  if (dtype != RGC_BF16) return RGC_ERR_DTYPE;
  if (style != RGC_ROPE_HALF && style != RGC_ROPE_INTERLEAVED) return RGC_ERR_ARG;
  if (!(base > 0.0) || !std::isfinite(base)) return RGC_ERR_ARG;
  if (B == 0) return RGC_OK;
  if (!o || !q || !k_new || !v_new || !k_cache || !v_cache || !seq_lens) return RGC_ERR_NULL;
  if (max_len < 1 || max_len > S_max) return RGC_ERR_CAPACITY;
  if (!(scale > 0.f) || !std::isfinite(scale)) return RGC_ERR_ARG;
  if (!aligned16(o) || !aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return RGC_ERR_LAYOUT;
  if (!stride_ok(q_sb, dtype) || !stride_ok(q_sh, dtype) || !stride_ok(n_sb, dtype) || !stride_ok(n_sh, dtype) ||
      !stride_ok(o_sb, dtype) || !stride_ok(o_sh, dtype) || !stride_ok(kv_sb, dtype) ||
      !stride_ok(kv_sh, dtype) || !stride_ok(kv_ss, dtype))
    return RGC_ERR_LAYOUT;
  const size_t need = decode_workspace_bytes(B, Hq, Hkv, D, max_len);
  if (use_static) {
    if (need > kDecodeStaticScratchBytes) return RGC_ERR_WORKSPACE;
    if (decode_static_scratch(&workspace) != hipSuccess) return RGC_ERR_HIP;
  } else {
    if (!workspace || ws_bytes < need) return RGC_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return RGC_ERR_LAYOUT;
  }
  AttnParams p = {};
  p.o = o;
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.B = B;
  p.Sq = 1;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  p.S_max = S_max;
  p.q_sb = q_sb;
  p.q_sh = q_sh;
  p.o_sb = o_sb;
  p.o_sh = o_sh;
  p.kv_sb = kv_sb;
  p.kv_sh = kv_sh;
  p.kv_ss = kv_ss;
  p.seq_lens = seq_lens;
  p.max_len = max_len;
  p.scale = scale;
  p.lse = lse;
  p.err = err_flag;
  DecodeRope r = {};
  r.k_new = k_new;
  r.v_new = v_new;
  r.k_cache = k_cache;
  r.v_cache = v_cache;
  r.n_sb = n_sb;
  r.n_sh = n_sh;
  r.style = style;
  for (int i = 0; i < 64; ++i) r.theta[i] = i < D / 2 ? std::pow(base, -2.0 * (double)i / (double)D) : 0.0;
  return hip_status(launch_decode_rope_bf16(p, r, workspace, reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

int rgc_gqa_attn_decode_rope_append(void* o, const void* q, const void* k_new, const void* v_new, void* k_cache,
                                    void* v_cache, int dtype, int B, int Hq, int Hkv, int D, int S_max,
                                    int64_t q_sb, int64_t q_sh, int64_t n_sb, int64_t n_sh, int64_t o_sb,
                                    int64_t o_sh, int64_t kv_sb, int64_t kv_sh, int64_t kv_ss,
                                    const int32_t* seq_lens, int max_len, double base, int style, float scale,
                                    void* workspace, size_t ws_bytes, float* lse, int32_t* err_flag,
                                    void* stream) {
  return decode_rope_append_impl(o, q, k_new, v_new, k_cache, v_cache, dtype, B, Hq, Hkv, D, S_max, q_sb, q_sh,
                                 n_sb, n_sh, o_sb, o_sh, kv_sb, kv_sh, kv_ss, seq_lens, max_len, base, style,
                                 scale, workspace, ws_bytes, false, lse, err_flag, stream);
}

int rgc_gqa_attn_decode_rope_append_static(void* o, const void* q, const void* k_new, const void* v_new,
                                           void* k_cache, void* v_cache, int dtype, int B, int Hq, int Hkv,
                                           int D, int S_max, int64_t q_sb, int64_t q_sh, int64_t n_sb,
                                           int64_t n_sh, int64_t o_sb, int64_t o_sh, int64_t kv_sb,
                                           int64_t kv_sh, int64_t kv_ss, const int32_t* seq_lens, int max_len,
                                           double base, int style, float scale, float* lse, int32_t* err_flag,
                                           void* stream) {
  return decode_rope_append_impl(o, q, k_new, v_new, k_cache, v_cache, dtype, B, Hq, Hkv, D, S_max, q_sb, q_sh,
                                 n_sb, n_sh, o_sb, o_sh, kv_sb, kv_sh, kv_ss, seq_lens, max_len, base, style,
                                 scale, nullptr, 0, true, lse, err_flag, stream);
}

}  // extern "C"
