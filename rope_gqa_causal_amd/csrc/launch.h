// launch.h -- internal launch interface between the C ABI (api.hip) and the
// kernels.  Every launcher enqueues on `stream` and returns the HIP status of
// the launch; argument checking happens before, in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rgc {

// Brackets one kernel launch with HIP events on its stream while per-kernel
// timing is on.  Only the instrumented build (RGC_KERNEL_TIMING, timing.hip)
// records anything; in the product build it is an empty object.  Construct
// it right before the launch, in the scope that ends right after it.
#ifdef RGC_KERNEL_TIMING
class KernelTimer {
 public:
  KernelTimer(const char* name, hipStream_t stream);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

 private:
  const char* name_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr, stop_ = nullptr;
};
int timing_enable(int on);
long timing_report(char* buf, size_t bytes);
#else
class KernelTimer {
 public:
  KernelTimer(const char*, hipStream_t) {}
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;
};
#endif

enum { DT_F32 = 0, DT_BF16 = 1 };
enum { ROPE_HALF = 0, ROPE_INTERLEAVED = 1 };

constexpr int kMaxRopeDim = 256;

struct RopeParams {
  void* x;
  int B, S, H, D;
  int64_t sb, ss, sh;
  const int32_t* pos0;
  float sin_sign;                 // +1: rotate by the angle; -1: rotate back (the gradient)
  double theta[kMaxRopeDim / 2];  // base^(-2i/D), formed on the host in fp64
};
hipError_t launch_rope(const RopeParams& p, int dtype, int style, hipStream_t stream);

// Fused prologue: RoPE on q (in place) and on the new k, then k and v into
// the caches; the token's position is its cache slot pos0[b] + s.
struct RopeAppendParams {
  void* q;
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  int B, S, Hq, Hkv, D, S_max;
  int64_t q_sb, q_ss, q_sh;
  int64_t n_sb, n_ss, n_sh;
  int64_t c_sb, c_sh, c_ss;
  const int32_t* pos0;
  int32_t* err;
  float eps;                      // QK normalisation (used by the normalising variant)
  double theta[kMaxRopeDim / 2];
};
hipError_t launch_rope_append(const RopeAppendParams& p, int dtype, int style, bool norm, hipStream_t stream);

struct AppendParams {
  void* k_cache;
  void* v_cache;
  const void* k_new;
  const void* v_new;
  int B, Hkv, D, S_max, S_new;
  int64_t c_sb, c_sh, c_ss;
  int64_t sb, ss, sh;
  const int32_t* pos0;
  int32_t* err;
};
hipError_t launch_append(const AppendParams& p, int dtype, hipStream_t stream);

// Causal attention over a cache.  Query row s of sequence b sits at slot
// q_start[b] + s (prefill), or at seq_lens[b] - 1 with Sq == 1 (decode).
struct AttnParams {
  void* o;
  const void* q;
  const void* k;
  const void* v;
  int B, Sq, Hq, Hkv, D, S_max;
  int64_t q_sb, q_ss, q_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t kv_sb, kv_sh, kv_ss;
  const int32_t* q_start;   // prefill
  const int32_t* cu_seqlens;  // packed-document prefill: [B + 1] token offsets (else NULL)
  const int32_t* seq_lens;  // decode
  int max_len;              // decode: host bound on seq_lens
  float scale;
  float* lse;               // [B,Hq,Sq] or NULL
  int32_t* err;
  int out_add;              // bf16 prefill: 0 stores o; 1 adds out_add_scale * (this pass's o) to o
  float out_add_scale;
};
hipError_t launch_prefill_bf16(const AttnParams& p, hipStream_t stream);
hipError_t launch_attn_f32(const AttnParams& p, bool decode, hipStream_t stream);

// Differential attention: q / k / v / o of `a` are q1, k1 cache, v cache
// and o; q2 and k2 share the strides of q1 and k1.
struct DiffParams {
  AttnParams a;
  const void* q2;
  const void* k2;
  float lambda;
};
hipError_t launch_diff_bf16(const DiffParams& p, hipStream_t stream);
// Cached decode of differential attention: a.seq_lens and a.max_len as in
// the decode; the caller's workspace holds both maps' chunk partials.
size_t diff_decode_workspace_bytes(int B, int Hq, int D, int max_len);
hipError_t launch_diff_decode_bf16(const DiffParams& p, void* ws, hipStream_t stream);

// Gradients of causal GQA self-attention: q, o, dO, dq share one layout
// [B,S,Hq,D]; k, v, dk, dv share [B,S,Hkv,D]; lse [B,Hq,S] from the forward.
struct BwdParams {
  void* dq;
  void* dk;
  void* dv;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;
  int B, S, Hq, Hkv, D;
  int64_t q_sb, q_ss, q_sh;
  int64_t kv_sb, kv_ss, kv_sh;
  float scale;
};
size_t backward_workspace_bytes(int B, int S, int Hq);
hipError_t launch_backward_bf16(const BwdParams& p, void* workspace, hipStream_t stream);
// The dQ kernel; it also writes Dlt = rowsum(dO * O) ([B,Hq,S] fp32) to dlt.
hipError_t launch_dq_bf16(const BwdParams& p, float* dlt, hipStream_t stream);

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int D, int max_len);
hipError_t launch_decode_bf16(const AttnParams& p, void* ws, hipStream_t stream);

// The new token's RoPE and cache append, done by the decode itself: q (read
// from AttnParams::q, left unrotated) and k_new are turned at position
// seq_lens[b] - 1, and the rotated k and v_new are written into the caches
// at that slot.
struct DecodeRope {
  const void* k_new;   // [B,Hkv,D] of bf16, strides (n_sb, n_sh)
  const void* v_new;
  void* k_cache;       // the caches of AttnParams, writable
  void* v_cache;
  int64_t n_sb, n_sh;
  int style;           // ROPE_HALF or ROPE_INTERLEAVED
  double theta[64];    // base^(-2i/D) for i < D/2, formed on the host in fp64
};
hipError_t launch_decode_rope_bf16(const AttnParams& p, const DecodeRope& r, void* ws, hipStream_t stream);

// A decode workspace the library owns, for callers that cannot allocate:
// a file-scope device array of kDecodeStaticScratchBytes per GPU.  Returns
// the current device's copy (its address is looked up once per device).
// Every call on one GPU shares it, so calls that overlap on a GPU race.
constexpr size_t kDecodeStaticScratchBytes = size_t(16) << 20;
hipError_t decode_static_scratch(void** ptr);

}  // namespace rgc
