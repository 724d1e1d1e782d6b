/*
 * orc.h -- plain fp64 CPU oracle for causal grouped-query attention (GQA) with
 * rotary position embedding (RoPE) over a key/value cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the HIP library's
 * results.  Only the test-suite, the smoke check and the benchmark's CPU
 * baseline load it.  It shares no source, header, table or helper with the HIP
 * library, and the HIP library never calls it.
 *
 * Every routine reads its inputs in their storage type exactly (fp32, or bf16
 * widened by a bit shift), computes in IEEE double with libm, sums in
 * ascending index order, and uses a two-pass (max, then exp-sum) softmax.
 *
 * Sources (web pages; cited by title and section):
 *  [P1] "750美元从零训练3个LLM：一位开发者的实战复盘" (kongchang.com)
 *       - section "V1：现代架构基线": RoPE rotates query and key vectors by a
 *         position-dependent angle so that a score depends only on the
 *         distance between the two tokens.
 *       - section "V2：引入前沿技术": GQA splits the query heads into groups
 *         that each share one key/value head; DiffAttn subtracts a second
 *         attention map from the first to cancel common-mode noise.
 *       - section "V3：扩容与推理优化": the KV cache stores every step's keys
 *         and values; a new token computes only its own q, k, v, appends k, v
 *         and attends over the cache; outputs with and without the cache agree.
 *       - section "五条来之不易的工程教训", lesson 4: check the configuration
 *         with assertions, including that the head counts divide.
 *  [P2] "从零手训LLaMa：125M模型11小时训练全记录" (kongchang.com)
 *       - section "核心架构：手动实现LLaMa的四个关键组件": RoPE is a rotation
 *         matrix; query heads share key/value heads; the per-layer cache of K
 *         and V makes each generation step linear in the sequence length.
 *  [P3] "训练3.8B LLM至0.384 CORE，成本998美元 – Hugo Vergnes"
 *       - section "设置" (setup): 24 query heads and 8 KV heads.
 *       - section "无效的方法" (what did not work): plain causal SDPA.
 *  [P5] m.nxbn.cn build-an-LLM-from-scratch page, section 3.1 (code
 *       skeleton): causal scaled-dot-product attention on (B,H,T,hd) views
 *       of (B,T,H,hd) activations; the causal mask includes the diagonal.
 *
 * Readings taken where the pages are silent (the pages print no formula):
 *  - theta_i = base^(-2i/D), i < D/2 (the rotary construction the [P1] V1
 *    paragraph attributes to Su, 2021); rotation by +pos*theta_i.
 *  - pairs (x_i, x_{i+D/2}) ("half") or (x_{2i}, x_{2i+1}) ("interleaved").
 *  - query head h reads KV head h / (Hq/Hkv) (contiguous groups).
 *  - query row s of batch b sits at absolute slot q_start[b] + s and sees
 *    keys 0..q_start[b]+s inclusive.
 *  - differential attention: o = sum_j (w1_j - lambda * w2_j) v_j with a
 *    constant lambda and no extra normalisation.
 *
 * Parity pins (what checks this oracle against something other than itself)
 * live in the test-suite: torch float64 SDPA, transformers' LLaMA/GPT-J
 * rotary helpers, closed forms and invariants, and brute-force loops.
 */
#ifndef ORC_H
#define ORC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_ROPE_HALF = 0, ORC_ROPE_INTERLEAVED = 1 };
enum {
  ORC_OK = 0,
  ORC_ERR_ARG = -1,      /* bad shape, dtype or style                     */
  ORC_ERR_GROUP = -3,    /* Hq is not a multiple of Hkv                   */
  ORC_ERR_CAPACITY = -7  /* a slot or position falls outside the cache    */
};

/* Round a double to the nearest bfloat16 (ties to even); returns the bits. */
uint16_t orc_bf16_bits(double x);

/*
 * RoPE, unrounded.  x: [B,S,H,D] elements of type dt with element strides
 * (sb, ss, sh) and unit stride along D.  Token (b,s) sits at position
 * pos0[b] + s (pos0 may be NULL: all zero).  out: contiguous [B,S,H,D]
 * doubles.  Follows [P1] V1 and [P2] (rotation of q and k).
 */
int orc_rope_f64(double* out, const void* x, int dt, int B, int S, int H,
                 int D, int64_t sb, int64_t ss, int64_t sh,
                 const int32_t* pos0, double base, int style);

/*
 * QK normalisation then RoPE, unrounded: each head vector is divided by
 * sqrt(mean of its squares + eps) (no weight), then rotated as by
 * orc_rope_f64.  Same layout and out as orc_rope_f64.  Follows [P2] (RMSNorm)
 * and [P3] 设置 (q and k are normalised).
 */
int orc_norm_rope_f64(double* out, const void* x, int dt, int B, int S, int H,
                      int D, int64_t sb, int64_t ss, int64_t sh,
                      const int32_t* pos0, double base, int style, double eps);

/* RoPE in place: the exact double result rounded once to dt. */
int orc_rope_apply(void* x, int dt, int B, int S, int H, int D, int64_t sb,
                   int64_t ss, int64_t sh, const int32_t* pos0, double base,
                   int style);

/*
 * Cache append ([P1] V3, [P2]): cache[b, h, pos0[b]+s, :] = new[b, s, h, :]
 * for k and v.  Caches use element strides (c_sb, c_sh, c_ss); new rows use
 * (sb, ss, sh).  A byte copy.  Slots outside [0, S_max) are not written and
 * the call returns ORC_ERR_CAPACITY after copying the valid ones.
 */
int orc_kv_cache_append(void* k_cache, void* v_cache, int dt, int B, int Hkv,
                        int D, int S_max, int64_t c_sb, int64_t c_sh,
                        int64_t c_ss, const void* k_new, const void* v_new,
                        int S_new, int64_t sb, int64_t ss, int64_t sh,
                        const int32_t* pos0);

/*
 * Causal GQA attention ([P1] V2/V3, [P2], [P3], [P5]).
 *   q:  [B,Sq,Hq,D] with strides (q_sb, q_ss, q_sh)
 *   k_cache, v_cache: [B,Hkv,S_max,D] with strides (kv_sb, kv_sh, kv_ss)
 *   row s of batch b at slot p = q_start[b] + s (q_start NULL: all zero)
 *   o:   contiguous [B,Sq,Hq,D] doubles
 *   lse: contiguous [B,Hq,Sq] doubles (natural log of the softmax
 *        denominator plus the row maximum), may be NULL
 * z_j = scale * <q, K_j>, w = softmax(z over j <= p), o = sum_j w_j V_j.
 */
int orc_attn(double* o, double* lse, const void* q, const void* k_cache,
             const void* v_cache, int dt, int B, int Sq, int Hq, int Hkv,
             int D, int S_max, int64_t q_sb, int64_t q_ss, int64_t q_sh,
             int64_t kv_sb, int64_t kv_sh, int64_t kv_ss,
             const int32_t* q_start, double scale, int nthreads);

/*
 * Cached decode: one query row per sequence at slot seq_lens[b] - 1, the
 * cache already holding the new token.  q: [B,Hq,D] with strides (q_sb,
 * q_sh); o: contiguous [B,Hq,D] doubles; lse: [B,Hq] or NULL.
 */
int orc_attn_decode(double* o, double* lse, const void* q,
                    const void* k_cache, const void* v_cache, int dt, int B,
                    int Hq, int Hkv, int D, int S_max, int64_t q_sb,
                    int64_t q_sh, int64_t kv_sb, int64_t kv_sh, int64_t kv_ss,
                    const int32_t* seq_lens, double scale, int nthreads);

/*
 * Differential attention ([P1] V2): two causal softmax maps over the same
 * keys' positions, w1 from (q1, k1) and w2 from (q2, k2); o = sum_j
 * (w1_j - lambda * w2_j) v_j.  q1, q2: [B,S,Hq,D] strides (q_sb, q_ss,
 * q_sh); k1, k2: [B,Hkv,S_max,D] strides (kv_sb, kv_sh, kv_ss); v:
 * [B,Hkv,S_max,Dv] strides (v_sb, v_sh, v_ss); o contiguous [B,S,Hq,Dv]
 * doubles.  Row s of batch b sits at slot q_start[b] + s.
 */
int orc_diff_attn(double* o, const void* q1, const void* q2, const void* k1,
                  const void* k2, const void* v, int dt, int B, int S, int Hq,
                  int Hkv, int D, int Dv, int S_max, int64_t q_sb,
                  int64_t q_ss, int64_t q_sh, int64_t kv_sb, int64_t kv_sh,
                  int64_t kv_ss, int64_t v_sb, int64_t v_sh, int64_t v_ss,
                  const int32_t* q_start, double lambda,
                  double scale, int nthreads);

/*
 * Gradients of causal GQA self-attention for output gradient dO (same layout
 * as q): dq [B,S,Hq,D], dk and dv [B,S,Hkv,D], contiguous doubles; dk and dv
 * sum over the query heads of each group.  k, v [B,S,Hkv,D] with element
 * strides (kv_sb, kv_ss, kv_sh).
 */
int orc_attn_backward(double* dq, double* dk, double* dv, const void* q,
                      const void* k, const void* v, const void* dO, int dt,
                      int B, int S, int Hq, int Hkv, int D, int64_t q_sb,
                      int64_t q_ss, int64_t q_sh, int64_t kv_sb, int64_t kv_ss,
                      int64_t kv_sh, double scale, int nthreads);

/*
 * Gradient through RoPE: g [B,S,H,D] (layout as orc_rope_f64) turned back by
 * the angle of its position; out contiguous doubles.
 */
int orc_rope_grad_f64(double* out, const void* g, int dt, int B, int S, int H,
                      int D, int64_t sb, int64_t ss, int64_t sh,
                      const int32_t* pos0, double base, int style);

#ifdef __cplusplus
}
#endif

#endif /* ORC_H */
