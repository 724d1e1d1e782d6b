/*
 * rgc.h -- C ABI of the MI355X (gfx950) library for causal grouped-query
 * attention with rotary position embedding over a key/value cache.
 *
 * The operations, and the pages that define them (cited by title and
 * section):
 *  - RoPE on q and k: page "750美元从零训练3个LLM：一位开发者的实战复盘"
 *    (kongchang.com), section "V1：现代架构基线"; page "从零手训LLaMa：125M
 *    模型11小时训练全记录" (kongchang.com), section "核心架构：手动实现LLaMa的
 *    四个关键组件" (RoPE as a rotation matrix).
 *  - KV cache append and cached decode: the first page, section
 *    "V3：扩容与推理优化"; the second page, the KV cache paragraph of the
 *    core-architecture section.
 *  - Grouped-query attention: the first page, section "V2：引入前沿技术";
 *    the second page, core-architecture section; page "训练3.8B LLM至0.384
 *    CORE，成本998美元 – Hugo Vergnes", section "设置" (24 query / 8 KV
 *    heads).
 *  - Causal attention with the diagonal included: the 3.8B page, section
 *    "无效的方法"; the m.nxbn.cn build-an-LLM page, section 3.1.
 *  - Differential attention: the first page, section "V2：引入前沿技术".
 *
 * Conventions shared by every entry point:
 *  - Every data pointer is a DEVICE pointer (HIP global memory) unless the
 *    argument says "host".  The caller owns every buffer; the library never
 *    allocates, frees or synchronises and keeps no mutable global state
 *    (per-kernel timing lives in a separate instrumented build,
 *    rgc_timing.h).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it and returns.
 *  - Shapes are element counts; strides are in ELEMENTS, not bytes.  The
 *    head-dimension stride is always 1.
 *  - dtype is RGC_F32 or RGC_BF16 and applies to every floating-point tensor
 *    of the call except lse (always fp32).
 *  - Base pointers must be 16-byte aligned and every stride a multiple of
 *    16 bytes' worth of elements (8 for bf16, 4 for fp32), so that rows load
 *    as 16-byte vectors; otherwise RGC_ERR_LAYOUT.
 *  - All arguments are checked on the host before anything is enqueued; a
 *    negative status means nothing was launched.  B == 0 or an empty
 *    sequence dimension is a successful no-op.
 *  - Facts only the device can see (a slot or length held in a device
 *    array that falls outside the cache) never cause an out-of-bounds
 *    access: the affected rows are skipped (append) or written as NaN
 *    (attention), and 1 is stored to *err_flag when err_flag is not NULL.
 *    The library never clears err_flag.
 *  - Query head h reads KV head h / (Hq / Hkv); Hq must be a multiple of
 *    Hkv (RGC_ERR_GROUP otherwise).
 *  - Supported head dims: 32, 64, 128 (RGC_ERR_HEADDIM otherwise).
 *  - Every attention entry point takes a softmax `scale` that must be
 *    positive and finite (RGC_ERR_ARG otherwise): the causal mask is the
 *    -inf score that a positive scale leaves at -inf.
 */
#ifndef RGC_H
#define RGC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RGC_ABI_VERSION 1

typedef enum { RGC_F32 = 0, RGC_BF16 = 1 } rgc_dtype;

typedef enum {
  RGC_OK = 0,
  RGC_ERR_NULL = -1,      /* a required pointer is NULL                      */
  RGC_ERR_SHAPE = -2,     /* a negative or inconsistent size                 */
  RGC_ERR_GROUP = -3,     /* Hq is not a multiple of Hkv                     */
  RGC_ERR_DTYPE = -4,     /* dtype is not RGC_F32 or RGC_BF16, or not one    */
                          /* the call supports                               */
  RGC_ERR_HEADDIM = -5,   /* head dim not supported                          */
  RGC_ERR_LAYOUT = -6,    /* misaligned pointer or stride                    */
  RGC_ERR_CAPACITY = -7,  /* a host-known length exceeds the cache           */
  RGC_ERR_WORKSPACE = -8, /* workspace missing or too small                  */
  RGC_ERR_HIP = -9,       /* the HIP runtime refused a launch                */
  RGC_ERR_ARG = -10       /* any other invalid argument                      */
} rgc_status;

typedef enum {
  RGC_ROPE_HALF = 0,       /* pairs (x_i, x_{i+D/2}), i < D/2                */
  RGC_ROPE_INTERLEAVED = 1 /* pairs (x_{2i}, x_{2i+1})                        */
} rgc_rope_style;

/* ABI version of the loaded library (RGC_ABI_VERSION at build time). */
int rgc_abi_version(void);

/* Static English text for a status code; never NULL. */
const char* rgc_status_string(int status);

/*
 * rgc_rope_apply -- rotary position embedding, in place.
 *   x     [B,S,H,D] of dtype, strides (sb, ss, sh); rotated in place.
 *   pos0  [B] int32 or NULL (all zero): token (b, s) sits at position
 *         pos0[b] + s.
 *   base  frequency base (10000 in the pages' models); theta_i =
 *         base^(-2i/D) for pair i < D/2.
 *   style RGC_ROPE_HALF or RGC_ROPE_INTERLEAVED.
 * Each pair (a, b) becomes (a cos t - b sin t, a sin t + b cos t) with
 * t = position * theta_i.  The angle is formed and reduced modulo 2*pi in
 * fp64; sine, cosine and the rotation run in fp32; bf16 results are rounded
 * to nearest even.  Apply to q and to k, never to v.  D may be any even
 * size from 2 to 256 here.
 */
int rgc_rope_apply(void* x, int dtype, int B, int S, int H, int D, int64_t sb,
                   int64_t ss, int64_t sh, const int32_t* pos0, double base,
                   int style, void* stream);

/*
 * rgc_rope_backward -- the gradient through RoPE: g [B,S,H,D] (layout as for
 * rgc_rope_apply) is turned back, in place, by the angle of its position.
 * The rotation is orthogonal, so this is exactly the gradient with respect
 * to the unrotated vector.  Arguments and errors as for rgc_rope_apply.
 */
int rgc_rope_backward(void* g, int dtype, int B, int S, int H, int D, int64_t sb, int64_t ss, int64_t sh,
                      const int32_t* pos0, double base, int style, void* stream);

/*
 * rgc_kv_cache_append -- copy new key and value rows into the caches.
 *   k_cache, v_cache  [B,Hkv,S_max,D] of dtype, strides (c_sb, c_sh, c_ss)
 *                     shared by both caches.
 *   k_new, v_new      [B,S_new,Hkv,D] of dtype, strides (sb, ss, sh) shared
 *                     by both.
 *   pos0              [B] int32, the first slot written for sequence b
 *                     (normally its current length).
 * cache[b, h, pos0[b] + s, :] = new[b, s, h, :], bit for bit.  Rows whose
 * slot falls outside [0, S_max) are skipped and flagged in *err_flag.  The
 * library never updates lengths: the caller advances its length array after
 * the append, on the same stream.  Store keys after RoPE (the cache holds
 * rotated keys and raw values).
 */
int rgc_kv_cache_append(void* k_cache, void* v_cache, int dtype, int B,
                        int Hkv, int D, int S_max, int64_t c_sb, int64_t c_sh,
                        int64_t c_ss, const void* k_new, const void* v_new,
                        int S_new, int64_t sb, int64_t ss, int64_t sh,
                        const int32_t* pos0, int32_t* err_flag, void* stream);

/*
 * rgc_rope_append -- the fused prologue of a generation step: RoPE on the
 * new tokens' q and k and the append of k and v to the caches, in one pass
 * over the data (the first page's section V3 describes the step: the new
 * token computes its q, k, v, which are rotated at its position, and its k
 * and v join the cache).
 *   q              [B,S,Hq,D] of dtype, strides (q_sb, q_ss, q_sh); rotated
 *                  in place.
 *   k_new, v_new   [B,S,Hkv,D] of dtype, strides (sb, ss, sh) shared by
 *                  both; read only.
 *   k_cache, v_cache  [B,Hkv,S_max,D] of dtype, strides (c_sb, c_sh, c_ss).
 *   pos0           [B] int32: token (b, s) has position and cache slot
 *                  pos0[b] + s.
 * Equivalent to rgc_rope_apply on q and on a copy of k_new, followed by
 * rgc_kv_cache_append of the rotated k and of v_new, bit for bit; k_new
 * itself is left unrotated.  A token whose slot falls outside [0, S_max)
 * still has its q rotated; its k and v are skipped and flagged.  Head dim
 * 32, 64 or 128; pointers and strides 16-byte aligned.
 */
int rgc_rope_append(void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache, int dtype,
                    int B, int S, int Hq, int Hkv, int D, int S_max, int64_t q_sb, int64_t q_ss,
                    int64_t q_sh, int64_t sb, int64_t ss, int64_t sh, int64_t c_sb, int64_t c_sh,
                    int64_t c_ss, const int32_t* pos0, double base, int style, int32_t* err_flag,
                    void* stream);

/*
 * rgc_norm_rope_append -- rgc_rope_append with QK normalisation first: each
 * q and k head vector is divided by sqrt(mean of its D squares + eps) before
 * it is rotated (RMS normalisation: page "从零手训LLaMa：125M模型11小时训练
 * 全记录", core-architecture section; q and k normalised: page "训练3.8B
 * LLM至0.384 CORE，成本998美元 – Hugo Vergnes", section 设置).  No learned
 * weight (the pages print none); v is copied unchanged.  Arguments as for
 * rgc_rope_append, plus eps >= 0 (finite; RGC_ERR_ARG otherwise).  The sum
 * of squares and the rotation run in fp32; the result is rounded once.
 */
int rgc_norm_rope_append(void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                         int dtype, int B, int S, int Hq, int Hkv, int D, int S_max, int64_t q_sb,
                         int64_t q_ss, int64_t q_sh, int64_t sb, int64_t ss, int64_t sh, int64_t c_sb,
                         int64_t c_sh, int64_t c_ss, const int32_t* pos0, double base, int style,
                         float eps, int32_t* err_flag, void* stream);

/*
 * rgc_gqa_attn_prefill -- causal GQA attention of a block of query rows over
 * the cache.
 *   o        [B,Sq,Hq,D] of dtype, strides (o_sb, o_ss, o_sh); written.
 *   q        [B,Sq,Hq,D] of dtype, strides (q_sb, q_ss, q_sh); already
 *            rotated.
 *   k_cache, v_cache  [B,Hkv,S_max,D], strides (kv_sb, kv_sh, kv_ss); a
 *            [B,S,Hkv,D] tensor stands in for a cache with kv_sb = S*Hkv*D,
 *            kv_sh = D, kv_ss = Hkv*D.
 *   q_start  [B] int32 or NULL (all zero): row s of sequence b sits at slot
 *            p = q_start[b] + s and attends to slots 0..p inclusive.
 *   scale    softmax scale (normally 1/sqrt(D)).
 *   lse      [B,Hq,Sq] fp32 contiguous or NULL: log-sum-exp of the scaled
 *            scores (natural log).
 * o[b,s,h,:] = sum_{j<=p} softmax_j(scale * q . K_j) V_j with KV head
 * h / (Hq/Hkv).  bf16: scores, softmax and accumulation in fp32, the
 * probabilities rounded to bf16 for the second product, the output rounded
 * to nearest even.  bf16: the token stride kv_ss must lie in [0, 2^24)
 * elements (RGC_ERR_LAYOUT otherwise).  A sequence whose q_start puts a row
 * outside [0, S_max) gets NaN rows and a flag.
 */
int rgc_gqa_attn_prefill(void* o, const void* q, const void* k_cache,
                         const void* v_cache, int dtype, int B, int Sq, int Hq,
                         int Hkv, int D, int S_max, int64_t q_sb, int64_t q_ss,
                         int64_t q_sh, int64_t o_sb, int64_t o_ss,
                         int64_t o_sh, int64_t kv_sb, int64_t kv_sh,
                         int64_t kv_ss, const int32_t* q_start, float scale,
                         float* lse, int32_t* err_flag, void* stream);

/*
 * rgc_gqa_attn_prefill_varlen -- causal GQA over packed documents: several
 * token sequences laid end to end, each token attending only to the tokens
 * of its own document at or before it (document masking with per-token
 * document ids: page "训练3.8B LLM至0.384 CORE，成本998美元 – Hugo Vergnes",
 * section 无效的方法).
 *   q, o       [T,Hq,D] bf16, strides (q_ts, q_hs) / (o_ts, o_hs); T =
 *              total_tokens.  o is written for every token of every document.
 *   k, v       [T,Hkv,D] bf16, both with strides (kv_ts, kv_hs): the packed,
 *              already rotated keys and values of the same tokens.
 *   cu_seqlens [n_docs + 1] int32, device: document i is tokens
 *              cu_seqlens[i] .. cu_seqlens[i+1]-1 (non-decreasing, from 0 to
 *              at most T).
 *   max_seqlen host: the longest document (sizes the launch).
 *   lse        [Hq,T] fp32 or NULL.
 * bf16 only; head dim 32, 64 or 128; kv_ts in [0, 2^24) elements
 * (RGC_ERR_LAYOUT otherwise).  Offsets that are decreasing, exceed T
 * or give a document longer than max_seqlen raise *err_flag and that
 * document is not computed.  Same arithmetic as rgc_gqa_attn_prefill.
 */
int rgc_gqa_attn_prefill_varlen(void* o, const void* q, const void* k, const void* v, int dtype, int n_docs,
                                const int32_t* cu_seqlens, int max_seqlen, int total_tokens, int Hq,
                                int Hkv, int D, int64_t q_ts, int64_t q_hs, int64_t o_ts, int64_t o_hs,
                                int64_t kv_ts, int64_t kv_hs, float scale, float* lse, int32_t* err_flag,
                                void* stream);

/*
 * rgc_gqa_attn_backward -- gradients of causal GQA self-attention (the
 * training pass of the attention the 3.8B page trains: page "训练3.8B LLM至
 * 0.384 CORE，成本998美元 – Hugo Vergnes", section 设置).  Row i of head h
 * attends to keys 0..i of its own sequence (no cache offset).
 *   dq               [B,S,Hq,D] bf16, written; q, o, d_o share its strides
 *                    (q_sb, q_ss, q_sh).
 *   dk, dv           [B,S,Hkv,D] bf16, written (summed over each group's
 *                    query heads); k, v share their strides (kv_sb, kv_ss,
 *                    kv_sh).
 *   q, k, v          the forward inputs (q and k already rotated).
 *   o, d_o           the forward output and its gradient.
 *   lse              [B,Hq,S] fp32: the forward's log-sum-exp
 *                    (rgc_gqa_attn_prefill's lse output, natural log).
 *   workspace        >= rgc_gqa_attn_backward_workspace_size bytes,
 *                    256-byte aligned, caller-owned scratch.
 * bf16 only (RGC_ERR_DTYPE); head dim 32, 64 or 128.  The token strides
 * q_ss and kv_ss must lie in [0, 2^24) elements (RGC_ERR_LAYOUT otherwise).  The
 * weights are recomputed from lse; P and dS are rounded to bf16 for the matrix cores and
 * accumulate in fp32.  For the gradient with respect to the unrotated q and
 * k, apply rgc_rope_backward to dq and dk.
 */
size_t rgc_gqa_attn_backward_workspace_size(int B, int S, int Hq);
int rgc_gqa_attn_backward(void* dq, void* dk, void* dv, const void* q, const void* k, const void* v,
                          const void* o, const void* d_o, const float* lse, int dtype, int B, int S, int Hq,
                          int Hkv, int D, int64_t q_sb, int64_t q_ss, int64_t q_sh, int64_t kv_sb,
                          int64_t kv_ss, int64_t kv_sh, float scale, void* workspace, size_t ws_bytes,
                          void* stream);

/*
 * rgc_diff_attn_prefill -- causal differential attention with grouped KV
 * heads (page "750美元从零训练3个LLM：一位开发者的实战复盘", section
 * "V2：引入前沿技术": a second attention map, weighted by lambda, is
 * subtracted from the first to cancel common-mode noise):
 *   o = (softmax(scale q1 K1^T) - lambda softmax(scale q2 K2^T)) V
 * over the keys at or before each row's slot, both maps causal, query head
 * h reading KV head h / (Hq/Hkv) for k1, k2 and v.
 *   o          [B,Sq,Hq,D] bf16, strides (o_sb, o_ss, o_sh); written.
 *   q1, q2     [B,Sq,Hq,D] bf16, both with strides (q_sb, q_ss, q_sh).
 *   k1_cache, k2_cache, v_cache  [B,Hkv,S_max,D] bf16, all three with
 *              strides (kv_sb, kv_sh, kv_ss); the value head dim equals D.
 *   q_start    [B] int32 or NULL, as in rgc_gqa_attn_prefill.
 *   lambda     the constant weight of the second map (no re-normalisation).
 *   scale      applied to both maps' scores (1/sqrt(D) is the usual value).
 * bf16 only (RGC_ERR_DTYPE otherwise); head dim 32, 64 or 128
 * (RGC_ERR_HEADDIM otherwise); kv_ss in [0, 2^24) elements (RGC_ERR_LAYOUT
 * otherwise).  Each map's weights are summed in fp32 and rounded to bf16
 * where they multiply V.  At head dim 64 (each map's head dim in the
 * differential workload) one kernel forms both maps and o is rounded once
 * from fp32.  At 32 and 128 the call is two launches of the causal prefill
 * on the stream: o = the first map's output (rounded to bf16), then o plus
 * -lambda times the second map's output (rounded to bf16), added in fp32
 * and rounded once more; with lambda = 0 the result is bit for bit that of
 * rgc_gqa_attn_prefill on (q1, K1, V).  A row whose slots fall outside the
 * cache gets NaN and raises *err_flag.
 */
int rgc_diff_attn_prefill(void* o, const void* q1, const void* q2,
                          const void* k1_cache, const void* k2_cache,
                          const void* v_cache, int dtype, int B, int Sq,
                          int Hq, int Hkv, int D, int S_max, int64_t q_sb,
                          int64_t q_ss, int64_t q_sh, int64_t o_sb,
                          int64_t o_ss, int64_t o_sh, int64_t kv_sb,
                          int64_t kv_sh, int64_t kv_ss,
                          const int32_t* q_start, float lambda, float scale,
                          int32_t* err_flag, void* stream);

/*
 * rgc_diff_attn_decode -- cached decode of differential attention (page
 * "750美元从零训练3个LLM：一位开发者的实战复盘", section "V2：引入前沿技术"):
 * one new query row per sequence,
 *   o = softmax(scale q1 K1^T) V - lambda softmax(scale q2 K2^T) V
 * over the L = seq_lens[b] cached slots of its KV head h / (Hq/Hkv).
 *   o          [B,Hq,D] bf16, strides (o_sb, o_sh); written.
 *   q1, q2     [B,Hq,D] bf16, both with strides (q_sb, q_sh); already
 *              rotated when RoPE is used.
 *   k1_cache, k2_cache, v_cache  [B,Hkv,S_max,D] bf16, all three with strides
 *              (kv_sb, kv_sh, kv_ss); the value head dim equals D.
 *   seq_lens   [B] int32: cache length including the new token (slot L-1
 *              is the query's own position); max_len as in
 *              rgc_gqa_attn_decode.
 *   lambda     the constant weight of the second map; scale as for the
 *              other attention calls.
 *   workspace  >= rgc_diff_attn_decode_workspace_size(B, Hq, Hkv, D,
 *              max_len) bytes, 256-byte aligned, caller-owned; its contents
 *              need no initialisation.  Calls that overlap in time must use
 *              different workspaces.
 * bf16 only (RGC_ERR_DTYPE); head dim 32, 64 or 128.  Each map is split
 * along the cache length, merged by max-rescaled sums, normalised by its own
 * sum of weights (fp32), and o is rounded once.  A sequence with seq_lens
 * outside [1, min(max_len, S_max)] gets NaN rows and the flag.
 */
size_t rgc_diff_attn_decode_workspace_size(int B, int Hq, int Hkv, int D, int max_len);
int rgc_diff_attn_decode(void* o, const void* q1, const void* q2, const void* k1_cache,
                         const void* k2_cache, const void* v_cache, int dtype, int B, int Hq,
                         int Hkv, int D, int S_max, int64_t q_sb, int64_t q_sh, int64_t o_sb,
                         int64_t o_sh, int64_t kv_sb, int64_t kv_sh, int64_t kv_ss,
                         const int32_t* seq_lens, int max_len, float lambda, float scale,
                         void* workspace, size_t ws_bytes, int32_t* err_flag, void* stream);

/*
 * Bytes of device workspace rgc_gqa_attn_decode needs for this shape
 * (max_len: the largest length it will be called with).  0 for an invalid
 * shape.
 */
size_t rgc_gqa_attn_decode_workspace_size(int B, int Hq, int Hkv, int D,
                                          int max_len);

/*
 * rgc_gqa_attn_decode -- one query row per sequence against its cache
 * (cached generation).
 *   o         [B,Hq,D] of dtype, strides (o_sb, o_sh); written.
 *   q         [B,Hq,D] of dtype, strides (q_sb, q_sh); already rotated.
 *   k_cache, v_cache  as in prefill.
 *   seq_lens  [B] int32: cache length of sequence b INCLUDING the new
 *             token, which sits at slot seq_lens[b] - 1 and is the query's
 *             own position.
 *   max_len   host: an upper bound of every seq_lens[b], 1..S_max; it sizes
 *             the launch.  Pass S_max when unknown.
 *   workspace device scratch of at least
 *             rgc_gqa_attn_decode_workspace_size(B, Hq, Hkv, D, max_len)
 *             bytes, 256-byte aligned, owned by the caller.  It holds the
 *             per-chunk partial results of one call; its contents need no
 *             initialisation and are meaningless afterwards.  Calls that
 *             overlap in time must use different workspaces.  With an
 *             fp32 dtype the workspace is not used (may be NULL).
 *   lse       [B,Hq] fp32 or NULL.
 * Same arithmetic as prefill.  The cache is split along its length; the
 * partial results are merged by max-rescaled sums.  When the split would not
 * give every compute unit a workgroup and max_len is short enough (at most
 * 2 x 12 x 128, 64 or 32 keys at D = 32, 64, 128), one workgroup per
 * (sequence, query head) walks the whole cache instead, in one launch.  A
 * sequence with
 * seq_lens outside [1, min(max_len, S_max)] gets NaN rows and a flag.
 */
int rgc_gqa_attn_decode(void* o, const void* q, const void* k_cache,
                        const void* v_cache, int dtype, int B, int Hq, int Hkv,
                        int D, int S_max, int64_t q_sb, int64_t q_sh,
                        int64_t o_sb, int64_t o_sh, int64_t kv_sb,
                        int64_t kv_sh, int64_t kv_ss, const int32_t* seq_lens,
                        int max_len, float scale, void* workspace,
                        size_t ws_bytes, float* lse, int32_t* err_flag,
                        void* stream);

/*
 * rgc_gqa_attn_decode_rope_append -- one whole cached-generation step for
 * one new token per sequence: RoPE on its q and k at its position, the
 * append of its k and v to the caches, and its attention over the cache, in
 * one decode launch (plus the chunk merge) instead of a prologue launch
 * before the decode (the first page's section V3 describes the step).
 *   o         [B,Hq,D] bf16, strides (o_sb, o_sh); written.
 *   q         [B,Hq,D] bf16, strides (q_sb, q_sh); NOT rotated, and left
 *             unrotated (read only).
 *   k_new, v_new  [B,Hkv,D] bf16, strides (n_sb, n_sh) shared by both;
 *             read only.
 *   k_cache, v_cache  [B,Hkv,S_max,D] bf16, strides (kv_sb, kv_sh, kv_ss):
 *             slot seq_lens[b] - 1 of each receives the rotated k_new and
 *             v_new; the other slots are read only.
 *   seq_lens  [B] int32: cache length INCLUDING the new token, whose
 *             position and slot is seq_lens[b] - 1.
 *   base, style  as rgc_rope_apply; max_len, scale, workspace, ws_bytes,
 *             lse as rgc_gqa_attn_decode.
 * o, lse and the caches are bit for bit those of rgc_rope_append (S = 1,
 * pos0 = seq_lens - 1) followed by rgc_gqa_attn_decode of the rotated q; the
 * only difference is that q itself is not rotated in place.  bf16 only
 * (RGC_ERR_DTYPE otherwise).  A sequence whose seq_lens is outside
 * [1, min(max_len, S_max)] gets NaN rows and the flag, and its cache is not
 * written.  Calls that overlap in time must use different workspaces.
 */
int rgc_gqa_attn_decode_rope_append(void* o, const void* q, const void* k_new,
                                    const void* v_new, void* k_cache, void* v_cache,
                                    int dtype, int B, int Hq, int Hkv, int D, int S_max,
                                    int64_t q_sb, int64_t q_sh, int64_t n_sb, int64_t n_sh,
                                    int64_t o_sb, int64_t o_sh, int64_t kv_sb,
                                    int64_t kv_sh, int64_t kv_ss, const int32_t* seq_lens,
                                    int max_len, double base, int style, float scale,
                                    void* workspace, size_t ws_bytes, float* lse,
                                    int32_t* err_flag, void* stream);

/*
 * rgc_gqa_attn_decode_rope_append_static -- rgc_gqa_attn_decode_rope_append
 * without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  The chunk partials go to a device array the library
 * owns, 16 MiB per GPU (each GPU the library runs on holds its copy until
 * the process ends); its address is looked up once per device, on the first
 * call made with that device current.  Nothing is allocated or freed.
 * Arguments, arithmetic and results are those of
 * rgc_gqa_attn_decode_rope_append, bit for bit.  A shape whose partials
 * need more than 16 MiB (rgc_gqa_attn_decode_workspace_size(B, Hq, Hkv, D,
 * max_len) > 16 MiB; at head dim 128 that is about 32,000 (sequence, query
 * head, 128-key chunk) triples) returns RGC_ERR_WORKSPACE and launches
 * nothing.  Every call on one GPU shares its array and leaves its partials
 * there: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be serialised by the caller.  RGC_ERR_HIP when the
 * array's address cannot be obtained.
 */
int rgc_gqa_attn_decode_rope_append_static(void* o, const void* q, const void* k_new,
                                           const void* v_new, void* k_cache, void* v_cache,
                                           int dtype, int B, int Hq, int Hkv, int D, int S_max,
                                           int64_t q_sb, int64_t q_sh, int64_t n_sb, int64_t n_sh,
                                           int64_t o_sb, int64_t o_sh, int64_t kv_sb,
                                           int64_t kv_sh, int64_t kv_ss, const int32_t* seq_lens,
                                           int max_len, double base, int style, float scale,
                                           float* lse, int32_t* err_flag, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RGC_H */
