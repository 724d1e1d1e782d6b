/*
 * orc.c -- fp64 CPU oracle (test infrastructure; see orc.h for the sources
 * and the readings).  Plain C11 + libm + OpenMP, built without fast-math so
 * that every sum runs in the order written here.
 */
#include "orc.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* ---- storage types ------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32; widening is a 16-bit shift. */
static double bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double load(const void* base, int dt, int64_t i) {
  if (dt == ORC_F32) return (double)((const float*)base)[i];
  return bf16_to_f64(((const uint16_t*)base)[i]);
}

/*
 * Nearest bfloat16 to x, ties to even, in one rounding step from the double.
 * bf16 keeps 8 significant bits and the binary32 exponent range, so the
 * quantum at |x| in [2^e, 2^(e+1)) is 2^(e-7), and 2^-133 below 2^-126.
 */
uint16_t orc_bf16_bits(double x) {
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
  if (isinf(x)) return (uint16_t)(sign | 0x7F80u);
  if (x == 0.0) return sign;
  int e = ilogb(x);
  if (e < -126) e = -126;
  double quantum = ldexp(1.0, e - 7);
  double r = rint(x / quantum) * quantum; /* default mode: ties to even */
  const double bf16_max = 3.3895313892515355e38; /* (2 - 2^-7) * 2^127 */
  if (fabs(r) > bf16_max) return (uint16_t)(sign | 0x7F80u);
  float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

static void store(void* base, int dt, int64_t i, double v) {
  if (dt == ORC_F32)
    ((float*)base)[i] = (float)v; /* C conversion: nearest, ties to even */
  else
    ((uint16_t*)base)[i] = orc_bf16_bits(v);
}

static int dtype_ok(int dt) { return dt == ORC_F32 || dt == ORC_BF16; }

/* ---- RoPE ---------------------------------------------------------------- */

/*
 * Rotation of one head vector at position pos ([P1] V1, [P2] core
 * architecture): pair i is (x_i, x_{i+D/2}) for the half style and
 * (x_{2i}, x_{2i+1}) for the interleaved style; each pair (a, b) turns by the
 * angle pos * theta_i with theta_i = base^(-2i/D):
 *   a' = a cos - b sin,   b' = a sin + b cos.
 */
static void rope_vec(double* out, const void* x, int dt, int64_t off, int D,
                     double pos, double base, int style) {
  int half = D / 2;
  for (int i = 0; i < half; ++i) {
    double theta = pow(base, -2.0 * (double)i / (double)D);
    double ang = pos * theta;
    double c = cos(ang), s = sin(ang);
    int ia = (style == ORC_ROPE_HALF) ? i : 2 * i;
    int ib = (style == ORC_ROPE_HALF) ? i + half : 2 * i + 1;
    double a = load(x, dt, off + ia);
    double b = load(x, dt, off + ib);
    out[ia] = a * c - b * s;
    out[ib] = a * s + b * c;
  }
}

static int rope_args_ok(int dt, int B, int S, int H, int D, int style) {
  if (!dtype_ok(dt) || B < 0 || S < 0 || H < 0) return 0;
  if (D <= 0 || (D % 2) != 0) return 0;
  return style == ORC_ROPE_HALF || style == ORC_ROPE_INTERLEAVED;
}

int orc_rope_f64(double* out, const void* x, int dt, int B, int S, int H,
                 int D, int64_t sb, int64_t ss, int64_t sh,
                 const int32_t* pos0, double base, int style) {
  if (!rope_args_ok(dt, B, S, H, D, style)) return ORC_ERR_ARG;
  for (int b = 0; b < B; ++b)
    for (int s = 0; s < S; ++s) {
      double pos = (double)((pos0 ? pos0[b] : 0) + s);
      for (int h = 0; h < H; ++h) {
        int64_t off = (int64_t)b * sb + (int64_t)s * ss + (int64_t)h * sh;
        double* dst = out + (((int64_t)b * S + s) * H + h) * D;
        rope_vec(dst, x, dt, off, D, pos, base, style);
      }
    }
  return ORC_OK;
}

int orc_rope_apply(void* x, int dt, int B, int S, int H, int D, int64_t sb,
                   int64_t ss, int64_t sh, const int32_t* pos0, double base,
                   int style) {
  if (!rope_args_ok(dt, B, S, H, D, style)) return ORC_ERR_ARG;
  double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
  if (!tmp) return ORC_ERR_ARG;
  for (int b = 0; b < B; ++b)
    for (int s = 0; s < S; ++s) {
      double pos = (double)((pos0 ? pos0[b] : 0) + s);
      for (int h = 0; h < H; ++h) {
        int64_t off = (int64_t)b * sb + (int64_t)s * ss + (int64_t)h * sh;
        rope_vec(tmp, x, dt, off, D, pos, base, style);
        for (int d = 0; d < D; ++d) store(x, dt, off + d, tmp[d]);
      }
    }
  free(tmp);
  return ORC_OK;
}

/*
 * Gradient through RoPE: the rotation is orthogonal, so the gradient with
 * respect to the unrotated vector is the output gradient turned back by the
 * same angle: (ga, gb) -> (ga cos + gb sin, -ga sin + gb cos).
 */
int orc_rope_grad_f64(double* out, const void* g, int dt, int B, int S, int H,
                      int D, int64_t sb, int64_t ss, int64_t sh,
                      const int32_t* pos0, double base, int style) {
  if (!rope_args_ok(dt, B, S, H, D, style)) return ORC_ERR_ARG;
  int half = D / 2;
  for (int b = 0; b < B; ++b)
    for (int s = 0; s < S; ++s) {
      double pos = (double)((pos0 ? pos0[b] : 0) + s);
      for (int h = 0; h < H; ++h) {
        int64_t off = (int64_t)b * sb + (int64_t)s * ss + (int64_t)h * sh;
        double* dst = out + (((int64_t)b * S + s) * H + h) * D;
        for (int i = 0; i < half; ++i) {
          double theta = pow(base, -2.0 * (double)i / (double)D);
          double c = cos(pos * theta), sn = sin(pos * theta);
          int ia = (style == ORC_ROPE_HALF) ? i : 2 * i;
          int ib = (style == ORC_ROPE_HALF) ? i + half : 2 * i + 1;
          double ga = load(g, dt, off + ia), gb = load(g, dt, off + ib);
          dst[ia] = ga * c + gb * sn;
          dst[ib] = -ga * sn + gb * c;
        }
      }
    }
  return ORC_OK;
}

/* ---- QK normalisation before RoPE ----------------------------------------- */

/*
 * RMS normalisation of one head vector ([P2] core architecture: RMSNorm
 * replaces LayerNorm; [P3] 设置: the model normalises q and k): the vector is
 * divided by the root of the mean of its squares plus eps.  No learned weight
 * (the pages print none).  Then the rotation of rope_vec, on the normalised
 * values.
 */
static void norm_rope_vec(double* out, double* y, const void* x, int dt, int64_t off, int D,
                          double pos, double base, int style, double eps) {
  double ss = 0.0;
  for (int d = 0; d < D; ++d) {
    double v = load(x, dt, off + d);
    y[d] = v;
    ss += v * v;
  }
  double r = 1.0 / sqrt(ss / (double)D + eps);
  for (int d = 0; d < D; ++d) y[d] *= r;
  int half = D / 2;
  for (int i = 0; i < half; ++i) {
    double theta = pow(base, -2.0 * (double)i / (double)D);
    double ang = pos * theta;
    double c = cos(ang), s = sin(ang);
    int ia = (style == ORC_ROPE_HALF) ? i : 2 * i;
    int ib = (style == ORC_ROPE_HALF) ? i + half : 2 * i + 1;
    double a = y[ia], b = y[ib];
    out[ia] = a * c - b * s;
    out[ib] = a * s + b * c;
  }
}

int orc_norm_rope_f64(double* out, const void* x, int dt, int B, int S, int H,
                      int D, int64_t sb, int64_t ss, int64_t sh,
                      const int32_t* pos0, double base, int style, double eps) {
  if (!rope_args_ok(dt, B, S, H, D, style) || !(eps >= 0.0)) return ORC_ERR_ARG;
  double* y = (double*)malloc(sizeof(double) * (size_t)D);
  if (!y) return ORC_ERR_ARG;
  for (int b = 0; b < B; ++b)
    for (int s = 0; s < S; ++s) {
      double pos = (double)((pos0 ? pos0[b] : 0) + s);
      for (int h = 0; h < H; ++h) {
        int64_t off = (int64_t)b * sb + (int64_t)s * ss + (int64_t)h * sh;
        double* dst = out + (((int64_t)b * S + s) * H + h) * D;
        norm_rope_vec(dst, y, x, dt, off, D, pos, base, style, eps);
      }
    }
  free(y);
  return ORC_OK;
}

/* ---- cache append -------------------------------------------------------- */

/* [P1] V3 and [P2]: the cache keeps every step's K and V rows in order. */
int orc_kv_cache_append(void* k_cache, void* v_cache, int dt, int B, int Hkv,
                        int D, int S_max, int64_t c_sb, int64_t c_sh,
                        int64_t c_ss, const void* k_new, const void* v_new,
                        int S_new, int64_t sb, int64_t ss, int64_t sh,
                        const int32_t* pos0) {
  if (!dtype_ok(dt) || B < 0 || Hkv < 0 || D <= 0 || S_new < 0 || S_max < 0)
    return ORC_ERR_ARG;
  size_t esz = (dt == ORC_F32) ? 4 : 2;
  int status = ORC_OK;
  for (int b = 0; b < B; ++b)
    for (int s = 0; s < S_new; ++s) {
      int64_t slot = (int64_t)(pos0 ? pos0[b] : 0) + s;
      if (slot < 0 || slot >= S_max) {
        status = ORC_ERR_CAPACITY;
        continue;
      }
      for (int h = 0; h < Hkv; ++h) {
        int64_t src = (int64_t)b * sb + (int64_t)s * ss + (int64_t)h * sh;
        int64_t dst = (int64_t)b * c_sb + (int64_t)h * c_sh + slot * c_ss;
        memcpy((char*)k_cache + dst * esz, (const char*)k_new + src * esz,
               esz * (size_t)D);
        memcpy((char*)v_cache + dst * esz, (const char*)v_new + src * esz,
               esz * (size_t)D);
      }
    }
  return status;
}

/* ---- attention ----------------------------------------------------------- */

/*
 * Softmax weights of one causal row, two passes: z_j = scale * <q, K_j> for
 * j = 0..p, m = max z, w_j = exp(z_j - m).  Returns the denominator
 * l = sum_j w_j (ascending j) and the maximum through *m_out.
 */
static double row_weights(double* w, const void* q, int64_t q_off,
                          const void* kc, int64_t k_off, int64_t kv_ss,
                          int dt, int D, int p, double scale, double* m_out) {
  double m = -INFINITY;
  for (int j = 0; j <= p; ++j) {
    double dot = 0.0;
    int64_t kr = k_off + (int64_t)j * kv_ss;
    for (int d = 0; d < D; ++d) dot += load(q, dt, q_off + d) * load(kc, dt, kr + d);
    w[j] = scale * dot;
    if (w[j] > m) m = w[j];
  }
  double l = 0.0;
  for (int j = 0; j <= p; ++j) {
    w[j] = exp(w[j] - m);
    l += w[j];
  }
  *m_out = m;
  return l;
}

/* o[d] = sum_j w_j V_j[d] / l, ascending j. */
static void row_output(double* o, const double* w, double l, const void* vc,
                       int64_t v_off, int64_t v_ss, int dt, int Dv, int p,
                       double coef) {
  for (int d = 0; d < Dv; ++d) {
    double acc = 0.0;
    for (int j = 0; j <= p; ++j)
      acc += w[j] * load(vc, dt, v_off + (int64_t)j * v_ss + d);
    o[d] += coef * acc / l;
  }
}

static int attn_args_ok(int dt, int B, int Sq, int Hq, int Hkv, int D,
                        int S_max) {
  if (!dtype_ok(dt) || B < 0 || Sq < 0 || D <= 0 || S_max < 0) return 0;
  return Hq > 0 && Hkv > 0;
}

int orc_attn(double* o, double* lse, const void* q, const void* k_cache,
             const void* v_cache, int dt, int B, int Sq, int Hq, int Hkv,
             int D, int S_max, int64_t q_sb, int64_t q_ss, int64_t q_sh,
             int64_t kv_sb, int64_t kv_sh, int64_t kv_ss,
             const int32_t* q_start, double scale, int nthreads) {
  if (!attn_args_ok(dt, B, Sq, Hq, Hkv, D, S_max)) return ORC_ERR_ARG;
  if (Hq % Hkv != 0) return ORC_ERR_GROUP; /* [P1] lesson 4 */
  for (int b = 0; b < B; ++b) {
    int64_t first = q_start ? q_start[b] : 0;
    if (Sq > 0 && (first < 0 || first + Sq > S_max)) return ORC_ERR_CAPACITY;
  }
  const int group = Hq / Hkv;
  const int64_t rows = (int64_t)B * Hq * Sq;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)(S_max > 0 ? S_max : 1));
#pragma omp for schedule(dynamic, 8)
    for (int64_t r = 0; r < rows; ++r) {
      int s = (int)(r % Sq);
      int h = (int)((r / Sq) % Hq);
      int b = (int)(r / ((int64_t)Sq * Hq));
      int kvh = h / group; /* contiguous groups ([P1] V2, [P2]) */
      int p = (q_start ? q_start[b] : 0) + s;
      int64_t q_off = (int64_t)b * q_sb + (int64_t)s * q_ss + (int64_t)h * q_sh;
      int64_t kv_off = (int64_t)b * kv_sb + (int64_t)kvh * kv_sh;
      double m;
      double l = row_weights(w, q, q_off, k_cache, kv_off, kv_ss, dt, D, p,
                             scale, &m);
      double* orow = o + (((int64_t)b * Sq + s) * Hq + h) * D;
      for (int d = 0; d < D; ++d) orow[d] = 0.0;
      row_output(orow, w, l, v_cache, kv_off, kv_ss, dt, D, p, 1.0);
      if (lse) lse[((int64_t)b * Hq + h) * Sq + s] = m + log(l);
    }
    free(w);
  }
  return ORC_OK;
}

/*
 * Gradients of causal GQA self-attention (the training pass: the pages train
 * the 24 q / 8 KV model of [P3] 设置 end to end).  For row i of query head h
 * (keys j <= i of the same sequence, KV head h / group) with softmax weights
 * w_ij, and the output gradient dO_i:
 *   dV_j += w_ij dO_i              (summed over the group's query heads)
 *   dP_ij = dO_i . V_j,   Dlt_i = sum_j w_ij dP_ij
 *   dS_ij = w_ij (dP_ij - Dlt_i)
 *   dQ_i  = scale sum_j dS_ij K_j
 *   dK_j += scale dS_ij Q_i        (summed over the group's query heads)
 * q and dO share one layout [B,S,Hq,D]; k and v [B,S,Hkv,D].  dq, dk, dv are
 * contiguous doubles of the same shapes.  OpenMP over (sequence, KV head)
 * units, so each dk/dv row is written by one thread.
 */
int orc_attn_backward(double* dq, double* dk, double* dv, const void* q,
                      const void* k, const void* v, const void* dO, int dt,
                      int B, int S, int Hq, int Hkv, int D, int64_t q_sb,
                      int64_t q_ss, int64_t q_sh, int64_t kv_sb, int64_t kv_ss,
                      int64_t kv_sh, double scale, int nthreads) {
  if (!attn_args_ok(dt, B, S, Hq, Hkv, D, S)) return ORC_ERR_ARG;
  if (Hq % Hkv != 0) return ORC_ERR_GROUP;
  const int group = Hq / Hkv;
  const int64_t units = (int64_t)B * Hkv;
  if (nthreads < 1) nthreads = 1;
  for (int64_t i = 0; i < (int64_t)B * S * Hkv * D; ++i) dk[i] = dv[i] = 0.0;
#pragma omp parallel num_threads(nthreads)
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    double* dp = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
      int b = (int)(u / Hkv), kvh = (int)(u % Hkv);
      int64_t kv_off = (int64_t)b * kv_sb + (int64_t)kvh * kv_sh;
      for (int hh = 0; hh < group; ++hh) {
        int h = kvh * group + hh;
        for (int i = 0; i < S; ++i) {
          int64_t q_off = (int64_t)b * q_sb + (int64_t)i * q_ss + (int64_t)h * q_sh;
          double m;
          double l = row_weights(w, q, q_off, k, kv_off, kv_ss, dt, D, i, scale, &m);
          double dlt = 0.0;
          for (int j = 0; j <= i; ++j) {
            w[j] /= l;
            double acc = 0.0;
            int64_t vr = kv_off + (int64_t)j * kv_ss;
            for (int d = 0; d < D; ++d) acc += load(dO, dt, q_off + d) * load(v, dt, vr + d);
            dp[j] = acc;
            dlt += w[j] * acc;
          }
          double* dqr = dq + (((int64_t)b * S + i) * Hq + h) * D;
          for (int d = 0; d < D; ++d) dqr[d] = 0.0;
          for (int j = 0; j <= i; ++j) {
            double ds = w[j] * (dp[j] - dlt);
            int64_t kr = kv_off + (int64_t)j * kv_ss;
            double* dkr = dk + (((int64_t)b * S + j) * Hkv + kvh) * D;
            double* dvr = dv + (((int64_t)b * S + j) * Hkv + kvh) * D;
            for (int d = 0; d < D; ++d) {
              dqr[d] += scale * ds * load(k, dt, kr + d);
              dkr[d] += scale * ds * load(q, dt, q_off + d);
              dvr[d] += w[j] * load(dO, dt, q_off + d);
            }
          }
        }
      }
    }
    free(w);
    free(dp);
  }
  return ORC_OK;
}

/*
 * Cached decode ([P1] V3, [P2]): the newest token is the last cache row, so
 * decode is the causal row at slot seq_lens[b] - 1.
 */
int orc_attn_decode(double* o, double* lse, const void* q,
                    const void* k_cache, const void* v_cache, int dt, int B,
                    int Hq, int Hkv, int D, int S_max, int64_t q_sb,
                    int64_t q_sh, int64_t kv_sb, int64_t kv_sh, int64_t kv_ss,
                    const int32_t* seq_lens, double scale, int nthreads) {
  if (!attn_args_ok(dt, B, 1, Hq, Hkv, D, S_max) || !seq_lens) return ORC_ERR_ARG;
  if (Hq % Hkv != 0) return ORC_ERR_GROUP;
  int32_t* start = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B > 0 ? B : 1));
  if (!start) return ORC_ERR_ARG;
  int status = ORC_OK;
  for (int b = 0; b < B; ++b) {
    if (seq_lens[b] < 1 || seq_lens[b] > S_max) status = ORC_ERR_CAPACITY;
    start[b] = seq_lens[b] - 1;
  }
  if (status == ORC_OK)
    status = orc_attn(o, lse, q, k_cache, v_cache, dt, B, 1, Hq, Hkv, D,
                      S_max, q_sb, 0, q_sh, kv_sb, kv_sh, kv_ss, start, scale,
                      nthreads);
  free(start);
  return status;
}

/*
 * Differential attention ([P1] V2): the first map minus lambda times the
 * second, both causal softmaxes over keys 0..p, applied to one V.
 */
int orc_diff_attn(double* o, const void* q1, const void* q2, const void* k1,
                  const void* k2, const void* v, int dt, int B, int S, int Hq,
                  int Hkv, int D, int Dv, int S_max, int64_t q_sb,
                  int64_t q_ss, int64_t q_sh, int64_t kv_sb, int64_t kv_sh,
                  int64_t kv_ss, int64_t v_sb, int64_t v_sh, int64_t v_ss,
                  const int32_t* q_start, double lambda, double scale,
                  int nthreads) {
  if (!attn_args_ok(dt, B, S, Hq, Hkv, D, S_max) || Dv <= 0) return ORC_ERR_ARG;
  if (Hq % Hkv != 0) return ORC_ERR_GROUP;
  for (int b = 0; b < B; ++b) {
    int64_t first = q_start ? q_start[b] : 0;
    if (S > 0 && (first < 0 || first + S > S_max)) return ORC_ERR_CAPACITY;
  }
  const int group = Hq / Hkv;
  const int64_t rows = (int64_t)B * Hq * S;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
  {
    size_t n = (size_t)(S_max > 0 ? S_max : 1);
    double* w1 = (double*)malloc(sizeof(double) * n);
    double* w2 = (double*)malloc(sizeof(double) * n);
#pragma omp for schedule(dynamic, 8)
    for (int64_t r = 0; r < rows; ++r) {
      int s = (int)(r % S);
      int h = (int)((r / S) % Hq);
      int b = (int)(r / ((int64_t)S * Hq));
      int kvh = h / group;
      int p = (q_start ? q_start[b] : 0) + s;
      int64_t q_off = (int64_t)b * q_sb + (int64_t)s * q_ss + (int64_t)h * q_sh;
      int64_t k_off = (int64_t)b * kv_sb + (int64_t)kvh * kv_sh;
      int64_t v_off = (int64_t)b * v_sb + (int64_t)kvh * v_sh;
      double m1, m2;
      double l1 = row_weights(w1, q1, q_off, k1, k_off, kv_ss, dt, D, p, scale, &m1);
      double l2 = row_weights(w2, q2, q_off, k2, k_off, kv_ss, dt, D, p, scale, &m2);
      double* orow = o + (((int64_t)b * S + s) * Hq + h) * Dv;
      for (int d = 0; d < Dv; ++d) orow[d] = 0.0;
      row_output(orow, w1, l1, v, v_off, v_ss, dt, Dv, p, 1.0);
      row_output(orow, w2, l2, v, v_off, v_ss, dt, Dv, p, -lambda);
    }
    free(w1);
    free(w2);
  }
  return ORC_OK;
}
