/*
 * ds_oracle.c -- plain, slow CPU oracle for Double Sparsity decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library and its Python binding) never calls it and shares no code with
 * it: no header, helper, table or constant generator is common to both.
 *
 * Sources (pages cited by title and section):
 *   [DS]    "Double Sparsity" article, joto.ai blog archive 2025060420469:
 *           section "offline calibration" (label cache; 4-bit labels) and
 *           section "online forward computation" (steps 1-3).
 *   [LeanK] LeanK article, aitangshan.cn news 1293675: section 1.1 (channel
 *           importance from the query-key product), section 2.2 (static
 *           hardware-aligned K-channel mask), section 3.2 (kernel speed).
 *   [GQA]   grouped-query attention article, trdm.cn news 80600: section 4
 *           (query heads split into groups sharing one K/V head).
 *
 * Every floating-point step is done in fp64 from fp16 inputs, except the
 * 4-bit quantiser, which is fixed to fp32 IEEE arithmetic because its integer
 * codes must match bit for bit (the pages only say "4 bits"; the procedure
 * below is this implementation's reading of it).
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_NONFINITE (-2)
#define ORC_ERR_NOMEM (-3)

/* ------------------------------------------------------------------------ */
/* IEEE binary16 <-> binary64/32, written from the format definition:        */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.                 */
/* ------------------------------------------------------------------------ */

double oracle_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int f = h & 0x3FF;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* Round a binary32 value to the nearest binary16, ties to even.  All scaling
 * below is by powers of two, so it is exact in fp64, and nearbyint() under the
 * default rounding mode is round-half-even. */
uint16_t oracle_float_to_half_rn(float xf) {
  double x = (double)xf;
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  double a = fabs(x);
  if (isnan(a)) return (uint16_t)0x7E00u;
  if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u); /* halfway to 2^16 rounds up */
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: integer multiples of 2^-24; 1024 lands on 2^-14 */
    double m = nearbyint(ldexp(a, 24));
    return (uint16_t)(sign | (uint16_t)m);
  }
  int e2;
  (void)frexp(a, &e2); /* a in [2^(e2-1), 2^e2) */
  int E = e2 - 1;
  double m = nearbyint(ldexp(a, 10 - E)); /* in [1024, 2048] */
  if (m == 2048.0) {
    m = 1024.0;
    E += 1;
  }
  if (E > 15) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | (uint16_t)(((E + 15) << 10) | ((int)m - 1024)));
}

/* ------------------------------------------------------------------------ */
/* Label cache ([DS] offline calibration: the heavy-channel values of K are   */
/* copied into a contiguous label cache at prefill, and only the new token's */
/* values are added at each decode step).                                   */
/* ------------------------------------------------------------------------ */

/* fp16 label: L[j] = K[chan[j]], a bit copy. */
void oracle_label_f16_row(const uint16_t* krow, const int32_t* chan, int r, uint16_t* out) {
  for (int j = 0; j < r; ++j) out[j] = krow[chan[j]];
}

/* 4-bit label ([DS]: labels tolerate low precision and may be stored in 4
 * bits).  Reading: symmetric codes in [-7, 7] with one fp16 absmax scale per
 * token; scale = fp16_rn(amax / 7); code = clamp(rint_half_even(x / scale));
 * byte j/2 holds code 2i in its low nibble and code 2i+1 in its high nibble,
 * two's complement. */
int oracle_label_int4_row(const uint16_t* krow, const int32_t* chan, int r, uint8_t* codes,
                          uint16_t* scale_out) {
  if (r <= 0 || (r & 1)) return ORC_ERR_ARG;
  float amax = 0.0f;
  for (int j = 0; j < r; ++j) {
    double xd = oracle_half_to_double(krow[chan[j]]);
    if (!isfinite(xd)) return ORC_ERR_NONFINITE;
    float ax = fabsf((float)xd);
    if (ax > amax) amax = ax;
  }
  float ratio = amax / 7.0f; /* IEEE fp32 division */
  uint16_t s16 = oracle_float_to_half_rn(ratio);
  float sf = (float)oracle_half_to_double(s16);
  for (int i = 0; i < r / 2; ++i) {
    int c[2];
    for (int u = 0; u < 2; ++u) {
      float x = (float)oracle_half_to_double(krow[chan[2 * i + u]]);
      int code = 0;
      if (sf != 0.0f) {
        float v = x / sf; /* IEEE fp32 division */
        float rv = nearbyintf(v);
        if (rv > 7.0f) rv = 7.0f;
        if (rv < -7.0f) rv = -7.0f;
        code = (int)rv;
      }
      c[u] = code;
    }
    codes[i] = (uint8_t)((c[0] & 0xF) | ((c[1] & 0xF) << 4));
  }
  *scale_out = s16;
  return ORC_OK;
}

static int nibble_value(uint8_t byte, int hi) {
  int v = hi ? (byte >> 4) & 0xF : byte & 0xF;
  return v >= 8 ? v - 16 : v;
}

/* ------------------------------------------------------------------------ */
/* Step 1 ([DS] online forward, step 1): gather the query at the heavy       */
/* channels into a contiguous vector.  Under GQA ([GQA] section 4) the k     */
/* tokens are shared by the group, and the group's score is read as the sum */
/* of its query heads' approximate scores, i.e. the gathered queries summed. */
/* keep maps a stored K column to its query channel (LeanK compaction,       */
/* [LeanK] section 2.2); NULL is the identity.                               */
/* ------------------------------------------------------------------------ */
void oracle_gather_query(const uint16_t* qg_heads /* [G][d_q] */, int G, int d_q,
                         const int32_t* keep /* [d_k] or NULL */, const int32_t* chan, int r,
                         double* qg /* [r] */) {
  for (int j = 0; j < r; ++j) {
    int col = chan[j];
    int qc = keep ? keep[col] : col;
    double acc = 0.0;
    for (int h = 0; h < G; ++h) acc += oracle_half_to_double(qg_heads[(size_t)h * d_q + qc]);
    qg[j] = acc;
  }
}

/* Step 2 ([DS] online forward, step 2): approximate score of every cached
 * token from the gathered query and the label cache.  Reading: the unscaled
 * dot product (any positive scale or softmax is monotone and leaves the
 * selection unchanged); int4 labels are dequantised as scale * code. */
void oracle_scores_row(const double* qg, int r, int is_int4, const uint16_t* lab_f16 /* [S][r] */,
                       const uint8_t* codes /* [S][r/2] */, const uint16_t* scales /* [S] */,
                       int S, double* s /* [S] */) {
  for (int t = 0; t < S; ++t) {
    double acc = 0.0;
    if (!is_int4) {
      for (int j = 0; j < r; ++j) acc += qg[j] * oracle_half_to_double(lab_f16[(size_t)t * r + j]);
    } else {
      const uint8_t* ct = codes + (size_t)t * (r / 2);
      for (int j = 0; j < r; ++j) acc += qg[j] * (double)nibble_value(ct[j / 2], j & 1);
      acc *= oracle_half_to_double(scales[t]);
    }
    s[t] = acc + 0.0; /* -0 becomes +0 */
  }
}

/* Step 3a ([DS] online forward, step 3): the k tokens with the largest
 * approximate scores, ties broken towards the lower token index.  k <= 0 or
 * k >= S selects every token (the dense fallback of the serving flags).  The
 * set is returned in ascending token order; the return value is its size. */
typedef struct {
  double s;
  int32_t t;
} orc_pair;

static int cmp_desc_score_asc_index(const void* a, const void* b) {
  const orc_pair* x = (const orc_pair*)a;
  const orc_pair* y = (const orc_pair*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->t > y->t) - (x->t < y->t);
}

static int cmp_int32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

int oracle_topk(const double* s, int S, int k, int32_t* idx_out) {
  if (S <= 0) return 0;
  if (k <= 0 || k >= S) {
    for (int t = 0; t < S; ++t) idx_out[t] = t;
    return S;
  }
  orc_pair* p = (orc_pair*)malloc(sizeof(orc_pair) * (size_t)S);
  if (!p) return ORC_ERR_NOMEM;
  for (int t = 0; t < S; ++t) {
    p[t].s = s[t];
    p[t].t = t;
  }
  qsort(p, (size_t)S, sizeof(orc_pair), cmp_desc_score_asc_index);
  for (int i = 0; i < k; ++i) idx_out[i] = p[i].t;
  free(p);
  qsort(idx_out, (size_t)k, sizeof(int32_t), cmp_int32);
  return k;
}

/* Step 3b ([DS] online forward, step 3): exact softmax attention with the
 * full (not channel-sparse) query, K and V over the selected tokens.  Logit
 * l_t = sm_scale * sum_c q[keep[c]] * K[t][c] over the stored K columns (all
 * columns unless LeanK-compacted); o = sum_t e^(l_t - m) V_t / sum_t e^(l_t - m).
 * An empty selection gives a zero output. */
void oracle_attend(const uint16_t* q_heads /* [G][d_q] */, int G, int d_q,
                   const int32_t* keep /* [d_k] or NULL */, const uint16_t* Kb, int64_t k_tok_stride,
                   int d_k, const uint16_t* Vb, int64_t v_tok_stride, int d_v, const int32_t* T,
                   int nT, double sm_scale, double* out /* [G][d_v] */) {
  double* l = (double*)malloc(sizeof(double) * (size_t)(nT > 0 ? nT : 1));
  for (int h = 0; h < G; ++h) {
    const uint16_t* qh = q_heads + (size_t)h * d_q;
    double* oh = out + (size_t)h * d_v;
    for (int c = 0; c < d_v; ++c) oh[c] = 0.0;
    if (nT <= 0) continue;
    double m = -INFINITY;
    for (int i = 0; i < nT; ++i) {
      const uint16_t* kr = Kb + (int64_t)T[i] * k_tok_stride;
      double acc = 0.0;
      for (int c = 0; c < d_k; ++c) {
        int qc = keep ? keep[c] : c;
        acc += oracle_half_to_double(qh[qc]) * oracle_half_to_double(kr[c]);
      }
      l[i] = sm_scale * acc;
      if (l[i] > m) m = l[i];
    }
    double den = 0.0;
    for (int i = 0; i < nT; ++i) {
      double w = exp(l[i] - m);
      den += w;
      const uint16_t* vr = Vb + (int64_t)T[i] * v_tok_stride;
      for (int c = 0; c < d_v; ++c) oh[c] += w * oracle_half_to_double(vr[c]);
    }
    for (int c = 0; c < d_v; ++c) oh[c] /= den;
  }
  free(l);
}

/* ------------------------------------------------------------------------ */
/* Whole tensors.  Layouts (row-major, last index fastest):                 */
/*   K  [B][H_kv][cap][d_k] fp16 with element strides ks[0..2] (channel 1)   */
/*   V  [B][H_kv][cap][d_v] fp16 with element strides vs[0..2]               */
/*   q  [B][H_q][d_q] fp16, query head h belongs to KV head h / G            */
/*   labels fp16 [B][H_kv][slots][r], or int4 codes [B][H_kv][slots][r/2]   */
/*   plus fp16 scales [B][H_kv][slots]                                       */
/* ------------------------------------------------------------------------ */
typedef struct {
  int32_t B, Hq, Hkv, d_q, d_k, d_v, cap;
  int64_t ks[3], vs[3];
  int32_t r, is_int4, slots;
} oracle_shape;

/* Label build over tokens [t_begin, t_end) of every (b, g). */
int oracle_label_build(const oracle_shape* sh, const uint16_t* K, const int32_t* chan /* [Hkv][r] */,
                       uint16_t* lab_f16, uint8_t* codes, uint16_t* scales, int t_begin, int t_end) {
  if (t_begin < 0 || t_end > sh->cap || t_begin > t_end) return ORC_ERR_ARG;
  int rc = ORC_OK;
  for (int b = 0; b < sh->B; ++b)
    for (int g = 0; g < sh->Hkv; ++g)
      for (int t = t_begin; t < t_end; ++t) {
        const uint16_t* kr = K + b * sh->ks[0] + g * sh->ks[1] + (int64_t)t * sh->ks[2];
        size_t row = ((size_t)b * sh->Hkv + g) * (size_t)sh->slots + (size_t)t;
        if (!sh->is_int4) {
          oracle_label_f16_row(kr, chan + (size_t)g * sh->r, sh->r, lab_f16 + row * sh->r);
        } else {
          int e = oracle_label_int4_row(kr, chan + (size_t)g * sh->r, sh->r,
                                        codes + row * (size_t)(sh->r / 2), scales + row);
          if (e) rc = e;
        }
      }
  return rc;
}

/* Label append: tokens pos[b] of every (b, g); rows with pos out of range are
 * left untouched. */
int oracle_label_append(const oracle_shape* sh, const uint16_t* K, const int32_t* chan,
                        uint16_t* lab_f16, uint8_t* codes, uint16_t* scales, const int32_t* pos) {
  int rc = ORC_OK;
  for (int b = 0; b < sh->B; ++b) {
    int t = pos[b];
    if (t < 0 || t >= sh->cap) continue;
    for (int g = 0; g < sh->Hkv; ++g) {
      const uint16_t* kr = K + b * sh->ks[0] + g * sh->ks[1] + (int64_t)t * sh->ks[2];
      size_t row = ((size_t)b * sh->Hkv + g) * (size_t)sh->slots + (size_t)t;
      if (!sh->is_int4) {
        oracle_label_f16_row(kr, chan + (size_t)g * sh->r, sh->r, lab_f16 + row * sh->r);
      } else {
        int e = oracle_label_int4_row(kr, chan + (size_t)g * sh->r, sh->r,
                                      codes + row * (size_t)(sh->r / 2), scales + row);
        if (e) rc = e;
      }
    }
  }
  return rc;
}

/* One decode step for the (b, g) rows listed in rows[0..n_rows) (pairs b, g).
 * Outputs (only the listed rows are written):
 *   out     [B][H_q][d_v] fp64
 *   topk    [B][H_kv][k_cap] int32, ascending, -1 padded (may be NULL)
 *   scores  [B][H_kv][score_stride] fp64 (may be NULL)
 * With k <= 0 no label is read and every token is attended.  seq_lens[b] is
 * the number of cached tokens, the current one included. */
int oracle_decode(const oracle_shape* sh, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                  const int32_t* seq_lens, const int32_t* keep /* [Hkv][d_k] or NULL */,
                  const int32_t* chan, const uint16_t* lab_f16, const uint8_t* codes,
                  const uint16_t* scales, int k, double sm_scale, const int32_t* rows, int n_rows,
                  double* out, int32_t* topk, int k_cap, double* scores, int64_t score_stride,
                  int n_threads) {
  if (sh->Hq % sh->Hkv) return ORC_ERR_ARG;
  int G = sh->Hq / sh->Hkv;
  int rc = ORC_OK;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int i = 0; i < n_rows; ++i) {
    int b = rows[2 * i], g = rows[2 * i + 1];
    int S = seq_lens[b];
    if (S < 0) S = 0;
    if (S > sh->cap) S = sh->cap;
    const uint16_t* qh = q + ((size_t)b * sh->Hq + (size_t)g * G) * sh->d_q;
    const int32_t* kp = keep ? keep + (size_t)g * sh->d_k : NULL;
    const uint16_t* Kb = K + b * sh->ks[0] + g * sh->ks[1];
    const uint16_t* Vb = V + b * sh->vs[0] + g * sh->vs[1];
    int32_t* T = (int32_t*)malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
    double* s = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    if (!T || !s) {
      rc = ORC_ERR_NOMEM;
      free(T);
      free(s);
      continue;
    }
    int nT;
    if (k <= 0 || k >= S) {
      nT = S;
      for (int t = 0; t < S; ++t) T[t] = t;
      if (k > 0 && scores) {
        /* scores are still reported for parity checks */
        double* qgv = (double*)malloc(sizeof(double) * (size_t)sh->r);
        oracle_gather_query(qh, G, sh->d_q, kp, chan + (size_t)g * sh->r, sh->r, qgv);
        size_t row = ((size_t)b * sh->Hkv + g) * (size_t)sh->slots;
        oracle_scores_row(qgv, sh->r, sh->is_int4, lab_f16 ? lab_f16 + row * sh->r : NULL,
                          codes ? codes + row * (size_t)(sh->r / 2) : NULL,
                          scales ? scales + row : NULL, S, s);
        free(qgv);
      }
    } else {
      double* qgv = (double*)malloc(sizeof(double) * (size_t)sh->r);
      oracle_gather_query(qh, G, sh->d_q, kp, chan + (size_t)g * sh->r, sh->r, qgv);
      size_t row = ((size_t)b * sh->Hkv + g) * (size_t)sh->slots;
      oracle_scores_row(qgv, sh->r, sh->is_int4, lab_f16 ? lab_f16 + row * sh->r : NULL,
                        codes ? codes + row * (size_t)(sh->r / 2) : NULL,
                        scales ? scales + row : NULL, S, s);
      free(qgv);
      nT = oracle_topk(s, S, k, T);
    }
    if (scores && k > 0) {
      double* dst = scores + ((size_t)b * sh->Hkv + g) * (size_t)score_stride;
      for (int t = 0; t < S; ++t) dst[t] = s[t];
    }
    if (topk) {
      int32_t* dst = topk + ((size_t)b * sh->Hkv + g) * (size_t)k_cap;
      for (int j = 0; j < k_cap; ++j) dst[j] = j < nT ? T[j] : -1;
    }
    oracle_attend(qh, G, sh->d_q, kp, Kb, sh->ks[2], sh->d_k, Vb, sh->vs[2], sh->d_v, T,
                  nT < 0 ? 0 : nT, sm_scale, out + ((size_t)b * sh->Hq + (size_t)g * G) * sh->d_v);
    free(T);
    free(s);
  }
  return rc;
}

/* Attention only, over a caller-given token set per (b, g) row (used to
 * re-check an output against another implementation's selection).
 * sets [B][H_kv][k_cap] int32, entries < 0 ignored. */
int oracle_attend_sets(const oracle_shape* sh, const uint16_t* q, const uint16_t* K,
                       const uint16_t* V, const int32_t* keep, const int32_t* sets, int k_cap,
                       double sm_scale, const int32_t* rows, int n_rows, double* out, int n_threads) {
  if (sh->Hq % sh->Hkv) return ORC_ERR_ARG;
  int G = sh->Hq / sh->Hkv;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int i = 0; i < n_rows; ++i) {
    int b = rows[2 * i], g = rows[2 * i + 1];
    const int32_t* src = sets + ((size_t)b * sh->Hkv + g) * (size_t)k_cap;
    int32_t* T = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k_cap > 0 ? k_cap : 1));
    int nT = 0;
    for (int j = 0; j < k_cap; ++j)
      if (src[j] >= 0 && src[j] < sh->cap) T[nT++] = src[j];
    const uint16_t* qh = q + ((size_t)b * sh->Hq + (size_t)g * G) * sh->d_q;
    oracle_attend(qh, G, sh->d_q, keep ? keep + (size_t)g * sh->d_k : NULL,
                  K + b * sh->ks[0] + g * sh->ks[1], sh->ks[2], sh->d_k,
                  V + b * sh->vs[0] + g * sh->vs[1], sh->vs[2], sh->d_v, T, nT, sm_scale,
                  out + ((size_t)b * sh->Hq + (size_t)g * G) * sh->d_v);
    free(T);
  }
  return ORC_OK;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Offline heavy-channel calibration ([DS] "offline calibration": the        */
/* channels that move the attention scores most are found once, from a few  */
/* sample tokens, by one of the K-, Q- or QK-outlier criteria; [LeanK]       */
/* section 1.1: the importance of channel i is the L2 norm of Q[i] K[i]^T,   */
/* Q the queries of an observation window, K the whole key matrix).          */
/* ------------------------------------------------------------------------ */

/* Agreement of two heavy-channel tables ([DS] "offline calibration": the
 * outlier channels found offline against those found online, whose overlap
 * the article reports): for every KV head g, the number of distinct channels
 * of a[g] that also occur in b[g], divided by r.  a, b: [Hkv][r].
 * Returns ORC_OK or ORC_ERR_ARG. */
int oracle_channel_overlap(const int32_t* a, const int32_t* b, int Hkv, int r, double* out) {
  if (!a || !b || !out || Hkv < 1 || r < 1) return ORC_ERR_ARG;
  for (int g = 0; g < Hkv; ++g) {
    const int32_t* ag = a + (int64_t)g * r;
    const int32_t* bg = b + (int64_t)g * r;
    int shared = 0;
    for (int i = 0; i < r; ++i) {
      int seen = 0, found = 0;
      for (int j = 0; j < i; ++j) seen |= ag[j] == ag[i];
      for (int j = 0; j < r; ++j) found |= bg[j] == ag[i];
      if (!seen && found) ++shared;
    }
    out[g] = (double)shared / (double)r;
  }
  return ORC_OK;
}

/* For KV head g and stored K column c (query channel qc = keep[g][c], or c):
 *   kn_b = sum_{t < n_tok} K[b][g][t][c]^2                 (sample b's K column)
 *   qn_b = sum_{w < n_win} sum_{h in group g} q[b][w][h][qc]^2
 *   K-outlier  (criterion 0): score = sum_b kn_b
 *   Q-outlier  (criterion 1): score = sum_b qn_b
 *   QK-outlier (criterion 2): score = sqrt(sum_b qn_b * kn_b), the Frobenius
 *     norm of the per-sample products Q_b[c] K_b[c]^T (column c of the
 *     window's query rows times column c of K; a rank-one matrix, whose norm
 *     is the product of the two column norms), taken together over samples.
 * chan[g] = the r columns with the largest score, ties to the lower column,
 * listed in ascending column order.  norms (optional): [Hkv][3][d_k] holding
 * sum_b kn_b, sum_b qn_b and the criterion's score.
 * K: fp16 bits with element strides ks = {batch, head, token}, unit channel
 * stride; qwin: fp16 bits [B][n_win][Hq][d_q]; keep: [Hkv][d_k] or NULL.
 * Returns ORC_OK, ORC_ERR_ARG or ORC_ERR_NONFINITE (a non-finite input). */
int oracle_calibrate(const uint16_t* K, const int64_t* ks, int B, int Hkv, int d_k, int n_tok,
                     const uint16_t* qwin, int n_win, int Hq, int d_q, const int32_t* keep,
                     int criterion, int r, int32_t* chan, double* norms) {
  if (B < 1 || Hkv < 1 || d_k < 1 || n_tok < 0 || n_win < 0 || r < 1 || r > d_k || !chan)
    return ORC_ERR_ARG;
  if (criterion < 0 || criterion > 2) return ORC_ERR_ARG;
  if (n_win > 0 && (!qwin || Hq < Hkv || Hq % Hkv || d_q < 1)) return ORC_ERR_ARG;
  if (n_tok > 0 && !K) return ORC_ERR_ARG;
  const int G = n_win > 0 ? Hq / Hkv : 1;
  orc_pair* p = (orc_pair*)malloc(sizeof(orc_pair) * (size_t)d_k);
  int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)r);
  if (!p || !sel) {
    free(p);
    free(sel);
    return ORC_ERR_NOMEM;
  }
  int rc = ORC_OK;
  for (int g = 0; g < Hkv && rc == ORC_OK; ++g) {
    for (int c = 0; c < d_k; ++c) {
      const int qc = keep ? keep[(size_t)g * d_k + c] : c;
      if (n_win > 0 && (qc < 0 || qc >= d_q)) {
        rc = ORC_ERR_ARG;
        break;
      }
      double kn = 0.0, qn = 0.0, qk = 0.0;
      for (int b = 0; b < B; ++b) {
        double knb = 0.0, qnb = 0.0;
        for (int t = 0; t < n_tok; ++t) {
          const double x = oracle_half_to_double(K[b * ks[0] + g * ks[1] + t * ks[2] + c]);
          knb += x * x;
        }
        for (int w = 0; w < n_win; ++w)
          for (int h = 0; h < G; ++h) {
            const double x = oracle_half_to_double(
                qwin[(((size_t)b * n_win + w) * Hq + (size_t)g * G + h) * d_q + qc]);
            qnb += x * x;
          }
        kn += knb;
        qn += qnb;
        qk += qnb * knb;
      }
      if (!isfinite(kn) || !isfinite(qn) || !isfinite(qk)) {
        rc = ORC_ERR_NONFINITE;
        break;
      }
      const double s = criterion == 0 ? kn : criterion == 1 ? qn : sqrt(qk);
      p[c].s = s;
      p[c].t = c;
      if (norms) {
        double* nd = norms + (size_t)g * 3 * d_k;
        nd[c] = kn;
        nd[d_k + c] = qn;
        nd[2 * d_k + c] = s;
      }
    }
    if (rc != ORC_OK) break;
    qsort(p, (size_t)d_k, sizeof(orc_pair), cmp_desc_score_asc_index);
    for (int j = 0; j < r; ++j) sel[j] = p[j].t;
    qsort(sel, (size_t)r, sizeof(int32_t), cmp_int32);
    memcpy(chan + (size_t)g * r, sel, sizeof(int32_t) * (size_t)r);
  }
  free(p);
  free(sel);
  return rc;
}
