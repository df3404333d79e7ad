/*
 * tq_oracle.c -- CPU oracle (TEST INFRASTRUCTURE; see tq_oracle.h for who may use it).
 *
 * Plain scalar C, fp64 arithmetic, sums in ascending index order. Rows (and tokens) are spread
 * over OpenMP threads; no sum is split, blocked or reordered.
 *
 * Block formats. The pages name Q4_K, Q6_K and Q8_0 as the quantization formats of the GGUF
 * files these engines load ("Titan Engine" page, sections "Aggressive quantization" and "Model
 * format support"; "Show HN: Llama 3.1 70B on a single RTX 3090 ..." page, section
 * "Quantization support"; KTransformers page, table of supported models and quantizations).
 * They print no bit layout. The oracle reads each name as the public GGUF block layout of that
 * name, with all multi-byte fields little-endian:
 *
 *   Q4_K, 256 weights in 144 bytes: [0,2) d fp16, [2,4) dmin fp16, [4,16) twelve bytes S holding
 *     eight 6-bit scales sc_j and eight 6-bit mins m_j, [16,144) 128 bytes qs of 4-bit quants.
 *     Weight i lies in sub-block j = i/32. With c = i/64 and r = i%64 its quant is the low
 *     nibble of qs[32c + r] when r < 32 and the high nibble of qs[32c + r - 32] otherwise.
 *     For j < 4: sc_j = S[j] & 63, m_j = S[j+4] & 63. For j >= 4: sc_j = (S[j+4] & 15) |
 *     ((S[j-4] >> 6) << 4) and m_j = (S[j+4] >> 4) | ((S[j] >> 6) << 4).
 *     Value: w = d*sc_j*q - dmin*m_j.
 *   Q6_K, 256 weights in 210 bytes: [0,128) ql low 4 bits, [128,192) qh high 2 bits, [192,208)
 *     sixteen int8 scales, [208,210) d fp16. With h = i/128, r = i%128, g = r/32, l = r%32:
 *     low4 = nibble (low if g < 2, high otherwise) of ql[64h + l + 32*(g%2)], high2 = bits
 *     2g..2g+1 of qh[32h + l], q = low4 + 16*high2 in 0..63. Value: w = d*sc[i/16]*(q - 32).
 *   Q8_0, 32 weights in 34 bytes: [0,2) d fp16, [2,34) int8 q. Value: w = d*q.
 *   Q5_K, 256 weights in 176 bytes: [0,2) d fp16, [2,4) dmin fp16, [4,16) the twelve scale/min
 *     bytes S of Q4_K, [16,48) 32 bytes qh of high bits, [48,176) 128 bytes qs of low 4 bits
 *     laid out as Q4_K's quants. Weight i (sub-block j = i/32, position l = i%32) has low4 from
 *     qs as in Q4_K and its fifth bit in bit j of qh[l]: q = low4 + 16*((qh[l] >> j) & 1), 0..31.
 *     Value: w = d*sc_j*q - dmin*m_j.
 *   Q4_0, 32 weights in 18 bytes: [0,2) d fp16, [2,18) 16 bytes of 4-bit quants; weight i < 16
 *     is the low nibble of byte 2+i, weight i >= 16 the high nibble of byte 2+i-16. Value:
 *     w = d*(q - 8).
 *
 * The pages list these two among the formats of the NTransformer loader ("Show HN" page,
 * section "Quantization support": Q4_0, Q8_0, Q4_K_M, Q5_K, Q6_K).
 *
 * Every product above has at most 23 significant bits and both Q4_K (and Q5_K) terms are
 * multiples of 2^-24 below 2^28 in magnitude, so the fp64 arithmetic here is exact;
 * orc_dequant_f32 then rounds once.
 */
#include "tq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int64_t orc_block_weights(int type) {
  switch (type) {
    case ORC_Q4_K: return 256;
    case ORC_Q6_K: return 256;
    case ORC_Q8_0: return 32;
    case ORC_Q5_K: return 256;
    case ORC_Q4_0: return 32;
    default: return 0;
  }
}

int64_t orc_block_bytes(int type) {
  switch (type) {
    case ORC_Q4_K: return 144;
    case ORC_Q6_K: return 210;
    case ORC_Q8_0: return 34;
    case ORC_Q5_K: return 176;
    case ORC_Q4_0: return 18;
    default: return 0;
  }
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double orc_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 31;
  int frac = h & 1023;
  double v;
  if (expo == 0) {
    v = ldexp((double)frac, -24); /* subnormal: frac * 2^-14 * 2^-10 */
  } else if (expo == 31) {
    v = frac ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/1024) * 2^(expo-15) */
  }
  return sign ? -v : v;
}

/* binary64 -> binary16 bit pattern, round to nearest, ties to even (used by the quantizers). */
static uint16_t double_to_half_rne(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return sign | 0x7E00;
  if (a >= 65520.0) return sign | 0x7C00; /* at or beyond the midpoint to 2^16: infinity */
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: the value in units of 2^-24, rounded to nearest even integer */
    double units = nearbyint(ldexp(a, 24));
    return sign | (uint16_t)units; /* units == 1024 lands exactly on the smallest normal */
  }
  int e;
  double m = frexp(a, &e);            /* a = m * 2^e, m in [0.5, 1) */
  double units = nearbyint(ldexp(m, 11)); /* 11 significant bits, in [1024, 2048] */
  if (units == 2048.0) {
    units = 1024.0;
    e += 1;
  }
  int expo = e - 1 + 15; /* a = units/1024 * 2^(e-1) */
  if (expo >= 31) return sign | 0x7C00;
  return sign | (uint16_t)(expo << 10) | (uint16_t)((int)units - 1024);
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t *p, uint16_t v) {
  p[0] = (uint8_t)(v & 255);
  p[1] = (uint8_t)(v >> 8);
}

/* Q4_K 6-bit scale and min of sub-block j from the twelve packed bytes S. */
static void q4k_scale_min(const uint8_t *S, int j, int *sc, int *m) {
  if (j < 4) {
    *sc = S[j] & 63;
    *m = S[j + 4] & 63;
  } else {
    *sc = (S[j + 4] & 15) | ((S[j - 4] >> 6) << 4);
    *m = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);
  }
}

static int q4k_quant(const uint8_t *qs, int i) {
  int c = i / 64, r = i % 64;
  return r < 32 ? (qs[32 * c + r] & 15) : (qs[32 * c + r - 32] >> 4);
}

static int q5k_quant(const uint8_t *qh, const uint8_t *qs, int i) {
  return q4k_quant(qs, i) + 16 * ((qh[i % 32] >> (i / 32)) & 1);
}

static int q40_quant(const uint8_t *qs, int i) {
  return i < 16 ? (qs[i] & 15) : (qs[i - 16] >> 4);
}

static int q6k_quant(const uint8_t *ql, const uint8_t *qh, int i) {
  int h = i / 128, r = i % 128, g = r / 32, l = r % 32;
  uint8_t lb = ql[64 * h + l + 32 * (g % 2)];
  int low4 = g < 2 ? (lb & 15) : (lb >> 4);
  int high2 = (qh[32 * h + l] >> (2 * g)) & 3;
  return low4 + 16 * high2;
}

double orc_block_weight(int type, const uint8_t *b, int i) {
  if (type == ORC_Q4_K) {
    double d = orc_half_to_double(rd16(b));
    double dmin = orc_half_to_double(rd16(b + 2));
    int sc, m;
    q4k_scale_min(b + 4, i / 32, &sc, &m);
    int q = q4k_quant(b + 16, i);
    return d * sc * q - dmin * m;
  }
  if (type == ORC_Q6_K) {
    double d = orc_half_to_double(rd16(b + 208));
    int sc = (int8_t)b[192 + i / 16];
    int q = q6k_quant(b, b + 128, i);
    return d * sc * (q - 32);
  }
  if (type == ORC_Q8_0) {
    double d = orc_half_to_double(rd16(b));
    return d * (int8_t)b[2 + i];
  }
  if (type == ORC_Q5_K) {
    double d = orc_half_to_double(rd16(b));
    double dmin = orc_half_to_double(rd16(b + 2));
    int sc, m;
    q4k_scale_min(b + 4, i / 32, &sc, &m);
    int q = q5k_quant(b + 16, b + 48, i);
    return d * sc * q - dmin * m;
  }
  if (type == ORC_Q4_0) {
    double d = orc_half_to_double(rd16(b));
    return d * (q40_quant(b + 2, i) - 8);
  }
  return NAN;
}

int orc_block_fields(int type, const uint8_t *b, double *d, double *dmin, int32_t *sc,
                     int32_t *m, int32_t *q) {
  if (type == ORC_Q4_K) {
    if (d) *d = orc_half_to_double(rd16(b));
    if (dmin) *dmin = orc_half_to_double(rd16(b + 2));
    for (int j = 0; j < 8; ++j) {
      int s, mm;
      q4k_scale_min(b + 4, j, &s, &mm);
      if (sc) sc[j] = s;
      if (m) m[j] = mm;
    }
    if (q)
      for (int i = 0; i < 256; ++i) q[i] = q4k_quant(b + 16, i);
    return 0;
  }
  if (type == ORC_Q6_K) {
    if (d) *d = orc_half_to_double(rd16(b + 208));
    if (sc)
      for (int s = 0; s < 16; ++s) sc[s] = (int8_t)b[192 + s];
    if (q)
      for (int i = 0; i < 256; ++i) q[i] = q6k_quant(b, b + 128, i);
    return 0;
  }
  if (type == ORC_Q8_0) {
    if (d) *d = orc_half_to_double(rd16(b));
    if (q)
      for (int i = 0; i < 32; ++i) q[i] = (int8_t)b[2 + i];
    return 0;
  }
  if (type == ORC_Q5_K) {
    if (d) *d = orc_half_to_double(rd16(b));
    if (dmin) *dmin = orc_half_to_double(rd16(b + 2));
    for (int j = 0; j < 8; ++j) {
      int s, mm;
      q4k_scale_min(b + 4, j, &s, &mm);
      if (sc) sc[j] = s;
      if (m) m[j] = mm;
    }
    if (q)
      for (int i = 0; i < 256; ++i) q[i] = q5k_quant(b + 16, b + 48, i);
    return 0;
  }
  if (type == ORC_Q4_0) {
    if (d) *d = orc_half_to_double(rd16(b));
    if (q)
      for (int i = 0; i < 32; ++i) q[i] = q40_quant(b + 2, i);
    return 0;
  }
  return -1;
}

static int shape_ok(int type, int64_t n, int64_t k) {
  int64_t bw = orc_block_weights(type);
  return bw > 0 && n >= 0 && k >= 0 && k % bw == 0;
}

/* Exact values of the weights of one block into out[]: the expressions of orc_block_weight,
 * evaluated in the same order, with the block's fp16 scales and sub-block fields read once per
 * block instead of once per weight (the values are the same bits). */
static void decode_block(int type, const uint8_t *b, double *out) {
  if (type == ORC_Q4_K) {
    double d = orc_half_to_double(rd16(b));
    double dmin = orc_half_to_double(rd16(b + 2));
    for (int j = 0; j < 8; ++j) {
      int sc, m;
      q4k_scale_min(b + 4, j, &sc, &m);
      for (int i = 32 * j; i < 32 * j + 32; ++i) out[i] = d * sc * q4k_quant(b + 16, i) - dmin * m;
    }
  } else if (type == ORC_Q6_K) {
    double d = orc_half_to_double(rd16(b + 208));
    for (int i = 0; i < 256; ++i) {
      int sc = (int8_t)b[192 + i / 16];
      out[i] = d * sc * (q6k_quant(b, b + 128, i) - 32);
    }
  } else if (type == ORC_Q8_0) {
    double d = orc_half_to_double(rd16(b));
    for (int i = 0; i < 32; ++i) out[i] = d * (int8_t)b[2 + i];
  } else if (type == ORC_Q5_K) {
    double d = orc_half_to_double(rd16(b));
    double dmin = orc_half_to_double(rd16(b + 2));
    for (int j = 0; j < 8; ++j) {
      int sc, m;
      q4k_scale_min(b + 4, j, &sc, &m);
      for (int i = 32 * j; i < 32 * j + 32; ++i)
        out[i] = d * sc * q5k_quant(b + 16, b + 48, i) - dmin * m;
    }
  } else if (type == ORC_Q4_0) {
    double d = orc_half_to_double(rd16(b));
    for (int i = 0; i < 32; ++i) out[i] = d * (q40_quant(b + 2, i) - 8);
  }
}

/* Exact values of row `row` into out[k]. */
static void decode_row(int type, const uint8_t *w, int64_t k, int64_t row, double *out) {
  int64_t bw = orc_block_weights(type), bb = orc_block_bytes(type);
  const uint8_t *rp = w + row * (k / bw) * bb;
  for (int64_t c = 0; c < k / bw; ++c) decode_block(type, rp + c * bb, out + c * bw);
}

int orc_dequant_f64(int type, const uint8_t *w, int64_t n, int64_t k, double *out) {
  if (!shape_ok(type, n, k)) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) decode_row(type, w, k, r, out + r * k);
  return 0;
}

int orc_dequant_f32(int type, const uint8_t *w, int64_t n, int64_t k, float *out) {
  if (!shape_ok(type, n, k)) return -1;
#pragma omp parallel
  {
    double *buf = (double *)malloc(sizeof(double) * (size_t)(k ? k : 1));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
      decode_row(type, w, k, r, buf);
      for (int64_t kk = 0; kk < k; ++kk) out[r * k + kk] = (float)buf[kk]; /* one RNE rounding */
    }
    free(buf);
  }
  return 0;
}

uint16_t orc_f32_to_bf16(float f) {
  uint32_t bits;
  memcpy(&bits, &f, 4);
  if (isnan(f)) return (uint16_t)((bits >> 16) | 0x40); /* stay NaN */
  uint32_t upper = bits >> 16, lower = bits & 0xFFFF;
  if (lower > 0x8000 || (lower == 0x8000 && (upper & 1))) upper += 1; /* nearest, ties to even */
  return (uint16_t)upper;
}

int orc_dequant_bf16(int type, const uint8_t *w, int64_t n, int64_t k, uint16_t *out) {
  if (!shape_ok(type, n, k)) return -1;
  float *tmp = (float *)malloc(sizeof(float) * (size_t)(n * k > 0 ? n * k : 1));
  if (!tmp) return -2;
  orc_dequant_f32(type, w, n, k, tmp);
  for (int64_t i = 0; i < n * k; ++i) out[i] = orc_f32_to_bf16(tmp[i]);
  free(tmp);
  return 0;
}

/* Shared body of the two GEMV entry points: xd is the activation matrix already widened to
 * fp64 ([batch][k]). */
static void gemv_body(int type, const uint8_t *w, int64_t n, int64_t k, const double *xd,
                      int64_t batch, const int64_t *rows, int64_t n_rows, double *y,
                      double *mag) {
  int64_t nr = rows ? n_rows : n;
#pragma omp parallel
  {
    double *wrow = (double *)malloc(sizeof(double) * (size_t)(k ? k : 1));
#pragma omp for schedule(static)
    for (int64_t ri = 0; ri < nr; ++ri) {
      int64_t row = rows ? rows[ri] : ri;
      decode_row(type, w, k, row, wrow);
      for (int64_t b = 0; b < batch; ++b) {
        const double *xb = xd + b * k;
        double s = 0.0, a = 0.0;
        for (int64_t kk = 0; kk < k; ++kk) {
          double p = wrow[kk] * xb[kk];
          s += p;
          a += fabs(p);
        }
        y[b * nr + ri] = s;
        if (mag) mag[b * nr + ri] = a;
      }
    }
    free(wrow);
  }
}

int orc_gemv(int type, const uint8_t *w, int64_t n, int64_t k, const float *x, int64_t batch,
             const int64_t *rows, int64_t n_rows, double *y, double *mag) {
  if (!shape_ok(type, n, k) || batch < 0) return -1;
  if (rows)
    for (int64_t i = 0; i < n_rows; ++i)
      if (rows[i] < 0 || rows[i] >= n) return -1;
  double *xd = (double *)malloc(sizeof(double) * (size_t)(batch * k > 0 ? batch * k : 1));
  if (!xd) return -2;
  for (int64_t i = 0; i < batch * k; ++i) xd[i] = x[i];
  gemv_body(type, w, n, k, xd, batch, rows, n_rows, y, mag);
  free(xd);
  return 0;
}

int orc_gemv_f64x(int type, const uint8_t *w, int64_t n, int64_t k, const double *x,
                  int64_t batch, const int64_t *rows, int64_t n_rows, double *y, double *mag) {
  if (!shape_ok(type, n, k) || batch < 0) return -1;
  if (rows)
    for (int64_t i = 0; i < n_rows; ++i)
      if (rows[i] < 0 || rows[i] >= n) return -1;
  gemv_body(type, w, n, k, x, batch, rows, n_rows, y, mag);
  return 0;
}

/* silu(g) * u = g * u / (1 + exp(-g)). For g < about -745, exp(-g) overflows to infinity and
 * the result is a signed zero, which is the limit. */
static double swiglu1(double g, double u) { return g * u / (1.0 + exp(-g)); }

void orc_swiglu_f32(const float *g, const float *u, int64_t n, double *h) {
  for (int64_t i = 0; i < n; ++i) h[i] = swiglu1((double)g[i], (double)u[i]);
}

void orc_swiglu_f64(const double *g, const double *u, int64_t n, double *h) {
  for (int64_t i = 0; i < n; ++i) h[i] = swiglu1(g[i], u[i]);
}

void orc_router_logits(const float *x, int64_t T, const float *wr, int64_t E, int64_t H,
                       double *logits) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t e = 0; e < E; ++e) {
      double s = 0.0;
      for (int64_t h = 0; h < H; ++h) s += (double)x[t * H + h] * (double)wr[e * H + h];
      logits[t * E + e] = s;
    }
}

/* Top-k of one token's logits (already fp64; fp32 inputs are widened exactly). Selection by
 * repeated arg-max: the largest remaining logit, the lower index on equality. */
static void topk_one(const double *l, int64_t E, int64_t k, int renormalize, int32_t *ids,
                     double *wts, unsigned char *taken) {
  memset(taken, 0, (size_t)E);
  for (int64_t j = 0; j < k; ++j) {
    int64_t best = -1;
    for (int64_t e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || l[e] > l[best]) best = e; /* strict '>' keeps the lower index on ties */
    }
    taken[best] = 1;
    ids[j] = (int32_t)best;
  }
  double lmax = l[ids[0]];
  double denom = 0.0;
  if (renormalize) {
    for (int64_t j = 0; j < k; ++j) denom += exp(l[ids[j]] - lmax);
  } else {
    for (int64_t e = 0; e < E; ++e) denom += exp(l[e] - lmax);
  }
  for (int64_t j = 0; j < k; ++j) wts[j] = exp(l[ids[j]] - lmax) / denom;
}

int orc_topk_f64(const double *logits, int64_t T, int64_t E, int64_t k, int renormalize,
                 int32_t *ids, double *weights) {
  if (k < 1 || k > E) return -1;
  unsigned char *taken = (unsigned char *)malloc((size_t)E);
  for (int64_t t = 0; t < T; ++t)
    topk_one(logits + t * E, E, k, renormalize, ids + t * k, weights + t * k, taken);
  free(taken);
  return 0;
}

int orc_topk_f32(const float *logits, int64_t T, int64_t E, int64_t k, int renormalize,
                 int32_t *ids, double *weights) {
  if (k < 1 || k > E) return -1;
  double *l = (double *)malloc(sizeof(double) * (size_t)E);
  unsigned char *taken = (unsigned char *)malloc((size_t)E);
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t e = 0; e < E; ++e) l[e] = (double)logits[t * E + e];
    topk_one(l, E, k, renormalize, ids + t * k, weights + t * k, taken);
  }
  free(taken);
  free(l);
  return 0;
}

int orc_group(const int32_t *ids, int64_t T, int64_t k, int64_t E, int32_t *counts,
              int32_t *offsets, int32_t *pairs) {
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < T * k; ++p) {
    if (ids[p] < 0 || ids[p] >= E) return -1;
    counts[ids[p]] += 1;
  }
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  /* walk the pairs in ascending (t, j); each lands after the earlier pairs of its expert */
  int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E ? E : 1));
  for (int64_t e = 0; e < E; ++e) fill[e] = offsets[e];
  for (int64_t p = 0; p < T * k; ++p) pairs[fill[ids[p]]++] = (int32_t)p;
  free(fill);
  return 0;
}

/* down . swiglu(gate . x, up . x) for one token, with the matching absolute sums. */
static void expert_ffn(int type, int64_t hidden, int64_t ffn, const orc_expert *ex,
                       const float *x, double *o, double *omag) {
  double *g = (double *)malloc(sizeof(double) * (size_t)ffn);
  double *u = (double *)malloc(sizeof(double) * (size_t)ffn);
  double *h = (double *)malloc(sizeof(double) * (size_t)ffn);
  orc_gemv(type, ex->gate, ffn, hidden, x, 1, NULL, 0, g, NULL);
  orc_gemv(type, ex->up, ffn, hidden, x, 1, NULL, 0, u, NULL);
  orc_swiglu_f64(g, u, ffn, h);
  orc_gemv_f64x(type, ex->down, hidden, ffn, h, 1, NULL, 0, o, omag);
  free(g);
  free(u);
  free(h);
}

/* The bf16 value of a bf16 bit pattern, widened exactly. */
static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* v rounded to fp32 and then to bf16 (each to nearest even). */
static double round_bf16(double v) { return bf16_value(orc_f32_to_bf16((float)v)); }

/* y[i] = sum_c bf16(w[i][c]) * xb[c] for the n rows of a blob, where bf16(w) is the bf16 rounding
 * of the fp32 weight and xb holds values already rounded to bf16; fp64, ascending c. */
static int gemv_bf16(int type, const uint8_t *w, int64_t n, int64_t k, const double *xb,
                     double *y, double *mag) {
  const int64_t rb = k / orc_block_weights(type) * orc_block_bytes(type);
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t i = 0; i < n; ++i) {
    uint16_t *wb = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)k);
    if (!wb || orc_dequant_bf16(type, w + i * rb, 1, k, wb) != 0) {
      bad = 1;
    } else {
      double s = 0.0, m = 0.0;
      for (int64_t c = 0; c < k; ++c) {
        double p = bf16_value(wb[c]) * xb[c];
        s += p;
        m += fabs(p);
      }
      y[i] = s;
      if (mag) mag[i] = m;
    }
    free(wb);
  }
  return bad ? -1 : 0;
}

/* The expert FFN with bf16 operands: x, every weight and h rounded to bf16, products summed in
 * fp64. */
static void expert_ffn_bf16(int type, int64_t hidden, int64_t ffn, const orc_expert *ex,
                            const float *x, double *o, double *omag) {
  double *xb = (double *)malloc(sizeof(double) * (size_t)hidden);
  double *g = (double *)malloc(sizeof(double) * (size_t)ffn);
  double *u = (double *)malloc(sizeof(double) * (size_t)ffn);
  double *h = (double *)malloc(sizeof(double) * (size_t)ffn);
  for (int64_t c = 0; c < hidden; ++c) xb[c] = round_bf16((double)x[c]);
  gemv_bf16(type, ex->gate, ffn, hidden, xb, g, NULL);
  gemv_bf16(type, ex->up, ffn, hidden, xb, u, NULL);
  orc_swiglu_f64(g, u, ffn, h);
  for (int64_t f = 0; f < ffn; ++f) h[f] = round_bf16(h[f]);
  gemv_bf16(type, ex->down, hidden, ffn, h, o, omag);
  free(xb);
  free(g);
  free(u);
  free(h);
}

typedef void (*expert_fn)(int, int64_t, int64_t, const orc_expert *, const float *, double *,
                          double *);

static int moe_body(expert_fn ffn_of, int type, int64_t hidden, int64_t ffn,
                    const orc_expert *experts, int64_t n_experts, const orc_expert *shared,
                    const float *x, int64_t T, int64_t k, const int32_t *ids,
                    const double *weights, const int64_t *tokens, int64_t n_tok, double *y,
                    double *mag) {
  int64_t bw = orc_block_weights(type);
  if (bw == 0 || hidden % bw || ffn % bw || k < 1) return -1;
  int64_t nt = tokens ? n_tok : T;
  double *o = (double *)malloc(sizeof(double) * (size_t)hidden);
  double *om = (double *)malloc(sizeof(double) * (size_t)hidden);
  for (int64_t ti = 0; ti < nt; ++ti) {
    int64_t t = tokens ? tokens[ti] : ti;
    if (t < 0 || t >= T) {
      free(o);
      free(om);
      return -1;
    }
    double *yt = y + ti * hidden;
    double *mt = mag ? mag + ti * hidden : NULL;
    for (int64_t i = 0; i < hidden; ++i) {
      yt[i] = 0.0;
      if (mt) mt[i] = 0.0;
    }
    for (int64_t j = 0; j < k; ++j) {
      int32_t e = ids[t * k + j];
      if (e < 0 || e >= n_experts) {
        free(o);
        free(om);
        return -1;
      }
      double wt = weights[t * k + j];
      ffn_of(type, hidden, ffn, &experts[e], x + t * hidden, o, om);
      for (int64_t i = 0; i < hidden; ++i) {
        yt[i] += wt * o[i];
        if (mt) mt[i] += fabs(wt) * om[i];
      }
    }
    if (shared) {
      ffn_of(type, hidden, ffn, shared, x + t * hidden, o, om);
      for (int64_t i = 0; i < hidden; ++i) {
        yt[i] += o[i];
        if (mt) mt[i] += om[i];
      }
    }
  }
  free(o);
  free(om);
  return 0;
}

int orc_moe(int type, int64_t hidden, int64_t ffn, const orc_expert *experts, int64_t n_experts,
            const orc_expert *shared, const float *x, int64_t T, int64_t k, const int32_t *ids,
            const double *weights, const int64_t *tokens, int64_t n_tok, double *y, double *mag) {
  return moe_body(expert_ffn, type, hidden, ffn, experts, n_experts, shared, x, T, k, ids,
                  weights, tokens, n_tok, y, mag);
}

int orc_moe_bf16(int type, int64_t hidden, int64_t ffn, const orc_expert *experts,
                 int64_t n_experts, const orc_expert *shared, const float *x, int64_t T,
                 int64_t k, const int32_t *ids, const double *weights, const int64_t *tokens,
                 int64_t n_tok, double *y, double *mag) {
  return moe_body(expert_ffn_bf16, type, hidden, ffn, experts, n_experts, shared, x, T, k, ids,
                  weights, tokens, n_tok, y, mag);
}

/* The result of orc_moe, bitwise, with the work grouped by expert so that large layers finish in
 * seconds: the tokens routed to one expert go through its three matrices together (orc_gemv
 * over a batch decodes each row once for all of them), each (token, slot) pair's output is kept,
 * and every token's output is then formed exactly as in moe_body: its pairs in slot order, then
 * the shared expert. Every value is computed by the same expressions in the same order as in
 * orc_moe, so nothing but the loop nesting differs. */
static int expert_batch(int type, int64_t hidden, int64_t ffn, const orc_expert *ex,
                        const float *xs, int64_t B, double *o, double *om) {
  double *g = (double *)malloc(sizeof(double) * (size_t)(B * ffn));
  double *u = (double *)malloc(sizeof(double) * (size_t)(B * ffn));
  double *h = (double *)malloc(sizeof(double) * (size_t)(B * ffn));
  int rc = (g && u && h) ? 0 : -2;
  if (rc == 0) rc = orc_gemv(type, ex->gate, ffn, hidden, xs, B, NULL, 0, g, NULL);
  if (rc == 0) rc = orc_gemv(type, ex->up, ffn, hidden, xs, B, NULL, 0, u, NULL);
  if (rc == 0) {
    orc_swiglu_f64(g, u, B * ffn, h);
    rc = orc_gemv_f64x(type, ex->down, hidden, ffn, h, B, NULL, 0, o, om);
  }
  free(g);
  free(u);
  free(h);
  return rc;
}

int orc_moe_grouped(int type, int64_t hidden, int64_t ffn, const orc_expert *experts,
                    int64_t n_experts, const orc_expert *shared, const float *x, int64_t T,
                    int64_t k, const int32_t *ids, const double *weights, const int64_t *tokens,
                    int64_t n_tok, double *y, double *mag) {
  int64_t bw = orc_block_weights(type);
  if (bw == 0 || hidden % bw || ffn % bw || k < 1) return -1;
  int64_t nt = tokens ? n_tok : T;
  for (int64_t ti = 0; ti < nt; ++ti) {
    int64_t t = tokens ? tokens[ti] : ti;
    if (t < 0 || t >= T) return -1;
    for (int64_t j = 0; j < k; ++j)
      if (ids[t * k + j] < 0 || ids[t * k + j] >= n_experts) return -1;
  }
  const int64_t np = nt * k;
  double *po = (double *)malloc(sizeof(double) * (size_t)((np ? np : 1) * hidden));
  double *pm = (double *)malloc(sizeof(double) * (size_t)((np ? np : 1) * hidden));
  double *so = (double *)malloc(sizeof(double) * (size_t)((nt ? nt : 1) * hidden));
  double *sm = (double *)malloc(sizeof(double) * (size_t)((nt ? nt : 1) * hidden));
  int64_t *which = (int64_t *)malloc(sizeof(int64_t) * (size_t)(np ? np : 1));
  float *xs = (float *)malloc(sizeof(float) * (size_t)((np > nt ? np : nt) + 1) * (size_t)hidden);
  double *o = (double *)malloc(sizeof(double) * (size_t)((np > nt ? np : nt) + 1) * (size_t)hidden);
  double *om = (double *)malloc(sizeof(double) * (size_t)((np > nt ? np : nt) + 1) * (size_t)hidden);
  int rc = (po && pm && so && sm && which && xs && o && om) ? 0 : -2;
  for (int64_t e = 0; rc == 0 && e < n_experts; ++e) {
    int64_t B = 0;
    for (int64_t p = 0; p < np; ++p) {
      int64_t t = tokens ? tokens[p / k] : p / k;
      if (ids[t * k + p % k] == e) {
        which[B] = p;
        memcpy(xs + B * hidden, x + t * hidden, sizeof(float) * (size_t)hidden);
        ++B;
      }
    }
    if (B == 0) continue;
    rc = expert_batch(type, hidden, ffn, &experts[e], xs, B, o, om);
    for (int64_t b = 0; rc == 0 && b < B; ++b) {
      memcpy(po + which[b] * hidden, o + b * hidden, sizeof(double) * (size_t)hidden);
      memcpy(pm + which[b] * hidden, om + b * hidden, sizeof(double) * (size_t)hidden);
    }
  }
  if (rc == 0 && shared && nt > 0) {
    for (int64_t ti = 0; ti < nt; ++ti) {
      int64_t t = tokens ? tokens[ti] : ti;
      memcpy(xs + ti * hidden, x + t * hidden, sizeof(float) * (size_t)hidden);
    }
    rc = expert_batch(type, hidden, ffn, shared, xs, nt, so, sm);
  }
  for (int64_t ti = 0; rc == 0 && ti < nt; ++ti) {
    int64_t t = tokens ? tokens[ti] : ti;
    double *yt = y + ti * hidden;
    double *mt = mag ? mag + ti * hidden : NULL;
    for (int64_t i = 0; i < hidden; ++i) {
      yt[i] = 0.0;
      if (mt) mt[i] = 0.0;
    }
    for (int64_t j = 0; j < k; ++j) {
      double wt = weights[t * k + j];
      const double *oo = po + (ti * k + j) * hidden, *mm = pm + (ti * k + j) * hidden;
      for (int64_t i = 0; i < hidden; ++i) {
        yt[i] += wt * oo[i];
        if (mt) mt[i] += fabs(wt) * mm[i];
      }
    }
    if (shared) {
      for (int64_t i = 0; i < hidden; ++i) {
        yt[i] += so[ti * hidden + i];
        if (mt) mt[i] += sm[ti * hidden + i];
      }
    }
  }
  free(po);
  free(pm);
  free(so);
  free(sm);
  free(which);
  free(xs);
  free(o);
  free(om);
  return rc;
}

/* ---- reference quantizers (round-trip tests only) ---- */

static int clampi(double v, int lo, int hi) {
  if (v < lo) return lo;
  if (v > hi) return hi;
  return (int)v;
}

/* Write quants q[256] into a Q4_K block's qs bytes (inverse of q4k_quant). */
static void q4k_put_quants(uint8_t *qs, const int *q) {
  for (int c = 0; c < 4; ++c)
    for (int l = 0; l < 32; ++l)
      qs[32 * c + l] = (uint8_t)((q[64 * c + l] & 15) | ((q[64 * c + 32 + l] & 15) << 4));
}

/* Write eight 6-bit scales and mins into the twelve bytes S (inverse of q4k_scale_min). */
static void q4k_put_scales(uint8_t *S, const int *sc, const int *m) {
  memset(S, 0, 12);
  for (int j = 0; j < 4; ++j) {
    S[j] = (uint8_t)(sc[j] & 63);
    S[j + 4] = (uint8_t)(m[j] & 63);
  }
  for (int j = 4; j < 8; ++j) {
    S[j + 4] = (uint8_t)((sc[j] & 15) | ((m[j] & 15) << 4));
    S[j - 4] |= (uint8_t)((sc[j] >> 4) << 6);
    S[j] |= (uint8_t)((m[j] >> 4) << 6);
  }
}

/* Write quants q[256] (0..31) into a Q5_K block's qh/qs bytes (inverse of q5k_quant). */
static void q5k_put_quants(uint8_t *qh, uint8_t *qs, const int *q) {
  int low[256];
  memset(qh, 0, 32);
  for (int i = 0; i < 256; ++i) {
    low[i] = q[i] & 15;
    qh[i % 32] |= (uint8_t)(((q[i] >> 4) & 1) << (i / 32));
  }
  q4k_put_quants(qs, low);
}

/* Write quants q[32] (0..15) into a Q4_0 block's 16 quant bytes (inverse of q40_quant). */
static void q40_put_quants(uint8_t *qs, const int *q) {
  for (int i = 0; i < 16; ++i) qs[i] = (uint8_t)((q[i] & 15) | ((q[i + 16] & 15) << 4));
}

/* Write quants q[256] (0..63) into a Q6_K block's ql/qh bytes (inverse of q6k_quant). */
static void q6k_put_quants(uint8_t *ql, uint8_t *qh, const int *q) {
  memset(ql, 0, 128);
  memset(qh, 0, 64);
  for (int i = 0; i < 256; ++i) {
    int h = i / 128, r = i % 128, g = r / 32, l = r % 32;
    int low4 = q[i] & 15, high2 = (q[i] >> 4) & 3;
    int li = 64 * h + l + 32 * (g % 2);
    ql[li] |= (uint8_t)(g < 2 ? low4 : low4 << 4);
    qh[32 * h + l] |= (uint8_t)(high2 << (2 * g));
  }
}

int orc_requant(int type, const uint8_t *w_blob, const double *w, int64_t n, int64_t k,
                uint8_t *out) {
  if (!shape_ok(type, n, k)) return -1;
  int64_t bw = orc_block_weights(type), bb = orc_block_bytes(type);
  int64_t nblk = n * (k / bw);
  for (int64_t blk = 0; blk < nblk; ++blk) {
    const uint8_t *b = w_blob + blk * bb;
    uint8_t *ob = out + blk * bb;
    const double *wv = w + blk * bw; /* blocks are contiguous along rows of [n][k] */
    memcpy(ob, b, (size_t)bb);
    int q[256];
    if (type == ORC_Q4_K || type == ORC_Q5_K) {
      double d, dmin;
      int32_t sc[8], m[8];
      const int qmax = type == ORC_Q4_K ? 15 : 31;
      orc_block_fields(type, b, &d, &dmin, sc, m, NULL);
      for (int i = 0; i < 256; ++i) {
        double step = d * sc[i / 32];
        q[i] = step != 0.0 ? clampi(nearbyint((wv[i] + dmin * m[i / 32]) / step), 0, qmax) : 0;
      }
      if (type == ORC_Q4_K)
        q4k_put_quants(ob + 16, q);
      else
        q5k_put_quants(ob + 16, ob + 48, q);
    } else if (type == ORC_Q4_0) {
      double d;
      orc_block_fields(type, b, &d, NULL, NULL, NULL, NULL);
      for (int i = 0; i < 32; ++i) q[i] = d != 0.0 ? clampi(nearbyint(wv[i] / d) + 8, 0, 15) : 8;
      q40_put_quants(ob + 2, q);
    } else if (type == ORC_Q6_K) {
      double d;
      int32_t sc[16];
      orc_block_fields(type, b, &d, NULL, sc, NULL, NULL);
      for (int i = 0; i < 256; ++i) {
        double step = d * sc[i / 16];
        q[i] = step != 0.0 ? clampi(nearbyint(wv[i] / step) + 32, 0, 63) : 32;
      }
      q6k_put_quants(ob, ob + 128, q);
    } else {
      double d;
      orc_block_fields(type, b, &d, NULL, NULL, NULL, NULL);
      for (int i = 0; i < 32; ++i) {
        int qi = d != 0.0 ? clampi(nearbyint(wv[i] / d), -128, 127) : 0;
        ob[2 + i] = (uint8_t)(int8_t)qi;
      }
    }
  }
  return 0;
}

int orc_quantize(int type, const float *w, int64_t n, int64_t k, uint8_t *out) {
  if (!shape_ok(type, n, k)) return -1;
  int64_t bw = orc_block_weights(type), bb = orc_block_bytes(type);
  int64_t nblk = n * (k / bw);
  for (int64_t blk = 0; blk < nblk; ++blk) {
    const float *wv = w + blk * bw;
    uint8_t *ob = out + blk * bb;
    memset(ob, 0, (size_t)bb);
    int q[256];
    if (type == ORC_Q4_0) {
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs((double)wv[i]));
      uint16_t dh = double_to_half_rne(amax / 7.0); /* |w| <= 7d: quants 1..15 */
      double d = orc_half_to_double(dh);
      wr16(ob, dh);
      for (int i = 0; i < 32; ++i) q[i] = d != 0.0 ? clampi(nearbyint(wv[i] / d) + 8, 0, 15) : 8;
      q40_put_quants(ob + 2, q);
    } else if (type == ORC_Q8_0) {
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs((double)wv[i]));
      uint16_t dh = double_to_half_rne(amax / 127.0);
      double d = orc_half_to_double(dh);
      wr16(ob, dh);
      for (int i = 0; i < 32; ++i) {
        int qi = d != 0.0 ? clampi(nearbyint(wv[i] / d), -127, 127) : 0;
        ob[2 + i] = (uint8_t)(int8_t)qi;
      }
    } else if (type == ORC_Q6_K) {
      double s[16], smax = 0.0;
      for (int g = 0; g < 16; ++g) {
        double amax = 0.0;
        for (int i = 0; i < 16; ++i) amax = fmax(amax, fabs((double)wv[16 * g + i]));
        s[g] = amax / 31.0; /* largest magnitude lands on quant offset +-31 */
        smax = fmax(smax, s[g]);
      }
      uint16_t dh = double_to_half_rne(smax / 127.0);
      double d = orc_half_to_double(dh);
      wr16(ob + 208, dh);
      int sc[16];
      for (int g = 0; g < 16; ++g) {
        sc[g] = d != 0.0 ? clampi(nearbyint(s[g] / d), -128, 127) : 0;
        ob[192 + g] = (uint8_t)(int8_t)sc[g];
      }
      for (int i = 0; i < 256; ++i) {
        double step = d * sc[i / 16];
        q[i] = step != 0.0 ? clampi(nearbyint(wv[i] / step) + 32, 0, 63) : 32;
      }
      q6k_put_quants(ob, ob + 128, q);
    } else { /* Q4_K, Q5_K */
      const int qmax = type == ORC_Q4_K ? 15 : 31;
      double s[8], mn[8], smax = 0.0, mmax = 0.0;
      for (int j = 0; j < 8; ++j) {
        double lo = 0.0, hi = -INFINITY;
        for (int i = 0; i < 32; ++i) {
          lo = fmin(lo, (double)wv[32 * j + i]);
          hi = fmax(hi, (double)wv[32 * j + i]);
        }
        if (hi < lo) hi = lo;
        mn[j] = -lo;              /* min offset, >= 0 */
        s[j] = (hi - lo) / qmax;  /* step spanning [lo, hi] with qmax + 1 levels */
        smax = fmax(smax, s[j]);
        mmax = fmax(mmax, mn[j]);
      }
      uint16_t dh = double_to_half_rne(smax / 63.0), mh = double_to_half_rne(mmax / 63.0);
      double d = orc_half_to_double(dh), dmin = orc_half_to_double(mh);
      wr16(ob, dh);
      wr16(ob + 2, mh);
      int sc[8], m[8];
      for (int j = 0; j < 8; ++j) {
        sc[j] = d != 0.0 ? clampi(nearbyint(s[j] / d), 0, 63) : 0;
        m[j] = dmin != 0.0 ? clampi(nearbyint(mn[j] / dmin), 0, 63) : 0;
      }
      q4k_put_scales(ob + 4, sc, m);
      for (int i = 0; i < 256; ++i) {
        double step = d * sc[i / 32];
        q[i] = step != 0.0 ? clampi(nearbyint((wv[i] + dmin * m[i / 32]) / step), 0, qmax) : 0;
      }
      if (type == ORC_Q4_K)
        q4k_put_quants(ob + 16, q);
      else
        q5k_put_quants(ob + 16, ob + 48, q);
    }
  }
  return 0;
}
