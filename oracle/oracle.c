/*
 * oracle.c -- plain fp64 CPU reference for the 4-bit quantized decode
 * projections.  TEST INFRASTRUCTURE ONLY: see oracle.h for who may use it and
 * for the page citations.  Plain C11, libm only, no fast-math, no blocking,
 * no reordering: every sum runs over its index in ascending order.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- O0 ---- */

double o_bf16_to_f64(uint16_t h) {
  /* A bf16 is the top half of an IEEE binary32; widening is exact. */
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double o_f16_to_f64(uint16_t h) {
  /* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24); /* subnormal: f * 2^-14 / 1024 */
  } else if (e == 31) {
    v = (f == 0) ? INFINITY : NAN;
  } else {
    v = ldexp(1024.0 + (double)f, e - 25); /* (1 + f/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

uint16_t o_f64_to_bf16_rne(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
  if (isinf(v)) return (uint16_t)(sign | 0x7F80u);
  if (a == 0.0) return sign;
  int e;
  (void)frexp(a, &e); /* a = f * 2^e, 0.5 <= f < 1 */
  int be = e - 1 + 127; /* biased exponent if a rounds to a normal bf16 */
  if (be <= 0) {
    /* subnormal range: value = r * 2^-133, r in 0..128 (128 = min normal) */
    double r = nearbyint(ldexp(a, 133));
    return (uint16_t)(sign | (uint16_t)r);
  }
  double r = nearbyint(ldexp(a, 8 - e)); /* 8 significant bits, in [128,256] */
  if (r >= 256.0) {
    r = 128.0;
    be += 1;
  }
  if (be >= 255) return (uint16_t)(sign | 0x7F80u);
  return (uint16_t)(sign | (uint16_t)(be << 7) | (uint16_t)((int)r - 128));
}

/* ---------------------------------------------------------------- O1 ---- */
/* Affine 4-bit, group 64 along K (MLX-style 4-bit weights named by the uzu
 * page's weight_matrix row; "4-bit group 64" in the TensorFold box table).
 * Reading: code k of row n sits in word k/8 of that row, bits 4*(k%8) ..
 * 4*(k%8)+3 (low nibble first); the weight is scale*code + bias with the bf16
 * scale and bias of group k/64. */
int oracle_dequant_affine4(const uint32_t* codes, const uint16_t* scales,
                           const uint16_t* biases, int64_t N, int64_t K,
                           int64_t n0, int64_t nr, double* w) {
  if (!codes || !scales || !biases || !w) return -1;
  if (N < 0 || K <= 0 || K % 64 != 0 || n0 < 0 || nr < 0 || n0 + nr > N)
    return -1;
  const int64_t words = K / 8, groups = K / 64;
  for (int64_t r = 0; r < nr; ++r) {
    const int64_t n = n0 + r;
    for (int64_t k = 0; k < K; ++k) {
      uint32_t word = codes[n * words + k / 8];
      unsigned q = (unsigned)((word >> (4 * (k % 8))) & 15u);
      double s = o_bf16_to_f64(scales[n * groups + k / 64]);
      double b = o_bf16_to_f64(biases[n * groups + k / 64]);
      w[r * K + k] = s * (double)q + b;
    }
  }
  return 0;
}

/* ---------------------------------------------------------------- O2 ---- */
/* GGUF Q4_K (the runNburn page runs Q4_K_M GGUF files as stored; the pages do
 * not print the block layout).  Reading -- the public 144-byte block:
 *   bytes 0-1 d (fp16), 2-3 dmin (fp16), 4-15 twelve bytes holding eight
 *   6-bit scales sc_j and eight 6-bit mins m_j, 16-143 the 256 codes.
 *   Weight o (0..255) of the block belongs to sub-block j = o/32; its code is
 *   the low nibble of code byte 32*(o/64) + o%32 when o%64 < 32, else the
 *   high nibble of that byte.  Its value is d*sc_j*q - dmin*m_j. */
static void q4k_scale_min(const uint8_t* s12, int j, unsigned* sc, unsigned* m) {
  if (j < 4) {
    *sc = s12[j] & 63u;
    *m = s12[j + 4] & 63u;
  } else {
    /* low four bits from byte j+4, top two bits from bits 6-7 of byte j-4
     * (scale) or byte j (min) */
    *sc = (unsigned)(s12[j + 4] & 15u) | ((unsigned)(s12[j - 4] >> 6) << 4);
    *m = (unsigned)(s12[j + 4] >> 4) | ((unsigned)(s12[j] >> 6) << 4);
  }
}

int oracle_dequant_q4k(const uint8_t* blocks, int64_t N, int64_t K, int64_t n0,
                       int64_t nr, double* w) {
  if (!blocks || !w) return -1;
  if (N < 0 || K <= 0 || K % 256 != 0 || n0 < 0 || nr < 0 || n0 + nr > N)
    return -1;
  const int64_t nb = K / 256;
  for (int64_t r = 0; r < nr; ++r) {
    const int64_t n = n0 + r;
    for (int64_t t = 0; t < nb; ++t) {
      const uint8_t* blk = blocks + (n * nb + t) * 144;
      double d = o_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
      double dmin = o_f16_to_f64((uint16_t)(blk[2] | (blk[3] << 8)));
      const uint8_t* s12 = blk + 4;
      const uint8_t* qs = blk + 16;
      for (int o = 0; o < 256; ++o) {
        int j = o / 32;
        uint8_t byte = qs[32 * (o / 64) + o % 32];
        unsigned q = (o % 64 < 32) ? (byte & 15u) : (unsigned)(byte >> 4);
        unsigned sc, m;
        q4k_scale_min(s12, j, &sc, &m);
        w[r * K + t * 256 + o] = d * (double)sc * (double)q - dmin * (double)m;
      }
    }
  }
  return 0;
}

/* ---------------------------------------------------------------- O3 ---- */

static double* decode_bf16_rows(const uint16_t* x, int M, int64_t K) {
  double* xd = (double*)malloc(sizeof(double) * (size_t)M * (size_t)K);
  if (!xd) return NULL;
  for (int64_t i = 0; i < (int64_t)M * K; ++i) xd[i] = o_bf16_to_f64(x[i]);
  return xd;
}

static double dot_asc(const double* a, const double* b, int64_t K) {
  double s = 0.0;
  for (int64_t k = 0; k < K; ++k) s += a[k] * b[k];
  return s;
}

int oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

int oracle_qgemv_affine4_f64x(const double* x, const uint32_t* codes,
                              const uint16_t* scales, const uint16_t* biases,
                              int M, int64_t N, int64_t K, double* y) {
  if (!x || !y || M < 1 || N < 0) return -1;
  int rc = 0;
#pragma omp parallel reduction(| : rc)
  {
    double* wrow = (double*)malloc(sizeof(double) * (size_t)K);
    if (!wrow) rc = -1;
#pragma omp for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
      if (rc) continue;
      if (oracle_dequant_affine4(codes, scales, biases, N, K, n, 1, wrow)) {
        rc = -1;
        continue;
      }
      for (int m = 0; m < M; ++m) y[(int64_t)m * N + n] = dot_asc(x + (int64_t)m * K, wrow, K);
    }
    free(wrow);
  }
  return rc;
}

int oracle_qgemv_affine4(const uint16_t* x, const uint32_t* codes,
                         const uint16_t* scales, const uint16_t* biases, int M,
                         int64_t N, int64_t K, double* y) {
  if (!x || M < 1 || K <= 0) return -1;
  double* xd = decode_bf16_rows(x, M, K);
  if (!xd) return -1;
  int rc = oracle_qgemv_affine4_f64x(xd, codes, scales, biases, M, N, K, y);
  free(xd);
  return rc;
}

static int qgemv_q4k_f64x(const double* x, const uint8_t* blocks, int M,
                          int64_t N, int64_t K, double* y) {
  if (!x || !y || M < 1 || N < 0) return -1;
  int rc = 0;
#pragma omp parallel reduction(| : rc)
  {
    double* wrow = (double*)malloc(sizeof(double) * (size_t)K);
    if (!wrow) rc = -1;
#pragma omp for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
      if (rc) continue;
      if (oracle_dequant_q4k(blocks, N, K, n, 1, wrow)) {
        rc = -1;
        continue;
      }
      for (int m = 0; m < M; ++m) y[(int64_t)m * N + n] = dot_asc(x + (int64_t)m * K, wrow, K);
    }
    free(wrow);
  }
  return rc;
}

int oracle_qgemv_q4k(const uint16_t* x, const uint8_t* blocks, int M, int64_t N,
                     int64_t K, double* y) {
  if (!x || M < 1 || K <= 0) return -1;
  double* xd = decode_bf16_rows(x, M, K);
  if (!xd) return -1;
  int rc = qgemv_q4k_f64x(xd, blocks, M, N, K, y);
  free(xd);
  return rc;
}

/* ---------------------------------------------------------------- O4 ---- */
/* RMSNorm ahead of the projection (the Husky page fuses the preceding norm
 * into each projection kernel).  Reading: gain multiplies, eps inside the
 * square root, mean over K, no centring. */
int oracle_rmsnorm(const uint16_t* x, const uint16_t* gamma, double eps, int M,
                   int64_t K, double* xn) {
  if (!x || !gamma || !xn || M < 1 || K <= 0) return -1;
  for (int m = 0; m < M; ++m) {
    double ss = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double v = o_bf16_to_f64(x[(int64_t)m * K + k]);
      ss += v * v;
    }
    double denom = sqrt(ss / (double)K + eps);
    for (int64_t k = 0; k < K; ++k) {
      double v = o_bf16_to_f64(x[(int64_t)m * K + k]);
      xn[(int64_t)m * K + k] = v * o_bf16_to_f64(gamma[k]) / denom;
    }
  }
  return 0;
}

/* ---------------------------------------------------------------- O5 ---- */

double oracle_silu(double g) { return g / (1.0 + exp(-g)); }

/* ---------------------------------------------------------------- O6 ---- */
/* Gate and up computed together (Husky page, fused kernels); gate rows come
 * first in the fused matrix, then up rows; h = silu(gate) * up. */
static int gateup_swiglu_f64x(const double* xn, const uint32_t* codes_gu,
                              const uint16_t* scales_gu,
                              const uint16_t* biases_gu, int M, int64_t I,
                              int64_t K, double* h) {
  double* gu = (double*)malloc(sizeof(double) * (size_t)M * (size_t)(2 * I));
  if (!gu) return -1;
  int rc = oracle_qgemv_affine4_f64x(xn, codes_gu, scales_gu, biases_gu, M,
                                     2 * I, K, gu);
  if (rc == 0) {
    for (int m = 0; m < M; ++m)
      for (int64_t i = 0; i < I; ++i) {
        double g = gu[(int64_t)m * 2 * I + i];
        double u = gu[(int64_t)m * 2 * I + I + i];
        h[(int64_t)m * I + i] = oracle_silu(g) * u;
      }
  }
  free(gu);
  return rc;
}

int oracle_rmsnorm_gateup_swiglu(const uint16_t* x, const uint16_t* gamma,
                                 double eps, const uint32_t* codes_gu,
                                 const uint16_t* scales_gu,
                                 const uint16_t* biases_gu, int M, int64_t I,
                                 int64_t K, double* h) {
  if (!h || M < 1 || I <= 0 || K <= 0) return -1;
  double* xn = (double*)malloc(sizeof(double) * (size_t)M * (size_t)K);
  if (!xn) return -1;
  int rc = oracle_rmsnorm(x, gamma, eps, M, K, xn);
  if (rc == 0) rc = gateup_swiglu_f64x(xn, codes_gu, scales_gu, biases_gu, M, I, K, h);
  free(xn);
  return rc;
}

int oracle_mlp_block(const uint16_t* x, const uint16_t* gamma, double eps,
                     const uint32_t* codes_gu, const uint16_t* scales_gu,
                     const uint16_t* biases_gu, const uint32_t* codes_d,
                     const uint16_t* scales_d, const uint16_t* biases_d, int M,
                     int64_t I, int64_t K, double* y) {
  if (!y || M < 1 || I <= 0 || K <= 0) return -1;
  double* h = (double*)malloc(sizeof(double) * (size_t)M * (size_t)I);
  if (!h) return -1;
  int rc = oracle_rmsnorm_gateup_swiglu(x, gamma, eps, codes_gu, scales_gu,
                                        biases_gu, M, I, K, h);
  if (rc == 0) rc = oracle_qgemv_affine4_f64x(h, codes_d, scales_d, biases_d, M, K, I, y);
  free(h);
  return rc;
}

/* ---------------------------------------------------------------- O7 ---- */
/* Routed experts (uzu page: MixtureOfExperts with a routing function; the
 * runNburn page: routing is never altered by the engine).  Readings: the
 * top_k largest logits are selected, larger first, equal logits -> lower
 * expert index; the weights are the softmax over the selected logits only;
 * each selected expert is a SwiGLU MLP stored in Q4_K; the output is the
 * weighted sum over the selected experts in ascending expert order; no norm,
 * no shared expert. */
int oracle_moe(const uint16_t* x, const float* logits, int top_k,
               const uint8_t* w_gu, const uint8_t* w_down, int E, int64_t D,
               int64_t I, double* y, int32_t* ids, double* p) {
  if (!x || !logits || !w_gu || !w_down || !y || !ids || !p) return -1;
  if (E < 1 || top_k < 1 || top_k > E || D <= 0 || I <= 0 || D % 256 || I % 256)
    return -1;
  char* taken = (char*)calloc((size_t)E, 1);
  if (!taken) return -1;
  for (int s = 0; s < top_k; ++s) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || logits[e] > logits[best]) best = e;
    }
    taken[best] = 1;
    ids[s] = best;
  }
  double lmax = (double)logits[ids[0]];
  double z = 0.0;
  for (int s = 0; s < top_k; ++s) z += exp((double)logits[ids[s]] - lmax);
  for (int s = 0; s < top_k; ++s) p[s] = exp((double)logits[ids[s]] - lmax) / z;

  double* xd = decode_bf16_rows(x, 1, D);
  double* gu = (double*)malloc(sizeof(double) * (size_t)(2 * I));
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  double* ye = (double*)malloc(sizeof(double) * (size_t)D);
  int rc = (xd && gu && h && ye) ? 0 : -1;
  for (int64_t n = 0; n < D; ++n) y[n] = 0.0;
  const size_t gu_bytes = (size_t)(2 * I) * (size_t)(D / 256) * 144;
  const size_t dn_bytes = (size_t)D * (size_t)(I / 256) * 144;
  for (int e = 0; e < E && rc == 0; ++e) {
    if (!taken[e]) continue;
    double pe = 0.0;
    for (int s = 0; s < top_k; ++s)
      if (ids[s] == e) pe = p[s];
    rc = qgemv_q4k_f64x(xd, w_gu + (size_t)e * gu_bytes, 1, 2 * I, D, gu);
    if (rc) break;
    for (int64_t i = 0; i < I; ++i) h[i] = oracle_silu(gu[i]) * gu[I + i];
    rc = qgemv_q4k_f64x(h, w_down + (size_t)e * dn_bytes, 1, D, I, ye);
    if (rc) break;
    for (int64_t n = 0; n < D; ++n) y[n] += pe * ye[n];
  }
  free(taken);
  free(xd);
  free(gu);
  free(h);
  free(ye);
  return rc;
}

/* ---------------------------------------------------------------- O8 ---- */
/* Untied readout (uzu page, linear row: untied_readout) with greedy choice and
 * the verify rule of speculative decoding (uzu page, DFlash + Weaver section:
 * the target scores the proposal and keeps the longest matching path; Husky
 * page: an 8-token block is verified and the matching candidates are kept).
 * Readings: ties -> lowest index; a NaN logit counts as the maximum and the
 * first NaN wins; row i is compared with draft[i]. */
int oracle_lmhead(const uint16_t* x, const uint32_t* codes,
                  const uint16_t* scales, const uint16_t* biases, int M,
                  int64_t V, int64_t K, double* logits, int32_t* ids,
                  double* gap, const int32_t* draft, int32_t* accepted) {
  if (!x || !codes || !scales || !biases || !ids || M < 1 || V < 1 || K <= 0)
    return -1;
  double* xd = decode_bf16_rows(x, M, K);
  /* every logit (O3's dot product over ascending k), then the selection in
   * ascending v */
  double* L_all = logits ? logits : (double*)malloc(sizeof(double) * (size_t)M * (size_t)V);
  double* bestv = (double*)malloc(sizeof(double) * (size_t)M);
  double* second = (double*)malloc(sizeof(double) * (size_t)M);
  int64_t* best = (int64_t*)malloc(sizeof(int64_t) * (size_t)M);
  char* isnan_best = (char*)calloc((size_t)M, 1);
  int rc = (xd && L_all && bestv && second && best && isnan_best) ? 0 : -1;
  /* L_all[m][v]: the projection O3 with N = V */
  if (rc == 0) rc = oracle_qgemv_affine4_f64x(xd, codes, scales, biases, M, V, K, L_all);
  for (int m = 0; m < M && rc == 0; ++m) {
    best[m] = -1;
    bestv[m] = -INFINITY;
    second[m] = -INFINITY;
  }
  for (int64_t v = 0; v < V && rc == 0; ++v) {
    for (int m = 0; m < M; ++m) {
      double L = L_all[(int64_t)m * V + v];
      if (isnan_best[m]) continue;
      if (isnan(L)) {
        best[m] = v;
        isnan_best[m] = 1;
      } else if (best[m] < 0) {
        best[m] = v;
        bestv[m] = L;
      } else if (L > bestv[m]) {
        second[m] = bestv[m];
        best[m] = v;
        bestv[m] = L;
      } else if (L > second[m]) {
        second[m] = L;
      }
    }
  }
  if (rc == 0) {
    for (int m = 0; m < M; ++m) {
      ids[m] = (int32_t)best[m];
      if (gap) gap[m] = isnan_best[m] ? NAN : bestv[m] - second[m];
    }
    if (accepted) {
      int32_t a = 0;
      if (draft)
        while (a < M && ids[a] == draft[a]) ++a;
      *accepted = a;
    }
  }
  free(xd);
  if (L_all != logits) free(L_all);
  free(bestv);
  free(second);
  free(best);
  free(isnan_best);
  return rc;
}

/* O9: all logits of the row in fp64 (O8's dot product), then k rounds of
 * "the best not yet chosen" under the order stated in oracle.h. */
static int topk_beats(double a, int64_t ia, double b, int64_t ib) {
  /* does (a, ia) come before (b, ib)? */
  const int na = isnan(a), nb = isnan(b);
  if (na || nb) {
    if (na && nb) return ia < ib;
    return na;
  }
  if (a != b) return a > b;
  return ia < ib;
}

int oracle_lmhead_topk(const uint16_t* x, const uint32_t* codes,
                       const uint16_t* scales, const uint16_t* biases, int M,
                       int64_t V, int64_t K, int k, int32_t* ids,
                       double* vals) {
  if (!x || !codes || !scales || !biases || !ids || M < 1 || V < 1 || K <= 0 ||
      k < 1 || k > V)
    return -1;
  double* xd = decode_bf16_rows(x, M, K);
  double* wrow = (double*)malloc(sizeof(double) * (size_t)K);
  double* L = (double*)malloc(sizeof(double) * (size_t)M * (size_t)V);
  char* taken = (char*)malloc((size_t)V);
  int rc = (xd && wrow && L && taken) ? 0 : -1;
  for (int64_t v = 0; v < V && rc == 0; ++v) {
    rc = oracle_dequant_affine4(codes, scales, biases, V, K, v, 1, wrow);
    if (rc) break;
    for (int m = 0; m < M; ++m) L[(int64_t)m * V + v] = dot_asc(xd + (int64_t)m * K, wrow, K);
  }
  for (int m = 0; m < M && rc == 0; ++m) {
    const double* row = L + (int64_t)m * V;
    memset(taken, 0, (size_t)V);
    for (int j = 0; j < k; ++j) {
      int64_t best = -1;
      for (int64_t v = 0; v < V; ++v) {
        if (taken[v]) continue;
        if (best < 0 || topk_beats(row[v], v, row[best], best)) best = v;
      }
      taken[best] = 1;
      ids[(int64_t)m * k + j] = (int32_t)best;
      if (vals) vals[(int64_t)m * k + j] = row[best];
    }
  }
  free(xd);
  free(wrow);
  free(L);
  free(taken);
  return rc;
}

/* --------------------------------------------------------------- O10 ---- */

static int popcount_u32(uint32_t v) {
  int c = 0;
  while (v) {
    c += (int)(v & 1u);
    v >>= 1;
  }
  return c;
}

int oracle_rht(const uint16_t* x, const int8_t* signs, int had, int M,
               int64_t K, double* xr) {
  if (!x || !signs || !xr || M < 1 || K <= 0 || had < 1) return -1;
  if ((had & (had - 1)) != 0 || K % had != 0) return -1;
  double* sx = (double*)malloc(sizeof(double) * (size_t)had);
  if (!sx) return -1;
  const double norm = 1.0 / sqrt((double)had);
  for (int m = 0; m < M; ++m) {
    for (int64_t b = 0; b < K / had; ++b) {
      const int64_t k0 = b * had;
      for (int j = 0; j < had; ++j) {
        const double v = o_bf16_to_f64(x[(int64_t)m * K + k0 + j]);
        sx[j] = signs[k0 + j] < 0 ? -v : v;
      }
      for (int i = 0; i < had; ++i) {
        double acc = 0.0; /* the plain matrix-vector product, j ascending */
        for (int j = 0; j < had; ++j) {
          const double h = (popcount_u32((uint32_t)(i & j)) & 1) ? -1.0 : 1.0;
          acc += h * sx[j];
        }
        xr[(int64_t)m * K + k0 + i] = acc * norm;
      }
    }
  }
  free(sx);
  return 0;
}

int oracle_qgemv_affine4_rht(const uint16_t* x, const int8_t* signs, int had,
                             const uint32_t* codes, const uint16_t* scales,
                             const uint16_t* biases, int M, int64_t N,
                             int64_t K, double* y) {
  if (M < 1 || K <= 0) return -1;
  double* xr = (double*)malloc(sizeof(double) * (size_t)M * (size_t)K);
  if (!xr) return -1;
  int rc = oracle_rht(x, signs, had, M, K, xr);
  if (rc == 0) rc = oracle_qgemv_affine4_f64x(xr, codes, scales, biases, M, N, K, y);
  free(xr);
  return rc;
}

/* ---------------------------------------------------------------- O12 --- */
/* Affine 8-bit, group 64 along K (the uzu page's weight_matrix row names MLX
 * 4- and 8-bit quantized weights).  Reading, the 8-bit twin of O1: code k of
 * row n is byte k%4 (least significant first) of word k/4 of that row, an
 * unsigned value 0..255; the weight is scale*code + bias with the bf16 scale
 * and bias of group k/64. */
int oracle_dequant_affine8(const uint32_t* codes, const uint16_t* scales,
                           const uint16_t* biases, int64_t N, int64_t K,
                           int64_t n0, int64_t nr, double* w) {
  if (!codes || !scales || !biases || !w) return -1;
  if (N < 0 || K <= 0 || K % 64 != 0 || n0 < 0 || nr < 0 || n0 + nr > N)
    return -1;
  const int64_t words = K / 4, groups = K / 64;
  for (int64_t r = 0; r < nr; ++r) {
    const int64_t n = n0 + r;
    for (int64_t k = 0; k < K; ++k) {
      uint32_t word = codes[n * words + k / 4];
      unsigned q = (unsigned)((word >> (8 * (k % 4))) & 255u);
      double s = o_bf16_to_f64(scales[n * groups + k / 64]);
      double b = o_bf16_to_f64(biases[n * groups + k / 64]);
      w[r * K + k] = s * (double)q + b;
    }
  }
  return 0;
}

/* ---------------------------------------------------------------- O13 --- */
/* O3 on affine-8 weights: y[m][n] = sum_k x[m][k] * w[n][k], ascending k. */
int oracle_qgemv_affine8(const uint16_t* x, const uint32_t* codes,
                         const uint16_t* scales, const uint16_t* biases, int M,
                         int64_t N, int64_t K, double* y) {
  if (!x || !y || M < 1 || N < 0 || K <= 0) return -1;
  double* xd = decode_bf16_rows(x, M, K);
  if (!xd) return -1;
  double* wrow = (double*)malloc(sizeof(double) * (size_t)K);
  if (!wrow) {
    free(xd);
    return -1;
  }
  int rc = 0;
  for (int64_t n = 0; n < N && rc == 0; ++n) {
    rc = oracle_dequant_affine8(codes, scales, biases, N, K, n, 1, wrow);
    for (int m = 0; m < M && rc == 0; ++m) y[(int64_t)m * N + n] = dot_asc(xd + (int64_t)m * K, wrow, K);
  }
  free(wrow);
  free(xd);
  return rc;
}

/* ---------------------------------------------------------------- O14 --- */
/* GGUF Q6_K (Q4_K_M files mix it in; the pages do not print the layout).
 * Reading -- the public 210-byte block of 256 weights:
 *   bytes 0-127 ql (low 4 bits), 128-191 qh (high 2 bits), 192-207 sixteen
 *   int8 scales (one per 16 weights), 208-209 d (fp16).
 *   Weight o of the block: half h = o/128, quarter j = (o%128)/32, l = o%32;
 *   its low bits are the low nibble of ql[64h + 32*(j%2) + l] for j < 2 and
 *   the high nibble for j >= 2; its high bits are bits 2j, 2j+1 of
 *   qh[32h + l]; q = (low | high << 4) - 32 and the weight is d * sc[o/16] * q. */
int oracle_dequant_q6k(const uint8_t* blocks, int64_t N, int64_t K, int64_t n0,
                       int64_t nr, double* w) {
  if (!blocks || !w) return -1;
  if (N < 0 || K <= 0 || K % 256 != 0 || n0 < 0 || nr < 0 || n0 + nr > N) return -1;
  const int64_t nb = K / 256;
  for (int64_t r = 0; r < nr; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t* blk = blocks + ((n0 + r) * nb + b) * 210;
      const uint8_t* ql = blk;
      const uint8_t* qh = blk + 128;
      const int8_t* sc = (const int8_t*)(blk + 192);
      const double d = o_f16_to_f64((uint16_t)(blk[208] | (blk[209] << 8)));
      for (int o = 0; o < 256; ++o) {
        const int h = o / 128, j = (o % 128) / 32, l = o % 32;
        const unsigned lb = ql[64 * h + 32 * (j % 2) + l];
        const unsigned lo = (j < 2) ? (lb & 15u) : (lb >> 4);
        const unsigned hi = (qh[32 * h + l] >> (2 * j)) & 3u;
        const int q = (int)(lo | (hi << 4)) - 32;
        w[r * K + b * 256 + o] = d * (double)sc[o / 16] * (double)q;
      }
    }
  }
  return 0;
}

/* ---------------------------------------------------------------- O15 --- */
/* O3 on Q6_K weights: y[m][n] = sum_k x[m][k] * w[n][k], ascending k. */
int oracle_qgemv_q6k(const uint16_t* x, const uint8_t* blocks, int M, int64_t N,
                     int64_t K, double* y) {
  if (!x || !y || M < 1 || N < 0 || K <= 0) return -1;
  double* xd = decode_bf16_rows(x, M, K);
  if (!xd) return -1;
  double* wrow = (double*)malloc(sizeof(double) * (size_t)K);
  if (!wrow) {
    free(xd);
    return -1;
  }
  int rc = 0;
  for (int64_t n = 0; n < N && rc == 0; ++n) {
    rc = oracle_dequant_q6k(blocks, N, K, n, 1, wrow);
    for (int m = 0; m < M && rc == 0; ++m) y[(int64_t)m * N + n] = dot_asc(xd + (int64_t)m * K, wrow, K);
  }
  free(wrow);
  free(xd);
  return rc;
}
