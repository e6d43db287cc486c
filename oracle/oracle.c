/*
 * oracle.c -- plain fp64 CPU oracle for sparse causal attention over a fixed
 * per-query neighbour graph.  TEST INFRASTRUCTURE ONLY (see oracle.h): only
 * the tests, the smoke check and the CPU-baseline leg of the benchmark use it.
 * It shares no code with the HIP path.
 *
 * Readings of the pages this file implements (each also listed with the
 * design notes):
 *  - the window {i-W+1, ..., i} contains the query itself (MiniGPT Part 6,
 *    "A mask is not enough": the mask keeps j with j <= i and i - j < w);
 *  - a long-range offset d adds key i - d when i - d >= 0; keys before the
 *    start are dropped, never clamped (SpatialLM-Mini news page, "How tokens
 *    choose whom to listen to": no look-ahead, fixed list of distances);
 *  - the neighbour set is a set: a distance listed twice, or an offset that
 *    falls inside the window, contributes its key once;
 *  - the weights are a softmax over the neighbour set only (same section: the
 *    distribution of attention within the fixed list depends on the text).
 *
 * Arithmetic: IEEE double, ascending key order, two-pass softmax (max, then
 * sum of exponentials), exp and log from libm.  No blocking or fusion.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact upcast of one stored element to double. */
static double rd(const void* base, int dtype, int64_t idx) {
  if (dtype == ORACLE_F64) return ((const double*)base)[idx];
  if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
  /* bf16: the stored 16 bits are the top half of an IEEE binary32 */
  uint32_t u = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static int cmp_i64(const void* a, const void* b) {
  int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
  return (x > y) - (x < y);
}

static int bad_graph_args(int64_t T, int64_t W, const int64_t* offs, int32_t n_offs) {
  if (T < 1 || W < 1 || n_offs < 0 || (n_offs > 0 && !offs)) return 1;
  for (int32_t t = 0; t < n_offs; ++t)
    if (offs[t] < 0) return 1; /* a negative distance would look ahead */
  return 0;
}

static int64_t row_cap(int64_t T, int64_t W, int32_t n_offs) {
  return (W < T ? W : T) + n_offs;
}

/* N(i) = { i - delta : delta in {0, ..., W-1} U offsets, i - delta >= 0 },
 * built literally as a set: collect every candidate key, sort, drop repeats.
 * (SpatialLM-Mini news page, "How tokens choose whom to listen to"; MiniGPT
 * Part 6, "A mask is not enough", window predicate.) */
int64_t oracle_row(int64_t T, int64_t W, const int64_t* offs, int32_t n_offs,
                   int64_t i, int64_t* out) {
  if (bad_graph_args(T, W, offs, n_offs) || i < 0 || i >= T || !out) return -1;
  int64_t n = 0;
  for (int64_t delta = 0; delta < W && delta <= i; ++delta) out[n++] = i - delta;
  for (int32_t t = 0; t < n_offs; ++t)
    if (i - offs[t] >= 0) out[n++] = i - offs[t];
  qsort(out, (size_t)n, sizeof(int64_t), cmp_i64);
  int64_t u = 0;
  for (int64_t t = 0; t < n; ++t)
    if (u == 0 || out[t] != out[u - 1]) out[u++] = out[t];
  return u;
}

int64_t oracle_graph_csr(int64_t T, int64_t W, const int64_t* offs, int32_t n_offs,
                         int64_t r0, int64_t r1, int64_t* row_ptr, int64_t* cols,
                         int64_t cols_cap) {
  if (bad_graph_args(T, W, offs, n_offs) || r0 < 0 || r1 < r0 || r1 > T || !row_ptr)
    return -1;
  int64_t* buf = (int64_t*)malloc(sizeof(int64_t) * (size_t)row_cap(T, W, n_offs));
  if (!buf) return -1;
  int64_t e = 0;
  row_ptr[0] = 0;
  for (int64_t i = r0; i < r1; ++i) {
    int64_t n = oracle_row(T, W, offs, n_offs, i, buf);
    if (cols && e + n <= cols_cap) memcpy(cols + e, buf, sizeof(int64_t) * (size_t)n);
    e += n;
    row_ptr[i - r0 + 1] = e;
  }
  free(buf);
  if (e > cols_cap || !cols) return -(e + 2);
  return e;
}

/* Score of edge (i, j).
 * Dot mode: s = scale * <q_i, k_j> (scaled dot product; the scale is a
 * parameter of the chunked_swa listing in MiniGPT Part 6, 1/sqrt(D) by
 * default).
 * Coordinate mode: s = -gamma * ||c_q,i - c_k,j||^2 + beta (SpatialLM-Mini
 * news page, "How tokens choose whom to listen to": learnable 3-D query and
 * key coordinates, nearer pairs weigh more, extra learnable parameters adjust
 * the score; gamma and beta are those parameters). */
static double score(int mode, int64_t D, double scale, int dtype, const void* q,
                    const void* k, int cdtype, const void* cq, const void* ck,
                    double gamma, double beta, int64_t i, int64_t j) {
  /* Uniform mode: one score for every admissible neighbour, so each of the
   * |N(i)| neighbours gets weight 1 / |N(i)| (SpatialLM-Mini news page, "What
   * to check before adopting it in your project": the same graph with fixed
   * weights). */
  if (mode == ORACLE_SCORE_UNIFORM) return 0.0;
  if (mode == ORACLE_SCORE_DOT) {
    double acc = 0.0;
    for (int64_t d = 0; d < D; ++d) acc += rd(q, dtype, i * D + d) * rd(k, dtype, j * D + d);
    return scale * acc;
  }
  double r2 = 0.0;
  for (int c = 0; c < 3; ++c) {
    double diff = rd(cq, cdtype, i * 3 + c) - rd(ck, cdtype, j * 3 + c);
    r2 += diff * diff;
  }
  return -gamma * r2 + beta;
}

static int bad_attn_args(int64_t T, int64_t D, int mode, const void* q, const void* k,
                         const void* v, const void* cq, const void* ck) {
  if (D < 1 || !v) return 1;
  if (mode == ORACLE_SCORE_DOT) return !q || !k;
  if (mode == ORACLE_SCORE_COORD) return !cq || !ck;
  if (mode == ORACLE_SCORE_UNIFORM) return 0;
  (void)T;
  return 1;
}

/* Softmax over the neighbour set only, then the weighted sum of values:
 *   m_i = max_j s_ij,  l_i = sum_j exp(s_ij - m_i),  LSE_i = m_i + ln l_i,
 *   P_ij = exp(s_ij - m_i) / l_i,  O_i = sum_j P_ij v_j.
 * (SpatialLM-Mini news page, "How tokens choose whom to listen to".)
 * One row i with neighbour list nb[0 .. n); s is scratch of n doubles. */
static void fwd_row(int64_t D, int score_mode, double scale, int dtype, const void* q,
                    const void* k, const void* v, int cdtype, const void* cq, const void* ck,
                    double gamma, double beta, int64_t i, const int64_t* nb, int64_t n,
                    double* s, double* O_row, double* LSE_out) {
  for (int64_t t = 0; t < n; ++t)
    s[t] = score(score_mode, D, scale, dtype, q, k, cdtype, cq, ck, gamma, beta, i, nb[t]);
  double m = -INFINITY;
  for (int64_t t = 0; t < n; ++t)
    if (s[t] > m) m = s[t];
  double l = 0.0;
  for (int64_t t = 0; t < n; ++t) l += exp(s[t] - m);
  *LSE_out = m + log(l);
  for (int64_t d = 0; d < D; ++d) O_row[d] = 0.0;
  for (int64_t t = 0; t < n; ++t) {
    const double p = exp(s[t] - m) / l;
    for (int64_t d = 0; d < D; ++d) O_row[d] += p * rd(v, dtype, nb[t] * D + d);
  }
}

int oracle_fwd(int64_t T, int64_t D, int64_t W, const int64_t* offs, int32_t n_offs,
               int score_mode, double scale, int dtype, const void* q, const void* k,
               const void* v, int cdtype, const void* cq, const void* ck, double gamma,
               double beta, const int64_t* rows, int64_t n_rows, double* O, double* LSE) {
  if (bad_graph_args(T, W, offs, n_offs) || bad_attn_args(T, D, score_mode, q, k, v, cq, ck))
    return -1;
  if (!rows) n_rows = T;
  if (n_rows < 0 || !O || !LSE) return -1;
  if (rows)
    for (int64_t r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= T) return -1;
  const int64_t cap = row_cap(T, W, n_offs);
  int failed = 0;
#pragma omp parallel
  {
    int64_t* nb = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
    double* s = (double*)malloc(sizeof(double) * (size_t)cap);
    if (!nb || !s) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 64)
      for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t i = rows ? rows[r] : r;
        const int64_t n = oracle_row(T, W, offs, n_offs, i, nb);
        fwd_row(D, score_mode, scale, dtype, q, k, v, cdtype, cq, ck, gamma, beta, i, nb, n, s,
                O + r * D, LSE + r);
      }
    }
    free(nb);
    free(s);
  }
  return failed ? -2 : 0;
}

/* An explicit graph: row i lists its keys cols[row_ptr[i] .. row_ptr[i+1]),
 * strictly ascending, each 0 <= j <= i, at least one per row (a softmax over
 * an empty list is undefined). */
static int bad_csr(int64_t T, const int64_t* row_ptr, const int64_t* cols) {
  if (T < 1 || !row_ptr || row_ptr[0] != 0) return 1;
  for (int64_t i = 0; i < T; ++i) {
    if (row_ptr[i + 1] <= row_ptr[i]) return 1;
    for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
      if (!cols || cols[e] < 0 || cols[e] > i) return 1;
      if (e > row_ptr[i] && cols[e] <= cols[e - 1]) return 1;
    }
  }
  return 0;
}

int oracle_fwd_csr(int64_t T, int64_t D, const int64_t* row_ptr, const int64_t* cols,
                   int score_mode, double scale, int dtype, const void* q, const void* k,
                   const void* v, int cdtype, const void* cq, const void* ck, double gamma,
                   double beta, double* O, double* LSE) {
  if (bad_csr(T, row_ptr, cols) || bad_attn_args(T, D, score_mode, q, k, v, cq, ck) || !O || !LSE)
    return -1;
  int64_t cap = 1;
  for (int64_t i = 0; i < T; ++i)
    if (row_ptr[i + 1] - row_ptr[i] > cap) cap = row_ptr[i + 1] - row_ptr[i];
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)cap);
    if (!s) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 64)
      for (int64_t i = 0; i < T; ++i)
        fwd_row(D, score_mode, scale, dtype, q, k, v, cdtype, cq, ck, gamma, beta, i,
                cols + row_ptr[i], row_ptr[i + 1] - row_ptr[i], s, O + i * D, LSE + i);
    }
    free(s);
  }
  return failed ? -2 : 0;
}

/* Backward of L = sum_i <dO_i, O_i> through the forward above, by the chain
 * rule over the edges of the graph:
 *   dP_ij = <dO_i, v_j>,  Delta_i = sum_j P_ij dP_ij,
 *   dS_ij = P_ij (dP_ij - Delta_i),
 *   dot mode:   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
 *   both modes: dV_j = sum_i P_ij dO_i,
 *   coordinate: dcq_i = sum_j dS_ij (-2 gamma)(c_q,i - c_k,j),
 *               dck_j = sum_i dS_ij ( 2 gamma)(c_q,i - c_k,j),
 *               dgamma = -sum_ij dS_ij ||c_q,i - c_k,j||^2,  dbeta = sum_ij dS_ij.
 * Sums over i for a fixed key j run over the transposed edge list, so every
 * output row has one writer. */
/* The backward over an explicit graph (row_ptr, cols as in oracle_fwd_csr);
 * the distance-graph backward below builds its lists and calls this. */
int oracle_bwd_csr(int64_t T, int64_t D, const int64_t* row_ptr, const int64_t* cols,
                   int score_mode, double scale, int dtype, const void* q, const void* k,
                   const void* v, int cdtype, const void* cq, const void* ck, double gamma,
                   double beta, const void* dO, double* dQ, double* dK, double* dV,
                   double* dcq, double* dck, double* dgamma, double* dbeta, double* l1) {
  if (bad_csr(T, row_ptr, cols) || bad_attn_args(T, D, score_mode, q, k, v, cq, ck) || !dO)
    return -1;
  int rc = -2;
  const int64_t E = row_ptr[T];
  int64_t* col_cnt = (int64_t*)calloc((size_t)(T + 1), sizeof(int64_t));
  int64_t* tptr = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T + 1));
  int64_t* tedge = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  int64_t* erow = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  double* P = (double*)malloc(sizeof(double) * (size_t)E);
  double* dS = (double*)malloc(sizeof(double) * (size_t)E);
  double* Delta = (double*)malloc(sizeof(double) * (size_t)T);
  if (!col_cnt || !tptr || !tedge || !erow || !P || !dS || !Delta) goto done;

  /* 2. per row: scores, softmax, dP, Delta, dS (stored per edge) */
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t i = 0; i < T; ++i) {
    const int64_t e0 = row_ptr[i], e1 = row_ptr[i + 1];
    double m = -INFINITY;
    for (int64_t e = e0; e < e1; ++e) {
      erow[e] = i;
      P[e] = score(score_mode, D, scale, dtype, q, k, cdtype, cq, ck, gamma, beta, i, cols[e]);
      if (P[e] > m) m = P[e];
    }
    double l = 0.0;
    for (int64_t e = e0; e < e1; ++e) l += exp(P[e] - m);
    for (int64_t e = e0; e < e1; ++e) P[e] = exp(P[e] - m) / l;
    double delta = 0.0;
    for (int64_t e = e0; e < e1; ++e) {
      double dp = 0.0;
      for (int64_t d = 0; d < D; ++d) dp += rd(dO, dtype, i * D + d) * rd(v, dtype, cols[e] * D + d);
      dS[e] = dp; /* dP for now */
      delta += P[e] * dp;
    }
    Delta[i] = delta;
    for (int64_t e = e0; e < e1; ++e) dS[e] = P[e] * (dS[e] - delta);
  }

  /* 3. gradients with respect to the query side, per row */
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t i = 0; i < T; ++i) {
    const int64_t e0 = row_ptr[i], e1 = row_ptr[i + 1];
    if (score_mode == ORACLE_SCORE_DOT && dQ) {
      for (int64_t d = 0; d < D; ++d) dQ[i * D + d] = 0.0;
      for (int64_t e = e0; e < e1; ++e)
        for (int64_t d = 0; d < D; ++d) dQ[i * D + d] += dS[e] * rd(k, dtype, cols[e] * D + d);
      for (int64_t d = 0; d < D; ++d) dQ[i * D + d] *= scale;
    }
    if (score_mode == ORACLE_SCORE_COORD && dcq) {
      for (int c = 0; c < 3; ++c) dcq[i * 3 + c] = 0.0;
      for (int64_t e = e0; e < e1; ++e)
        for (int c = 0; c < 3; ++c) {
          const double diff = rd(cq, cdtype, i * 3 + c) - rd(ck, cdtype, cols[e] * 3 + c);
          dcq[i * 3 + c] += dS[e] * (-2.0 * gamma) * diff;
        }
    }
  }

  /* 4. transpose the edge list (counting sort by key index, stable in i) */
  for (int64_t e = 0; e < row_ptr[T]; ++e) col_cnt[cols[e] + 1]++;
  tptr[0] = 0;
  for (int64_t j = 0; j < T; ++j) tptr[j + 1] = tptr[j] + col_cnt[j + 1];
  for (int64_t j = 0; j < T; ++j) col_cnt[j] = tptr[j];
  for (int64_t e = 0; e < row_ptr[T]; ++e) tedge[col_cnt[cols[e]]++] = e;

  /* 5. gradients with respect to the key side, per key */
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t j = 0; j < T; ++j) {
    if (dV) {
      for (int64_t d = 0; d < D; ++d) dV[j * D + d] = 0.0;
      for (int64_t t = tptr[j]; t < tptr[j + 1]; ++t) {
        const int64_t e = tedge[t], i = erow[e];
        for (int64_t d = 0; d < D; ++d) dV[j * D + d] += P[e] * rd(dO, dtype, i * D + d);
      }
    }
    if (score_mode == ORACLE_SCORE_DOT && dK) {
      for (int64_t d = 0; d < D; ++d) dK[j * D + d] = 0.0;
      for (int64_t t = tptr[j]; t < tptr[j + 1]; ++t) {
        const int64_t e = tedge[t], i = erow[e];
        for (int64_t d = 0; d < D; ++d) dK[j * D + d] += dS[e] * rd(q, dtype, i * D + d);
      }
      for (int64_t d = 0; d < D; ++d) dK[j * D + d] *= scale;
    }
    if (score_mode == ORACLE_SCORE_COORD && dck) {
      for (int c = 0; c < 3; ++c) dck[j * 3 + c] = 0.0;
      for (int64_t t = tptr[j]; t < tptr[j + 1]; ++t) {
        const int64_t e = tedge[t], i = erow[e];
        for (int c = 0; c < 3; ++c) {
          const double diff = rd(cq, cdtype, i * 3 + c) - rd(ck, cdtype, j * 3 + c);
          dck[j * 3 + c] += dS[e] * (2.0 * gamma) * diff;
        }
      }
    }
  }

  /* 6. per-head parameter gradients, summed over edges in edge order */
  if (score_mode == ORACLE_SCORE_COORD) {
    double g = 0.0, b = 0.0, mass = 0.0;
    for (int64_t e = 0; e < row_ptr[T]; ++e) {
      const int64_t i = erow[e], j = cols[e];
      double r2 = 0.0;
      for (int c = 0; c < 3; ++c) {
        const double diff = rd(cq, cdtype, i * 3 + c) - rd(ck, cdtype, j * 3 + c);
        r2 += diff * diff;
      }
      g += -dS[e] * r2;
      b += dS[e];
      mass += fabs(dS[e]) * (1.0 + r2);
    }
    if (dgamma) *dgamma = g;
    if (dbeta) *dbeta = b;
    if (l1) *l1 = mass;
  }
  (void)beta;
  rc = 0;

done:
  free(col_cnt);
  free(erow);
  free(P);
  free(dS);
  free(tedge);
  free(tptr);
  free(Delta);
  return rc;
}

int oracle_bwd(int64_t T, int64_t D, int64_t W, const int64_t* offs, int32_t n_offs,
               int score_mode, double scale, int dtype, const void* q, const void* k,
               const void* v, int cdtype, const void* cq, const void* ck, double gamma,
               double beta, const void* dO, double* dQ, double* dK, double* dV,
               double* dcq, double* dck, double* dgamma, double* dbeta, double* l1) {
  if (bad_graph_args(T, W, offs, n_offs) ||
      bad_attn_args(T, D, score_mode, q, k, v, cq, ck) || !dO)
    return -1;
  /* the graph, row by row, then the explicit-list backward */
  int64_t* row_ptr = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T + 1));
  if (!row_ptr) return -2;
  const int64_t E = -(oracle_graph_csr(T, W, offs, n_offs, 0, T, row_ptr, NULL, 0) + 2);
  int64_t* cols = E >= 0 ? (int64_t*)malloc(sizeof(int64_t) * (size_t)(E > 0 ? E : 1)) : NULL;
  int rc = -2;
  if (cols && oracle_graph_csr(T, W, offs, n_offs, 0, T, row_ptr, cols, E) == E)
    rc = oracle_bwd_csr(T, D, row_ptr, cols, score_mode, scale, dtype, q, k, v, cdtype, cq, ck,
                        gamma, beta, dO, dQ, dK, dV, dcq, dck, dgamma, dbeta, l1);
  free(row_ptr);
  free(cols);
  return rc;
}

/* Causal attention over every key j <= i, ascending j: the result the
 * windowed op must equal exactly once W >= T (MiniGPT Part 6, "A mask is not
 * enough", the claim after the chunked_swa listing). */
int oracle_dense_causal(int64_t T, int64_t D, double scale, int dtype, const void* q,
                        const void* k, const void* v, double* O, double* LSE) {
  if (T < 1 || D < 1 || !q || !k || !v || !O || !LSE) return -1;
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)T);
    if (!s) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t i = 0; i < T; ++i) {
        double m = -INFINITY;
        for (int64_t j = 0; j <= i; ++j) {
          double acc = 0.0;
          for (int64_t d = 0; d < D; ++d) acc += rd(q, dtype, i * D + d) * rd(k, dtype, j * D + d);
          s[j] = scale * acc;
          if (s[j] > m) m = s[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j <= i; ++j) l += exp(s[j] - m);
        LSE[i] = m + log(l);
        for (int64_t d = 0; d < D; ++d) O[i * D + d] = 0.0;
        for (int64_t j = 0; j <= i; ++j) {
          const double p = exp(s[j] - m) / l;
          for (int64_t d = 0; d < D; ++d) O[i * D + d] += p * rd(v, dtype, j * D + d);
        }
      }
    }
    free(s);
  }
  return failed ? -2 : 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
