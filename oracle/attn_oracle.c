/*
 * Plain fp64 CPU oracle for exact softmax attention: the forward, and its gradients
 * (oracle_attn_bwd_f64 near the end of the file).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load
 * this file or the library built from it; only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg do. It shares no code with the HIP path.
 *
 * What it computes (the definition, written out, no tiling and no online update):
 *   For one (batch, head) slice with Q in R^{Nq x d}, K, V in R^{Nk x d} and a
 *   positive scale s:
 *       x_ij = sum_c Q[i,c] K[j,c]                  raw score, S = Q K^T
 *       P_i. = softmax over the valid keys j of s*x_ij
 *       O_i. = sum_j P_ij V[j,.]
 *       LSE_i = ln sum_{valid j} exp(s*x_ij)
 *   Sources: "用 CuTe 读懂 FlashAttention" (blog.qingsen.net), the notation block
 *   that defines S = QK^T, P = softmax_row(sS), O = PV, s = 1/sqrt(D), and its final
 *   section ("最后：归一化并写回 O"), which defines LSE = s*m + log(l) with m the
 *   raw (unscaled) row maximum and checks it against log(sum(exp(s*S))); "CUDA
 *   算子工程" ch. 14 §14.1 (the scaled dot-product definition).
 *
 * Safe softmax in three passes over the stored score row (max, exponential sum,
 * weighted sum of V), as the pwwt.cn FlashAttention-forward notes §3.1 and
 * ch. 14 §14.2 describe the naive softmax. With z_j = s*x_j and m = max z_j,
 *   l = sum exp(z_j - m),  O = (sum exp(z_j - m) V_j) / l,  LSE = m + ln l,
 * which equals s*m_raw + ln l of the blog's final section because s > 0.
 *
 * Causal masking (argument `causal`): 0 = none; 1 = top-left aligned, key j is
 * valid for query i iff j <= i (the blog's causal section, Fig. 11); 2 =
 * bottom-right aligned, key j valid iff j <= i + Nk - Nq, the other alignment that
 * section names as differing from top-left only when the query and key lengths
 * differ (the last query sees every key). A row with no valid key (Nk = 0, or
 * bottom-right with i < Nq - Nk) gets O = 0 and LSE = -inf (the limit of an
 * empty sum; the pages leave the case open).
 *
 * Arithmetic: IEEE double, libm exp/log, compiled without fast-math, so the
 * sums are evaluated strictly in loop order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One output row. z is caller scratch of length Nk. Returns nothing; writes
 * o_row[0..d) and *lse_out. */
static void oracle_one_row(const double* q_row, const double* k, const double* v,
                           int64_t Nq, int64_t Nk, int64_t d, double scale, int causal,
                           int64_t i, double* z, double* o_row, double* lse_out) {
  int64_t nvalid = Nk;
  if (causal == 1) nvalid = (i + 1 < Nk) ? (i + 1) : Nk;   /* keys 0..i are valid */
  if (causal == 2) {                                       /* keys 0..i+Nk-Nq are valid */
    const int64_t last = i + Nk - Nq;
    nvalid = (last + 1 < Nk) ? (last + 1) : Nk;
  }
  if (nvalid <= 0) {
    for (int64_t c = 0; c < d; ++c) o_row[c] = 0.0;
    *lse_out = -INFINITY;
    return;
  }
  /* scores z_j = s * (q . k_j) over the valid keys */
  for (int64_t j = 0; j < nvalid; ++j) {
    const double* k_row = k + j * d;
    double x = 0.0;
    for (int64_t c = 0; c < d; ++c) x += q_row[c] * k_row[c];
    z[j] = scale * x;
  }
  /* pass 1: row maximum */
  double m = z[0];
  for (int64_t j = 1; j < nvalid; ++j)
    if (z[j] > m) m = z[j];
  /* pass 2: sum of exponentials relative to the maximum */
  double l = 0.0;
  for (int64_t j = 0; j < nvalid; ++j) l += exp(z[j] - m);
  /* pass 3: normalised weights times V */
  for (int64_t c = 0; c < d; ++c) o_row[c] = 0.0;
  for (int64_t j = 0; j < nvalid; ++j) {
    double p = exp(z[j] - m) / l;
    const double* v_row = v + j * d;
    for (int64_t c = 0; c < d; ++c) o_row[c] += p * v_row[c];
  }
  *lse_out = m + log(l);
}

static int oracle_check_args(const void* q, const void* k, const void* v, const void* o,
                             const void* lse, int64_t BH, int64_t Nq, int64_t Nk, int64_t d,
                             double scale, int causal) {
  if (BH < 0 || Nq < 0 || Nk < 0 || d < 0) return 2;
  if (!(scale > 0.0) || !isfinite(scale)) return 3;
  if (causal < 0 || causal > 2) return 6;
  if (BH * Nq == 0) return 0;
  if (!q || !o || !lse) return 1;
  if (Nk > 0 && (!k || !v)) return 1;
  return 0;
}

/* Full forward over every row.
 * q: [BH, Nq, d], k, v: [BH, Nk, d], o: [BH, Nq, d], lse: [BH, Nq]; all row-major
 * contiguous doubles, owned by the caller. causal: 0, 1 (top-left) or 2
 * (bottom-right). Returns 0 on success, 1 for a null pointer, 2 for a negative
 * size, 3 for a scale that is not finite and > 0, 4 when scratch memory cannot be
 * allocated, 6 for an unknown causal mode. */
int oracle_attn_fwd_f64(const double* q, const double* k, const double* v, double* o,
                        double* lse, int64_t BH, int64_t Nq, int64_t Nk, int64_t d,
                        double scale, int causal) {
  int rc = oracle_check_args(q, k, v, o, lse, BH, Nq, Nk, d, scale, causal);
  if (rc || BH * Nq == 0) return rc;
  int fail = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
    if (!z) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 8)
      for (int64_t r = 0; r < BH * Nq; ++r) {
        int64_t bh = r / Nq, i = r % Nq;
        oracle_one_row(q + r * d, k + bh * Nk * d, v + bh * Nk * d, Nq, Nk, d, scale, causal, i, z,
                       o + r * d, lse + r);
      }
      free(z);
    }
  }
  return fail ? 4 : 0;
}

/* Selected rows only. rows[t] is a flat row index bh*Nq + i in [0, BH*Nq);
 * o_rows: [nrows, d], lse_rows: [nrows]. Same return codes, plus 5 for a row
 * index out of range. */
int oracle_attn_rows_f64(const double* q, const double* k, const double* v, int64_t BH,
                         int64_t Nq, int64_t Nk, int64_t d, double scale, int causal,
                         const int64_t* rows, int64_t nrows, double* o_rows, double* lse_rows) {
  int rc = oracle_check_args(q, k, v, o_rows, lse_rows, BH, Nq, Nk, d, scale, causal);
  if (rc) return rc;
  if (nrows <= 0) return 0;
  if (!rows) return 1;
  for (int64_t t = 0; t < nrows; ++t)
    if (rows[t] < 0 || rows[t] >= BH * Nq) return 5;
  int fail = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
    if (!z) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t t = 0; t < nrows; ++t) {
        int64_t r = rows[t];
        int64_t bh = r / Nq, i = r % Nq;
        oracle_one_row(q + r * d, k + bh * Nk * d, v + bh * Nk * d, Nq, Nk, d, scale, causal, i, z,
                       o_rows + t * d, lse_rows + t);
      }
      free(z);
    }
  }
  return fail ? 4 : 0;
}

/*
 * Backward pass: the gradients of a scalar loss L with respect to Q, K and V, given
 * dO = dL/dO, for the forward defined at the top of this file.
 *
 * The pages define only the forward; "CUDA 算子工程" ch. 14 §14.5 says its LSE
 * output exists for the backward pass and §14.7 gives the backward's loop order.
 * The gradients are the forward definition differentiated (chain rule), per row i
 * over its valid keys j, with z_ij = s q_i . k_j, P_i. = softmax(z_i.), O_i = sum_j P_ij v_j:
 *   dL/dP_ij = dO_i . v_j                                  (dP)
 *   dL/dz_ij = P_ij (dP_ij - sum_k P_ik dP_ik)             (softmax Jacobian; the sum is
 *                                                           dO_i . O_i, called D_i)
 *   dL/dq_i  = s sum_j dL/dz_ij k_j
 *   dL/dk_j  = s sum_i dL/dz_ij q_i
 *   dL/dv_j  = sum_i P_ij dO_i
 * A row with no valid key has O_i = 0 whatever the inputs and contributes nothing.
 * P is recomputed here from the scores with the row's own maximum and sum (three
 * passes, as in the forward), not from a stored LSE.
 *
 * q, dout: [BH, Nq, d]; k, v: [BH, Nk, d]; dq: [BH, Nq, d]; dk, dv: [BH, Nk, d];
 * row-major contiguous doubles owned by the caller, all outputs overwritten.
 * Slices run in parallel; within a slice the rows run in order. Return codes as
 * oracle_attn_fwd_f64.
 */
int oracle_attn_bwd_f64(const double* q, const double* k, const double* v, const double* dout,
                        double* dq, double* dk, double* dv, int64_t BH, int64_t Nq, int64_t Nk,
                        int64_t d, double scale, int causal) {
  if (BH < 0 || Nq < 0 || Nk < 0 || d < 0) return 2;
  if (!(scale > 0.0) || !isfinite(scale)) return 3;
  if (causal < 0 || causal > 2) return 6;
  if (BH == 0) return 0;
  if ((Nq > 0 && (!q || !dout || !dq)) || (Nk > 0 && (!k || !v || !dk || !dv))) return 1;
  int fail = 0;
#pragma omp parallel
  {
    const size_t n = (size_t)(Nk > 0 ? Nk : 1);
    double* z = (double*)malloc(sizeof(double) * n);
    double* pr = (double*)malloc(sizeof(double) * n);
    double* dp = (double*)malloc(sizeof(double) * n);
    if (!z || !pr || !dp) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t bh = 0; bh < BH; ++bh) {
        const double* qs = q + bh * Nq * d;
        const double* ks = k + bh * Nk * d;
        const double* vs = v + bh * Nk * d;
        const double* dos = dout + bh * Nq * d;
        double* dqs = dq + bh * Nq * d;
        double* dks = dk + bh * Nk * d;
        double* dvs = dv + bh * Nk * d;
        for (int64_t t = 0; t < Nk * d; ++t) { dks[t] = 0.0; dvs[t] = 0.0; }
        for (int64_t i = 0; i < Nq; ++i) {
          const double* qi = qs + i * d;
          const double* doi = dos + i * d;
          double* dqi = dqs + i * d;
          for (int64_t c = 0; c < d; ++c) dqi[c] = 0.0;
          int64_t nv = Nk;
          if (causal == 1) nv = (i + 1 < Nk) ? (i + 1) : Nk;
          if (causal == 2) nv = (i + Nk - Nq + 1 < Nk) ? (i + Nk - Nq + 1) : Nk;
          if (nv <= 0) continue;
          /* scores and the row's softmax (max, sum, normalised weights) */
          for (int64_t j = 0; j < nv; ++j) {
            double x = 0.0;
            for (int64_t c = 0; c < d; ++c) x += qi[c] * ks[j * d + c];
            z[j] = scale * x;
          }
          double m = z[0];
          for (int64_t j = 1; j < nv; ++j)
            if (z[j] > m) m = z[j];
          double l = 0.0;
          for (int64_t j = 0; j < nv; ++j) l += exp(z[j] - m);
          for (int64_t j = 0; j < nv; ++j) pr[j] = exp(z[j] - m) / l;
          /* dP_ij = dO_i . v_j and D_i = sum_j P_ij dP_ij */
          double Di = 0.0;
          for (int64_t j = 0; j < nv; ++j) {
            double x = 0.0;
            for (int64_t c = 0; c < d; ++c) x += doi[c] * vs[j * d + c];
            dp[j] = x;
            Di += pr[j] * x;
          }
          for (int64_t j = 0; j < nv; ++j) {
            const double dz = pr[j] * (dp[j] - Di);
            for (int64_t c = 0; c < d; ++c) {
              dqi[c] += scale * dz * ks[j * d + c];
              dks[j * d + c] += scale * dz * qi[c];
              dvs[j * d + c] += pr[j] * doi[c];
            }
          }
        }
      }
    }
    free(z);
    free(pr);
    free(dp);
  }
  return fail ? 4 : 0;
}

/* Number of threads the parallel regions above use. */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
