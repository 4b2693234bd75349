/*
 * Oracle: plain fp64 CPU softmax attention, forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it. It shares no code with the HIP library.
 *
 * What it computes. The pages (DASH: Deterministic Attention Scheduling for
 * High-throughput Reproducible LLM Training; zskr.cn explainer, section 2.1;
 * gist.science summary, section 1) say that the attention backward produces the
 * partial gradients dQ, dK, dV of tiled softmax attention and that the
 * deterministic variants differ from the atomic one only in the order in which
 * dQ partials are summed. They never write the gradient out, so the oracle is
 * the textbook definition, evaluated exactly once per term in fp64:
 *
 *   s_ij  = scale * <q_i, k_j>          for visible j (full: all j; causal: j <= i)
 *   lse_i = m_i + log(sum_j exp(s_ij - m_i)),  m_i = max_j s_ij   (natural log)
 *   P_ij  = exp(s_ij - lse_i)
 *   o_i   = sum_j P_ij v_j
 *   dP_ij = <do_i, v_j>
 *   D_i   = sum_j P_ij dP_ij
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dq_i  = scale * sum_j dS_ij k_j
 *   dk_j  = scale * sum_i dS_ij q_i
 *   dv_j  = sum_i P_ij do_i
 *
 * Layout: every tensor is contiguous [B, H, S, D] (row-major, D fastest);
 * lse and delta are [B, H, S]. Self-attention only (one S for queries and keys).
 *
 * Parallelism does not change any result: every output element is produced by
 * exactly one loop nest that sums its terms in ascending index order. The
 * backward is split into three passes (row statistics, dq rows, dk/dv columns),
 * each embarrassingly parallel over its own index.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static double dot(const double* a, const double* b, int D) {
  double s = 0.0;
  for (int d = 0; d < D; ++d) s += a[d] * b[d];
  return s;
}

/* Number of keys query i may attend to: all S under the full mask, i+1 under causal. */
static int visible(int i, int S, int causal) { return causal ? i + 1 : S; }

/* Scores s_ij and log-sum-exp of one query row; s has room for S values. */
static double row_scores(const double* qi, const double* k, int S, int D, double scale, int nvis, double* s) {
  double m = -INFINITY;
  for (int j = 0; j < nvis; ++j) {
    s[j] = scale * dot(qi, k + (size_t)j * D, D);
    if (s[j] > m) m = s[j];
  }
  double l = 0.0;
  for (int j = 0; j < nvis; ++j) l += exp(s[j] - m);
  (void)S;
  return m + log(l);
}

/*
 * Forward for all (b, h, i): o and lse. Inputs q, k, v as fp64 [B,H,S,D].
 */
void oracle_attn_fwd(int B, int H, int S, int D, const double* q, const double* k, const double* v, double scale,
                     int causal, double* o, double* lse, int nthreads) {
  set_threads(nthreads);
  const size_t hs = (size_t)S * D;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)S);
#pragma omp for schedule(dynamic, 4) collapse(2)
    for (int bh = 0; bh < B * H; ++bh) {
      for (int i = 0; i < S; ++i) {
        const double* qh = q + bh * hs;
        const double* kh = k + bh * hs;
        const double* vh = v + bh * hs;
        int nvis = visible(i, S, causal);
        double L = row_scores(qh + (size_t)i * D, kh, S, D, scale, nvis, s);
        double* oi = o + bh * hs + (size_t)i * D;
        for (int d = 0; d < D; ++d) oi[d] = 0.0;
        for (int j = 0; j < nvis; ++j) {
          double p = exp(s[j] - L);
          const double* vj = vh + (size_t)j * D;
          for (int d = 0; d < D; ++d) oi[d] += p * vj[d];
        }
        lse[(size_t)bh * S + i] = L;
      }
    }
    free(s);
  }
}

/* Row statistics of one head: lse_i and D_i = sum_j P_ij dP_ij for every row i. */
static void head_row_stats(int S, int D, const double* qh, const double* kh, const double* vh, const double* doh,
                           double scale, int causal, double* lse_h, double* delta_h) {
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)S);
#pragma omp for schedule(dynamic, 8)
    for (int i = 0; i < S; ++i) {
      int nvis = visible(i, S, causal);
      const double* qi = qh + (size_t)i * D;
      const double* doi = doh + (size_t)i * D;
      double L = row_scores(qi, kh, S, D, scale, nvis, s);
      double acc = 0.0;
      for (int j = 0; j < nvis; ++j) {
        double p = exp(s[j] - L);
        double dp = dot(doi, vh + (size_t)j * D, D);
        acc += p * dp;
      }
      lse_h[i] = L;
      delta_h[i] = acc;
    }
    free(s);
  }
}

/* dq for one row i of one head, given that row's lse and D. */
static void head_dq_row(int i, int S, int D, const double* qh, const double* kh, const double* vh, const double* doh,
                        double scale, int causal, double L, double Di, double* dqi) {
  int nvis = visible(i, S, causal);
  const double* qi = qh + (size_t)i * D;
  const double* doi = doh + (size_t)i * D;
  for (int d = 0; d < D; ++d) dqi[d] = 0.0;
  for (int j = 0; j < nvis; ++j) {
    const double* kj = kh + (size_t)j * D;
    double p = exp(scale * dot(qi, kj, D) - L);
    double dp = dot(doi, vh + (size_t)j * D, D);
    double ds = p * (dp - Di);
    for (int d = 0; d < D; ++d) dqi[d] += ds * kj[d];
  }
  for (int d = 0; d < D; ++d) dqi[d] *= scale;
}

/* dk and dv for one key column j of one head, given every row's lse and D. */
static void head_dkdv_col(int j, int S, int D, const double* qh, const double* kh, const double* vh, const double* doh,
                          double scale, int causal, const double* lse_h, const double* delta_h, double* dkj,
                          double* dvj) {
  const double* kj = kh + (size_t)j * D;
  const double* vj = vh + (size_t)j * D;
  for (int d = 0; d < D; ++d) { dkj[d] = 0.0; dvj[d] = 0.0; }
  int i0 = causal ? j : 0; /* under the causal mask only queries i >= j see key j */
  for (int i = i0; i < S; ++i) {
    const double* qi = qh + (size_t)i * D;
    const double* doi = doh + (size_t)i * D;
    double p = exp(scale * dot(qi, kj, D) - lse_h[i]);
    double dp = dot(doi, vj, D);
    double ds = p * (dp - delta_h[i]);
    for (int d = 0; d < D; ++d) {
      dkj[d] += ds * qi[d];
      dvj[d] += p * doi[d];
    }
  }
  for (int d = 0; d < D; ++d) dkj[d] *= scale;
}

/*
 * Full backward for all heads: dq, dk, dv, plus lse and delta (D_i) per row.
 * The forward statistics are recomputed here from q, k, v; nothing from any
 * other implementation is consumed.
 */
void oracle_attn_bwd(int B, int H, int S, int D, const double* q, const double* k, const double* v, const double* dout,
                     double scale, int causal, double* dq, double* dk, double* dv, double* lse, double* delta,
                     int nthreads) {
  set_threads(nthreads);
  const size_t hs = (size_t)S * D;
  for (int bh = 0; bh < B * H; ++bh) {
    const double* qh = q + bh * hs;
    const double* kh = k + bh * hs;
    const double* vh = v + bh * hs;
    const double* doh = dout + bh * hs;
    double* lse_h = lse + (size_t)bh * S;
    double* delta_h = delta + (size_t)bh * S;
    head_row_stats(S, D, qh, kh, vh, doh, scale, causal, lse_h, delta_h);
#pragma omp parallel for schedule(dynamic, 8)
    for (int i = 0; i < S; ++i)
      head_dq_row(i, S, D, qh, kh, vh, doh, scale, causal, lse_h[i], delta_h[i], dq + bh * hs + (size_t)i * D);
#pragma omp parallel for schedule(dynamic, 8)
    for (int j = 0; j < S; ++j)
      head_dkdv_col(j, S, D, qh, kh, vh, doh, scale, causal, lse_h, delta_h, dk + bh * hs + (size_t)j * D,
                    dv + bh * hs + (size_t)j * D);
  }
}

/*
 * Sampled backward for one head (tensors of shape [S, D]): computes every row's
 * lse and D (needed by any key column), then dq for the listed rows and dk, dv
 * for the listed key columns. Used where the full problem is too large for the
 * CPU; each sampled value is the same expression as in oracle_attn_bwd.
 */
void oracle_attn_bwd_sampled(int S, int D, const double* qh, const double* kh, const double* vh, const double* doh,
                             double scale, int causal, int nrows, const int32_t* rows, int ncols, const int32_t* cols,
                             double* dq_rows, double* dk_cols, double* dv_cols, double* lse_h, double* delta_h,
                             int nthreads) {
  set_threads(nthreads);
  head_row_stats(S, D, qh, kh, vh, doh, scale, causal, lse_h, delta_h);
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < nrows; ++r)
    head_dq_row(rows[r], S, D, qh, kh, vh, doh, scale, causal, lse_h[rows[r]], delta_h[rows[r]],
                dq_rows + (size_t)r * D);
#pragma omp parallel for schedule(dynamic, 1)
  for (int c = 0; c < ncols; ++c)
    head_dkdv_col(cols[c], S, D, qh, kh, vh, doh, scale, causal, lse_h, delta_h, dk_cols + (size_t)c * D,
                  dv_cols + (size_t)c * D);
}
