/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the gated delta rule prefill.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this code.  The product path
 * (the HIP library) never links, loads or calls it, and this file shares no
 * code, header, table or helper with that library.
 *
 * What it computes (sources, cited by page title and section):
 *   - "Add opt-in fused Qwen3.5 inference kernels" (JevAny PR #29), Summary:
 *     each Gated DeltaNet layer's chunked kernel applies the decay gate built
 *     from A_log and dt_bias, a sigmoid beta, L2 normalisation of q and k and
 *     grouped value heads; a fused gated RMSNorm follows.
 *   - "feat(qwen35): add SM120 FlashInfer GDN prefill candidate" (pegainfer
 *     PR #862), Correctness: the production geometry Hq/Hk/Hv/D = 16/16/32/128,
 *     a 128x128 recurrent state per value head, chunked prefill carrying state
 *     between calls, and an FP64 oracle as the accuracy reference.
 * The pages print no formula.  The operator is the gated delta rule, written
 * here token by token, which is its plain definition (the chunked form only
 * reorders the same arithmetic):
 *     g_t     = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])
 *     alpha_t = exp(g_t),  beta_t = sigmoid(b[t,h])
 *     qn_t    = scale * q_t / sqrt(|q_t|^2 + eps_l2),  kn_t = k_t / sqrt(|k_t|^2 + eps_l2)
 *     S_t     = alpha_t * S_{t-1} (I - beta_t kn_t kn_t^T) + beta_t v_t kn_t^T
 *     o_t     = S_t qn_t
 *     y_t     = o_t / sqrt(mean(o_t^2) + eps_n) * w * silu(z_t)   (when z is given)
 * with S an Dv x Dk matrix per (sequence, value head), stored row-major
 * [N, Hv, Dv, Dk], and value head h reading key head floor(h / (Hv/Hk)).
 * The two update lines are evaluated as "decay, then delta write":
 *     S' = alpha_t S_{t-1};  e = v_t - S' kn_t;  S_t = S' + beta_t e kn_t^T
 * which equals the product form above exactly in real arithmetic.
 *
 * Readings where the pages are silent:
 * scale defaults to Dk^-1/2 (callers pass it), eps_l2 = eps_n = 1e-6 by
 * default (callers pass them), softplus is the exact stable form, the norm
 * weight multiplies plainly (not 1+w), a NULL state_in means zeros, and a
 * zero-length sequence passes its state through unchanged.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(x) = log(1 + e^x), evaluated without overflow. */
double gdn_oracle_softplus(double x) {
  return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

/* sigmoid(x) = 1 / (1 + e^-x); IEEE inf handling gives exactly 0 and 1 at the
 * extremes. */
double gdn_oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/*
 * The recurrence alone, on already-prepared per-token quantities:
 *   alpha[T], beta[T], kn[T,Dk], qn[T,Dk], v[T,Dv]; S[Dv,Dk] is read and
 *   overwritten with the final state; o[T,Dv] receives S_t qn_t.
 * Strides let the caller point into strided [T, H, D] tensors.
 */
/*
 * The same recurrence, also returning the size of the terms of each output
 * element: rss[t, i] = sqrt(sum_j (S_t[i,j] qn_t[j])^2), the root-sum-square
 * of the Dk products whose sum is o_t[i] (rss may be NULL).  This is a
 * diagnostic for the tests: a dot product evaluated from operands rounded to
 * a relative precision u carries an error of the order of u times the size
 * of its terms, not of its result, so an element that is small through
 * cancellation is determined by low-precision operands only to that
 * absolute accuracy.
 */
void gdn_oracle_delta_core_terms(int64_t T, int Dk, int Dv,
                                 const double* alpha, const double* beta,
                                 const double* kn, int64_t kn_stride,
                                 const double* qn, int64_t qn_stride,
                                 const double* v, int64_t v_stride,
                                 double* S, double* o, int64_t o_stride,
                                 double* rss, int64_t rss_stride) {
  double* e = (double*)malloc(sizeof(double) * (size_t)(Dv > 0 ? Dv : 1));
  for (int64_t t = 0; t < T; ++t) {
    const double* kt = kn + t * kn_stride;
    const double* qt = qn + t * qn_stride;
    const double* vt = v + t * v_stride;
    /* decay */
    for (int64_t i = 0; i < (int64_t)Dv * Dk; ++i) S[i] *= alpha[t];
    /* e = v_t - S' kn_t */
    for (int i = 0; i < Dv; ++i) {
      double acc = 0.0;
      for (int j = 0; j < Dk; ++j) acc += S[(int64_t)i * Dk + j] * kt[j];
      e[i] = vt[i] - acc;
    }
    /* S_t = S' + beta e kn^T */
    for (int i = 0; i < Dv; ++i) {
      double be = beta[t] * e[i];
      for (int j = 0; j < Dk; ++j) S[(int64_t)i * Dk + j] += be * kt[j];
    }
    /* o_t = S_t qn_t */
    if (o) {
      double* ot = o + t * o_stride;
      for (int i = 0; i < Dv; ++i) {
        double acc = 0.0;
        for (int j = 0; j < Dk; ++j) acc += S[(int64_t)i * Dk + j] * qt[j];
        ot[i] = acc;
      }
    }
    if (rss) {
      double* rt = rss + t * rss_stride;
      for (int i = 0; i < Dv; ++i) {
        double ss = 0.0;
        for (int j = 0; j < Dk; ++j) {
          const double term = S[(int64_t)i * Dk + j] * qt[j];
          ss += term * term;
        }
        rt[i] = sqrt(ss);
      }
    }
  }
  free(e);
}

void gdn_oracle_delta_core(int64_t T, int Dk, int Dv,
                           const double* alpha, const double* beta,
                           const double* kn, int64_t kn_stride,
                           const double* qn, int64_t qn_stride,
                           const double* v, int64_t v_stride,
                           double* S, double* o, int64_t o_stride) {
  gdn_oracle_delta_core_terms(T, Dk, Dv, alpha, beta, kn, kn_stride, qn,
                              qn_stride, v, v_stride, S, o, o_stride, NULL, 0);
}

/* y = o / sqrt(mean(o^2) + eps) * w * z * sigmoid(z), over one row of D. */
void gdn_oracle_gated_rmsnorm_row(int D, const double* o, const double* z,
                                  const double* w, double eps, double* y) {
  double ss = 0.0;
  for (int i = 0; i < D; ++i) ss += o[i] * o[i];
  double r = 1.0 / sqrt(ss / (double)D + eps);
  for (int i = 0; i < D; ++i) {
    double silu = z[i] * gdn_oracle_sigmoid(z[i]);
    y[i] = o[i] * r * w[i] * silu;
  }
}

/*
 * Full prefill.  All arrays are host fp64, row-major:
 *   q [T_tot, Hk, Dk], k [T_tot, Hk, Dk], v [T_tot, Hv, Dv],
 *   a, b [T_tot, Hv], A_log, dt_bias [Hv],
 *   z [T_tot, Hv, Dv] and norm_w [Dv] (both NULL: no gated norm),
 *   state_in [N, Hv, Dv, Dk] (NULL: zeros),
 *   cu_seqlens int32 [N+1] (NULL: one sequence of T_tot tokens),
 *   o [T_tot, Hv, Dv] out, state_out [N, Hv, Dv, Dk] out (may be NULL),
 *   and two optional diagnostics for the tests (each may be NULL):
 *   o_raw [T_tot, Hv, Dv], the output before the gated norm, and
 *   term_rss [T_tot, Hv, Dv], the size of the terms of each element of
 *   o_raw (see gdn_oracle_delta_core_terms).
 * Returns 0, or -1 on inconsistent arguments.
 */
int gdn_oracle_prefill_ex(int N, int64_t T_tot, int Hk, int Hv, int Dk, int Dv,
                          const double* q, const double* k, const double* v,
                          const double* a, const double* b,
                          const double* A_log, const double* dt_bias,
                          const double* z, const double* norm_w,
                          const double* state_in, const int32_t* cu_seqlens,
                          double scale, double l2_eps, double norm_eps,
                          double* o, double* state_out, double* o_raw,
                          double* term_rss, int num_threads) {
  if (N < 1 || T_tot < 0 || Hk < 1 || Hv < 1 || Dk < 1 || Dv < 1) return -1;
  if (Hv % Hk != 0) return -1;
  if ((z == NULL) != (norm_w == NULL)) return -1;
  if (cu_seqlens == NULL && N != 1) return -1;
  if (cu_seqlens) {
    if (cu_seqlens[0] != 0 || cu_seqlens[N] != T_tot) return -1;
    for (int n = 0; n < N; ++n)
      if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  }
  const int r = Hv / Hk;
  const int64_t units = (int64_t)N * Hv;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t u = 0; u < units; ++u) {
    const int n = (int)(u / Hv);
    const int h = (int)(u % Hv);
    const int kh = h / r; /* grouped value heads: blocked map */
    const int64_t t0 = cu_seqlens ? cu_seqlens[n] : 0;
    const int64_t t1 = cu_seqlens ? cu_seqlens[n + 1] : T_tot;
    const int64_t L = t1 - t0;
    const size_t SD = (size_t)Dv * Dk;
    double* S = (double*)malloc(sizeof(double) * SD);
    if (state_in)
      memcpy(S, state_in + (size_t)u * SD, sizeof(double) * SD);
    else
      memset(S, 0, sizeof(double) * SD);
    if (L > 0) {
      double* alpha = (double*)malloc(sizeof(double) * (size_t)L);
      double* beta = (double*)malloc(sizeof(double) * (size_t)L);
      double* kn = (double*)malloc(sizeof(double) * (size_t)L * Dk);
      double* qn = (double*)malloc(sizeof(double) * (size_t)L * Dk);
      double* vv = (double*)malloc(sizeof(double) * (size_t)L * Dv);
      double* oo = (double*)malloc(sizeof(double) * (size_t)L * Dv);
      const double decay_rate = exp(A_log[h]);
      for (int64_t t = 0; t < L; ++t) {
        const int64_t row = t0 + t;
        const double x = a[row * Hv + h] + dt_bias[h];
        const double g = -decay_rate * gdn_oracle_softplus(x);
        alpha[t] = exp(g);
        beta[t] = gdn_oracle_sigmoid(b[row * Hv + h]);
        const double* qr = q + (row * Hk + kh) * Dk;
        const double* kr = k + (row * Hk + kh) * Dk;
        double sq = 0.0, sk = 0.0;
        for (int j = 0; j < Dk; ++j) {
          sq += qr[j] * qr[j];
          sk += kr[j] * kr[j];
        }
        const double fq = scale / sqrt(sq + l2_eps);
        const double fk = 1.0 / sqrt(sk + l2_eps);
        for (int j = 0; j < Dk; ++j) {
          qn[t * Dk + j] = qr[j] * fq;
          kn[t * Dk + j] = kr[j] * fk;
        }
        memcpy(vv + t * Dv, v + (row * Hv + h) * Dv, sizeof(double) * Dv);
      }
      gdn_oracle_delta_core_terms(L, Dk, Dv, alpha, beta, kn, Dk, qn, Dk, vv,
                                  Dv, S, oo, Dv,
                                  term_rss ? term_rss + (t0 * Hv + h) * Dv : NULL,
                                  (int64_t)Hv * Dv);
      for (int64_t t = 0; t < L; ++t) {
        const int64_t row = t0 + t;
        double* dst = o + (row * Hv + h) * Dv;
        if (o_raw)
          memcpy(o_raw + (row * Hv + h) * Dv, oo + t * Dv, sizeof(double) * Dv);
        if (z)
          gdn_oracle_gated_rmsnorm_row(Dv, oo + t * Dv, z + (row * Hv + h) * Dv,
                                       norm_w, norm_eps, dst);
        else
          memcpy(dst, oo + t * Dv, sizeof(double) * Dv);
      }
      free(alpha);
      free(beta);
      free(kn);
      free(qn);
      free(vv);
      free(oo);
    }
    if (state_out) memcpy(state_out + (size_t)u * SD, S, sizeof(double) * SD);
    free(S);
  }
  return 0;
}

int gdn_oracle_prefill(int N, int64_t T_tot, int Hk, int Hv, int Dk, int Dv,
                       const double* q, const double* k, const double* v,
                       const double* a, const double* b,
                       const double* A_log, const double* dt_bias,
                       const double* z, const double* norm_w,
                       const double* state_in, const int32_t* cu_seqlens,
                       double scale, double l2_eps, double norm_eps,
                       double* o, double* state_out, int num_threads) {
  return gdn_oracle_prefill_ex(N, T_tot, Hk, Hv, Dk, Dv, q, k, v, a, b, A_log,
                               dt_bias, z, norm_w, state_in, cu_seqlens, scale,
                               l2_eps, norm_eps, o, state_out, NULL, NULL,
                               num_threads);
}

/*
 * Depthwise causal convolution of width W over channels, zero history, then
 * SiLU: y[t,c] = silu( sum_{j=0}^{W-1} w[c,j] * x[t-(W-1)+j, c] ),
 * x[t<0] = 0.  Tap w[c,W-1] multiplies the current token.
 */
void gdn_oracle_causal_conv_silu(int64_t T, int C, int W, const double* x,
                                 const double* w, double* y) {
#ifdef _OPENMP
#pragma omp parallel for
#endif
  for (int c = 0; c < C; ++c) {
    for (int64_t t = 0; t < T; ++t) {
      double acc = 0.0;
      for (int j = 0; j < W; ++j) {
        int64_t src = t - (W - 1) + j;
        if (src >= 0) acc += w[(int64_t)c * W + j] * x[src * C + c];
      }
      y[t * C + c] = acc * gdn_oracle_sigmoid(acc);
    }
  }
}
