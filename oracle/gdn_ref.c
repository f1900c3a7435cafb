/*
 * CPU oracle, plain C twin of gdn_ref.py (float64, token by token).
 *
 * TEST INFRASTRUCTURE ONLY: called by the tests, the smoke check and the
 * CPU-baseline leg of the benchmark, never by the HIP library.  It shares no
 * code with the library.
 *
 * Recurrence (gated delta rule, Yang et al., "Gated Delta Networks", ICLR 2025):
 *   S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *   o_t = scale * S_t^T q_t
 * Interfaces follow "GDN CTE Kernel API Reference" (gdn_cte) and
 * "GDN TKG Kernel API Reference" (gdn_tkg).  The only parallelism is an
 * OpenMP loop over independent (batch, value head) pairs: heads never
 * interact (TKG page, Notes: per-head independent recurrence).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* gdn_cte: q,k [B,Hk,S,Dk]; v [B,Hv,S,Dv]; g,beta [B,Hv,S];
 * s0 [B,Hv,Dk,Dv] or NULL (zero state); out [B,Hv,S,Dv]; state [B,Hv,Dk,Dv]. */
void gdn_ref_cte(const double* q, const double* k, const double* v,
                 const double* g, const double* beta, double scale,
                 const double* s0, double* out, double* state,
                 int B, int Hk, int Hv, int S, int Dk, int Dv) {
  const int grp = Hv / Hk;
#pragma omp parallel for schedule(dynamic, 1)
  for (int bh = 0; bh < B * Hv; ++bh) {
    const int b = bh / Hv, h = bh % Hv, hk = h / grp;
    double* St = state + (size_t)bh * Dk * Dv;
    if (s0)
      memcpy(St, s0 + (size_t)bh * Dk * Dv, sizeof(double) * Dk * Dv);
    else
      memset(St, 0, sizeof(double) * Dk * Dv);
    double* kS = (double*)malloc(sizeof(double) * Dv);
    for (int t = 0; t < S; ++t) {
      const double* kt = k + (((size_t)b * Hk + hk) * S + t) * Dk;
      const double* qt = q + (((size_t)b * Hk + hk) * S + t) * Dk;
      const double* vt = v + (((size_t)b * Hv + h) * S + t) * Dv;
      const double a = exp(g[((size_t)b * Hv + h) * S + t]);
      const double bt = beta[((size_t)b * Hv + h) * S + t];
      /* kS = k^T S */
      for (int j = 0; j < Dv; ++j) kS[j] = 0.0;
      for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) kS[j] += kt[i] * St[i * Dv + j];
      /* S = a (S - bt k kS^T) + bt k v^T */
      for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j)
          St[i * Dv + j] = a * (St[i * Dv + j] - bt * kt[i] * kS[j]) + bt * kt[i] * vt[j];
      /* o = scale S^T q */
      double* ot = out + (((size_t)b * Hv + h) * S + t) * Dv;
      for (int j = 0; j < Dv; ++j) ot[j] = 0.0;
      for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) ot[j] += St[i * Dv + j] * qt[i];
      for (int j = 0; j < Dv; ++j) ot[j] *= scale;
    }
    free(kS);
  }
}

static double softplus_d(double x) {
  /* log(1 + exp(x)) without overflow */
  return x > 0 ? x + log1p(exp(-x)) : log1p(exp(x));
}

/* gdn_tkg core + prologue + RMSNormGated epilogue (no bf16 rounding of y;
 * the caller rounds).  q,k [BH,K]; v,z [BH,V]; b,a [BH]; A_log, dt_bias [Hv];
 * w [V]; s_in, s_out [BH,K,V]; y [BH,V]. */
void gdn_ref_tkg(const double* q, const double* k, const double* v,
                 const double* b, const double* a, const double* A_log,
                 const double* dt_bias, const double* z, const double* w,
                 const double* s_in, double* s_out, double* y,
                 int BH, int Hv, int K, int V, double l2_eps, double rms_eps) {
#pragma omp parallel for schedule(static)
  for (int n = 0; n < BH; ++n) {
    const int h = n % Hv;
    const double* qn = q + (size_t)n * K;
    const double* kn = k + (size_t)n * K;
    double qq = 0, kk = 0;
    for (int i = 0; i < K; ++i) { qq += qn[i] * qn[i]; kk += kn[i] * kn[i]; }
    const double qs = 1.0 / sqrt(qq + l2_eps) / sqrt((double)K);
    const double ks = 1.0 / sqrt(kk + l2_eps);
    const double bt = 1.0 / (1.0 + exp(-b[n]));
    const double g = -exp(A_log[h]) * softplus_d(a[n] + dt_bias[h]);
    const double al = exp(g);
    const double* S0 = s_in + (size_t)n * K * V;
    double* S1 = s_out + (size_t)n * K * V;
    double* o = y + (size_t)n * V;
    for (int j = 0; j < V; ++j) {
      double kS = 0;
      for (int i = 0; i < K; ++i) kS += kn[i] * ks * S0[i * V + j];
      double oj = 0;
      for (int i = 0; i < K; ++i) {
        const double ki = kn[i] * ks;
        const double s = al * (S0[i * V + j] - bt * ki * kS) + bt * ki * v[(size_t)n * V + j];
        S1[i * V + j] = s;
        oj += s * qn[i] * qs;
      }
      o[j] = oj;
    }
    double ms = 0;
    for (int j = 0; j < V; ++j) ms += o[j] * o[j];
    const double r = 1.0 / sqrt(ms / V + rms_eps);
    for (int j = 0; j < V; ++j) {
      const double zj = z[(size_t)n * V + j];
      o[j] = w[j] * o[j] * r * (zj / (1.0 + exp(-zj)));
    }
  }
}

int gdn_ref_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
