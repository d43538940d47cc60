/*
 * KDA oracle: plain, slow, token-by-token fp64 evaluation of the Kimi Delta
 * Attention recurrence on the host.  TEST INFRASTRUCTURE ONLY: only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg load this file's
 * library.  It shares no code with the HIP kernels.
 *
 * What it computes (the KDA recurrence: a delta rule with a channel-wise forget
 * gate, "Kimi K3 technical report summary", section 1, pre-training table, KDA
 * row; the per-head fixed matrix state updated token by token at decode time,
 * "Kimi K3 NPU Training", section "confirmed skeleton", list item 4):
 *
 *   for every sequence n and head h independently, with S a dk x dv matrix
 *   (rows indexed by key channel, columns by value channel):
 *     S <- h0[n,h]  (zeros when no initial state is given)
 *     for each token t of sequence n, in order:
 *       S <- Diag(alpha_t) S              alpha_t = exp(log_alpha[t,h,:]) decays the key rows
 *       S <- S - beta_t k_t (k_t^T S)     the delta-rule erase, (I - beta k k^T) applied to the decayed state
 *       S <- S + beta_t k_t v_t^T         the write
 *       o[t,h,:] = S^T q_t                the read-out uses the state after the write
 *     hT[n,h] <- S
 *
 * Packed sequences: sequence n covers tokens [cu[n], cu[n+1]); the state is reset
 * at every sequence start (state reset at packed boundaries, "Kimi K3 NPU
 * Training", section "TND is not a layout switch", item 2).
 *
 * Inputs are read exactly as stored (bf16 and fp32 widen exactly to fp32, which
 * the caller passes) and widened to fp64.  Nothing is re-normalised.
 *
 * Parallelism: OpenMP over (sequence, head) and over blocks of value columns.
 * The columns of S evolve independently given k, alpha and beta, so splitting
 * them changes no arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One (sequence, head) chain restricted to value columns [j0, j1). */
static void chain(const float *q, const float *k, const float *v, const float *log_alpha,
                  const float *beta, const float *h0_nh, int64_t t_begin, int64_t t_end,
                  int H, int h, int dk, int dv, int j0, int j1, double *o, double *hT_nh,
                  double *S, double *y, double *a) {
  const int w = j1 - j0;
  for (int c = 0; c < dk; ++c)
    for (int j = 0; j < w; ++j) S[(size_t)c * w + j] = h0_nh ? (double)h0_nh[(size_t)c * dv + j0 + j] : 0.0;

  for (int64_t t = t_begin; t < t_end; ++t) {
    const float *qt = q + ((size_t)t * H + h) * dk;
    const float *kt = k + ((size_t)t * H + h) * dk;
    const float *vt = v + ((size_t)t * H + h) * dv + j0;
    const float *lat = log_alpha + ((size_t)t * H + h) * dk;
    const double bt = (double)beta[(size_t)t * H + h];

    /* decay: S <- Diag(alpha_t) S */
    for (int c = 0; c < dk; ++c) a[c] = exp((double)lat[c]);
    for (int c = 0; c < dk; ++c) {
      double *row = S + (size_t)c * w;
      const double ac = a[c];
      for (int j = 0; j < w; ++j) row[j] *= ac;
    }
    /* y = k_t^T S */
    for (int j = 0; j < w; ++j) y[j] = 0.0;
    for (int c = 0; c < dk; ++c) {
      const double kc = (double)kt[c];
      const double *row = S + (size_t)c * w;
      for (int j = 0; j < w; ++j) y[j] += kc * row[j];
    }
    /* S <- S - beta k y^T + beta k v^T */
    for (int c = 0; c < dk; ++c) {
      const double bk = bt * (double)kt[c];
      double *row = S + (size_t)c * w;
      for (int j = 0; j < w; ++j) row[j] = row[j] - bk * y[j] + bk * (double)vt[j];
    }
    /* o_t = S^T q_t */
    double *ot = o + ((size_t)t * H + h) * dv + j0;
    for (int j = 0; j < w; ++j) y[j] = 0.0;
    for (int c = 0; c < dk; ++c) {
      const double qc = (double)qt[c];
      const double *row = S + (size_t)c * w;
      for (int j = 0; j < w; ++j) y[j] += qc * row[j];
    }
    for (int j = 0; j < w; ++j) ot[j] = y[j];
  }
  if (hT_nh)
    for (int c = 0; c < dk; ++c)
      for (int j = 0; j < w; ++j) hT_nh[(size_t)c * dv + j0 + j] = S[(size_t)c * w + j];
}

/*
 * q, k: [T, H, dk] fp32; v: [T, H, dv] fp32; log_alpha: [T, H, dk] fp32; beta: [T, H] fp32.
 * h0: [N, H, dk, dv] fp32 or NULL (zeros).  cu_seqlens: [N+1] int64, cu[0] = 0, cu[N] = T.
 * o: [T, H, dv] fp64 (written for every token); hT: [N, H, dk, dv] fp64 or NULL.
 * n_threads <= 0 uses the OpenMP default.  Returns 0, or -1 on a bad argument.
 */
int kda_oracle_fwd(const float *q, const float *k, const float *v, const float *log_alpha,
                   const float *beta, const float *h0, const int64_t *cu_seqlens, int n_seqs,
                   int64_t total_tokens, int n_heads, int dk, int dv, double *o, double *hT,
                   int n_threads) {
  if (!q || !k || !v || !log_alpha || !beta || !cu_seqlens || !o) return -1;
  if (n_seqs < 0 || n_heads <= 0 || dk <= 0 || dv <= 0 || total_tokens < 0) return -1;
  if (cu_seqlens[0] != 0 || cu_seqlens[n_seqs] != total_tokens) return -1;
  for (int n = 0; n < n_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;

  int nt = 1;
#ifdef _OPENMP
  nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#endif
  const int64_t pairs = (int64_t)n_seqs * n_heads;
  /* split value columns until there are at least 2 tasks per thread (or 8 columns per task) */
  int nblk = 1;
  while (pairs * nblk < 2 * nt && dv / (nblk * 2) >= 8 && dv % (nblk * 2) == 0) nblk *= 2;
  const int64_t tasks = pairs * nblk;
  const int bw = dv / nblk;
  int err = 0;

#pragma omp parallel num_threads(nt)
  {
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * bw);
    double *y = (double *)malloc(sizeof(double) * (size_t)bw);
    double *a = (double *)malloc(sizeof(double) * (size_t)dk);
    if (!S || !y || !a) {
#pragma omp atomic write
      err = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t task = 0; task < tasks; ++task) {
        const int64_t pair = task / nblk;
        const int blk = (int)(task % nblk);
        const int n = (int)(pair / n_heads), h = (int)(pair % n_heads);
        const float *h0_nh = h0 ? h0 + ((size_t)n * n_heads + h) * dk * dv : NULL;
        double *hT_nh = hT ? hT + ((size_t)n * n_heads + h) * dk * dv : NULL;
        chain(q, k, v, log_alpha, beta, h0_nh, cu_seqlens[n], cu_seqlens[n + 1], n_heads, h, dk, dv,
              blk * bw, (blk + 1) * bw, o, hT_nh, S, y, a);
      }
    }
    free(S);
    free(y);
    free(a);
  }
  return err ? -1 : 0;
}

int kda_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
