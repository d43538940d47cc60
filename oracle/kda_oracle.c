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

/*
 * Reverse mode of the same recurrence (the backward pass), plain and slow: for every
 * (sequence, head) the forward states S_0 = h0, S_1 .. S_L are kept, then the adjoint
 * dS runs backwards from dS_L = dhT.  Token t (with P = Diag(alpha_t) S_{t-1},
 * u = P^T k_t, delta = beta_t (v_t - u), S_t = P + k_t delta^T, o_t = S_t^T q_t) gives:
 *   dS      += q_t do_t^T                      (read-out)
 *   dq_t     = S_t do_t
 *   ddelta   = dS^T k_t                        (S_t = P + k delta^T)
 *   dk_t     = dS delta
 *   dv_t     = beta_t ddelta,   dbeta_t = ddelta . (v_t - u),   du = -beta_t ddelta
 *   dP       = dS + k_t du^T,   dk_t    += P du                  (u = P^T k)
 *   dlog_alpha_t[c] = sum_j dP[c][j] P[c][j]                     (P = Diag(e^{log alpha}) S_{t-1})
 *   dS       = Diag(alpha_t) dP                 (adjoint of S_{t-1})
 * and dh0 = dS after the first token.  The loss these are gradients of is
 * sum_t o_t . do_t + sum hT . dhT.
 *
 * do_: [T, H, dv] fp32; dhT: [N, H, dk, dv] fp32 or NULL (zeros).  Outputs fp64: dq, dk_out,
 * dla [T, H, dk]; dv_out [T, H, dv]; dbeta [T, H]; dh0 [N, H, dk, dv] or NULL.
 * Memory: (longest sequence + 1) * dk * dv doubles per thread.  Returns 0, or -1.
 */
int kda_oracle_bwd(const float *q, const float *k, const float *v, const float *log_alpha,
                   const float *beta, const float *h0, const int64_t *cu_seqlens, int n_seqs,
                   int64_t total_tokens, int n_heads, int dk, int dv, const float *do_,
                   const float *dhT, double *dq, double *dk_out, double *dv_out, double *dla,
                   double *dbeta, double *dh0, int n_threads) {
  if (!q || !k || !v || !log_alpha || !beta || !cu_seqlens || !do_ || !dq || !dk_out || !dv_out || !dla ||
      !dbeta)
    return -1;
  if (n_seqs < 0 || n_heads <= 0 || dk <= 0 || dv <= 0 || total_tokens < 0) return -1;
  if (cu_seqlens[0] != 0 || cu_seqlens[n_seqs] != total_tokens) return -1;
  int64_t maxlen = 0;
  for (int n = 0; n < n_seqs; ++n) {
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    if (cu_seqlens[n + 1] - cu_seqlens[n] > maxlen) maxlen = cu_seqlens[n + 1] - cu_seqlens[n];
  }
  int nt = 1;
#ifdef _OPENMP
  nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#endif
  const int64_t pairs = (int64_t)n_seqs * n_heads;
  const size_t DD = (size_t)dk * dv;
  int err = 0;

#pragma omp parallel num_threads(nt)
  {
    double *St = (double *)malloc(sizeof(double) * DD * (size_t)(maxlen + 1));
    double *dS = (double *)malloc(sizeof(double) * DD);
    double *P = (double *)malloc(sizeof(double) * DD);
    double *a = (double *)malloc(sizeof(double) * (size_t)dk);
    double *u = (double *)malloc(sizeof(double) * (size_t)dv);
    double *dl = (double *)malloc(sizeof(double) * (size_t)dv);
    double *dd = (double *)malloc(sizeof(double) * (size_t)dv);
    double *du = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!St || !dS || !P || !a || !u || !dl || !dd || !du) {
#pragma omp atomic write
      err = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t pair = 0; pair < pairs; ++pair) {
        const int n = (int)(pair / n_heads), h = (int)(pair % n_heads);
        const int64_t t0 = cu_seqlens[n], L = cu_seqlens[n + 1] - cu_seqlens[n];
        const float *h0p = h0 ? h0 + ((size_t)n * n_heads + h) * DD : NULL;
        for (size_t i = 0; i < DD; ++i) St[i] = h0p ? (double)h0p[i] : 0.0;
        /* forward, keeping every state */
        for (int64_t s = 0; s < L; ++s) {
          const int64_t t = t0 + s;
          const float *kt = k + ((size_t)t * n_heads + h) * dk;
          const float *vt = v + ((size_t)t * n_heads + h) * dv;
          const float *lat = log_alpha + ((size_t)t * n_heads + h) * dk;
          const double bt = (double)beta[(size_t)t * n_heads + h];
          const double *Sp = St + (size_t)s * DD;
          double *Sn = St + (size_t)(s + 1) * DD;
          for (int c = 0; c < dk; ++c) {
            const double ac = exp((double)lat[c]);
            for (int j = 0; j < dv; ++j) P[(size_t)c * dv + j] = ac * Sp[(size_t)c * dv + j];
          }
          for (int j = 0; j < dv; ++j) u[j] = 0.0;
          for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) u[j] += (double)kt[c] * P[(size_t)c * dv + j];
          for (int j = 0; j < dv; ++j) dl[j] = bt * ((double)vt[j] - u[j]); /* delta */
          for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) Sn[(size_t)c * dv + j] = P[(size_t)c * dv + j] + (double)kt[c] * dl[j];
        }
        /* backward */
        const float *dhTp = dhT ? dhT + ((size_t)n * n_heads + h) * DD : NULL;
        for (size_t i = 0; i < DD; ++i) dS[i] = dhTp ? (double)dhTp[i] : 0.0;
        for (int64_t s = L - 1; s >= 0; --s) {
          const int64_t t = t0 + s;
          const size_t ik = ((size_t)t * n_heads + h) * dk, iv = ((size_t)t * n_heads + h) * dv;
          const float *qt = q + ik, *kt = k + ik, *lat = log_alpha + ik, *vt = v + iv, *dot = do_ + iv;
          const double bt = (double)beta[(size_t)t * n_heads + h];
          const double *Sp = St + (size_t)s * DD, *Sn = St + (size_t)(s + 1) * DD;
          for (int c = 0; c < dk; ++c) {
            a[c] = exp((double)lat[c]);
            for (int j = 0; j < dv; ++j) P[(size_t)c * dv + j] = a[c] * Sp[(size_t)c * dv + j];
          }
          for (int j = 0; j < dv; ++j) u[j] = 0.0;
          for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) u[j] += (double)kt[c] * P[(size_t)c * dv + j];
          for (int j = 0; j < dv; ++j) dl[j] = bt * ((double)vt[j] - u[j]); /* delta */
          /* read-out */
          for (int c = 0; c < dk; ++c) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) {
              dS[(size_t)c * dv + j] += (double)qt[c] * (double)dot[j];
              acc += Sn[(size_t)c * dv + j] * (double)dot[j];
            }
            dq[ik + c] = acc;
          }
          /* write: S_t = P + k delta^T */
          for (int j = 0; j < dv; ++j) dd[j] = 0.0;
          for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) dd[j] += dS[(size_t)c * dv + j] * (double)kt[c];
          double db = 0.0;
          for (int j = 0; j < dv; ++j) {
            dv_out[iv + j] = bt * dd[j];
            db += dd[j] * ((double)vt[j] - u[j]);
            du[j] = -bt * dd[j];
          }
          dbeta[(size_t)t * n_heads + h] = db;
          for (int c = 0; c < dk; ++c) {
            double g = 0.0, gP = 0.0, gl = 0.0;
            for (int j = 0; j < dv; ++j) {
              const double dSc = dS[(size_t)c * dv + j];
              g += dSc * dl[j];
              gP += P[(size_t)c * dv + j] * du[j];
              const double dP = dSc + (double)kt[c] * du[j];
              gl += dP * P[(size_t)c * dv + j];
              dS[(size_t)c * dv + j] = a[c] * dP; /* adjoint of S_{t-1} */
            }
            dk_out[ik + c] = g + gP;
            dla[ik + c] = gl;
          }
        }
        if (dh0) {
          double *d0 = dh0 + ((size_t)n * n_heads + h) * DD;
          for (size_t i = 0; i < DD; ++i) d0[i] = dS[i];
        }
      }
    }
    free(St); free(dS); free(P); free(a); free(u); free(dl); free(dd); free(du);
  }
  return err ? -1 : 0;
}
