/*
 * KDA reference gradient -- TEST INFRASTRUCTURE ONLY.
 *
 * Reverse-mode derivative of the token-by-token recurrence of kda_oracle.c,
 * in IEEE fp64.  Only the test suite may load it; it shares no code with the
 * HIP path (nor with kda_oracle.c: the forward steps are written out again
 * here so that each file can be read on its own).
 *
 * Forward step t (per sequence and head), as in kda_oracle.c:
 *   a   = exp(max(g_t, g_floor))          per key channel
 *   S'  = diag(a) S_{t-1}
 *   w   = S'^T k_t
 *   u   = beta_t (v_t - w)
 *   S_t = S' + k_t u^T
 *   o_t = S_t^T q_t
 * Sources: the delta rule with erase-then-write and read after the write,
 * "Kimi K3 深度拆解" (chenxutan.com), 4.2 "线性注意力与 Delta Rule"; the
 * channel-wise gate, "Kimi K3 技術報告：三個架構改動一次看懂" (akiraxclaw.com),
 * "長度：KDA 為什麼還要搭配 Gated MLA？"; the floor on the log-decay,
 * "3 分钟看懂 Kimi K3" (landx.limxdynamics.com), "第一条主线", Figure 3.  The
 * pages give no gradient: what follows is the chain rule applied to the six
 * lines above, last line first.
 *
 * Given dL/do_t and dL/dS_t (called dS, accumulated from later tokens; the
 * caller's dht at the end of the sequence), step t in reverse:
 *   dS  += q_t do_t^T                     o_t = S_t^T q_t
 *   dq_t = S_t do_t
 *   du   = dS^T k_t ;  dk_t = dS u        S_t = S' + k u^T   (dS' = dS)
 *   dbeta_t = du . (v_t - w) ; dv_t = beta_t du ; dw = -beta_t du
 *   dS' += k_t dw^T ;  dk_t += S' dw      w = S'^T k
 *   da_c = sum_j dS'_cj S_{t-1,cj} ;  dS_{t-1} = diag(a) dS'
 *   dg_t,c = a_c da_c   where g_t,c >= g_floor, else 0
 * The floor max(g, g_floor) passes the gradient where g equals the floor
 * (inputs are normally floored already, so the tie is the common case) and
 * blocks it strictly below.
 *
 * States S_{t-1} are recomputed: the forward pass keeps the state at the
 * start of every block of BLK tokens; each block is replayed forward into a
 * buffer before it is walked backward.  The replay is the same arithmetic as
 * the first pass, so the states are bit-identical.
 *
 * Layout: as kda_oracle.c.  do_: [T_total, H, dv] double; dht, dh0:
 * [n_seqs, H, dk, dv] double (dht may be NULL = zero); gradients dq, dk, dg:
 * [T_total, H, dk]; dv: [T_total, H, dv]; dbeta: [T_total, H]; all double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define BLK 64

typedef struct {
  int64_t H, dk, dv;
  double g_floor;
  const float *q, *k, *v, *g, *beta;
} fwd_in;

/* One forward step from S (in place).  w, u: scratch of dv. */
static void step(const fwd_in* in, int64_t t, int64_t h, double* S, double* w, double* u) {
  const int64_t H = in->H, dk = in->dk, dv = in->dv;
  const float* kt = in->k + (t * H + h) * dk;
  const float* gt = in->g + (t * H + h) * dk;
  const float* vt = in->v + (t * H + h) * dv;
  const double bt = (double)in->beta[t * H + h];
  for (int64_t c = 0; c < dk; ++c) {
    double gc = (double)gt[c];
    if (gc < in->g_floor) gc = in->g_floor;
    const double a = exp(gc);
    for (int64_t j = 0; j < dv; ++j) S[c * dv + j] *= a;
  }
  for (int64_t j = 0; j < dv; ++j) w[j] = 0.0;
  for (int64_t c = 0; c < dk; ++c) {
    const double kc = (double)kt[c];
    for (int64_t j = 0; j < dv; ++j) w[j] += S[c * dv + j] * kc;
  }
  for (int64_t j = 0; j < dv; ++j) u[j] = bt * ((double)vt[j] - w[j]);
  for (int64_t c = 0; c < dk; ++c) {
    const double kc = (double)kt[c];
    for (int64_t j = 0; j < dv; ++j) S[c * dv + j] += kc * u[j];
  }
}

/* Gradient of one (sequence, head) pair over tokens [t0, t1). */
static int bwd_pair(const fwd_in* in, int64_t t0, int64_t t1, int64_t h,
                    const double* S0, const double* do_, const double* dST,
                    double* dq, double* dk_, double* dv_, double* dg, double* dbeta,
                    double* dS0) {
  const int64_t H = in->H, dk = in->dk, dv = in->dv, dd = dk * dv;
  const int64_t L = t1 - t0, nb = (L + BLK - 1) / BLK;
  double* ck = (double*)malloc(sizeof(double) * (size_t)((nb > 0 ? nb : 1) * dd));
  double* st = (double*)malloc(sizeof(double) * (size_t)((BLK + 1) * dd));
  double* dS = (double*)malloc(sizeof(double) * (size_t)dd);
  double* Sp = (double*)malloc(sizeof(double) * (size_t)dd);
  double* w = (double*)malloc(sizeof(double) * (size_t)dv);
  double* u = (double*)malloc(sizeof(double) * (size_t)dv);
  double* du = (double*)malloc(sizeof(double) * (size_t)dv);
  double* a = (double*)malloc(sizeof(double) * (size_t)dk);
  if (!ck || !st || !dS || !Sp || !w || !u || !du || !a) {
    free(ck); free(st); free(dS); free(Sp); free(w); free(u); free(du); free(a);
    return 2;
  }
  /* forward pass: the state at the start of every block */
  double* S = st;
  if (S0) memcpy(S, S0, sizeof(double) * (size_t)dd);
  else memset(S, 0, sizeof(double) * (size_t)dd);
  for (int64_t b = 0; b < nb; ++b) {
    memcpy(ck + b * dd, S, sizeof(double) * (size_t)dd);
    const int64_t e = t0 + (b + 1) * BLK < t1 ? t0 + (b + 1) * BLK : t1;
    for (int64_t t = t0 + b * BLK; t < e; ++t) step(in, t, h, S, w, u);
  }

  if (dST) memcpy(dS, dST, sizeof(double) * (size_t)dd);
  else memset(dS, 0, sizeof(double) * (size_t)dd);

  for (int64_t b = nb - 1; b >= 0; --b) {
    const int64_t s = t0 + b * BLK;
    const int64_t e = s + BLK < t1 ? s + BLK : t1;
    /* replay: st[i] = state before token s + i, st[e - s] = after the block */
    memcpy(st, ck + b * dd, sizeof(double) * (size_t)dd);
    for (int64_t t = s; t < e; ++t) {
      memcpy(st + (t - s + 1) * dd, st + (t - s) * dd, sizeof(double) * (size_t)dd);
      step(in, t, h, st + (t - s + 1) * dd, w, u);
    }
    for (int64_t t = e - 1; t >= s; --t) {
      const double* Sprev = st + (t - s) * dd;
      const double* St = st + (t - s + 1) * dd;
      const float* qt = in->q + (t * H + h) * dk;
      const float* kt = in->k + (t * H + h) * dk;
      const float* gt = in->g + (t * H + h) * dk;
      const float* vt = in->v + (t * H + h) * dv;
      const double bt = (double)in->beta[t * H + h];
      const double* dot = do_ + (t * H + h) * dv;
      double* dqt = dq + (t * H + h) * dk;
      double* dkt = dk_ + (t * H + h) * dk;
      double* dgt = dg + (t * H + h) * dk;
      double* dvt = dv_ + (t * H + h) * dv;

      /* quantities of the forward step: a, S' = diag(a) S_{t-1}, w, u */
      for (int64_t c = 0; c < dk; ++c) {
        double gc = (double)gt[c];
        if (gc < in->g_floor) gc = in->g_floor;
        a[c] = exp(gc);
        for (int64_t j = 0; j < dv; ++j) Sp[c * dv + j] = a[c] * Sprev[c * dv + j];
      }
      for (int64_t j = 0; j < dv; ++j) w[j] = 0.0;
      for (int64_t c = 0; c < dk; ++c)
        for (int64_t j = 0; j < dv; ++j) w[j] += Sp[c * dv + j] * (double)kt[c];
      for (int64_t j = 0; j < dv; ++j) u[j] = bt * ((double)vt[j] - w[j]);

      /* o_t = S_t^T q_t */
      for (int64_t c = 0; c < dk; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < dv; ++j) {
          dS[c * dv + j] += (double)qt[c] * dot[j];
          acc += St[c * dv + j] * dot[j];
        }
        dqt[c] = acc;
      }
      /* S_t = S' + k u^T */
      for (int64_t j = 0; j < dv; ++j) du[j] = 0.0;
      for (int64_t c = 0; c < dk; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < dv; ++j) {
          du[j] += dS[c * dv + j] * (double)kt[c];
          acc += dS[c * dv + j] * u[j];
        }
        dkt[c] = acc;
      }
      /* u = beta (v - w) */
      double db = 0.0;
      for (int64_t j = 0; j < dv; ++j) {
        db += du[j] * ((double)vt[j] - w[j]);
        dvt[j] = bt * du[j];
        du[j] = -bt * du[j]; /* du now holds dw */
      }
      dbeta[t * H + h] = db;
      /* w = S'^T k */
      for (int64_t c = 0; c < dk; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < dv; ++j) {
          dS[c * dv + j] += (double)kt[c] * du[j];
          acc += Sp[c * dv + j] * du[j];
        }
        dkt[c] += acc;
      }
      /* S' = diag(a) S_{t-1} */
      for (int64_t c = 0; c < dk; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < dv; ++j) {
          acc += dS[c * dv + j] * Sprev[c * dv + j];
          dS[c * dv + j] *= a[c];
        }
        dgt[c] = (double)gt[c] >= in->g_floor ? a[c] * acc : 0.0;
      }
    }
  }
  memcpy(dS0, dS, sizeof(double) * (size_t)dd);
  free(ck); free(st); free(dS); free(Sp); free(w); free(u); free(du); free(a);
  return 0;
}

/* Returns 0 on success, 1 on a bad argument, 2 on allocation failure. */
int kda_oracle_backward(int64_t n_seqs, const int64_t* cu, int64_t H,
                        int64_t dk, int64_t dv, double g_floor,
                        const float* q, const float* k, const float* v,
                        const float* g, const float* beta, const double* h0,
                        const double* do_, const double* dht,
                        double* dq, double* dk_, double* dv_, double* dg,
                        double* dbeta, double* dh0, int n_threads) {
  if (n_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu || !q || !k || !v ||
      !g || !beta || !do_ || !dq || !dk_ || !dv_ || !dg || !dbeta || !dh0)
    return 1;
  for (int64_t n = 0; n < n_seqs; ++n)
    if (cu[n + 1] < cu[n]) return 1;
  const fwd_in in = {H, dk, dv, g_floor, q, k, v, g, beta};
  const int64_t pairs = n_seqs * H;
  int status = 0;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t p = 0; p < pairs; ++p) {
    const int64_t n = p / H, h = p % H;
    const double* S0 = h0 ? h0 + p * dk * dv : NULL;
    const double* dST = dht ? dht + p * dk * dv : NULL;
    if (bwd_pair(&in, cu[n], cu[n + 1], h, S0, do_, dST, dq, dk_, dv_, dg, dbeta,
                 dh0 + p * dk * dv) != 0) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      status = 2;
    }
  }
  return status;
}
