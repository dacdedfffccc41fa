/*
 * KDA (Kimi Delta Attention) reference recurrence -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the oracle that the HIP library is checked against.  Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the HIP path.
 *
 * What it computes, per (sequence, head), token by token, in IEEE fp64:
 *
 *   a_t   = exp(max(g_t, g_floor))                 per key channel
 *   S'    = diag(a_t) S_{t-1}                      decay (channel-wise gate)
 *   u_t   = beta_t (v_t - S'^T k_t)                delta-rule error
 *   S_t   = S' + k_t u_t^T                         erase-then-write
 *   o_t   = S_t^T q_t                              read after the write
 *
 * which is S_t = (I - beta_t k_t k_t^T) diag(a_t) S_{t-1} + beta_t k_t v_t^T.
 *
 * Sources:
 *  - Delta rule S_t = S_{t-1}(I - b k k^T) + b k v^T, erase before write and
 *    output read from the updated state: "Kimi K3 深度拆解" (chenxutan.com),
 *    section 4.2 "线性注意力与 Delta Rule" (update formula and the toy
 *    single-head loop, whose state is [d, d_v] and whose output is q @ S).
 *  - Channel-wise forget gate (one rate per key channel instead of one per
 *    head): "Kimi K3 技術報告：三個架構改動一次看懂" (akiraxclaw.com), section
 *    "長度：KDA 為什麼還要搭配 Gated MLA？".
 *  - Lower bound on the per-step log-decay: "3 分钟看懂 Kimi K3"
 *    (landx.limxdynamics.com), section "第一条主线", Figure 3 caption; and
 *    "Kimi K3 发布 47 页技术报告" (163.com), section 01.
 *  The pages do not fix where the gate sits relative to the erase; this file
 *  decays first, then erases and writes (the gated form written above).
 *
 * Layout (all row-major, innermost dimension last):
 *   q, k, g : [T_total, H, dk]   float (bf16 inputs are passed up-converted)
 *   v       : [T_total, H, dv]   float
 *   beta    : [T_total, H]       float
 *   h0, ht  : [n_seqs, H, dk, dv] double (h0 may be NULL = zero state)
 *   o       : [T_total, H, dv]   double
 * Sequence n owns packed tokens [cu[n], cu[n+1]).
 *
 * Deliberately plain: no blocking, no fast-math.  The loops over the state
 * run row by row with the value index innermost so that each sum over the key
 * index is accumulated in the natural order c = 0, 1, 2, ...
 * OpenMP splits only the independent (sequence, head) pairs, so the result
 * does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void kda_pair(int64_t t0, int64_t t1, int64_t h, int64_t H,
                     int64_t dk, int64_t dv, double g_floor,
                     const float* q, const float* k, const float* v,
                     const float* g, const float* beta,
                     const double* S0, double* S, double* o,
                     double* w, double* u) {
  if (S0)
    memcpy(S, S0, sizeof(double) * (size_t)(dk * dv));
  else
    memset(S, 0, sizeof(double) * (size_t)(dk * dv));

  for (int64_t t = t0; t < t1; ++t) {
    const float* qt = q + (t * H + h) * dk;
    const float* kt = k + (t * H + h) * dk;
    const float* gt = g + (t * H + h) * dk;
    const float* vt = v + (t * H + h) * dv;
    const double bt = (double)beta[t * H + h];
    double* ot = o + (t * H + h) * dv;

    /* S' = diag(exp(max(g, floor))) S */
    for (int64_t c = 0; c < dk; ++c) {
      double gc = (double)gt[c];
      if (gc < g_floor) gc = g_floor;
      const double a = exp(gc);
      for (int64_t j = 0; j < dv; ++j) S[c * dv + j] *= a;
    }
    /* w = S'^T k */
    for (int64_t j = 0; j < dv; ++j) w[j] = 0.0;
    for (int64_t c = 0; c < dk; ++c) {
      const double kc = (double)kt[c];
      for (int64_t j = 0; j < dv; ++j) w[j] += S[c * dv + j] * kc;
    }
    /* u = beta (v - w) */
    for (int64_t j = 0; j < dv; ++j) u[j] = bt * ((double)vt[j] - w[j]);
    /* S = S' + k u^T */
    for (int64_t c = 0; c < dk; ++c) {
      const double kc = (double)kt[c];
      for (int64_t j = 0; j < dv; ++j) S[c * dv + j] += kc * u[j];
    }
    /* o = S^T q */
    for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;
    for (int64_t c = 0; c < dk; ++c) {
      const double qc = (double)qt[c];
      for (int64_t j = 0; j < dv; ++j) ot[j] += S[c * dv + j] * qc;
    }
  }
}

/* Returns 0 on success, 1 on a bad argument, 2 on allocation failure. */
int kda_oracle_forward(int64_t n_seqs, const int64_t* cu, int64_t H,
                       int64_t dk, int64_t dv, double g_floor,
                       const float* q, const float* k, const float* v,
                       const float* g, const float* beta, const double* h0,
                       double* o, double* ht, int n_threads) {
  if (n_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu || !q || !k || !v ||
      !g || !beta || !o || !ht)
    return 1;
  for (int64_t n = 0; n < n_seqs; ++n)
    if (cu[n + 1] < cu[n]) return 1;

  const int64_t pairs = n_seqs * H;
  int status = 0;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t p = 0; p < pairs; ++p) {
    const int64_t n = p / H, h = p % H;
    double* w = (double*)malloc(sizeof(double) * (size_t)dv);
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    if (w && u) {
      const double* S0 = h0 ? h0 + p * dk * dv : NULL;
      kda_pair(cu[n], cu[n + 1], h, H, dk, dv, g_floor, q, k, v, g, beta, S0,
               ht + p * dk * dv, o, w, u);
    } else {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      status = 2;
    }
    free(w);
    free(u);
  }
  return status;
}

int kda_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
