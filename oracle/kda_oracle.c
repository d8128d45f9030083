/*
 * kda_oracle.c -- plain fp64 CPU oracle for the Kimi Delta Attention (KDA)
 * forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The GPU product path
 * never links, imports or calls it, and it shares no code, header, table or
 * helper with the HIP sources.
 *
 * Citation key (the pages this follows):
 *   P1 = blog post "FlashKDA：月之暗面开源的 Kimi Delta Attention 高性能内核"
 *        (guancyxx.cn).  §一 gives the gated recurrent state update with a
 *        decay gate g, a sigmoid weight beta and a [K,V] state; §二 2.2 lists
 *        the per-token stages (gate activation, L2 normalisation, decay,
 *        delta-rule recurrence, output).
 *   P2 = FlashKDA README mirror (ai-feeds.com), section "内核 API" (Kernel API):
 *        the argument table of flash_kda.fwd (shapes, dtypes, the K = V = 128
 *        rule, the [B|N, H, V, K] state layout, the cu_seqlens rule) and the
 *        chunk_kda call in "将 FlashKDA 用作 FLA 后端" with the in-kernel gate,
 *        L2-norm, sigmoid and transposed-state flags.
 *
 * What is computed (token by token, no chunking, all in fp64):
 *   for every sequence n and head h, with the K x V state S (math layout,
 *   S[i][j], i = key channel, j = value channel):
 *     a_t[i]  = lower_bound * sigmoid(exp(A_log[h]) * (g_t[i] + dt_bias[h][i]))
 *     beta_t  = sigmoid(beta_logit_t)
 *     kn_t    = k_t / sqrt(|k_t|^2 + eps)
 *     qn_t    = scale * q_t / sqrt(|q_t|^2 + eps)
 *     S      <- diag(exp(a_t)) S                     (decay each key channel)
 *     r       = v_t - S^T kn_t                        (delta-rule residual)
 *     S      <- S + beta_t kn_t r^T                   (rank-1 correction)
 *     o_t     = S^T qn_t                              (read-out after update)
 *   The pages print only a simplified form of this update (P1 §一, scalar
 *   gate, no correction); the per-channel gate shape (P2 Kernel API, g is
 *   [B,T,H,K]) and the "delta rule" wording of P1 §二 2.2 fix the full form.
 *   The gate activation formula itself is not printed anywhere: the reading
 *   taken is the bounded sigmoid form above, which maps any raw gate into
 *   (lower_bound, 0) as P1 §二 2.1 and the lower_bound row of P2's table need.
 *   eps = 1e-6 sits inside the square root (not stated on the pages).
 *
 * Layouts (P2 Kernel API):
 *   q, k, g : bf16 bit patterns, [B, T, H, K]
 *   v       : bf16 bit patterns, [B, T, H, V]
 *   beta    : bf16 bit patterns, [B, T, H]
 *   A_log   : fp32 [H];  dt_bias : fp32 [H, K]
 *   state   : fp64 [Nseq, H, V, K]  (stored [n,h,j,i] = S[i][j]: V-major,
 *             K contiguous, the transposed-state layout of P2)
 *   out     : fp64 [B, T, H, V]
 *   cu_seqlens (optional, int64 [Nseq+1]): then B must be 1 and sequence n is
 *   tokens [cu[n], cu[n+1]) of batch row 0; without it, sequence n = batch
 *   row n over all T tokens (P2 Kernel API notes).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDA_ORACLE_EPS 1e-6

/* bf16 -> fp64, exact: a bf16 value is the upper 16 bits of an fp32. */
static double bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Gate activation (reading: bounded sigmoid form, see file header). */
static double gate_activation(double g, double A_log, double dt_bias, double lower_bound) {
  return lower_bound * sigmoid(exp(A_log) * (g + dt_bias));
}

/* One (sequence, head) pair: tokens [t0, t1) of batch row b. */
static void run_pair(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
                     const uint16_t* beta, double scale, const float* A_log, const float* dt_bias,
                     double lower_bound, const double* s_in, double* out, double* s_out,
                     int64_t b, int64_t t0, int64_t t1, int64_t h, int64_t T, int64_t H, int64_t K,
                     int64_t V, double* S, double* work) {
  double* qn = work;
  double* kn = qn + K;
  double* a = kn + K;
  double* r = a + K;
  double* vv = r + V;

  for (int64_t i = 0; i < K; ++i)
    for (int64_t j = 0; j < V; ++j) S[i * V + j] = s_in ? s_in[j * K + i] : 0.0;

  for (int64_t t = t0; t < t1; ++t) {
    const int64_t row = (b * T + t) * H + h; /* token-head index */
    const uint16_t* qt = q + row * K;
    const uint16_t* kt = k + row * K;
    const uint16_t* gt = g + row * K;
    const uint16_t* vt = v + row * V;

    /* gate, beta, L2 normalisation */
    double sq = 0.0, sk = 0.0;
    for (int64_t i = 0; i < K; ++i) {
      const double qi = bf16_to_f64(qt[i]), ki = bf16_to_f64(kt[i]);
      qn[i] = qi;
      kn[i] = ki;
      sq += qi * qi;
      sk += ki * ki;
      a[i] = gate_activation(bf16_to_f64(gt[i]), (double)A_log[h], (double)dt_bias[h * K + i],
                             lower_bound);
    }
    const double rq = scale / sqrt(sq + KDA_ORACLE_EPS);
    const double rk = 1.0 / sqrt(sk + KDA_ORACLE_EPS);
    for (int64_t i = 0; i < K; ++i) {
      qn[i] *= rq;
      kn[i] *= rk;
    }
    const double bt = sigmoid(bf16_to_f64(beta[row]));
    for (int64_t j = 0; j < V; ++j) vv[j] = bf16_to_f64(vt[j]);

    /* decay: S <- diag(exp(a)) S */
    for (int64_t i = 0; i < K; ++i) {
      const double d = exp(a[i]);
      for (int64_t j = 0; j < V; ++j) S[i * V + j] *= d;
    }
    /* residual r = v - S^T kn */
    for (int64_t j = 0; j < V; ++j) r[j] = vv[j];
    for (int64_t i = 0; i < K; ++i)
      for (int64_t j = 0; j < V; ++j) r[j] -= S[i * V + j] * kn[i];
    /* rank-1 correction S <- S + beta kn r^T */
    for (int64_t i = 0; i < K; ++i) {
      const double c = bt * kn[i];
      for (int64_t j = 0; j < V; ++j) S[i * V + j] += c * r[j];
    }
    /* read-out o = S^T qn */
    double* ot = out + row * V;
    for (int64_t j = 0; j < V; ++j) ot[j] = 0.0;
    for (int64_t i = 0; i < K; ++i)
      for (int64_t j = 0; j < V; ++j) ot[j] += S[i * V + j] * qn[i];
  }

  if (s_out)
    for (int64_t i = 0; i < K; ++i)
      for (int64_t j = 0; j < V; ++j) s_out[j * K + i] = S[i * V + j];
}

/*
 * Returns 0 on success, 1 on bad arguments, 2 on allocation failure.
 * initial_state / final_state may be NULL (P2 Kernel API: state None).
 * nthreads <= 0 means the OpenMP default.
 */
int kda_oracle_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
                   const uint16_t* beta, double scale, const float* A_log, const float* dt_bias,
                   double lower_bound, const double* initial_state, double* out,
                   double* final_state, const int64_t* cu_seqlens, int64_t num_seqs, int64_t B,
                   int64_t T, int64_t H, int64_t K, int64_t V, int nthreads) {
  if (B < 0 || T < 0 || H < 1 || K < 1 || V < 1) return 1;
  if (cu_seqlens && B != 1) return 1;
  const int64_t N = cu_seqlens ? num_seqs : B;
  if (N < 0) return 1;
  if (cu_seqlens) {
    if (cu_seqlens[0] != 0 || cu_seqlens[N] != T) return 1;
    for (int64_t n = 0; n < N; ++n)
      if (cu_seqlens[n + 1] < cu_seqlens[n]) return 1;
  }
  const int64_t pairs = N * H;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel reduction(| : failed)
#endif
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)(K * V));
    double* work = (double*)malloc(sizeof(double) * (size_t)(3 * K + 2 * V));
    if (!S || !work) {
      failed = 1;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
      for (int64_t p = 0; p < pairs; ++p) {
        const int64_t n = p / H, h = p % H;
        const int64_t b = cu_seqlens ? 0 : n;
        const int64_t t0 = cu_seqlens ? cu_seqlens[n] : 0;
        const int64_t t1 = cu_seqlens ? cu_seqlens[n + 1] : T;
        const double* s_in = initial_state ? initial_state + (n * H + h) * V * K : NULL;
        double* s_out = final_state ? final_state + (n * H + h) * V * K : NULL;
        run_pair(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, s_in, out, s_out, b, t0,
                 t1, h, T, H, K, V, S, work);
      }
    }
    free(S);
    free(work);
  }
  return failed ? 2 : 0;
}

/* The number of threads an OpenMP parallel region would use (for reports). */
int kda_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
