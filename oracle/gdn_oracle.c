/*
 * fp64 CPU oracle of the gated delta rule, token by token.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  It shares no code with the
 * HIP library and is never on the product path.
 *
 * What it computes ("SuffixReplay", Theoretical Foundation, Eq. 4; "Tail-Replay"
 * section 2 for the gate in (0,1] and the rank-one correction):
 *
 *   S_t = A_t(S_{t-1}) + B_t,   S_0 = 0 (or a given initial state),
 *
 * with, per sequence n and value head h, S a d_v x d_k matrix and
 *
 *   erase mode (Gated DeltaNet):
 *       S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T
 *           = a_t S_{t-1} - a_t b_t (S_{t-1} k_t) k_t^T + b_t v_t k_t^T
 *   erase-free mode (scalar per-head decay, Mamba2 style):
 *       S_t = a_t S_{t-1} + b_t v_t k_t^T
 *   optional output after the update:  o_t = scale * S_t q_t.
 *
 * Value head h reads key/query head h / (h_v / h_k).  Inputs are the stored
 * values widened exactly to double by the caller (bf16, fp16 and fp32 all
 * widen exactly), or fp64 intermediates of the group oracle; every operation
 * below is done in double precision, in the order written, with no blocking
 * or reordering.  The final state is returned transposed, as
 * [d_k][d_v] per (sequence, value head).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation failure. */
int oracle_gdn_f64(int32_t n_seqs, const int32_t* cu, int32_t h_k, int32_t h_v,
                   int32_t d_k, int32_t d_v, const double* q, const double* k,
                   const double* v, const double* alpha, int32_t alpha_is_log,
                   const double* beta, int32_t erase, double scale,
                   const double* initial_state, double* final_state, double* o,
                   int32_t n_threads) {
  if (n_seqs < 0 || h_k <= 0 || h_v <= 0 || d_k <= 0 || d_v <= 0) return -1;
  if (h_v % h_k != 0) return -1;
  if (!cu || !k || !v || !alpha || !final_state) return -1;
  if (o && !q) return -1;
  const int32_t group = h_v / h_k;
  const int64_t units = (int64_t)n_seqs * h_v;
  int failed = 0;
#ifdef _OPENMP
  if (n_threads <= 0) n_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
#endif
  for (int64_t u = 0; u < units; ++u) {
    const int32_t n = (int32_t)(u / h_v);
    const int32_t h = (int32_t)(u % h_v);
    const int32_t g = h / group;
    double* S = (double*)malloc(sizeof(double) * (size_t)d_v * d_k);  /* S[i][j] */
    double* x = (double*)malloc(sizeof(double) * (size_t)d_v);
    if (!S || !x) {
      free(S);
      free(x);
#ifdef _OPENMP
#pragma omp atomic write
#endif
      failed = 1;
      continue;
    }
    /* S_0: the stored initial state is [d_k][d_v]; S is [d_v][d_k]. */
    for (int32_t i = 0; i < d_v; ++i)
      for (int32_t j = 0; j < d_k; ++j)
        S[(size_t)i * d_k + j] =
            initial_state
                ? initial_state[(((size_t)n * h_v + h) * d_k + j) * d_v + i]
                : 0.0;
    for (int32_t t = cu[n]; t < cu[n + 1]; ++t) {
      const double a = alpha_is_log ? exp(alpha[(size_t)t * h_v + h])
                                    : alpha[(size_t)t * h_v + h];
      const double b = beta ? beta[(size_t)t * h_v + h] : 1.0;
      const double* kk = k + ((size_t)t * h_k + g) * d_k;
      const double* vv = v + ((size_t)t * h_v + h) * d_v;
      if (erase) {
        for (int32_t i = 0; i < d_v; ++i) { /* x = S_{t-1} k_t */
          double acc = 0.0;
          for (int32_t j = 0; j < d_k; ++j) acc += S[(size_t)i * d_k + j] * kk[j];
          x[i] = acc;
        }
        for (int32_t i = 0; i < d_v; ++i) {
          const double ax = a * b * x[i];
          const double bv = b * vv[i];
          for (int32_t j = 0; j < d_k; ++j) {
            const double kj = kk[j];
            S[(size_t)i * d_k + j] = a * S[(size_t)i * d_k + j] - ax * kj + bv * kj;
          }
        }
      } else {
        for (int32_t i = 0; i < d_v; ++i) {
          const double bv = b * vv[i];
          for (int32_t j = 0; j < d_k; ++j)
            S[(size_t)i * d_k + j] = a * S[(size_t)i * d_k + j] + bv * kk[j];
        }
      }
      if (o) { /* o_t = scale * S_t q_t */
        const double* qq = q + ((size_t)t * h_k + g) * d_k;
        double* oo = o + ((size_t)t * h_v + h) * d_v;
        for (int32_t i = 0; i < d_v; ++i) {
          double acc = 0.0;
          for (int32_t j = 0; j < d_k; ++j) acc += S[(size_t)i * d_k + j] * qq[j];
          oo[i] = scale * acc;
        }
      }
    }
    for (int32_t j = 0; j < d_k; ++j)
      for (int32_t i = 0; i < d_v; ++i)
        final_state[(((size_t)n * h_v + h) * d_k + j) * d_v + i] = S[(size_t)i * d_k + j];
    free(S);
    free(x);
  }
  return failed ? -2 : 0;
}
