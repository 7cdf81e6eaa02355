/* recurrent.c -- the gated delta-rule recurrence in plain C, fp64.
 *
 * TEST INFRASTRUCTURE ONLY (see linattn_oracle.py's header): only the tests,
 * the package smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code with the HIP library.
 *
 * Same definition as linattn_oracle.recurrent_fwd, token by token, with the
 * state stored as h = S^T (Dk x Dv, row-major):
 *     kh   = k_t^T h                        (Dv)
 *     h    = a_t (h - b_t k_t kh^T) + b_t k_t v_t^T,   a_t = exp(g_t)
 *     o_t  = h^T q_t                        (after the update)
 * ("Evaluating Next-Gen Sparse MoE and Long-Context LLMs", sec. 2 item 2: a
 * fixed-size matrix state, delta-rule write, data-dependent decay.)
 *
 * oracle_head_fwd runs one (batch, head) stream over T tokens.  q, k, v point
 * at the stream's first token and advance by the given strides (in elements)
 * per token; g and beta likewise.  h (Dk*Dv doubles) is the state, read and
 * overwritten.  o receives T*Dv doubles (or nothing when NULL).
 */
#include <math.h>
#include <stdlib.h>

int oracle_head_fwd(const double* q, const double* k, const double* v,
                    const double* g, const double* beta,
                    long long sq, long long sv, long long sg,
                    int T, int Dk, int Dv, double* h, double* o) {
  double* kh = (double*)malloc(sizeof(double) * (size_t)Dv);
  if (!kh) return 1;
  for (int t = 0; t < T; ++t) {
    const double* kt = k + (long long)t * sq;
    const double* qt = q + (long long)t * sq;
    const double* vt = v + (long long)t * sv;
    const double a = exp(g[(long long)t * sg]);
    const double b = beta[(long long)t * sg];
    for (int j = 0; j < Dv; ++j) kh[j] = 0.0;
    for (int i = 0; i < Dk; ++i) {
      const double ki = kt[i];
      const double* hi = h + (long long)i * Dv;
      for (int j = 0; j < Dv; ++j) kh[j] += ki * hi[j];
    }
    /* update the state; with o, accumulate o_t = h_t^T q_t in the same pass */
    if (o) {
      double* ot = o + (long long)t * Dv;
      for (int j = 0; j < Dv; ++j) ot[j] = 0.0;
      for (int i = 0; i < Dk; ++i) {
        const double bki = b * kt[i];
        const double qi = qt[i];
        double* hi = h + (long long)i * Dv;
        for (int j = 0; j < Dv; ++j) {
          const double x = a * (hi[j] - bki * kh[j]) + bki * vt[j];
          hi[j] = x;
          ot[j] += qi * x;
        }
      }
    } else {
      for (int i = 0; i < Dk; ++i) {
        const double bki = b * kt[i];
        double* hi = h + (long long)i * Dv;
        for (int j = 0; j < Dv; ++j) hi[j] = a * (hi[j] - bki * kh[j]) + bki * vt[j];
      }
    }
  }
  free(kh);
  return 0;
}
