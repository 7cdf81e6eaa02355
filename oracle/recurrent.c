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

/* oracle_head_fwd_channel -- the same stream with one log-decay per key
 * channel (g_t is a Dk-vector, advancing by sgc elements per token):
 *     d    = diag(exp(g_t)) h                decay on the key side first
 *     kd   = k_t^T d                         (Dv)
 *     h    = d - b_t k_t kd^T + b_t k_t v_t^T
 *     o_t  = h^T q_t
 * (the per-channel reading of the same update: decay, then the delta-rule
 * erase and write act on the decayed state; with every channel equal it is
 * oracle_head_fwd).  beta advances by sg elements per token. */
int oracle_head_fwd_channel(const double* q, const double* k, const double* v,
                            const double* g, const double* beta,
                            long long sq, long long sv, long long sgc, long long sg,
                            int T, int Dk, int Dv, double* h, double* o) {
  double* kd = (double*)malloc(sizeof(double) * (size_t)Dv);
  if (!kd) return 1;
  for (int t = 0; t < T; ++t) {
    const double* kt = k + (long long)t * sq;
    const double* qt = q + (long long)t * sq;
    const double* vt = v + (long long)t * sv;
    const double* gt = g + (long long)t * sgc;
    const double b = beta[(long long)t * sg];
    for (int j = 0; j < Dv; ++j) kd[j] = 0.0;
    for (int i = 0; i < Dk; ++i) {
      const double a = exp(gt[i]);
      const double ki = kt[i];
      double* hi = h + (long long)i * Dv;
      for (int j = 0; j < Dv; ++j) {
        hi[j] *= a;
        kd[j] += ki * hi[j];
      }
    }
    if (o) {
      double* ot = o + (long long)t * Dv;
      for (int j = 0; j < Dv; ++j) ot[j] = 0.0;
      for (int i = 0; i < Dk; ++i) {
        const double bki = b * kt[i];
        const double qi = qt[i];
        double* hi = h + (long long)i * Dv;
        for (int j = 0; j < Dv; ++j) {
          const double x = hi[j] - bki * kd[j] + bki * vt[j];
          hi[j] = x;
          ot[j] += qi * x;
        }
      }
    } else {
      for (int i = 0; i < Dk; ++i) {
        const double bki = b * kt[i];
        double* hi = h + (long long)i * Dv;
        for (int j = 0; j < Dv; ++j) hi[j] = hi[j] - bki * kd[j] + bki * vt[j];
      }
    }
  }
  free(kd);
  return 0;
}

/* One token of the scalar-gate recurrence on state h (in place). */
static void step_fwd(const double* kt, const double* vt, double a, double b, int Dk, int Dv,
                     double* h, double* kh) {
  for (int j = 0; j < Dv; ++j) kh[j] = 0.0;
  for (int i = 0; i < Dk; ++i) {
    const double ki = kt[i];
    const double* hi = h + (long long)i * Dv;
    for (int j = 0; j < Dv; ++j) kh[j] += ki * hi[j];
  }
  for (int i = 0; i < Dk; ++i) {
    const double bki = b * kt[i];
    double* hi = h + (long long)i * Dv;
    for (int j = 0; j < Dv; ++j) hi[j] = a * (hi[j] - bki * kh[j]) + bki * vt[j];
  }
}

/* oracle_head_bwd -- reverse mode of oracle_head_fwd for one stream: the
 * gradients of L = <o, do> + <h_T, dh_T> with respect to q, k, v, g, beta and
 * the initial state, by the chain rule applied to each step of the
 * recurrence, walked backwards.  With h_p the state before step t, h_t after
 * it, a = exp(g_t), b = beta_t and dh the gradient flowing into h_t:
 *     dh   += q_t do_t^T                    (o_t = h_t^T q_t)
 *     dq_t  = h_t do_t
 *     c     = k_t^T h_p,  e = h_p - b k_t c^T   (h_t = a e + b k_t v_t^T)
 *     dg_t  = a <dh, e>,  dv_t = b dh^T k_t
 *     de    = a dh,       kde = k_t^T de
 *     dbeta_t = k_t^T dh v_t - kde . c
 *     dk_t  = b (dh v_t - de c - h_p kde)
 *     dh    <- de - b k_t kde^T             (the gradient flowing into h_p)
 * States are recomputed forward from checkpoints every `seg` tokens.  h0
 * (Dk*Dv) may be NULL (zeros); dh holds dh_T on entry (zeros allowed) and the
 * gradient of h0 on return.  Strides as oracle_head_fwd; do advances by sv. */
int oracle_head_bwd(const double* q, const double* k, const double* v,
                    const double* g, const double* beta, const double* dout,
                    long long sq, long long sv, long long sg, int T, int Dk, int Dv,
                    const double* h0, double* dh, double* dq, double* dk, double* dv,
                    double* dg, double* dbeta, int seg) {
  const long long S = (long long)Dk * Dv;
  if (seg < 1) seg = 1;
  const int nseg = (T + seg - 1) / seg;
  double* ck = (double*)malloc(sizeof(double) * (size_t)(S * (nseg > 0 ? nseg : 1)));
  double* st = (double*)malloc(sizeof(double) * (size_t)(S * (seg + 1)));
  double* tmp = (double*)malloc(sizeof(double) * (size_t)(4 * Dv + S));
  if (!ck || !st || !tmp) { free(ck); free(st); free(tmp); return 1; }
  double* kh = tmp;
  double* c = tmp + Dv;
  double* kde = tmp + 2 * Dv;
  double* de = tmp + 4 * Dv;
  /* forward: checkpoints at every segment start */
  double* h = st;
  for (long long x = 0; x < S; ++x) h[x] = h0 ? h0[x] : 0.0;
  for (int s = 0; s < nseg; ++s) {
    for (long long x = 0; x < S; ++x) ck[s * S + x] = h[x];
    const int t1 = (s + 1) * seg < T ? (s + 1) * seg : T;
    for (int t = s * seg; t < t1; ++t)
      step_fwd(k + t * sq, v + t * sv, exp(g[t * sg]), beta[t * sg], Dk, Dv, h, kh);
  }
  /* backward, segment by segment */
  for (int s = nseg - 1; s >= 0; --s) {
    const int t0 = s * seg, t1 = (s + 1) * seg < T ? (s + 1) * seg : T;
    for (long long x = 0; x < S; ++x) st[x] = ck[s * S + x];
    for (int t = t0; t < t1; ++t) {
      double* hn = st + (long long)(t - t0 + 1) * S;
      for (long long x = 0; x < S; ++x) hn[x] = st[(long long)(t - t0) * S + x];
      step_fwd(k + t * sq, v + t * sv, exp(g[t * sg]), beta[t * sg], Dk, Dv, hn, kh);
    }
    for (int t = t1 - 1; t >= t0; --t) {
      const double* hp = st + (long long)(t - t0) * S;
      const double* ht = hp + S;
      const double* qt = q + t * sq;
      const double* kt = k + t * sq;
      const double* vt = v + t * sv;
      const double* dot = dout + t * sv;
      const double a = exp(g[t * sg]), b = beta[t * sg];
      for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) dh[(long long)i * Dv + j] += qt[i] * dot[j];
      for (int i = 0; i < Dk; ++i) {
        double sacc = 0.0;
        for (int j = 0; j < Dv; ++j) sacc += ht[(long long)i * Dv + j] * dot[j];
        dq[t * sq + i] = sacc;
      }
      for (int j = 0; j < Dv; ++j) c[j] = 0.0;
      for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) c[j] += kt[i] * hp[(long long)i * Dv + j];
      double dgs = 0.0;
      for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) {
          const double e = hp[(long long)i * Dv + j] - b * kt[i] * c[j];
          dgs += dh[(long long)i * Dv + j] * e;
        }
      dg[t * sg] = a * dgs;
      for (int j = 0; j < Dv; ++j) {
        double sacc = 0.0;
        for (int i = 0; i < Dk; ++i) sacc += dh[(long long)i * Dv + j] * kt[i];
        dv[t * sv + j] = b * sacc;
      }
      for (long long x = 0; x < S; ++x) de[x] = a * dh[x];
      for (int j = 0; j < Dv; ++j) kde[j] = 0.0;
      for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) kde[j] += kt[i] * de[(long long)i * Dv + j];
      double db1 = 0.0, db2 = 0.0;
      for (int i = 0; i < Dk; ++i) {
        double r = 0.0;
        for (int j = 0; j < Dv; ++j) r += dh[(long long)i * Dv + j] * vt[j];
        db1 += kt[i] * r;
      }
      for (int j = 0; j < Dv; ++j) db2 += kde[j] * c[j];
      dbeta[t * sg] = db1 - db2;
      for (int i = 0; i < Dk; ++i) {
        double r1 = 0.0, r2 = 0.0, r3 = 0.0;
        for (int j = 0; j < Dv; ++j) {
          r1 += dh[(long long)i * Dv + j] * vt[j];
          r2 += de[(long long)i * Dv + j] * c[j];
          r3 += hp[(long long)i * Dv + j] * kde[j];
        }
        dk[t * sq + i] = b * (r1 - r2 - r3);
      }
      for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j)
          dh[(long long)i * Dv + j] = de[(long long)i * Dv + j] - b * kt[i] * kde[j];
    }
  }
  free(ck);
  free(st);
  free(tmp);
  return 0;
}
