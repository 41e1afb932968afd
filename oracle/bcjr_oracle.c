/*
 * Plain CPU oracle for BCJR-QAT soft trellis decoding -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg load this
 * file's library. The product path (the HIP library) never calls it and shares no code
 * with it.
 *
 * Source of the method: "BCJR-QAT: A Differentiable Relaxation of Trellis-Coded Weight
 * Quantization" (V. Iyengar, arXiv 2605.10655), as summarised on
 *   - the paper abstract (gptget.net/papers/2605.10655, "Abstract"): Viterbi's argmax over
 *     trellis paths is replaced by the BCJR forward-backward sum-product recursion at
 *     temperature T; the soft codeword is the Boltzmann expectation over trellis paths; it
 *     is exactly differentiable; T -> 0 recovers the hard code; the computation is the
 *     transfer-matrix computation of a 1D Ising-like chain;
 *   - the gist.science technical summary, "Core mechanism" (soft codeword
 *     w_hat_t(T) = sum_s c(s) p_T(s_t = s | w)) and "Key technical innovations"
 *     (forward-backward recursions, O(L*S^2), exact gradients, fp32 parity).
 *
 * The pages never write the energy or the trellis shape. The readings used here:
 *   energy of a path s_1..s_L:  E = sum_t (w_t - c(s_t))^2  [dense: - sum_t theta(s_{t-1}, s_t)],
 *   path weight exp(-E / T), natural log throughout, free start and free end state;
 *   bitshift trellis with S = 2^n states and K = 2^k branches, s' = ((s << k) | b) & (S-1);
 *   dense trellis: every state may follow every state, transition log-potential theta/T.
 *
 * Everything is computed in double precision, state by state, in the order the method
 * states it (alpha, beta, posterior, soft codeword, then the gradient recursions). The
 * only exception is the Viterbi decoder, which is deliberately fp32 with no contraction so
 * that the GPU decoder can be checked bit for bit (op order in the function's comment).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------------------------------- */
/* Trellis view: one description shared by the bitshift and the dense trellis.               */
/* ---------------------------------------------------------------------------------------- */
typedef struct {
  int S;             /* number of states                                                  */
  int dense;         /* 0: bitshift trellis (n, k); 1: fully connected with phi = theta/T   */
  int n, k;          /* bitshift parameters                                               */
  int npred;         /* predecessors per state: K for bitshift, S for dense                 */
  const double* phi; /* dense only: phi[s*S + s'] = theta(s, s') / T                         */
} tview;

/* a-th predecessor of state sp, a increasing. Bitshift: (sp >> k) | (a << (n-k)). */
static int pred_state(const tview* v, int sp, int a) {
  if (v->dense) return a;
  return (sp >> v->k) | (a << (v->n - v->k));
}
/* b-th successor of state s. Bitshift: ((s << k) | b) & (S-1). */
static int succ_state(const tview* v, int s, int b) {
  if (v->dense) return b;
  return ((s << v->k) | b) & (v->S - 1);
}
/* log-potential of the edge s -> sp (0 on every bitshift edge). */
static double edge_phi(const tview* v, int s, int sp) {
  if (v->dense) return v->phi[(size_t)s * (size_t)v->S + (size_t)sp];
  return 0.0;
}

/* log(sum_i exp(x_i)) with the largest term factored out. */
static double lse(const double* x, int m) {
  double mx = -INFINITY;
  for (int i = 0; i < m; ++i)
    if (x[i] > mx) mx = x[i];
  if (mx == -INFINITY) return -INFINITY;
  double s = 0.0;
  for (int i = 0; i < m; ++i) s += exp(x[i] - mx);
  return mx + log(s);
}

/* Per-sequence scratch of the forward-backward. */
typedef struct {
  double* ell;   /* [L][S] emission log-potentials        */
  double* alpha; /* [L][S]                                */
  double* beta;  /* [L][S]                                */
  double* tmp;   /* [npred]                               */
} fb_buf;

static int fb_alloc(fb_buf* b, long L, int S, int npred) {
  size_t LS = (size_t)L * (size_t)S;
  b->ell = (double*)malloc(LS * sizeof(double));
  b->alpha = (double*)malloc(LS * sizeof(double));
  b->beta = (double*)malloc(LS * sizeof(double));
  b->tmp = (double*)malloc((size_t)npred * sizeof(double));
  return (b->ell && b->alpha && b->beta && b->tmp) ? 0 : -1;
}
static void fb_free(fb_buf* b) {
  free(b->ell);
  free(b->alpha);
  free(b->beta);
  free(b->tmp);
}

/*
 * Forward-backward of one sequence (abstract: BCJR forward-backward sum-product at
 * temperature T; technical summary: forward-backward recursions).
 *   ell_t(s)   = -(w_t - c(s))^2 / T
 *   alpha_1(s) = ell_1(s);  alpha_t(s') = ell_t(s') + LSE_{s in pred(s')} (alpha_{t-1}(s) + phi(s,s'))
 *   beta_L(s)  = 0;         beta_t(s)   = LSE_{s' in succ(s)} (phi(s,s') + ell_{t+1}(s') + beta_{t+1}(s'))
 *   log Z      = LSE_s alpha_L(s)
 * Returns log Z.
 */
static double fb_sequence(const tview* v, const float* c, const float* w, long L, double T,
                          fb_buf* b) {
  const int S = v->S, P = v->npred;
  for (long t = 0; t < L; ++t)
    for (int s = 0; s < S; ++s) {
      double d = (double)w[t] - (double)c[s];
      b->ell[t * S + s] = -(d * d) / T;
    }
  for (int s = 0; s < S; ++s) b->alpha[s] = b->ell[s];
  for (long t = 1; t < L; ++t)
    for (int sp = 0; sp < S; ++sp) {
      for (int a = 0; a < P; ++a) {
        int s = pred_state(v, sp, a);
        b->tmp[a] = b->alpha[(t - 1) * S + s] + edge_phi(v, s, sp);
      }
      b->alpha[t * S + sp] = b->ell[t * S + sp] + lse(b->tmp, P);
    }
  for (int s = 0; s < S; ++s) b->beta[(L - 1) * S + s] = 0.0;
  for (long t = L - 2; t >= 0; --t)
    for (int s = 0; s < S; ++s) {
      for (int bb = 0; bb < P; ++bb) {
        int sp = succ_state(v, s, bb);
        b->tmp[bb] = edge_phi(v, s, sp) + b->ell[(t + 1) * S + sp] + b->beta[(t + 1) * S + sp];
      }
      b->beta[t * S + s] = lse(b->tmp, P);
    }
  return lse(b->alpha + (size_t)(L - 1) * S, S);
}

/*
 * Posterior and soft codeword (technical summary, "Core mechanism"):
 *   gamma_t(s) = exp(alpha_t(s) + beta_t(s) - log Z),  w_hat_t = sum_s c(s) gamma_t(s).
 */
static void posterior(const tview* v, const float* c, long L, const fb_buf* b, double logz,
                      double* gamma /* [L][S] or NULL */, double* what /* [L] */) {
  const int S = v->S;
  for (long t = 0; t < L; ++t) {
    double acc = 0.0;
    for (int s = 0; s < S; ++s) {
      double g = exp(b->alpha[t * S + s] + b->beta[t * S + s] - logz);
      if (gamma) gamma[t * S + s] = g;
      acc += (double)c[s] * g;
    }
    what[t] = acc;
  }
}

static int set_view(tview* v, int n, int k) {
  if (n < 1 || n > 20 || k < 1 || k > n) return -1;
  v->S = 1 << n;
  v->dense = 0;
  v->n = n;
  v->k = k;
  v->npred = 1 << k;
  v->phi = NULL;
  return 0;
}

/* ---------------------------------------------------------------------------------------- */
/* Forward: soft codeword, log Z, optional posterior / alpha / beta dumps.                    */
/* ---------------------------------------------------------------------------------------- */
static int forward_impl(const tview* v, const float* c, const float* w, long B, long L, double T,
                        double* what, double* logz, double* gamma, double* alpha_out,
                        double* beta_out) {
  const int S = v->S;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (long q = 0; q < B; ++q) {
    fb_buf b;
    if (fb_alloc(&b, L, S, v->npred)) {
      fb_free(&b);
      err |= 1;
      continue;
    }
    const float* wq = w + q * L;
    double lz = fb_sequence(v, c, wq, L, T, &b);
    logz[q] = lz;
    posterior(v, c, L, &b, lz, gamma ? gamma + (size_t)q * L * S : NULL, what + q * L);
    if (alpha_out) memcpy(alpha_out + (size_t)q * L * S, b.alpha, (size_t)L * S * sizeof(double));
    if (beta_out) memcpy(beta_out + (size_t)q * L * S, b.beta, (size_t)L * S * sizeof(double));
    fb_free(&b);
  }
  return err ? -2 : 0;
}

/*
 * Gradient of  F = sum_t g_t w_hat_t + h * log Z  with respect to w, c and (dense) theta
 * ("exactly differentiable ... exact gradients" -- abstract; technical summary, "Key
 * technical innovations"). With Lambda = -E/T the log-weight of a path:
 *   d E_p[F] / d x = E_p[dF/dx] + Cov_p(F, dLambda/dx),  d log Z / d x = E_p[dLambda/dx].
 * The posterior is a Markov chain, so E[sum_u g_u c(s_u) | s_t = s] = Fwd_t(s) + g_t c(s) + Bwd_t(s):
 *   Fwd_1 = 0;  Fwd_t(s') = sum_{s in pred(s')} q_t(s|s') (Fwd_{t-1}(s) + g_{t-1} c(s)),
 *               q_t(s|s') = exp(alpha_{t-1}(s) + phi(s,s') + ell_t(s') - alpha_t(s'))
 *   Bwd_L = 0;  Bwd_t(s)  = sum_{s' in succ(s)} r_t(s'|s) (Bwd_{t+1}(s') + g_{t+1} c(s')),
 *               r_t(s'|s) = exp(phi(s,s') + ell_{t+1}(s') + beta_{t+1}(s') - beta_t(s))
 *   mu = sum_t g_t w_hat_t,  D_t(s) = gamma_t(s) (Fwd_t(s) + g_t c(s) + Bwd_t(s) - mu)
 *   dF/dw_t  = (2/T) sum_s c(s) D_t(s) - (2h/T)(w_t - w_hat_t)
 *   dF/dc(s) = sum_t [ g_t gamma_t(s) + (2/T)(w_t - c(s)) (D_t(s) + h gamma_t(s)) ]
 *   dF/dtheta(s,s') = (1/T) sum_{t>=2} xi_t(s,s') (Fwd_{t-1}(s) + g_{t-1} c(s) + g_t c(s')
 *                                                  + Bwd_t(s') - mu + h),
 *               xi_t(s,s') = exp(alpha_{t-1}(s) + phi(s,s') + ell_t(s') + beta_t(s') - log Z)
 * grad_c and grad_theta are summed over all B sequences (overwritten, not accumulated).
 */
static int backward_impl(const tview* v, const float* c, const float* w, long B, long L, double T,
                         const float* g, const float* h, double* grad_w, double* grad_c,
                         double* grad_theta) {
  const int S = v->S, P = v->npred;
  int nthr = 1;
#ifdef _OPENMP
  nthr = omp_get_max_threads();
#endif
  double* gc_part = (double*)calloc((size_t)nthr * S, sizeof(double));
  double* gt_part = NULL;
  if (grad_theta) gt_part = (double*)calloc((size_t)nthr * S * S, sizeof(double));
  if (!gc_part || (grad_theta && !gt_part)) {
    free(gc_part);
    free(gt_part);
    return -2;
  }
  int err = 0;
#pragma omp parallel reduction(| : err)
  {
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
    double* gcp = gc_part + (size_t)tid * S;
    double* gtp = gt_part ? gt_part + (size_t)tid * S * S : NULL;
    size_t LS = (size_t)L * S;
    double* fwd = (double*)malloc(LS * sizeof(double));
    double* bwd = (double*)malloc(LS * sizeof(double));
    double* gam = (double*)malloc(LS * sizeof(double));
    double* what = (double*)malloc((size_t)L * sizeof(double));
    fb_buf b;
    int ok = fwd && bwd && gam && what && (fb_alloc(&b, L, S, P) == 0);
    if (!ok) err |= 1;
#pragma omp for schedule(static)
    for (long q = 0; q < B; ++q) {
      if (!ok) continue;
      const float* wq = w + q * L;
      const float* gq = g + q * L;
      const double hq = h ? (double)h[q] : 0.0;
      double lz = fb_sequence(v, c, wq, L, T, &b);
      posterior(v, c, L, &b, lz, gam, what);
      /* forward conditional expectation */
      for (int s = 0; s < S; ++s) fwd[s] = 0.0;
      for (long t = 1; t < L; ++t)
        for (int sp = 0; sp < S; ++sp) {
          double acc = 0.0;
          for (int a = 0; a < P; ++a) {
            int s = pred_state(v, sp, a);
            double qw = exp(b.alpha[(t - 1) * S + s] + edge_phi(v, s, sp) + b.ell[t * S + sp] -
                            b.alpha[t * S + sp]);
            acc += qw * (fwd[(t - 1) * S + s] + (double)gq[t - 1] * (double)c[s]);
          }
          fwd[t * S + sp] = acc;
        }
      /* backward conditional expectation */
      for (int s = 0; s < S; ++s) bwd[(L - 1) * S + s] = 0.0;
      for (long t = L - 2; t >= 0; --t)
        for (int s = 0; s < S; ++s) {
          double acc = 0.0;
          for (int bb = 0; bb < P; ++bb) {
            int sp = succ_state(v, s, bb);
            double rw = exp(edge_phi(v, s, sp) + b.ell[(t + 1) * S + sp] +
                            b.beta[(t + 1) * S + sp] - b.beta[t * S + s]);
            acc += rw * (bwd[(t + 1) * S + sp] + (double)gq[t + 1] * (double)c[sp]);
          }
          bwd[t * S + s] = acc;
        }
      double mu = 0.0;
      for (long t = 0; t < L; ++t) mu += (double)gq[t] * what[t];
      for (long t = 0; t < L; ++t) {
        double wt = (double)wq[t], gt = (double)gq[t];
        double acc = 0.0;
        for (int s = 0; s < S; ++s) {
          double gm = gam[t * S + s];
          double D = gm * (fwd[t * S + s] + gt * (double)c[s] + bwd[t * S + s] - mu);
          acc += (double)c[s] * D;
          gcp[s] += gt * gm + (2.0 / T) * (wt - (double)c[s]) * (D + hq * gm);
        }
        grad_w[q * L + t] = (2.0 / T) * acc - (2.0 * hq / T) * (wt - what[t]);
      }
      if (gtp) {
        for (long t = 1; t < L; ++t)
          for (int s = 0; s < S; ++s) {
            double left = fwd[(t - 1) * S + s] + (double)gq[t - 1] * (double)c[s];
            for (int sp = 0; sp < S; ++sp) {
              double xi = exp(b.alpha[(t - 1) * S + s] + edge_phi(v, s, sp) + b.ell[t * S + sp] +
                              b.beta[t * S + sp] - lz);
              gtp[(size_t)s * S + sp] +=
                  xi * (left + (double)gq[t] * (double)c[sp] + bwd[t * S + sp] - mu + hq) / T;
            }
          }
      }
    }
    if (ok) fb_free(&b);
    free(fwd);
    free(bwd);
    free(gam);
    free(what);
  }
  if (!err) {
    for (int s = 0; s < S; ++s) {
      double acc = 0.0;
      for (int i = 0; i < nthr; ++i) acc += gc_part[(size_t)i * S + s];
      grad_c[s] = acc;
    }
    if (grad_theta)
      for (size_t e = 0; e < (size_t)S * S; ++e) {
        double acc = 0.0;
        for (int i = 0; i < nthr; ++i) acc += gt_part[(size_t)i * S * S + e];
        grad_theta[e] = acc;
      }
  }
  free(gc_part);
  free(gt_part);
  return err ? -2 : 0;
}

/* ---------------------------------------------------------------------------------------- */
/* Exported entry points (bitshift trellis)                                                   */
/* ---------------------------------------------------------------------------------------- */
int oracle_sparse_forward(int n, int k, const float* c, const float* w, long B, long L, double T,
                          double* what, double* logz, double* gamma, double* alpha,
                          double* beta) {
  tview v;
  if (set_view(&v, n, k) || B < 0 || L < 1 || !(T > 0.0)) return -1;
  return forward_impl(&v, c, w, B, L, T, what, logz, gamma, alpha, beta);
}

int oracle_sparse_backward(int n, int k, const float* c, const float* w, long B, long L, double T,
                           const float* g, const float* h, double* grad_w, double* grad_c) {
  tview v;
  if (set_view(&v, n, k) || B < 0 || L < 1 || !(T > 0.0)) return -1;
  return backward_impl(&v, c, w, B, L, T, g, h, grad_w, grad_c, NULL);
}

/* ---------------------------------------------------------------------------------------- */
/* Dense (fully connected) trellis: theta is the S x S transition log-potential, divided by   */
/* T together with the emission energy (the Ising transfer-matrix reading of the abstract).    */
/* ---------------------------------------------------------------------------------------- */
static double* dense_phi(int S, const float* theta, double T) {
  double* phi = (double*)malloc((size_t)S * S * sizeof(double));
  if (!phi) return NULL;
  for (size_t e = 0; e < (size_t)S * S; ++e) phi[e] = (double)theta[e] / T;
  return phi;
}

int oracle_dense_forward(int S, const float* theta, const float* c, const float* w, long B, long L,
                         double T, double* what, double* logz, double* gamma) {
  if (S < 1 || B < 0 || L < 1 || !(T > 0.0)) return -1;
  double* phi = dense_phi(S, theta, T);
  if (!phi) return -2;
  tview v = {S, 1, 0, 0, S, phi};
  int r = forward_impl(&v, c, w, B, L, T, what, logz, gamma, NULL, NULL);
  free(phi);
  return r;
}

int oracle_dense_backward(int S, const float* theta, const float* c, const float* w, long B,
                          long L, double T, const float* g, const float* h, double* grad_w,
                          double* grad_c, double* grad_theta) {
  if (S < 1 || B < 0 || L < 1 || !(T > 0.0)) return -1;
  double* phi = dense_phi(S, theta, T);
  if (!phi) return -2;
  tview v = {S, 1, 0, 0, S, phi};
  int r = backward_impl(&v, c, w, B, L, T, g, h, grad_w, grad_c, grad_theta);
  free(phi);
  return r;
}

/* ---------------------------------------------------------------------------------------- */
/* Viterbi: the zero-temperature limit (abstract: "recovering the hard QTIP code as T -> 0"). */
/* fp32, no contraction, fixed op order, so that a GPU decoder can match it bit for bit:      */
/*   e_t(s)  = fl(d * d) with d = fl(w_t - c(s))                                              */
/*   m_1(s)  = e_1(s)                                                                         */
/*   m_t(s') = fl(best + e_t(s')), best = the first strict minimum of m_{t-1}(p_a(s'))         */
/*             over a = 0, 1, ..., K-1 (lowest predecessor index wins a tie); bp_t(s') = a     */
/*   s*_L    = the smallest s attaining min_s m_L(s);  s*_{t-1} = p_{bp_t(s*_t)}(s*_t)         */
/* The same recursion is also offered in double precision so that a caller can tell a         */
/* near-tie (the two precisions choose different paths) from a bug.                           */
/* ---------------------------------------------------------------------------------------- */
#define VITERBI_BODY(REAL)                                                                     \
  tview v;                                                                                     \
  if (set_view(&v, n, k) || B < 0 || L < 1) return -1;                                         \
  const int S = v.S, K = v.npred;                                                              \
  int err = 0;                                                                                 \
  _Pragma("omp parallel for schedule(dynamic, 1) reduction(| : err)")                          \
  for (long q = 0; q < B; ++q) {                                                               \
    REAL* m = (REAL*)malloc(2 * (size_t)S * sizeof(REAL));                                     \
    uint8_t* bp = (uint8_t*)malloc((size_t)L * S);                                             \
    if (!m || !bp) {                                                                           \
      free(m);                                                                                 \
      free(bp);                                                                                \
      err |= 1;                                                                                \
      continue;                                                                                \
    }                                                                                          \
    const float* wq = w + q * L;                                                               \
    REAL* cur = m;                                                                             \
    REAL* nxt = m + S;                                                                         \
    for (int s = 0; s < S; ++s) {                                                              \
      REAL d = (REAL)wq[0] - (REAL)c[s];                                                       \
      REAL e = d * d;                                                                          \
      cur[s] = e;                                                                              \
    }                                                                                          \
    for (long t = 1; t < L; ++t) {                                                             \
      for (int sp = 0; sp < S; ++sp) {                                                         \
        REAL best = cur[pred_state(&v, sp, 0)];                                                \
        int ba = 0;                                                                            \
        for (int a = 1; a < K; ++a) {                                                          \
          REAL x = cur[pred_state(&v, sp, a)];                                                 \
          if (x < best) {                                                                      \
            best = x;                                                                          \
            ba = a;                                                                            \
          }                                                                                    \
        }                                                                                      \
        REAL d = (REAL)wq[t] - (REAL)c[sp];                                                    \
        REAL e = d * d;                                                                        \
        nxt[sp] = best + e;                                                                    \
        bp[t * S + sp] = (uint8_t)ba;                                                          \
      }                                                                                        \
      REAL* tmp = cur;                                                                         \
      cur = nxt;                                                                               \
      nxt = tmp;                                                                               \
    }                                                                                          \
    int sb = 0;                                                                                \
    for (int s = 1; s < S; ++s)                                                                \
      if (cur[s] < cur[sb]) sb = s;                                                            \
    if (energy) energy[q] = (double)cur[sb];                                                   \
    int32_t* st = states + q * L;                                                              \
    st[L - 1] = sb;                                                                            \
    for (long t = L - 1; t >= 1; --t) st[t - 1] = pred_state(&v, st[t], bp[t * S + st[t]]);    \
    if (w_hard)                                                                                \
      for (long t = 0; t < L; ++t) w_hard[q * L + t] = c[st[t]];                               \
    free(m);                                                                                   \
    free(bp);                                                                                  \
  }                                                                                            \
  return err ? -2 : 0;

int oracle_viterbi_f32(int n, int k, const float* c, const float* w, long B, long L,
                       int32_t* states, float* w_hard, double* energy) {
  if (k > 8) return -1; /* backpointers are stored as bytes */
  VITERBI_BODY(float)
}

int oracle_viterbi_f64(int n, int k, const float* c, const float* w, long B, long L,
                       int32_t* states, float* w_hard, double* energy) {
  if (k > 8) return -1;
  VITERBI_BODY(double)
}

/* ---------------------------------------------------------------------------------------- */
/* Hard-code export, the zero-temperature end of the method (abstract: the hard QTIP code is   */
/* recovered as T -> 0). In the bitshift trellis a state path is fixed by its first state and  */
/* the k bits every step shifts in: s_t = ((s_{t-1} << k) | b_t) & (S-1), b_t = s_t mod K.     */
/* The code of a chain is the bit string s_0 (n bits, most significant first) followed by      */
/* b_1, ..., b_{L-1} (k bits each, most significant first), n + k (L-1) bits in 32-bit words,  */
/* the first bit in the most significant position of word 0 and the unused tail of the last   */
/* word zero. (The pages do not give a packing; this is the reading.)                          */
/* ---------------------------------------------------------------------------------------- */
long oracle_code_words(int n, int k, long L) { return ((long)n + (long)k * (L - 1) + 31) / 32; }

static void put_bits(uint32_t* words, long* pos, uint32_t value, int nbits) {
  for (int i = nbits - 1; i >= 0; --i) {
    const uint32_t bit = (value >> i) & 1u;
    words[*pos / 32] |= bit << (31 - (int)(*pos % 32));
    ++*pos;
  }
}

static uint32_t get_bits(const uint32_t* words, long* pos, int nbits) {
  uint32_t v = 0;
  for (int i = 0; i < nbits; ++i) {
    const uint32_t bit = (words[*pos / 32] >> (31 - (int)(*pos % 32))) & 1u;
    v = (v << 1) | bit;
    ++*pos;
  }
  return v;
}

/* Pack each chain's state path; *bad counts the steps whose state is not a successor of the   */
/* previous one (such a path cannot be represented and packs to its successor-consistent code). */
int oracle_pack_states(int n, int k, const int32_t* states, long B, long L, uint32_t* code,
                       long* bad) {
  if (n < 1 || n > 16 || k < 1 || k > n || B < 0 || L < 1) return -1;
  const long W = oracle_code_words(n, k, L);
  const uint32_t S = 1u << n, K = 1u << k;
  long nbad = 0;
  for (long q = 0; q < B; ++q) {
    uint32_t* words = code + q * W;
    for (long i = 0; i < W; ++i) words[i] = 0;
    const int32_t* st = states + q * L;
    long pos = 0;
    put_bits(words, &pos, (uint32_t)st[0] & (S - 1), n);
    for (long t = 1; t < L; ++t) {
      const uint32_t prev = (uint32_t)st[t - 1], cur = (uint32_t)st[t];
      if ((((prev << k) | (cur & (K - 1))) & (S - 1)) != cur) ++nbad;
      put_bits(words, &pos, cur & (K - 1), k);
    }
  }
  if (bad) *bad = nbad;
  return 0;
}

/* Replay the shift register from the code; w_hard (may be NULL) gets c(s_t). */
int oracle_unpack_code(int n, int k, const float* c, const uint32_t* code, long B, long L,
                       int32_t* states, float* w_hard) {
  if (n < 1 || n > 16 || k < 1 || k > n || B < 0 || L < 1) return -1;
  const long W = oracle_code_words(n, k, L);
  const uint32_t S = 1u << n;
  for (long q = 0; q < B; ++q) {
    const uint32_t* words = code + q * W;
    long pos = 0;
    uint32_t s = get_bits(words, &pos, n);
    states[q * L] = (int32_t)s;
    for (long t = 1; t < L; ++t) {
      s = ((s << k) | get_bits(words, &pos, k)) & (S - 1);
      states[q * L + t] = (int32_t)s;
    }
    if (w_hard)
      for (long t = 0; t < L; ++t) w_hard[q * L + t] = c[states[q * L + t]];
  }
  return 0;
}

/* Thread count used by the OpenMP loops (the CPU baseline reports it). */
int oracle_set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
  return omp_get_max_threads();
#else
  (void)nthreads;
  return 1;
#endif
}
