/*
 * Plain fp64 CPU oracle for the gated delta rule (GatedDeltaNet) recurrence:
 * forward scan and its reverse-mode VJP.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU product path
 * shares no code, header, table or helper with it.
 *
 * What it computes (sources: the mlx-lm pull request "Add gated_delta_update
 * VJP -- trainable GatedDeltaNet on Apple Silicon", sections "What this PR
 * adds", "Numerical correctness" and "Design notes"; the torch-to-nnef page
 * "Gated delta net recurrence export to tract_transformers_gdn_recurrent",
 * its "Op contract" paragraph):
 *
 *   For batch b and value head h, the key/query head is j = h / G with
 *   G = Hv / Hk (the op contract's GQA rule: value head h reads q/k head h//G).
 *   q and k are L2-normalised with eps 1e-6 inside the square root, and q is
 *   then scaled by 1/sqrt(Dk) (the op contract normalises q and k with an
 *   eps of 1e-6 and scales q by one over the square root of the key width).
 *   Gates: x = a + dt_bias, x_c = min(x, 20) (the PR clamps the argument of
 *   the softplus without giving bounds; read: upper bound only),
 *   l = -exp(A_log) * softplus(x_c), g = exp(l),
 *   beta = sigmoid(b).
 *   Step (valid step):  S' = g*S;  u = S'^T k;  delta = beta*(v - u);
 *                       S  = S' + k delta^T;  o = S^T q.
 *   Masked step: S is left unchanged (PR, "Covered corner cases": the final
 *   state of a half-masked run equals the state after the unmasked prefix);
 *   the output is still o = S^T q.
 *   State checkpoints are the states at t = 64c, c = 1..ceil(T/64)-1 (PR,
 *   "Why chunked instead of single-shot?": CHUNK_SIZE = 64).
 *
 * The backward is the plain reverse sweep of that step (chain rule applied to
 * each assignment above, in reverse order), evaluated in fp64 with the states
 * either all stored (chunk = 0) or stored every `chunk` steps and recomputed
 * inside each chunk; both modes perform the same fp64 operations in the same
 * order, so they agree bit for bit.
 *
 * The per-key-channel gate (oracle_gdn_fwd_vg / oracle_gdn_bwd_vg) replaces the
 * scalar g by a vector that scales the state's rows; see its section below.
 *
 * Everything is sequential per (b, h); the optional OpenMP loop only runs
 * independent (b, h) pairs on different threads.  The sums over the G value
 * heads of a key head and over (b, t) for the per-head parameters run
 * afterwards in a fixed order (b, then t, then h inside the group).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int64_t B, T, Hk, Hv, Dk, Dv;
} oracle_dims;

#define ORACLE_EPS 1e-6
#define ORACLE_CLAMP 20.0
#define ORACLE_CKPT 64

/* ---------------------------------------------------------------- scalars */

/* softplus(x) = log(1 + e^x), evaluated without overflow. */
static double softplus(double x) {
  if (x > 0.0) return x + log1p(exp(-x));
  return log1p(exp(x));
}

static double sigmoid(double x) {
  if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
  double e = exp(x);
  return e / (1.0 + e);
}

typedef struct {
  double g, ell, beta, lam, xc, x;
} gate_t;

/* Gate scalars of one (b, t, h) (see header comment). */
static gate_t gates(double a, double b, double A_log, double dt_bias) {
  gate_t r;
  r.x = a + dt_bias;
  r.xc = r.x < ORACLE_CLAMP ? r.x : ORACLE_CLAMP;
  r.lam = exp(A_log);
  r.ell = -r.lam * softplus(r.xc);
  r.g = exp(r.ell);
  r.beta = sigmoid(b);
  return r;
}

/* Exported for direct pins of the gate scalars. */
void oracle_gates(double a, double b, double A_log, double dt_bias,
                  double* g, double* ell, double* beta) {
  gate_t r = gates(a, b, A_log, dt_bias);
  *g = r.g;
  *ell = r.ell;
  *beta = r.beta;
}

/* xhat = x * (sum x^2 + eps)^(-1/2); returns the factor r. */
static double l2norm(const double* x, int64_t n, double* xhat) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
  double r = 1.0 / sqrt(ss + ORACLE_EPS);
  for (int64_t i = 0; i < n; ++i) xhat[i] = x[i] * r;
  return r;
}

/* ---------------------------------------------------------------- layout */

static size_t at_qk(const oracle_dims* d, int64_t b, int64_t t, int64_t j) {
  return ((size_t)(b * d->T + t) * d->Hk + j) * d->Dk;
}
static size_t at_v(const oracle_dims* d, int64_t b, int64_t t, int64_t h) {
  return ((size_t)(b * d->T + t) * d->Hv + h) * d->Dv;
}
static size_t at_g(const oracle_dims* d, int64_t b, int64_t t, int64_t h) {
  return (size_t)(b * d->T + t) * d->Hv + h;
}
static size_t at_s(const oracle_dims* d, int64_t b, int64_t h) {
  return ((size_t)b * d->Hv + h) * d->Dk * d->Dv;
}

static int check_dims(const oracle_dims* d) {
  if (d->B < 1 || d->T < 0 || d->Hk < 1 || d->Hv < 1 || d->Dk < 1 || d->Dv < 1)
    return 1;
  if (d->Hv % d->Hk != 0) return 1;
  return 0;
}

/* Per-step inputs of one (b, t, h), read and transformed as in the header. */
typedef struct {
  double *khat, *qhat, *qt; /* Dk each: normalised k, normalised q, scaled q */
  double rk, rq;
  gate_t gt;
  int valid;
} step_in;

static void load_step(const oracle_dims* d, int64_t b, int64_t t, int64_t h,
                      const double* q, const double* k, const double* a,
                      const double* bb, const double* A_log,
                      const double* dt_bias, const uint8_t* mask, step_in* s) {
  int64_t G = d->Hv / d->Hk, j = h / G;
  double scale = 1.0 / sqrt((double)d->Dk);
  s->rk = l2norm(k + at_qk(d, b, t, j), d->Dk, s->khat);
  s->rq = l2norm(q + at_qk(d, b, t, j), d->Dk, s->qhat);
  for (int64_t i = 0; i < d->Dk; ++i) s->qt[i] = scale * s->qhat[i];
  size_t gi = at_g(d, b, t, h);
  s->gt = gates(a[gi], bb[gi], A_log[h], dt_bias[h]);
  s->valid = mask ? (mask[b * d->T + t] != 0) : 1;
}

/* One forward step on S (Dk x Dv, row-major).  Writes u and delta (Dv each)
 * when the step is valid, and o (Dv).  Returns nothing; S is updated. */
static void fwd_step(const oracle_dims* d, double* S, const step_in* s,
                     const double* v, double* u, double* delta, double* o) {
  int64_t Dk = d->Dk, Dv = d->Dv;
  if (s->valid) {
    for (int64_t i = 0; i < Dk; ++i)
      for (int64_t c = 0; c < Dv; ++c) S[i * Dv + c] *= s->gt.g;
    for (int64_t c = 0; c < Dv; ++c) {
      double acc = 0.0;
      for (int64_t i = 0; i < Dk; ++i) acc += S[i * Dv + c] * s->khat[i];
      u[c] = acc;
      delta[c] = s->gt.beta * (v[c] - acc);
    }
    for (int64_t i = 0; i < Dk; ++i)
      for (int64_t c = 0; c < Dv; ++c) S[i * Dv + c] += s->khat[i] * delta[c];
  }
  for (int64_t c = 0; c < Dv; ++c) {
    double acc = 0.0;
    for (int64_t i = 0; i < Dk; ++i) acc += S[i * Dv + c] * s->qt[i];
    o[c] = acc;
  }
}

typedef struct {
  double *khat, *qhat, *qt, *u, *delta, *otmp;
} scratch_t;

static int scratch_alloc(const oracle_dims* d, scratch_t* w) {
  w->khat = malloc(sizeof(double) * d->Dk);
  w->qhat = malloc(sizeof(double) * d->Dk);
  w->qt = malloc(sizeof(double) * d->Dk);
  w->u = malloc(sizeof(double) * d->Dv);
  w->delta = malloc(sizeof(double) * d->Dv);
  w->otmp = malloc(sizeof(double) * d->Dv);
  return !(w->khat && w->qhat && w->qt && w->u && w->delta && w->otmp);
}
static void scratch_free(scratch_t* w) {
  free(w->khat); free(w->qhat); free(w->qt);
  free(w->u); free(w->delta); free(w->otmp);
}

/* ---------------------------------------------------------------- forward */

/*
 * o [B,T,Hv,Dv], state_out [B,Hv,Dk,Dv]; ckpt (nullable)
 * [ceil(T/64)-1, B, Hv, Dk, Dv].  state0 and mask may be NULL (zeros / all
 * valid).  Returns 0 on success, 1 on bad dims, 2 on allocation failure.
 */
int oracle_gdn_fwd(const oracle_dims* d, const double* q, const double* k,
                   const double* v, const double* a, const double* b,
                   const double* A_log, const double* dt_bias,
                   const double* state0, const uint8_t* mask, double* o,
                   double* state_out, double* ckpt, int nthreads) {
  if (check_dims(d)) return 1;
  int64_t BH = d->B * d->Hv;
  size_t SS = (size_t)d->Dk * d->Dv;
  int err = 0;
  (void)nthreads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
  for (int64_t bh = 0; bh < BH; ++bh) {
    int64_t bi = bh / d->Hv, h = bh % d->Hv;
    scratch_t w;
    double* S = malloc(sizeof(double) * SS);
    if (scratch_alloc(d, &w) || !S) {
#pragma omp atomic write
      err = 2;
      free(S);
      scratch_free(&w);
      continue;
    }
    if (state0) memcpy(S, state0 + at_s(d, bi, h), sizeof(double) * SS);
    else memset(S, 0, sizeof(double) * SS);
    step_in s;
    memset(&s, 0, sizeof s);
    s.khat = w.khat;
    s.qhat = w.qhat;
    s.qt = w.qt;
    for (int64_t t = 0; t < d->T; ++t) {
      load_step(d, bi, t, h, q, k, a, b, A_log, dt_bias, mask, &s);
      fwd_step(d, S, &s, v + at_v(d, bi, t, h), w.u, w.delta,
               o + at_v(d, bi, t, h));
      if (ckpt && (t + 1) % ORACLE_CKPT == 0 && t + 1 < d->T) {
        int64_t c = (t + 1) / ORACLE_CKPT - 1;
        memcpy(ckpt + (size_t)c * BH * SS + at_s(d, bi, h), S,
               sizeof(double) * SS);
      }
    }
    memcpy(state_out + at_s(d, bi, h), S, sizeof(double) * SS);
    free(S);
    scratch_free(&w);
  }
  return err;
}

/* --------------------------------------------------------------- backward */

/*
 * Reverse sweep.  Inputs as oracle_gdn_fwd plus dO [B,T,Hv,Dv] and dS_final
 * [B,Hv,Dk,Dv] (nullable = zeros).  Outputs (all overwritten):
 *   dq, dk [B,T,Hk,Dk]; dv [B,T,Hv,Dv]; da, db [B,T,Hv];
 *   dA_log, ddt_bias [Hv]; dstate [B,Hv,Dk,Dv].
 * chunk = 0 stores every state; chunk > 0 stores the state every `chunk`
 * steps and recomputes inside each chunk.
 */
int oracle_gdn_bwd(const oracle_dims* d, const double* q, const double* k,
                   const double* v, const double* a, const double* b,
                   const double* A_log, const double* dt_bias,
                   const double* state0, const uint8_t* mask, const double* dO,
                   const double* dS_final, double* dq, double* dk, double* dv,
                   double* da, double* db, double* dA_log, double* ddt_bias,
                   double* dstate, int64_t chunk, int nthreads) {
  if (check_dims(d) || chunk < 0) return 1;
  int64_t B = d->B, T = d->T, Hk = d->Hk, Hv = d->Hv, Dk = d->Dk, Dv = d->Dv;
  int64_t G = Hv / Hk, BH = B * Hv;
  size_t SS = (size_t)Dk * Dv;
  int64_t span = chunk > 0 ? chunk : (T > 0 ? T : 1); /* states kept per pass */
  int64_t nspan = T > 0 ? (T + span - 1) / span : 0;

  /* Per value head contributions, summed over the group afterwards. */
  size_t nvk = (size_t)B * T * Hv * Dk;
  double* dqt_h = calloc(nvk ? nvk : 1, sizeof(double));
  double* dkt_h = calloc(nvk ? nvk : 1, sizeof(double));
  double* dAl_part = calloc((size_t)B * T * Hv + 1, sizeof(double));
  if (!dqt_h || !dkt_h || !dAl_part) {
    free(dqt_h); free(dkt_h); free(dAl_part);
    return 2;
  }
  int err = 0;
  (void)nthreads;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
  for (int64_t bh = 0; bh < BH; ++bh) {
    int64_t bi = bh / Hv, h = bh % Hv;
    scratch_t w;
    double* S = malloc(sizeof(double) * SS);
    double* D = malloc(sizeof(double) * SS);
    double* Sp = malloc(sizeof(double) * SS);   /* S' = g * S_prev */
    double* St = malloc(sizeof(double) * SS);   /* S_t */
    double* dSp = malloc(sizeof(double) * SS);  /* dL/dS' */
    double* starts = malloc(sizeof(double) * SS * (nspan ? nspan : 1));
    double* hist = malloc(sizeof(double) * SS * span);
    double* ddel = malloc(sizeof(double) * Dv);
    double* du = malloc(sizeof(double) * Dv);
    if (scratch_alloc(d, &w) || !S || !D || !Sp || !St || !dSp || !starts ||
        !hist || !ddel || !du) {
#pragma omp atomic write
      err = 2;
      free(S); free(D); free(Sp); free(St); free(dSp); free(starts);
      free(hist); free(ddel); free(du);
      scratch_free(&w);
      continue;
    }
    step_in s;
    memset(&s, 0, sizeof s);
    s.khat = w.khat;
    s.qhat = w.qhat;
    s.qt = w.qt;

    /* Forward pass, keeping the state at the start of every span. */
    if (state0) memcpy(S, state0 + at_s(d, bi, h), sizeof(double) * SS);
    else memset(S, 0, sizeof(double) * SS);
    for (int64_t t = 0; t < T; ++t) {
      if (t % span == 0) memcpy(starts + (size_t)(t / span) * SS, S, sizeof(double) * SS);
      load_step(d, bi, t, h, q, k, a, b, A_log, dt_bias, mask, &s);
      fwd_step(d, S, &s, v + at_v(d, bi, t, h), w.u, w.delta, w.otmp);
    }

    /* Reverse sweep. */
    if (dS_final) memcpy(D, dS_final + at_s(d, bi, h), sizeof(double) * SS);
    else memset(D, 0, sizeof(double) * SS);
    for (int64_t c = nspan - 1; c >= 0; --c) {
      int64_t t0 = c * span, t1 = t0 + span < T ? t0 + span : T;
      /* Recompute the states S_prev of every step of this span. */
      memcpy(S, starts + (size_t)c * SS, sizeof(double) * SS);
      for (int64_t t = t0; t < t1; ++t) {
        memcpy(hist + (size_t)(t - t0) * SS, S, sizeof(double) * SS);
        load_step(d, bi, t, h, q, k, a, b, A_log, dt_bias, mask, &s);
        fwd_step(d, S, &s, v + at_v(d, bi, t, h), w.u, w.delta, w.otmp);
      }
      for (int64_t t = t1 - 1; t >= t0; --t) {
        const double* Sprev = hist + (size_t)(t - t0) * SS;
        const double* vt = v + at_v(d, bi, t, h);
        const double* dOt = dO + at_v(d, bi, t, h);
        load_step(d, bi, t, h, q, k, a, b, A_log, dt_bias, mask, &s);
        size_t gi = at_g(d, bi, t, h);
        double* dqt = dqt_h + ((size_t)(bi * T + t) * Hv + h) * Dk;
        double* dkt = dkt_h + ((size_t)(bi * T + t) * Hv + h) * Dk;
        double* dvt = dv + at_v(d, bi, t, h);
        double g = s.gt.g, beta = s.gt.beta;

        /* Recompute this step's forward quantities from S_prev. */
        if (s.valid) {
          for (size_t e = 0; e < SS; ++e) Sp[e] = g * Sprev[e];
          for (int64_t cc = 0; cc < Dv; ++cc) {
            double acc = 0.0;
            for (int64_t i = 0; i < Dk; ++i) acc += Sp[i * Dv + cc] * s.khat[i];
            w.u[cc] = acc;
            w.delta[cc] = beta * (vt[cc] - acc);
          }
          for (int64_t i = 0; i < Dk; ++i)
            for (int64_t cc = 0; cc < Dv; ++cc)
              St[i * Dv + cc] = Sp[i * Dv + cc] + s.khat[i] * w.delta[cc];
        } else {
          memcpy(St, Sprev, sizeof(double) * SS);
        }

        /* o_t = S_t^T qt:  dL/dS_t += qt dO^T,  dL/dqt = S_t dO. */
        for (int64_t i = 0; i < Dk; ++i)
          for (int64_t cc = 0; cc < Dv; ++cc) D[i * Dv + cc] += s.qt[i] * dOt[cc];
        for (int64_t i = 0; i < Dk; ++i) {
          double acc = 0.0;
          for (int64_t cc = 0; cc < Dv; ++cc) acc += St[i * Dv + cc] * dOt[cc];
          dqt[i] = acc;
        }

        if (!s.valid) {
          /* S_t = S_prev: D passes through unchanged. */
          for (int64_t i = 0; i < Dk; ++i) dkt[i] = 0.0;
          for (int64_t cc = 0; cc < Dv; ++cc) dvt[cc] = 0.0;
          da[gi] = 0.0;
          db[gi] = 0.0;
          dAl_part[gi] = 0.0;
          continue;
        }

        /* S_t = S' + k delta^T. */
        for (int64_t cc = 0; cc < Dv; ++cc) {
          double acc = 0.0;
          for (int64_t i = 0; i < Dk; ++i) acc += D[i * Dv + cc] * s.khat[i];
          ddel[cc] = acc;
        }
        /* delta = beta (v - u). */
        double dbeta = 0.0;
        for (int64_t cc = 0; cc < Dv; ++cc) {
          dvt[cc] = beta * ddel[cc];
          dbeta += ddel[cc] * (vt[cc] - w.u[cc]);
          du[cc] = -beta * ddel[cc];
        }
        /* u = S'^T k:  dS' = D + k du^T;  dk = D delta + S' du. */
        for (int64_t i = 0; i < Dk; ++i)
          for (int64_t cc = 0; cc < Dv; ++cc)
            dSp[i * Dv + cc] = D[i * Dv + cc] + s.khat[i] * du[cc];
        for (int64_t i = 0; i < Dk; ++i) {
          double acc = 0.0;
          for (int64_t cc = 0; cc < Dv; ++cc)
            acc += D[i * Dv + cc] * w.delta[cc] + Sp[i * Dv + cc] * du[cc];
          dkt[i] = acc;
        }
        /* S' = g S_prev:  dg = <dS', S_prev>,  dL/dS_prev = g dS'. */
        double dg = 0.0;
        for (size_t e = 0; e < SS; ++e) dg += dSp[e] * Sprev[e];
        for (size_t e = 0; e < SS; ++e) D[e] = g * dSp[e];

        /* Gate chain: g = exp(l), l = -lam softplus(xc), xc = min(x, 20),
         * x = a + dt_bias, lam = exp(A_log); beta = sigmoid(b). */
        double dl = dg * g;
        double pass = s.gt.x <= ORACLE_CLAMP ? 1.0 : 0.0;
        da[gi] = dl * (-s.gt.lam) * sigmoid(s.gt.xc) * pass;
        db[gi] = dbeta * beta * (1.0 - beta);
        dAl_part[gi] = dl == 0.0 ? 0.0 : dl * s.gt.ell;
      }
    }
    memcpy(dstate + at_s(d, bi, h), D, sizeof(double) * SS);

    free(S); free(D); free(Sp); free(St); free(dSp); free(starts);
    free(hist); free(ddel); free(du);
    scratch_free(&w);
  }

  if (!err) {
    /* Sum over the G value heads of each key head (h ascending), then the
     * L2-normalisation backward:  with xhat = x r,
     *   dx = r (dxhat - xhat (xhat . dxhat)),  and dxhat = scale * dqt for q. */
    double scale = 1.0 / sqrt((double)Dk);
    double* tmp = malloc(sizeof(double) * Dk * 3);
    double *xhat = tmp, *acc = tmp + Dk;
    for (int64_t bi = 0; bi < B && tmp; ++bi)
      for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < Hk; ++j) {
          for (int pass = 0; pass < 2; ++pass) {
            const double* src = pass == 0 ? dqt_h : dkt_h;
            const double* x = (pass == 0 ? q : k) + at_qk(d, bi, t, j);
            double* out = (pass == 0 ? dq : dk) + at_qk(d, bi, t, j);
            for (int64_t i = 0; i < Dk; ++i) acc[i] = 0.0;
            for (int64_t hh = j * G; hh < (j + 1) * G; ++hh) {
              const double* p = src + ((size_t)(bi * T + t) * Hv + hh) * Dk;
              for (int64_t i = 0; i < Dk; ++i) acc[i] += p[i];
            }
            if (pass == 0)
              for (int64_t i = 0; i < Dk; ++i) acc[i] *= scale;
            double r = l2norm(x, Dk, xhat);
            double dotp = 0.0;
            for (int64_t i = 0; i < Dk; ++i) dotp += xhat[i] * acc[i];
            for (int64_t i = 0; i < Dk; ++i) out[i] = r * (acc[i] - xhat[i] * dotp);
          }
        }
    if (!tmp) err = 2;
    free(tmp);
    for (int64_t h = 0; h < Hv; ++h) {
      double sa = 0.0, sd = 0.0;
      for (int64_t bi = 0; bi < B; ++bi)
        for (int64_t t = 0; t < T; ++t) {
          size_t gi = at_g(d, bi, t, h);
          sa += dAl_part[gi];
          sd += da[gi];
        }
      dA_log[h] = sa;
      ddt_bias[h] = sd;
    }
  }
  free(dqt_h); free(dkt_h); free(dAl_part);
  return err;
}

/* ------------------------------------------------- per-channel (vector) gate */

/*
 * Vectorised gating (mlx-lm PR, "Models covered": Kimi-Linear runs the same
 * rule with a gate per key channel, g.ndim == 4; "Scope and follow-ups": the
 * Python path supports it).  The gate of step t, value head h is a vector
 * g_t in R^Dk that scales the rows of the state: S' = diag(g_t) S.  The pages
 * give no formula that produces it, so the caller passes its logarithm
 * lg[b,t,h,i] = log g_{t,i} directly (as the torch-to-nnef op contract passes
 * a log-decay).  beta = sigmoid(b) and everything else is the scalar-gate
 * step above:
 *   S' = diag(g) S;  u = S'^T k;  delta = beta (v - u);  S = S' + k delta^T;
 *   o = S^T q.
 * A masked step leaves S unchanged and reads o from it.
 */
typedef struct {
  double *khat, *qhat, *qt, *g; /* Dk each; g = exp(lg) */
  double beta;
  int valid;
} step_vg;

static size_t at_lg(const oracle_dims* d, int64_t b, int64_t t, int64_t h) {
  return ((size_t)(b * d->T + t) * d->Hv + h) * d->Dk;
}

static void load_step_vg(const oracle_dims* d, int64_t b, int64_t t, int64_t h,
                         const double* q, const double* k, const double* lg,
                         const double* bb, const uint8_t* mask, step_vg* s) {
  int64_t G = d->Hv / d->Hk, j = h / G;
  double scale = 1.0 / sqrt((double)d->Dk);
  l2norm(k + at_qk(d, b, t, j), d->Dk, s->khat);
  l2norm(q + at_qk(d, b, t, j), d->Dk, s->qhat);
  for (int64_t i = 0; i < d->Dk; ++i) s->qt[i] = scale * s->qhat[i];
  const double* l = lg + at_lg(d, b, t, h);
  for (int64_t i = 0; i < d->Dk; ++i) s->g[i] = exp(l[i]);
  s->beta = sigmoid(bb[at_g(d, b, t, h)]);
  s->valid = mask ? (mask[b * d->T + t] != 0) : 1;
}

static void fwd_step_vg(const oracle_dims* d, double* S, const step_vg* s,
                        const double* v, double* u, double* delta, double* o) {
  int64_t Dk = d->Dk, Dv = d->Dv;
  if (s->valid) {
    for (int64_t i = 0; i < Dk; ++i)
      for (int64_t c = 0; c < Dv; ++c) S[i * Dv + c] *= s->g[i];
    for (int64_t c = 0; c < Dv; ++c) {
      double acc = 0.0;
      for (int64_t i = 0; i < Dk; ++i) acc += S[i * Dv + c] * s->khat[i];
      u[c] = acc;
      delta[c] = s->beta * (v[c] - acc);
    }
    for (int64_t i = 0; i < Dk; ++i)
      for (int64_t c = 0; c < Dv; ++c) S[i * Dv + c] += s->khat[i] * delta[c];
  }
  for (int64_t c = 0; c < Dv; ++c) {
    double acc = 0.0;
    for (int64_t i = 0; i < Dk; ++i) acc += S[i * Dv + c] * s->qt[i];
    o[c] = acc;
  }
}

static int vg_alloc(const oracle_dims* d, scratch_t* w, step_vg* s) {
  memset(s, 0, sizeof *s);
  int bad = scratch_alloc(d, w);
  s->g = malloc(sizeof(double) * d->Dk);
  s->khat = w->khat;
  s->qhat = w->qhat;
  s->qt = w->qt;
  return bad || !s->g;
}

/*
 * lg [B,T,Hv,Dk] log-gates; the rest as oracle_gdn_fwd without the scalar
 * gate inputs.  Returns 0, 1 on bad dims, 2 on allocation failure.
 */
int oracle_gdn_fwd_vg(const oracle_dims* d, const double* q, const double* k,
                      const double* v, const double* lg, const double* b,
                      const double* state0, const uint8_t* mask, double* o,
                      double* state_out, double* ckpt, int nthreads) {
  if (check_dims(d)) return 1;
  int64_t BH = d->B * d->Hv;
  size_t SS = (size_t)d->Dk * d->Dv;
  int err = 0;
  (void)nthreads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
  for (int64_t bh = 0; bh < BH; ++bh) {
    int64_t bi = bh / d->Hv, h = bh % d->Hv;
    scratch_t w;
    step_vg s;
    double* S = malloc(sizeof(double) * SS);
    if (vg_alloc(d, &w, &s) || !S) {
#pragma omp atomic write
      err = 2;
      free(S); free(s.g);
      scratch_free(&w);
      continue;
    }
    if (state0) memcpy(S, state0 + at_s(d, bi, h), sizeof(double) * SS);
    else memset(S, 0, sizeof(double) * SS);
    for (int64_t t = 0; t < d->T; ++t) {
      load_step_vg(d, bi, t, h, q, k, lg, b, mask, &s);
      fwd_step_vg(d, S, &s, v + at_v(d, bi, t, h), w.u, w.delta, o + at_v(d, bi, t, h));
      if (ckpt && (t + 1) % ORACLE_CKPT == 0 && t + 1 < d->T) {
        int64_t c = (t + 1) / ORACLE_CKPT - 1;
        memcpy(ckpt + (size_t)c * BH * SS + at_s(d, bi, h), S, sizeof(double) * SS);
      }
    }
    memcpy(state_out + at_s(d, bi, h), S, sizeof(double) * SS);
    free(S); free(s.g);
    scratch_free(&w);
  }
  return err;
}

/*
 * Reverse sweep of the per-channel-gate step.  Outputs (overwritten):
 *   dq, dk [B,T,Hk,Dk]; dv [B,T,Hv,Dv]; dlg [B,T,Hv,Dk]; db [B,T,Hv];
 *   dstate [B,Hv,Dk,Dv].  chunk as in oracle_gdn_bwd.
 * With S' = diag(g) S_prev the gate enters row by row, so its gradient is a
 * row-wise sum:  dg_i = sum_c dS'[i,c] S_prev[i,c],  dlg_i = g_i dg_i, and
 * dL/dS_prev = diag(g) dS'.  Masked steps get dv = dlg = db = 0.
 */
int oracle_gdn_bwd_vg(const oracle_dims* d, const double* q, const double* k,
                      const double* v, const double* lg, const double* b,
                      const double* state0, const uint8_t* mask, const double* dO,
                      const double* dS_final, double* dq, double* dk, double* dv,
                      double* dlg, double* db, double* dstate, int64_t chunk,
                      int nthreads) {
  if (check_dims(d) || chunk < 0) return 1;
  int64_t B = d->B, T = d->T, Hk = d->Hk, Hv = d->Hv, Dk = d->Dk, Dv = d->Dv;
  int64_t G = Hv / Hk, BH = B * Hv;
  size_t SS = (size_t)Dk * Dv;
  int64_t span = chunk > 0 ? chunk : (T > 0 ? T : 1);
  int64_t nspan = T > 0 ? (T + span - 1) / span : 0;
  size_t nvk = (size_t)B * T * Hv * Dk;
  double* dqt_h = calloc(nvk ? nvk : 1, sizeof(double));
  double* dkt_h = calloc(nvk ? nvk : 1, sizeof(double));
  if (!dqt_h || !dkt_h) {
    free(dqt_h); free(dkt_h);
    return 2;
  }
  int err = 0;
  (void)nthreads;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
  for (int64_t bh = 0; bh < BH; ++bh) {
    int64_t bi = bh / Hv, h = bh % Hv;
    scratch_t w;
    step_vg s;
    double* S = malloc(sizeof(double) * SS);
    double* D = malloc(sizeof(double) * SS);
    double* Sp = malloc(sizeof(double) * SS);
    double* St = malloc(sizeof(double) * SS);
    double* dSp = malloc(sizeof(double) * SS);
    double* starts = malloc(sizeof(double) * SS * (nspan ? nspan : 1));
    double* hist = malloc(sizeof(double) * SS * span);
    double* ddel = malloc(sizeof(double) * Dv);
    double* du = malloc(sizeof(double) * Dv);
    if (vg_alloc(d, &w, &s) || !S || !D || !Sp || !St || !dSp || !starts || !hist ||
        !ddel || !du) {
#pragma omp atomic write
      err = 2;
      free(S); free(D); free(Sp); free(St); free(dSp); free(starts);
      free(hist); free(ddel); free(du); free(s.g);
      scratch_free(&w);
      continue;
    }

    if (state0) memcpy(S, state0 + at_s(d, bi, h), sizeof(double) * SS);
    else memset(S, 0, sizeof(double) * SS);
    for (int64_t t = 0; t < T; ++t) {
      if (t % span == 0) memcpy(starts + (size_t)(t / span) * SS, S, sizeof(double) * SS);
      load_step_vg(d, bi, t, h, q, k, lg, b, mask, &s);
      fwd_step_vg(d, S, &s, v + at_v(d, bi, t, h), w.u, w.delta, w.otmp);
    }

    if (dS_final) memcpy(D, dS_final + at_s(d, bi, h), sizeof(double) * SS);
    else memset(D, 0, sizeof(double) * SS);
    for (int64_t c = nspan - 1; c >= 0; --c) {
      int64_t t0 = c * span, t1 = t0 + span < T ? t0 + span : T;
      memcpy(S, starts + (size_t)c * SS, sizeof(double) * SS);
      for (int64_t t = t0; t < t1; ++t) {
        memcpy(hist + (size_t)(t - t0) * SS, S, sizeof(double) * SS);
        load_step_vg(d, bi, t, h, q, k, lg, b, mask, &s);
        fwd_step_vg(d, S, &s, v + at_v(d, bi, t, h), w.u, w.delta, w.otmp);
      }
      for (int64_t t = t1 - 1; t >= t0; --t) {
        const double* Sprev = hist + (size_t)(t - t0) * SS;
        const double* vt = v + at_v(d, bi, t, h);
        const double* dOt = dO + at_v(d, bi, t, h);
        load_step_vg(d, bi, t, h, q, k, lg, b, mask, &s);
        double* dqt = dqt_h + ((size_t)(bi * T + t) * Hv + h) * Dk;
        double* dkt = dkt_h + ((size_t)(bi * T + t) * Hv + h) * Dk;
        double* dlt = dlg + at_lg(d, bi, t, h);
        double* dvt = dv + at_v(d, bi, t, h);
        double beta = s.beta;

        if (s.valid) {
          for (int64_t i = 0; i < Dk; ++i)
            for (int64_t cc = 0; cc < Dv; ++cc) Sp[i * Dv + cc] = s.g[i] * Sprev[i * Dv + cc];
          for (int64_t cc = 0; cc < Dv; ++cc) {
            double acc = 0.0;
            for (int64_t i = 0; i < Dk; ++i) acc += Sp[i * Dv + cc] * s.khat[i];
            w.u[cc] = acc;
            w.delta[cc] = beta * (vt[cc] - acc);
          }
          for (int64_t i = 0; i < Dk; ++i)
            for (int64_t cc = 0; cc < Dv; ++cc)
              St[i * Dv + cc] = Sp[i * Dv + cc] + s.khat[i] * w.delta[cc];
        } else {
          memcpy(St, Sprev, sizeof(double) * SS);
        }

        /* o_t = S_t^T qt. */
        for (int64_t i = 0; i < Dk; ++i)
          for (int64_t cc = 0; cc < Dv; ++cc) D[i * Dv + cc] += s.qt[i] * dOt[cc];
        for (int64_t i = 0; i < Dk; ++i) {
          double acc = 0.0;
          for (int64_t cc = 0; cc < Dv; ++cc) acc += St[i * Dv + cc] * dOt[cc];
          dqt[i] = acc;
        }

        if (!s.valid) {
          for (int64_t i = 0; i < Dk; ++i) dkt[i] = dlt[i] = 0.0;
          for (int64_t cc = 0; cc < Dv; ++cc) dvt[cc] = 0.0;
          db[at_g(d, bi, t, h)] = 0.0;
          continue;
        }

        /* S_t = S' + k delta^T;  delta = beta (v - u). */
        for (int64_t cc = 0; cc < Dv; ++cc) {
          double acc = 0.0;
          for (int64_t i = 0; i < Dk; ++i) acc += D[i * Dv + cc] * s.khat[i];
          ddel[cc] = acc;
        }
        double dbeta = 0.0;
        for (int64_t cc = 0; cc < Dv; ++cc) {
          dvt[cc] = beta * ddel[cc];
          dbeta += ddel[cc] * (vt[cc] - w.u[cc]);
          du[cc] = -beta * ddel[cc];
        }
        /* u = S'^T k. */
        for (int64_t i = 0; i < Dk; ++i)
          for (int64_t cc = 0; cc < Dv; ++cc)
            dSp[i * Dv + cc] = D[i * Dv + cc] + s.khat[i] * du[cc];
        for (int64_t i = 0; i < Dk; ++i) {
          double acc = 0.0;
          for (int64_t cc = 0; cc < Dv; ++cc)
            acc += D[i * Dv + cc] * w.delta[cc] + Sp[i * Dv + cc] * du[cc];
          dkt[i] = acc;
        }
        /* S' = diag(g) S_prev:  dg_i = sum_c dS'[i,c] S_prev[i,c],
         * dlg_i = g_i dg_i,  dL/dS_prev = diag(g) dS'. */
        for (int64_t i = 0; i < Dk; ++i) {
          double acc = 0.0;
          for (int64_t cc = 0; cc < Dv; ++cc) acc += dSp[i * Dv + cc] * Sprev[i * Dv + cc];
          dlt[i] = s.g[i] * acc;
        }
        for (int64_t i = 0; i < Dk; ++i)
          for (int64_t cc = 0; cc < Dv; ++cc) D[i * Dv + cc] = s.g[i] * dSp[i * Dv + cc];
        db[at_g(d, bi, t, h)] = dbeta * beta * (1.0 - beta);
      }
    }
    memcpy(dstate + at_s(d, bi, h), D, sizeof(double) * SS);

    free(S); free(D); free(Sp); free(St); free(dSp); free(starts);
    free(hist); free(ddel); free(du); free(s.g);
    scratch_free(&w);
  }

  if (!err) {
    /* Group sums over the G value heads (h ascending), then the L2 backward,
     * exactly as for the scalar gate. */
    double scale = 1.0 / sqrt((double)Dk);
    double* tmp = malloc(sizeof(double) * Dk * 2);
    double *xhat = tmp, *acc = tmp ? tmp + Dk : NULL;
    for (int64_t bi = 0; bi < B && tmp; ++bi)
      for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < Hk; ++j)
          for (int pass = 0; pass < 2; ++pass) {
            const double* src = pass == 0 ? dqt_h : dkt_h;
            const double* x = (pass == 0 ? q : k) + at_qk(d, bi, t, j);
            double* out = (pass == 0 ? dq : dk) + at_qk(d, bi, t, j);
            for (int64_t i = 0; i < Dk; ++i) acc[i] = 0.0;
            for (int64_t hh = j * G; hh < (j + 1) * G; ++hh) {
              const double* p = src + ((size_t)(bi * T + t) * Hv + hh) * Dk;
              for (int64_t i = 0; i < Dk; ++i) acc[i] += p[i];
            }
            if (pass == 0)
              for (int64_t i = 0; i < Dk; ++i) acc[i] *= scale;
            double r = l2norm(x, Dk, xhat);
            double dotp = 0.0;
            for (int64_t i = 0; i < Dk; ++i) dotp += xhat[i] * acc[i];
            for (int64_t i = 0; i < Dk; ++i) out[i] = r * (acc[i] - xhat[i] * dotp);
          }
    if (!tmp) err = 2;
    free(tmp);
  }
  free(dqt_h); free(dkt_h);
  return err;
}

/*
 * Depthwise causal conv1d + SiLU update with a k-sample carry state, the op
 * that precedes the recurrence in a decode step (torch-to-nnef GDN page, the
 * causal-conv-update drop-in: layout hidden_states [b, C, S], conv_state
 * [b, C, k], weight [C, k] -> out [b, C, S], final_state [b, C, k]; the conv is
 * an unfold, a multiply and a sum).  Per batch row and channel the S new
 * samples follow the k carried ones; output s is SiLU(z) = z sigmoid(z) of the
 * tap-weighted sum z of the k most recent samples up to and including new
 * sample s (taps oldest first), and the final state holds the last k samples.
 * Returns 0, or 2 when out of memory.
 */
int oracle_conv_update(int64_t B, int64_t C, int64_t K, int64_t S, const double* x, const double* state,
                       const double* w, double* out, double* final_state) {
  double* ext = malloc((size_t)(K + S) * sizeof(double));
  if (!ext) return 2;
  for (int64_t bi = 0; bi < B; ++bi)
    for (int64_t c = 0; c < C; ++c) {
      const size_t row = (size_t)(bi * C + c);
      for (int64_t j = 0; j < K; ++j) ext[j] = state[row * K + j];
      for (int64_t s = 0; s < S; ++s) ext[K + s] = x[row * S + s];
      for (int64_t s = 0; s < S; ++s) {
        double z = 0.0;
        for (int64_t j = 0; j < K; ++j) z += w[c * K + j] * ext[s + 1 + j];
        out[row * S + s] = z * sigmoid(z);
      }
      for (int64_t j = 0; j < K; ++j) final_state[row * K + j] = ext[S + j];
    }
  free(ext);
  return 0;
}
