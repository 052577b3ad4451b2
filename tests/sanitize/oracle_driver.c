/* Driver of the fp64 oracle for the sanitizer build (gcc with
 * AddressSanitizer + UndefinedBehaviorSanitizer): forward, backward in both
 * storage modes (every state kept / recomputed from checkpoints), the
 * per-key-channel gate and the conv update, over shapes that cover a ragged
 * last chunk, masks, an empty sequence, a single step and GQA.  Checks that
 * every call succeeds, that the outputs are finite and that the two backward
 * modes agree bit for bit.  Exits 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int64_t B, T, Hk, Hv, Dk, Dv;
} oracle_dims;
int oracle_gdn_fwd(const oracle_dims*, const double*, const double*, const double*, const double*, const double*,
                   const double*, const double*, const double*, const uint8_t*, double*, double*, double*, int);
int oracle_gdn_bwd(const oracle_dims*, const double*, const double*, const double*, const double*, const double*,
                   const double*, const double*, const double*, const uint8_t*, const double*, const double*,
                   double*, double*, double*, double*, double*, double*, double*, double*, int64_t, int);
int oracle_gdn_fwd_vg(const oracle_dims*, const double*, const double*, const double*, const double*, const double*,
                      const double*, const uint8_t*, double*, double*, double*, int);
int oracle_gdn_bwd_vg(const oracle_dims*, const double*, const double*, const double*, const double*, const double*,
                      const double*, const uint8_t*, const double*, const double*, double*, double*, double*,
                      double*, double*, double*, int64_t, int);
int oracle_conv_update(int64_t, int64_t, int64_t, int64_t, const double*, const double*, const double*, double*,
                       double*);

static uint64_t g_rng = 88172645463325252ull;
static double uni(void) { /* xorshift64, uniform in (-1, 1) */
  g_rng ^= g_rng << 13;
  g_rng ^= g_rng >> 7;
  g_rng ^= g_rng << 17;
  return (double)(g_rng >> 11) / 4503599627370496.0 - 1.0;
}
static double* arr(size_t n, double scale) {
  double* p = malloc((n ? n : 1) * sizeof(double));
  for (size_t i = 0; i < n; ++i) p[i] = scale * uni();
  return p;
}
static int finite(const double* p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

static int run(int64_t B, int64_t T, int64_t Hk, int64_t Hv, int64_t Dk, int64_t Dv, int masked) {
  oracle_dims d = {B, T, Hk, Hv, Dk, Dv};
  const size_t nq = (size_t)(B * T * Hk * Dk), nv = (size_t)(B * T * Hv * Dv), ng = (size_t)(B * T * Hv);
  const size_t ns = (size_t)(B * Hv * Dk * Dv), nc = T > 0 ? (size_t)((T + 63) / 64 - 1) : 0;
  double *q = arr(nq, 1), *k = arr(nq, 1), *v = arr(nv, 1), *a = arr(ng, 2), *b = arr(ng, 2);
  double *Al = arr((size_t)Hv, 1), *dtb = arr((size_t)Hv, 0.5), *s0 = arr(ns, 0.1), *dO = arr(nv, 1),
         *dS = arr(ns, 1), *lg = arr((size_t)(B * T * Hv * Dk), 1);
  for (size_t i = 0; i < (size_t)(B * T * Hv * Dk); ++i) lg[i] = -fabs(lg[i]) * 2.0;
  uint8_t* m = NULL;
  if (masked) {
    m = malloc((size_t)(B * T) + 1);
    for (int64_t i = 0; i < B * T; ++i) m[i] = (uint8_t)((i % T) < T / 2 || (i / T) % 2 == 0);
  }
  double *o = arr(nv, 0), *so = arr(ns, 0), *ck = arr(nc * ns, 0);
  int rc = oracle_gdn_fwd(&d, q, k, v, a, b, Al, dtb, s0, m, o, so, nc ? ck : NULL, 2);
  int ok = rc == 0 && finite(o, nv) && finite(so, ns) && finite(ck, nc * ns);
  double* g1[8];
  double* g2[8];
  const size_t sz[8] = {nq, nq, nv, ng, ng, (size_t)Hv, (size_t)Hv, ns};
  for (int i = 0; i < 8; ++i) {
    g1[i] = arr(sz[i], 0);
    g2[i] = arr(sz[i], 0);
  }
  rc = oracle_gdn_bwd(&d, q, k, v, a, b, Al, dtb, s0, m, dO, dS, g1[0], g1[1], g1[2], g1[3], g1[4], g1[5], g1[6],
                      g1[7], 64, 2);
  ok = ok && rc == 0;
  rc = oracle_gdn_bwd(&d, q, k, v, a, b, Al, dtb, s0, m, dO, dS, g2[0], g2[1], g2[2], g2[3], g2[4], g2[5], g2[6],
                      g2[7], 0, 1);
  ok = ok && rc == 0;
  for (int i = 0; i < 8; ++i) ok = ok && finite(g1[i], sz[i]) && memcmp(g1[i], g2[i], sz[i] * sizeof(double)) == 0;
  rc = oracle_gdn_fwd_vg(&d, q, k, v, lg, b, s0, m, o, so, nc ? ck : NULL, 2);
  ok = ok && rc == 0 && finite(o, nv);
  rc = oracle_gdn_bwd_vg(&d, q, k, v, lg, b, s0, m, dO, dS, g1[0], g1[1], g1[2], lg, g1[4], g1[7], 64, 2);
  ok = ok && rc == 0 && finite(g1[0], nq) && finite(lg, (size_t)(B * T * Hv * Dk));
  if (!ok) fprintf(stderr, "FAIL oracle B%ld T%ld Hk%ld Hv%ld Dk%ld Dv%ld masked %d\n", (long)B, (long)T, (long)Hk,
                   (long)Hv, (long)Dk, (long)Dv, masked);
  free(q); free(k); free(v); free(a); free(b); free(Al); free(dtb); free(s0); free(dO); free(dS); free(lg);
  free(m); free(o); free(so); free(ck);
  for (int i = 0; i < 8; ++i) {
    free(g1[i]);
    free(g2[i]);
  }
  return ok;
}

int main(void) {
  const int64_t shapes[][6] = {{1, 8, 2, 4, 16, 8}, {2, 65, 1, 2, 8, 4}, {2, 130, 2, 2, 16, 8},
                               {1, 0, 1, 2, 4, 4},  {3, 1, 1, 3, 8, 8}, {1, 200, 1, 1, 32, 16}};
  for (int s = 0; s < 6; ++s)
    for (int masked = 0; masked < 2; ++masked)
      if (!run(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], shapes[s][4], shapes[s][5], masked)) return 1;
  /* conv update: 2 rows, 5 channels, 4 taps, 3 new samples */
  double *x = arr(2 * 5 * 3, 1), *st = arr(2 * 5 * 4, 1), *w = arr(5 * 4, 1), *out = arr(2 * 5 * 3, 0),
         *fin = arr(2 * 5 * 4, 0);
  int rc = oracle_conv_update(2, 5, 4, 3, x, st, w, out, fin);
  int ok = rc == 0 && finite(out, 30) && finite(fin, 40);
  free(x); free(st); free(w); free(out); free(fin);
  if (!ok) {
    fprintf(stderr, "FAIL conv update\n");
    return 1;
  }
  printf("ok\n");
  return 0;
}
