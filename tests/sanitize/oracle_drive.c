/*
 * Drives every entry point of oracle/oracle.c on small seeded inputs, and
 * with bad arguments, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  Exit status 0:
 * every call returned the expected code and every output is finite.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void ora_rope(const double *x, double *y, int64_t d, const int64_t pos[3], double theta);
int64_t ora_num_blocks(int64_t T, int64_t F);
int ora_state(const float *k, const float *v, int64_t B, int64_t H, int64_t T, int64_t Hs,
              int64_t Ws, int64_t d, int64_t F, double theta, const int64_t *pos0, double *S,
              double *z);
int ora_apply(const float *q, const float *g, const double *S, const double *z, int64_t B,
              int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d, int64_t F, double theta,
              double eps, const int64_t *pos0, const int64_t *tokens, int64_t ntok, double *out);
int ora_gated_forward(const float *q, const float *k, const float *v, const float *g,
                      const float *beta, const float *w, int64_t B, int64_t H, int64_t T,
                      int64_t Hs, int64_t Ws, int64_t d, int64_t F, double theta, double eps,
                      double rms_eps, double *out);
int ora_backward(const float *q, const float *k, const float *v, const float *g,
                 const float *dout, int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws,
                 int64_t d, int64_t F, double theta, double eps, double *dq, double *dk,
                 double *dv, double *dg);
int ora_forward(const float *q, const float *k, const float *v, const float *g, int64_t B,
                int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d, int64_t F,
                double theta, double eps, const int64_t *pos0, double *out);
int ora_block_step(const float *q, const float *k, const float *v, const float *g,
                   const double *S_cache, const double *z_cache, int64_t B, int64_t H,
                   int64_t Tb, int64_t Hs, int64_t Ws, int64_t d, int64_t t_offset, double theta,
                   double eps, double *out, double *S_new, double *z_new);
int ora_token_causal(const float *q, const float *k, const float *v, const float *g, int64_t B,
                     int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d, double theta,
                     double eps, double *out);

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static float uniform(void) { /* xorshift64, in (-1, 1) */
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (float)((double)(rng >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}
static float *fill(size_t n) {
  float *p = malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) p[i] = uniform();
  return p;
}
static int all_finite(const double *p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

static void run_shape(int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                      int64_t F) {
  const int64_t N = T * Hs * Ws, nb = ora_num_blocks(T, F);
  const size_t n = (size_t)(B * N * H * d);
  float *q = fill(n), *k = fill(n), *v = fill(n), *g = fill(n), *dout = fill(n);
  float *beta = fill((size_t)(B * N * H)), *w = fill((size_t)d);
  double *out = malloc(n * sizeof(double)), *out2 = malloc(n * sizeof(double));
  double *S = malloc((size_t)(B * H * nb * d * d) * sizeof(double));
  double *z = malloc((size_t)(B * H * nb * d) * sizeof(double));
  double *grads[4];
  for (int i = 0; i < 4; ++i) grads[i] = malloc(n * sizeof(double));

  EXPECT(ora_forward(q, k, v, g, B, H, T, Hs, Ws, d, F, 1e4, 1e-6, NULL, out) == 0);
  EXPECT(all_finite(out, n));
  EXPECT(ora_state(k, v, B, H, T, Hs, Ws, d, F, 1e4, NULL, S, z) == 0);
  EXPECT(all_finite(S, (size_t)(B * H * nb * d * d)) && all_finite(z, (size_t)(B * H * nb * d)));
  EXPECT(ora_apply(q, g, S, z, B, H, T, Hs, Ws, d, F, 1e4, 1e-6, NULL, NULL, N, out2) == 0);
  EXPECT(all_finite(out2, n));
  const int64_t tokens[3] = {0, N / 2, N - 1};
  EXPECT(ora_apply(q, g, S, z, B, H, T, Hs, Ws, d, F, 1e4, 1e-6, NULL, tokens, 3, out2) == 0);
  EXPECT(ora_gated_forward(q, k, v, g, beta, w, B, H, T, Hs, Ws, d, F, 1e4, 1e-6, 1e-6, out) == 0);
  EXPECT(all_finite(out, n));
  EXPECT(ora_backward(q, k, v, g, dout, B, H, T, Hs, Ws, d, F, 1e4, 1e-6, grads[0], grads[1],
                      grads[2], grads[3]) == 0);
  for (int i = 0; i < 4; ++i) EXPECT(all_finite(grads[i], n));
  if (F == 0) {
    EXPECT(ora_token_causal(q, k, v, g, B, H, T, Hs, Ws, d, 1e4, 1e-6, out) == 0);
    EXPECT(all_finite(out, n));
    /* one block step over the whole grid from a zero cache */
    double *S0 = calloc((size_t)(B * H * d * d), sizeof(double));
    double *z0 = calloc((size_t)(B * H * d), sizeof(double));
    EXPECT(ora_block_step(q, k, v, g, S0, z0, B, H, T, Hs, Ws, d, 2, 1e4, 1e-6, out, S, z) == 0);
    EXPECT(all_finite(out, n));
    free(S0);
    free(z0);
  }
  double y[128], x[128];
  const int64_t pos[3] = {T - 1, Hs - 1, Ws - 1};
  for (int64_t i = 0; i < d; ++i) x[i] = uniform();
  ora_rope(x, y, d, pos, 1e4);
  EXPECT(all_finite(y, (size_t)d));

  free(q); free(k); free(v); free(g); free(dout); free(beta); free(w);
  free(out); free(out2); free(S); free(z);
  for (int i = 0; i < 4; ++i) free(grads[i]);
}

int main(void) {
  run_shape(2, 2, 4, 3, 5, 32, 0);
  run_shape(1, 3, 4, 2, 3, 64, 2);
  run_shape(1, 1, 3, 2, 2, 16, 1);
  run_shape(1, 2, 2, 3, 3, 128, 0);

  /* bad arguments: a code, never a crash */
  float a[64] = {0};
  double o[64];
  EXPECT(ora_forward(a, a, a, a, 0, 1, 1, 1, 1, 16, 0, 1e4, 1e-6, NULL, o) != 0);
  EXPECT(ora_forward(a, a, a, a, 1, 1, 1, 1, 1, 24, 0, 1e4, 1e-6, NULL, o) != 0);
  EXPECT(ora_forward(a, a, a, a, 1, 1, 3, 1, 1, 16, 2, 1e4, 1e-6, NULL, o) != 0);
  EXPECT(ora_backward(NULL, a, a, a, a, 1, 1, 1, 1, 1, 16, 0, 1e4, 1e-6, o, o, o, o) != 0);
  EXPECT(ora_token_causal(a, a, a, NULL, 1, 1, 1, 1, 1, 16, 1e4, 1e-6, o) != 0);
  EXPECT(ora_block_step(a, a, a, a, NULL, NULL, 1, 1, 1, 1, 1, 16, 0, 1e4, 1e-6, o, o, o) != 0);
  if (failures) fprintf(stderr, "%d expectation(s) failed\n", failures);
  return failures ? 1 : 0;
}
