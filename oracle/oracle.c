/*
 * Oracle for the gated ReLU linear-attention token mixer: a plain, slow,
 * fp64 CPU implementation of what the GPU path computes.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code, header, table or helper with the HIP library; neither includes the
 * other.
 *
 * Sources (pages, sections):
 *  [V2]  "SANA-Video 2.0: Hybrid Linear Attention with Attention Residuals for
 *        Efficient Video Generation" (arXiv 2607.21553), Section 2, paragraph
 *        "Gated linear attention", Eq. (1): state, denominator with +eps,
 *        sigmoid output gate.
 *  [V1]  "SANA-Video: Efficient Video Generation with Block Linear Diffusion
 *        Transformer" (paper notes), Section 3.2 "Linear Attention with RoPE":
 *        phi = ReLU; RoPE applied after ReLU, in the numerator only; the
 *        denominator keeps the un-rotated phi; layout (B, N, H, D).
 *  [V1c] same page, Section 3.4 "Block Linear Attention with Constant-Memory
 *        KV Cache": the causal form carries the running sum of states
 *        phi(K)^T V and the running sum of phi(K) across blocks.
 *
 * Readings where the pages are silent (each one is listed in the design
 * notes of the repository):
 *  - 3D RoPE: d is split (d/4, 3d/8, 3d/8) over the (t, h, w) axes, in that
 *    order; on each axis a independent rotary rotation of adjacent pairs
 *    (2i, 2i+1) of that axis' slice by angle pos_a * theta^(-2i/d_a).
 *    theta <= 0 turns the rotation off (identity).
 *  - positions are integer grid indices; token n of a [T, Hs, Ws] grid has
 *    t = n / (Hs*Ws), h = (n / Ws) % Hs, w = n % Ws; pos0[] shifts them.
 *  - eps is added to the dot product (den = phi(q).z + eps).
 *  - the gate g has the shape of the output; sigma(x) = 1 / (1 + exp(-x)).
 *  - block-causal: blocks of F latent frames; a token of block b uses the
 *    state and normaliser summed over every token of blocks 0..b (its own
 *    block included, so attention inside a block is bidirectional).
 *
 * Arithmetic: inputs arrive as float (every bf16 value is exact in float);
 * everything is computed and returned in double.  Sums run in increasing
 * token order.  OpenMP only distributes independent (batch, head) or
 * (batch, token) work; it never splits a sum.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

#define ORA_OK 0
#define ORA_BAD_ARG 1
#define ORA_NO_MEM 2

/* Token n of a t-major [T, Hs, Ws] latent grid -> (t, h, w) ([V1] Section 3.3
 * pseudocode reshapes (B, T*H*W, D) to (B, T, H, W, D): t slowest, w fastest). */
static void grid_position(int64_t n, int64_t Hs, int64_t Ws, const int64_t *pos0,
                          int64_t pos[3]) {
  pos[0] = n / (Hs * Ws);
  pos[1] = (n / Ws) % Hs;
  pos[2] = n % Ws;
  if (pos0) {
    pos[0] += pos0[0];
    pos[1] += pos0[1];
    pos[2] += pos0[2];
  }
}

/* 3D rotary embedding of one feature vector x (length d) at grid position
 * pos = (t, h, w), written to y (y may not alias x). */
void ora_rope(const double *x, double *y, int64_t d, const int64_t pos[3], double theta) {
  int64_t width[3] = {d / 4, 3 * d / 8, 3 * d / 8};
  int64_t offset = 0;
  if (!(theta > 0.0)) {
    memcpy(y, x, (size_t)d * sizeof(double));
    return;
  }
  for (int a = 0; a < 3; ++a) {
    int64_t da = width[a];
    for (int64_t i = 0; i < da / 2; ++i) {
      double freq = pow(theta, -2.0 * (double)i / (double)da);
      double angle = (double)pos[a] * freq;
      double c = cos(angle), s = sin(angle);
      double x0 = x[offset + 2 * i], x1 = x[offset + 2 * i + 1];
      y[offset + 2 * i] = x0 * c - x1 * s;
      y[offset + 2 * i + 1] = x0 * s + x1 * c;
    }
    offset += da;
  }
}

static int check_shape(int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                       int64_t F) {
  if (B < 1 || H < 1 || T < 1 || Hs < 1 || Ws < 1) return ORA_BAD_ARG;
  if (d < 16 || d % 16 != 0) return ORA_BAD_ARG;
  if (F < 0 || (F > 0 && T % F != 0)) return ORA_BAD_ARG;
  return ORA_OK;
}

/* Number of temporal blocks: F = 0 (or F = T) is the non-causal operator. */
int64_t ora_num_blocks(int64_t T, int64_t F) { return (F <= 0) ? 1 : T / F; }

/*
 * State and normaliser ([V1] Section 3.2 pseudocode steps 1-4, [V2] Eq. 1):
 *   z        = sum_n phi(k_n)
 *   S[p][e]  = sum_n RoPE_n(phi(k_n))[p] * v_n[e]        (d x d, rows = key dim)
 * In block-causal mode ([V1c]) the values written for block b are the sums
 * over every token of blocks 0..b.
 *
 * k, v : [B, N, H, d] float, N = T*Hs*Ws
 * S    : [B, H, nb, d, d] double (output)   z : [B, H, nb, d] double (output)
 */
/* beta (optional, [B, N, H]): the write gate of [V2] Eq. (1), a factor on
 * each token's rotated key in the state only (z keeps the plain phi(k)). */
static int state_impl(const float *k, const float *v, const float *beta, int64_t B, int64_t H,
                      int64_t T, int64_t Hs, int64_t Ws, int64_t d, int64_t F, double theta,
                      const int64_t *pos0, double *S, double *z) {
  if (!k || !v || !S || !z) return ORA_BAD_ARG;
  int rc = check_shape(B, H, T, Hs, Ws, d, F);
  if (rc) return rc;
  const int64_t N = T * Hs * Ws;
  const int64_t nb = ora_num_blocks(T, F);
  const int64_t tokens_per_block = N / nb;
  int failed = 0;

#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t h = 0; h < H; ++h) {
      double *Sacc = (double *)calloc((size_t)(d * d), sizeof(double));
      double *zacc = (double *)calloc((size_t)d, sizeof(double));
      double *phik = (double *)malloc((size_t)d * sizeof(double));
      double *rotk = (double *)malloc((size_t)d * sizeof(double));
      double *vrow = (double *)malloc((size_t)d * sizeof(double));
      if (!Sacc || !zacc || !phik || !rotk || !vrow) {
#pragma omp atomic write
        failed = 1;
      } else {
        for (int64_t n = 0; n < N; ++n) {
          const float *kn = k + ((b * N + n) * H + h) * d;
          const float *vn = v + ((b * N + n) * H + h) * d;
          int64_t pos[3];
          grid_position(n, Hs, Ws, pos0, pos);
          for (int64_t p = 0; p < d; ++p) {
            double x = (double)kn[p];
            phik[p] = x > 0.0 ? x : 0.0; /* phi = ReLU */
            vrow[p] = (double)vn[p];
          }
          ora_rope(phik, rotk, d, pos, theta); /* RoPE after ReLU, numerator only */
          if (beta) { /* write gate: scales what this token writes into S */
            const double bt = (double)beta[(b * N + n) * H + h];
            for (int64_t p = 0; p < d; ++p) rotk[p] *= bt;
          }
          for (int64_t p = 0; p < d; ++p) {
            zacc[p] += phik[p]; /* normaliser: un-rotated phi(k) */
            for (int64_t e = 0; e < d; ++e) Sacc[p * d + e] += rotk[p] * vrow[e];
          }
          if ((n + 1) % tokens_per_block == 0) { /* end of a temporal block */
            int64_t blk = n / tokens_per_block;
            double *Sout = S + ((b * H + h) * nb + blk) * d * d;
            double *zout = z + ((b * H + h) * nb + blk) * d;
            memcpy(Sout, Sacc, (size_t)(d * d) * sizeof(double));
            memcpy(zout, zacc, (size_t)d * sizeof(double));
          }
        }
      }
      free(Sacc);
      free(zacc);
      free(phik);
      free(rotk);
      free(vrow);
    }
  }
  return failed ? ORA_NO_MEM : ORA_OK;
}

int ora_state(const float *k, const float *v, int64_t B, int64_t H, int64_t T, int64_t Hs,
              int64_t Ws, int64_t d, int64_t F, double theta, const int64_t *pos0, double *S,
              double *z) {
  return state_impl(k, v, NULL, B, H, T, Hs, Ws, d, F, theta, pos0, S, z);
}

/*
 * Output for a list of tokens ([V1] Section 3.2 steps 3-5 with the gate of
 * [V2] Eq. 1):
 *   num[e] = sum_p RoPE_i(phi(q_i))[p] * S[p][e]
 *   den    = sum_p phi(q_i)[p] * z[p] + eps
 *   out[e] = num[e] / den * sigma(g_i[e])
 * using the state of the token's block (block-causal) or the single state.
 *
 * q, g   : [B, N, H, d] float
 * S, z   : as written by ora_state
 * tokens : ntok token indices in [0, N), or NULL for all N tokens in order
 * out    : [B, ntok, H, d] double
 */
/* w (optional, [d]): RMSNorm of [V2] Eq. (1) on num/den over the d features,
 * y / sqrt(mean_e y[e]^2 + rms_eps) * w, before the sigmoid gate. */
static int apply_impl(const float *q, const float *g, const double *S, const double *z,
                      const float *w, double rms_eps, int64_t B, int64_t H, int64_t T, int64_t Hs,
                      int64_t Ws, int64_t d, int64_t F, double theta, double eps,
                      const int64_t *pos0, const int64_t *tokens, int64_t ntok, double *out) {
  if (!q || !g || !S || !z || !out) return ORA_BAD_ARG;
  int rc = check_shape(B, H, T, Hs, Ws, d, F);
  if (rc) return rc;
  const int64_t N = T * Hs * Ws;
  const int64_t nb = ora_num_blocks(T, F);
  const int64_t tokens_per_block = N / nb;
  if (!tokens) ntok = N;
  if (ntok < 0) return ORA_BAD_ARG;
  for (int64_t j = 0; tokens && j < ntok; ++j)
    if (tokens[j] < 0 || tokens[j] >= N) return ORA_BAD_ARG;
  int failed = 0;

#pragma omp parallel for collapse(2) schedule(dynamic, 64)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t j = 0; j < ntok; ++j) {
      double *phiq = (double *)malloc((size_t)d * sizeof(double));
      double *rotq = (double *)malloc((size_t)d * sizeof(double));
      if (!phiq || !rotq) {
#pragma omp atomic write
        failed = 1;
      } else {
        int64_t n = tokens ? tokens[j] : j;
        int64_t blk = n / tokens_per_block;
        int64_t pos[3];
        grid_position(n, Hs, Ws, pos0, pos);
        for (int64_t h = 0; h < H; ++h) {
          const float *qn = q + ((b * N + n) * H + h) * d;
          const float *gn = g + ((b * N + n) * H + h) * d;
          const double *Sh = S + ((b * H + h) * nb + blk) * d * d;
          const double *zh = z + ((b * H + h) * nb + blk) * d;
          double *on = out + ((b * ntok + j) * H + h) * d;
          for (int64_t p = 0; p < d; ++p) {
            double x = (double)qn[p];
            phiq[p] = x > 0.0 ? x : 0.0;
          }
          ora_rope(phiq, rotq, d, pos, theta);
          double den = 0.0;
          for (int64_t p = 0; p < d; ++p) den += phiq[p] * zh[p];
          den += eps;
          for (int64_t e = 0; e < d; ++e) {
            double num = 0.0;
            for (int64_t p = 0; p < d; ++p) num += rotq[p] * Sh[p * d + e];
            on[e] = num / den;
          }
          if (w) { /* RMSNorm over the d features of y = num / den */
            double ss = 0.0;
            for (int64_t e = 0; e < d; ++e) ss += on[e] * on[e];
            const double inv_rms = 1.0 / sqrt(ss / (double)d + rms_eps);
            for (int64_t e = 0; e < d; ++e) on[e] = on[e] * inv_rms * (double)w[e];
          }
          for (int64_t e = 0; e < d; ++e) {
            double gate = 1.0 / (1.0 + exp(-(double)gn[e]));
            on[e] *= gate;
          }
        }
      }
      free(phiq);
      free(rotq);
    }
  }
  return failed ? ORA_NO_MEM : ORA_OK;
}

int ora_apply(const float *q, const float *g, const double *S, const double *z, int64_t B,
              int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d, int64_t F, double theta,
              double eps, const int64_t *pos0, const int64_t *tokens, int64_t ntok,
              double *out) {
  return apply_impl(q, g, S, z, NULL, 0.0, B, H, T, Hs, Ws, d, F, theta, eps, pos0, tokens, ntok,
                    out);
}

/* The full gated mixer of [V2] Eq. (1), short of the output projection W_o:
 *   S   = sum_n beta_n RoPE_n(phi(k_n))^T v_n,   z = sum_n phi(k_n)
 *   y_i = (RoPE_i(phi(q_i)) S) / (phi(q_i) . z + eps)
 *   o_i = y_i / sqrt(mean_e y_i[e]^2 + rms_eps) * w  *  sigmoid(g_i)
 * beta: [B, N, H] (NULL: every beta_n = 1); w: [d] (NULL: no RMSNorm,
 * o_i = y_i * sigmoid(g_i)).  Block-causal like ora_forward.
 * out: [B, N, H, d] double. */
int ora_gated_forward(const float *q, const float *k, const float *v, const float *g,
                      const float *beta, const float *w, int64_t B, int64_t H, int64_t T,
                      int64_t Hs, int64_t Ws, int64_t d, int64_t F, double theta, double eps,
                      double rms_eps, double *out) {
  int rc = check_shape(B, H, T, Hs, Ws, d, F);
  if (rc) return rc;
  if (!q || !g || !out) return ORA_BAD_ARG;
  const int64_t nb = ora_num_blocks(T, F);
  double *S = (double *)malloc((size_t)(B * H * nb * d * d) * sizeof(double));
  double *z = (double *)malloc((size_t)(B * H * nb * d) * sizeof(double));
  if (!S || !z) {
    free(S);
    free(z);
    return ORA_NO_MEM;
  }
  rc = state_impl(k, v, beta, B, H, T, Hs, Ws, d, F, theta, NULL, S, z);
  if (rc == ORA_OK)
    rc = apply_impl(q, g, S, z, w, rms_eps, B, H, T, Hs, Ws, d, F, theta, eps, NULL, NULL, 0,
                    out);
  free(S);
  free(z);
  return rc;
}

/* Gradients of the operator (the loss L = sum dout . out), derived from the
 * forward definition above by the chain rule; [V2] Section 3 trains the
 * model from scratch, so the mixer needs them.  Per (batch, head), with the
 * state S^b and normaliser z^b each token of block b reads (ora_state):
 *   y_i    = num_i / den_i,   num_i = RoPE_i(phi(q_i)) S^b,   den_i = phi(q_i) . z^b + eps
 *   dg_i   = dout_i * y_i * s_i (1 - s_i),   s_i = sigmoid(g_i)
 *   dnum_i = dout_i * s_i / den_i,   dden_i = - (dout_i * s_i) . y_i / den_i
 *   dq_i   = [ RoPE_i^T(S^b dnum_i) + dden_i z^b ] * 1[q_i > 0]
 *   dS^b  += RoPE_i(phi(q_i))^T dnum_i,   dz^b += dden_i phi(q_i)
 * S^b sums the per-block states of blocks 0..b, so the gradient of block c's
 * own state is the suffix sum G^c = sum over b >= c of dS^b (likewise for z):
 *   dv_n   = RoPE_n(phi(k_n)) G^c
 *   dk_n   = [ RoPE_n^T(G^c v_n) + Gz^c ] * 1[k_n > 0]         (n in block c)
 * RoPE^T, the transpose of a rotation, is the rotation by minus the angle.
 * All inputs [B, N, H, d] float; outputs dq, dk, dv, dg [B, N, H, d] double. */
int ora_backward(const float *q, const float *k, const float *v, const float *g,
                 const float *dout, int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws,
                 int64_t d, int64_t F, double theta, double eps, double *dq, double *dk,
                 double *dv, double *dg) {
  if (!q || !k || !v || !g || !dout || !dq || !dk || !dv || !dg) return ORA_BAD_ARG;
  int rc = check_shape(B, H, T, Hs, Ws, d, F);
  if (rc) return rc;
  const int64_t N = T * Hs * Ws;
  const int64_t nb = ora_num_blocks(T, F);
  const int64_t tpb = N / nb;
  const int64_t dd = d * d;
  double *S = (double *)malloc((size_t)(B * H * nb * dd) * sizeof(double));
  double *z = (double *)malloc((size_t)(B * H * nb * d) * sizeof(double));
  if (!S || !z) {
    free(S);
    free(z);
    return ORA_NO_MEM;
  }
  rc = ora_state(k, v, B, H, T, Hs, Ws, d, F, theta, NULL, S, z);
  int failed = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t h = 0; h < H; ++h) {
      if (rc != ORA_OK) continue;
      double *dS = (double *)calloc((size_t)(nb * dd), sizeof(double));
      double *dz = (double *)calloc((size_t)(nb * d), sizeof(double));
      double *w = (double *)malloc((size_t)(8 * d) * sizeof(double));
      if (!dS || !dz || !w) {
#pragma omp atomic write
        failed = 1;
      } else {
        double *phi = w, *rot = w + d, *dy = w + 2 * d, *dnum = w + 3 * d, *t1 = w + 4 * d,
               *t2 = w + 5 * d, *vrow = w + 6 * d, *y = w + 7 * d;
        /* the q side: dq, dg and the per-block dS, dz */
        for (int64_t n = 0; n < N; ++n) {
          const int64_t row = ((b * N + n) * H + h) * d, blk = n / tpb;
          const double *Sb = S + ((b * H + h) * nb + blk) * dd;
          const double *zb = z + ((b * H + h) * nb + blk) * d;
          int64_t pos[3], neg[3];
          grid_position(n, Hs, Ws, NULL, pos);
          for (int a = 0; a < 3; ++a) neg[a] = -pos[a];
          for (int64_t p = 0; p < d; ++p) {
            const double x = (double)q[row + p];
            phi[p] = x > 0.0 ? x : 0.0;
          }
          ora_rope(phi, rot, d, pos, theta);
          double den = eps;
          for (int64_t p = 0; p < d; ++p) den += phi[p] * zb[p];
          double dyy = 0.0;
          for (int64_t e = 0; e < d; ++e) {
            double num = 0.0;
            for (int64_t p = 0; p < d; ++p) num += rot[p] * Sb[p * d + e];
            y[e] = num / den;
            const double s = 1.0 / (1.0 + exp(-(double)g[row + e]));
            dg[row + e] = (double)dout[row + e] * y[e] * s * (1.0 - s);
            dy[e] = (double)dout[row + e] * s;
            dyy += dy[e] * y[e];
          }
          const double dden = -dyy / den;
          for (int64_t e = 0; e < d; ++e) dnum[e] = dy[e] / den;
          for (int64_t p = 0; p < d; ++p) {
            double acc = 0.0;
            for (int64_t e = 0; e < d; ++e) acc += Sb[p * d + e] * dnum[e];
            t1[p] = acc; /* gradient of the rotated phi(q) */
          }
          ora_rope(t1, t2, d, neg, theta); /* back through the rotation */
          for (int64_t p = 0; p < d; ++p)
            dq[row + p] = (double)q[row + p] > 0.0 ? t2[p] + dden * zb[p] : 0.0;
          double *dSb = dS + blk * dd, *dzb = dz + blk * d;
          for (int64_t p = 0; p < d; ++p) {
            dzb[p] += dden * phi[p];
            for (int64_t e = 0; e < d; ++e) dSb[p * d + e] += rot[p] * dnum[e];
          }
        }
        /* suffix sums over blocks: the gradients of each block's own sums */
        for (int64_t blk = nb - 2; blk >= 0; --blk) {
          for (int64_t i = 0; i < dd; ++i) dS[blk * dd + i] += dS[(blk + 1) * dd + i];
          for (int64_t i = 0; i < d; ++i) dz[blk * d + i] += dz[(blk + 1) * d + i];
        }
        /* the k, v side */
        for (int64_t n = 0; n < N; ++n) {
          const int64_t row = ((b * N + n) * H + h) * d, blk = n / tpb;
          const double *G = dS + blk * dd, *Gz = dz + blk * d;
          int64_t pos[3], neg[3];
          grid_position(n, Hs, Ws, NULL, pos);
          for (int a = 0; a < 3; ++a) neg[a] = -pos[a];
          for (int64_t p = 0; p < d; ++p) {
            const double x = (double)k[row + p];
            phi[p] = x > 0.0 ? x : 0.0;
            vrow[p] = (double)v[row + p];
          }
          ora_rope(phi, rot, d, pos, theta);
          for (int64_t e = 0; e < d; ++e) {
            double acc = 0.0;
            for (int64_t p = 0; p < d; ++p) acc += rot[p] * G[p * d + e];
            dv[row + e] = acc;
          }
          for (int64_t p = 0; p < d; ++p) {
            double acc = 0.0;
            for (int64_t e = 0; e < d; ++e) acc += G[p * d + e] * vrow[e];
            t1[p] = acc;
          }
          ora_rope(t1, t2, d, neg, theta);
          for (int64_t p = 0; p < d; ++p)
            dk[row + p] = (double)k[row + p] > 0.0 ? t2[p] + Gz[p] : 0.0;
        }
      }
      free(dS);
      free(dz);
      free(w);
    }
  }
  free(S);
  free(z);
  if (rc != ORA_OK) return rc;
  return failed ? ORA_NO_MEM : ORA_OK;
}

/* Whole operator: ora_state followed by ora_apply over every token.
 * out : [B, N, H, d] double. */
int ora_forward(const float *q, const float *k, const float *v, const float *g, int64_t B,
                int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d, int64_t F,
                double theta, double eps, const int64_t *pos0, double *out) {
  int rc = check_shape(B, H, T, Hs, Ws, d, F);
  if (rc) return rc;
  const int64_t nb = ora_num_blocks(T, F);
  double *S = (double *)malloc((size_t)(B * H * nb * d * d) * sizeof(double));
  double *z = (double *)malloc((size_t)(B * H * nb * d) * sizeof(double));
  if (!S || !z) {
    free(S);
    free(z);
    return ORA_NO_MEM;
  }
  rc = ora_state(k, v, B, H, T, Hs, Ws, d, F, theta, pos0, S, z);
  if (rc == ORA_OK)
    rc = ora_apply(q, g, S, z, B, H, T, Hs, Ws, d, F, theta, eps, pos0, NULL, 0, out);
  free(S);
  free(z);
  return rc;
}

/* One step of the streaming block-causal mode ([V1c], and Algorithm 1 on the
 * same page: a block is generated with the cache of the earlier blocks, and
 * the cache is then updated with the block's own sums).  The block holds Tb
 * latent frames of a Tb x Hs x Ws grid whose first frame sits at absolute
 * temporal position t_offset; (S_cache, z_cache) are the sums over every
 * earlier block ([B, H, d, d] and [B, H, d] double).  The block attends to
 * itself and to the cache, as in the causal form on that page:
 *   S_tot = S_cache + S_blk,  z_tot = z_cache + z_blk,
 *   out   = the apply step with (S_tot, z_tot)        (skipped if out is NULL)
 *   S_new = S_tot, z_new = z_tot                      (if non-NULL)
 * q and g may be NULL when out is NULL. */
int ora_block_step(const float *q, const float *k, const float *v, const float *g,
                   const double *S_cache, const double *z_cache, int64_t B, int64_t H,
                   int64_t Tb, int64_t Hs, int64_t Ws, int64_t d, int64_t t_offset, double theta,
                   double eps, double *out, double *S_new, double *z_new) {
  if (!k || !v || !S_cache || !z_cache || t_offset < 0) return ORA_BAD_ARG;
  if (out && (!q || !g)) return ORA_BAD_ARG;
  int rc = check_shape(B, H, Tb, Hs, Ws, d, 0);
  if (rc) return rc;
  const int64_t pos0[3] = {t_offset, 0, 0};
  double *S = (double *)malloc((size_t)(B * H * d * d) * sizeof(double));
  double *z = (double *)malloc((size_t)(B * H * d) * sizeof(double));
  if (!S || !z) {
    free(S);
    free(z);
    return ORA_NO_MEM;
  }
  rc = ora_state(k, v, B, H, Tb, Hs, Ws, d, 0, theta, pos0, S, z); /* the block's own sums */
  if (rc == ORA_OK) {
    for (int64_t i = 0; i < B * H * d * d; ++i) S[i] += S_cache[i];
    for (int64_t i = 0; i < B * H * d; ++i) z[i] += z_cache[i];
    if (out) rc = ora_apply(q, g, S, z, B, H, Tb, Hs, Ws, d, 0, theta, eps, pos0, NULL, 0, out);
    if (S_new) memcpy(S_new, S, (size_t)(B * H * d * d) * sizeof(double));
    if (z_new) memcpy(z_new, z, (size_t)(B * H * d) * sizeof(double));
  }
  free(S);
  free(z);
  return rc;
}

/* Token-causal form ([V1c], the causal linear-attention output of token i
 * derived there for the KV cache): token i attends to tokens 0..i, itself
 * included, through the running sums of the states and of phi(k):
 *   S_i = sum_{j<=i} RoPE_j(phi(k_j))^T v_j,   z_i = sum_{j<=i} phi(k_j)
 *   out_i = RoPE_i(phi(q_i)) S_i / (phi(q_i).z_i + eps) * sigma(g_i)
 * with the same RoPE, eps and gate readings as the other forms.  One pass per
 * (batch, head) in increasing token order: token n is added to the sums,
 * then read them.  out : [B, N, H, d] double. */

/* S += RoPE_n(phi(k_n))^T v_n and z += phi(k_n) for the row at k + row, v + row. */
static void causal_add(const float *k, const float *v, int64_t row, int64_t d,
                       const int64_t pos[3], double theta, double *phik, double *rotk, double *S,
                       double *z) {
  for (int64_t p = 0; p < d; ++p) {
    double x = (double)k[row + p];
    phik[p] = x > 0.0 ? x : 0.0;
  }
  ora_rope(phik, rotk, d, pos, theta);
  for (int64_t p = 0; p < d; ++p) {
    z[p] += phik[p];
    for (int64_t e = 0; e < d; ++e) S[p * d + e] += rotk[p] * (double)v[row + e];
  }
}

/* out_n from the current sums. */
static void causal_read(const float *q, const float *g, int64_t row, int64_t d,
                        const int64_t pos[3], double theta, double eps, double *phiq,
                        double *rotq, const double *S, const double *z, double *out) {
  for (int64_t p = 0; p < d; ++p) {
    double x = (double)q[row + p];
    phiq[p] = x > 0.0 ? x : 0.0;
  }
  ora_rope(phiq, rotq, d, pos, theta);
  double den = 0.0;
  for (int64_t p = 0; p < d; ++p) den += phiq[p] * z[p];
  den += eps;
  for (int64_t e = 0; e < d; ++e) {
    double num = 0.0;
    for (int64_t p = 0; p < d; ++p) num += rotq[p] * S[p * d + e];
    out[row + e] = num / den / (1.0 + exp(-(double)g[row + e]));
  }
}

int ora_token_causal(const float *q, const float *k, const float *v, const float *g, int64_t B,
                     int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d, double theta,
                     double eps, double *out) {
  if (!q || !k || !v || !g || !out) return ORA_BAD_ARG;
  int rc = check_shape(B, H, T, Hs, Ws, d, 0);
  if (rc) return rc;
  const int64_t N = T * Hs * Ws;
  int failed = 0;

#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t h = 0; h < H; ++h) {
      double *S = (double *)calloc((size_t)(d * d), sizeof(double));
      double *z = (double *)calloc((size_t)d, sizeof(double));
      double *tmp = (double *)malloc((size_t)(4 * d) * sizeof(double));
      if (!S || !z || !tmp) {
#pragma omp atomic write
        failed = 1;
      } else {
        for (int64_t n = 0; n < N; ++n) {
          const int64_t row = ((b * N + n) * H + h) * d;
          int64_t pos[3];
          grid_position(n, Hs, Ws, NULL, pos);
          causal_add(k, v, row, d, pos, theta, tmp, tmp + d, S, z);
          causal_read(q, g, row, d, pos, theta, eps, tmp + 2 * d, tmp + 3 * d, S, z, out);
        }
      }
      free(S);
      free(z);
      free(tmp);
    }
  }
  return failed ? ORA_NO_MEM : ORA_OK;
}

/* Number of threads OpenMP will use (reported by the benchmark's CPU leg). */
int ora_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      n = omp_get_num_threads();
#endif
    }
  }
  return n;
}
