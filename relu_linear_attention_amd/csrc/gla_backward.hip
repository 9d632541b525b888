// Gradients of the operator (vector kernels, fp32 arithmetic, every
// supported head size, bf16 or fp32 tensors): with the loss L = sum dout *
// out, per (batch, head) and token i of temporal block b,
//
//   y_i    = num_i / den_i,   num_i = RoPE_i(phi(q_i)) S^b,   den_i = phi(q_i).z^b + eps
//   dg_i   = dout_i * y_i * s_i (1 - s_i),   s_i = sigmoid(g_i)
//   dnum_i = dout_i * s_i / den_i,   dden_i = -(dout_i * s_i) . y_i / den_i
//   dq_i   = [RoPE_i^T(S^b dnum_i) + dden_i z^b] * 1[q_i > 0]
//   dS^b  += RoPE_i(phi(q_i))^T dnum_i,   dz^b += dden_i phi(q_i)
//   G^c    = sum over b >= c of dS^b (likewise Gz^c)
//   dv_n   = RoPE_n(phi(k_n)) G^c,   dk_n = [RoPE_n^T(G^c v_n) + Gz^c] * 1[k_n > 0]
//
// (the chain rule through "SANA-Video 2.0" Section 2 Eq. (1) and the
// "SANA-Video" notes page Sections 3.2 and 3.4).  RoPE^T rotates by minus
// the angle.  S^b, z^b come from the forward state stage (re-run by the
// backward call).  Three kernels: the q side (dq, dg and the dS, dz
// partials of each token range), the reduce (chunk sums, then the suffix
// sums over blocks), the k/v side (dk, dv).

#include <hip/hip_runtime.h>

#include "gla_internal.h"

namespace gla {
namespace {

struct BwdArgs {
  int64_t N, H, Hs, Ws;
  int64_t nb, L, Rb, Lb;
  int64_t tab_h_off, tab_w_off;
  float eps;
};

template <typename TIn>
__device__ __forceinline__ float ld(const TIn *p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float *p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t *p, int64_t i) {
  return bf16_bits_to_float(p[i]);
}
template <typename TIn>
__device__ __forceinline__ void st(TIn *p, int64_t i, float x);
template <>
__device__ __forceinline__ void st<float>(float *p, int64_t i, float x) {
  p[i] = x;
}
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t *p, int64_t i, float x) {
  __bf16 h = (__bf16)x;  // round to nearest even
  p[i] = __builtin_bit_cast(uint16_t, h);
}

// (cos, sin) of feature pair P of a token at (t, h, w), from the fp64-built
// table (t rows, then h rows, then w rows).
template <int D>
__device__ __forceinline__ float2 pair_cs(const float2 *__restrict__ tab, const BwdArgs &a, int P,
                                          int t, int h, int w) {
  constexpr int pt = D / 8, ph = 3 * D / 16;
  if (P < pt) return tab[(int64_t)t * pt + P];
  if (P < pt + ph) return tab[a.tab_h_off + (int64_t)h * ph + (P - pt)];
  return tab[a.tab_w_off + (int64_t)w * ph + (P - pt - ph)];
}

constexpr int kTokB = 16;  // tokens per tile

// LDS row stride of the d x d matrices (S, G): four floats of padding per
// row keep the rows 16-byte aligned for float4 reads and put lanes that read
// four-wide chunks of different rows (the dq and dk loops) into different
// banks eight lanes at a time, the rate of any 16-byte wave read.
template <int D>
constexpr int kRow = D + 4;

// Register blocking of the small products: a thread computes two tokens of
// one four-wide group of output features (row reads of S), or two tokens of
// one feature pair (column reads of S, four-wide chunks along e).
__device__ __forceinline__ float4 lds4(const float *p) {
  return *reinterpret_cast<const float4 *>(p);
}
__device__ __forceinline__ void fma4(float (&acc)[4], float a, const float4 b) {
  acc[0] = __builtin_fmaf(a, b.x, acc[0]);
  acc[1] = __builtin_fmaf(a, b.y, acc[1]);
  acc[2] = __builtin_fmaf(a, b.z, acc[2]);
  acc[3] = __builtin_fmaf(a, b.w, acc[3]);
}
__device__ __forceinline__ float dot4(const float4 a, const float4 b, float acc) {
  acc = __builtin_fmaf(a.x, b.x, acc);
  acc = __builtin_fmaf(a.y, b.y, acc);
  acc = __builtin_fmaf(a.z, b.z, acc);
  return __builtin_fmaf(a.w, b.w, acc);
}

// One workgroup per (unit, token range of Lb tokens).  The unit's S, z sit
// in LDS; thread t owns a (D/16) x (D/16) block of the range's dS partial,
// rows (t/16)*D/16.., columns (t%16)*D/16.. (and dz[t] for t < D), written to
// slot unit*Rb + r.  Per token a thread reads D/16 values of RoPE(phi(q))
// and of dnum and updates (D/16)^2 sums.
template <typename TIn, int D>
__global__ __launch_bounds__(kBlock) void bwd_q_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ g, const TIn *__restrict__ dout,
    const float *__restrict__ states, const float2 *__restrict__ tab, TIn *__restrict__ dq,
    TIn *__restrict__ dg, float *__restrict__ partials, BwdArgs a) {
  constexpr int BK = D / 16;
  constexpr int SP = kRow<D>;
  extern __shared__ float lds[];
  float *s_S = lds;                  // D rows of SP
  float *s_z = s_S + D * SP;         // D
  float *s_phi = s_z + D;            // kTok*D   phi(q)
  float *s_rot = s_phi + kTokB * D;  // kTok*D   RoPE(phi(q))
  float *s_dn = s_rot + kTokB * D;   // kTok*D   dnum
  float *s_t = s_dn + kTokB * D;     // kTok*D   dy * y
  float *s_den = s_t + kTokB * D;    // kTok
  float *s_dd = s_den + kTokB;       // kTok     dden

  const int64_t wg = blockIdx.x;
  const int64_t unit = wg / a.Rb, r = wg % a.Rb;
  const int64_t bh = unit / a.nb, blk = unit % a.nb;
  const int64_t b = bh / a.H, hd = bh % a.H;
  const int64_t n_begin = blk * a.L + r * a.Lb;
  const int64_t n_end = min(n_begin + a.Lb, (blk + 1) * a.L);
  const int tid = threadIdx.x;

  const float *stt = states + unit * (int64_t)(D * D + D);
  for (int i = tid; i < D * D; i += kBlock) s_S[(i / D) * SP + i % D] = stt[i];
  for (int i = tid; i < D; i += kBlock) s_z[i] = stt[D * D + i];

  const int pb = tid / 16, eb = tid % 16;  // this thread's block of dS
  float acc[BK * BK];
#pragma unroll
  for (int m = 0; m < BK * BK; ++m) acc[m] = 0.f;
  float zacc = 0.f;
  __syncthreads();

  for (int64_t n0 = n_begin; n0 < n_end; n0 += kTokB) {
    // phi(q) and its rotation
    for (int i = tid; i < kTokB * (D / 2); i += kBlock) {
      const int s = i / (D / 2), P = i % (D / 2);
      const int64_t n = n0 + s;
      float q0 = 0.f, q1 = 0.f, r0 = 0.f, r1 = 0.f;
      if (n < n_end) {
        const int64_t base = ((b * a.N + n) * a.H + hd) * D + 2 * P;
        q0 = fmaxf(ld(q, base), 0.f);
        q1 = fmaxf(ld(q, base + 1), 0.f);
        int t, h, w;
        grid_pos(n, a.Hs, a.Ws, t, h, w);
        const float2 cs = pair_cs<D>(tab, a, P, t, h, w);
        r0 = q0 * cs.x - q1 * cs.y;
        r1 = q0 * cs.y + q1 * cs.x;
      }
      s_phi[s * D + 2 * P] = q0;
      s_phi[s * D + 2 * P + 1] = q1;
      s_rot[s * D + 2 * P] = r0;
      s_rot[s * D + 2 * P + 1] = r1;
    }
    __syncthreads();
    if (tid < kTokB) {
      float den = 0.f;
      for (int p = 0; p < D; ++p) den += s_phi[tid * D + p] * s_z[p];
      s_den[tid] = den + a.eps;
    }
    __syncthreads();
    // y, dg, dnum and dy * y: tokens (2j, 2j+1) x features 4i..4i+3 per item
    for (int it = tid; it < (kTokB / 2) * (D / 4); it += kBlock) {
      const int s0 = 2 * (it / (D / 4)), e0 = 4 * (it % (D / 4));
      float num[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll 4
      for (int p = 0; p < D; ++p) {
        const float4 sv = lds4(s_S + p * SP + e0);
        fma4(num[0], s_rot[s0 * D + p], sv);
        fma4(num[1], s_rot[(s0 + 1) * D + p], sv);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int s = s0 + u;
        const int64_t n = n0 + s;
        const float den = s_den[s];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = e0 + j;
          float dn = 0.f, t = 0.f;
          if (n < n_end) {
            const float y = num[u][j] / den;
            const int64_t idx = ((b * a.N + n) * a.H + hd) * D + e;
            const float sg = 1.f / (1.f + expf(-ld(g, idx)));
            const float go = ld(dout, idx);
            st(dg, idx, go * y * sg * (1.f - sg));
            const float dy = go * sg;
            dn = dy / den;
            t = dy * y;
          }
          s_dn[s * D + e] = dn;
          s_t[s * D + e] = t;
        }
      }
    }
    __syncthreads();
    if (tid < kTokB) {
      float sum = 0.f;
      for (int e = 0; e < D; ++e) sum += s_t[tid * D + e];
      s_dd[tid] = -sum / s_den[tid];
    }
    __syncthreads();
    // dq: back through S (S dnum), the rotation and the ReLU, plus dden z;
    // tokens (2j, 2j+1) x feature pair P per item
    for (int it = tid; it < (kTokB / 2) * (D / 2); it += kBlock) {
      const int s0 = 2 * (it / (D / 2)), P = it % (D / 2);
      float d[2][2] = {{0.f, 0.f}, {0.f, 0.f}};  // [token][row 2P, 2P+1]
#pragma unroll 4
      for (int e = 0; e < D; e += 4) {
        const float4 r0 = lds4(s_S + (2 * P) * SP + e), r1 = lds4(s_S + (2 * P + 1) * SP + e);
        const float4 x0 = lds4(s_dn + s0 * D + e), x1 = lds4(s_dn + (s0 + 1) * D + e);
        d[0][0] = dot4(r0, x0, d[0][0]);
        d[0][1] = dot4(r1, x0, d[0][1]);
        d[1][0] = dot4(r0, x1, d[1][0]);
        d[1][1] = dot4(r1, x1, d[1][1]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int s = s0 + u;
        const int64_t n = n0 + s;
        if (n < n_end) {
          int t, h, w;
          grid_pos(n, a.Hs, a.Ws, t, h, w);
          const float2 cs = pair_cs<D>(tab, a, P, t, h, w);
          const float dd = s_dd[s];
          const float u0 = d[u][0] * cs.x + d[u][1] * cs.y + dd * s_z[2 * P];
          const float u1 = -d[u][0] * cs.y + d[u][1] * cs.x + dd * s_z[2 * P + 1];
          const int64_t base = ((b * a.N + n) * a.H + hd) * D + 2 * P;
          st(dq, base, s_phi[s * D + 2 * P] > 0.f ? u0 : 0.f);
          st(dq, base + 1, s_phi[s * D + 2 * P + 1] > 0.f ? u1 : 0.f);
        }
      }
    }
    // this range's dS and dz
#pragma unroll 2
    for (int s = 0; s < kTokB; ++s) {
      float rv[BK], dv[BK];
#pragma unroll
      for (int i = 0; i < BK; ++i) rv[i] = s_rot[s * D + pb * BK + i];
#pragma unroll
      for (int j = 0; j < BK; ++j) dv[j] = s_dn[s * D + eb * BK + j];
#pragma unroll
      for (int i = 0; i < BK; ++i)
#pragma unroll
        for (int j = 0; j < BK; ++j) acc[i * BK + j] = __builtin_fmaf(rv[i], dv[j], acc[i * BK + j]);
    }
    if (tid < D) {
#pragma unroll
      for (int s = 0; s < kTokB; ++s) zacc += s_dd[s] * s_phi[s * D + tid];
    }
    __syncthreads();
  }
  float *dst = partials + wg * (int64_t)(D * D + D);
#pragma unroll
  for (int i = 0; i < BK; ++i)
#pragma unroll
    for (int j = 0; j < BK; ++j) dst[(pb * BK + i) * D + eb * BK + j] = acc[i * BK + j];
  if (tid < D) dst[D * D + tid] = zacc;
}

// Fixed-order sums of the Rb range partials of each unit, then the suffix
// sums over the temporal blocks of a (batch, head), last block first:
// G[unit of block c] = sum over blocks b >= c.  One thread owns four
// consecutive floats of the d*d + d vector.
__global__ __launch_bounds__(kBlock) void bwd_reduce_kernel(const float *__restrict__ partials,
                                                            float *__restrict__ grads,
                                                            int64_t nb, int64_t Rb, int d) {
  const int64_t stride = (int64_t)d * d + d;
  const int64_t bh = blockIdx.x;
  const int64_t i4 = ((int64_t)blockIdx.y * blockDim.x + threadIdx.x) * 4;
  if (i4 >= stride) return;
  float4 run = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t blk = nb - 1; blk >= 0; --blk) {
    const int64_t unit = bh * nb + blk;
    add_partials(run, partials + unit * Rb * stride + i4, stride, 0, Rb);
    *reinterpret_cast<float4 *>(grads + unit * stride + i4) = run;
  }
}

// One workgroup per (unit, token range): dv and dk of the range's tokens,
// with the unit's G, Gz in LDS.
template <typename TIn, int D>
__global__ __launch_bounds__(kBlock) void bwd_kv_kernel(
    const TIn *__restrict__ k, const TIn *__restrict__ v, const float *__restrict__ grads,
    const float2 *__restrict__ tab, TIn *__restrict__ dk, TIn *__restrict__ dv, BwdArgs a) {
  constexpr int SP = kRow<D>;
  extern __shared__ float lds[];
  float *s_G = lds;                  // D rows of SP
  float *s_Gz = s_G + D * SP;        // D
  float *s_phi = s_Gz + D;           // kTok*D   phi(k)
  float *s_rot = s_phi + kTokB * D;  // kTok*D   RoPE(phi(k))
  float *s_v = s_rot + kTokB * D;    // kTok*D

  const int64_t wg = blockIdx.x;
  const int64_t unit = wg / a.Rb, r = wg % a.Rb;
  const int64_t bh = unit / a.nb, blk = unit % a.nb;
  const int64_t b = bh / a.H, hd = bh % a.H;
  const int64_t n_begin = blk * a.L + r * a.Lb;
  const int64_t n_end = min(n_begin + a.Lb, (blk + 1) * a.L);
  const int tid = threadIdx.x;

  const float *gr = grads + unit * (int64_t)(D * D + D);
  for (int i = tid; i < D * D; i += kBlock) s_G[(i / D) * SP + i % D] = gr[i];
  for (int i = tid; i < D; i += kBlock) s_Gz[i] = gr[D * D + i];
  __syncthreads();

  for (int64_t n0 = n_begin; n0 < n_end; n0 += kTokB) {
    for (int i = tid; i < kTokB * (D / 2); i += kBlock) {
      const int s = i / (D / 2), P = i % (D / 2);
      const int64_t n = n0 + s;
      float k0 = 0.f, k1 = 0.f, r0 = 0.f, r1 = 0.f, v0 = 0.f, v1 = 0.f;
      if (n < n_end) {
        const int64_t base = ((b * a.N + n) * a.H + hd) * D + 2 * P;
        k0 = fmaxf(ld(k, base), 0.f);
        k1 = fmaxf(ld(k, base + 1), 0.f);
        v0 = ld(v, base);
        v1 = ld(v, base + 1);
        int t, h, w;
        grid_pos(n, a.Hs, a.Ws, t, h, w);
        const float2 cs = pair_cs<D>(tab, a, P, t, h, w);
        r0 = k0 * cs.x - k1 * cs.y;
        r1 = k0 * cs.y + k1 * cs.x;
      }
      s_phi[s * D + 2 * P] = k0;
      s_phi[s * D + 2 * P + 1] = k1;
      s_rot[s * D + 2 * P] = r0;
      s_rot[s * D + 2 * P + 1] = r1;
      s_v[s * D + 2 * P] = v0;
      s_v[s * D + 2 * P + 1] = v1;
    }
    __syncthreads();
    // dv = RoPE(phi(k)) G: tokens (2j, 2j+1) x features 4i..4i+3 per item
    for (int it = tid; it < (kTokB / 2) * (D / 4); it += kBlock) {
      const int s0 = 2 * (it / (D / 4)), e0 = 4 * (it % (D / 4));
      float x[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll 4
      for (int p = 0; p < D; ++p) {
        const float4 gv = lds4(s_G + p * SP + e0);
        fma4(x[0], s_rot[s0 * D + p], gv);
        fma4(x[1], s_rot[(s0 + 1) * D + p], gv);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t n = n0 + s0 + u;
        if (n < n_end) {
          const int64_t base = ((b * a.N + n) * a.H + hd) * D + e0;
#pragma unroll
          for (int j = 0; j < 4; ++j) st(dv, base + j, x[u][j]);
        }
      }
    }
    // dk = [RoPE^T(G v) + Gz] * 1[k > 0]: tokens (2j, 2j+1) x pair P per item
    for (int it = tid; it < (kTokB / 2) * (D / 2); it += kBlock) {
      const int s0 = 2 * (it / (D / 2)), P = it % (D / 2);
      float d[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
#pragma unroll 4
      for (int e = 0; e < D; e += 4) {
        const float4 r0 = lds4(s_G + (2 * P) * SP + e), r1 = lds4(s_G + (2 * P + 1) * SP + e);
        const float4 x0 = lds4(s_v + s0 * D + e), x1 = lds4(s_v + (s0 + 1) * D + e);
        d[0][0] = dot4(r0, x0, d[0][0]);
        d[0][1] = dot4(r1, x0, d[0][1]);
        d[1][0] = dot4(r0, x1, d[1][0]);
        d[1][1] = dot4(r1, x1, d[1][1]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int s = s0 + u;
        const int64_t n = n0 + s;
        if (n < n_end) {
          int t, h, w;
          grid_pos(n, a.Hs, a.Ws, t, h, w);
          const float2 cs = pair_cs<D>(tab, a, P, t, h, w);
          const float u0 = d[u][0] * cs.x + d[u][1] * cs.y + s_Gz[2 * P];
          const float u1 = -d[u][0] * cs.y + d[u][1] * cs.x + s_Gz[2 * P + 1];
          const int64_t base = ((b * a.N + n) * a.H + hd) * D + 2 * P;
          st(dk, base, s_phi[s * D + 2 * P] > 0.f ? u0 : 0.f);
          st(dk, base + 1, s_phi[s * D + 2 * P + 1] > 0.f ? u1 : 0.f);
        }
      }
    }
    __syncthreads();
  }
}

BwdArgs make_bargs(const Plan &p) {
  BwdArgs a;
  a.N = p.N; a.H = p.H; a.Hs = p.Hs; a.Ws = p.Ws;
  a.nb = p.nb; a.L = p.L; a.Rb = p.Rb; a.Lb = p.Lb;
  a.tab_h_off = p.tab_h_off; a.tab_w_off = p.tab_w_off;
  a.eps = p.eps;
  return a;
}

template <typename TIn, int D>
hipError_t bwd_d(const Plan &p, const void *q, const void *k, const void *v, const void *g,
                 const void *dout, const float *states, const float2 *tab, float *partials,
                 float *grads, float2 *dd, void *dq, void *dk, void *dv, void *dg,
                 hipStream_t stream) {
  const int64_t stride = kPartialStride(p.d), per_block = (int64_t)kBlock * 4;
  const dim3 rgrid((unsigned)(p.B * p.H), (unsigned)((stride + per_block - 1) / per_block));
  if (p.mfma && (D == 64 || D == 128) && sizeof(TIn) == 2 &&
      bwd_query_lds_bytes(p) <= 160 * 1024 && (p.Lr % 128) == 0) {
    // matrix-core kernels: the token pass over the output stage's ranges
    // (R x Lr), the state pass over the state stage's chunks (C x Lc), the
    // block sums over the chunks, then the key/value side
    hipError_t e = launch_bwd_token_mfma(p, q, g, dout, states, tab, dq, dg, dd, stream);
    if (e != hipSuccess) return e;
    e = launch_bwd_dstate_mfma(p, q, g, dout, dd, tab, partials, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_reduce_kernel, rgrid, dim3(kBlock), 0, stream, partials, grads, p.nb,
                       p.C, (int)p.d);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_bwd_kv_mfma(p, k, v, grads, tab, dk, dv, stream);
  }
  const BwdArgs a = make_bargs(p);
  const dim3 grid((unsigned)(p.units * p.Rb));
  const size_t lds_q = sizeof(float) * (D * kRow<D> + D + 4 * kTokB * D + 2 * kTokB);
  auto kq = bwd_q_kernel<TIn, D>;
  hipError_t e = lds_limit_once((const void *)kq);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kq, grid, dim3(kBlock), lds_q, stream, (const TIn *)q, (const TIn *)g,
                     (const TIn *)dout, states, tab, (TIn *)dq, (TIn *)dg, partials, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_reduce_kernel, rgrid, dim3(kBlock), 0, stream, partials, grads, p.nb,
                     p.Rb, (int)p.d);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds_kv = sizeof(float) * (D * kRow<D> + D + 3 * kTokB * D);
  auto kkv = bwd_kv_kernel<TIn, D>;
  e = lds_limit_once((const void *)kkv);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kkv, grid, dim3(kBlock), lds_kv, stream, (const TIn *)k, (const TIn *)v,
                     grads, tab, (TIn *)dk, (TIn *)dv, a);
  return hipGetLastError();
}

template <typename TIn>
hipError_t bwd_t(const Plan &p, const void *q, const void *k, const void *v, const void *g,
                 const void *dout, const float *states, const float2 *tab, float *partials,
                 float *grads, float2 *dd, void *dq, void *dk, void *dv, void *dg, hipStream_t s) {
#define GLA_BWD_CASE(DD)                                                                        \
  case DD:                                                                                      \
    return bwd_d<TIn, DD>(p, q, k, v, g, dout, states, tab, partials, grads, dd, dq, dk, dv, dg, \
                          s);
  switch (p.d) {
    GLA_BWD_CASE(16)
    GLA_BWD_CASE(32)
    GLA_BWD_CASE(48)
    GLA_BWD_CASE(64)
    GLA_BWD_CASE(80)
    GLA_BWD_CASE(96)
    GLA_BWD_CASE(112)
    GLA_BWD_CASE(128)
  }
#undef GLA_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace

template <typename TIn>
hipError_t backward_vector_limits() {
  return lds_limits({(const void *)bwd_q_kernel<TIn, 16>,  (const void *)bwd_kv_kernel<TIn, 16>,
                     (const void *)bwd_q_kernel<TIn, 32>,  (const void *)bwd_kv_kernel<TIn, 32>,
                     (const void *)bwd_q_kernel<TIn, 48>,  (const void *)bwd_kv_kernel<TIn, 48>,
                     (const void *)bwd_q_kernel<TIn, 64>,  (const void *)bwd_kv_kernel<TIn, 64>,
                     (const void *)bwd_q_kernel<TIn, 80>,  (const void *)bwd_kv_kernel<TIn, 80>,
                     (const void *)bwd_q_kernel<TIn, 96>,  (const void *)bwd_kv_kernel<TIn, 96>,
                     (const void *)bwd_q_kernel<TIn, 112>, (const void *)bwd_kv_kernel<TIn, 112>,
                     (const void *)bwd_q_kernel<TIn, 128>, (const void *)bwd_kv_kernel<TIn, 128>});
}

hipError_t backward_vector_lds_limits() {
  const hipError_t e = backward_vector_limits<uint16_t>();
  return e != hipSuccess ? e : backward_vector_limits<float>();
}

hipError_t launch_backward(const Plan &p, const void *q, const void *k, const void *v,
                           const void *g, const void *dout, const float *states,
                           const float2 *tab, float *partials, float *grads, float2 *dd,
                           void *dq, void *dk, void *dv, void *dg, hipStream_t stream) {
  return p.bf16 ? bwd_t<uint16_t>(p, q, k, v, g, dout, states, tab, partials, grads, dd, dq, dk,
                                  dv, dg, stream)
                : bwd_t<float>(p, q, k, v, g, dout, states, tab, partials, grads, dd, dq, dk, dv,
                               dg, stream);
}

}  // namespace gla
