// Token-causal form of the operator ("SANA-Video" notes page, Section 3.4:
// the causal linear-attention output of token i, derived there for the
// constant-memory cache): token i attends to tokens 0..i of its (batch,
// head) through the running sums
//
//   S_i = sum_{j<=i} RoPE_j(phi(k_j))^T v_j,   z_i = sum_{j<=i} phi(k_j)
//   o_i = RoPE_i(phi(q_i)) S_i / (phi(q_i) . z_i + eps) * sigmoid(g_i)
//
// Chunkwise evaluation: the state stage writes one partial (S_c, z_c) per
// chunk of Lc tokens; range_prefix_kernel turns them into the exclusive
// prefix at the start of every range of Lr = m * Lc tokens; one workgroup per
// range then walks its range tile by tile.  For a tile of tokens T with the
// sums S, z of everything before it,
//
//   num_i = RoPE(phi(q_i)) S + sum_{j in T, j<=i} (RoPE(phi(q_i)) . RoPE(phi(k_j))) v_j
//   den_i = phi(q_i) . z + sum_{j in T, j<=i} phi(q_i) . phi(k_j) + eps
//
// and then S, z take the tile's keys.  This file holds the prefix kernel and
// the vector (fp32 VALU) tile kernel used for fp32 tensors, head sizes other
// than 64 and 128, and unaligned tensors.

#include <hip/hip_runtime.h>

#include "gla_internal.h"

namespace gla {
namespace {

// Exclusive prefix of the chunk partials at range starts: for every unit u
// and range r, states[u][r] = sum over chunks c < r*m of partials[u][c], in
// chunk order (bitwise deterministic).  One thread owns four consecutive
// floats of the d*d + d vector.
__global__ __launch_bounds__(kBlock) void range_prefix_kernel(const float *__restrict__ partials,
                                                              float *__restrict__ states,
                                                              int64_t C, int64_t R, int64_t m,
                                                              int d) {
  const int64_t stride = (int64_t)d * d + d;
  const int64_t unit = blockIdx.x;
  const int64_t i4 = ((int64_t)blockIdx.y * blockDim.x + threadIdx.x) * 4;
  if (i4 >= stride) return;
  const float *src = partials + unit * C * stride + i4;
  float *dst = states + unit * R * stride + i4;
  float4 run = make_float4(0.f, 0.f, 0.f, 0.f);
  int64_t c = 0;
  for (int64_t r = 0; r < R; ++r) {
    *reinterpret_cast<float4 *>(dst + r * stride) = run;
    const int64_t c_end = min((r + 1) * m, C);
    add_partials(run, src, stride, c, c_end);
    c = max(c, c_end);
  }
}

struct CArgs {
  int64_t N, H, Hs, Ws;
  int64_t R, Lr;
  int64_t tab_h_off, tab_w_off;
  float eps;
};

template <typename TIn>
__device__ __forceinline__ float ldx(const TIn *p, int64_t i);
template <>
__device__ __forceinline__ float ldx<float>(const float *p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float ldx<uint16_t>(const uint16_t *p, int64_t i) {
  return bf16_bits_to_float(p[i]);
}
template <typename TIn>
__device__ __forceinline__ void stx(TIn *p, int64_t i, float x);
template <>
__device__ __forceinline__ void stx<float>(float *p, int64_t i, float x) {
  p[i] = x;
}
template <>
__device__ __forceinline__ void stx<uint16_t>(uint16_t *p, int64_t i, float x) {
  __bf16 h = (__bf16)x;  // round to nearest even
  p[i] = __builtin_bit_cast(uint16_t, h);
}

// (cos, sin) of feature pair P of a token at (t, h, w) from the table (t
// rows, then h rows, then w rows).
template <int D>
__device__ __forceinline__ float2 cs_of(const float2 *__restrict__ tab, const CArgs &a, int P,
                                        int t, int h, int w) {
  constexpr int pt = D / 8, ph = 3 * D / 16;
  if (P < pt) return tab[(int64_t)t * pt + P];
  if (P < pt + ph) return tab[a.tab_h_off + (int64_t)h * ph + (P - pt)];
  return tab[a.tab_w_off + (int64_t)w * ph + (P - pt - ph)];
}

__device__ __forceinline__ float4 lds4f(const float *p) {
  return *reinterpret_cast<const float4 *>(p);
}
__device__ __forceinline__ float dot4f(const float4 a, const float4 b, float acc) {
  acc = __builtin_fmaf(a.x, b.x, acc);
  acc = __builtin_fmaf(a.y, b.y, acc);
  acc = __builtin_fmaf(a.z, b.z, acc);
  return __builtin_fmaf(a.w, b.w, acc);
}

constexpr int kCTok = 16;  // tokens per tile of the vector kernel

// LDS row stride (floats) of S and of the token tiles: four floats of
// padding keep rows 16-byte aligned and put the rows that neighbouring
// threads read into different banks.
template <int D>
constexpr int kCRow = D + 4;

// One workgroup (256 threads) per (unit, range).  S sits in LDS for the
// numerator reads and, split into (D/16) x (D/16) blocks, in the registers
// of its owner thread, which adds each tile's keys to its block and writes
// it back.  Per tile of 16 tokens:
//   1. phi and RoPE of q and k, and v, into LDS;
//   2. the 16 x 16 intra-tile products (one (i, j) pair per thread);
//   3. den per token;
//   4. num, the gate and the store (two tokens x four features per item);
//   5. S and z take the tile's keys.
template <typename TIn, int D>
__global__ __launch_bounds__(kBlock) void causal_vector_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const TIn *__restrict__ g, const float *__restrict__ states, const float2 *__restrict__ tab,
    TIn *__restrict__ out, CArgs a) {
  constexpr int BK = D / 16;
  constexpr int SP = kCRow<D>;
  constexpr int AP = kCTok + 1;
  extern __shared__ float lds[];
  float *s_S = lds;                  // D rows of SP
  float *s_z = s_S + D * SP;         // D
  float *s_pq = s_z + D;             // kCTok rows of SP: phi(q)
  float *s_rq = s_pq + kCTok * SP;   // RoPE(phi(q))
  float *s_pk = s_rq + kCTok * SP;   // phi(k)
  float *s_rk = s_pk + kCTok * SP;   // RoPE(phi(k))
  float *s_v = s_rk + kCTok * SP;    // v
  float *s_A = s_v + kCTok * SP;     // kCTok x AP: RoPE(phi(q_i)) . RoPE(phi(k_j)), j <= i
  float *s_D = s_A + kCTok * AP;     // kCTok x AP: phi(q_i) . phi(k_j), j <= i
  float *s_den = s_D + kCTok * AP;   // kCTok

  const int64_t wg = blockIdx.x;
  const int64_t unit = wg / a.R, r = wg % a.R;
  const int64_t b = unit / a.H, hd = unit % a.H;
  const int64_t n_begin = r * a.Lr;
  const int64_t n_end = min(n_begin + a.Lr, a.N);
  const int tid = threadIdx.x;

  // the sums of every token before the range
  const float *stt = states + wg * (int64_t)(D * D + D);
  const int pb = tid / 16, eb = tid % 16;  // this thread's block of S
  float acc[BK * BK];
#pragma unroll
  for (int i = 0; i < BK; ++i)
#pragma unroll
    for (int j = 0; j < BK; ++j) {
      const float x = stt[(pb * BK + i) * D + eb * BK + j];
      acc[i * BK + j] = x;
      s_S[(pb * BK + i) * SP + eb * BK + j] = x;
    }
  for (int i = tid; i < D; i += kBlock) s_z[i] = stt[D * D + i];
  __syncthreads();

  for (int64_t n0 = n_begin; n0 < n_end; n0 += kCTok) {
    // 1. phi and RoPE of q and k, and v (zeros past the range)
    for (int i = tid; i < kCTok * (D / 2); i += kBlock) {
      const int s = i / (D / 2), P = i % (D / 2);
      const int64_t n = n0 + s;
      float q0 = 0.f, q1 = 0.f, k0 = 0.f, k1 = 0.f, v0 = 0.f, v1 = 0.f;
      float2 cs = make_float2(1.f, 0.f);
      if (n < n_end) {
        const int64_t base = ((b * a.N + n) * a.H + hd) * D + 2 * P;
        q0 = fmaxf(ldx(q, base), 0.f);
        q1 = fmaxf(ldx(q, base + 1), 0.f);
        k0 = fmaxf(ldx(k, base), 0.f);
        k1 = fmaxf(ldx(k, base + 1), 0.f);
        v0 = ldx(v, base);
        v1 = ldx(v, base + 1);
        int t, h, w;
        grid_pos(n, a.Hs, a.Ws, t, h, w);
        cs = cs_of<D>(tab, a, P, t, h, w);
      }
      const int o = s * SP + 2 * P;
      s_pq[o] = q0;
      s_pq[o + 1] = q1;
      s_rq[o] = q0 * cs.x - q1 * cs.y;
      s_rq[o + 1] = q0 * cs.y + q1 * cs.x;
      s_pk[o] = k0;
      s_pk[o + 1] = k1;
      s_rk[o] = k0 * cs.x - k1 * cs.y;
      s_rk[o + 1] = k0 * cs.y + k1 * cs.x;
      s_v[o] = v0;
      s_v[o + 1] = v1;
    }
    __syncthreads();
    // 2. intra-tile products, one (i, j) pair per thread (j <= i)
    {
      const int i = tid / kCTok, j = tid % kCTok;
      float av = 0.f, dv = 0.f;
      if (j <= i) {
#pragma unroll 4
        for (int p = 0; p < D; p += 4) {
          av = dot4f(lds4f(s_rq + i * SP + p), lds4f(s_rk + j * SP + p), av);
          dv = dot4f(lds4f(s_pq + i * SP + p), lds4f(s_pk + j * SP + p), dv);
        }
      }
      s_A[i * AP + j] = av;
      s_D[i * AP + j] = dv;
    }
    __syncthreads();
    // 3. den per token
    if (tid < kCTok) {
      float den = 0.f;
      for (int p = 0; p < D; ++p) den = __builtin_fmaf(s_pq[tid * SP + p], s_z[p], den);
      for (int j = 0; j <= tid; ++j) den += s_D[tid * AP + j];
      s_den[tid] = den + a.eps;
    }
    __syncthreads();
    // 4. num, gate and store: tokens (2u, 2u+1) x features 4i..4i+3 per item
    for (int it = tid; it < (kCTok / 2) * (D / 4); it += kBlock) {
      const int s0 = 2 * (it / (D / 4)), e0 = 4 * (it % (D / 4));
      float num[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll 4
      for (int p = 0; p < D; ++p) {
        const float4 sv = lds4f(s_S + p * SP + e0);
        const float x0 = s_rq[s0 * SP + p], x1 = s_rq[(s0 + 1) * SP + p];
        num[0][0] = __builtin_fmaf(x0, sv.x, num[0][0]);
        num[0][1] = __builtin_fmaf(x0, sv.y, num[0][1]);
        num[0][2] = __builtin_fmaf(x0, sv.z, num[0][2]);
        num[0][3] = __builtin_fmaf(x0, sv.w, num[0][3]);
        num[1][0] = __builtin_fmaf(x1, sv.x, num[1][0]);
        num[1][1] = __builtin_fmaf(x1, sv.y, num[1][1]);
        num[1][2] = __builtin_fmaf(x1, sv.z, num[1][2]);
        num[1][3] = __builtin_fmaf(x1, sv.w, num[1][3]);
      }
      for (int j = 0; j <= s0 + 1; ++j) {
        const float4 vv = lds4f(s_v + j * SP + e0);
        const float a0 = s_A[s0 * AP + j], a1 = s_A[(s0 + 1) * AP + j];  // 0 where j > i
        num[0][0] = __builtin_fmaf(a0, vv.x, num[0][0]);
        num[0][1] = __builtin_fmaf(a0, vv.y, num[0][1]);
        num[0][2] = __builtin_fmaf(a0, vv.z, num[0][2]);
        num[0][3] = __builtin_fmaf(a0, vv.w, num[0][3]);
        num[1][0] = __builtin_fmaf(a1, vv.x, num[1][0]);
        num[1][1] = __builtin_fmaf(a1, vv.y, num[1][1]);
        num[1][2] = __builtin_fmaf(a1, vv.z, num[1][2]);
        num[1][3] = __builtin_fmaf(a1, vv.w, num[1][3]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t n = n0 + s0 + u;
        if (n < n_end) {
          const float den = s_den[s0 + u];
          const int64_t base = ((b * a.N + n) * a.H + hd) * D + e0;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            stx(out, base + j, num[u][j] / den / (1.f + expf(-ldx(g, base + j))));
        }
      }
    }
    __syncthreads();
    // 5. S and z take the tile's keys (rows past the range are zeros)
#pragma unroll 2
    for (int s = 0; s < kCTok; ++s) {
      float rv[BK], vv[BK];
#pragma unroll
      for (int i = 0; i < BK; ++i) rv[i] = s_rk[s * SP + pb * BK + i];
#pragma unroll
      for (int j = 0; j < BK; ++j) vv[j] = s_v[s * SP + eb * BK + j];
#pragma unroll
      for (int i = 0; i < BK; ++i)
#pragma unroll
        for (int j = 0; j < BK; ++j) acc[i * BK + j] = __builtin_fmaf(rv[i], vv[j], acc[i * BK + j]);
    }
#pragma unroll
    for (int i = 0; i < BK; ++i)
#pragma unroll
      for (int j = 0; j < BK; ++j) s_S[(pb * BK + i) * SP + eb * BK + j] = acc[i * BK + j];
    if (tid < D) {
      float zs = s_z[tid];
#pragma unroll
      for (int s = 0; s < kCTok; ++s) zs += s_pk[s * SP + tid];
      s_z[tid] = zs;
    }
    __syncthreads();
  }
}

CArgs make_cargs(const Plan &p) {
  CArgs a;
  a.N = p.N; a.H = p.H; a.Hs = p.Hs; a.Ws = p.Ws;
  a.R = p.R; a.Lr = p.Lr;
  a.tab_h_off = p.tab_h_off; a.tab_w_off = p.tab_w_off;
  a.eps = p.eps;
  return a;
}

template <typename TIn, int D>
hipError_t causal_vec_d(const Plan &p, const void *q, const void *k, const void *v, const void *g,
                        const float *states, const float2 *tab, void *out, hipStream_t stream) {
  constexpr int SP = kCRow<D>;
  const size_t lds =
      sizeof(float) * (D * SP + D + 5 * kCTok * SP + 2 * kCTok * (kCTok + 1) + kCTok);
  auto kern = causal_vector_kernel<TIn, D>;
  hipError_t e = lds_limit_once((const void *)kern);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.units * p.R)), dim3(kBlock), lds, stream,
                     (const TIn *)q, (const TIn *)k, (const TIn *)v, (const TIn *)g, states, tab,
                     (TIn *)out, make_cargs(p));
  return hipGetLastError();
}

template <typename TIn>
hipError_t causal_vec_t(const Plan &p, const void *q, const void *k, const void *v, const void *g,
                        const float *states, const float2 *tab, void *out, hipStream_t s) {
#define GLA_CAUSAL_CASE(DD) \
  case DD:                  \
    return causal_vec_d<TIn, DD>(p, q, k, v, g, states, tab, out, s);
  switch (p.d) {
    GLA_CAUSAL_CASE(16)
    GLA_CAUSAL_CASE(32)
    GLA_CAUSAL_CASE(48)
    GLA_CAUSAL_CASE(64)
    GLA_CAUSAL_CASE(80)
    GLA_CAUSAL_CASE(96)
    GLA_CAUSAL_CASE(112)
    GLA_CAUSAL_CASE(128)
  }
#undef GLA_CAUSAL_CASE
  return hipErrorInvalidValue;
}

}  // namespace

template <typename TIn>
hipError_t causal_vector_limits() {
  return lds_limits({(const void *)causal_vector_kernel<TIn, 16>,
                     (const void *)causal_vector_kernel<TIn, 32>,
                     (const void *)causal_vector_kernel<TIn, 48>,
                     (const void *)causal_vector_kernel<TIn, 64>,
                     (const void *)causal_vector_kernel<TIn, 80>,
                     (const void *)causal_vector_kernel<TIn, 96>,
                     (const void *)causal_vector_kernel<TIn, 112>,
                     (const void *)causal_vector_kernel<TIn, 128>});
}

hipError_t causal_vector_lds_limits() {
  const hipError_t e = causal_vector_limits<uint16_t>();
  return e != hipSuccess ? e : causal_vector_limits<float>();
}

hipError_t launch_range_prefix(const Plan &p, const float *partials, float *states,
                               hipStream_t stream) {
  const int64_t stride = kPartialStride(p.d);
  const int64_t per_block = (int64_t)kBlock * 4;
  const int64_t m = p.Lr / p.Lc;
  dim3 grid((unsigned)p.units, (unsigned)((stride + per_block - 1) / per_block));
  hipLaunchKernelGGL(range_prefix_kernel, grid, dim3(kBlock), 0, stream, partials, states, p.C,
                     p.R, m, (int)p.d);
  return hipGetLastError();
}

hipError_t launch_causal_generic(const Plan &p, const void *q, const void *k, const void *v,
                                 const void *g, const float *states, const float2 *tab, void *out,
                                 hipStream_t stream) {
  return p.bf16 ? causal_vec_t<uint16_t>(p, q, k, v, g, states, tab, out, stream)
                : causal_vec_t<float>(p, q, k, v, g, states, tab, out, stream);
}

}  // namespace gla
