// Vector (VALU) kernels of the operator for every supported head size and
// for fp32 tensors: the state partials and the output stage.  All arithmetic
// is fp32.  Used for fp32 tensors and for bf16 head sizes other than 64/128.
//
// "SANA-Video" notes page, Section 3.2 (pseudocode steps 1-5): phi = ReLU,
// RoPE after ReLU on q and k for the numerator only, state
// sum_j RoPE(phi(k_j))^T v_j, denominator phi(q_i) . sum_j phi(k_j);
// "SANA-Video 2.0" Section 2 Eq. (1): + eps and the sigmoid output gate.

#include <hip/hip_runtime.h>

#include "gla_internal.h"

namespace gla {
namespace {

struct VecArgs {
  int64_t N, H, T, Hs, Ws;
  int64_t nb, L, C, Lc, R, Lr;
  int64_t tab_h_off, tab_w_off;  // entry offsets of the h and w tables (t starts at 0)
  float eps;
  float rms_eps;
};

template <typename TIn>
__device__ __forceinline__ float load_elem(const TIn *p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float *p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t *p, int64_t i) {
  return bf16_bits_to_float(p[i]);
}

template <typename TIn>
__device__ __forceinline__ void store_elem(TIn *p, int64_t i, float x);
template <>
__device__ __forceinline__ void store_elem<float>(float *p, int64_t i, float x) {
  p[i] = x;
}
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t *p, int64_t i, float x) {
  __bf16 h = (__bf16)x;  // round to nearest even
  p[i] = __builtin_bit_cast(uint16_t, h);
}

// (cos, sin) of feature pair P (0 <= P < D/2) of a token at (t, h, w).
template <int D>
__device__ __forceinline__ float2 rope_cs(const float2 *__restrict__ tab, const VecArgs &a, int P,
                                          int t, int h, int w) {
  constexpr int pt = D / 8, ph = 3 * D / 16;
  if (P < pt) return tab[(int64_t)t * pt + P];
  if (P < pt + ph) return tab[a.tab_h_off + (int64_t)h * ph + (P - pt)];
  return tab[a.tab_w_off + (int64_t)w * ph + (P - pt - ph)];
}

constexpr int kTok = 16;  // tokens staged in LDS per step

// One workgroup per (unit, chunk): S_c = sum RoPE(phi(k))^T v and
// z_c = sum phi(k) over the chunk's tokens, written row-major to the partial
// slot unit*C + c.  Thread t owns the (D/16)^2 state entries t + 256*m.
// beta (optional): the write gate, scaling a token's rotated key in S only.
template <typename TIn, int D>
__global__ __launch_bounds__(kBlock) void state_vector_kernel(const TIn *__restrict__ k,
                                                              const TIn *__restrict__ v,
                                                              const TIn *__restrict__ beta,
                                                              const float2 *__restrict__ tab,
                                                              float *__restrict__ partials,
                                                              VecArgs a) {
  constexpr int kPer = (D / 16) * (D / 16);
  __shared__ float s_phi[kTok][D];
  __shared__ float s_rot[kTok][D];
  __shared__ float s_v[kTok][D];

  const int64_t wg = blockIdx.x;
  const int64_t unit = wg / a.C, c = wg % a.C;
  const int64_t bh = unit / a.nb, blk = unit % a.nb;
  const int64_t b = bh / a.H, hd = bh % a.H;
  const int64_t n_begin = blk * a.L + c * a.Lc;
  const int64_t n_end = min(n_begin + a.Lc, (blk + 1) * a.L);
  const int tid = threadIdx.x;

  float acc[kPer];
#pragma unroll
  for (int m = 0; m < kPer; ++m) acc[m] = 0.f;
  float zacc = 0.f;

  for (int64_t n0 = n_begin; n0 < n_end; n0 += kTok) {
    for (int i = tid; i < kTok * (D / 2); i += kBlock) {
      const int s = i / (D / 2), P = i % (D / 2);
      const int64_t n = n0 + s;
      float k0 = 0.f, k1 = 0.f, v0 = 0.f, v1 = 0.f, r0 = 0.f, r1 = 0.f;
      if (n < n_end) {
        const int64_t base = ((b * a.N + n) * a.H + hd) * D + 2 * P;
        k0 = fmaxf(load_elem(k, base), 0.f);
        k1 = fmaxf(load_elem(k, base + 1), 0.f);
        v0 = load_elem(v, base);
        v1 = load_elem(v, base + 1);
        int t, h, w;
        grid_pos(n, a.Hs, a.Ws, t, h, w);
        const float2 cs = rope_cs<D>(tab, a, P, t, h, w);
        r0 = k0 * cs.x - k1 * cs.y;
        r1 = k0 * cs.y + k1 * cs.x;
        if (beta != nullptr) {
          const float bt = load_elem(beta, (b * a.N + n) * a.H + hd);
          r0 *= bt;
          r1 *= bt;
        }
      }
      s_phi[s][2 * P] = k0;
      s_phi[s][2 * P + 1] = k1;
      s_rot[s][2 * P] = r0;
      s_rot[s][2 * P + 1] = r1;
      s_v[s][2 * P] = v0;
      s_v[s][2 * P + 1] = v1;
    }
    __syncthreads();
    if (tid < D) {
#pragma unroll
      for (int s = 0; s < kTok; ++s) zacc += s_phi[s][tid];
    }
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int idx = tid + kBlock * m;
      const int p = idx / D, e = idx % D;
      float x = acc[m];
#pragma unroll
      for (int s = 0; s < kTok; ++s) x += s_rot[s][p] * s_v[s][e];
      acc[m] = x;
    }
    __syncthreads();
  }
  float *dst = partials + wg * (int64_t)(D * D + D);
#pragma unroll
  for (int m = 0; m < kPer; ++m) dst[tid + kBlock * m] = acc[m];
  if (tid < D) dst[D * D + tid] = zacc;
}

// One workgroup per (unit, token range): out = num / den * sigmoid(g) with
// num = RoPE(phi(q)) S and den = phi(q) . z + eps, S and z of the unit read
// from the reduced fp32 states.  S sits in dynamic LDS (64 KiB at D = 128).
// rms_w (optional): y = num / den passes an RMSNorm over its D features
// with weight rms_w before the gate.
template <typename TIn, int D>
__global__ __launch_bounds__(kBlock) void apply_vector_kernel(const TIn *__restrict__ q,
                                                              const TIn *__restrict__ g,
                                                              const float *__restrict__ states,
                                                              const float2 *__restrict__ tab,
                                                              const TIn *__restrict__ rms_w,
                                                              TIn *__restrict__ out, VecArgs a) {
  extern __shared__ float lds[];
  float *s_S = lds;                   // D*D
  float *s_z = s_S + D * D;           // D
  float *s_phi = s_z + D;             // kTok*D (y = num / den when normalising)
  float *s_rot = s_phi + kTok * D;    // kTok*D
  float *s_den = s_rot + kTok * D;    // kTok (1 / rms when normalising)

  const int64_t wg = blockIdx.x;
  const int64_t unit = wg / a.R, r = wg % a.R;
  const int64_t bh = unit / a.nb, blk = unit % a.nb;
  const int64_t b = bh / a.H, hd = bh % a.H;
  const int64_t n_begin = blk * a.L + r * a.Lr;
  const int64_t n_end = min(n_begin + a.Lr, (blk + 1) * a.L);
  const int tid = threadIdx.x;

  const float *st = states + unit * (int64_t)(D * D + D);
  for (int i = tid; i < D * D + D; i += kBlock) lds[i] = st[i];
  __syncthreads();

  for (int64_t n0 = n_begin; n0 < n_end; n0 += kTok) {
    for (int i = tid; i < kTok * (D / 2); i += kBlock) {
      const int s = i / (D / 2), P = i % (D / 2);
      const int64_t n = n0 + s;
      float q0 = 0.f, q1 = 0.f, r0 = 0.f, r1 = 0.f;
      if (n < n_end) {
        const int64_t base = ((b * a.N + n) * a.H + hd) * D + 2 * P;
        q0 = fmaxf(load_elem(q, base), 0.f);
        q1 = fmaxf(load_elem(q, base + 1), 0.f);
        int t, h, w;
        grid_pos(n, a.Hs, a.Ws, t, h, w);
        const float2 cs = rope_cs<D>(tab, a, P, t, h, w);
        r0 = q0 * cs.x - q1 * cs.y;
        r1 = q0 * cs.y + q1 * cs.x;
      }
      s_phi[s * D + 2 * P] = q0;
      s_phi[s * D + 2 * P + 1] = q1;
      s_rot[s * D + 2 * P] = r0;
      s_rot[s * D + 2 * P + 1] = r1;
    }
    __syncthreads();
    if (tid < kTok) {
      float den = 0.f;
      for (int p = 0; p < D; ++p) den += s_phi[tid * D + p] * s_z[p];
      s_den[tid] = den + a.eps;
    }
    __syncthreads();
    if (rms_w == nullptr) {
      for (int o = tid; o < kTok * D; o += kBlock) {
        const int s = o / D, e = o % D;
        const int64_t n = n0 + s;
        if (n < n_end) {
          float num = 0.f;
#pragma unroll 8
          for (int p = 0; p < D; ++p) num += s_rot[s * D + p] * s_S[p * D + e];
          const int64_t idx = ((b * a.N + n) * a.H + hd) * D + e;
          const float gate = 1.f / (1.f + expf(-load_elem(g, idx)));
          store_elem(out, idx, num / s_den[s] * gate);
        }
      }
    } else {
      // y = num / den into s_phi (phi(q) is no longer needed), 1 / rms into
      // s_den, then the normalised and gated output
      for (int o = tid; o < kTok * D; o += kBlock) {
        const int s = o / D, e = o % D;
        float num = 0.f;
#pragma unroll 8
        for (int p = 0; p < D; ++p) num += s_rot[s * D + p] * s_S[p * D + e];
        s_phi[s * D + e] = num;  // (every thread has read s_phi before the last barrier)
      }
      __syncthreads();
      if (tid < kTok) {
        const float inv_den = 1.f / s_den[tid];
        float ss = 0.f;
        for (int e = 0; e < D; ++e) {
          const float y = s_phi[tid * D + e] * inv_den;
          s_phi[tid * D + e] = y;
          ss += y * y;
        }
        s_den[tid] = 1.f / sqrtf(ss / D + a.rms_eps);
      }
      __syncthreads();
      for (int o = tid; o < kTok * D; o += kBlock) {
        const int s = o / D, e = o % D;
        const int64_t n = n0 + s;
        if (n < n_end) {
          const int64_t idx = ((b * a.N + n) * a.H + hd) * D + e;
          const float gate = 1.f / (1.f + expf(-load_elem(g, idx)));
          store_elem(out, idx, s_phi[s * D + e] * s_den[s] * load_elem(rms_w, e) * gate);
        }
      }
    }
    __syncthreads();
  }
}

VecArgs make_args(const Plan &p) {
  VecArgs a;
  a.N = p.N; a.H = p.H; a.T = p.T; a.Hs = p.Hs; a.Ws = p.Ws;
  a.nb = p.nb; a.L = p.L; a.C = p.C; a.Lc = p.Lc; a.R = p.R; a.Lr = p.Lr;
  a.tab_h_off = p.tab_h_off; a.tab_w_off = p.tab_w_off;
  a.eps = p.eps;
  a.rms_eps = p.rms_eps;
  return a;
}

template <typename TIn, int D>
hipError_t state_d(const Plan &p, const void *k, const void *v, const void *beta,
                   const float2 *tab, float *part, hipStream_t stream) {
  hipLaunchKernelGGL((state_vector_kernel<TIn, D>), dim3((unsigned)(p.units * p.C)), dim3(kBlock),
                     0, stream, (const TIn *)k, (const TIn *)v, (const TIn *)beta, tab, part,
                     make_args(p));
  return hipGetLastError();
}

template <typename TIn, int D>
hipError_t apply_d(const Plan &p, const void *q, const void *g, const float *states,
                   const float2 *tab, const void *rms_w, void *out, hipStream_t stream) {
  const size_t lds = sizeof(float) * (D * D + D + 2 * kTok * D + kTok);
  auto kern = apply_vector_kernel<TIn, D>;
  hipError_t e = lds_limit_once((const void *)kern);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.units * p.R)), dim3(kBlock), lds, stream,
                     (const TIn *)q, (const TIn *)g, states, tab, (const TIn *)rms_w, (TIn *)out,
                     make_args(p));
  return hipGetLastError();
}

template <typename TIn>
hipError_t state_t(const Plan &p, const void *k, const void *v, const void *beta,
                   const float2 *tab, float *part, hipStream_t s) {
  switch (p.d) {
    case 16: return state_d<TIn, 16>(p, k, v, beta, tab, part, s);
    case 32: return state_d<TIn, 32>(p, k, v, beta, tab, part, s);
    case 48: return state_d<TIn, 48>(p, k, v, beta, tab, part, s);
    case 64: return state_d<TIn, 64>(p, k, v, beta, tab, part, s);
    case 80: return state_d<TIn, 80>(p, k, v, beta, tab, part, s);
    case 96: return state_d<TIn, 96>(p, k, v, beta, tab, part, s);
    case 112: return state_d<TIn, 112>(p, k, v, beta, tab, part, s);
    case 128: return state_d<TIn, 128>(p, k, v, beta, tab, part, s);
  }
  return hipErrorInvalidValue;
}

template <typename TIn>
hipError_t apply_t(const Plan &p, const void *q, const void *g, const float *st,
                   const float2 *tab, const void *w, void *out, hipStream_t s) {
  switch (p.d) {
    case 16: return apply_d<TIn, 16>(p, q, g, st, tab, w, out, s);
    case 32: return apply_d<TIn, 32>(p, q, g, st, tab, w, out, s);
    case 48: return apply_d<TIn, 48>(p, q, g, st, tab, w, out, s);
    case 64: return apply_d<TIn, 64>(p, q, g, st, tab, w, out, s);
    case 80: return apply_d<TIn, 80>(p, q, g, st, tab, w, out, s);
    case 96: return apply_d<TIn, 96>(p, q, g, st, tab, w, out, s);
    case 112: return apply_d<TIn, 112>(p, q, g, st, tab, w, out, s);
    case 128: return apply_d<TIn, 128>(p, q, g, st, tab, w, out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

template <typename TIn>
hipError_t apply_vector_limits() {
  return lds_limits({(const void *)apply_vector_kernel<TIn, 16>,
                     (const void *)apply_vector_kernel<TIn, 32>,
                     (const void *)apply_vector_kernel<TIn, 48>,
                     (const void *)apply_vector_kernel<TIn, 64>,
                     (const void *)apply_vector_kernel<TIn, 80>,
                     (const void *)apply_vector_kernel<TIn, 96>,
                     (const void *)apply_vector_kernel<TIn, 112>,
                     (const void *)apply_vector_kernel<TIn, 128>});
}

hipError_t vector_lds_limits() {
  const hipError_t e = apply_vector_limits<uint16_t>();
  return e != hipSuccess ? e : apply_vector_limits<float>();
}

hipError_t launch_state_generic(const Plan &p, const void *k, const void *v, const void *beta,
                                const float2 *tab, float *partials, hipStream_t stream) {
  return p.bf16 ? state_t<uint16_t>(p, k, v, beta, tab, partials, stream)
                : state_t<float>(p, k, v, beta, tab, partials, stream);
}

hipError_t launch_apply_generic(const Plan &p, const void *q, const void *g, const float *states,
                                const float2 *tab, const void *rms_w, void *out,
                                hipStream_t stream) {
  return p.bf16 ? apply_t<uint16_t>(p, q, g, states, tab, rms_w, out, stream)
                : apply_t<float>(p, q, g, states, tab, rms_w, out, stream);
}

}  // namespace gla
