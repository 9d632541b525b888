// Kernels shared by both paths: the RoPE table and the fixed-order reduce /
// block prefix of the state partials.
//
// "SANA-Video" notes page, Section 3.2: RoPE rotates phi(q) and phi(k) in the
// numerator; Section 3.4: a block reads the running sums of the states and
// normalisers of all earlier blocks plus its own.

#include <hip/hip_runtime.h>

#include "gla_internal.h"

namespace gla {
namespace {

// One (cos, sin) entry per (axis, position, pair).  The angle
// pos * theta^(-2i/d_axis) and its cosine and sine are evaluated in fp64 and
// rounded once to fp32, so large positions (t up to several hundred) keep
// full fp32 accuracy.  theta <= 0 gives the identity rotation (1, 0).
__global__ __launch_bounds__(kBlock) void rope_table_kernel(float2 *__restrict__ tab, int64_t T,
                                                            int64_t Hs, int64_t Ws, int d,
                                                            double theta, int64_t t0) {
  const int64_t pt = d / 8, ph = 3 * d / 16, pw = 3 * d / 16;
  const int64_t nt = T * pt, nh = Hs * ph, nw = Ws * pw;
  const int64_t total = nt + nh + nw;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t pos, pair, width;
    if (i < nt) {
      pos = t0 + i / pt; pair = i % pt; width = d / 4;  // frames sit at t0, t0 + 1, ...
    } else if (i < nt + nh) {
      pos = (i - nt) / ph; pair = (i - nt) % ph; width = 3 * d / 8;
    } else {
      pos = (i - nt - nh) / pw; pair = (i - nt - nh) % pw; width = 3 * d / 8;
    }
    float2 cs = make_float2(1.f, 0.f);
    if (theta > 0.0) {
      double freq = pow(theta, -2.0 * (double)pair / (double)width);
      double angle = (double)pos * freq;
      cs = make_float2((float)cos(angle), (float)sin(angle));
    }
    tab[i] = cs;
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// Sum of the C chunk partials of every unit, in chunk order, followed by the
// inclusive prefix over the nb temporal blocks of a (batch, head), in block
// order.  One thread owns four consecutive floats of the d*d + d state
// vector; no two threads touch the same output, so the result is the same on
// every run.
//
// frags (optional): S in two bf16 parts, S ~ hi + lo (hi = S rounded to
// bf16, lo = the remainder rounded to bf16), each row-major [p][e]; the d*d
// lo values follow the d*d hi values of a unit.
// S_in/z_in (optional): the sums carried in from earlier blocks, where the
// running sums start; S_out/z_out (optional): the final running sums.  Each
// thread reads its four values of S_in/z_in before it writes the same four
// of S_out/z_out, so the two may be the same arrays (an in-place update).
__device__ __forceinline__ float *cache_ptr(float *S, float *z, int64_t bh, int64_t i4, int d) {
  const int64_t dd = (int64_t)d * d;
  return i4 < dd ? S + bh * dd + i4 : z + bh * d + (i4 - dd);
}

__global__ __launch_bounds__(kBlock) void reduce_prefix_kernel(
    const float *__restrict__ partials, float *__restrict__ states, uint16_t *__restrict__ frags,
    const float *S_in, const float *z_in, float *S_out, float *z_out, int64_t nb, int64_t C,
    int d) {
  const int64_t stride = (int64_t)d * d + d;
  const int64_t bh = blockIdx.x;
  const int64_t i4 = ((int64_t)blockIdx.y * blockDim.x + threadIdx.x) * 4;
  if (i4 >= stride) return;
  float4 run = make_float4(0.f, 0.f, 0.f, 0.f);
  if (S_in != nullptr) {
    // four consecutive values of one row (d % 4 == 0, so they never straddle S and z)
    const float *c = cache_ptr(const_cast<float *>(S_in), const_cast<float *>(z_in), bh, i4, d);
    run = make_float4(c[0], c[1], c[2], c[3]);
  }
  for (int64_t blk = 0; blk < nb; ++blk) {
    const int64_t unit = bh * nb + blk;
    add_partials(run, partials + unit * C * stride + i4, stride, 0, C);
    *reinterpret_cast<float4 *>(states + unit * stride + i4) = run;
    if (frags != nullptr && i4 < (int64_t)d * d) {
      const float vals[4] = {run.x, run.y, run.z, run.w};
      uint16_t hi[4], lo[4];
      for (int r = 0; r < 4; ++r) {
        const __bf16 h = (__bf16)vals[r];
        hi[r] = __builtin_bit_cast(uint16_t, h);
        lo[r] = f32_to_bf16_bits(vals[r] - (float)h);
      }
      uint16_t *base = frags + unit * (int64_t)d * d * 2 + i4;
      *reinterpret_cast<uint2 *>(base) =
          make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
      *reinterpret_cast<uint2 *>(base + (int64_t)d * d) =
          make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
    }
  }
  if (S_out != nullptr) {
    float *c = cache_ptr(S_out, z_out, bh, i4, d);
    c[0] = run.x;
    c[1] = run.y;
    c[2] = run.z;
    c[3] = run.w;
  }
}

}  // namespace

hipError_t launch_rope_table(const Plan &p, float2 *tab, hipStream_t stream) {
  int64_t blocks = (p.tab_entries + kBlock - 1) / kBlock;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, stream, tab, p.T,
                     p.Hs, p.Ws, (int)p.d, (double)p.theta, p.t0);
  return hipGetLastError();
}

hipError_t launch_reduce(const Plan &p, const float *partials, float *states, uint16_t *frags,
                         const float *S_in, const float *z_in, float *S_out, float *z_out,
                         hipStream_t stream) {
  const int64_t stride = kPartialStride(p.d);
  const int64_t per_block = (int64_t)kBlock * 4;
  dim3 grid((unsigned)(p.B * p.H), (unsigned)((stride + per_block - 1) / per_block));
  hipLaunchKernelGGL(reduce_prefix_kernel, grid, dim3(kBlock), 0, stream, partials, states, frags,
                     S_in, z_in, S_out, z_out, p.nb, p.C, (int)p.d);
  return hipGetLastError();
}

}  // namespace gla
