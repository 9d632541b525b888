// Kernels shared by both paths: the RoPE table and the fixed-order reduce /
// block prefix of the state partials.
//
// "SANA-Video" notes page, Section 3.2: RoPE rotates phi(q) and phi(k) in the
// numerator; Section 3.4: a block reads the running sums of the states and
// normalisers of all earlier blocks plus its own.

#include <hip/hip_runtime.h>

#include <mutex>
#include <utility>
#include <vector>

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

// The fixed-order reduce and block prefix of the state partials
// (reduce_prefix_values), one (batch, head) per blockIdx.x, four consecutive
// floats of its d*d + d state vector per thread.
__global__ __launch_bounds__(kBlock) void reduce_prefix_kernel(
    const float *__restrict__ partials, float *__restrict__ states, uint16_t *__restrict__ frags,
    const float *S_in, const float *z_in, float *S_out, float *z_out, int64_t nb, int64_t C,
    int d) {
  const int64_t stride = (int64_t)d * d + d;
  const int64_t i4 = ((int64_t)blockIdx.y * blockDim.x + threadIdx.x) * 4;
  if (i4 >= stride) return;
  reduce_prefix_values(partials, states, frags, S_in, z_in, S_out, z_out, blockIdx.x, nb, C, d,
                       i4);
}

}  // namespace

hipError_t lds_limit_once(const void *kern) {
  static std::mutex mu;
  static std::vector<std::pair<const void *, int>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  for (const auto &x : done)
    if (x.first == kern && x.second == dev) return hipSuccess;
  // a CU's 160 KiB less the kernel's static LDS
  hipFuncAttributes fa;
  e = hipFuncGetAttributes(&fa, kern);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                          160 * 1024 - (int)fa.sharedSizeBytes);
  if (e == hipSuccess) done.emplace_back(kern, dev);
  return e;
}

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
