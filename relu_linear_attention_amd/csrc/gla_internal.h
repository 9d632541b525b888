// Internal declarations shared by the host launcher (gla_api.cpp) and the
// kernel translation units.  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gla {

// Work decomposition of one call, computed on the host.
//
// A "unit" is one (batch, head, temporal block); the non-causal operator is
// the one-block case.  The state stage splits each unit's L tokens into C
// chunks of Lc tokens (the last one ragged) and writes one fp32 partial
// (S_c, z_c) per chunk; the reduce stage sums the partials of a unit in chunk
// order and runs the inclusive prefix over the blocks of a (batch, head) in
// block order; the apply stage splits each unit's tokens into R ranges of Lr
// tokens.
struct Plan {
  int64_t B, H, T, Hs, Ws, d;
  int64_t F;      // frames per block (== T when non-causal)
  int64_t t0;     // absolute temporal position of frame 0 (streaming blocks)
  int64_t nb;     // temporal blocks per (batch, head)
  int64_t N;      // tokens per batch entry, T*Hs*Ws
  int64_t L;      // tokens per block
  int64_t units;  // B*H*nb
  int64_t C, Lc;  // state chunks per unit, tokens per chunk
  int64_t R, Lr;  // apply ranges per unit, tokens per range
  int64_t Rb, Lb; // backward ranges per unit, tokens per range
  bool bf16;      // element type of q, k, v, g, out
  bool mfma;      // matrix-core kernels (bf16, d = 64 or 128)
  float theta, eps;
  float rms_eps;  // RMSNorm epsilon (gated mixer only)
  int64_t tab_entries;  // RoPE table entries (cos, sin pairs)
  int64_t tab_t_off, tab_h_off, tab_w_off;  // entry offsets of the axis tables
  // workspace layout, byte offsets
  size_t off_tab, off_part, off_state, off_frag, total_bytes;
  // the backward call's extra sections (after total_bytes): the per-range
  // dS, dz partials and the suffix-summed gradients of the block states
  size_t off_bpart, off_grad, bwd_total_bytes;
};

constexpr int kBlock = 256;          // threads per workgroup for every kernel
constexpr int64_t kStateTile = 64;   // tokens per step of the matrix-core state kernel
constexpr int64_t kApplyTile = 16;   // tokens per wave step of the matrix-core apply kernel (8 waves)
constexpr int64_t kPartialStride(int64_t d) { return d * d + d; }

// run += src[c * stride .. + 3] for c = c0, c0 + 1, ..., c1 - 1, added in
// that order (so the sum is bitwise that of the plain loop), with eight
// loads in flight: the reduce kernels are latency-bound with one partial per
// round trip.  Indices past c1 - 1 are clamped (their values are loaded and
// dropped), so every load is unconditional.
__device__ __forceinline__ void add_partials(float4 &run, const float *src, int64_t stride,
                                             int64_t c0, int64_t c1) {
  for (int64_t c = c0; c < c1; c += 8) {
    float4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t cj = c + j < c1 ? c + j : c1 - 1;
      x[j] = *reinterpret_cast<const float4 *>(src + cj * stride);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (c + j < c1) {
        run.x += x[j].x;
        run.y += x[j].y;
        run.z += x[j].z;
        run.w += x[j].w;
      }
    }
  }
}

// LDS budget of the RoPE table slice kept by the matrix-core kernels
// (float2 entries).
constexpr int64_t kStateTabEntries = 6144;  // 48 KiB
constexpr int64_t kApplyTabEntries = 5120;  // 40 KiB

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  All enqueue on `stream`.

// RoPE table: cos/sin per (axis, position, pair), computed in fp64 and
// stored as float2.
hipError_t launch_rope_table(const Plan &p, float2 *tab, hipStream_t stream);

// State partials, vector kernels (any supported d, bf16 or f32).  beta
// (optional, [B, N, H] of the tensors' type): the write gate, a factor on
// each token's rotated key in S only.
hipError_t launch_state_generic(const Plan &p, const void *k, const void *v, const void *beta,
                                const float2 *tab, float *partials, hipStream_t stream);
// Fixed-order reduce of the partials plus the inclusive block prefix.
// Writes fp32 states [units][d*d + d] and, for the matrix-core path, S as
// row-major bf16 hi and lo parts [units][2][d][d].  S_in/z_in (optional,
// [B*H][d][d] and [B*H][d]) start the running sums of each (batch, head);
// S_out/z_out (optional, may alias S_in/z_in) receive the final sums.
hipError_t launch_reduce(const Plan &p, const float *partials, float *states,
                         uint16_t *frags, const float *S_in, const float *z_in, float *S_out,
                         float *z_out, hipStream_t stream);
// Output stage, vector kernels.  rms_w (optional, [d] of the tensors' type):
// RMSNorm of num/den with that weight (epsilon p.rms_eps) before the gate.
hipError_t launch_apply_generic(const Plan &p, const void *q, const void *g, const float *states,
                                const float2 *tab, const void *rms_w, void *out,
                                hipStream_t stream);

// Matrix-core kernels (bf16, d = 64 or 128).
hipError_t launch_state_mfma(const Plan &p, const void *k, const void *v, const void *beta,
                             const float2 *tab, float *partials, hipStream_t stream);
hipError_t launch_apply_mfma(const Plan &p, const void *q, const void *g, const float *states,
                             const uint16_t *frags, const float2 *tab, const void *rms_w,
                             void *out, hipStream_t stream);

// Token-causal form.  The state stage writes one partial per chunk of Lc
// tokens (units = B*H, one block each); the prefix kernel writes, for every
// range of Lr = m*Lc tokens, the exclusive sum of the partials before it
// ([units][R][d*d + d]); the tile kernels walk each range from that sum.
hipError_t launch_range_prefix(const Plan &p, const float *partials, float *states,
                               hipStream_t stream);
// Matrix-core tile kernel (bf16, d = 64 or 128, Lr a multiple of 64) and its
// LDS bytes for the plan's ranges.
hipError_t launch_causal_mfma(const Plan &p, const void *q, const void *k, const void *v,
                              const void *g, const float *states, const float2 *tab, void *out,
                              hipStream_t stream);
size_t causal_mfma_lds_bytes(const Plan &p);
hipError_t launch_causal_generic(const Plan &p, const void *q, const void *k, const void *v,
                                 const void *g, const float *states, const float2 *tab, void *out,
                                 hipStream_t stream);

// Gradients (vector kernels): with the forward states of the call in
// `states`, writes dq, dk, dv, dg; `partials` holds units*Rb and `grads`
// units state vectors of d*d + d floats.
hipError_t launch_backward(const Plan &p, const void *q, const void *k, const void *v,
                           const void *g, const void *dout, const float *states,
                           const float2 *tab, float *partials, float *grads, void *dq, void *dk,
                           void *dv, void *dg, hipStream_t stream);

// Matrix-core kernel of the key/value side of the gradients (bf16, d = 64 or
// 128): dk, dv from G, Gz (`grads`, [units][d*d + d]); ranges R x Lr.
// Matrix-core kernel of the query side of the gradients (bf16, d = 64 or
// 128): dq, dg and the per-range dS, dz partials ([units][R][d*d + d]) from
// the forward states; ranges R x Lr (Lr a multiple of 64).
hipError_t launch_bwd_q_mfma(const Plan &p, const void *q, const void *g, const void *dout,
                             const float *states, const float2 *tab, void *dq, void *dg,
                             float *partials, hipStream_t stream);
size_t bwd_q_mfma_lds_bytes(const Plan &p);
hipError_t launch_bwd_kv_mfma(const Plan &p, const void *k, const void *v, const float *grads,
                              const float2 *tab, void *dk, void *dv, hipStream_t stream);

// Division by a fixed divisor d >= 1 for dividends 0 <= n < 2^31, by a
// multiply-high and a shift: with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1, n / d = (mulhi(n, m) + n) >> s.
struct FastDiv {
  uint32_t d, m, s;
  static FastDiv make(uint32_t d) {
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    uint32_t m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << s) - d)) / d + 1);
    return FastDiv{d, m, s};
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    return (__umulhi(n, m) + n) >> s;
  }
};

// ------------------------------------------------------------ device helpers
__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Token index -> (t, h, w) of the t-major latent grid.
__device__ __forceinline__ void grid_pos(int64_t n, int64_t Hs, int64_t Ws, int &t, int &h,
                                         int &w) {
  int64_t hw = Hs * Ws;
  t = (int)(n / hw);
  int64_t r = n - (int64_t)t * hw;
  h = (int)(r / Ws);
  w = (int)(r - (int64_t)h * Ws);
}

}  // namespace gla
