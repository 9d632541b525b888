// Internal declarations shared by the host launcher (gla_api.cpp) and the
// kernel translation units.  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <initializer_list>

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
  // output stage (matrix cores): a workgroup owns hpw heads of one (batch,
  // block) (hpw = 1); ag such units, each block cut into ar super-ranges of
  // air items of 128 tokens, am workgroups per super-range taking its items
  // in turn
  int64_t hpw, ag, ar, air, am;
  bool apair;     // output stage: two 16-token blocks per wave at a time
  bool bf16;      // element type of q, k, v, g, out
  bool mfma;      // matrix-core kernels (bf16, d = 64 or 128)
  float theta, eps;
  float rms_eps;  // RMSNorm epsilon (gated mixer only)
  int64_t tab_entries;  // RoPE table entries (cos, sin pairs)
  int64_t tab_t_off, tab_h_off, tab_w_off;  // entry offsets of the axis tables
  // workspace layout, byte offsets
  size_t off_tab, off_part, off_state, off_frag, total_bytes;
  // the backward call's extra sections (after total_bytes): the per-range
  // (or, on the matrix cores, per-chunk) dS, dz partials, the suffix-summed
  // gradients of the block states, and (matrix cores) each token's
  // (den, dden), float2 [B*H][N]
  size_t off_bpart, off_grad, off_dd, bwd_total_bytes;
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
// `load` reads the four floats at a pointer (PlainLoad4: an ordinary load).
struct PlainLoad4 {
  __device__ __forceinline__ float4 operator()(const float *p) const {
    return *reinterpret_cast<const float4 *>(p);
  }
};
template <class Load = PlainLoad4>
__device__ __forceinline__ void add_partials(float4 &run, const float *src, int64_t stride,
                                             int64_t c0, int64_t c1, Load load = Load()) {
  for (int64_t c = c0; c < c1; c += 8) {
    float4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t cj = c + j < c1 ? c + j : c1 - 1;
      x[j] = load(src + cj * stride);
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

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// The element i4 of the carried cache (S rows then z) of (batch, head) bh.
__device__ __forceinline__ float *cache_ptr(float *S, float *z, int64_t bh, int64_t i4, int d) {
  const int64_t dd = (int64_t)d * d;
  return i4 < dd ? S + bh * dd + i4 : z + bh * d + (i4 - dd);
}

// The running sums `run` of floats i4..i4+3 of unit `unit`'s state (d*d + d
// floats: S rows, then z): written to `states` and, for S and when `frags` is
// given, as bf16 hi + lo parts (hi = the value rounded to bf16, lo = the
// remainder rounded to bf16; the d*d lo values follow the d*d hi values of a
// unit, each row-major [p][e]).
__device__ __forceinline__ void store_state4(const float4 &run, float *states, uint16_t *frags,
                                             int64_t unit, int d, int64_t i4) {
  const int64_t stride = (int64_t)d * d + d;
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

// Sum of the C chunk partials of every block unit of (batch, head) bh, in
// chunk order, followed by the inclusive prefix over its nb temporal blocks,
// in block order, for the four consecutive floats i4..i4+3 of the d*d + d
// state vector (d % 4 == 0, so they never straddle S and z).  Every output
// value is owned by one caller, so the result is the same on every run; the
// separate reduce kernel and the state kernel's last workgroup both run
// this, so their results agree bit for bit.
//
// states: [unit][d*d + d] running sums (unit = bh * nb + block).
// frags (optional): S in two bf16 parts, S ~ hi + lo (hi = S rounded to
// bf16, lo = the remainder rounded to bf16), each row-major [p][e]; the d*d
// lo values follow the d*d hi values of a unit.
// S_in/z_in (optional): the sums carried in from earlier blocks, where the
// running sums start; S_out/z_out (optional): the final running sums.  The
// four values of S_in/z_in are read before the same four of S_out/z_out are
// written, so the two may be the same arrays (an in-place update).
template <class Load = PlainLoad4>
__device__ __forceinline__ void reduce_prefix_values(const float *partials, float *states,
                                                     uint16_t *frags, const float *S_in,
                                                     const float *z_in, float *S_out,
                                                     float *z_out, int64_t bh, int64_t nb,
                                                     int64_t C, int d, int64_t i4,
                                                     Load load = Load()) {
  const int64_t stride = (int64_t)d * d + d;
  float4 run = make_float4(0.f, 0.f, 0.f, 0.f);
  if (S_in != nullptr) {
    const float *c = cache_ptr(const_cast<float *>(S_in), const_cast<float *>(z_in), bh, i4, d);
    run = make_float4(c[0], c[1], c[2], c[3]);
  }
  for (int64_t blk = 0; blk < nb; ++blk) {
    const int64_t unit = bh * nb + blk;
    add_partials(run, partials + unit * C * stride + i4, stride, 0, C, load);
    store_state4(run, states, frags, unit, d, i4);
  }
  if (S_out != nullptr) {
    float *c = cache_ptr(S_out, z_out, bh, i4, d);
    c[0] = run.x;
    c[1] = run.y;
    c[2] = run.z;
    c[3] = run.w;
  }
}

// Size of the static scratch array behind gla_forward_noalloc (one copy per
// device, held until the process ends).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
// Device address of the current device's scratch array (looked up once per
// device).
hipError_t noalloc_scratch(void **ptr);

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
// Raises a kernel's dynamic-LDS limit to a compute unit's 160 KiB less the
// kernel's static LDS, once per (kernel, device) rather than before every
// launch; thread-safe.
hipError_t lds_limit_once(const void *kern);
// lds_limit_once for each kernel of a list (stops at the first failure).
inline hipError_t lds_limits(std::initializer_list<const void *> kerns) {
  for (const void *k : kerns) {
    const hipError_t e = lds_limit_once(k);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
// The limits of every kernel of one translation unit; the library sets them
// all once per device, before its first launch there, so that no call fails
// on an attribute after it has enqueued work.
hipError_t apply_mfma_lds_limits();
hipError_t state_mfma_lds_limits();
hipError_t causal_mfma_lds_limits();
hipError_t backward_mfma_lds_limits();
hipError_t backward_query_lds_limits();
hipError_t vector_lds_limits();
hipError_t causal_vector_lds_limits();
hipError_t backward_vector_lds_limits();
// dynamic LDS of the matrix-core state kernel
size_t state_mfma_lds_bytes(const Plan &p);
// The reduce folded into the state kernel (one temporal block, nb == 1):
// each workgroup counts itself done on cnt[unit] (an agent-scope atomic),
// and the last of a unit's C workgroups runs reduce_prefix_values for the
// unit and puts cnt[unit] back to 0.  cnt must hold zeros when the kernel
// starts, and no other kernel may use it meanwhile.  cnt == nullptr: the
// partials are left for the separate reduce kernel.
struct FusedReduce {
  unsigned *cnt = nullptr;
  float *states = nullptr;
  uint16_t *frags = nullptr;
  const float *S_in = nullptr, *z_in = nullptr;
  float *S_out = nullptr, *z_out = nullptr;
};
hipError_t launch_state_mfma(const Plan &p, const void *k, const void *v, const void *beta,
                             const float2 *tab, float *partials, const FusedReduce &fuse,
                             hipStream_t stream);
// Output stage on the matrix cores (bf16, d = 64 or 128): frags holds S of
// every unit as bf16 hi and lo parts, [units][part][d][d] row-major (written
// by the reduce); its LDS bytes for the plan.
hipError_t launch_apply_mfma(const Plan &p, const void *q, const void *g, const float *states,
                            const uint16_t *frags, const float2 *tab, const void *rms_w,
                            void *out, hipStream_t stream);
size_t apply_mfma_lds_bytes(const Plan &p);
// tokens of one work item of the output stage
int64_t apply_mfma_item_tokens();

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

// Gradients: with the forward states of the call in `states`, writes dq,
// dk, dv, dg; `partials` holds units * max(Rb, C) and `grads` units state
// vectors of d*d + d floats; `dd` (matrix-core path) B*H*N float2.
hipError_t launch_backward(const Plan &p, const void *q, const void *k, const void *v,
                           const void *g, const void *dout, const float *states,
                           const float2 *tab, float *partials, float *grads, float2 *dd,
                           void *dq, void *dk, void *dv, void *dg, hipStream_t stream);

// Query side of the gradients on the matrix cores (bf16, d = 64 or 128), in
// two passes: the token pass writes dq, dg and each token's (den, dden)
// (ranges R x Lr, Lr a multiple of 128); the state pass re-reads q, g, dout
// and writes the per-chunk dS, dz partials ([units][C][d*d + d]).
hipError_t launch_bwd_token_mfma(const Plan &p, const void *q, const void *g, const void *dout,
                                 const float *states, const float2 *tab, void *dq, void *dg,
                                 float2 *dd, hipStream_t stream);
hipError_t launch_bwd_dstate_mfma(const Plan &p, const void *q, const void *g, const void *dout,
                                  const float2 *dd, const float2 *tab, float *partials,
                                  hipStream_t stream);
size_t bwd_query_lds_bytes(const Plan &p);
// Matrix-core kernel of the key/value side of the gradients (bf16, d = 64 or
// 128): dk, dv from G, Gz (`grads`, [units][d*d + d]); ranges R x Lr.
hipError_t launch_bwd_kv_mfma(const Plan &p, const void *k, const void *v, const float *grads,
                              const float2 *tab, void *dk, void *dv, hipStream_t stream);

// Division by a fixed divisor d >= 1 for dividends 0 <= n < 2^31, by a
// multiply-high and a shift: the division by invariant integers using
// multiplication of Granlund and Montgomery (PLDI 1994), in its N+1-bit
// multiplier form.  With s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d)
// + 1, n / d = (mulhi(n, m) + n) >> s (the sum stays below 2^32 because
// n < 2^31).
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
