// Matrix-core kernel of the key/value side of the gradients (bf16 tensors,
// head size 64 or 128).  With G, Gz the gradients that reach the state and
// the normaliser of a unit (the suffix sums over blocks of the per-range
// dS, dz partials of the query side), per token n:
//
//   dv_n = RoPE_n(phi(k_n)) G
//   dk_n = [RoPE_n^T(G v_n) + Gz] * 1[k_n > 0]
//
// (the chain rule through "SANA-Video 2.0" Section 2 Eq. (1) and the
// "SANA-Video" notes page, Sections 3.2 and 3.4; RoPE^T rotates by minus the
// angle).  One workgroup (8 waves) per (unit, token range), as the forward
// apply stage: G sits in LDS as bf16 hi + lo parts (row-major [p][e], the
// layout of S there), each wave takes 16-token tiles:
//   dv: A = G^T fragments (transposing reads), B = RoPE(phi(k)) hi / lo in
//       the B layout (k rows loaded 16 bytes per lane): 3 products;
//   dk: A = G rows (16-byte row pieces), B = v in the B layout (exact in
//       bf16): 2 products; then the inverse rotation, + Gz and the mask, in
//       the accumulator layout (four consecutive features per lane).

#include <hip/hip_runtime.h>

#include "gla_mfma_common.h"

namespace gla {
namespace {

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBwdThreads = 512;  // 8 waves

__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kCacheNormal);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2 x) {
  const u32x2 v = {x.x, x.y};
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, kCacheNormal);
}

// Sixteen wait states after the last matrix-core instruction of a chain,
// with the scheduler kept from moving anything across, before vector code
// reads the results or reuses the accumulator registers.
__device__ __forceinline__ void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_kv_mfma_kernel(
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ grads, const float2 *__restrict__ tab,
    uint16_t *__restrict__ dk, uint16_t *__restrict__ dv, MArgs a) {
  constexpr int KS = D / 32;  // 32-feature contraction steps
  constexpr int ET = D / 16;  // 16-feature output tiles
  constexpr int NW = kBwdThreads / 64;
  extern __shared__ __align__(16) unsigned char lds[];
  unsigned char *s_gh = lds;              // G hi, row-major [p][e], units permuted (SRow)
  unsigned char *s_gl = lds + D * D * 2;  // G lo
  float *s_gz = reinterpret_cast<float *>(lds + D * D * 4);  // Gz (D)
  float2 *s_tab = reinterpret_cast<float2 *>(s_gz + D);

  const int64_t wg = blockIdx.x;
  const int64_t unit = wg / a.R, r = wg % a.R;
  const int64_t bh = unit / a.nb, blk = unit % a.nb;
  const int64_t b = bh / a.H, hd = bh % a.H;
  const int64_t n_begin = blk * a.L + r * a.Lr;
  const int64_t n_end = min(n_begin + a.Lr, (blk + 1) * a.L);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  {
    // G (fp32, row-major) -> bf16 hi + lo in LDS; four consecutive e per thread
    const float *gsrc = grads + unit * (int64_t)(D * D + D);
    for (int i = tid; i < D * D / 4; i += kBwdThreads) {
      const float4 x = reinterpret_cast<const float4 *>(gsrc)[i];
      const int p = (4 * i) / D, e0 = (4 * i) % D;
      uint32_t h0, l0, h1, l1;
      split_bf16x2(x.x, x.y, h0, l0);
      split_bf16x2(x.z, x.w, h1, l1);
      const int o = SRow<D>::off(p, e0 >> 3) + 2 * (e0 & 7);
      *reinterpret_cast<uint2 *>(s_gh + o) = make_uint2(h0, h1);
      *reinterpret_cast<uint2 *>(s_gl + o) = make_uint2(l0, l1);
    }
    for (int i = tid; i < D; i += kBwdThreads) s_gz[i] = gsrc[D * D + i];
  }
  const TabSlice<D> ts = load_tab_slice<D>(s_tab, tab, a, n_begin, n_end);
  __syncthreads();

  const int nl = lane & 15, kg = lane >> 4;
  // transposing-read offsets of G^T fragments (as S^T in the apply stage)
  int rd_t[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et)
    rd_t[et] = SRow<D>::off(8 * kg + (nl >> 2), 2 * et + ((nl & 3) >> 1)) + 8 * (nl & 1);

  const int64_t first = ((b * a.N + n_begin) * a.H + hd) * D;
  const uint32_t row_bytes = (uint32_t)(a.H * D * 2);
  const uint32_t range_bytes = (uint32_t)(n_end - n_begin - 1) * row_bytes + 2 * D;
  const __amdgpu_buffer_rsrc_t rk = head_rows_rsrc(k + first, range_bytes);
  const __amdgpu_buffer_rsrc_t rv = head_rows_rsrc(v + first, range_bytes);
  const __amdgpu_buffer_rsrc_t rdk = head_rows_rsrc(dk + first, range_bytes);
  const __amdgpu_buffer_rsrc_t rdv = head_rows_rsrc(dv + first, range_bytes);

  auto fetch = [&](int64_t tile, uint4 (&kb)[KS], uint4 (&vb)[KS]) {
    const uint32_t off = ((uint32_t)(tile - n_begin) + nl) * row_bytes + 16 * kg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kb[ks] = buf_load16<kCacheStream>(rk, off + 64 * ks);
      vb[ks] = buf_load16<kCacheStream>(rv, off + 64 * ks);
    }
  };

  auto process = [&](int64_t tile, const uint4 (&kb)[KS], const uint4 (&vb)[KS]) {
    // loop-invariant LDS offsets kept inside the loop (as in the apply stage)
    int opaque = 0;
    asm volatile("" : "+v"(opaque));
    const unsigned char *gh = s_gh + opaque, *gl = s_gl + opaque;
    const int64_t n = tile + nl;
    int t, h, w;
    token_pos(a, n < n_end ? n : n_end - 1, t, h, w);
    const uint32_t toff = ((uint32_t)(tile - n_begin) + nl) * row_bytes + 8 * kg;

    // ---- dv = RoPE(phi(k)) G
    {
      f32x4 acc[ET];
#pragma unroll
      for (int et = 0; et < ET; ++et) acc[et] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t kw[4] = {relu_bf16x2(kb[ks].x), relu_bf16x2(kb[ks].y),
                                relu_bf16x2(kb[ks].z), relu_bf16x2(kb[ks].w)};
        float x[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          x[2 * m] = lo_bf16(kw[m]);
          x[2 * m + 1] = hi_bf16(kw[m]);
        }
        int axis, pia;
        pair_axis<D>(16 * ks + 4 * kg, axis, pia);
        float2 c4[4];
        ts.read(s_tab, ts.lookup(axis, pia).at(t, h, w), c4);
        rotate4(x, c4);
        uint32_t hw4[4], lw4[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) split_bf16x2(x[2 * m], x[2 * m + 1], hw4[m], lw4[m]);
        const bf16x8 bh = __builtin_bit_cast(bf16x8, make_uint4(hw4[0], hw4[1], hw4[2], hw4[3]));
        const bf16x8 bl = __builtin_bit_cast(bf16x8, make_uint4(lw4[0], lw4[1], lw4[2], lw4[3]));
#pragma unroll
        for (int eg = 0; eg < ET; eg += 4) {
          bf16x8 ah[4], al[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int o0 = rd_t[eg + u] + (32 * ks) * (2 * D);
            const int o1 = o0 + 4 * (2 * D);
            const uint2 h0 = lds_read_tr16(gh + o0), h1 = lds_read_tr16(gh + o1);
            const uint2 l0 = lds_read_tr16(gl + o0), l1 = lds_read_tr16(gl + o1);
            ah[u] = __builtin_bit_cast(bf16x8, make_uint4(h0.x, h0.y, h1.x, h1.y));
            al[u] = __builtin_bit_cast(bf16x8, make_uint4(l0.x, l0.y, l1.x, l1.y));
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
            acc[eg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[u], bl, acc[eg + u], 0, 0, 0);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            acc[eg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[u], bh, acc[eg + u], 0, 0, 0);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            acc[eg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[u], bh, acc[eg + u], 0, 0, 0);
        }
      }
      mfma_drain();
      // value i of acc[et]: feature 16*et + 4*kg + i of token nl
#pragma unroll
      for (int et = 0; et < ET; ++et)
        buf_store8(rdv, toff + 32 * et,
                   make_uint2(pack_bf16x2(acc[et][0], acc[et][1]), pack_bf16x2(acc[et][2], acc[et][3])));
    }

    // ---- dk = [RoPE^T(G v) + Gz] * 1[k > 0]
    {
      f32x4 acc[ET];
#pragma unroll
      for (int pt = 0; pt < ET; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, vb[ks]);
#pragma unroll
        for (int pt = 0; pt < ET; ++pt) {
          // A = G rows p = 16*pt + nl, features 32*ks + 8*kg..+7 (one 16-byte unit)
          const int o = SRow<D>::off(16 * pt + nl, 4 * ks + kg);
          const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(gh + o);
          const bf16x8 al = *reinterpret_cast<const bf16x8 *>(gl + o);
          acc[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bv, acc[pt], 0, 0, 0);
          acc[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bv, acc[pt], 0, 0, 0);
        }
      }
      // k in the accumulator layout, for the ReLU mask
      uint2 kc[ET];
#pragma unroll
      for (int pt = 0; pt < ET; ++pt) kc[pt] = buf_load8(rk, toff + 32 * pt);
      mfma_drain();
#pragma unroll
      for (int pt = 0; pt < ET; ++pt) {
        // features p0..p0+3 = pairs P0, P0 + 1 (half of a table group)
        const int p0 = 16 * pt + 4 * kg;
        int axis, pia;
        pair_axis<D>(p0 / 2 - ((p0 / 2) & 3), axis, pia);
        float2 c4[4];
        ts.read(s_tab, ts.lookup(axis, pia).at(t, h, w), c4);
        const bool upper = ((p0 / 2) & 3) != 0;  // pairs 2, 3 of the group (else 0, 1)
        const float2 c0 = upper ? c4[2] : c4[0], c1 = upper ? c4[3] : c4[1];
        const float4 gz = *reinterpret_cast<const float4 *>(s_gz + p0);
        const float d0 = acc[pt][0], d1 = acc[pt][1], d2 = acc[pt][2], d3 = acc[pt][3];
        float o[4];
        o[0] = d0 * c0.x + d1 * c0.y + gz.x;
        o[1] = -d0 * c0.y + d1 * c0.x + gz.y;
        o[2] = d2 * c1.x + d3 * c1.y + gz.z;
        o[3] = -d2 * c1.y + d3 * c1.x + gz.w;
        const float kv[4] = {lo_bf16(kc[pt].x), hi_bf16(kc[pt].x), lo_bf16(kc[pt].y),
                             hi_bf16(kc[pt].y)};
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = kv[i] > 0.f ? o[i] : 0.f;
        buf_store8(rdk, toff + 32 * pt, make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])));
      }
    }
  };

  // two tiles of loads in flight per wave (as in the apply stage)
  constexpr int64_t kStep = 16 * NW;
  uint4 ka[KS], va[KS], kb2[KS], vb2[KS];
  int64_t tile = n_begin + 16 * wave;
  if (tile < n_end) fetch(tile, ka, va);
  if (tile + kStep < n_end) fetch(tile + kStep, kb2, vb2);
  while (tile < n_end) {
    process(tile, ka, va);
    if (tile + 2 * kStep < n_end) fetch(tile + 2 * kStep, ka, va);
    tile += kStep;
    if (tile >= n_end) break;
    process(tile, kb2, vb2);
    if (tile + 2 * kStep < n_end) fetch(tile + 2 * kStep, kb2, vb2);
    tile += kStep;
  }
}

template <int D>
size_t bwd_kv_lds(const Plan &p) {
  return (size_t)D * D * 4 + (size_t)D * 4 + (size_t)tab_slice_entries(p, p.Lr) * sizeof(float2);
}

template <int D>
hipError_t bwd_kv_d(const Plan &p, const void *k, const void *v, const float *grads,
                    const float2 *tab, void *dk, void *dv, hipStream_t stream) {
  const size_t lds = bwd_kv_lds<D>(p);
  auto kern = bwd_kv_mfma_kernel<D>;
  hipError_t e = hipFuncSetAttribute((const void *)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.units * p.R)), dim3(kBwdThreads), lds, stream,
                     (const uint16_t *)k, (const uint16_t *)v, grads, tab, (uint16_t *)dk,
                     (uint16_t *)dv, make_margs(p));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_kv_mfma(const Plan &p, const void *k, const void *v, const float *grads,
                              const float2 *tab, void *dk, void *dv, hipStream_t stream) {
  if (p.d == 128) return bwd_kv_d<128>(p, k, v, grads, tab, dk, dv, stream);
  if (p.d == 64) return bwd_kv_d<64>(p, k, v, grads, tab, dk, dv, stream);
  return hipErrorInvalidValue;
}

}  // namespace gla
