// Matrix-core kernel of the key/value side of the gradients (bf16 tensors,
// head size 64 or 128), the chain rule through "SANA-Video 2.0" Section 2
// Eq. (1) and the "SANA-Video" notes page, Sections 3.2 and 3.4 (RoPE^T
// rotates by minus the angle).  With G, Gz the suffix sums over temporal
// blocks of the query side's dS, dz (block b's output reads the states of
// blocks 0..b):
//
//   dv_n = RoPE_n(phi(k_n)) G,  dk_n = [RoPE_n^T(G v_n) + Gz] * 1[k_n > 0]
//
// Every product of a rotated or fp32 operand runs on bf16 hi + lo parts (3
// products; 2 where the other operand is exact in bf16).

#include <hip/hip_runtime.h>

#include "gla_mfma_common.h"

namespace gla {
namespace {

constexpr int kBwdThreads = 512;  // 8 waves

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
  unsigned char *s_stage = reinterpret_cast<unsigned char *>(s_gz + D);  // NW staging tiles
  float2 *s_tab = reinterpret_cast<float2 *>(s_stage + NW * Stage<D>::kBytes);

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
  // G-row reads of G v: A row nl of output tile pt is G row 32 (pt / 2) +
  // 8 (nl / 4) + 4 (pt % 2) + nl % 4; the unit permutation of a row depends
  // only on nl (row bits 0, 1, 3), the tile adds a uniform row offset
  int grd[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) grd[ks] = SRow<D>::off(8 * (nl >> 2) + (nl & 3), 4 * ks + kg);

  const int64_t first = ((b * a.N + n_begin) * a.H + hd) * D;
  const uint32_t row_bytes = (uint32_t)(a.H * D * 2);
  const uint32_t range_bytes = (uint32_t)(n_end - n_begin - 1) * row_bytes + 2 * D;
  const __amdgpu_buffer_rsrc_t rk = head_rows_rsrc(k + first, range_bytes);
  const __amdgpu_buffer_rsrc_t rv = head_rows_rsrc(v + first, range_bytes);
  const __amdgpu_buffer_rsrc_t rdk = head_rows_rsrc(dk + first, range_bytes);
  const __amdgpu_buffer_rsrc_t rdv = head_rows_rsrc(dv + first, range_bytes);

  using St = Stage<D>;
  // k and v come in as whole rows (pass i, lane l: token i*kRowsPerPass +
  // l/kLanesPerRow, features 8*(l%kLanesPerRow)..+7) and reach the operand
  // layout (token nl, features 32*ks + 8*kg..+7) through the staging tile;
  // dk leaves the same way
  const int rl = lane / St::kLanesPerRow, rc = 8 * (lane % St::kLanesPerRow);
  auto fetch = [&](int64_t tile, uint4 (&kr)[St::kPasses], uint4 (&vr)[St::kPasses]) {
    const uint32_t base = (uint32_t)(tile - n_begin) * row_bytes + 2 * rc;
#pragma unroll
    for (int i = 0; i < St::kPasses; ++i) {
      const uint32_t off = base + (uint32_t)(i * St::kRowsPerPass + rl) * row_bytes;
      kr[i] = buf_load16<kCacheNormal>(rk, off);
      vr[i] = buf_load16<kCacheNormal>(rv, off);
    }
  };
  auto wave_sync = []() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // rows -> staging tile -> operand layout (the tile is free again on return)
  auto to_operand = [&](unsigned char *stage, const uint4 (&rows)[St::kPasses], uint4 (&ops)[KS]) {
#pragma unroll
    for (int i = 0; i < St::kPasses; ++i)
      *reinterpret_cast<uint4 *>(stage + (i * St::kRowsPerPass + rl) * St::kRowBytes + 2 * rc) =
          rows[i];
    wave_sync();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      ops[ks] = *reinterpret_cast<const uint4 *>(stage + nl * St::kRowBytes + 2 * (32 * ks + 8 * kg));
    wave_sync();
  };

  auto process = [&](int64_t tile, const uint4 (&kr)[St::kPasses], const uint4 (&vr)[St::kPasses]) {
    // loop-invariant LDS offsets kept inside the loop (as in the apply stage)
    int opaque = 0;
    asm volatile("" : "+v"(opaque));
    const unsigned char *gh = s_gh + opaque, *gl = s_gl + opaque;
    const int64_t n = tile + nl;
    int t, h, w;
    token_pos(a, n < n_end ? n : n_end - 1, t, h, w);
    const uint32_t row0 = (uint32_t)(tile - n_begin) * row_bytes;
    unsigned char *stage = s_stage + wave * Stage<D>::kBytes;
    uint4 kb[KS];
    to_operand(stage, kr, kb);
    uint32_t kw[KS][4];  // ReLU(k), packed bf16, in the B-operand layout
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kw[ks][0] = relu_bf16x2(kb[ks].x);
      kw[ks][1] = relu_bf16x2(kb[ks].y);
      kw[ks][2] = relu_bf16x2(kb[ks].z);
      kw[ks][3] = relu_bf16x2(kb[ks].w);
    }

    // raised wave priority while this wave issues matrix-core products (as in
    // the output stage: the other wave of the SIMD fills the gaps with its
    // vector work)
    __builtin_amdgcn_s_setprio(1);
    // ---- dv = RoPE(phi(k)) G
    {
      f32x4 acc[ET];
#pragma unroll
      for (int et = 0; et < ET; ++et) acc[et] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float x[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          x[2 * m] = lo_bf16(kw[ks][m]);
          x[2 * m + 1] = hi_bf16(kw[ks][m]);
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
      uint2 vals[ET];
#pragma unroll
      for (int et = 0; et < ET; ++et)
        vals[et] = make_uint2(pack_bf16x2(acc[et][0], acc[et][1]), pack_bf16x2(acc[et][2], acc[et][3]));
      store_tile_rows<D>(stage, vals, rdv, row0, row_bytes);
    }

    // ---- dk = [RoPE^T(G v) + Gz] * 1[k > 0], in k's operand layout: output
    // tile pt = 2 ks' + half takes A rows nl = G rows 32 ks' + 8 (nl / 4) +
    // 4 half + nl % 4, so that lane (token, kg) receives features 32 ks' +
    // 8 kg + 0..7, the features of k it holds (the mask and the pairs stay
    // in the lane); the rows then leave through the staging tile
    {
      uint4 vb[KS];
      to_operand(stage, vr, vb);
      f32x4 acc[ET];
#pragma unroll
      for (int pt = 0; pt < ET; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, vb[ks]);
#pragma unroll
        for (int pt = 0; pt < ET; ++pt) {
          // A = G rows, features 32*ks + 8*kg..+7 (one 16-byte unit)
          const int o = grd[ks] + (32 * (pt >> 1) + 4 * (pt & 1)) * (2 * D);
          const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(gh + o);
          const bf16x8 al = *reinterpret_cast<const bf16x8 *>(gl + o);
          acc[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bv, acc[pt], 0, 0, 0);
          acc[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bv, acc[pt], 0, 0, 0);
        }
      }
      mfma_drain();
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        int axis, pia;
        pair_axis<D>(16 * ks + 4 * kg, axis, pia);
        float2 c4[4];
        ts.read(s_tab, ts.lookup(axis, pia).at(t, h, w), c4);
        const float4 z0 = *reinterpret_cast<const float4 *>(s_gz + 32 * ks + 8 * kg);
        const float4 z1 = *reinterpret_cast<const float4 *>(s_gz + 32 * ks + 8 * kg + 4);
        const float gz[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
        *reinterpret_cast<uint4 *>(stage + nl * St::kRowBytes + 2 * (32 * ks + 8 * kg)) =
            rope_t_add_mask(acc[2 * ks], acc[2 * ks + 1], c4, gz, kw[ks]);
      }
      wave_sync();
#pragma unroll
      for (int i = 0; i < St::kPasses; ++i) {
        const int tok = i * St::kRowsPerPass + rl;
        buf_store16<kCacheNormal>(
            rdk, row0 + (uint32_t)tok * row_bytes + 2 * rc,
            *reinterpret_cast<const uint4 *>(stage + tok * St::kRowBytes + 2 * rc));
      }
      wave_sync();
    }
  };

  // two tiles of loads in flight per wave (as in the apply stage)
  constexpr int64_t kStep = 16 * NW;
  uint4 ka[St::kPasses], va[St::kPasses], kb2[St::kPasses], vb2[St::kPasses];
  int64_t tile = n_begin + 16 * wave;
  fetch(tile, ka, va);
  asm volatile("" ::: "memory");  // the first tile's loads are issued first
  fetch(tile + kStep, kb2, vb2);
  while (tile < n_end) {
    process(tile, ka, va);
    fetch(tile + 2 * kStep, ka, va);
    if (tile + kStep < n_end) process(tile + kStep, kb2, vb2);
    fetch(tile + 3 * kStep, kb2, vb2);
    tile += 2 * kStep;
  }
  __builtin_amdgcn_s_waitcnt(0);  // prefetches past the range are still in flight
}

template <int D>
size_t bwd_kv_lds(const Plan &p) {
  return (size_t)D * D * 4 + (size_t)D * 4 + (size_t)(kBwdThreads / 64) * Stage<D>::kBytes +
         (size_t)tab_slice_entries(p, p.Lr) * sizeof(float2);
}

template <int D>
hipError_t bwd_kv_d(const Plan &p, const void *k, const void *v, const float *grads,
                    const float2 *tab, void *dk, void *dv, hipStream_t stream) {
  const size_t lds = bwd_kv_lds<D>(p);
  auto kern = bwd_kv_mfma_kernel<D>;
  hipError_t e = lds_limit_once((const void *)kern);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.units * p.R)), dim3(kBwdThreads), lds, stream,
                     (const uint16_t *)k, (const uint16_t *)v, grads, tab, (uint16_t *)dk,
                     (uint16_t *)dv, make_margs(p));
  return hipGetLastError();
}

}  // namespace

hipError_t backward_mfma_lds_limits() {
  return lds_limits({(const void *)bwd_kv_mfma_kernel<128>, (const void *)bwd_kv_mfma_kernel<64>});
}

hipError_t launch_bwd_kv_mfma(const Plan &p, const void *k, const void *v, const float *grads,
                              const float2 *tab, void *dk, void *dv, hipStream_t stream) {
  if (p.d == 128) return bwd_kv_d<128>(p, k, v, grads, tab, dk, dv, stream);
  if (p.d == 64) return bwd_kv_d<64>(p, k, v, grads, tab, dk, dv, stream);
  return hipErrorInvalidValue;
}

}  // namespace gla
