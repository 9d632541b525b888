// Matrix-core kernels of the gradients (bf16 tensors, head size 64 or 128),
// the chain rule through "SANA-Video 2.0" Section 2 Eq. (1) and the
// "SANA-Video" notes page, Sections 3.2 and 3.4 (RoPE^T rotates by minus the
// angle).  Per (batch, head) and token i of temporal block b, with the block's
// state S, z (the forward's), y = num / den, s = sigmoid(g):
//
//   query side   dg_i   = dout_i * y_i * s_i (1 - s_i)
//                dnum_i = dout_i * s_i / den_i,  dden_i = -(dout_i * s_i) . y_i / den_i
//                dq_i   = [RoPE_i^T(S dnum_i) + dden_i z] * 1[q_i > 0]
//                dS    += RoPE_i(phi(q_i))^T dnum_i,  dz += dden_i phi(q_i)   (per range)
//   key side     with G, Gz the suffix sums over blocks of dS, dz:
//                dv_n = RoPE_n(phi(k_n)) G,  dk_n = [RoPE_n^T(G v_n) + Gz] * 1[k_n > 0]
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
      kb[ks] = buf_load16<kCacheNormal>(rk, off + 64 * ks);
      vb[ks] = buf_load16<kCacheNormal>(rv, off + 64 * ks);
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
    const uint32_t row0 = (uint32_t)(tile - n_begin) * row_bytes;
    unsigned char *stage = s_stage + wave * Stage<D>::kBytes;
    // the ReLU mask of dk in the accumulator layout (bit 4*pt + i: feature
    // 16*pt + 4*kg + i of token nl).  Each lane marks its own k values
    // (bit 8*ks + jj: feature 32*ks + 8*kg + jj); feature p sits in lane
    // (nl, kg' = (p % 32) / 8) at bit 8*(p / 32) + p % 8, so the two lanes
    // kg' = 2*b + kg/2 (b = 0, 1) hold everything this lane needs.
    uint32_t kmask = 0;
    {
      uint32_t own = 0;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t kw[4] = {kb[ks].x, kb[ks].y, kb[ks].z, kb[ks].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          own |= (lo_bf16(kw[m]) > 0.f ? 1u : 0u) << (8 * ks + 2 * m);
          own |= (hi_bf16(kw[m]) > 0.f ? 1u : 0u) << (8 * ks + 2 * m + 1);
        }
      }
      const uint32_t m0 = (uint32_t)__shfl((int)own, nl + 16 * (kg >> 1));
      const uint32_t m1 = (uint32_t)__shfl((int)own, nl + 16 * (2 + (kg >> 1)));
      const int sh = 4 * (kg & 1);
#pragma unroll
      for (int pt = 0; pt < ET; ++pt)
        kmask |= (((pt & 1 ? m1 : m0) >> (8 * (pt >> 1) + sh)) & 0xFu) << (4 * pt);
    }

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
      uint2 vals[ET];
#pragma unroll
      for (int et = 0; et < ET; ++et)
        vals[et] = make_uint2(pack_bf16x2(acc[et][0], acc[et][1]), pack_bf16x2(acc[et][2], acc[et][3]));
      store_tile_rows<D>(stage, vals, rdv, row0, row_bytes);
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
      mfma_drain();
      uint2 vals[ET];
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
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (kmask >> (4 * pt + i)) & 1u ? o[i] : 0.f;
        vals[pt] = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
      }
      store_tile_rows<D>(stage, vals, rdk, row0, row_bytes);
    }
  };

  // two tiles of loads in flight per wave (as in the apply stage)
  constexpr int64_t kStep = 16 * NW;
  uint4 ka[KS], va[KS], kb2[KS], vb2[KS];
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

// ---------------------------------------------------------------- query side

constexpr int kBwdStep = 64;  // tokens per step of the query-side kernel

template <int D>
struct BwdQCfg {
  static constexpr int NW = kBwdThreads / 64;
  static constexpr int STEP = kBwdStep;
  static constexpr int KS = D / 32;
  static constexpr int ET = D / 16;
  static constexpr int ETW = ET / 2;               // 16-feature tiles per wave (one half)
  static constexpr int TILE = STEP * 2 * D;        // bytes of one token tile
  static constexpr int ST = (D / 32) * (D / 32);   // 32x32 tiles of dS^T
  static constexpr int STW = ST >= NW ? ST / NW : 1;
  static constexpr int SW = ST >= NW ? NW : ST;    // waves that hold dS
  static constexpr size_t kFixedLds =
      (size_t)D * D * 4 + 4 * (size_t)TILE + (size_t)D * 4 + 2 * (size_t)STEP * 4;
};

// One workgroup (8 waves) per (unit, token range), in steps of 64 tokens.
// Wave w takes query tile qt(w) of the step and half eh(w) of the features.
//   phase 1: phi(q), RoPE(phi(q)) hi + lo (its half of the features to an LDS
//            tile), den; num for its half of the output features (S^T
//            fragments, 3 products), y, dg (stored), dnum hi + lo (to an LDS
//            tile), its half of dout*s . y;
//   phase 2: dden; S dnum for its half of the query features (S rows x dnum
//            rows, 3 products), the inverse rotation, + dden z, the mask and
//            the store of dq; dz in registers; dS^T += dnum^T RoPE(phi(q))
//            over the step's tokens (32x32 tiles, two per wave at d = 128).
// At the end the range's dS, dz partial is written for the block sums.
template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_q_mfma_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ g,
    const uint16_t *__restrict__ dout, const float *__restrict__ states,
    const float2 *__restrict__ tab, uint16_t *__restrict__ dq, uint16_t *__restrict__ dg,
    float *__restrict__ partials, MArgs a) {
  using Cfg = BwdQCfg<D>;
  constexpr int KS = Cfg::KS, ETW = Cfg::ETW, STEP = Cfg::STEP, STW = Cfg::STW;
  constexpr int TILE = Cfg::TILE;
  extern __shared__ __align__(16) unsigned char lds[];
  unsigned char *s_sh = lds;              // S hi, [p][e] (SRow)
  unsigned char *s_sl = lds + D * D * 2;  // S lo
  unsigned char *s_rh = lds + D * D * 4;  // RoPE(phi(q)) hi, [token][feature] (KRow)
  unsigned char *s_rl = s_rh + TILE;      // RoPE(phi(q)) lo
  unsigned char *s_nh = s_rl + TILE;      // dnum hi, [token][feature] (KRow)
  unsigned char *s_nl = s_nh + TILE;      // dnum lo
  float *s_z = reinterpret_cast<float *>(s_nl + TILE);  // z (D)
  float *s_dyy = s_z + D;                               // dout*s . y per half (2 x STEP)
  float2 *s_tab = reinterpret_cast<float2 *>(s_dyy + 2 * STEP);

  const int64_t wg = blockIdx.x;
  const int64_t unit = wg / a.R, r = wg % a.R;
  const int64_t bh = unit / a.nb, blk = unit % a.nb;
  const int64_t b = bh / a.H, hd = bh % a.H;
  const int64_t n_begin = blk * a.L + r * a.Lr;
  const int64_t n_end = min(n_begin + a.Lr, (blk + 1) * a.L);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, kg = lane >> 4;
  const int qt = wave < 4 ? wave : 7 - wave;  // waves w, w + 4 share a SIMD
  const int eh = wave >> 2;

  {
    const float *ssrc = states + unit * (int64_t)(D * D + D);
    for (int i = tid; i < D * D / 4; i += kBwdThreads) {
      const float4 x = reinterpret_cast<const float4 *>(ssrc)[i];
      const int p = (4 * i) / D, e0 = (4 * i) % D;
      uint32_t h0, l0, h1, l1;
      split_bf16x2(x.x, x.y, h0, l0);
      split_bf16x2(x.z, x.w, h1, l1);
      const int o = SRow<D>::off(p, e0 >> 3) + 2 * (e0 & 7);
      *reinterpret_cast<uint2 *>(s_sh + o) = make_uint2(h0, h1);
      *reinterpret_cast<uint2 *>(s_sl + o) = make_uint2(l0, l1);
    }
    for (int i = tid; i < D; i += kBwdThreads) s_z[i] = ssrc[D * D + i];
  }
  const TabSlice<D> ts = load_tab_slice<D>(s_tab, tab, a, n_begin, n_end);

  const int64_t first = ((b * a.N + n_begin) * a.H + hd) * D;
  const uint32_t row_bytes = (uint32_t)(a.H * D * 2);
  const uint32_t range_bytes = (uint32_t)(n_end - n_begin - 1) * row_bytes + 2 * D;
  const __amdgpu_buffer_rsrc_t rq = head_rows_rsrc(q + first, range_bytes);
  const __amdgpu_buffer_rsrc_t rg = head_rows_rsrc(g + first, range_bytes);
  const __amdgpu_buffer_rsrc_t rdo = head_rows_rsrc(dout + first, range_bytes);
  const __amdgpu_buffer_rsrc_t rdq = head_rows_rsrc(dq + first, range_bytes);
  const __amdgpu_buffer_rsrc_t rdg = head_rows_rsrc(dg + first, range_bytes);

  // dS^T tiles of this wave (rows e, columns p), as the state tiles of the
  // token-causal kernel
  const bool s_owner = wave < Cfg::SW;
  int t_e[STW], t_p[STW];
  f32x16 sacc[STW];
#pragma unroll
  for (int t = 0; t < STW; ++t) {
    const int idx = wave * STW + t;
    t_e[t] = idx / (D / 32);
    t_p[t] = idx % (D / 32);
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[t][i] = 0.f;
  }
  // dz of features 16*(eh*ETW + u) + 4*kg + i, summed over this lane's tokens
  float dzacc[ETW][4];
#pragma unroll
  for (int u = 0; u < ETW; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) dzacc[u][i] = 0.f;

  uint4 qraw[KS];
  uint2 graw[ETW], draw[ETW], qc[ETW];
  // q of the wave's query tile in the B layout; g, dout and q in the
  // accumulator layout (features of half eh)
  auto load_step = [&](int64_t n0) {
    const uint32_t rel = (uint32_t)(n0 - n_begin) + 16 * qt + nl;
    const uint32_t qoff = rel * row_bytes + 16 * kg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qraw[ks] = buf_load16<kCacheNormal>(rq, qoff + 64 * ks);
    const uint32_t coff = rel * row_bytes + 8 * kg;
#pragma unroll
    for (int u = 0; u < ETW; ++u) {
      const uint32_t o = coff + 32 * (eh * ETW + u);
      graw[u] = buf_load8(rg, o);
      draw[u] = buf_load8(rdo, o);
      qc[u] = buf_load8(rq, o);
    }
  };
  // LDS offsets of the read patterns (the row swizzles depend only on low
  // row bits, which tile and k-step offsets leave alone): lane-constant
  // bases plus uniform offsets
  int tbase[KS];  // the query tile's rows in the token tiles (+ 0 per k-step unit)
  int srow[KS];   // S rows of tile 0 (+ 16 rows per tile)
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    tbase[ks] = KRow<D>::off(nl, 4 * ks + kg) + qt * (32 * D);
    srow[ks] = SRow<D>::off(nl, 4 * ks + kg);
  }
  int sbase[ETW];  // S^T fragments of the output tiles of half eh (+ 32*ks rows, + 4 rows)
#pragma unroll
  for (int u = 0; u < ETW; ++u) {
    const int et = eh * ETW + u;
    sbase[u] = SRow<D>::off(8 * kg + (nl >> 2), 2 * et + ((nl & 3) >> 1)) + 8 * (nl & 1);
  }
  int pe[STW][2], pp[STW][2];  // dS^T update reads (+ 16*kk rows)
  {
    const int g16 = lane >> 4, s16 = lane & 15;
    const int r0 = 8 * (g16 >> 1) + (s16 >> 2);
#pragma unroll
    for (int tt = 0; tt < STW; ++tt) {
      const int ce = 32 * t_e[tt] + 16 * (g16 & 1) + 4 * (s16 & 3);
      const int cp = 32 * t_p[tt] + 16 * (g16 & 1) + 4 * (s16 & 3);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        pe[tt][hh] = KRow<D>::off(r0 + 4 * hh, ce >> 3) + 2 * (ce & 7);
        pp[tt][hh] = KRow<D>::off(r0 + 4 * hh, cp >> 3) + 2 * (cp & 7);
      }
    }
  }
  load_step(n_begin);

  for (int64_t n0 = n_begin; n0 < n_end; n0 += STEP) {
    __syncthreads();  // the previous step's second phase is done with the tiles

    // ---------------- phase 1
    int t, h, w;
    {
      int64_t nq = n0 + 16 * qt + nl;
      if (nq >= n_end) nq = n_end - 1;  // position only; the row reads as zero
      token_pos(a, nq, t, h, w);
    }
    bf16x8 qh[KS], ql[KS];
    float dpart = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t qw[4] = {relu_bf16x2(qraw[ks].x), relu_bf16x2(qraw[ks].y),
                              relu_bf16x2(qraw[ks].z), relu_bf16x2(qraw[ks].w)};
      float x[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        x[2 * m] = lo_bf16(qw[m]);
        x[2 * m + 1] = hi_bf16(qw[m]);
      }
      const float4 z0 = *reinterpret_cast<const float4 *>(s_z + 32 * ks + 8 * kg);
      const float4 z1 = *reinterpret_cast<const float4 *>(s_z + 32 * ks + 8 * kg + 4);
      dpart = __builtin_fmaf(x[0], z0.x, dpart);
      dpart = __builtin_fmaf(x[1], z0.y, dpart);
      dpart = __builtin_fmaf(x[2], z0.z, dpart);
      dpart = __builtin_fmaf(x[3], z0.w, dpart);
      dpart = __builtin_fmaf(x[4], z1.x, dpart);
      dpart = __builtin_fmaf(x[5], z1.y, dpart);
      dpart = __builtin_fmaf(x[6], z1.z, dpart);
      dpart = __builtin_fmaf(x[7], z1.w, dpart);
      int ax, pi;
      pair_axis<D>(16 * ks + 4 * kg, ax, pi);
      float2 c4[4];
      ts.read(s_tab, ts.lookup(ax, pi).at(t, h, w), c4);
      rotate4(x, c4);
      uint32_t hw4[4], lw4[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) split_bf16x2(x[2 * m], x[2 * m + 1], hw4[m], lw4[m]);
      qh[ks] = __builtin_bit_cast(bf16x8, make_uint4(hw4[0], hw4[1], hw4[2], hw4[3]));
      ql[ks] = __builtin_bit_cast(bf16x8, make_uint4(lw4[0], lw4[1], lw4[2], lw4[3]));
      if ((ks >= KS / 2) == (eh == 1)) {  // this wave's half of the features
        const int o = tbase[ks];
        *reinterpret_cast<bf16x8 *>(s_rh + o) = qh[ks];
        *reinterpret_cast<bf16x8 *>(s_rl + o) = ql[ks];
      }
    }
    dpart += __shfl_xor(dpart, 16);
    dpart += __shfl_xor(dpart, 32);
    const float den = dpart + a.eps;

    // num for the output features of half eh: S^T fragments x RoPE(phi(q))
    f32x4 acc[ETW];
#pragma unroll
    for (int u = 0; u < ETW; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int u = 0; u < ETW; ++u) {
        const int o0 = sbase[u] + (32 * ks) * (2 * D);
        const int o1 = o0 + 4 * (2 * D);
        const uint2 h0 = lds_read_tr16(s_sh + o0), h1 = lds_read_tr16(s_sh + o1);
        const uint2 l0 = lds_read_tr16(s_sl + o0), l1 = lds_read_tr16(s_sl + o1);
        const bf16x8 fa = __builtin_bit_cast(bf16x8, make_uint4(h0.x, h0.y, h1.x, h1.y));
        const bf16x8 fb = __builtin_bit_cast(bf16x8, make_uint4(l0.x, l0.y, l1.x, l1.y));
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, ql[ks], acc[u], 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, qh[ks], acc[u], 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, qh[ks], acc[u], 0, 0, 0);
      }
    }
    mfma_drain();

    // y, dg, dnum, dout*s . y (value i of acc[u]: feature 16*et + 4*kg + i, token nl)
    const uint32_t coff = ((uint32_t)(n0 - n_begin) + 16 * qt + nl) * row_bytes + 8 * kg;
    const float inv_den = __builtin_amdgcn_rcpf(den);
    float dyy = 0.f;
#pragma unroll
    for (int u = 0; u < ETW; ++u) {
      const int et = eh * ETW + u;
      const float gv[4] = {lo_bf16(graw[u].x), hi_bf16(graw[u].x), lo_bf16(graw[u].y),
                           hi_bf16(graw[u].y)};
      const float dv[4] = {lo_bf16(draw[u].x), hi_bf16(draw[u].x), lo_bf16(draw[u].y),
                           hi_bf16(draw[u].y)};
      float dgo[4], dn[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y = acc[u][i] * inv_den;
        const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-gv[i]));
        const float dy = dv[i] * sg;
        dgo[i] = dy * y * (1.f - sg);
        dn[i] = dy * inv_den;
        dyy = __builtin_fmaf(dy, y, dyy);
      }
      buf_store8(rdg, coff + 32 * et, make_uint2(pack_bf16x2(dgo[0], dgo[1]), pack_bf16x2(dgo[2], dgo[3])));
      uint32_t h0, l0, h1, l1;
      split_bf16x2(dn[0], dn[1], h0, l0);
      split_bf16x2(dn[2], dn[3], h1, l1);
      const int o = KRow<D>::off(16 * qt + nl, 2 * et + (kg >> 1)) + 8 * (kg & 1);
      *reinterpret_cast<uint2 *>(s_nh + o) = make_uint2(h0, h1);
      *reinterpret_cast<uint2 *>(s_nl + o) = make_uint2(l0, l1);
    }
    dyy += __shfl_xor(dyy, 16);
    dyy += __shfl_xor(dyy, 32);
    if (kg == 0) s_dyy[eh * STEP + 16 * qt + nl] = dyy;
    // the q rows of the next step are in flight through the second phase
    // (rows past the range read as zeros)
    uint2 qcur[ETW];
#pragma unroll
    for (int u = 0; u < ETW; ++u) qcur[u] = qc[u];
    load_step(n0 + STEP);
    __syncthreads();

    // ---------------- phase 2
    const float dden = -(s_dyy[16 * qt + nl] + s_dyy[STEP + 16 * qt + nl]) * inv_den;
    // S dnum for the query features p of half eh: A = S rows p (16-byte
    // pieces), B = dnum rows of the query tile (16-byte pieces)
    f32x4 acc2[ETW];
#pragma unroll
    for (int u = 0; u < ETW; ++u) acc2[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int on = tbase[ks];
      const bf16x8 nh = *reinterpret_cast<const bf16x8 *>(s_nh + on);
      const bf16x8 nlo = *reinterpret_cast<const bf16x8 *>(s_nl + on);
#pragma unroll
      for (int u = 0; u < ETW; ++u) {
        const int o = srow[ks] + (eh * ETW + u) * (32 * D);
        const bf16x8 sh = *reinterpret_cast<const bf16x8 *>(s_sh + o);
        const bf16x8 sl = *reinterpret_cast<const bf16x8 *>(s_sl + o);
        acc2[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sl, nh, acc2[u], 0, 0, 0);
        acc2[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sh, nlo, acc2[u], 0, 0, 0);
        acc2[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sh, nh, acc2[u], 0, 0, 0);
      }
    }
    mfma_drain();
    // dq = [RoPE^T(S dnum) + dden z] * 1[q > 0]; dz += dden phi(q)
#pragma unroll
    for (int u = 0; u < ETW; ++u) {
      const int p0 = 16 * (eh * ETW + u) + 4 * kg;
      int ax, pi;
      pair_axis<D>(p0 / 2 - ((p0 / 2) & 3), ax, pi);
      float2 c4[4];
      ts.read(s_tab, ts.lookup(ax, pi).at(t, h, w), c4);
      const bool upper = ((p0 / 2) & 3) != 0;  // pairs 2, 3 of the group (else 0, 1)
      const float2 c0 = upper ? c4[2] : c4[0], c1 = upper ? c4[3] : c4[1];
      const float4 zz = *reinterpret_cast<const float4 *>(s_z + p0);
      const float d0 = acc2[u][0], d1 = acc2[u][1], d2 = acc2[u][2], d3 = acc2[u][3];
      float o[4];
      o[0] = d0 * c0.x + d1 * c0.y + dden * zz.x;
      o[1] = -d0 * c0.y + d1 * c0.x + dden * zz.y;
      o[2] = d2 * c1.x + d3 * c1.y + dden * zz.z;
      o[3] = -d2 * c1.y + d3 * c1.x + dden * zz.w;
      const float qv[4] = {lo_bf16(qcur[u].x), hi_bf16(qcur[u].x), lo_bf16(qcur[u].y),
                           hi_bf16(qcur[u].y)};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool pos = qv[i] > 0.f;
        o[i] = pos ? o[i] : 0.f;
        dzacc[u][i] = __builtin_fmaf(dden, pos ? qv[i] : 0.f, dzacc[u][i]);
      }
      buf_store8(rdq, coff + 32 * (eh * ETW + u),
                 make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])));
    }
    // dS^T += dnum^T RoPE(phi(q)) over the step's 64 tokens
    if (s_owner) {
#pragma unroll
      for (int tt = 0; tt < STW; ++tt) {
#pragma unroll
        for (int kk = 0; kk < STEP / 16; ++kk) {
          const int oe0 = pe[tt][0] + kk * (32 * D), oe1 = pe[tt][1] + kk * (32 * D);
          const int op0 = pp[tt][0] + kk * (32 * D), op1 = pp[tt][1] + kk * (32 * D);
          const uint2 a0 = lds_read_tr16(s_nh + oe0), a1 = lds_read_tr16(s_nh + oe1);
          const uint2 b0 = lds_read_tr16(s_nl + oe0), b1 = lds_read_tr16(s_nl + oe1);
          const uint2 c0 = lds_read_tr16(s_rh + op0), c1 = lds_read_tr16(s_rh + op1);
          const uint2 e0 = lds_read_tr16(s_rl + op0), e1 = lds_read_tr16(s_rl + op1);
          const bf16x8 fnh = __builtin_bit_cast(bf16x8, make_uint4(a0.x, a0.y, a1.x, a1.y));
          const bf16x8 fnl = __builtin_bit_cast(bf16x8, make_uint4(b0.x, b0.y, b1.x, b1.y));
          const bf16x8 frh = __builtin_bit_cast(bf16x8, make_uint4(c0.x, c0.y, c1.x, c1.y));
          const bf16x8 frl = __builtin_bit_cast(bf16x8, make_uint4(e0.x, e0.y, e1.x, e1.y));
          sacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fnl, frh, sacc[tt], 0, 0, 0);
          sacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fnh, frl, sacc[tt], 0, 0, 0);
          sacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fnh, frh, sacc[tt], 0, 0, 0);
        }
      }
    }
  }
  mfma_drain();

  // ---- the range's partial: dS row-major [p][e], then dz
  float *dst = partials + wg * (int64_t)(D * D + D);
  if (s_owner) {
#pragma unroll
    for (int tt = 0; tt < STW; ++tt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int e0 = 32 * t_e[tt] + 8 * i4 + 4 * (lane >> 5);
        const int p = 32 * t_p[tt] + (lane & 31);
        *reinterpret_cast<float4 *>(dst + p * D + e0) =
            make_float4(sacc[tt][4 * i4], sacc[tt][4 * i4 + 1], sacc[tt][4 * i4 + 2],
                        sacc[tt][4 * i4 + 3]);
      }
  }
  // dz: the 16 tokens of a tile sit in lanes l % 16 (fixed-order butterfly),
  // then the four query tiles of each half in order
#pragma unroll
  for (int u = 0; u < ETW; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = dzacc[u][i];
      x += __shfl_xor(x, 1);
      x += __shfl_xor(x, 2);
      x += __shfl_xor(x, 4);
      x += __shfl_xor(x, 8);
      dzacc[u][i] = x;
    }
  __syncthreads();  // the tiles are free: s_rh holds the per-tile dz sums
  float *s_dzw = reinterpret_cast<float *>(s_rh);  // [4 query tiles][D]
  if (nl == 0) {
#pragma unroll
    for (int u = 0; u < ETW; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_dzw[qt * D + 16 * (eh * ETW + u) + 4 * kg + i] = dzacc[u][i];
  }
  __syncthreads();
  if (tid < D) dst[D * D + tid] = ((s_dzw[tid] + s_dzw[D + tid]) + s_dzw[2 * D + tid]) + s_dzw[3 * D + tid];
}

template <int D>
hipError_t bwd_q_d(const Plan &p, const void *q, const void *g, const void *dout,
                   const float *states, const float2 *tab, void *dq, void *dg, float *partials,
                   hipStream_t stream) {
  const size_t lds = BwdQCfg<D>::kFixedLds + (size_t)tab_slice_entries(p, p.Lr) * sizeof(float2);
  auto kern = bwd_q_mfma_kernel<D>;
  hipError_t e = lds_limit_once((const void *)kern);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.units * p.R)), dim3(kBwdThreads), lds, stream,
                     (const uint16_t *)q, (const uint16_t *)g, (const uint16_t *)dout, states, tab,
                     (uint16_t *)dq, (uint16_t *)dg, partials, make_margs(p));
  return hipGetLastError();
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

size_t bwd_q_mfma_lds_bytes(const Plan &p) {
  if (p.d == 128) return BwdQCfg<128>::kFixedLds + (size_t)tab_slice_entries(p, p.Lr) * 8;
  if (p.d == 64) return BwdQCfg<64>::kFixedLds + (size_t)tab_slice_entries(p, p.Lr) * 8;
  return 0;
}

hipError_t backward_mfma_lds_limits() {
  return lds_limits({(const void *)bwd_q_mfma_kernel<128>, (const void *)bwd_q_mfma_kernel<64>,
                     (const void *)bwd_kv_mfma_kernel<128>, (const void *)bwd_kv_mfma_kernel<64>});
}

hipError_t launch_bwd_q_mfma(const Plan &p, const void *q, const void *g, const void *dout,
                             const float *states, const float2 *tab, void *dq, void *dg,
                             float *partials, hipStream_t stream) {
  if (p.d == 128) return bwd_q_d<128>(p, q, g, dout, states, tab, dq, dg, partials, stream);
  if (p.d == 64) return bwd_q_d<64>(p, q, g, dout, states, tab, dq, dg, partials, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_kv_mfma(const Plan &p, const void *k, const void *v, const float *grads,
                              const float2 *tab, void *dk, void *dv, hipStream_t stream) {
  if (p.d == 128) return bwd_kv_d<128>(p, k, v, grads, tab, dk, dv, stream);
  if (p.d == 64) return bwd_kv_d<64>(p, k, v, grads, tab, dk, dv, stream);
  return hipErrorInvalidValue;
}

}  // namespace gla
