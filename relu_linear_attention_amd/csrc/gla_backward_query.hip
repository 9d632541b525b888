// Query-side gradient kernels on the matrix cores (bf16, head size 64 or
// 128), the chain rule through "SANA-Video 2.0" Section 2 Eq. (1) and the
// "SANA-Video" notes page, Sections 3.2 and 3.4 (RoPE^T rotates by minus the
// angle).  Per (batch, head) and token i of temporal block b, with the
// block's state S, z, x_i = RoPE_i(phi(q_i)), y = num / den, s = sigmoid(g):
//
//   token pass   dg_i   = dout_i * y_i * s_i (1 - s_i)
//                dnum_i = dout_i * s_i / den_i,  dden_i = -(dout_i * s_i) . y_i / den_i
//                dq_i   = [RoPE_i^T(S dnum_i) + dden_i z] * 1[q_i > 0]
//   state pass   dS    += x_i^T dnum_i,  dz += dden_i phi(q_i)   (per chunk)
//
// The token pass (bwd_token_mfma_kernel) works like the forward's output
// stage: every wave takes 16-token tiles on its own, with no barrier, and
// keeps (den, dden) of each token for the state pass.  The state pass
// (bwd_dstate_mfma_kernel) works like the forward's state stage: it re-reads
// q, g and dout, rebuilds x and dnum, and contracts them over the chunk's
// tokens.  Every product of a rotated or fp32 operand runs on bf16 hi + lo
// parts (3 products, dropping lo * lo).

#include <hip/hip_runtime.h>

#include <algorithm>

#include "gla_mfma_common.h"

namespace gla {
namespace {

constexpr int kTokThreads = 512;  // 8 waves, a 16-token tile each

// One workgroup (8 waves) per (unit, token range).  LDS: S hi and lo parts
// (row-major [p][e], SRow layout), the z fragments of the denominator
// product (as in the output stage), z in fp32, a staging tile per wave, and
// the RoPE table slice of the range.  Per 16-token tile a wave
//   1. loads q in the B-operand layout of v_mfma_f32_16x16x32_bf16 (lane l:
//      token l % 16, features 32 ks + 8 (l / 16) + 0..7), and g and dout as
//      whole rows, which pass through a per-wave staging tile into the
//      accumulator layout (features 16 et + 4 (l / 16) + 0..3);
//   2. forms x = RoPE(ReLU(q)) hi + lo and num = x S (3 products per tile of
//      S^T fragments), den = ReLU(q) . z + eps on the matrix cores;
//   3. computes y, s, dg (stored as whole rows through the staging tile),
//      dnum (split into hi + lo) and the sum
//      dout s . y over the token's features (its four lanes);
//   4. moves dnum into the B-operand layout with two in-register lane swaps
//      per register (lane (token, kg) then holds features 32 ks + 8 kg +
//      0..7), and forms S dnum on the matrix cores, A = S rows read as one
//      16-byte piece per part; the output rows are chosen so that lane
//      (token, kg) receives query features 32 ks' + 8 kg + 0..7, the
//      features it loaded of q;
//   5. applies RoPE^T, adds dden z, masks by q > 0 and stores dq in q's
//      layout, and writes (den, dden) of its token.
template <int D>
__global__ __launch_bounds__(kTokThreads) void bwd_token_mfma_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ g,
    const uint16_t *__restrict__ dout, const float *__restrict__ states,
    const float2 *__restrict__ tab, uint16_t *__restrict__ dq, uint16_t *__restrict__ dg,
    float2 *__restrict__ dd, MArgs a) {
  constexpr int KS = D / 32;  // 32-feature contraction steps
  constexpr int ET = D / 16;  // 16-feature output tiles
  constexpr int NW = kTokThreads / 64;
  extern __shared__ __align__(16) unsigned char lds[];
  unsigned char *s_sh = lds;              // S hi, [p][e] (SRow)
  unsigned char *s_sl = lds + D * D * 2;  // S lo
  bf16x8 *s_zf = reinterpret_cast<bf16x8 *>(lds + D * D * 4);  // KS fragments x 64 lanes
  float *s_z = reinterpret_cast<float *>(s_zf + KS * 64);       // z (D)
  using St = Stage<D>;
  unsigned char *s_stage = reinterpret_cast<unsigned char *>(s_z + D);  // NW staging tiles
  float2 *s_tab = reinterpret_cast<float2 *>(s_stage + NW * St::kBytes);

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

  {
    // S (fp32, row-major) -> bf16 hi + lo in LDS; z fragments and z
    const float *ssrc = states + unit * (int64_t)(D * D + D);
    for (int i = tid; i < D * D / 4; i += kTokThreads) {
      const float4 x = reinterpret_cast<const float4 *>(ssrc)[i];
      const int p = (4 * i) / D, e0 = (4 * i) % D;
      uint32_t h0, l0, h1, l1;
      split_bf16x2(x.x, x.y, h0, l0);
      split_bf16x2(x.z, x.w, h1, l1);
      const int o = SRow<D>::off(p, e0 >> 3) + 2 * (e0 & 7);
      *reinterpret_cast<uint2 *>(s_sh + o) = make_uint2(h0, h1);
      *reinterpret_cast<uint2 *>(s_sl + o) = make_uint2(l0, l1);
    }
    const float *zsrc = ssrc + D * D;
    // rows 0, 4, 8, 12 of a fragment carry z rounded to bf16, rows 1, 5, 9,
    // 13 the rounding of the remainder: values 0 and 1 of every lane's
    // accumulator sum to ReLU(q) . z
    for (int i = tid; i < KS * 64; i += kTokThreads) {
      const int ks = i >> 6, l = i & 63, row = l & 15;
      bf16x8 f;
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = (__bf16)0.f;
      if ((row & 3) < 2) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float zv = zsrc[32 * ks + 8 * (l >> 4) + j];
          const __bf16 zh = (__bf16)zv;
          f[j] = (row & 1) ? (__bf16)(zv - (float)zh) : zh;
        }
      }
      s_zf[i] = f;
    }
    for (int i = tid; i < D; i += kTokThreads) s_z[i] = zsrc[i];
  }
  const TabSlice<D> ts = load_tab_slice<D>(s_tab, tab, a, n_begin, n_end);
  __syncthreads();

  // transposing-read offsets of the S^T fragments (num): as in the output stage
  int rd_s[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et)
    rd_s[et] = SRow<D>::off(8 * kg + (nl >> 2), 2 * et + ((nl & 3) >> 1)) + 8 * (nl & 1);
  // S-row reads of S dnum: output tile pt = 2 ks' + half, A row nl is S row
  // 32 ks' + 8 (nl / 4) + 4 half + nl % 4; the row's unit permutation depends
  // only on nl (row bits 0, 1 and 3), the tile adds a uniform row offset
  int srd[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) srd[ks] = SRow<D>::off(8 * (nl >> 2) + (nl & 3), 4 * ks + kg);

  const uint32_t row_bytes = (uint32_t)(a.H * D * 2);
  const int64_t head0 = (b * a.N * a.H + hd) * D;
  const uint16_t *q_head = q + head0, *g_head = g + head0, *d_head = dout + head0;
  uint16_t *dq_head = dq + head0, *dg_head = dg + head0;
  float2 *dd_head = dd + bh * a.N;

  // row-wise lane mapping of the staging tile: in pass i lane l covers token
  // i*kRowsPerPass + l/kLanesPerRow, features 8*(l%kLanesPerRow)..+7
  const int rl = lane / St::kLanesPerRow, rc = 8 * (lane % St::kLanesPerRow);
  // loads of one tile: q in the B-operand layout, g and dout as whole rows
  // (they pass through the staging tile into the accumulator layout)
  auto fetch = [&](int64_t tile, uint4 (&qr)[KS], uint4 (&gr)[St::kPasses],
                   uint4 (&dr)[St::kPasses]) {
    const __amdgpu_buffer_rsrc_t rq = tile_rsrc(q_head + tile * a.H * D, tile, n_end, row_bytes, D);
    const __amdgpu_buffer_rsrc_t rg = tile_rsrc(g_head + tile * a.H * D, tile, n_end, row_bytes, D);
    const __amdgpu_buffer_rsrc_t rd = tile_rsrc(d_head + tile * a.H * D, tile, n_end, row_bytes, D);
    const uint32_t qoff = (uint32_t)nl * row_bytes + 16 * kg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qr[ks] = buf_load16<kCacheNormal>(rq, qoff + 64 * ks);
#pragma unroll
    for (int i = 0; i < St::kPasses; ++i) {
      const uint32_t o = (uint32_t)(i * St::kRowsPerPass + rl) * row_bytes + 2 * rc;
      gr[i] = buf_load16<kCacheNormal>(rg, o);
      dr[i] = buf_load16<kCacheNormal>(rd, o);
    }
  };
  // a tile's rows (in row-wise registers) into the staging tile and back in
  // the accumulator layout: value et holds features 16 et + 4 kg + 0..3 of
  // token nl
  unsigned char *stage = s_stage + wave * St::kBytes;
  auto staged = [&](const uint4 (&rows)[St::kPasses], uint2 (&acc_layout)[ET]) {
#pragma unroll
    for (int i = 0; i < St::kPasses; ++i)
      *reinterpret_cast<uint4 *>(stage + (i * St::kRowsPerPass + rl) * St::kRowBytes + 2 * rc) =
          rows[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int et = 0; et < ET; ++et)
      acc_layout[et] =
          *reinterpret_cast<const uint2 *>(stage + nl * St::kRowBytes + 2 * (16 * et + 4 * kg));
    // the next writes into the tile must not overtake these reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  auto process = [&](int64_t tile, const uint4 (&cq)[KS], const uint4 (&gr)[St::kPasses],
                     const uint4 (&dr)[St::kPasses]) {
    // (an offset the compiler cannot see through keeps the loop-invariant
    // S reads inside the loop, as in the output stage)
    int opaque = 0;
    asm volatile("" : "+v"(opaque));
    const unsigned char *sh = s_sh + opaque, *sl = s_sl + opaque;
    const int64_t n = tile + nl;
    const bool valid = n < n_end;
    int t, h, w;
    token_pos(a, valid ? n : n_end - 1, t, h, w);

    // raised wave priority while this wave issues matrix-core products (as in
    // the output stage: the other wave of the SIMD fills the gaps with its
    // vector work)
    __builtin_amdgcn_s_setprio(1);
    // ---- num = x S and den on the matrix cores
    uint32_t qw[KS][4];  // ReLU(q), packed bf16
    f32x4 acc[ET], accd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int et = 0; et < ET; ++et) acc[et] = accd;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qw[ks][0] = relu_bf16x2(cq[ks].x);
      qw[ks][1] = relu_bf16x2(cq[ks].y);
      qw[ks][2] = relu_bf16x2(cq[ks].z);
      qw[ks][3] = relu_bf16x2(cq[ks].w);
      const bf16x8 bden =
          __builtin_bit_cast(bf16x8, make_uint4(qw[ks][0], qw[ks][1], qw[ks][2], qw[ks][3]));
      float x[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        x[2 * m] = lo_bf16(qw[ks][m]);
        x[2 * m + 1] = hi_bf16(qw[ks][m]);
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
      accd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s_zf[ks * 64 + lane], bden, accd, 0, 0, 0);
#pragma unroll
      for (int eg = 0; eg < ET; eg += 4) {
        bf16x8 ah[4], al[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int o0 = rd_s[eg + u] + (32 * ks) * (2 * D);
          const int o1 = o0 + 4 * (2 * D);
          const uint2 h0 = lds_read_tr16(sh + o0), h1 = lds_read_tr16(sh + o1);
          const uint2 l0 = lds_read_tr16(sl + o0), l1 = lds_read_tr16(sl + o1);
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
    __builtin_amdgcn_s_setprio(0);

    // ---- y, s, dg, dnum and dout s . y (value i of acc[et]: feature
    // 16 et + 4 kg + i of token nl)
    const float den = accd[0] + accd[1] + a.eps;
    const float inv_den = __builtin_amdgcn_rcpf(den);
    const __amdgpu_buffer_rsrc_t rdg = tile_rsrc(dg_head + tile * a.H * D, tile, n_end, row_bytes, D);
    uint2 cg[ET], cd[ET], dgw[ET];
    staged(gr, cg);
    staged(dr, cd);
    // dnum hi / lo, packed pairs: X from tile 2 ks (features 32 ks + 4 kg +
    // 0..3), Y from tile 2 ks + 1 (32 ks + 16 + 4 kg + 0..3)
    uint32_t xh[KS][2], yh[KS][2], xl[KS][2], yl[KS][2];
    float dyy = 0.f;
#pragma unroll
    for (int et = 0; et < ET; ++et) {
      const float gv[4] = {lo_bf16(cg[et].x), hi_bf16(cg[et].x), lo_bf16(cg[et].y),
                           hi_bf16(cg[et].y)};
      const float dv[4] = {lo_bf16(cd[et].x), hi_bf16(cd[et].x), lo_bf16(cd[et].y),
                           hi_bf16(cd[et].y)};
      // with s' = s / den: dnum = dout s', dout s . y = dnum num, and
      // dg = dout y s (1 - s) = (dnum num)(e s), since 1 - s = e s
      float dgo[4], dn[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __expf(-gv[i]);
        const float sg = __builtin_amdgcn_rcpf(1.f + e);
        dn[i] = dv[i] * (sg * inv_den);
        const float t = dn[i] * acc[et][i];
        dyy += t;
        dgo[i] = t * (e * sg);
      }
      dgw[et] = make_uint2(pack_bf16x2(dgo[0], dgo[1]), pack_bf16x2(dgo[2], dgo[3]));
      const int ks = et >> 1;
      if (et & 1) {
        split_bf16x2(dn[0], dn[1], yh[ks][0], yl[ks][0]);
        split_bf16x2(dn[2], dn[3], yh[ks][1], yl[ks][1]);
      } else {
        split_bf16x2(dn[0], dn[1], xh[ks][0], xl[ks][0]);
        split_bf16x2(dn[2], dn[3], xh[ks][1], xl[ks][1]);
      }
    }
    store_tile_rows<D>(stage, dgw, rdg, 0, row_bytes);
    // Transpose across the token's four lanes (rows of 16 lanes, row = kg):
    // row r needs X of rows 2r, 2r + 1 (r < 2) or Y of rows 2r - 4, 2r - 3.
    // A 32-lane swap of (X, Y) gives X' = (X0, X1, Y0, Y1), Y' = (X2, X3, Y2,
    // Y3) by row; a 16-lane swap of (X', Y') gives X'' = (X'0, Y'0, X'2, Y'2),
    // Y'' = (X'1, Y'1, X'3, Y'3): row kg then holds features 32 ks + 8 kg +
    // 0..3 in X'' and + 4..7 in Y''.
    auto transpose = [](uint32_t &x, uint32_t &y) {
      const auto s32 = __builtin_amdgcn_permlane32_swap(x, y, false, false);
      const auto s16 = __builtin_amdgcn_permlane16_swap(s32[0], s32[1], false, false);
      x = s16[0];
      y = s16[1];
    };
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int w2 = 0; w2 < 2; ++w2) {
        transpose(xh[ks][w2], yh[ks][w2]);
        transpose(xl[ks][w2], yl[ks][w2]);
      }
    // the token's other three lanes hold the rest of its features (lanes
    // l ^ 16, l ^ 32, l ^ 48): two in-register exchanges (gfx950
    // permlane16/32 swap, each returning this lane's and its partner's value)
    {
      const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(dyy),
                                                        __float_as_uint(dyy), false, false);
      dyy = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
      const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(dyy),
                                                        __float_as_uint(dyy), false, false);
      dyy = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
    }
    const float dden = -dyy * inv_den;

    // ---- S dnum on the matrix cores: A = S rows (16-byte pieces), B =
    // dnum (features 32 ks + 8 kg + 0..7); output tile pt = 2 ks' + half
    __builtin_amdgcn_s_setprio(1);
    f32x4 acc2[ET];
#pragma unroll
    for (int pt = 0; pt < ET; ++pt) acc2[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 bnh = __builtin_bit_cast(bf16x8, make_uint4(xh[ks][0], xh[ks][1], yh[ks][0], yh[ks][1]));
      const bf16x8 bnl = __builtin_bit_cast(bf16x8, make_uint4(xl[ks][0], xl[ks][1], yl[ks][0], yl[ks][1]));
#pragma unroll
      for (int pg = 0; pg < ET; pg += 4) {
        bf16x8 ah[4], al[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int pt = pg + u;
          const int ro = (32 * (pt >> 1) + 4 * (pt & 1)) * (2 * D);
          ah[u] = *reinterpret_cast<const bf16x8 *>(sh + ro + srd[ks]);
          al[u] = *reinterpret_cast<const bf16x8 *>(sl + ro + srd[ks]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc2[pg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[u], bnl, acc2[pg + u], 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc2[pg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[u], bnh, acc2[pg + u], 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc2[pg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[u], bnh, acc2[pg + u], 0, 0, 0);
      }
    }
    mfma_drain();
    __builtin_amdgcn_s_setprio(0);

    // ---- dq = [RoPE^T(S dnum) + dden z] * 1[q > 0], in q's layout: lane
    // (token, kg) holds features 32 ks' + 8 kg + 4 half + i in acc2[2 ks' + half][i]
    const __amdgpu_buffer_rsrc_t rdq = tile_rsrc(dq_head + tile * a.H * D, tile, n_end, row_bytes, D);
    const uint32_t qoff = (uint32_t)nl * row_bytes + 16 * kg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      int axis, pia;
      pair_axis<D>(16 * ks + 4 * kg, axis, pia);
      float2 c4[4];
      ts.read(s_tab, ts.lookup(axis, pia).at(t, h, w), c4);
      const float4 z0 = *reinterpret_cast<const float4 *>(s_z + 32 * ks + 8 * kg);
      const float4 z1 = *reinterpret_cast<const float4 *>(s_z + 32 * ks + 8 * kg + 4);
      const float dz[8] = {dden * z0.x, dden * z0.y, dden * z0.z, dden * z0.w,
                           dden * z1.x, dden * z1.y, dden * z1.z, dden * z1.w};
      buf_store16<kCacheNormal>(rdq, qoff + 64 * ks,
                                rope_t_add_mask(acc2[2 * ks], acc2[2 * ks + 1], c4, dz, qw[ks]));
    }
    if (valid && kg == 0) dd_head[n] = make_float2(den, dden);
  };

  // Tiles wave, wave + NW, ... of the range, two in flight per wave (as in
  // the output stage: unconditional refills, tiles past the range read as
  // zeros and are never processed).
  const int64_t kStep = 16 * NW;
  uint4 qa[KS], qb[KS];
  uint4 ga[St::kPasses], da[St::kPasses], gb[St::kPasses], db[St::kPasses];
  int64_t tile = n_begin + 16 * wave;
  fetch(tile, qa, ga, da);
  asm volatile("" ::: "memory");
  fetch(tile + kStep, qb, gb, db);
  while (tile < n_end) {
    process(tile, qa, ga, da);
    fetch(tile + 2 * kStep, qa, ga, da);
    if (tile + kStep < n_end) process(tile + kStep, qb, gb, db);
    fetch(tile + 3 * kStep, qb, gb, db);
    tile += 2 * kStep;
  }
  __builtin_amdgcn_s_waitcnt(0);  // prefetches past the range are still in flight
}

// ---------------------------------------------------------------- state pass

// Workgroups of the state pass: twelve waves at d = 128 (one workgroup per
// compute unit), six at d = 64; two thirds producers, one third matrix-core
// consumers (waves w, w + NWV/3 and w + 2 NWV/3 share a SIMD), as in the
// forward's state stage, with 32-token steps: a step's operand set holds
// four tiles (x hi, x lo, dnum hi, dnum lo).
template <int D>
constexpr int kDsThreads = D == 128 ? 768 : 384;
constexpr int kDsStep = 32;      // tokens per step
constexpr int kDsPrefetch = 2;   // steps of rows in flight per producer thread

template <int D>
struct DsCfg {
  static constexpr int NT = kDsThreads<D>;
  static constexpr int NWV = NT / 64;
  static constexpr int NCW = NWV / 3;
  static constexpr int NPW = NWV - NCW;
  static constexpr int FPT = D / 8;              // threads per token row (16 B each)
  static constexpr int TPP = NPW * 64 / FPT;     // tokens per load pass
  static constexpr int TPW = D / 32;             // 32x32 tiles per consumer wave
  static constexpr int ROW = 2 * D;
  static constexpr int OP_BYTES = kDsStep * ROW;
  static constexpr int SET_BYTES = 4 * OP_BYTES;
  static constexpr int POS_BYTES = kDsStep * 16;
  static_assert(NCW * 32 == D, "consumer wave w owns rows 32w.. of dS");
  static_assert(TPP == kDsStep, "one load pass per step");
  // 16-byte units of a tile row XOR-permuted by the row (as in the forward
  // state stage)
  static __device__ __forceinline__ int swz(int row) {
    return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
  }
  static __device__ __forceinline__ int off(int row, int unit) {
    return row * ROW + ((unit ^ swz(row)) << 4);
  }
};

// One workgroup per (unit, chunk), with one barrier per 32-token step.  In
// round i the producers take step i's rows of q, g and dout (and each token's
// den, dden from the token pass) from registers, form x = RoPE(ReLU(q)) split
// into bf16 hi + lo, dnum = dout s / den split into hi + lo, and
// dz += dden ReLU(q), write the four tiles into LDS set i % 2 and refill
// their registers two steps ahead; the consumers accumulate rows 32 cw.. of
// dS = x^T dnum from set (i - 1) % 2 (x hi^T dnum lo
// + x lo^T dnum hi + x hi^T dnum hi, v_mfma_f32_32x32x16_bf16, transposing
// LDS reads of both operands), and consumer 0 writes step i + 1's token
// positions.  The chunk's partial (dS row-major [p][e], then dz) is written
// for the block sums.
template <int D>
__global__ __launch_bounds__(kDsThreads<D>, 3) void bwd_dstate_mfma_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ g,
    const uint16_t *__restrict__ dout, const float2 *__restrict__ dd,
    const float2 *__restrict__ tab, float *__restrict__ partials, MArgs a) {
  using Cfg = DsCfg<D>;
  constexpr int FPT = Cfg::FPT, TPP = Cfg::TPP, ROW = Cfg::ROW, TPW = Cfg::TPW;
  constexpr int P = kDsPrefetch;
  extern __shared__ __align__(16) unsigned char lds[];
  unsigned char *s_pos = lds + 2 * Cfg::SET_BYTES;
  float2 *s_tab = reinterpret_cast<float2 *>(s_pos + 2 * Cfg::POS_BYTES);

  const int64_t wg = blockIdx.x;
  const int64_t unit = wg / a.C, c = wg % a.C;
  const int64_t bh = unit / a.nb, blk = unit % a.nb;
  const int64_t b = bh / a.H, hd = bh % a.H;
  const int64_t n_begin = blk * a.L + c * a.Lc;
  const int64_t n_end = min(n_begin + a.Lc, (blk + 1) * a.L);
  const int64_t steps = (n_end - n_begin + kDsStep - 1) / kDsStep;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wave < Cfg::NPW;

  // producers: token row tg of a step, 16-byte unit fc
  const int fc = tid % FPT, tg = (tid / FPT) % TPP;
  const int wr_off = Cfg::off(tg, fc);

  // consumers: rows 32 cw.. of dS; transposing-read offsets as in the
  // forward state stage (A from the x tiles at feature column 32 cw, B from
  // the dnum tiles at feature column 32 t)
  const int cw = producer ? 0 : wave - Cfg::NPW;
  int rd_p, rd_e[TPW];
  {
    const int gq = lane >> 4, sl = lane & 15;
    const int rrow = 8 * (gq >> 1) + (sl >> 2);
    const int cp = 32 * cw + 16 * (gq & 1) + 4 * (sl & 3);
    rd_p = Cfg::off(rrow, cp >> 3) + ((cp & 7) << 1);
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int ce = 32 * t + 16 * (gq & 1) + 4 * (sl & 3);
      rd_e[t] = Cfg::off(rrow, ce >> 3) + ((ce & 7) << 1);
    }
  }

  const int64_t first = ((b * a.N + n_begin) * a.H + hd) * D;
  const uint32_t row_bytes = (uint32_t)(a.H * D * 2);
  const uint32_t range_bytes = (uint32_t)(n_end - n_begin - 1) * row_bytes + 2 * D;
  const __amdgpu_buffer_rsrc_t rq = head_rows_rsrc(q + first, range_bytes);
  const __amdgpu_buffer_rsrc_t rg = head_rows_rsrc(g + first, range_bytes);
  const __amdgpu_buffer_rsrc_t rdo = head_rows_rsrc(dout + first, range_bytes);
  // (den, dden) of the chunk's tokens: 8 bytes each, contiguous per head
  const __amdgpu_buffer_rsrc_t rdd = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float2 *>(dd + bh * a.N + n_begin), 0, (int)((n_end - n_begin) * 8), 0x00020000);
  const uint32_t my_off = (uint32_t)tg * row_bytes + 16 * fc;

  uint4 qr[P], gr[P], dr[P];
  float2 ddr[P];
  auto load_rows = [&](auto js, int64_t n0) {
    constexpr int j = decltype(js)::value;
    const uint32_t base = (uint32_t)(n0 - n_begin) * row_bytes + my_off;
    qr[j] = buf_load16<kCacheStream>(rq, base);
    gr[j] = buf_load16<kCacheStream>(rg, base);
    dr[j] = buf_load16<kCacheStream>(rdo, base);
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(
        rdd, (int)(((uint32_t)(n0 - n_begin) + tg) * 8u), 0, kCacheNormal);
    ddr[j] = make_float2(__uint_as_float(v.x), __uint_as_float(v.y));
  };
  constexpr int gt = D / 32, gh = 3 * D / 64;
  auto write_pos = [&](int64_t i) {
    if (lane < kDsStep) {
      int64_t n = n_begin + i * kDsStep + lane;
      if (n >= n_end) n = n_end - 1;
      int t, h, w;
      token_pos(a, n, t, h, w);
      *reinterpret_cast<int4 *>(s_pos + (int)(i & 1) * Cfg::POS_BYTES + 16 * lane) =
          make_int4(t * gt, h * gh, w * gh, 0);
    }
  };

  TabLoad<D> tload;
  tload.issue(tab, a, n_begin, n_end);
  asm volatile("" ::: "memory");
  if (producer) {
    load_rows(std::integral_constant<int, 0>{}, n_begin);
    load_rows(std::integral_constant<int, 1>{}, n_begin + kDsStep);
  }
  asm volatile("" ::: "memory");
  tload.store(s_tab, tab);
  if (!producer && cw == 0) write_pos(0);
  int axis, pia;
  pair_axis<D>(4 * fc, axis, pia);
  const int tab_base = tload.ts.lookup(axis, pia).base;
  const TabSlice<D> ts = tload.ts;
  __syncthreads();

  f32x16 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
  float dzacc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) dzacc[j] = 0.f;

  if (producer) {
    auto round = [&](auto js, int64_t i) {
      constexpr int j = decltype(js)::value;
      if (i < steps) {
        unsigned char *s_xh = lds + (int)(i & 1) * Cfg::SET_BYTES;
        unsigned char *s_xl = s_xh + Cfg::OP_BYTES;
        unsigned char *s_nh = s_xh + 2 * Cfg::OP_BYTES;
        unsigned char *s_nl = s_xh + 3 * Cfg::OP_BYTES;
        const int *pos = reinterpret_cast<const int *>(s_pos + (int)(i & 1) * Cfg::POS_BYTES);
        const int64_t n0 = n_begin + i * kDsStep;
        const int grp = tab_base + pos[4 * tg + axis];
        const uint32_t qw[4] = {relu_bf16x2(qr[j].x), relu_bf16x2(qr[j].y),
                                relu_bf16x2(qr[j].z), relu_bf16x2(qr[j].w)};
        const float dden = ddr[j].y;
        float x[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          x[2 * m] = lo_bf16(qw[m]);
          x[2 * m + 1] = hi_bf16(qw[m]);
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) dzacc[m] = __builtin_fmaf(dden, x[m], dzacc[m]);
        float2 c4[4];
        ts.read(s_tab, grp, c4);
        rotate4(x, c4);
        uint4 xh, xl;
        split_bf16x2(x[0], x[1], xh.x, xl.x);
        split_bf16x2(x[2], x[3], xh.y, xl.y);
        split_bf16x2(x[4], x[5], xh.z, xl.z);
        split_bf16x2(x[6], x[7], xh.w, xl.w);
        // dnum = dout s / den = dout / (den (1 + exp(-g))); rows past the
        // chunk read den and dout as 0, and take den = 1 so that their dnum
        // is 0 (0 / 0 would put NaN into every element of dS)
        const bool valid = n0 + tg < n_end;
        const float den = valid ? ddr[j].x : 1.f;
        const uint32_t gw[4] = {gr[j].x, gr[j].y, gr[j].z, gr[j].w};
        const uint32_t dw[4] = {dr[j].x, dr[j].y, dr[j].z, dr[j].w};
        float dn[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float e0 = __expf(-lo_bf16(gw[m])), e1 = __expf(-hi_bf16(gw[m]));
          dn[2 * m] = lo_bf16(dw[m]) * __builtin_amdgcn_rcpf(__builtin_fmaf(den, e0, den));
          dn[2 * m + 1] = hi_bf16(dw[m]) * __builtin_amdgcn_rcpf(__builtin_fmaf(den, e1, den));
        }
        uint4 nh, nlo;
        split_bf16x2(dn[0], dn[1], nh.x, nlo.x);
        split_bf16x2(dn[2], dn[3], nh.y, nlo.y);
        split_bf16x2(dn[4], dn[5], nh.z, nlo.z);
        split_bf16x2(dn[6], dn[7], nh.w, nlo.w);
        *reinterpret_cast<uint4 *>(s_xh + wr_off) = xh;
        *reinterpret_cast<uint4 *>(s_xl + wr_off) = xl;
        *reinterpret_cast<uint4 *>(s_nh + wr_off) = nh;
        *reinterpret_cast<uint4 *>(s_nl + wr_off) = nlo;
        load_rows(js, n0 + P * kDsStep);
      }
      __syncthreads();
    };
    for (int64_t i = 0; i <= steps; i += P) {
      round(std::integral_constant<int, 0>{}, i);
      if (i + 1 > steps) break;
      round(std::integral_constant<int, 1>{}, i + 1);
    }
  } else {
    for (int64_t i = 0; i <= steps; ++i) {
      if (cw == 0 && i + 1 < steps) write_pos(i + 1);
      if (i >= 1) {
        const unsigned char *s_xh = lds + (int)((i - 1) & 1) * Cfg::SET_BYTES;
        const unsigned char *s_xl = s_xh + Cfg::OP_BYTES;
        const unsigned char *s_nh = s_xh + 2 * Cfg::OP_BYTES;
        const unsigned char *s_nl = s_xh + 3 * Cfg::OP_BYTES;
#pragma unroll
        for (int ks = 0; ks < kDsStep / 16; ++ks) {
          const int o0 = (16 * ks) * ROW, o1 = (16 * ks + 4) * ROW;
          const uint2 h0 = lds_read_tr16(s_xh + rd_p + o0), h1 = lds_read_tr16(s_xh + rd_p + o1);
          const uint2 l0 = lds_read_tr16(s_xl + rd_p + o0), l1 = lds_read_tr16(s_xl + rd_p + o1);
          const bf16x8 fa = __builtin_bit_cast(bf16x8, make_uint4(h0.x, h0.y, h1.x, h1.y));
          const bf16x8 fl = __builtin_bit_cast(bf16x8, make_uint4(l0.x, l0.y, l1.x, l1.y));
          bf16x8 fbh[TPW], fbl[TPW];
#pragma unroll
          for (int t = 0; t < TPW; ++t) {
            const uint2 v0 = lds_read_tr16(s_nh + rd_e[t] + o0), v1 = lds_read_tr16(s_nh + rd_e[t] + o1);
            const uint2 w0 = lds_read_tr16(s_nl + rd_e[t] + o0), w1 = lds_read_tr16(s_nl + rd_e[t] + o1);
            fbh[t] = __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
            fbl[t] = __builtin_bit_cast(bf16x8, make_uint4(w0.x, w0.y, w1.x, w1.y));
          }
#pragma unroll
          for (int t = 0; t < TPW; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fl, fbh[t], acc[t], 0, 0, 0);
#pragma unroll
          for (int t = 0; t < TPW; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fbl[t], acc[t], 0, 0, 0);
#pragma unroll
          for (int t = 0; t < TPW; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fbh[t], acc[t], 0, 0, 0);
        }
      }
      __syncthreads();
    }
  }
  mfma_drain();

  // the chunk's partial: dS row-major [p][e] (consumers), then dz summed over
  // the token groups in a fixed order (the operand sets are no longer read)
  float *dst = partials + wg * (int64_t)(D * D + D);
  float *zs = reinterpret_cast<float *>(lds);
  if (producer) {
#pragma unroll
    for (int j = 0; j < 8; ++j) zs[tg * D + 8 * fc + j] = dzacc[j];
  } else {
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int p = 32 * cw + 8 * i4 + 4 * (lane >> 5);
        const int e = 32 * t + (lane & 31);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(p + i) * D + e] = acc[t][4 * i4 + i];
      }
  }
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
    for (int gidx = 0; gidx < TPP; ++gidx) s += zs[gidx * D + tid];
    dst[D * D + tid] = s;
  }
  __builtin_amdgcn_s_waitcnt(0);  // prefetches past the chunk are still in flight
}

template <int D>
size_t token_lds(const Plan &p) {
  return (size_t)D * D * 4 + (size_t)(D / 32) * 64 * 16 + (size_t)D * 4 +
         (size_t)(kTokThreads / 64) * Stage<D>::kBytes +
         (size_t)tab_slice_entries(p, p.Lr) * sizeof(float2);
}
template <int D>
size_t dstate_lds(const Plan &p) {
  return 2 * (size_t)(DsCfg<D>::SET_BYTES + DsCfg<D>::POS_BYTES) +
         (size_t)tab_slice_entries(p, p.Lc) * sizeof(float2);
}

template <int D>
hipError_t token_d(const Plan &p, const void *q, const void *g, const void *dout,
                   const float *states, const float2 *tab, void *dq, void *dg, float2 *dd,
                   hipStream_t stream) {
  auto kern = bwd_token_mfma_kernel<D>;
  hipError_t e = lds_limit_once((const void *)kern);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.units * p.R)), dim3(kTokThreads), token_lds<D>(p),
                     stream, (const uint16_t *)q, (const uint16_t *)g, (const uint16_t *)dout,
                     states, tab, (uint16_t *)dq, (uint16_t *)dg, dd, make_margs(p));
  return hipGetLastError();
}

template <int D>
hipError_t dstate_d(const Plan &p, const void *q, const void *g, const void *dout,
                    const float2 *dd, const float2 *tab, float *partials, hipStream_t stream) {
  auto kern = bwd_dstate_mfma_kernel<D>;
  hipError_t e = lds_limit_once((const void *)kern);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.units * p.C)), dim3(DsCfg<D>::NT), dstate_lds<D>(p),
                     stream, (const uint16_t *)q, (const uint16_t *)g, (const uint16_t *)dout, dd,
                     tab, partials, make_margs(p));
  return hipGetLastError();
}

}  // namespace

size_t bwd_query_lds_bytes(const Plan &p) {
  if (p.d == 128) return std::max(token_lds<128>(p), dstate_lds<128>(p));
  if (p.d == 64) return std::max(token_lds<64>(p), dstate_lds<64>(p));
  return 0;
}

hipError_t backward_query_lds_limits() {
  return lds_limits({(const void *)bwd_token_mfma_kernel<128>,
                     (const void *)bwd_token_mfma_kernel<64>,
                     (const void *)bwd_dstate_mfma_kernel<128>,
                     (const void *)bwd_dstate_mfma_kernel<64>});
}

hipError_t launch_bwd_token_mfma(const Plan &p, const void *q, const void *g, const void *dout,
                                 const float *states, const float2 *tab, void *dq, void *dg,
                                 float2 *dd, hipStream_t stream) {
  if (p.d == 128) return token_d<128>(p, q, g, dout, states, tab, dq, dg, dd, stream);
  if (p.d == 64) return token_d<64>(p, q, g, dout, states, tab, dq, dg, dd, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dstate_mfma(const Plan &p, const void *q, const void *g, const void *dout,
                                  const float2 *dd, const float2 *tab, float *partials,
                                  hipStream_t stream) {
  if (p.d == 128) return dstate_d<128>(p, q, g, dout, dd, tab, partials, stream);
  if (p.d == 64) return dstate_d<64>(p, q, g, dout, dd, tab, partials, stream);
  return hipErrorInvalidValue;
}

}  // namespace gla
