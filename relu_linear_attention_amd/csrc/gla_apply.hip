// Output stage of the operator on the matrix cores (bf16, head size 64 or
// 128; gfx950, v_mfma_f32_16x16x32_bf16 with fp32 accumulation):
//
//   o_i = (RoPE_i(phi(q_i)) S) / (phi(q_i) . z + eps) * sigmoid(g_i)
//
// "SANA-Video" notes page, Section 3.2 (phi = ReLU, RoPE after ReLU in the
// numerator only, the un-rotated denominator); "SANA-Video 2.0" Section 2
// Eq. (1) (+eps and the sigmoid output gate; the optional RMSNorm of num/den
// before the gate).
//
// Work layout.  A workgroup is eight waves, two per SIMD of a compute unit,
// and owns a group of up to four heads of one (batch, temporal block).  The
// waves form four pairs; a pair takes one head and one 16-token tile per
// item, and each wave of the pair keeps half of that head's transposed
// state, S^T split into bf16 hi + lo parts, in registers as matrix-core A
// operands (128 registers at d = 128): wave half s produces output features
// [s d/2, (s+1) d/2) of all 16 tokens.  The items of a block are dealt to the
// workgroups of its head group in turn (workgroup s of m takes items s,
// s + m, s + 2m, ...), so that at any moment the workgroups of every head
// read and write neighbouring tokens: all heads of a token row are touched
// together, which keeps HBM pages open, where contiguous token ranges per
// workgroup left hundreds of streams far apart.  q, g and out move as whole
// 2d-byte rows with the non-temporal hint; nothing here is read twice.
//
// Per tile: each wave of the pair loads 8 of the 16 q and g rows (two tiles
// ahead) and, in the row layout, computes ReLU(q), the denominator phi(q).z
// (a sum over the row's lanes), RoPE and the hi/lo split, writing
// RoPE(phi(q)) hi/lo and g into the pair's LDS tiles; after a workgroup
// barrier both waves read all 16 tokens in the B-operand layout, accumulate
// their half of num = S^T (qh + ql) with three products (hi.hi, hi.lo,
// lo.hi), read g in the accumulator layout and write o = num / (den (1 +
// e^-g)) back in place; after a second barrier each wave stores its 8 rows
// whole.  The pair's tiles are double-buffered, so two barriers per tile
// suffice.
//
// 16x16x32 operand layout (lane l of 64):
//   A (16 x 32):  lane l holds A[l % 16][8*(l/16) + j], j = 0..7
//   B (32 x 16):  lane l holds B[8*(l/16) + j][l % 16]
//   C (16 x 16):  lane l, value i holds C[4*(l/16) + i][l % 16]
// With A = S^T (rows e, columns p), B = RoPE(phi(q))^T (rows p, columns
// tokens) and C = num^T (rows e, columns tokens).

#include <hip/hip_runtime.h>

#include <algorithm>

#include "gla_mfma_common.h"

namespace gla {
namespace {

constexpr int kApplyWaves = 8;  // four pairs
constexpr int kApplyPairs = 4;

template <int D>
struct ApplyCfg {
  static constexpr int KS = D / 32;          // 32-feature contraction steps
  static constexpr int ET = D / 16;          // 16-feature output tiles
  static constexpr int EH = ET / 2;          // output tiles of one wave (its half)
  static constexpr int NFRAG = 2 * KS * EH;  // A fragments of a wave's half of S^T (hi, lo)
  static constexpr int LPR = D / 8;          // lanes per token row, 16 B each
  static constexpr int RPI = 64 / LPR;       // token rows per load instruction
  static constexpr int NI = 16 / RPI;        // load instructions per 16-row tile
  static constexpr int NH = NI / 2 > 0 ? NI / 2 : 1;  // ... per wave (its 8 rows)
  static constexpr int QROW = 2 * D;         // bytes of one staged row of one part
  static constexpr int QPART = 16 * QROW;    // one part (hi or lo) of the staged q tile
  // one buffer of a pair: q hi, q lo, 16 denominators, 2 x 16 RMS partial
  // sums, the g/out staging tile
  static constexpr int kBufBytes = 2 * QPART + 64 + 128 + Stage<D>::kBytes;
  static constexpr int kPairBytes = 2 * kBufBytes;  // double-buffered
  // 16-byte units of a staged q row are XOR-permuted by qswz(row) so that the
  // B-operand reads (16 rows, one unit each, per 16 lanes) and the row
  // writes both spread over all banks
  static __device__ __forceinline__ int qswz(int row) {
    return D == 128 ? (row & 15) : ((row >> 1) & 7);
  }
  static __device__ __forceinline__ int qoff(int row, int unit) {
    return row * QROW + ((unit ^ qswz(row)) << 4);
  }
};

// Buffer resource over the rows [n, n + 16) of one head that lie inside
// [.., n_end): rows past n_end (and whole tiles past it) read as zeros and
// are not written.  `base` points at feature 0 of row n.
// Every input is uniform across the wave; the values pass through
// readfirstlane so that the compiler keeps the descriptor in scalar
// registers (a descriptor it believes divergent costs a loop around every
// access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t *base, int64_t n,
                                                            int64_t n_end, uint32_t row_bytes,
                                                            int D) {
  const int64_t left = n_end - n;
  const uint32_t rows = left <= 0 ? 0u : (left >= 16 ? 16u : (uint32_t)left);
  const uint32_t bytes = __builtin_amdgcn_readfirstlane(
      rows == 0 ? 0u : (rows - 1) * row_bytes + 2u * (uint32_t)D);
  const uint64_t addr = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
  const uint16_t *p = (const uint16_t *)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(p), 0, (int)bytes,
                                           0x00020000);
}

// Sum over the lanes of each 16-lane row (D = 128: a token row) or each
// 8-lane half row (D = 64), left in every lane of it, by DPP lane moves.
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, true));
}
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_mov<0x141>(x);  // row_half_mirror: the other quad of each 8 lanes
  if (LPR == 16) x += dpp_mov<0x140>(x);  // row_mirror: the other 8 lanes of the row
  return x;
}

template <int D, bool kNorm>
__global__ __launch_bounds__(kApplyWaves * 64, 1) void apply_reg_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ g,
    const float *__restrict__ states, const uint16_t *__restrict__ frags,
    const float2 *__restrict__ tab, const uint16_t *__restrict__ rms_w,
    uint16_t *__restrict__ out, MArgs a) {
  using Cfg = ApplyCfg<D>;
  using St = Stage<D>;
  constexpr int KS = Cfg::KS, ET = Cfg::ET, EH = Cfg::EH, LPR = Cfg::LPR, RPI = Cfg::RPI;
  constexpr int NH = Cfg::NH;
  extern __shared__ __align__(16) unsigned char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave % kApplyPairs, half = wave / kApplyPairs;
  unsigned char *s_pair = lds + pair * Cfg::kPairBytes;
  float *s_w = reinterpret_cast<float *>(lds + kApplyPairs * Cfg::kPairBytes);  // D floats
  float2 *s_tab = reinterpret_cast<float2 *>(s_w + D);

  // workgroup -> (head group, super-range, slot); pair -> (head, tile of the item)
  const int64_t wg = blockIdx.x;
  const int64_t grp = wg % a.ag;
  const int64_t rest = wg / a.ag;
  const int64_t sr = rest / a.am, slot = rest % a.am;
  const int64_t hg = grp % (a.H / a.hpw);
  const int64_t bb = grp / (a.H / a.hpw);  // (batch, block)
  const int64_t b = bb / a.nb, blk = bb % a.nb;
  const int hw = pair % a.hpw, tw = pair / a.hpw;
  const int64_t hd = hg * a.hpw + hw;
  const int64_t unit = (b * a.H + hd) * a.nb + blk;
  const int item_tokens = 16 * (kApplyPairs / a.hpw);
  const int64_t blk_begin = blk * a.L, blk_end = blk_begin + a.L;
  const int64_t sr_begin = blk_begin + sr * a.air * item_tokens;
  const int64_t sr_end = min(blk_end, sr_begin + a.air * item_tokens);

  // this wave's half of S^T: fragments (part, ks, et) for et in [half*EH, half*EH + EH)
  // of frags[unit][part][ks][et][lane][8]
  bf16x8 sf[Cfg::NFRAG];
  {
    const uint4 *src = reinterpret_cast<const uint4 *>(frags + unit * (int64_t)(2 * KS * ET) * 512);
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < EH; ++e)
          sf[(pt * KS + ks) * EH + e] =
              __builtin_bit_cast(bf16x8, src[((pt * KS + ks) * ET + half * EH + e) * 64 + lane]);
  }
  // z entries of this lane's eight features (its 16-byte unit of a row)
  const int fc = lane % LPR, rl = lane / LPR;
  float zr[8];
  {
    const float4 *zs = reinterpret_cast<const float4 *>(states + unit * (int64_t)(D * D + D) +
                                                        D * D + 8 * fc);
    const float4 z0 = zs[0], z1 = zs[1];
    zr[0] = z0.x; zr[1] = z0.y; zr[2] = z0.z; zr[3] = z0.w;
    zr[4] = z1.x; zr[5] = z1.y; zr[6] = z1.z; zr[7] = z1.w;
  }
  if (kNorm)
    for (int i = tid; i < D; i += kApplyWaves * 64) s_w[i] = bf16_bits_to_float(rms_w[i]);
  const TabSlice<D> ts = load_tab_slice<D>(s_tab, tab, a, sr_begin, sr_end);
  __syncthreads();

  int axis, pia;
  pair_axis<D>(4 * fc, axis, pia);
  const typename TabSlice<D>::Lookup tl = ts.lookup(axis, pia);
  const int nl = lane & 15, kg = lane >> 4;
  const uint32_t row_bytes = (uint32_t)(a.H * D * 2);
  const uint16_t *q_head = q + (b * a.N * a.H + hd) * D;
  const uint16_t *g_head = g + (b * a.N * a.H + hd) * D;
  uint16_t *o_head = out + (b * a.N * a.H + hd) * D;
  // this wave's rows of a tile: rl + RPI * (half * NH + j), j < NH (D = 64:
  // one instruction covers 8 rows, the wave's half of the tile)
  const int row0 = rl + RPI * half * NH;
  const uint32_t lane_off = (uint32_t)row0 * row_bytes + 16 * fc;

  auto tile_of = [&](int64_t it) -> int64_t { return sr_begin + it * item_tokens + 16 * tw; };
  auto fetch = [&](int64_t n0, uint4 (&qv)[NH], uint4 (&gv)[NH]) {
    const int64_t e = n0 * a.H * D;
    const __amdgpu_buffer_rsrc_t rq = tile_rsrc(q_head + e, n0, sr_end, row_bytes, D);
    const __amdgpu_buffer_rsrc_t rg = tile_rsrc(g_head + e, n0, sr_end, row_bytes, D);
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      qv[j] = buf_load16<kCacheStream>(rq, lane_off + (uint32_t)(RPI * j) * row_bytes);
      gv[j] = buf_load16<kCacheStream>(rg, lane_off + (uint32_t)(RPI * j) * row_bytes);
    }
  };

  // LDS of buffer `buf` of this pair
  auto bufp = [&](int buf) { return s_pair + buf * Cfg::kBufBytes; };
  auto s_den_of = [&](int buf) { return reinterpret_cast<float *>(bufp(buf) + 2 * Cfg::QPART); };
  auto s_stage_of = [&](int buf) { return bufp(buf) + 2 * Cfg::QPART + 64 + 128; };

  // Row work of row-instruction j of a tile: ReLU, denominator, RoPE, hi/lo
  // split into the q tiles; g into the staging tile.
  auto rows = [&](int64_t n0, int buf, int j, uint4 qv, uint4 gv) {
    unsigned char *s_qh = bufp(buf);
    unsigned char *s_ql = s_qh + Cfg::QPART;
    const int row = row0 + RPI * j;
    int64_t n = n0 + row;
    if (n >= sr_end) n = sr_end - 1;  // position only; the row reads as zero
    int t, h, w;
    token_pos(a, n, t, h, w);
    const uint32_t qw[4] = {relu_bf16x2(qv.x), relu_bf16x2(qv.y), relu_bf16x2(qv.z),
                            relu_bf16x2(qv.w)};
    float x[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      x[2 * m] = lo_bf16(qw[m]);
      x[2 * m + 1] = hi_bf16(qw[m]);
    }
    float dp = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) dp = __builtin_fmaf(x[i], zr[i], dp);
    dp = row_sum<LPR>(dp);
    // every lane of the row holds the same sum; all of them write it (a
    // branch here would split the scheduling region that interleaves this
    // work with the matrix-core products)
    s_den_of(buf)[row] = dp;
    float2 c4[4];
    ts.read(s_tab, tl.at(t, h, w), c4);
    rotate4(x, c4);
    uint4 hi, lo;
    split_bf16x2(x[0], x[1], hi.x, lo.x);
    split_bf16x2(x[2], x[3], hi.y, lo.y);
    split_bf16x2(x[4], x[5], hi.z, lo.z);
    split_bf16x2(x[6], x[7], hi.w, lo.w);
    *reinterpret_cast<uint4 *>(s_qh + Cfg::qoff(row, fc)) = hi;
    *reinterpret_cast<uint4 *>(s_ql + Cfg::qoff(row, fc)) = lo;
    *reinterpret_cast<uint4 *>(s_stage_of(buf) + row * St::kRowBytes + 16 * fc) = gv;
  };

  // One contraction step of this wave's half of num^T = S^T RoPE(phi(q))^T
  // (three products: hi.lo, lo.hi, hi.hi) for the tile in buffer `buf`.
  auto mma_step = [&](int buf, int ks, f32x4 (&acc)[EH]) {
    const unsigned char *s_qh = bufp(buf);
    const int u = 4 * ks + kg;
    const bf16x8 bh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(s_qh + Cfg::qoff(nl, u)));
    const bf16x8 bl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(s_qh + Cfg::QPART + Cfg::qoff(nl, u)));
#pragma unroll
    for (int e = 0; e < EH; ++e)
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[(0 * KS + ks) * EH + e], bl, acc[e], 0, 0, 0);
#pragma unroll
    for (int e = 0; e < EH; ++e)
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[(1 * KS + ks) * EH + e], bh, acc[e], 0, 0, 0);
#pragma unroll
    for (int e = 0; e < EH; ++e)
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[(0 * KS + ks) * EH + e], bh, acc[e], 0, 0, 0);
  };

  // The products of the tile in `buf` interleaved with the row work of the
  // next tile (into the other buffer): the matrix cores run while the
  // vector units prepare the next tile.
  auto mma_and_rows = [&](int buf, f32x4 (&acc)[EH], bool rows_next, int64_t n_next,
                          const uint4 (&qv)[NH], const uint4 (&gv)[NH]) {
#pragma unroll
    for (int e = 0; e < EH; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int NS = KS > NH ? KS : NH;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s < KS) mma_step(buf, s, acc);
      if (s < NH && rows_next) rows(n_next, buf ^ 1, s, qv[s], gv[s]);
    }
    // schedule: one product, then a few vector instructions, throughout
#pragma unroll
    for (int i = 0; i < 3 * KS * EH; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
    }
  };

  // Epilogue of the tile in `buf` in the accumulator layout: token nl,
  // features 16 (half EH + e) + 4 kg + i; o = num / (den (1 + e^-g)) written
  // over g in the staging tile.
  auto epilogue = [&](int buf, const f32x4 (&acc)[EH]) {
    unsigned char *s_stage = s_stage_of(buf);
    float *s_ss = s_den_of(buf) + 16;  // [half][16] partial sums of num^2 (RMSNorm)
    const float den = s_den_of(buf)[nl] + a.eps;
    float scale = 0.f;  // (kNorm) 1 / (den * rms(num / den))
    if (kNorm) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < EH; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) ss = __builtin_fmaf(acc[e][i], acc[e][i], ss);
      // this half's other features of the token sit in lanes l ^ 16, l ^ 32,
      // l ^ 48; the other half's sum comes through LDS
      const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(ss), __float_as_uint(ss),
                                                        false, false);
      ss = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
      const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss),
                                                        false, false);
      ss = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
      if (kg == 0) s_ss[half * 16 + nl] = ss;
      __syncthreads();
      ss = s_ss[nl] + s_ss[16 + nl];  // the two halves in a fixed order
      const float inv_den = __builtin_amdgcn_rcpf(den);
      scale = inv_den * rsqrtf(ss * inv_den * inv_den * (1.f / D) + a.rms_eps);
    }
#pragma unroll
    for (int e = 0; e < EH; ++e) {
      const int et = half * EH + e;
      uint2 *slot = reinterpret_cast<uint2 *>(s_stage + nl * St::kRowBytes + 2 * (16 * et + 4 * kg));
      const uint2 gw = *slot;
      const float gvf[4] = {lo_bf16(gw.x), hi_bf16(gw.x), lo_bf16(gw.y), hi_bf16(gw.y)};
      float o[4];
      if (kNorm) {
        const float4 w4 = *reinterpret_cast<const float4 *>(s_w + 16 * et + 4 * kg);
        const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ex = __expf(-gvf[i]);
          o[i] = acc[e][i] * scale * wv[i] * __builtin_amdgcn_rcpf(1.f + ex);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // num / den * sigmoid(g) = num / (den * (1 + exp(-g)))
          const float ex = __expf(-gvf[i]);
          o[i] = acc[e][i] * __builtin_amdgcn_rcpf(__builtin_fmaf(den, ex, den));
        }
      }
      *slot = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    }
  };

  // This wave's rows of the tile in `buf` leave whole (both halves'
  // features are in place).
  auto store_rows = [&](int64_t n0, int buf) {
    const unsigned char *s_stage = s_stage_of(buf);
    const __amdgpu_buffer_rsrc_t ro = tile_rsrc(o_head + n0 * a.H * D, n0, sr_end, row_bytes, D);
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const int row = row0 + RPI * j;
      const uint4 ov = *reinterpret_cast<const uint4 *>(s_stage + row * St::kRowBytes + 16 * fc);
      buf_store16<kCacheStream>(ro, lane_off + (uint32_t)(RPI * j) * row_bytes, ov);
    }
  };

  // Items slot, slot + m, ... of this super-range (tile k = item slot + k m).
  // Software pipeline over the tiles, with two tiles of loads in flight:
  //   rows(0); barrier
  //   for k: [products(k) | rows(k+1)]; barrier; epilogue(k); barrier; stores(k)
  // Tile k lives in LDS buffer k % 2.  rows(k+1) overwrites the buffer of
  // tile k-1, whose last readers (epilogue and stores) finished before the
  // previous barrier.  Loads are refilled unconditionally: tiles past the
  // range read as zeros, and their results are never stored.  Every wave
  // runs the same number of iterations (the bounds depend on the workgroup
  // only), as the barriers need.
  const int64_t n_items = (sr_end - sr_begin + item_tokens - 1) / item_tokens;
  const int64_t step = a.am;
  uint4 qa[NH], ga[NH], qb[NH], gb[NH];
  int64_t it = slot;
  fetch(tile_of(it), qa, ga);
  asm volatile("" ::: "memory");
  fetch(tile_of(it + step), qb, gb);
#pragma unroll
  for (int j = 0; j < NH; ++j) rows(tile_of(it), 0, j, qa[j], ga[j]);
  fetch(tile_of(it + 2 * step), qa, ga);
  __syncthreads();
  f32x4 acc[EH];
  while (it < n_items) {
    // tile it in buffer 0 (registers: qb = tile it + step, qa = it + 2 step)
    mma_and_rows(0, acc, true, tile_of(it + step), qb, gb);
    fetch(tile_of(it + 3 * step), qb, gb);
    __syncthreads();
    epilogue(0, acc);
    __syncthreads();
    store_rows(tile_of(it), 0);
    if (it + step >= n_items) break;
    // tile it + step in buffer 1 (qa = it + 2 step, qb = it + 3 step)
    mma_and_rows(1, acc, true, tile_of(it + 2 * step), qa, ga);
    fetch(tile_of(it + 4 * step), qa, ga);
    __syncthreads();
    epilogue(1, acc);
    __syncthreads();
    store_rows(tile_of(it + step), 1);
    it += 2 * step;
  }
  __builtin_amdgcn_s_waitcnt(0);  // prefetches past the range are still in flight
}

template <int D, bool kNorm>
hipError_t apply_reg_d(const Plan &p, const void *q, const void *g, const float *states,
                       const uint16_t *frags, const float2 *tab, const void *rms_w, void *out,
                       hipStream_t stream) {
  const size_t lds = apply_reg_lds_bytes(p);
  auto kern = apply_reg_kernel<D, kNorm>;
  const hipError_t attr = lds_limit_once((const void *)kern);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.ag * p.ar * p.am)), dim3(kApplyWaves * 64), lds,
                     stream, (const uint16_t *)q, (const uint16_t *)g, states, frags, tab,
                     (const uint16_t *)rms_w, (uint16_t *)out, make_margs(p));
  return hipGetLastError();
}

}  // namespace

size_t apply_reg_lds_bytes(const Plan &p) {
  const int64_t d = p.d;
  const int64_t pair_bytes = 2 * (2 * (16 * 2 * d) + 64 + 128 + 16 * (2 * d + 16));
  const int64_t hw = p.Hs * p.Ws;
  const int64_t sr_tokens = p.air * 16 * (kApplyPairs / p.hpw);
  const int64_t rows = std::min<int64_t>(p.T, (std::min<int64_t>(sr_tokens, p.L) + hw - 1) / hw + 1);
  const int64_t entries = (p.Hs + p.Ws) * (3 * d / 16) + rows * (d / 8);
  return (size_t)(kApplyPairs * pair_bytes + d * 4 + entries * 8);
}

hipError_t launch_apply_reg(const Plan &p, const void *q, const void *g, const float *states,
                            const uint16_t *frags, const float2 *tab, const void *rms_w,
                            void *out, hipStream_t stream) {
  if (p.d == 128)
    return rms_w ? apply_reg_d<128, true>(p, q, g, states, frags, tab, rms_w, out, stream)
                 : apply_reg_d<128, false>(p, q, g, states, frags, tab, rms_w, out, stream);
  if (p.d == 64)
    return rms_w ? apply_reg_d<64, true>(p, q, g, states, frags, tab, rms_w, out, stream)
                 : apply_reg_d<64, false>(p, q, g, states, frags, tab, rms_w, out, stream);
  return hipErrorInvalidValue;
}

}  // namespace gla
