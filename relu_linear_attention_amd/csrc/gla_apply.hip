// Output stage of the operator on the matrix cores (bf16, head size 64 or
// 128; gfx950, v_mfma_f32_16x16x32_bf16 with fp32 accumulation):
//
//   o_i = (RoPE_i(phi(q_i)) S) / (phi(q_i) . z + eps) * sigmoid(g_i)
//
// "SANA-Video" notes page, Section 3.2 (phi = ReLU, RoPE after ReLU in the
// numerator only, the un-rotated denominator); "SANA-Video 2.0" Section 2
// Eq. (1) (+eps and the sigmoid output gate; the optional RMSNorm of num/den
// before the gate).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "gla_mfma_common.h"

namespace gla {
namespace {

// 16x16x32 bf16 matrix-core layout used by the apply stage:
//   A (16 x 32):  lane l holds A[l % 16][8*(l/16) + j], j = 0..7
//   B (32 x 16):  lane l holds B[8*(l/16) + j][l % 16]
//   C (16 x 16):  lane l, value i holds C[4*(l/16) + i][l % 16]
//
// One workgroup (8 waves) per (unit, token range); each wave takes 16-token
// tiles.  LDS holds the unit's S^T as bf16 A fragments in two parts, S ~
// S_hi + S_lo (written by the reduce stage), the A fragments of the
// denominator (rows 0, 4, 8, 12 carry z rounded to bf16 and rows 1, 5, 9, 13
// the bf16 rounding of the remainder, so C values 0 and 1 of every lane sum
// to phi(q).z), the RoPE table rows of the range, and one staging tile per
// wave.  Per tile and 32-feature step a lane loads 16 B of its token's q row;
// ReLU(q) is exact in bf16 and is the B operand of the denominator;
// RoPE(ReLU(q)) is split into bf16 hi + lo parts, and the numerator
// accumulates hi*S_hi + lo*S_hi + hi*S_lo in fp32, which carries about 16
// significant bits of every operand.  The gate g is loaded as whole 256-B
// rows into the staging tile, read back in the accumulator layout, combined
// with num / den, written back in place as bf16, and the tile leaves as whole
// 256-B rows: full-row accesses keep HBM efficient where 8-B pieces per token
// do not.
constexpr int kApplyThreads = 512;
constexpr int64_t kItem = 16 * (kApplyThreads / 64);  // tokens of an item: a tile per wave


//
// kNorm: the RMSNorm of "SANA-Video 2.0" Eq. (1) between num/den and the
// gate: y = num/den is scaled by 1/sqrt(mean over the D features of y^2 +
// rms_eps) and by the weight w [D].  A token's D values are spread over the
// four lanes l % 16 == token (32 each), summed with two lane exchanges.
//
// kPair: a wave takes two 16-token blocks at a time (below); otherwise one.
template <int D, bool kNorm, bool kPair>
__global__ __launch_bounds__(kApplyThreads) void apply_mfma_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ g,
    const float *__restrict__ states, const uint16_t *__restrict__ frags,
    const float2 *__restrict__ tab, const uint16_t *__restrict__ rms_w,
    uint16_t *__restrict__ out, MArgs a) {
  constexpr int KS = D / 32;  // 32-feature contraction steps
  constexpr int ET = D / 16;  // 16-feature output tiles
  constexpr int NW = kApplyThreads / 64;
  extern __shared__ __align__(16) unsigned char lds[];
  unsigned char *s_sh = lds;             // S hi part, row-major [p][e], units permuted
  unsigned char *s_sl = lds + D * D * 2;  // S lo part
  bf16x8 *s_zf = reinterpret_cast<bf16x8 *>(lds + D * D * 4);  // KS fragments x 64 lanes
  float *s_w = reinterpret_cast<float *>(s_zf + KS * 64);        // RMSNorm weight (D)
  using St = Stage<D>;
  unsigned char *s_stage = reinterpret_cast<unsigned char *>(s_w + D);  // NW tiles
  float2 *s_tab = reinterpret_cast<float2 *>(s_stage + NW * St::kBytes);

  // workgroup -> (unit, super-range, slot): the workgroups of a unit take
  // its items (kItem consecutive tokens, one 16-token tile per wave) in
  // turn, and the unit index runs fastest, so that at any moment all heads
  // of a token row are read and written together
  const int64_t wg = blockIdx.x;
  const int64_t unit = wg % a.ag;
  const int64_t rest = wg / a.ag;
  const int64_t sr = rest / a.am, slot = rest % a.am;
  const int64_t bh = unit / a.nb, blk = unit % a.nb;
  const int64_t b = bh / a.H, hd = bh % a.H;
  const int64_t blk_end = (blk + 1) * a.L;
  const int64_t n_begin = blk * a.L + sr * a.air * kItem;
  const int64_t n_end = min(n_begin + a.air * kItem, blk_end);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave

  {
    // S hi then lo, 16-byte units i = (part, row, unit), unit permuted by row
    const uint4 *src = reinterpret_cast<const uint4 *>(frags + unit * (int64_t)D * D * 2);
    for (int i = tid; i < D * D * 2 / 8; i += kApplyThreads) {
      const int u = i % (D / 8), row = (i / (D / 8)) % D, part = i / (D * D / 8);
      *reinterpret_cast<uint4 *>(lds + part * D * D * 2 + SRow<D>::off(row, u)) = src[i];
    }
    const float *zsrc = states + unit * (int64_t)(D * D + D) + D * D;
    for (int i = tid; i < KS * 64; i += kApplyThreads) {
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
  }
  if (kNorm)
    for (int i = tid; i < D; i += kApplyThreads) s_w[i] = bf16_bits_to_float(rms_w[i]);
  const TabSlice<D> ts = load_tab_slice<D>(s_tab, tab, a, n_begin, n_end);
  __syncthreads();

  const int nl = lane & 15, kg = lane >> 4;
  // transposing-read offsets of the S parts: lane l (s = l%16, group
  // g = l/16) points at row 8*g + s/4 (+ 32*ks + 4*half), column
  // 16*et + 4*(s%4); the row's unit permutation depends only on s and g
  int rd_s[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et)
    rd_s[et] = SRow<D>::off(8 * kg + (nl >> 2), 2 * et + ((nl & 3) >> 1)) + 8 * (nl & 1);
  // row-wise lane mapping of the staging tile: in pass i lane l covers token
  // i*kRowsPerPass + l/kLanesPerRow, features 8*(l%kLanesPerRow)..+7
  const int rl = lane / St::kLanesPerRow, rc = 8 * (lane % St::kLanesPerRow);
  // buffer resources over each tile's rows of q, g and out (64-bit base,
  // rows past the range read as zeros and are not written)
  const uint32_t row_bytes = (uint32_t)(a.H * D * 2);
  const uint16_t *q_head = q + (b * a.N * a.H + hd) * D;
  const uint16_t *g_head = g + (b * a.N * a.H + hd) * D;
  uint16_t *o_head = out + (b * a.N * a.H + hd) * D;
  // loads of one 16-token block: q in the B-operand layout, g as whole rows
  auto fetch_q = [&](int64_t tile, uint4 (&qraw)[KS]) {
    const __amdgpu_buffer_rsrc_t rq = tile_rsrc(q_head + tile * a.H * D, tile, n_end, row_bytes, D);
    const uint32_t qoff = (uint32_t)nl * row_bytes + 2 * 8 * kg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qraw[ks] = buf_load16<kCacheStream>(rq, qoff + 2 * 32 * ks);
  };
  auto fetch_g = [&](int64_t tile, uint4 (&grow)[St::kPasses]) {
    const __amdgpu_buffer_rsrc_t rg = tile_rsrc(g_head + tile * a.H * D, tile, n_end, row_bytes, D);
#pragma unroll
    for (int i = 0; i < St::kPasses; ++i)
      grow[i] = buf_load16<kCacheStream>(rg, (uint32_t)(i * St::kRowsPerPass + rl) * row_bytes + 2 * rc);
  };

  // RoPE(ReLU(q)) of one block's k-step ks as bf16 hi + lo B operands, and
  // ReLU(q) itself (exact in bf16) for the denominator
  auto q_operands = [&](const uint4 &cq, int ks, int t, int h, int w, bf16x8 &bh, bf16x8 &bl,
                        bf16x8 &bden) {
    const uint32_t qw[4] = {relu_bf16x2(cq.x), relu_bf16x2(cq.y), relu_bf16x2(cq.z),
                            relu_bf16x2(cq.w)};
    bden = __builtin_bit_cast(bf16x8, make_uint4(qw[0], qw[1], qw[2], qw[3]));
    float x[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      x[2 * m] = lo_bf16(qw[m]);
      x[2 * m + 1] = hi_bf16(qw[m]);
    }
    int axis, pia;
    pair_axis<D>(16 * ks + 4 * kg, axis, pia);
    float2 c4[4];
    ts.read(s_tab, ts.lookup(axis, pia).at(t, h, w), c4);
    rotate4(x, c4);
    uint32_t hw4[4], lw4[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) split_bf16x2(x[2 * m], x[2 * m + 1], hw4[m], lw4[m]);
    bh = __builtin_bit_cast(bf16x8, make_uint4(hw4[0], hw4[1], hw4[2], hw4[3]));
    bl = __builtin_bit_cast(bf16x8, make_uint4(lw4[0], lw4[1], lw4[2], lw4[3]));
  };

  // num and den of two 16-token blocks (A, B) that share every S fragment
  // read: per k-step, each pair of S^T fragments (hi, lo) of an output tile
  // feeds six products, three per block (nb2 false: block A alone)
  auto products = [&](auto nb2, auto row16, int64_t tA, int64_t tB, const uint4 (&cqA)[KS],
                      const uint4 (&cqB)[KS], f32x4 (&accA)[ET], f32x4 (&accB)[ET], float &denA,
                      float &denB) {
    constexpr bool kTwo = decltype(nb2)::value;
    constexpr bool kCarry = decltype(row16)::value;
    // An offset the compiler cannot see through (always 0) keeps the
    // loop-invariant S-part reads inside the loop: hoisting all of them
    // would need 256 registers per lane.  It is a register-only asm, so it
    // does not make the compiler drain outstanding memory operations.
    int opaque = 0;
    asm volatile("" : "+v"(opaque));
    const unsigned char *sh = s_sh + opaque, *sl = s_sl + opaque;
    int pA[3], pB[3];
    block_token_pos<kCarry>(a, tA, n_end, nl, pA[0], pA[1], pA[2]);
    if (kTwo) block_token_pos<kCarry>(a, tB, n_end, nl, pB[0], pB[1], pB[2]);
    // Raised wave priority while this wave issues its products: of the two
    // waves on a SIMD, the one in its product phase then issues first, and
    // the other's gate and store work fills the gaps (the products phase
    // mixes matrix-core and vector work, the gate phase is vector work only).
    // Measured: -4% for this kernel and -2% per call over calls 5-24 at
    // 720p/81f, where the shader clock is low and the kernels issue-bound.
    // The stores of a block's rows run at a middle priority (below).
    __builtin_amdgcn_s_setprio(2);
    f32x4 adA = {0.f, 0.f, 0.f, 0.f}, adB = adA;
#pragma unroll
    for (int et = 0; et < ET; ++et) accA[et] = accB[et] = adA;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 bhA, blA, bdA, bhB, blB, bdB;
      q_operands(cqA[ks], ks, pA[0], pA[1], pA[2], bhA, blA, bdA);
      if (kTwo) q_operands(cqB[ks], ks, pB[0], pB[1], pB[2], bhB, blB, bdB);
      adA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s_zf[ks * 64 + lane], bdA, adA, 0, 0, 0);
      if (kTwo) adB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s_zf[ks * 64 + lane], bdB, adB, 0, 0, 0);
      // A = S^T fragments (rows e = 16*et + l%16, columns p = 32*ks +
      // 8*(l/16) + j), read transposed from the row-major S parts, two
      // output tiles at a time; the products are issued so that consecutive
      // matrix-core instructions do not depend on each other
#pragma unroll
      for (int eg = 0; eg < ET; eg += 2) {
        bf16x8 ah[2], al[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int o0 = rd_s[eg + u] + (32 * ks) * (2 * D);
          const int o1 = o0 + 4 * (2 * D);
          const uint2 h0 = lds_read_tr16(sh + o0), h1 = lds_read_tr16(sh + o1);
          const uint2 l0 = lds_read_tr16(sl + o0), l1 = lds_read_tr16(sl + o1);
          ah[u] = __builtin_bit_cast(bf16x8, make_uint4(h0.x, h0.y, h1.x, h1.y));
          al[u] = __builtin_bit_cast(bf16x8, make_uint4(l0.x, l0.y, l1.x, l1.y));
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          accA[eg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[u], blA, accA[eg + u], 0, 0, 0);
          if (kTwo)
            accB[eg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[u], blB, accB[eg + u], 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          accA[eg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[u], bhA, accA[eg + u], 0, 0, 0);
          if (kTwo)
            accB[eg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[u], bhB, accB[eg + u], 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          accA[eg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[u], bhA, accA[eg + u], 0, 0, 0);
          if (kTwo)
            accB[eg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[u], bhB, accB[eg + u], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    denA = adA[0] + adA[1] + a.eps;
    denB = kTwo ? adB[0] + adB[1] + a.eps : 0.f;
  };

  // the gate, the divide and the store of one 16-token block
  auto finish = [&](int64_t tile, const f32x4 (&acc)[ET], float den,
                    const uint4 (&cg)[St::kPasses]) {
      unsigned char *stage = s_stage + wave * St::kBytes;
#pragma unroll
      for (int i = 0; i < St::kPasses; ++i)
        *reinterpret_cast<uint4 *>(stage + (i * St::kRowsPerPass + rl) * St::kRowBytes + 2 * rc) =
            cg[i];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float scale = 0.f;  // (kNorm) 1 / (den * rms(num / den))
      if (kNorm) {
        // sum of num^2 over the token's D features: 32 in this lane, the rest
        // in lanes l ^ 16, l ^ 32 and l ^ 48, added by two in-register lane
        // swaps (gfx950 permlane16/32 swap: each returns the pair of values
        // exchanged between rows, whose sum is this lane's plus its partner's)
        float ss = 0.f;
#pragma unroll
        for (int et = 0; et < ET; ++et)
#pragma unroll
          for (int i = 0; i < 4; ++i) ss = __builtin_fmaf(acc[et][i], acc[et][i], ss);
        const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(ss), __float_as_uint(ss),
                                                          false, false);
        ss = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
        const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss),
                                                          false, false);
        ss = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
        // rms(num / den) = sqrt(sum num^2 / (D den^2) + rms_eps)
        const float inv_den = __builtin_amdgcn_rcpf(den);
        scale = inv_den * rsqrtf(ss * inv_den * inv_den * (1.f / D) + a.rms_eps);
      }
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        uint2 *slot = reinterpret_cast<uint2 *>(stage + nl * St::kRowBytes + 2 * (16 * et + 4 * kg));
        const uint2 gw = *slot;
        const float gv[4] = {lo_bf16(gw.x), hi_bf16(gw.x), lo_bf16(gw.y), hi_bf16(gw.y)};
        float o[4];
        if (kNorm) {
          const float4 w4 = *reinterpret_cast<const float4 *>(s_w + 16 * et + 4 * kg);
          const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // num / den / rms * w * sigmoid(g)
            const float e = __expf(-gv[i]);
            o[i] = acc[et][i] * scale * wv[i] * __builtin_amdgcn_rcpf(1.f + e);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // num / den * sigmoid(g) = num / (den * (1 + exp(-g)))
            const float e = __expf(-gv[i]);
            o[i] = acc[et][i] * __builtin_amdgcn_rcpf(__builtin_fmaf(den, e, den));
          }
        }
        *slot = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // the block's rows leave at a priority between the product phase and
      // the gate work (measured -1.6% for this kernel at the settled clock)
      __builtin_amdgcn_s_setprio(1);
      const __amdgpu_buffer_rsrc_t ro = tile_rsrc(o_head + tile * a.H * D, tile, n_end, row_bytes, D);
#pragma unroll
      for (int i = 0; i < St::kPasses; ++i) {
        const int tok = i * St::kRowsPerPass + rl;
        const uint4 ov = *reinterpret_cast<const uint4 *>(stage + tok * St::kRowBytes + 2 * rc);
        buf_store16<kCacheStream>(ro, (uint32_t)tok * row_bytes + 2 * rc, ov);
      }
      __builtin_amdgcn_s_setprio(0);
      // the next block's first staging writes must not overtake these reads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // The main loop is compiled twice, for grid rows of at least 16 tokens
  // (the positions of a block's tokens from its first token's plus one carry
  // per axis) and for shorter rows (a division per token), so that no branch
  // on the row length sits inside it.
  auto run = [&](auto row16) {
    const int64_t kStep = kItem * a.am;
    int64_t tile = n_begin + slot * kItem + 16 * wave;
    if constexpr (kPair) {
      // The workgroup takes the items slot, slot + m, ... of its super-range; a
      // wave takes the 16-token block 16 wave of two consecutive ones (A, B) at
      // a time.  q of the next pair is in flight during the current pair's
      // products and gates; g of a block is refilled right after its gate and
      // arrives during the next pair's products.  Refills are unconditional
      // (blocks past the range read as zeros and their stores are dropped):
      // with a branch around them the compiler waits for every outstanding
      // load at the join.  With an odd item count the last pair's second block
      // lies past the range; the plan takes pairs only where that block is
      // off the critical path or a small share of it.
      uint4 q0[KS], q1[KS], q2[KS], q3[KS], gA[St::kPasses], gB[St::kPasses];
      fetch_q(tile, q0);
      fetch_q(tile + kStep, q1);
      fetch_g(tile, gA);
      fetch_g(tile + kStep, gB);
      asm volatile("" ::: "memory");  // the first pair's loads are issued first
      auto pair = [&](int64_t t0, const uint4 (&qa)[KS], const uint4 (&qb)[KS], uint4 (&na)[KS],
                      uint4 (&nb)[KS]) {
        fetch_q(t0 + 2 * kStep, na);
        fetch_q(t0 + 3 * kStep, nb);
        f32x4 accA[ET], accB[ET];
        float denA, denB;
        products(std::true_type{}, row16, t0, t0 + kStep, qa, qb, accA, accB, denA, denB);
        finish(t0, accA, denA, gA);
        fetch_g(t0 + 2 * kStep, gA);
        finish(t0 + kStep, accB, denB, gB);
        fetch_g(t0 + 3 * kStep, gB);
      };
      while (tile < n_end) {
        pair(tile, q0, q1, q2, q3);
        tile += 2 * kStep;
        if (tile >= n_end) break;
        pair(tile, q2, q3, q0, q1);
        tile += 2 * kStep;
      }
    } else {
      // One block at a time, two in flight: buffer A holds block i while B
      // receives block i + 1; once block i is done, A is refilled with block
      // i + 2 before block i + 1 (in B) is processed, and so on (refills
      // unconditional, as above).
      uint4 qa[KS], ga[St::kPasses], qb[KS], gb[St::kPasses];
      auto single = [&](int64_t t0, const uint4 (&cq)[KS], const uint4 (&cg)[St::kPasses]) {
        f32x4 acc[ET], unused[ET];
        float den, unused_den;
        products(std::false_type{}, row16, t0, t0, cq, cq, acc, unused, den, unused_den);
        finish(t0, acc, den, cg);
      };
      fetch_q(tile, qa);
      fetch_g(tile, ga);
      asm volatile("" ::: "memory");  // the first block's loads are issued first
      fetch_q(tile + kStep, qb);
      fetch_g(tile + kStep, gb);
      while (tile < n_end) {
        single(tile, qa, ga);
        fetch_q(tile + 2 * kStep, qa);
        fetch_g(tile + 2 * kStep, ga);
        if (tile + kStep < n_end) single(tile + kStep, qb, gb);
        fetch_q(tile + 3 * kStep, qb);
        fetch_g(tile + 3 * kStep, gb);
        tile += 2 * kStep;
      }
    }
  };
  if (a.Ws >= 16)
    run(std::true_type{});
  else
    run(std::false_type{});
  __builtin_amdgcn_s_waitcnt(0);  // prefetches past the range are still in flight
}

template <int D, bool kNorm, bool kPair>
hipError_t apply_mfma_d(const Plan &p, const void *q, const void *g, const float *states,
                       const uint16_t *frags, const float2 *tab, const void *rms_w, void *out,
                       hipStream_t stream) {
  const size_t lds = apply_mfma_lds_bytes(p);
  auto kern = apply_mfma_kernel<D, kNorm, kPair>;
  const hipError_t attr = lds_limit_once((const void *)kern);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.ag * p.ar * p.am)), dim3(kApplyThreads), lds,
                     stream, (const uint16_t *)q, (const uint16_t *)g, states, frags, tab,
                     (const uint16_t *)rms_w, (uint16_t *)out, make_margs(p));
  return hipGetLastError();
}

}  // namespace

size_t apply_mfma_lds_bytes(const Plan &p) {
  const int64_t d = p.d;
  const int64_t hw = p.Hs * p.Ws;
  const int64_t sr_tokens = p.air * kItem;
  const int64_t rows = std::min<int64_t>(p.T, (std::min<int64_t>(sr_tokens, p.L) + hw - 1) / hw + 1);
  const int64_t entries = (p.Hs + p.Ws) * (3 * d / 16) + rows * (d / 8);
  return (size_t)(d * d * 4 + (d / 32) * 64 * 16 + d * 4 +
                  (kApplyThreads / 64) * (16 * (2 * d + 16)) + entries * 8);
}

int64_t apply_mfma_item_tokens() { return kItem; }

hipError_t apply_mfma_lds_limits() {
  return lds_limits({(const void *)apply_mfma_kernel<128, false, false>,
                     (const void *)apply_mfma_kernel<128, true, false>,
                     (const void *)apply_mfma_kernel<64, false, false>,
                     (const void *)apply_mfma_kernel<64, true, false>,
                     (const void *)apply_mfma_kernel<128, false, true>,
                     (const void *)apply_mfma_kernel<128, true, true>,
                     (const void *)apply_mfma_kernel<64, false, true>,
                     (const void *)apply_mfma_kernel<64, true, true>});
}

hipError_t launch_apply_mfma(const Plan &p, const void *q, const void *g, const float *states,
                            const uint16_t *frags, const float2 *tab, const void *rms_w,
                            void *out, hipStream_t stream) {
#define GLA_APPLY_CASE(DD, NORM)                                                                \
  return p.apair ? apply_mfma_d<DD, NORM, true>(p, q, g, states, frags, tab, rms_w, out, stream)  \
                 : apply_mfma_d<DD, NORM, false>(p, q, g, states, frags, tab, rms_w, out, stream);
  if (p.d == 128) {
    if (rms_w) GLA_APPLY_CASE(128, true)
    GLA_APPLY_CASE(128, false)
  }
  if (p.d == 64) {
    if (rms_w) GLA_APPLY_CASE(64, true)
    GLA_APPLY_CASE(64, false)
  }
#undef GLA_APPLY_CASE
  return hipErrorInvalidValue;
}

}  // namespace gla
