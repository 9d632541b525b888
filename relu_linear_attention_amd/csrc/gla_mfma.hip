// Matrix-core kernels of the operator for bf16 tensors with head size 64 or
// 128 (gfx950, v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
//   state:  S_c = sum_{n in chunk} RoPE_n(phi(k_n))^T v_n,  z_c = sum phi(k_n)
//   apply:  o_i = (RoPE_i(phi(q_i)) S) / (phi(q_i) . z + eps) * sigmoid(g_i)
//
// "SANA-Video" notes page, Section 3.2 (phi = ReLU, RoPE after ReLU for the
// numerator only, un-rotated denominator); "SANA-Video 2.0" Section 2
// Eq. (1) (+eps, sigmoid output gate).
//
// Operand layout of v_mfma_f32_32x32x16_bf16 used throughout (lane l of a
// 64-wide wave, eight bf16 per operand register group):
//   A (32 x 16):  lane l holds A[l % 32][8*(l/32) + j], j = 0..7
//   B (16 x 32):  lane l holds B[8*(l/32) + j][l % 32]
//   C (32 x 32):  lane l, value i holds C[8*(i/4) + 4*(l/32) + i%4][l % 32]
//
// The contraction of the state is over tokens, so k and v are staged in LDS
// transposed (feature-major); the contraction of the apply stage is over
// features, so q is loaded straight from HBM in the B layout.

#include <hip/hip_runtime.h>

#include "gla_mfma_common.h"


namespace gla {
namespace {

// Policies of the streams of the two stages.  Measured over whole
// forward calls at 720p/81f: streaming the k and v reads of the state stage
// saves about 3% per call; streaming the q and g reads or the out writes of
// the apply stage (non-temporal, also at system scope) changes nothing
// measurable, since apply's limit is its operand-layout q loads.
constexpr int kStateLoadPolicy = kCacheStream;
constexpr int kApplyLoadPolicy = kCacheNormal;
constexpr int kApplyStorePolicy = kCacheNormal;

// ---------------------------------------------------------------- state

// Threads per workgroup of the state kernel: d = 128 runs eight waves (two
// workgroups, 16 waves, per compute unit, in at most 128 registers per
// lane: the eight waves share one RoPE table slice, and twice the waves hide
// more of the load latency than four waves with 4 tiles each), d = 64 four.
template <int D>
constexpr int kStateThreads = D == 128 ? 512 : 256;

template <int D>
struct StateCfg {
  static constexpr int NT = kStateThreads<D>;
  static constexpr int NWV = NT / 64;                // waves
  static constexpr int FPT = D / 8;                  // threads per token row (16 B each)
  static constexpr int TPP = NT / FPT;               // tokens per load pass
  static constexpr int R = (int)kStateTile / TPP;    // passes per tile
  static constexpr int TILES = (D / 32) * (D / 32);  // 32x32 output tiles of S
  static constexpr int TPW = TILES / NWV;            // tiles per wave
  static constexpr int ROW = 2 * D;                  // bytes per token row
  static constexpr int OP_BYTES = (int)kStateTile * ROW;
  // Operand tiles are row-major [token][feature] with the 16-byte units of a
  // row XOR-permuted by the row index, so that the 16-B row writes and the
  // 8-B transposing reads (4 rows x 64 B per 32 lanes) both spread over all
  // banks.  The permutation depends on row bits that neither the token
  // passes nor the k-steps of a read change.
  static __device__ __forceinline__ int swz(int row) {
    return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
  }
  static __device__ __forceinline__ int off(int row, int unit) {
    return row * ROW + ((unit ^ swz(row)) << 4);
  }
};

// One workgroup per (unit, chunk).  Each 64-token step: the threads load the
// k and v rows (16 B per thread per row, whole rows per instruction), apply
// ReLU (accumulating z) and RoPE to k in fp32, and write RoPE(phi(k)) split
// into bf16 hi + lo parts, and v (exact in bf16), as row-major tiles into
// LDS.  Each wave then reads its operands transposed (four tokens of one
// feature per lane and read) and accumulates its share of the 32x32 tiles of
// S = hi^T v + lo^T v on the matrix cores.  The rows of the next step are in
// flight in registers meanwhile.
//
// kBeta: the write gate ("SANA-Video 2.0" Eq. (1)): beta [B, N, H] scales each
// token's rotated key before it enters S (z keeps the plain phi(k)).
template <int D, bool kBeta>
__global__ __launch_bounds__(kStateThreads<D>, kStateThreads<D> / 128) void state_mfma_kernel(const uint16_t *__restrict__ k,
                                                            const uint16_t *__restrict__ v,
                                                            const uint16_t *__restrict__ beta,
                                                            const float2 *__restrict__ tab,
                                                            float *__restrict__ partials,
                                                            MArgs a) {
  using Cfg = StateCfg<D>;
  constexpr int FPT = Cfg::FPT, TPP = Cfg::TPP, R = Cfg::R, ROW = Cfg::ROW;
  extern __shared__ __align__(16) unsigned char lds[];
  unsigned char *s_kh = lds;                      // RoPE(phi(k)), bf16 hi part
  unsigned char *s_kl = lds + Cfg::OP_BYTES;      // bf16 lo part
  unsigned char *s_v = lds + 2 * Cfg::OP_BYTES;   // v
  float2 *s_tab = reinterpret_cast<float2 *>(lds + 3 * Cfg::OP_BYTES);

  const int64_t wg = blockIdx.x;
  const int64_t unit = wg / a.C, c = wg % a.C;
  const int64_t bh = unit / a.nb, blk = unit % a.nb;
  const int64_t b = bh / a.H, hd = bh % a.H;
  const int64_t n_begin = blk * a.L + c * a.Lc;
  const int64_t n_end = min(n_begin + a.Lc, (blk + 1) * a.L);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave

  const int fc = tid % FPT, tg = tid / FPT;
  // this thread's rows of a tile: tg + TPP*r, 16-byte unit fc
  const int wr_off = Cfg::off(tg, fc);

  // output tiles of this wave and their transposing-read offsets: lane l
  // (group g = l/16, s = l%16) points at row 8*(g/2) + s/4 (+ 16*ks +
  // 4*half), column 32*tile + 16*(g%2) + 4*(s%4)
  int tile_p[Cfg::TPW], tile_e[Cfg::TPW], rd_p[Cfg::TPW], rd_e[Cfg::TPW];
  {
    const int g = lane >> 4, sl = lane & 15;
    const int rrow = 8 * (g >> 1) + (sl >> 2);
#pragma unroll
    for (int t = 0; t < Cfg::TPW; ++t) {
      if (D == 128 && Cfg::NWV == 8) {
        tile_p[t] = wave >> 1;
        tile_e[t] = 2 * (wave & 1) + t;
      } else if (D == 128) {
        tile_p[t] = 2 * (wave >> 1) + (t >> 1);
        tile_e[t] = 2 * (wave & 1) + (t & 1);
      } else {
        tile_p[t] = wave >> 1;
        tile_e[t] = wave & 1;
      }
      const int cp = 32 * tile_p[t] + 16 * (g & 1) + 4 * (sl & 3);
      const int ce = 32 * tile_e[t] + 16 * (g & 1) + 4 * (sl & 3);
      rd_p[t] = Cfg::off(rrow, cp >> 3) + ((cp & 7) << 1);
      rd_e[t] = Cfg::off(rrow, ce >> 3) + ((ce & 7) << 1);
    }
  }

  // buffer resources over this chunk's rows of k and v (rows past the chunk
  // read as zeros)
  const int64_t first = ((b * a.N + n_begin) * a.H + hd) * D;
  const uint32_t row_bytes = (uint32_t)(a.H * D * 2);
  const uint32_t range_bytes = (uint32_t)(n_end - n_begin - 1) * row_bytes + 2 * D;
  const __amdgpu_buffer_rsrc_t rk = head_rows_rsrc(k + first, range_bytes);
  const __amdgpu_buffer_rsrc_t rv = head_rows_rsrc(v + first, range_bytes);
  const uint32_t my_off = (uint32_t)tg * row_bytes + 16 * fc;
  // the write gates of this chunk's tokens (a 2-byte column of [B, N, H])
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(kBeta ? beta + (b * a.N + n_begin) * a.H + hd : k), 0,
      kBeta ? (int)((n_end - n_begin - 1) * a.H * 2 + 2) : 0, 0x00020000);
  uint4 kr[R], vr[R];
  uint32_t br[R];
  auto load_rows = [&](int64_t n0) {
    const uint32_t base = (uint32_t)(n0 - n_begin) * row_bytes + my_off;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      kr[r] = buf_load16<kStateLoadPolicy>(rk, base + (uint32_t)(TPP * r) * row_bytes);
      vr[r] = buf_load16<kStateLoadPolicy>(rv, base + (uint32_t)(TPP * r) * row_bytes);
      if (kBeta)
        br[r] = __builtin_amdgcn_raw_buffer_load_b16(
            rb, (int)(((uint32_t)(n0 - n_begin) + tg + TPP * r) * (uint32_t)a.H * 2), 0, 0);
    }
  };

  // The table slice goes to LDS while the first step's rows are in flight:
  // its loads, then the rows' loads, then its stores (which wait for the
  // older table loads alone).  The compiler-only barriers keep the two groups
  // of loads in that order.
  TabLoad<D> tload;
  tload.issue(tab, a, n_begin, n_end);
  asm volatile("" ::: "memory");
  load_rows(n_begin);
  asm volatile("" ::: "memory");
  tload.store(s_tab, tab);
  const TabSlice<D> ts = tload.ts;
  int axis, pia;
  pair_axis<D>(4 * fc, axis, pia);
  const typename TabSlice<D>::Lookup tl = ts.lookup(axis, pia);

  f32x16 acc[Cfg::TPW];
#pragma unroll
  for (int t = 0; t < Cfg::TPW; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
  float zacc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) zacc[j] = 0.f;

  // Each 64-token step: ReLU/RoPE/split of the rows in (kr, vr) into the LDS
  // tiles; once they are there, the same registers are refilled with the
  // next step's rows, which stay in flight during the matrix-core phase.
  for (int64_t n0 = n_begin; n0 < n_end; n0 += kStateTile) {
    __syncthreads();  // the previous step's operand reads are done
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int64_t n = n0 + tg + TPP * r;
      if (n >= n_end) n = n_end - 1;  // position only; the row itself reads as zero
      int t, h, w;
      token_pos(a, n, t, h, w);
      const uint32_t kw[4] = {kr[r].x, kr[r].y, kr[r].z, kr[r].w};
      float x[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t rl = relu_bf16x2(kw[m]);
        x[2 * m] = lo_bf16(rl);
        x[2 * m + 1] = hi_bf16(rl);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) zacc[j] += x[j];
      float2 c4[4];
      ts.read(s_tab, tl.at(t, h, w), c4);
      rotate4(x, c4);
      if (kBeta) {
        const float bt = bf16_bits_to_float(br[r]);
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] *= bt;
      }
      uint4 hi, lo;
      split_bf16x2(x[0], x[1], hi.x, lo.x);
      split_bf16x2(x[2], x[3], hi.y, lo.y);
      split_bf16x2(x[4], x[5], hi.z, lo.z);
      split_bf16x2(x[6], x[7], hi.w, lo.w);
      const int o = wr_off + r * TPP * ROW;
      *reinterpret_cast<uint4 *>(s_kh + o) = hi;
      *reinterpret_cast<uint4 *>(s_kl + o) = lo;
      *reinterpret_cast<uint4 *>(s_v + o) = vr[r];
    }
    // unconditional (rows past the chunk read as zeros): a conditional load
    // here would make the compiler wait for it before the matrix-core phase
    load_rows(n0 + kStateTile);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < (int)kStateTile / 16; ++ks) {
#pragma unroll
      for (int t = 0; t < Cfg::TPW; ++t) {
        const int o0 = (16 * ks) * ROW, o1 = (16 * ks + 4) * ROW;
        const uint2 h0 = lds_read_tr16(s_kh + rd_p[t] + o0), h1 = lds_read_tr16(s_kh + rd_p[t] + o1);
        const uint2 l0 = lds_read_tr16(s_kl + rd_p[t] + o0), l1 = lds_read_tr16(s_kl + rd_p[t] + o1);
        const uint2 v0 = lds_read_tr16(s_v + rd_e[t] + o0), v1 = lds_read_tr16(s_v + rd_e[t] + o1);
        const bf16x8 fa = __builtin_bit_cast(bf16x8, make_uint4(h0.x, h0.y, h1.x, h1.y));
        const bf16x8 fl = __builtin_bit_cast(bf16x8, make_uint4(l0.x, l0.y, l1.x, l1.y));
        const bf16x8 fb = __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fl, fb, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc[t], 0, 0, 0);
      }
    }
  }

  // S_c, row-major: lanes 0..31 write 32 consecutive floats of one row
  float *dst = partials + wg * (int64_t)(D * D + D);
#pragma unroll
  for (int t = 0; t < Cfg::TPW; ++t) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int p = 32 * tile_p[t] + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      const int e = 32 * tile_e[t] + (lane & 31);
      dst[p * D + e] = acc[t][i];
    }
  }
  // z_c: per-thread sums over its tokens, then a fixed-order sum over the
  // TPP token groups
  __syncthreads();
  float *zs = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int j = 0; j < 8; ++j) zs[tg * D + 8 * fc + j] = zacc[j];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
    for (int gidx = 0; gidx < TPP; ++gidx) s += zs[gidx * D + tid];
    dst[D * D + tid] = s;
  }
}

// ---------------------------------------------------------------- apply

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


//
// kNorm: the RMSNorm of "SANA-Video 2.0" Eq. (1) between num/den and the
// gate: y = num/den is scaled by 1/sqrt(mean over the D features of y^2 +
// rms_eps) and by the weight w [D].  A token's D values are spread over the
// four lanes l % 16 == token (32 each), summed with two lane exchanges.
template <int D, bool kNorm>
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

  const int64_t wg = blockIdx.x;
  const int64_t unit = wg / a.R, r = wg % a.R;
  const int64_t bh = unit / a.nb, blk = unit % a.nb;
  const int64_t b = bh / a.H, hd = bh % a.H;
  const int64_t n_begin = blk * a.L + r * a.Lr;
  const int64_t n_end = min(n_begin + a.Lr, (blk + 1) * a.L);
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
  // buffer resources over this range's rows of q, g and out
  const int64_t first = ((b * a.N + n_begin) * a.H + hd) * D;
  const uint32_t row_bytes = (uint32_t)(a.H * D * 2);
  const uint32_t range_bytes = (uint32_t)(n_end - n_begin - 1) * row_bytes + 2 * D;
  const __amdgpu_buffer_rsrc_t rq = head_rows_rsrc(q + first, range_bytes);
  const __amdgpu_buffer_rsrc_t rg = head_rows_rsrc(g + first, range_bytes);
  const __amdgpu_buffer_rsrc_t ro = head_rows_rsrc(out + first, range_bytes);
  // loads of one tile: q in the B-operand layout, g as whole rows (rows past
  // the range read as zeros)
  auto fetch = [&](int64_t tile, uint4 (&qraw)[KS], uint4 (&grow)[St::kPasses]) {
    const uint32_t rel = (uint32_t)(tile - n_begin);
    const uint32_t qoff = (rel + nl) * row_bytes + 2 * 8 * kg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qraw[ks] = buf_load16<kApplyLoadPolicy>(rq, qoff + 2 * 32 * ks);
#pragma unroll
    for (int i = 0; i < St::kPasses; ++i)
      grow[i] = buf_load16<kApplyLoadPolicy>(rg, (rel + i * St::kRowsPerPass + rl) * row_bytes + 2 * rc);
  };
  // everything after the loads of one tile
  auto process = [&](int64_t tile, const uint4 (&cq)[KS], const uint4 (&cg)[St::kPasses]) {
      // An offset the compiler cannot see through (always 0) keeps the
      // loop-invariant S-part reads inside the loop: hoisting all of them
      // would need 256 registers per lane.  It is a register-only asm, so it
      // does not make the compiler drain outstanding memory operations.
      int opaque = 0;
      asm volatile("" : "+v"(opaque));
      const unsigned char *sh = s_sh + opaque, *sl = s_sl + opaque;
      const int64_t n = tile + nl;
      const bool valid = n < n_end;
      int t, h, w;
      token_pos(a, valid ? n : n_end - 1, t, h, w);

      f32x4 acc[ET], accd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int et = 0; et < ET; ++et) acc[et] = accd;

#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t qw[4] = {relu_bf16x2(cq[ks].x), relu_bf16x2(cq[ks].y),
                                relu_bf16x2(cq[ks].z), relu_bf16x2(cq[ks].w)};
        const bf16x8 bden = __builtin_bit_cast(bf16x8, make_uint4(qw[0], qw[1], qw[2], qw[3]));
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
        const bf16x8 bh = __builtin_bit_cast(bf16x8, make_uint4(hw4[0], hw4[1], hw4[2], hw4[3]));
        const bf16x8 bl = __builtin_bit_cast(bf16x8, make_uint4(lw4[0], lw4[1], lw4[2], lw4[3]));
        accd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s_zf[ks * 64 + lane], bden, accd, 0, 0, 0);
        // A = S^T fragments (rows e = 16*et + l%16, columns p = 32*ks +
        // 8*(l/16) + j), read transposed from the row-major S parts, four
        // output tiles at a time; the three products of a tile are issued
        // round-robin over the four tiles so that consecutive matrix-core
        // instructions do not depend on each other
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

      const float den = accd[0] + accd[1] + a.eps;
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
#pragma unroll
      for (int i = 0; i < St::kPasses; ++i) {
        const int tok = i * St::kRowsPerPass + rl;
        const uint4 ov = *reinterpret_cast<const uint4 *>(stage + tok * St::kRowBytes + 2 * rc);
        buf_store16<kApplyStorePolicy>(ro, ((uint32_t)(tile - n_begin) + tok) * row_bytes + 2 * rc, ov);
      }
      // the next tile's first staging writes must not overtake these reads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Two tiles of loads stay in flight per wave: buffer A holds tile i while
  // B receives tile i+1; once tile i is done, A is refilled with tile i+2
  // before tile i+1 (in B) is processed, and so on.  The refills are
  // unconditional (tiles past the range read as zeros and are never
  // processed): with a branch around them the compiler cannot tell which
  // loads are still outstanding at the top of the loop and waits for all of
  // them, the next tile's included, which leaves one tile in flight.
  constexpr int64_t kStep = 16 * NW;
  uint4 qa[KS], ga[St::kPasses], qb[KS], gb[St::kPasses];
  int64_t tile = n_begin + 16 * wave;
  fetch(tile, qa, ga);
  asm volatile("" ::: "memory");  // the first tile's loads are issued first
  fetch(tile + kStep, qb, gb);
  while (tile < n_end) {
    process(tile, qa, ga);
    fetch(tile + 2 * kStep, qa, ga);
    if (tile + kStep < n_end) process(tile + kStep, qb, gb);
    fetch(tile + 3 * kStep, qb, gb);
    tile += 2 * kStep;
  }
  __builtin_amdgcn_s_waitcnt(0);  // prefetches past the range are still in flight
}

template <int D, bool kBeta>
hipError_t state_d(const Plan &p, const void *k, const void *v, const void *beta,
                   const float2 *tab, float *part, hipStream_t stream) {
  const size_t lds = 3 * StateCfg<D>::OP_BYTES + tab_slice_entries(p, p.Lc) * sizeof(float2);
  auto kern = state_mfma_kernel<D, kBeta>;
  hipError_t e = hipFuncSetAttribute((const void *)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.units * p.C)), dim3(StateCfg<D>::NT), lds, stream,
                     (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)beta, tab, part,
                     make_margs(p));
  return hipGetLastError();
}

template <int D, bool kNorm>
hipError_t apply_d(const Plan &p, const void *q, const void *g, const float *states,
                   const uint16_t *frags, const float2 *tab, const void *rms_w, void *out,
                   hipStream_t stream) {
  const size_t lds = (size_t)D * D * 2 * 2 + (size_t)(D / 32) * 64 * 16 + (size_t)D * 4 +
                     (size_t)(kApplyThreads / 64) * Stage<D>::kBytes +
                     tab_slice_entries(p, p.Lr) * sizeof(float2);
  auto kern = apply_mfma_kernel<D, kNorm>;
  hipError_t e = hipFuncSetAttribute((const void *)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.units * p.R)), dim3(kApplyThreads), lds, stream,
                     (const uint16_t *)q, (const uint16_t *)g, states, frags, tab,
                     (const uint16_t *)rms_w, (uint16_t *)out,
                     make_margs(p));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_state_mfma(const Plan &p, const void *k, const void *v, const void *beta,
                             const float2 *tab, float *partials, hipStream_t stream) {
  if (p.d == 128)
    return beta ? state_d<128, true>(p, k, v, beta, tab, partials, stream)
                : state_d<128, false>(p, k, v, beta, tab, partials, stream);
  if (p.d == 64)
    return beta ? state_d<64, true>(p, k, v, beta, tab, partials, stream)
                : state_d<64, false>(p, k, v, beta, tab, partials, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_apply_mfma(const Plan &p, const void *q, const void *g, const float *states,
                             const uint16_t *frags, const float2 *tab, const void *rms_w,
                             void *out, hipStream_t stream) {
  if (p.d == 128)
    return rms_w ? apply_d<128, true>(p, q, g, states, frags, tab, rms_w, out, stream)
                 : apply_d<128, false>(p, q, g, states, frags, tab, rms_w, out, stream);
  if (p.d == 64)
    return rms_w ? apply_d<64, true>(p, q, g, states, frags, tab, rms_w, out, stream)
                 : apply_d<64, false>(p, q, g, states, frags, tab, rms_w, out, stream);
  return hipErrorInvalidValue;
}

}  // namespace gla
