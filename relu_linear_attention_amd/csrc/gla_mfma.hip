// State stage of the operator on the matrix cores for bf16 tensors with head
// size 64 or 128 (gfx950, v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//
//   S_c = sum_{n in chunk} RoPE_n(phi(k_n))^T v_n,  z_c = sum phi(k_n)
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
// The contraction is over tokens, so k and v are staged in LDS and read
// back transposed (feature-major).

#include <hip/hip_runtime.h>

#include "gla_mfma_common.h"


namespace gla {
namespace {

// k and v are read once: streaming (non-temporal) loads, measured about 3%
// faster per call at 720p/81f than normal ones.
constexpr int kStateLoadPolicy = kCacheStream;

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

}  // namespace gla
