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

#include <type_traits>

#include "gla_mfma_common.h"


namespace gla {
namespace {

// k and v are read once: streaming (non-temporal) loads, measured about 3%
// faster per call at 720p/81f than normal ones.
constexpr int kStateLoadPolicy = kCacheStream;

// 16-byte loads of chunk partials at device scope (the SC1 cache-policy
// bit): coherent with the device-scope stores other workgroups made, from
// any XCD.  `base` is where the resource starts.
constexpr int kCacheDevice = 16;
struct DeviceLoad4 {
  __amdgpu_buffer_rsrc_t r;
  const float *base;
  __device__ __forceinline__ float4 operator()(const float *p) const {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)((p - base) * 4), 0,
                                                          kCacheDevice);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                       __uint_as_float(v.w));
  }
};

// The reduce of one unit (one temporal block) by the NT threads of its last
// state workgroup: thread t owns the four-float slots i4 = 4 (t + k NT),
// k = 0..K-1, of the d*d + d state vector.  The loads of all its slots are
// interleaved, kBatch partials of every slot in flight at once, while each
// float still adds the C partials in chunk order from its start value (the
// carried cache or 0), so the sums are bitwise those of reduce_prefix_values
// (one slot after another, with C / 8 round trips each, this left the other
// compute units idle for about a dozen memory latencies at the end of a
// small call).
template <int D, int NT>
__device__ __forceinline__ void fused_reduce_unit(const FusedReduce &fz, const float *partials,
                                                  int64_t unit, int64_t C) {
  constexpr int64_t stride = (int64_t)D * D + D;
  constexpr int K = (int)((stride + 4 * NT - 1) / (4 * NT));
  constexpr int kBatch = 4;
  const float *base = partials + unit * C * stride;
  const DeviceLoad4 load{head_rows_rsrc(reinterpret_cast<const uint16_t *>(base),
                                        (uint32_t)(C * stride * 4)),
                         base};
  const int tid = threadIdx.x;
  float4 run[K];
  int i4[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    i4[k] = 4 * (tid + k * NT);
    run[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (fz.S_in != nullptr && i4[k] < stride) {
      const float *c = cache_ptr(const_cast<float *>(fz.S_in), const_cast<float *>(fz.z_in),
                                 unit, i4[k], D);
      run[k] = make_float4(c[0], c[1], c[2], c[3]);
    }
  }
  for (int64_t c0 = 0; c0 < C; c0 += kBatch) {
    float4 x[kBatch][K];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t cj = c0 + j < C ? c0 + j : C - 1;  // clamped: loaded, not added
#pragma unroll
      for (int k = 0; k < K; ++k) x[j][k] = load(base + cj * stride + (i4[k] < stride ? i4[k] : 0));
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (c0 + j < C) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
          run[k].x += x[j][k].x;
          run[k].y += x[j][k].y;
          run[k].z += x[j][k].z;
          run[k].w += x[j][k].w;
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (i4[k] >= stride) continue;
    store_state4(run[k], fz.states, fz.frags, unit, D, i4[k]);
    if (fz.S_out != nullptr) {
      float *c = cache_ptr(fz.S_out, fz.z_out, unit, i4[k], D);
      c[0] = run[k].x;
      c[1] = run[k].y;
      c[2] = run[k].z;
      c[3] = run[k].w;
    }
  }
}

// ---------------------------------------------------------------- state

// Workgroups of the state kernel: twelve waves at d = 128 (one workgroup per
// compute unit), six at d = 64 (two per CU).  Two thirds of the waves are
// producers, one third consumers (below).  Waves w, w + NWV/3 and
// w + 2 NWV/3 of a workgroup share a SIMD, so every SIMD runs two producers
// and one consumer: the consumers' matrix-core products overlap the
// producers' vector work.  One workgroup per CU with several 64-token steps
// of k and v in flight reads the two tensors faster than two workgroups per
// CU with one step each (measured at 720p/81f: about 188 against 206 us for
// the reads alone).
template <int D>
constexpr int kStateThreads = D == 128 ? 768 : 384;
// 64-token steps of k and v in flight per producer thread (three rather than
// two: -2.5% per call over calls 5-24 at 720p/81f, where the shader clock is
// low; unchanged at the settled clock)
constexpr int kStatePrefetch = 3;

template <int D>
struct StateCfg {
  static constexpr int NT = kStateThreads<D>;
  static constexpr int NWV = NT / 64;                // waves
  static constexpr int NCW = NWV / 3;                // consumer waves
  static constexpr int NPW = NWV - NCW;              // producer waves
  static constexpr int FPT = D / 8;                  // threads per token row (16 B each)
  static constexpr int TPP = NPW * 64 / FPT;         // tokens per load pass
  static constexpr int R = (int)kStateTile / TPP;    // passes per step
  static constexpr int TPW = D / 32;                 // tiles per consumer wave (one row of tiles)
  static constexpr int ROW = 2 * D;                  // bytes per token row
  static constexpr int OP_BYTES = (int)kStateTile * ROW;
  static constexpr int SET_BYTES = 3 * OP_BYTES;     // one set of operand tiles
  static constexpr int POS_BYTES = (int)kStateTile * 16;  // one step of token positions
  static_assert(NCW * 32 == D, "consumer wave w owns row w of the 32x32 output tiles");
  static_assert(R * TPP == (int)kStateTile, "whole passes per step");
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

// One workgroup per (unit, chunk), 64-token steps, one barrier per step
// ("round" i below).  In round i the producer waves take the k and v rows of
// step i from registers (16 B per thread per row, whole rows per load
// instruction), apply ReLU (accumulating z) and RoPE to k in fp32, write
// RoPE(phi(k)) split into bf16 hi + lo parts, and v (exact in bf16), as
// row-major tiles into LDS set i % 2, and refill the registers with the rows
// kStatePrefetch steps ahead.  Meanwhile the consumer waves read the operands
// of step i - 1 transposed from set (i - 1) % 2 (four tokens of one feature
// per lane and read) and accumulate S = hi^T v + lo^T v on the matrix cores,
// each wave one row of 32x32 tiles; consumer wave 0 also writes the grid
// positions of step i + 1's tokens, as offsets into the RoPE table slice, to
// LDS (integer divisions the producers would otherwise repeat per feature
// unit).  Set i % 2 and positions (i + 1) % 2 are complete after barrier i;
// set (i - 1) % 2, which round i + 1 writes, was consumed before it.
//
// kBeta: the write gate ("SANA-Video 2.0" Eq. (1)): beta [B, N, H] scales each
// token's rotated key before it enters S (z keeps the plain phi(k)).
template <int D, bool kBeta>
__global__ __launch_bounds__(kStateThreads<D>, 3) void state_mfma_kernel(
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const uint16_t *__restrict__ beta, const float2 *__restrict__ tab,
    float *__restrict__ partials, MArgs a, FusedReduce fz) {
  using Cfg = StateCfg<D>;
  constexpr int FPT = Cfg::FPT, TPP = Cfg::TPP, R = Cfg::R, ROW = Cfg::ROW, TPW = Cfg::TPW;
  constexpr int P = kStatePrefetch;
  extern __shared__ __align__(16) unsigned char lds[];
  // set s: RoPE(phi(k)) hi part, lo part, v at lds + s * SET_BYTES; then the
  // two position buffers, then the table slice
  unsigned char *s_pos = lds + 2 * Cfg::SET_BYTES;
  float2 *s_tab = reinterpret_cast<float2 *>(s_pos + 2 * Cfg::POS_BYTES);

  const int64_t wg = blockIdx.x;
  const int64_t unit = wg / a.C, c = wg % a.C;
  const int64_t bh = unit / a.nb, blk = unit % a.nb;
  const int64_t b = bh / a.H, hd = bh % a.H;
  const int64_t n_begin = blk * a.L + c * a.Lc;
  const int64_t n_end = min(n_begin + a.Lc, (blk + 1) * a.L);
  const int64_t steps = (n_end - n_begin + kStateTile - 1) / kStateTile;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
  const bool producer = wave < Cfg::NPW;

  // producers: rows tg + TPP*r of a step, 16-byte unit fc
  const int fc = tid % FPT, tg = (tid / FPT) % TPP;
  const int wr_off = Cfg::off(tg, fc);

  // consumers: output tiles (cw, t), t = 0..TPW-1, and their transposing-read
  // offsets: lane l (group g = l/16, s = l%16) points at row 8*(g/2) + s/4
  // (+ 16*ks + 4*half), column 32*tile + 16*(g%2) + 4*(s%4)
  const int cw = producer ? 0 : wave - Cfg::NPW;
  int rd_p, rd_e[TPW];
  {
    const int g = lane >> 4, sl = lane & 15;
    const int rrow = 8 * (g >> 1) + (sl >> 2);
    const int cp = 32 * cw + 16 * (g & 1) + 4 * (sl & 3);
    rd_p = Cfg::off(rrow, cp >> 3) + ((cp & 7) << 1);
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int ce = 32 * t + 16 * (g & 1) + 4 * (sl & 3);
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
  // producers: ring of P steps of rows in registers
  uint4 kr[P][R], vr[P][R];
  uint32_t br[P][R];
  auto load_rows = [&](auto js, int64_t n0) {
    constexpr int j = decltype(js)::value;
    const uint32_t base = (uint32_t)(n0 - n_begin) * row_bytes + my_off;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      kr[j][r] = buf_load16<kStateLoadPolicy>(rk, base + (uint32_t)(TPP * r) * row_bytes);
      vr[j][r] = buf_load16<kStateLoadPolicy>(rv, base + (uint32_t)(TPP * r) * row_bytes);
      if (kBeta)
        br[j][r] = __builtin_amdgcn_raw_buffer_load_b16(
            rb, (int)(((uint32_t)(n0 - n_begin) + tg + TPP * r) * (uint32_t)a.H * 2), 0, 0);
    }
  };
  // consumer wave 0: the table offsets of step i's 64 tokens along each axis
  // (t, h, w rows; the slice's row bases are added by the reader)
  constexpr int gt = D / 32, gh = 3 * D / 64;  // groups per t row, per h or w row
  // (rows past the chunk take its last token's position; they read as zero
  // anyway).  Where a grid row holds at least the step's 64 tokens, the
  // step's first token is divided on the scalar unit and each lane carries
  // from it (no quarter-rate multiplies on this wave, whose SIMD also runs
  // two producers).
  auto write_pos = [&](int64_t i) {
    const int64_t n0 = n_begin + i * kStateTile;
    int t, h, w;
    if (a.Ws >= kStateTile)
      block_token_pos<true>(a, n0, n_end, lane, t, h, w);
    else
      block_token_pos<false>(a, n0, n_end, lane, t, h, w);
    *reinterpret_cast<int4 *>(s_pos + (int)(i & 1) * Cfg::POS_BYTES + 16 * lane) =
        make_int4((int)__umul24((unsigned)t, gt), (int)__umul24((unsigned)h, gh),
                  (int)__umul24((unsigned)w, gh), 0);
  };

  // The table slice goes to LDS while the first steps' rows are in flight:
  // its loads, then the rows' loads, then its stores (which wait for the
  // older table loads alone).  The compiler-only barriers keep the two groups
  // of loads in that order.
  TabLoad<D> tload;
  tload.issue(tab, a, n_begin, n_end);
  asm volatile("" ::: "memory");
  static_assert(P == 2 || P == 3, "the ring holds two or three steps");
  if (producer) {
    load_rows(std::integral_constant<int, 0>{}, n_begin);
    load_rows(std::integral_constant<int, 1>{}, n_begin + kStateTile);
    if constexpr (P == 3) load_rows(std::integral_constant<int, P - 1>{}, n_begin + 2 * kStateTile);
  }
  asm volatile("" ::: "memory");
  tload.store(s_tab, tab);
  if (!producer && cw == 0) write_pos(0);
  // a producer thread's table group: slice base of its axis and pair group,
  // plus the token's offset along that axis
  int axis, pia;
  pair_axis<D>(4 * fc, axis, pia);
  const int tab_base = tload.ts.lookup(axis, pia).base;
  const TabSlice<D> ts = tload.ts;
  __syncthreads();  // the table slice and the first positions are in LDS

  f32x16 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
  float zacc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) zacc[j] = 0.f;

  // The two roles run loops of their own with one barrier per round, steps +
  // 1 rounds each (a barrier counts waves, wherever in the code they wait),
  // so that neither role's registers stay live in the other's loop.
  if (producer) {
    // round i: step i (ring slot i % P) into set i % 2
    auto round = [&](auto js, int64_t i) {
      constexpr int j = decltype(js)::value;
      if (i < steps) {
        unsigned char *s_kh = lds + (int)(i & 1) * Cfg::SET_BYTES;
        unsigned char *s_kl = s_kh + Cfg::OP_BYTES;
        unsigned char *s_v = s_kh + 2 * Cfg::OP_BYTES;
        const int *pos = reinterpret_cast<const int *>(s_pos + (int)(i & 1) * Cfg::POS_BYTES);
        const int64_t n0 = n_begin + i * kStateTile;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int grp = tab_base + pos[4 * (tg + TPP * r) + axis];
          const uint32_t kw[4] = {kr[j][r].x, kr[j][r].y, kr[j][r].z, kr[j][r].w};
          float x[8];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const uint32_t rl = relu_bf16x2(kw[m]);
            x[2 * m] = lo_bf16(rl);
            x[2 * m + 1] = hi_bf16(rl);
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) zacc[q] += x[q];
          float2 c4[4];
          ts.read(s_tab, grp, c4);
          rotate4(x, c4);
          if (kBeta) {
            const float bt = bf16_bits_to_float(br[j][r]);
#pragma unroll
            for (int q = 0; q < 8; ++q) x[q] *= bt;
          }
          uint4 hi, lo;
          split_bf16x2(x[0], x[1], hi.x, lo.x);
          split_bf16x2(x[2], x[3], hi.y, lo.y);
          split_bf16x2(x[4], x[5], hi.z, lo.z);
          split_bf16x2(x[6], x[7], hi.w, lo.w);
          const int o = wr_off + r * TPP * ROW;
          *reinterpret_cast<uint4 *>(s_kh + o) = hi;
          *reinterpret_cast<uint4 *>(s_kl + o) = lo;
          *reinterpret_cast<uint4 *>(s_v + o) = vr[j][r];
        }
        // unconditional (rows past the chunk read as zeros): a conditional
        // load here would make the compiler wait for it at the join
        load_rows(js, n0 + P * kStateTile);
      }
      __syncthreads();
    };
    for (int64_t i = 0; i <= steps; i += P) {
      round(std::integral_constant<int, 0>{}, i);
      if (i + 1 > steps) break;
      round(std::integral_constant<int, 1>{}, i + 1);
      if constexpr (P == 3) {
        if (i + 2 > steps) break;
        round(std::integral_constant<int, P - 1>{}, i + 2);
      }
    }
  } else {
    // round i: positions of step i + 1, products of step i - 1
    for (int64_t i = 0; i <= steps; ++i) {
      if (cw == 0 && i + 1 < steps) write_pos(i + 1);
      if (i >= 1) {
        const unsigned char *s_kh = lds + (int)((i - 1) & 1) * Cfg::SET_BYTES;
        const unsigned char *s_kl = s_kh + Cfg::OP_BYTES;
        const unsigned char *s_v = s_kh + 2 * Cfg::OP_BYTES;
#pragma unroll
        for (int ks = 0; ks < (int)kStateTile / 16; ++ks) {
          const int o0 = (16 * ks) * ROW, o1 = (16 * ks + 4) * ROW;
          const uint2 h0 = lds_read_tr16(s_kh + rd_p + o0), h1 = lds_read_tr16(s_kh + rd_p + o1);
          const uint2 l0 = lds_read_tr16(s_kl + rd_p + o0), l1 = lds_read_tr16(s_kl + rd_p + o1);
          const bf16x8 fa = __builtin_bit_cast(bf16x8, make_uint4(h0.x, h0.y, h1.x, h1.y));
          const bf16x8 fl = __builtin_bit_cast(bf16x8, make_uint4(l0.x, l0.y, l1.x, l1.y));
          bf16x8 fb[TPW];
#pragma unroll
          for (int t = 0; t < TPW; ++t) {
            const uint2 v0 = lds_read_tr16(s_v + rd_e[t] + o0), v1 = lds_read_tr16(s_v + rd_e[t] + o1);
            fb[t] = __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
          }
          // the lo products of all tiles, then the hi products: no product
          // waits for the one just issued
#pragma unroll
          for (int t = 0; t < TPW; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fl, fb[t], acc[t], 0, 0, 0);
#pragma unroll
          for (int t = 0; t < TPW; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb[t], acc[t], 0, 0, 0);
        }
      }
      __syncthreads();
    }
  }

  // The partials are written with device-scope stores (through to memory,
  // past this XCD's L2), so that the unit's last workgroup, on any XCD, reads
  // them with device-scope loads and no whole-cache fence.
  float *dst = partials + wg * (int64_t)(D * D + D);
  float *zs = reinterpret_cast<float *>(lds);
  if (producer) {
    // z_c: per-thread sums over its tokens, then a fixed-order sum over the
    // TPP token groups (the operand sets are no longer read)
#pragma unroll
    for (int j = 0; j < 8; ++j) zs[tg * D + 8 * fc + j] = zacc[j];
  } else {
    // S_c, row-major: lanes 0..31 write 32 consecutive floats of one row
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int p = 32 * cw + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        const int e = 32 * t + (lane & 31);
        __hip_atomic_store(dst + p * D + e, acc[t][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
    for (int gidx = 0; gidx < TPP; ++gidx) s += zs[gidx * D + tid];
    __hip_atomic_store(dst + D * D + tid, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (fz.cnt != nullptr) {
    // The unit's last workgroup to finish sums its C partials (the reduce
    // stage, folded in).  Each thread waits until its device-scope stores
    // are complete, then one thread counts the workgroup done; the count
    // only picks which workgroup sums, never the order of the sums.
    __shared__ unsigned s_last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const unsigned before = __hip_atomic_fetch_add(fz.cnt + unit, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
      s_last = before == (unsigned)(a.C - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (s_last != 0u) {
      fused_reduce_unit<D, Cfg::NT>(fz, partials, unit, a.C);
      if (tid == 0)
        __hip_atomic_store(fz.cnt + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // prefetches past the chunk are still in flight
}

template <int D, bool kBeta>
hipError_t state_d(const Plan &p, const void *k, const void *v, const void *beta,
                   const float2 *tab, float *part, const FusedReduce &fz, hipStream_t stream) {
  const size_t lds = state_mfma_lds_bytes(p);
  auto kern = state_mfma_kernel<D, kBeta>;
  const hipError_t e = lds_limit_once((const void *)kern);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.units * p.C)), dim3(StateCfg<D>::NT), lds, stream,
                     (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)beta, tab, part,
                     make_margs(p), fz);
  return hipGetLastError();
}

}  // namespace

hipError_t state_mfma_lds_limits() {
  return lds_limits({(const void *)state_mfma_kernel<128, false>,
                     (const void *)state_mfma_kernel<128, true>,
                     (const void *)state_mfma_kernel<64, false>,
                     (const void *)state_mfma_kernel<64, true>});
}

size_t state_mfma_lds_bytes(const Plan &p) {
  const size_t ops = p.d == 128 ? 2 * (StateCfg<128>::SET_BYTES + StateCfg<128>::POS_BYTES)
                                 : 2 * (StateCfg<64>::SET_BYTES + StateCfg<64>::POS_BYTES);
  return ops + tab_slice_entries(p, p.Lc) * sizeof(float2);
}

hipError_t launch_state_mfma(const Plan &p, const void *k, const void *v, const void *beta,
                             const float2 *tab, float *partials, const FusedReduce &fuse,
                             hipStream_t stream) {
  if (fuse.cnt != nullptr && p.nb != 1) return hipErrorInvalidValue;
  if (p.d == 128)
    return beta ? state_d<128, true>(p, k, v, beta, tab, partials, fuse, stream)
                : state_d<128, false>(p, k, v, beta, tab, partials, fuse, stream);
  if (p.d == 64)
    return beta ? state_d<64, true>(p, k, v, beta, tab, partials, fuse, stream)
                : state_d<64, false>(p, k, v, beta, tab, partials, fuse, stream);
  return hipErrorInvalidValue;
}

}  // namespace gla
