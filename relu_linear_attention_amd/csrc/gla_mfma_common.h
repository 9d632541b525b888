// Helpers of the matrix-core kernels (gfx950): vector types, buffer
// resources over a head's rows, bf16 packing and hi/lo splitting, the RoPE
// table slice kept in LDS, the transposing LDS read, and the LDS layout of
// the bf16 parts of S.  Included by the matrix-core translation units only;
// everything here has internal linkage.
#pragma once

#include <hip/hip_runtime.h>

#include <mutex>
#include <utility>
#include <vector>

#include "gla_internal.h"

namespace gla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

struct MArgs {
  int64_t N, H, Hs, Ws;
  int64_t nb, L, C, Lc, R, Lr;
  int64_t hpw, ag, ar, air, am;  // the output stage's work layout (Plan)
  int64_t tab_h_off;  // global entry offset of the h rows (the w rows follow)
  FastDiv div_hw, div_w;  // by Hs*Ws and by Ws (token indices < 2^31)
  float eps;
  float rms_eps;  // epsilon of the optional RMSNorm of num/den
};

// Buffer resource over the rows of one head for a token range: byte 0 is
// feature 0 of the first token, row r starts at r * row_bytes, and the
// range ends after the last token's d features.  Loads past the end return
// zeros and stores past the end are dropped by the hardware, so ragged token
// tiles need neither masks nor branches.  (Raw buffer, stride 0; the last
// descriptor word selects 32-bit untyped data.)
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rows_rsrc(const uint16_t *first_row,
                                                                 uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(first_row), 0, (int)bytes,
                                           0x00020000);
}
// Cache policy of a buffer access: kCacheNormal, or kCacheStream for data
// touched exactly once (the non-temporal hint: the line is not kept for
// reuse).
constexpr int kCacheNormal = 0;
constexpr int kCacheStream = 2;
template <int Policy = kCacheNormal>
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, Policy);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <int Policy = kCacheNormal>
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 x) {
  const u32x4 v = {x.x, x.y, x.z, x.w};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, Policy);
}

// Buffer resource over the rows [n, n + 16) of one head that lie inside
// [.., n_end): rows past n_end (and whole tiles past it) read as zeros and
// are not written.  `base` points at feature 0 of row n.  Every input is
// uniform across the wave; the values pass through readfirstlane so that the
// compiler keeps the descriptor in scalar registers (a descriptor it
// believes divergent costs a loop around every access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t *base, int64_t n,
                                                            int64_t n_end, uint32_t row_bytes,
                                                            int D) {
  // rows = clamp(n_end - n, 0, 16) from the 32-bit halves of the difference,
  // so that the comparisons stay on the scalar unit (it has no 64-bit
  // ordered compares; the vector unit's would also pull the multiply below
  // onto a quarter-rate vector instruction)
  const int64_t left = n_end - n;
  int32_t left_hi = __builtin_amdgcn_readfirstlane((int32_t)(left >> 32));
  uint32_t left_lo = __builtin_amdgcn_readfirstlane((uint32_t)left);
  asm("" : "+s"(left_hi), "+s"(left_lo));  // opaque: not folded back into a 64-bit compare
  const uint32_t rows = left_hi < 0 ? 0u : (left_hi > 0 || left_lo >= 16u ? 16u : left_lo);
  // (rows - 1) * row_bytes + 2 D, or 0 without rows
  int32_t bytes = max((int32_t)(rows * row_bytes) - (int32_t)(row_bytes - 2u * (uint32_t)D), 0);
  asm("" : "+s"(bytes));  // computed and kept on the scalar unit
  const uint64_t addr = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
  const uint16_t *p = (const uint16_t *)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(p), 0, (int)bytes,
                                           0x00020000);
}

// 8-byte buffer accesses (four bf16 of one token row)
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kCacheNormal);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2 x) {
  const u32x2 v = {x.x, x.y};
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, kCacheNormal);
}

// Sixteen wait states after the last matrix-core instruction of an
// accumulation chain, with the scheduler kept from moving anything across:
// the vector instructions that follow may read the chain's result.  (Without
// it the compiler let a vector read of an 8-pass v_mfma_f32_16x16x32_bf16
// result follow a branch one wait state after the instruction issued, and
// the read saw the previous value.)
__device__ __forceinline__ void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Token index (within a batch entry, < 2^31) -> (t, h, w) of the t-major grid.
__device__ __forceinline__ void token_pos(const MArgs &a, int64_t n, int &t, int &h, int &w) {
  const uint32_t u = (uint32_t)n;
  const uint32_t tt = a.div_hw.div(u);
  const uint32_t r = u - tt * a.div_hw.d;
  const uint32_t hh = a.div_w.div(r);
  t = (int)tt;
  h = (int)hh;
  w = (int)(r - hh * a.div_w.d);
}

// Grid position of the token t0 + o, for a block of tokens that starts at
// token t0 (uniform across the wave) and a lane offset o (tokens past the
// range take the position of its last token, n_end - 1).  kCarry (the
// caller guarantees o < Ws, the tokens of a grid row): the block's first
// token is divided once on the scalar unit and each lane adds its offset
// with at most one carry into h and one into t; otherwise each lane divides
// its own index.  Token indices are below 2^31.
template <bool kCarry>
__device__ __forceinline__ void block_token_pos(const MArgs &a, int64_t t0, int64_t n_end, int o,
                                                int &t, int &h, int &w) {
  const uint32_t last = (uint32_t)(n_end - 1);
  const uint32_t f0 = __builtin_amdgcn_readfirstlane((uint32_t)t0);
  const uint32_t n = min(f0 + (uint32_t)o, last);
  if constexpr (kCarry) {
    const uint32_t first = f0 < last ? f0 : last;
    int t0p, h0p, w0p;
    token_pos(a, first, t0p, h0p, w0p);
    const int ws = (int)a.div_w.d, hs = (int)a.Hs;
    w = w0p + (int)(n - first);
    const bool cw = w >= ws;
    w = cw ? w - ws : w;
    h = h0p + (cw ? 1 : 0);
    const bool ch = h >= hs;
    h = ch ? h - hs : h;
    t = t0p + (ch ? 1 : 0);
  } else {
    token_pos(a, n, t, h, w);
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 h = __builtin_convertvector(f, bf16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

// ReLU of two packed bf16 values: a bf16 is negative exactly when its sign
// bit is set, so a signed 16-bit max with 0 keeps x >= 0 and maps x < 0
// (and -0) to +0.
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t x) {
  s16x2 v = __builtin_bit_cast(s16x2, x);
  s16x2 zero = {0, 0};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(v, zero));
}

// 0xffff in each 16-bit half of x that is nonzero, else 0, for x a packed
// pair of ReLU results (each half in 0..0x7f80): the mask of the elements
// with x > 0.  A nonzero half h has -h in 0x8080..0xffff, so the arithmetic
// shift of -h by 15 gives 0xffff, and 0 gives 0: two packed 16-bit ops.  (An
// empty register-only asm between them keeps the compiler from turning the
// pair into per-half compares and selects, four to five instructions.)
__device__ __forceinline__ uint32_t nonzero_mask16(uint32_t x) {
  s16x2 neg = s16x2{0, 0} - __builtin_bit_cast(s16x2, x);
  asm("" : "+v"(neg));
  return __builtin_bit_cast(uint32_t, neg >> s16x2{15, 15});
}

__device__ __forceinline__ float lo_bf16(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Split two floats into packed bf16 hi parts (round to nearest even) and
// packed bf16 lo parts, the rounded remainders: x ~ hi + lo to about 16
// significant bits.
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16x2(x0, x1);
  lo = pack_bf16x2(x0 - lo_bf16(hi), x1 - hi_bf16(hi));
}

// Feature pair P0 (a multiple of 4) -> axis (0 t, 1 h, 2 w) and the pair's
// index within that axis.  For d = 64 and 128 a group of four pairs never
// straddles two axes.
template <int D>
__device__ __forceinline__ void pair_axis(int P0, int &axis, int &pia) {
  constexpr int pt = D / 8, ph = 3 * D / 16;
  if (P0 < pt) {
    axis = 0; pia = P0;
  } else if (P0 < pt + ph) {
    axis = 1; pia = P0 - pt;
  } else {
    axis = 2; pia = P0 - pt - ph;
  }
}

// LDS copy of the RoPE table rows a workgroup touches: the h rows and the w
// rows (both whole), then the temporal rows t_lo..t_hi of its token range.
// A lane always needs the (cos, sin) entries of four consecutive pairs (a
// "group"; every axis row holds a whole number of groups).  The slice is
// stored as two planes of 16-byte units, pairs 0-1 of every group in the
// first and pairs 2-3 in the second, so that lanes reading neighbouring
// groups read neighbouring 16-byte units (the direct 32-byte layout leaves
// half the LDS banks idle and serialises on the other half).
template <int D>
struct TabSlice {
  int sp_groups;  // (Hs + Ws) * 3D/64 groups of the spatial rows
  int groups;     // groups in the slice (size of one plane)
  int Hs;
  int t_lo;
  // Group of the pair group pia/4 of an axis at grid position (t, h, w):
  // g = base + t*mt + h*mh + w*mw.  Written as arithmetic (two of the
  // multipliers are 0) so that the compiler cannot turn the axis choice into
  // a divergent branch, which would make it wait for every outstanding load
  // at the join.
  struct Lookup {
    int base, mt, mh, mw;
    // 24-bit multiplies (full rate; grid positions and multipliers are far
    // below 2^24)
    __device__ __forceinline__ int at(int t, int h, int w) const {
      return base + (int)(__umul24((unsigned)t, (unsigned)mt) + __umul24((unsigned)h, (unsigned)mh) +
                          __umul24((unsigned)w, (unsigned)mw));
    }
  };
  __device__ __forceinline__ Lookup lookup(int axis, int pia) const {
    constexpr int gt = D / 32, gh = 3 * D / 64;  // groups per t row, per h or w row
    Lookup l;
    l.mt = axis == 0 ? gt : 0;
    l.mh = axis == 1 ? gh : 0;
    l.mw = axis == 2 ? gh : 0;
    l.base = pia / 4 + (axis == 0 ? sp_groups - t_lo * gt : (axis == 2 ? Hs * gh : 0));
    return l;
  }
  // the four (cos, sin) entries of group g
  __device__ __forceinline__ void read(const float2 *s_tab, int g, float2 (&c4)[4]) const {
    const float4 a = reinterpret_cast<const float4 *>(s_tab)[g];
    const float4 b = reinterpret_cast<const float4 *>(s_tab)[groups + g];
    c4[0] = make_float2(a.x, a.y);
    c4[1] = make_float2(a.z, a.w);
    c4[2] = make_float2(b.x, b.y);
    c4[3] = make_float2(b.z, b.w);
  }
};

// Copy of the table rows of tokens [n_begin, n_end) into LDS in two parts:
// issue() loads the first kBatch entries per thread into registers, store()
// writes them to s_tab and copies any further entries.  A kernel issues the
// first loads of its main loop (and any other set-up loads) between the two,
// so that their HBM latency overlaps the table's: the stores wait only for
// the older table loads.  Indices are clamped so that every load is
// unconditional.
template <int D, int kBatch = 8>
struct TabLoad {
  TabSlice<D> ts;
  int sp_entries, entries;
  int64_t h_off, t_off;
  float2 v[kBatch];
  __device__ __forceinline__ float2 fetch(const float2 *__restrict__ tab, int i) const {
    return i < sp_entries ? tab[h_off + i] : tab[t_off + (i - sp_entries)];
  }
  // entry i = pair i % 4 of group i / 4
  __device__ __forceinline__ int slot(int i) const {
    return (i & 2) * ts.groups + 2 * (i >> 2) + (i & 1);
  }
  __device__ __forceinline__ void issue(const float2 *__restrict__ tab, const MArgs &a,
                                        int64_t n_begin, int64_t n_end) {
    constexpr int ph = 3 * D / 16;
    const int64_t hw = a.Hs * a.Ws;
    ts.Hs = (int)a.Hs;
    sp_entries = (int)((a.Hs + a.Ws) * ph);
    ts.sp_groups = sp_entries / 4;
    ts.t_lo = (int)(n_begin / hw);
    const int t_hi = (int)((n_end - 1) / hw);
    entries = sp_entries + (t_hi - ts.t_lo + 1) * (D / 8);
    ts.groups = entries / 4;
    h_off = a.tab_h_off;
    t_off = (int64_t)ts.t_lo * (D / 8);
    const int nt = blockDim.x;
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      v[j] = fetch(tab, min((int)threadIdx.x + j * nt, entries - 1));
  }
  __device__ __forceinline__ void store(float2 *s_tab, const float2 *__restrict__ tab) const {
    const int nt = blockDim.x;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = (int)threadIdx.x + j * nt;
      if (i < entries) s_tab[slot(i)] = v[j];
    }
    for (int i = (int)threadIdx.x + kBatch * nt; i < entries; i += nt) s_tab[slot(i)] = fetch(tab, i);
  }
};

template <int D>
__device__ TabSlice<D> load_tab_slice(float2 *s_tab, const float2 *__restrict__ tab,
                                      const MArgs &a, int64_t n_begin, int64_t n_end) {
  TabLoad<D> tl;
  tl.issue(tab, a, n_begin, n_end);
  tl.store(s_tab, tab);
  return tl.ts;
}

// The gradient of a rotated operand, in the B-operand layout of the
// feature: lane (token, kg) holds features 32 ks + 8 kg + 4 half + i in
// value i of a[half] (half = 0, 1), the pairs' (cos, sin) entries in cs[0..3].
// Returns RoPE^T(a) + add, zero where the packed ReLU words relu[0..3] are
// zero, as eight packed bf16.
__device__ __forceinline__ uint4 rope_t_add_mask(const f32x4 &a0, const f32x4 &a1,
                                                 const float2 (&cs)[4], const float (&add)[8],
                                                 const uint32_t (&relu)[4]) {
  float o[8];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const f32x4 d4 = half ? a1 : a0;
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const float2 c = cs[2 * half + pr];
      const float d0 = d4[2 * pr], d1 = d4[2 * pr + 1];
      const int j = 4 * half + 2 * pr;
      o[j] = d0 * c.x + __builtin_fmaf(d1, c.y, add[j]);
      o[j + 1] = d1 * c.x - __builtin_fmaf(d0, c.y, -add[j + 1]);
    }
  }
  uint32_t w[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) w[m] = pack_bf16x2(o[2 * m], o[2 * m + 1]) & nonzero_mask16(relu[m]);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Rotate four adjacent pairs x[0..7] by the (cos, sin) entries cs[0..3].
__device__ __forceinline__ void rotate4(float *x, const float2 *cs) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float2 c = cs[i];
    const float x0 = x[2 * i], x1 = x[2 * i + 1];
    x[2 * i] = x0 * c.x - x1 * c.y;
    x[2 * i + 1] = x0 * c.y + x1 * c.x;
  }
}

// Transposing LDS read of gfx950 (ds_read_b64_tr_b16).  Within each group of
// 16 lanes, lane s supplies the address of a row of four 16-bit values
// M[s][0..3], and lane i receives M[i/4 + 4k][i%4] for k = 0..3.  With lane
// s pointing at row tok0 + s/4, column c0 + 4*(s%4) of a row-major
// [token][feature] tile, lane i receives X[tok0 + k][c0 + i], k = 0..3: four
// consecutive tokens of one feature, half of the eight a lane contributes to
// a matrix-core operand whose contraction runs over tokens.  This read moves
// 512 B in two LDS cycles (plain 16-byte reads: 1 KiB in four).
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char *p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(p));
  return __builtin_bit_cast(uint2, r);
}

// LDS layout of the S parts in the apply stage: row-major [p][e] bf16 with
// the 16-byte units of row p XOR-permuted by f(p).  The A operand of the
// 16x16x32 instruction (S^T: rows e, columns p) is read with the transposing
// LDS read: lane s of a 16-lane group points at row p0 + s/4, column
// e0 + 4*(s%4), and lane i receives S[p0 + k][e0 + i], k = 0..3.  A read
// touches rows p0..p0+3 and p0+8..p0+11 per 32 lanes, 32 B each; f gives
// those eight rows distinct unit pairs, so a read covers all banks once.
// f depends only on row bits that the k-step and half offsets (multiples of
// 4 rows, bit 3 untouched) leave alone.
template <int D>
struct SRow {
  static __device__ __forceinline__ int f(int row) {
    return D == 128 ? 2 * ((row & 3) + 4 * ((row >> 3) & 1))
                    : 2 * (((row >> 1) & 1) + 2 * ((row >> 3) & 1));
  }
  static __device__ __forceinline__ int off(int row, int unit) {
    return row * (2 * D) + ((unit ^ f(row)) << 4);
  }
};

// LDS layout of token tiles (the rows of one step of tokens): row-major
// [token][feature] bf16, the 16-byte units of row r XOR-permuted by f(r),
// which depends on row bits 0-3 only.  The transposing reads of these tiles
// serve 32 lanes per LDS cycle: two 16-lane groups, each on 4 consecutive
// rows and 2 adjacent units, either on the same rows and the next unit pair
// (the contractions over a step's tokens) or on the next 4 rows and the same
// units (scores x v).  At d = 128, f(r) = 4(r&3) + 2((r>>2)&1) + ((r>>3)&1)
// puts both pairs of groups on 16 distinct units (measured on MI355X with
// rocprofv3 SQ_LDS_BANK_CONFLICT: no conflict cycles for either, where the
// previous 4(r&3) + ((r>>2)&3) doubled the second pattern).  16-byte row
// pieces cost the same under any permutation.
template <int D>
struct KRow {
  static __device__ __forceinline__ int f(int row) {
    return D == 128 ? 4 * (row & 3) + 2 * ((row >> 2) & 1) + ((row >> 3) & 1)
                    : 2 * (row & 3) + ((row >> 2) & 1);
  }
  static __device__ __forceinline__ int off(int row, int unit) {
    return row * (2 * D) + ((unit ^ f(row)) << 4);
  }
};

// per-wave LDS staging tile of the epilogue: 16 token rows of D bf16, rows
// 2D + 16 bytes apart (an odd number of 16-byte units), so that the 16
// rows read by a fragment-wise 8-B access start in 16 different 4-bank
// groups and the row-wise 16-B accesses stay contiguous
template <int D>
struct Stage {
  static constexpr int kRowBytes = 2 * D + 16;
  static constexpr int kBytes = 16 * kRowBytes;
  static constexpr int kLanesPerRow = D / 8;             // 16 B per lane
  static constexpr int kRowsPerPass = 64 / kLanesPerRow;  // token rows per instruction
  static constexpr int kPasses = 16 / kRowsPerPass;
};

// Writes a wave's 16-token output tile to HBM as whole rows through its
// staging tile.  vals[et] holds four bf16 (packed) of token l % 16, features
// 16*et + 4*(l/16)..+3: the accumulator layout of a 16x16 product whose
// columns are tokens.  row_off is the byte offset of the tile's first token
// row in `dst`; rows past the resource's end are dropped.
template <int D, int Policy = kCacheNormal>
__device__ __forceinline__ void store_tile_rows(unsigned char *stage, const uint2 (&vals)[D / 16],
                                                __amdgpu_buffer_rsrc_t dst, uint32_t row_off,
                                                uint32_t row_bytes) {
  using St = Stage<D>;
  const int lane = threadIdx.x & 63, nl = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int et = 0; et < D / 16; ++et)
    *reinterpret_cast<uint2 *>(stage + nl * St::kRowBytes + 2 * (16 * et + 4 * kg)) = vals[et];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int rl = lane / St::kLanesPerRow, rc = 8 * (lane % St::kLanesPerRow);
#pragma unroll
  for (int i = 0; i < St::kPasses; ++i) {
    const int tok = i * St::kRowsPerPass + rl;
    const uint4 ov = *reinterpret_cast<const uint4 *>(stage + tok * St::kRowBytes + 2 * rc);
    buf_store16<Policy>(dst, row_off + (uint32_t)tok * row_bytes + 2 * rc, ov);
  }
  // the next writes into the tile must not overtake these reads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

inline MArgs make_margs(const Plan &p) {
  MArgs a;
  a.N = p.N; a.H = p.H; a.Hs = p.Hs; a.Ws = p.Ws;
  a.nb = p.nb; a.L = p.L; a.C = p.C; a.Lc = p.Lc; a.R = p.R; a.Lr = p.Lr;
  a.hpw = p.hpw; a.ag = p.ag; a.ar = p.ar; a.air = p.air; a.am = p.am;
  a.tab_h_off = p.tab_h_off;
  a.div_hw = FastDiv::make((uint32_t)(p.Hs * p.Ws));
  a.div_w = FastDiv::make((uint32_t)p.Ws);
  a.eps = p.eps;
  a.rms_eps = p.rms_eps;
  return a;
}

// LDS entries of the RoPE table slice for a token range of at most `len`
// tokens: the spatial rows plus the temporal rows it can span.
inline int64_t tab_slice_entries(const Plan &p, int64_t len) {
  const int64_t hw = p.Hs * p.Ws;
  const int64_t rows = (len + hw - 1) / hw + 1;
  return (p.Hs + p.Ws) * (3 * p.d / 16) + rows * (p.d / 8);
}

}  // namespace
}  // namespace gla
