// Matrix-core tile kernel of the token-causal form (bf16 tensors, head size
// 64 or 128; "SANA-Video" notes page, Section 3.4, the causal output of
// token i).  One workgroup (8 waves) per (batch, head, token range) walks its
// range in steps of 64 tokens, starting from the exclusive prefix of the
// chunk partials (S, z before the range).  For a step with the sums S, z of
// every earlier token:
//
//   num_i = RoPE(phi(q_i)) S + sum_{j in step, j<=i} (RoPE(phi(q_i)) . RoPE(phi(k_j))) v_j
//   den_i = phi(q_i) . z + sum_{j in step, j<=i} phi(q_i) . phi(k_j) + eps
//   o_i   = num_i / den_i * sigmoid(g_i)
//
// and then S, z take the step's keys.  S lives in fp32 matrix-core
// accumulators spread over the waves and, after every step, as bf16 hi + lo
// parts in LDS (the operand of the numerator, as in the non-causal apply
// stage).  Every bf16 product of a rotated or fp32 operand is split into hi
// + lo parts, which carries about 16 significant bits through the matrix
// cores: 3 products for RoPE(phi(q)) x S and for the intra-step scores,
// 2 for scores x v and for the state update (v and phi() are exact in bf16).
//
// Work of one step (64 tokens = 4 query tiles of 16):
//   prologue   all threads: k, v rows -> LDS tiles (RoPE(phi(k)) hi, lo,
//              phi(k), v); the step's phi(k) sums per wave; each wave turns
//              its query tile's q rows (loaded in the operand layout) into
//              phi(q) and RoPE(phi(q)) hi, lo in registers.
//   outputs    wave w: query tile qt(w), output features of half eh(w):
//              den, the intra-step scores against key tiles 0..qt (masked
//              on the diagonal tile) and num; after a barrier, the gate and
//              the store as whole half rows through the wave's piece of the
//              phi(k) tile.
//   state      S^T += v^T RoPE(phi(k)) (32x32 tiles, two per wave at
//              d = 128), published as bf16 hi + lo; z += the step's sums.

#include <hip/hip_runtime.h>

#include "gla_mfma_common.h"

namespace gla {
namespace {

constexpr int kCausalThreads = 512;  // 8 waves
constexpr int kCausalStep = 64;      // tokens per step

template <int D>
struct CausalCfg {
  static constexpr int NT = kCausalThreads;
  static constexpr int NW = NT / 64;
  static constexpr int STEP = kCausalStep;
  static constexpr int KS = D / 32;                 // 32-feature steps of a feature contraction
  static constexpr int ET = D / 16;                 // 16-feature output tiles
  static constexpr int ETW = ET / 2;                // output tiles per wave
  static constexpr int TILE = STEP * 2 * D;         // bytes of one step tile
  static constexpr int FPT = D / 8;                 // prologue threads per row (16 B each)
  static constexpr int TPP = NT / FPT;              // rows per prologue pass
  static constexpr int RP = STEP / TPP;             // prologue passes
  static constexpr int ST = (D / 32) * (D / 32);    // 32x32 tiles of S^T
  static constexpr int STW = ST >= NW ? ST / NW : 1;  // tiles per state wave
  static constexpr int SW = ST >= NW ? NW : ST;       // waves that hold S
  static constexpr size_t kFixedLds =
      (size_t)D * D * 4 + 4 * (size_t)TILE + (size_t)D * 4 + (size_t)NW * D * 4;
};

template <int D>
__global__ __launch_bounds__(kCausalThreads) void causal_mfma_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ g,
    const float *__restrict__ states, const float2 *__restrict__ tab,
    uint16_t *__restrict__ out, MArgs a) {
  using Cfg = CausalCfg<D>;
  constexpr int KS = Cfg::KS, ETW = Cfg::ETW, STEP = Cfg::STEP, NW = Cfg::NW;
  constexpr int FPT = Cfg::FPT, TPP = Cfg::TPP, RP = Cfg::RP, STW = Cfg::STW;
  constexpr int TILE = Cfg::TILE;
  extern __shared__ __align__(16) unsigned char lds[];
  unsigned char *s_sh = lds;                  // S hi, [p][e], units permuted (SRow)
  unsigned char *s_sl = lds + D * D * 2;      // S lo
  unsigned char *s_kh = lds + D * D * 4;      // RoPE(phi(k)) hi, [token][feature] (KRow)
  unsigned char *s_kl = s_kh + TILE;          // RoPE(phi(k)) lo
  unsigned char *s_kp = s_kl + TILE;          // phi(k)
  unsigned char *s_v = s_kp + TILE;           // v
  float *s_z = reinterpret_cast<float *>(s_v + TILE);  // z before the step (D)
  float *s_zp = s_z + D;                                // the step's phi(k) sums per wave (NW x D)
  float2 *s_tab = reinterpret_cast<float2 *>(s_zp + NW * D);

  const int64_t wg = blockIdx.x;
  const int64_t unit = wg / a.R, r = wg % a.R;
  const int64_t b = unit / a.H, hd = unit % a.H;
  const int64_t n_begin = r * a.Lr;
  const int64_t n_end = min(n_begin + a.Lr, a.N);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
  const int nl = lane & 15, kg = lane >> 4;
  // query tile and output half of this wave.  Waves w and w + 4 share a SIMD;
  // their query tiles (0 and 3, or 1 and 2) carry equal intra-step work.
  const int qt = wave < 4 ? wave : 7 - wave;
  const int eh = wave >> 2;

  const TabSlice<D> ts = load_tab_slice<D>(s_tab, tab, a, n_begin, n_end);

  // ---- the sums before the range: S^T tiles of this wave, and z
  const float *stt = states + wg * (int64_t)(D * D + D);
  const bool s_owner = wave < Cfg::SW;  // uniform
  int t_e[STW], t_p[STW];
  f32x16 sacc[STW];
#pragma unroll
  for (int t = 0; t < STW; ++t) {
    const int idx = wave * STW + t;
    t_e[t] = idx / (D / 32);
    t_p[t] = idx % (D / 32);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // C layout of the 32x32 products: value i of lane l is S^T[e][p]
      const int e = 32 * t_e[t] + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      const int p = 32 * t_p[t] + (lane & 31);
      sacc[t][i] = s_owner ? stt[p * D + e] : 0.f;
    }
  }
  // S -> bf16 hi + lo in LDS.  Lanes l and l + 32 hold e0..e0+3 and
  // e0+4..e0+7 of row p; one lane swap per dword (gfx950 permlane32 swap:
  // the upper half of its first operand trades places with the lower half of
  // its second) leaves the lower lane with the row's 16-byte hi unit and the
  // upper lane with its lo unit, one 16-byte store each (half the stores of
  // 8-byte pieces, and fewer bank conflicts).
  auto publish = [&]() {
    if (!s_owner) return;
    unsigned char *dst = s_sh + (lane >> 5) * (D * D * 2);  // hi, or lo (s_sl)
#pragma unroll
    for (int t = 0; t < STW; ++t) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int e0 = 32 * t_e[t] + 8 * i4;
        const int p = 32 * t_p[t] + (lane & 31);
        uint32_t h0, l0, h1, l1;
        split_bf16x2(sacc[t][4 * i4], sacc[t][4 * i4 + 1], h0, l0);
        split_bf16x2(sacc[t][4 * i4 + 2], sacc[t][4 * i4 + 3], h1, l1);
        const auto s0 = __builtin_amdgcn_permlane32_swap(h0, l0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(h1, l1, false, false);
        *reinterpret_cast<uint4 *>(dst + SRow<D>::off(p, e0 >> 3)) =
            make_uint4(s0[0], s1[0], s0[1], s1[1]);
      }
    }
  };
  publish();
  for (int i = tid; i < D; i += Cfg::NT) s_z[i] = stt[D * D + i];

  // ---- buffer resources over the range's rows (rows past the end read as
  // zeros, stores past it are dropped)
  const int64_t first = ((b * a.N + n_begin) * a.H + hd) * D;
  const uint32_t row_bytes = (uint32_t)(a.H * D * 2);
  const uint32_t range_bytes = (uint32_t)(n_end - n_begin - 1) * row_bytes + 2 * D;
  const __amdgpu_buffer_rsrc_t rq = head_rows_rsrc(q + first, range_bytes);
  const __amdgpu_buffer_rsrc_t rk = head_rows_rsrc(k + first, range_bytes);
  const __amdgpu_buffer_rsrc_t rv = head_rows_rsrc(v + first, range_bytes);
  const __amdgpu_buffer_rsrc_t rg = head_rows_rsrc(g + first, range_bytes);
  const __amdgpu_buffer_rsrc_t ro = head_rows_rsrc(out + first, range_bytes);

  // prologue mapping: rows tg + TPP*rr, 16-byte unit fc (features 8fc..8fc+7)
  const int fc = tid % FPT, tg = tid / FPT;
  int axis, pia;
  pair_axis<D>(4 * fc, axis, pia);
  const typename TabSlice<D>::Lookup tl = ts.lookup(axis, pia);

  // The gate comes in, and the output leaves, as whole half rows (the D/2
  // features of half eh of the wave's 16 tokens): pass i, lane l covers
  // token 16 qt + i*HRP + l/HU, 16-byte unit l%HU of the half row.  They
  // reach the accumulator layout through the wave's piece of the phi(k) tile
  // (free from the end of a step's outputs to the next step's prologue), 16
  // half rows of D bytes whose 16-byte units are XOR-permuted by hswz(row):
  // the 32 lanes of an 8-byte fragment access then fall on distinct banks.
  constexpr int HU = D / 16;      // 16-byte units of a half row
  constexpr int HRP = 64 / HU;    // half rows per pass
  constexpr int HP = 16 / HRP;    // passes
  auto hswz = [](int row) { return (row / (256 / D)) & (HU - 1); };
  uint4 kr[RP], vr[RP], qraw[KS];
  uint4 grow[HP];
  auto load_kvq = [&](int64_t n0) {
    const uint32_t rel = (uint32_t)(n0 - n_begin);
#pragma unroll
    for (int rr = 0; rr < RP; ++rr) {
      const uint32_t off = (rel + tg + TPP * rr) * row_bytes + 16 * fc;
      kr[rr] = buf_load16<kCacheStream>(rk, off);
      vr[rr] = buf_load16<kCacheStream>(rv, off);
    }
    // this wave's query tile in the B-operand layout: token nl, 16 bytes at
    // feature 32*ks + 8*kg
    const uint32_t qoff = (rel + 16 * qt + nl) * row_bytes + 16 * kg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qraw[ks] = buf_load16<kCacheNormal>(rq, qoff + 64 * ks);
  };
  const int hr = lane / HU, hc = lane % HU;  // whole-row mapping
  auto load_g = [&](int64_t n0) {
    const uint32_t goff =
        ((uint32_t)(n0 - n_begin) + 16 * qt + hr) * row_bytes + eh * D + 16 * hc;
#pragma unroll
    for (int i = 0; i < HP; ++i) grow[i] = buf_load16<kCacheStream>(rg, goff + i * HRP * row_bytes);
  };
  unsigned char *hs = s_kp + wave * (16 * D);  // this wave's half-row tile
  int hrow[HP], hfrag[ETW];
#pragma unroll
  for (int i = 0; i < HP; ++i) {
    const int row = i * HRP + hr;
    hrow[i] = row * D + 16 * (hc ^ hswz(row));
  }
  // accumulator layout: token nl, features 16*u + 4*kg..+3 of the half
#pragma unroll
  for (int u = 0; u < ETW; ++u)
    hfrag[u] = nl * D + 16 * ((2 * u + (kg >> 1)) ^ hswz(nl)) + 8 * (kg & 1);
  auto wave_sync = []() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // LDS offsets of the read patterns of a step.  The row swizzles of both
  // layouts depend only on the low row bits (KRow: bits 0-3; SRow: bits 0, 1
  // and 3), which the tile, key-step and k-step offsets below leave alone,
  // so every read is a lane-constant base plus a uniform offset.
  int kbase[KS];  // key rows of key tile 0: + kt * 16 rows
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kbase[ks] = KRow<D>::off(nl, 4 * ks + kg);
  int vbase[ETW];  // v^T reads of keys 4*kg.. (+ 32*js rows, + 16 rows)
  int sbase[ETW];  // S^T fragments (+ 32*ks rows, + 4 rows)
#pragma unroll
  for (int u = 0; u < ETW; ++u) {
    const int et = eh * ETW + u;
    const int c = 16 * et + 4 * (nl & 3);
    vbase[u] = KRow<D>::off(4 * kg + (nl >> 2), c >> 3) + 2 * (c & 7);
    sbase[u] = SRow<D>::off(8 * kg + (nl >> 2), 2 * et + ((nl & 3) >> 1)) + 8 * (nl & 1);
  }
  int pv[STW][2], pk[STW][2];  // state-update reads (+ 16*kk rows)
  {
    const int g16 = lane >> 4, s16 = lane & 15;
    const int r0 = 8 * (g16 >> 1) + (s16 >> 2);
#pragma unroll
    for (int t = 0; t < STW; ++t) {
      const int ce = 32 * t_e[t] + 16 * (g16 & 1) + 4 * (s16 & 3);
      const int cp = 32 * t_p[t] + 16 * (g16 & 1) + 4 * (s16 & 3);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        pv[t][hh] = KRow<D>::off(r0 + 4 * hh, ce >> 3) + 2 * (ce & 7);
        pk[t][hh] = KRow<D>::off(r0 + 4 * hh, cp >> 3) + 2 * (cp & 7);
      }
    }
  }

  load_kvq(n_begin);
  load_g(n_begin);

  for (int64_t n0 = n_begin; n0 < n_end; n0 += STEP) {
    __syncthreads();  // the previous step's state phase is done with the tiles

    // ---------------- prologue
    float zp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) zp[j] = 0.f;
#pragma unroll
    for (int rr = 0; rr < RP; ++rr) {
      int64_t n = n0 + tg + TPP * rr;
      if (n >= n_end) n = n_end - 1;  // position only; the row itself reads as zero
      int t, h, w;
      token_pos(a, n, t, h, w);
      const uint32_t rl[4] = {relu_bf16x2(kr[rr].x), relu_bf16x2(kr[rr].y),
                              relu_bf16x2(kr[rr].z), relu_bf16x2(kr[rr].w)};
      float x[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        x[2 * m] = lo_bf16(rl[m]);
        x[2 * m + 1] = hi_bf16(rl[m]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) zp[j] += x[j];
      float2 c4[4];
      ts.read(s_tab, tl.at(t, h, w), c4);
      rotate4(x, c4);
      uint4 hi, lo;
      split_bf16x2(x[0], x[1], hi.x, lo.x);
      split_bf16x2(x[2], x[3], hi.y, lo.y);
      split_bf16x2(x[4], x[5], hi.z, lo.z);
      split_bf16x2(x[6], x[7], hi.w, lo.w);
      const int o = KRow<D>::off(tg + TPP * rr, fc);
      *reinterpret_cast<uint4 *>(s_kh + o) = hi;
      *reinterpret_cast<uint4 *>(s_kl + o) = lo;
      *reinterpret_cast<uint4 *>(s_kp + o) = make_uint4(rl[0], rl[1], rl[2], rl[3]);
      *reinterpret_cast<uint4 *>(s_v + o) = vr[rr];
    }
    // the wave's phi(k) sums per feature: lanes l, l ^ FPT, ... hold the same features
#pragma unroll
    for (int m = FPT; m < 64; m <<= 1)
#pragma unroll
      for (int j = 0; j < 8; ++j) zp[j] += __shfl_xor(zp[j], m);
    if (lane < FPT) {
      float4 *dst = reinterpret_cast<float4 *>(s_zp + wave * D + 8 * lane);
      dst[0] = make_float4(zp[0], zp[1], zp[2], zp[3]);
      dst[1] = make_float4(zp[4], zp[5], zp[6], zp[7]);
    }
    // this wave's queries: phi(q) (exact in bf16) and RoPE(phi(q)) hi + lo
    bf16x8 qp[KS], qh[KS], ql[KS];
    {
      int64_t nq = n0 + 16 * qt + nl;
      if (nq >= n_end) nq = n_end - 1;
      int t, h, w;
      token_pos(a, nq, t, h, w);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t qw[4] = {relu_bf16x2(qraw[ks].x), relu_bf16x2(qraw[ks].y),
                                relu_bf16x2(qraw[ks].z), relu_bf16x2(qraw[ks].w)};
        qp[ks] = __builtin_bit_cast(bf16x8, make_uint4(qw[0], qw[1], qw[2], qw[3]));
        float x[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          x[2 * m] = lo_bf16(qw[m]);
          x[2 * m + 1] = hi_bf16(qw[m]);
        }
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
      }
    }
    // the next step's rows stay in flight through the rest of this step
    // (unconditional: rows past the range read as zeros)
    load_kvq(n0 + STEP);
    __syncthreads();

    // ---------------- outputs of query tile qt, features of half eh
    // den: phi(q) . z over this lane's 8 features per step
    float dpart = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4 z0 = *reinterpret_cast<const float4 *>(s_z + 32 * ks + 8 * kg);
      const float4 z1 = *reinterpret_cast<const float4 *>(s_z + 32 * ks + 8 * kg + 4);
      const uint4 qw = __builtin_bit_cast(uint4, qp[ks]);
      dpart = __builtin_fmaf(lo_bf16(qw.x), z0.x, dpart);
      dpart = __builtin_fmaf(hi_bf16(qw.x), z0.y, dpart);
      dpart = __builtin_fmaf(lo_bf16(qw.y), z0.z, dpart);
      dpart = __builtin_fmaf(hi_bf16(qw.y), z0.w, dpart);
      dpart = __builtin_fmaf(lo_bf16(qw.z), z1.x, dpart);
      dpart = __builtin_fmaf(hi_bf16(qw.z), z1.y, dpart);
      dpart = __builtin_fmaf(lo_bf16(qw.w), z1.z, dpart);
      dpart = __builtin_fmaf(hi_bf16(qw.w), z1.w, dpart);
    }
    f32x4 acc[ETW];
#pragma unroll
    for (int u = 0; u < ETW; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};

    // intra-step part, 32 keys (key tiles 2js, 2js + 1) at a time.  Scores^T
    // (keys x queries): A = key rows (16-byte pieces), B = queries.
    auto score_tile = [&](int kt, f32x4 &at, f32x4 &dm) {
      at = f32x4{0.f, 0.f, 0.f, 0.f};
      dm = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int o = kbase[ks] + kt * (32 * D);
        const bf16x8 fh = *reinterpret_cast<const bf16x8 *>(s_kh + o);
        const bf16x8 fl = *reinterpret_cast<const bf16x8 *>(s_kl + o);
        const bf16x8 fp = *reinterpret_cast<const bf16x8 *>(s_kp + o);
        at = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fl, qh[ks], at, 0, 0, 0);
        at = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fh, ql[ks], at, 0, 0, 0);
        at = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fh, qh[ks], at, 0, 0, 0);
        dm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp, qp[ks], dm, 0, 0, 0);
      }
      mfma_drain();
    };
    for (int js = 0; 2 * js <= qt; ++js) {
      f32x4 at[2], dm[2];
      score_tile(2 * js, at[0], dm[0]);
      if (2 * js + 1 <= qt) {
        score_tile(2 * js + 1, at[1], dm[1]);
      } else {
        at[1] = f32x4{0.f, 0.f, 0.f, 0.f};
        dm[1] = at[1];
      }
      // value i: key 4*kg + i of the tile, query nl; on the diagonal tile the
      // keys after the query drop (branch-free: lim = nl there, 15 elsewhere)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int lim = 2 * js + h2 == qt ? nl : 15;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool keep = 4 * kg + i <= lim;
          at[h2][i] = keep ? at[h2][i] : 0.f;
          dm[h2][i] = keep ? dm[h2][i] : 0.f;
        }
        dpart += (dm[h2][0] + dm[h2][1]) + (dm[h2][2] + dm[h2][3]);
      }
      // num += v^T scores^T: the B operand is the two score tiles (keys
      // 4*kg..+3 of each), split into hi + lo; the A operand reads the same
      // keys of v transposed
      uint32_t ah[4], al[4];
      split_bf16x2(at[0][0], at[0][1], ah[0], al[0]);
      split_bf16x2(at[0][2], at[0][3], ah[1], al[1]);
      split_bf16x2(at[1][0], at[1][1], ah[2], al[2]);
      split_bf16x2(at[1][2], at[1][3], ah[3], al[3]);
      const bf16x8 bh = __builtin_bit_cast(bf16x8, make_uint4(ah[0], ah[1], ah[2], ah[3]));
      const bf16x8 bl = __builtin_bit_cast(bf16x8, make_uint4(al[0], al[1], al[2], al[3]));
#pragma unroll
      for (int u = 0; u < ETW; ++u) {
        const int o = vbase[u] + js * (64 * D);  // keys 32*js + 4*kg.. and + 16
        const uint2 v0 = lds_read_tr16(s_v + o);
        const uint2 v1 = lds_read_tr16(s_v + o + 16 * (2 * D));
        const bf16x8 vt = __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, bl, acc[u], 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, bh, acc[u], 0, 0, 0);
      }
      mfma_drain();  // the next iteration's vector code rewrites the operands
    }

    // the sums before the step: num += S^T RoPE(phi(q))^T (A = S^T read
    // transposed from the bf16 parts, three products per step)
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

    // den over the token's four lanes (fixed order)
    dpart += __shfl_xor(dpart, 16);
    dpart += __shfl_xor(dpart, 32);
    const float den = dpart + a.eps;
    __syncthreads();  // every wave is done with the step's tiles

    // the gate and the store through the wave's half-row tile: g rows in,
    // g fragments out, output fragments in (each lane on its own places),
    // output rows out
#pragma unroll
    for (int i = 0; i < HP; ++i) *reinterpret_cast<uint4 *>(hs + hrow[i]) = grow[i];
    wave_sync();
#pragma unroll
    for (int u = 0; u < ETW; ++u) {
      const uint2 gw = *reinterpret_cast<const uint2 *>(hs + hfrag[u]);
      const float gv[4] = {lo_bf16(gw.x), hi_bf16(gw.x), lo_bf16(gw.y), hi_bf16(gw.y)};
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // num / den * sigmoid(g) = num / (den * (1 + exp(-g)))
        const float e = __expf(-gv[i]);
        o[i] = acc[u][i] * __builtin_amdgcn_rcpf(__builtin_fmaf(den, e, den));
      }
      *reinterpret_cast<uint2 *>(hs + hfrag[u]) =
          make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    }
    wave_sync();
    {
      const uint32_t ooff =
          ((uint32_t)(n0 - n_begin) + 16 * qt + hr) * row_bytes + eh * D + 16 * hc;
#pragma unroll
      for (int i = 0; i < HP; ++i)
        buf_store16<kCacheStream>(ro, ooff + i * HRP * row_bytes,
                                  *reinterpret_cast<const uint4 *>(hs + hrow[i]));
    }
    load_g(n0 + STEP);

    // ---------------- state: S^T += v^T RoPE(phi(k)) over the step's keys
    if (s_owner) {
#pragma unroll
      for (int t = 0; t < STW; ++t) {
#pragma unroll
        for (int kk = 0; kk < STEP / 16; ++kk) {
          const int ov0 = pv[t][0] + kk * (32 * D), ov1 = pv[t][1] + kk * (32 * D);
          const int ok0 = pk[t][0] + kk * (32 * D), ok1 = pk[t][1] + kk * (32 * D);
          const uint2 v0 = lds_read_tr16(s_v + ov0), v1 = lds_read_tr16(s_v + ov1);
          const uint2 h0 = lds_read_tr16(s_kh + ok0), h1 = lds_read_tr16(s_kh + ok1);
          const uint2 l0 = lds_read_tr16(s_kl + ok0), l1 = lds_read_tr16(s_kl + ok1);
          const bf16x8 fv = __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
          const bf16x8 fh = __builtin_bit_cast(bf16x8, make_uint4(h0.x, h0.y, h1.x, h1.y));
          const bf16x8 fl = __builtin_bit_cast(bf16x8, make_uint4(l0.x, l0.y, l1.x, l1.y));
          sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fv, fl, sacc[t], 0, 0, 0);
          sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fv, fh, sacc[t], 0, 0, 0);
        }
      }
      mfma_drain();
    }
    publish();
    // z takes the step's keys: the per-wave sums, in wave order
    if (tid < D) {
      float zs = s_z[tid];
#pragma unroll
      for (int w = 0; w < NW; ++w) zs += s_zp[w * D + tid];
      s_z[tid] = zs;
    }
  }
}

template <int D>
size_t causal_lds(const Plan &p) {
  return CausalCfg<D>::kFixedLds + (size_t)tab_slice_entries(p, p.Lr) * sizeof(float2);
}

template <int D>
hipError_t causal_d(const Plan &p, const void *q, const void *k, const void *v, const void *g,
                    const float *states, const float2 *tab, void *out, hipStream_t stream) {
  const size_t lds = causal_lds<D>(p);
  auto kern = causal_mfma_kernel<D>;
  hipError_t e = lds_limit_once((const void *)kern);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.units * p.R)), dim3(kCausalThreads), lds, stream,
                     (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v,
                     (const uint16_t *)g, states, tab, (uint16_t *)out, make_margs(p));
  return hipGetLastError();
}

}  // namespace

size_t causal_mfma_lds_bytes(const Plan &p) {
  if (p.d == 128) return causal_lds<128>(p);
  if (p.d == 64) return causal_lds<64>(p);
  return 0;
}

hipError_t causal_mfma_lds_limits() {
  return lds_limits({(const void *)causal_mfma_kernel<128>, (const void *)causal_mfma_kernel<64>});
}

hipError_t launch_causal_mfma(const Plan &p, const void *q, const void *k, const void *v,
                              const void *g, const float *states, const float2 *tab, void *out,
                              hipStream_t stream) {
  if (p.d == 128) return causal_d<128>(p, q, k, v, g, states, tab, out, stream);
  if (p.d == 64) return causal_d<64>(p, q, k, v, g, states, tab, out, stream);
  return hipErrorInvalidValue;
}

}  // namespace gla
