// Host side of libgla.so: argument validation, work decomposition, workspace
// handling, stage timing and the C entry points declared in include/gla.h.
//
// The operator and its sources are described in include/gla.h ("SANA-Video
// 2.0" Section 2 Eq. (1); "SANA-Video" Sections 3.2 and 3.4).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "gla.h"
#include "gla_internal.h"

using gla::Plan;

namespace {

thread_local char g_last_error[512] = "";

gla_status fail(gla_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

gla_status hip_fail(hipError_t e, const char *what) {
  return fail(GLA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool mul_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_mul_overflow(a, b, out); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Streaming block step arguments of forward_impl (absent for the one-call
// operators): the absolute position of the block's first frame and the
// caller's cache.
struct Step {
  int64_t t0 = 0;
  float *S_io = nullptr, *z_io = nullptr;
  bool update = false;
};

// ---------------------------------------------------------------- devices
std::mutex g_dev_mu;
std::vector<int> g_cu_count;  // per device id, 0 = unknown

gla_status device_cus(int *cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_cu_count.size() <= dev) g_cu_count.resize(dev + 1, 0);
  if (g_cu_count[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(multiprocessor count)");
    // every kernel's dynamic-LDS limit, before the first launch on this
    // device: no later call can then fail on an attribute mid-plan
    for (auto set : {gla::state_mfma_lds_limits, gla::apply_mfma_lds_limits,
                     gla::causal_mfma_lds_limits, gla::backward_mfma_lds_limits,
                     gla::backward_query_lds_limits,
                     gla::vector_lds_limits, gla::causal_vector_lds_limits,
                     gla::backward_vector_lds_limits}) {
      e = set();
      if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute (dynamic LDS limit)");
    }
    g_cu_count[dev] = n > 0 ? n : 1;
  }
  *cus = g_cu_count[dev];
  return GLA_OK;
}

// ---------------------------------------------------------------- validation
gla_status check_sizes(int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                       int64_t F, gla_dtype dtype) {
  if (B < 1 || H < 1 || T < 1 || Hs < 1 || Ws < 1)
    return fail(GLA_ERR_INVALID_ARG, "B, H, T, Hs, Ws must be >= 1 (got %lld %lld %lld %lld %lld)",
                (long long)B, (long long)H, (long long)T, (long long)Hs, (long long)Ws);
  if (d < 16 || d > 128 || d % 16 != 0)
    return fail(GLA_ERR_INVALID_ARG, "d must be a multiple of 16 in [16, 128] (got %lld)",
                (long long)d);
  if (F < 0) return fail(GLA_ERR_INVALID_ARG, "frames_per_block must be >= 0");
  if (F > 0 && T % F != 0)
    return fail(GLA_ERR_INVALID_ARG, "frames_per_block (%lld) must divide T (%lld)",
                (long long)F, (long long)T);
  if (dtype != GLA_BF16 && dtype != GLA_F32)
    return fail(GLA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  int64_t hw, n, bn, bnh, elems, bytes;
  if (!mul_ok(Hs, Ws, &hw) || !mul_ok(hw, T, &n) || !mul_ok(n, B, &bn) || !mul_ok(bn, H, &bnh) ||
      !mul_ok(bnh, d, &elems) || !mul_ok(elems, 4, &bytes))
    return fail(GLA_ERR_INVALID_ARG, "tensor size B*T*Hs*Ws*H*d overflows int64");
  return GLA_OK;
}

bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb) {
  uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

gla_status check_pointers(const void *q, const void *k, const void *v, const void *g,
                          const void *out, size_t bytes) {
  if (!q || !k || !v || !g || !out) return fail(GLA_ERR_INVALID_ARG, "null tensor pointer");
  const void *ins[4] = {q, k, v, g};
  const char *names[4] = {"q", "k", "v", "g"};
  for (int i = 0; i < 4; ++i)
    if (ranges_overlap(out, bytes, ins[i], bytes))
      return fail(GLA_ERR_INVALID_ARG, "out overlaps input %s", names[i]);
  return GLA_OK;
}

// gla_block_step: k and v always; q, g and out unless the call only updates
// the cache; a cache that overlaps nothing; t_offset + Tb within int32.
gla_status check_step(const void *q, const void *k, const void *v, const void *g, const void *out,
                      size_t bytes, const Step &s, int64_t BH, int64_t d, int64_t Tb) {
  if (!k || !v) return fail(GLA_ERR_INVALID_ARG, "null tensor pointer");
  if (!s.S_io || !s.z_io) return fail(GLA_ERR_INVALID_ARG, "null cache pointer (S_io or z_io)");
  if (out == nullptr && !s.update)
    return fail(GLA_ERR_INVALID_ARG, "out is null and update is 0: the call would do nothing");
  if (out != nullptr) {
    gla_status st = check_pointers(q, k, v, g, out, bytes);
    if (st != GLA_OK) return st;
  }
  if (s.t0 < 0 || s.t0 > (int64_t)INT32_MAX - Tb)
    return fail(GLA_ERR_INVALID_ARG, "t_offset (%lld) must be in [0, 2^31 - 1 - Tb]",
                (long long)s.t0);
  if ((((uintptr_t)s.S_io) | ((uintptr_t)s.z_io)) & 3)
    return fail(GLA_ERR_INVALID_ARG, "S_io and z_io must be 4-byte aligned");
  const size_t sb = (size_t)(BH * d * d) * sizeof(float), zb = (size_t)(BH * d) * sizeof(float);
  if (ranges_overlap(s.S_io, sb, s.z_io, zb))
    return fail(GLA_ERR_INVALID_ARG, "S_io and z_io overlap");
  const void *ts[5] = {q, k, v, g, out};
  const char *names[5] = {"q", "k", "v", "g", "out"};
  for (int i = 0; i < 5; ++i)
    if (ts[i] != nullptr &&
        (ranges_overlap(s.S_io, sb, ts[i], bytes) || ranges_overlap(s.z_io, zb, ts[i], bytes)))
      return fail(GLA_ERR_INVALID_ARG, "the cache overlaps %s", names[i]);
  return GLA_OK;
}

// gla_gated_forward: beta [B, N, H] and rms_w [d] of the tensors' type, each
// optional, aligned to their element size, not overlapping out;
// rms_eps finite and > 0 when the RMSNorm is on.
struct Gates;
gla_status check_gates(const Gates &gt, const void *out, size_t bytes, int64_t BNH, int64_t d,
                       gla_dtype dtype, float rms_eps);

// ---------------------------------------------------------------- planning
// Number of pieces to cut each of `units` token runs of `len` tokens into
// (pieces of a multiple of `tile` tokens, at least `min_len` long), such that
// the units * pieces workgroups fill whole rounds of `slots` workgroups that
// are resident at once: the fewest rounds (up to four) whose last round is at
// least 90% full, else the fullest last round.  A ragged last round leaves
// compute units idle at the end of the stage, and fewer, longer workgroups
// stream HBM better than many short ones.
int64_t pick_pieces(int64_t units, int64_t len, int64_t tile, int64_t min_len, int64_t slots) {
  const int64_t max_pieces = std::max<int64_t>(1, len / std::max(min_len, tile));
  int64_t best = 1;
  double best_fill = -1.0;
  for (int64_t rounds = 1; rounds <= 4; ++rounds) {
    int64_t n = std::min(max_pieces, std::max<int64_t>(1, rounds * slots / units));
    n = ceil_div(len, round_up(ceil_div(len, n), tile));  // after rounding to the tile
    const int64_t wgs = units * n;
    const double fill = (double)wgs / (double)(ceil_div(wgs, slots) * slots);
    if (fill >= 0.9) return n;
    if (fill > best_fill) {
      best_fill = fill;
      best = n;
    }
  }
  return best;
}

// aligned16: every tensor pointer is 16-byte aligned (the matrix-core
// kernels move 16-byte vectors).
gla_status make_plan(int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                     int64_t F, gla_dtype dtype, float theta, float eps, int cus, bool aligned16,
                     Plan *p) {
  gla_status st = check_sizes(B, H, T, Hs, Ws, d, F, dtype);
  if (st != GLA_OK) return st;
  Plan P{};
  P.B = B; P.H = H; P.T = T; P.Hs = Hs; P.Ws = Ws; P.d = d;
  P.F = (F == 0) ? T : F;
  P.nb = T / P.F;
  P.N = T * Hs * Ws;
  P.L = P.F * Hs * Ws;
  P.units = B * H * P.nb;
  P.bf16 = (dtype == GLA_BF16);
  P.theta = theta;
  P.eps = eps;

  // RoPE table: T*(d/8) + Hs*(3d/16) + Ws*(3d/16) (cos, sin) entries.
  const int64_t pt = d / 8, ph = 3 * d / 16, pw = 3 * d / 16;
  P.tab_t_off = 0;
  P.tab_h_off = T * pt;
  P.tab_w_off = P.tab_h_off + Hs * ph;
  P.tab_entries = P.tab_w_off + Ws * pw;

  // Matrix-core kernels keep the rows of the table they touch in LDS; the
  // spatial rows must fit next to at least two temporal rows.
  const int64_t spatial_entries = Hs * ph + Ws * pw;
  // (token indices and positions are 32-bit in the matrix-core kernels)
  P.mfma = aligned16 && P.bf16 && (d == 64 || d == 128) && P.N < ((int64_t)1 << 31) &&
           spatial_entries + 2 * pt <= std::min(gla::kStateTabEntries, gla::kApplyTabEntries);

  const int64_t hw = Hs * Ws;
  const int64_t tile_s = P.mfma ? gla::kStateTile : 16;
  const int64_t tile_a = P.mfma ? gla::kApplyTile * 8 : 16;

  // State stage: one twelve-wave workgroup resident per compute unit at
  // d = 128 (two six-wave ones at d = 64), chunks of at least 256 tokens.
  const int64_t C0 = pick_pieces(P.units, P.L, tile_s, 256, (d == 128 ? 1 : 2) * (int64_t)cus);
  int64_t Lc = round_up(ceil_div(P.L, C0), tile_s);
  if (P.mfma) {
    // temporal rows of a chunk: at most ceil(Lc / hw) + 1
    int64_t max_rows = (gla::kStateTabEntries - spatial_entries) / pt;
    int64_t max_len = std::max<int64_t>(tile_s, ((max_rows - 1) * hw) / tile_s * tile_s);
    Lc = std::min(Lc, max_len);
  }
  P.Lc = Lc;
  P.C = ceil_div(P.L, Lc);

  // Apply stage: the matrix-core kernel holds one workgroup per compute unit
  // (its LDS); the vector kernel takes about four per compute unit of
  // 16..4096 tokens each.
  int64_t Lr;
  if (P.mfma) {
    Lr = round_up(ceil_div(P.L, pick_pieces(P.units, P.L, tile_a, tile_a, cus)), tile_a);
  } else {
    Lr = round_up(ceil_div(P.units * P.L, 4 * (int64_t)cus), tile_a);
    Lr = std::max<int64_t>(tile_a, std::min<int64_t>(Lr, 4096));
  }
  if (P.mfma) {
    int64_t max_rows = (gla::kApplyTabEntries - spatial_entries) / pt;
    int64_t max_len = std::max<int64_t>(tile_a, ((max_rows - 1) * hw) / tile_a * tile_a);
    Lr = std::min(Lr, max_len);
  }
  Lr = std::min(Lr, round_up(P.L, tile_a));
  P.Lr = Lr;
  P.R = ceil_div(P.L, Lr);

  if (P.mfma) {
    // buffer offsets of a token range are 32-bit: keep range bytes < 2^31
    const int64_t row_bytes = H * d * 2;
    // (the state kernel also addresses up to three 64-token steps past a
    // chunk, the apply and key/value gradient kernels up to three 128-token
    // wave steps past a range: 512 rows cover both)
    const int64_t max_tokens = (((int64_t)1 << 31) - 2 * d) / row_bytes - 512;
    if (P.Lc > max_tokens) {
      P.Lc = std::max<int64_t>(tile_s, max_tokens / tile_s * tile_s);
      P.C = ceil_div(P.L, P.Lc);
    }
    if (P.Lr > max_tokens) {
      P.Lr = std::max<int64_t>(tile_a, max_tokens / tile_a * tile_a);
      P.R = ceil_div(P.L, P.Lr);
    }
    if (P.Lc > max_tokens || P.Lr > max_tokens) P.mfma = false;
  }
  if (P.mfma) {
    // Output stage: a workgroup takes one (batch, block, head) unit and items
    // of kItem tokens (one 16-token tile per wave).  One workgroup per compute
    // unit: am workgroups per unit share its items in turn.  A block is cut
    // into super-ranges only when the RoPE table rows of the whole block
    // would not fit in LDS beside S and the staging tiles.
    P.hpw = 1;
    P.ag = B * P.nb * H;
    const int64_t item = gla::apply_mfma_item_tokens();
    const int64_t items = ceil_div(P.L, item);
    P.ar = 1;
    for (;;) {
      P.air = ceil_div(items, P.ar);
      if (gla::apply_mfma_lds_bytes(P) <= 160 * 1024 || P.air == 1) break;
      P.ar *= 2;
    }
    if (gla::apply_mfma_lds_bytes(P) > 160 * 1024) P.mfma = false;
    const int64_t sranges = P.ag * P.ar;
    P.am = std::max<int64_t>(1, std::min<int64_t>(P.air, cus / std::max<int64_t>(1, sranges)));
    // Pairs of blocks per wave read half of S per block, but a workgroup
    // with an odd item count computes one dead block in its last pair: take
    // pairs where the busiest workgroups' item count is even or that block
    // is a small share of their work (measured: -1.3 to -2.2% per call at
    // 720p/81f with 74 items; +5% for the streaming block step with 9)
    const int64_t most = ceil_div(P.air, P.am);
    P.apair = (most % 2) == 0 || most >= 16;
    if (sranges * P.am > 0x7fffffff) P.mfma = false;
    // token indices stay below 2^31 up to the prefetches four items past a range
    if (P.N + 4 * P.am * item + 16 >= ((int64_t)1 << 31)) P.mfma = false;
    // a 16-row tile of one head must be addressable with 32-bit offsets
    if ((int64_t)16 * H * d * 2 >= ((int64_t)1 << 31)) P.mfma = false;
  }
  if (P.mfma) {
    // LDS of the two matrix-core kernels must fit the 160 KiB of a CU
    // (+ 64 bytes for the state kernel's static LDS)
    const int64_t lds_state = (int64_t)gla::state_mfma_lds_bytes(P) + 64;
    if (lds_state > 160 * 1024) return fail(GLA_ERR_UNSUPPORTED,
        "internal: LDS plan of %lld bytes exceeds the CU", (long long)lds_state);
  }
  // Backward: vector kernels, about four workgroups per compute unit of
  // 16..4096 tokens each.
  P.Lb = round_up(ceil_div(P.units * P.L, 4 * (int64_t)cus), 16);
  P.Lb = std::max<int64_t>(16, std::min<int64_t>(P.Lb, 4096));
  P.Lb = std::min(P.Lb, round_up(P.L, 16));
  P.Rb = ceil_div(P.L, P.Lb);

  const int64_t max_grid = 0x7fffffff;
  if (P.units * P.C > max_grid || P.units * P.R > max_grid || P.units * P.Rb > max_grid ||
      B * H > max_grid)
    return fail(GLA_ERR_UNSUPPORTED, "too many (batch, head, block) units for one launch");

  // Workspace layout.
  size_t off = 0;
  P.off_tab = off;
  off = align256(off + (size_t)P.tab_entries * sizeof(float2));
  P.off_part = off;
  off = align256(off + (size_t)P.units * P.C * gla::kPartialStride(d) * sizeof(float));
  P.off_state = off;
  off = align256(off + (size_t)P.units * gla::kPartialStride(d) * sizeof(float));
  P.off_frag = off;
  if (P.mfma) off = align256(off + (size_t)P.units * 2 * d * d * sizeof(uint16_t));
  P.total_bytes = off;
  P.off_bpart = off;
  // (the vector gradient kernels write Rb range partials per unit, the
  // matrix-core ones C chunk partials)
  off = align256(off + (size_t)P.units * std::max(P.Rb, P.C) * gla::kPartialStride(d) *
                           sizeof(float));
  P.off_grad = off;
  off = align256(off + (size_t)P.units * gla::kPartialStride(d) * sizeof(float));
  P.off_dd = off;
  if (P.mfma) off = align256(off + (size_t)(B * H * P.N) * 2 * sizeof(float));
  P.bwd_total_bytes = off;
  *p = P;
  return GLA_OK;
}

// Token-causal plan: one unit per (batch, head) over all N tokens.  The
// tile kernel walks a range of Lr tokens per workgroup (about one workgroup
// per compute unit); ranges are whole multiples of the state chunks
// (Lr = m * Lc), so the prefix at a range start is a sum of whole chunk
// partials.  The matrix-core path takes two chunks per range (two state
// workgroups per compute unit).  Workspace: the table, the chunk partials,
// and the range prefixes [units][R][d*d + d].
gla_status make_causal_plan(int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                            gla_dtype dtype, float theta, float eps, int cus, bool aligned16,
                            Plan *p) {
  Plan P;
  gla_status st = make_plan(B, H, T, Hs, Ws, d, 0, dtype, theta, eps, cus, aligned16, &P);
  if (st != GLA_OK) return st;
  if (P.mfma) {
    const int64_t tile = 2 * gla::kStateTile;
    int64_t Lr = round_up(ceil_div(P.N, pick_pieces(P.units, P.N, tile, 256, cus)), tile);
    Lr = std::min(Lr, round_up(P.N, tile));
    // the table slice of a range must fit beside the tile kernel's other
    // LDS, and the state kernel's slice of a chunk in its own budget
    const int64_t hw = Hs * Ws, pt = d / 8, spatial = Hs * (3 * d / 16) + Ws * (3 * d / 16);
    const int64_t state_rows = (gla::kStateTabEntries - spatial) / pt;
    const int64_t state_max = ((state_rows - 1) * hw) / gla::kStateTile * gla::kStateTile;
    Lr = std::min(Lr, 2 * state_max / tile * tile);
    // buffer offsets are 32-bit: the range plus one step of prefetch
    const int64_t row_bytes = H * d * 2;
    const int64_t max_tokens = (((int64_t)1 << 31) - 2 * d) / row_bytes - 2 * gla::kStateTile;
    Lr = std::min(Lr, max_tokens / tile * tile);
    auto set_ranges = [&](int64_t len) {
      P.Lr = len;
      P.R = ceil_div(P.N, len);
      P.Lc = len / 2;
      P.C = ceil_div(P.N, P.Lc);
    };
    set_ranges(std::max(Lr, tile));
    // fewer temporal table rows per range until the tile kernel's LDS fits
    while (gla::causal_mfma_lds_bytes(P) > 160 * 1024 && P.Lr > tile)
      set_ranges(std::max(tile, (P.Lr - hw) / tile * tile));
    if (Lr < tile || state_max < gla::kStateTile || gla::causal_mfma_lds_bytes(P) > 160 * 1024)
      P.mfma = false;
  }
  if (!P.mfma) {  // vector tile kernel
    const int64_t tile = 16;
    int64_t Lr = round_up(ceil_div(P.N, pick_pieces(P.units, P.N, tile, 256, cus)), tile);
    Lr = std::min(Lr, round_up(P.N, tile));
    P.Lr = Lr;
    P.R = ceil_div(P.N, Lr);
    P.Lc = Lr;  // m = 1
    P.C = P.R;
  }
  if (P.units * P.C > 0x7fffffff)
    return fail(GLA_ERR_UNSUPPORTED, "too many (batch, head, range) units for one launch");
  size_t off = 0;
  P.off_tab = off;
  off = align256(off + (size_t)P.tab_entries * sizeof(float2));
  P.off_part = off;
  off = align256(off + (size_t)P.units * P.C * gla::kPartialStride(d) * sizeof(float));
  P.off_state = off;
  off = align256(off + (size_t)P.units * P.R * gla::kPartialStride(d) * sizeof(float));
  P.off_frag = off;
  P.total_bytes = off;
  P.off_bpart = P.off_grad = P.off_dd = P.bwd_total_bytes = off;
  *p = P;
  return GLA_OK;
}

// ---------------------------------------------------------------- profiling
struct StageRecord {
  int stage;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<StageRecord> g_prof;

const char *kStageNames[GLA_NUM_STAGES] = {"rope_table", "state_partials", "reduce_prefix",
                                           "apply", "backward", "causal_apply"};

void prof_clear_locked() {
  for (auto &r : g_prof) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_prof.clear();
}

// Runs one launch, bracketed by events when timing is enabled.
template <class F>
gla_status timed_launch(int stage, hipStream_t stream, const char *what, F &&launch) {
  bool on;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    on = g_prof_on;
  }
  StageRecord rec{stage, nullptr, nullptr};
  if (on) {
    // timing-only events: without the system-scope fence (a write-back and
    // invalidation of the caches) a recorded event does not change how the
    // next kernel runs, so each stage takes the time it takes between the
    // other stages of an unprofiled call
    hipError_t e = hipEventCreateWithFlags(&rec.start, hipEventDisableSystemFence);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&rec.stop, hipEventDisableSystemFence);
    if (e == hipSuccess) e = hipEventRecord(rec.start, stream);
    if (e != hipSuccess) return hip_fail(e, "stage timing event");
  }
  hipError_t e = launch();
  if (e != hipSuccess) {
    if (on) {
      (void)hipEventDestroy(rec.start);
      (void)hipEventDestroy(rec.stop);
    }
    return hip_fail(e, what);
  }
  if (on) {
    e = hipEventRecord(rec.stop, stream);
    if (e != hipSuccess) return hip_fail(e, "stage timing event");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof.push_back(rec);
  }
  return GLA_OK;
}

// ---------------------------------------------------------------- RoPE table cache
// The (cos, sin) table depends only on (T, Hs, Ws, d, theta, t0).  The first
// call of a shape on a device computes it, on that call's stream, into
// library memory that lives until the process ends; later calls read it and
// skip the table kernel.  A call on another stream before the table kernel
// has finished waits for it (an event).  The per-call table in the workspace
// remains for calls that must not allocate (gla_forward_noalloc, which reads
// a finished cached table but never creates one), for calls made during
// stream capture while an entry is missing or unfinished (capture must not
// record the library's one-off work or wait on an event outside the graph),
// and once kMaxCachedTables shapes are cached.
struct TabKey {
  int dev;
  int64_t T, Hs, Ws, d, t0;
  uint32_t theta;
  bool operator<(const TabKey &o) const {
    return std::tie(dev, T, Hs, Ws, d, t0, theta) <
           std::tie(o.dev, o.T, o.Hs, o.Ws, o.d, o.t0, o.theta);
  }
};
struct TabEntry {
  float2 *ptr = nullptr;
  hipEvent_t done = nullptr;  // recorded after the table kernel
  bool ready = false;         // the event has completed
};
constexpr size_t kMaxCachedTables = 256;
std::mutex g_tab_mu;
std::map<TabKey, TabEntry> g_tabs;

// The RoPE table for P on `stream`: the cached one when it exists (creating
// it when may_create), else computed into the workspace's table ws_tab.
gla_status rope_table_for(const Plan &P, float2 *ws_tab, hipStream_t stream, bool may_create,
                          const float2 **tab) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  const bool capturing = cap != hipStreamCaptureStatusNone;
  uint32_t theta_bits;
  std::memcpy(&theta_bits, &P.theta, sizeof(theta_bits));
  const TabKey key{dev, P.T, P.Hs, P.Ws, P.d, P.t0, theta_bits};
  {
    std::lock_guard<std::mutex> lk(g_tab_mu);
    auto it = g_tabs.find(key);
    if (it != g_tabs.end()) {
      TabEntry &t = it->second;
      // (no event query during capture: only a table known to be finished
      // serves a captured call)
      if (!t.ready && !capturing) {
        e = hipEventQuery(t.done);
        if (e == hipSuccess) {
          t.ready = true;
        } else if (e == hipErrorNotReady) {
          (void)hipGetLastError();  // not an error; keep it from the next launch check
        } else {
          return hip_fail(e, "RoPE table event");
        }
      }
      if (t.ready) {
        *tab = t.ptr;
        return GLA_OK;
      }
      if (!capturing) {
        e = hipStreamWaitEvent(stream, t.done, 0);
        if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent (RoPE table)");
        *tab = t.ptr;
        return GLA_OK;
      }
    } else if (may_create && !capturing && g_tabs.size() < kMaxCachedTables) {
      TabEntry t;
      e = hipMalloc((void **)&t.ptr, (size_t)P.tab_entries * sizeof(float2));
      if (e == hipSuccess) e = hipEventCreateWithFlags(&t.done, hipEventDisableTiming);
      if (e != hipSuccess) {
        // no cache entry: the per-call table below still works
        (void)hipGetLastError();
        if (t.ptr != nullptr) (void)hipFree(t.ptr);
      } else {
        gla_status st = timed_launch(0, stream, "rope table kernel",
                                     [&] { return gla::launch_rope_table(P, t.ptr, stream); });
        if (st == GLA_OK) {
          e = hipEventRecord(t.done, stream);
          if (e != hipSuccess) st = hip_fail(e, "hipEventRecord (RoPE table)");
        }
        if (st != GLA_OK) {
          // the stream may still reach the kernel: keep the memory, drop the entry
          (void)hipEventDestroy(t.done);
          return st;
        }
        g_tabs.emplace(key, t);
        *tab = t.ptr;
        return GLA_OK;
      }
    }
  }
  *tab = ws_tab;
  return timed_launch(0, stream, "rope table kernel",
                      [&] { return gla::launch_rope_table(P, ws_tab, stream); });
}

// ---------------------------------------------------------------- reduce counters
// The counters of the reduce folded into the state kernel, one set per
// (device, stream): calls on one stream run in order, so a set is never used
// by two kernels at once.  A set is allocated on a stream's first call and
// zeroed stream-ordered on that stream; the last workgroup of each unit puts
// its counter back to zero, so the set stays zeroed between kernels.  Calls
// during stream capture, calls that must not allocate, calls with more than
// kMaxCounterUnits units and calls beyond kMaxCounterSets streams run the
// separate reduce kernel instead (bitwise the same sums).  (A stream that is
// destroyed while its last call still runs and whose handle a new stream
// reuses at once would share the set with it; the library cannot see that.)
constexpr int64_t kMaxCounterUnits = (int64_t)1 << 16;
constexpr size_t kMaxCounterSets = 64;
std::mutex g_cnt_mu;
std::map<std::pair<int, hipStream_t>, unsigned *> g_cnts;

// The counter set of `stream` (nullptr when the fold is not available).
gla_status reduce_counters(hipStream_t stream, bool may_alloc, unsigned **cnt) {
  *cnt = nullptr;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (cap != hipStreamCaptureStatusNone) return GLA_OK;
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_cnt_mu);
  auto it = g_cnts.find({dev, stream});
  if (it != g_cnts.end()) {
    *cnt = it->second;
    return GLA_OK;
  }
  if (!may_alloc || g_cnts.size() >= kMaxCounterSets) return GLA_OK;
  unsigned *p = nullptr;
  const size_t bytes = (size_t)kMaxCounterUnits * sizeof(unsigned);
  e = hipMalloc((void **)&p, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // no set: the separate reduce kernel still works
    return GLA_OK;
  }
  e = hipMemsetAsync(p, 0, bytes, stream);
  if (e != hipSuccess) {
    (void)hipFree(p);
    return hip_fail(e, "hipMemsetAsync (reduce counters)");
  }
  g_cnts.emplace(std::make_pair(dev, stream), p);
  *cnt = p;
  return GLA_OK;
}

// ---------------------------------------------------------------- execution
// The carried cache of a streaming block step: the reduce stage starts its
// running sums from (S_in, z_in) and writes the final sums to (S_out, z_out)
// (any of them may be null; S_out may be S_in).
struct Cache {
  const float *S_in = nullptr, *z_in = nullptr;
  float *S_out = nullptr, *z_out = nullptr;
};

// The gates of the full mixer (gla_gated_forward): the write gate beta
// [B, N, H] and the RMSNorm weight rms_w [d] (either may be null).
struct Gates {
  const void *beta = nullptr, *rms_w = nullptr;
};

gla_status check_gates(const Gates &gt, const void *out, size_t bytes, int64_t BNH, int64_t d,
                       gla_dtype dtype, float rms_eps) {
  const size_t es = dtype == GLA_BF16 ? 2 : 4;
  if (gt.beta != nullptr) {
    if ((uintptr_t)gt.beta % es) return fail(GLA_ERR_INVALID_ARG, "beta is misaligned");
    if (ranges_overlap(out, bytes, gt.beta, (size_t)BNH * es))
      return fail(GLA_ERR_INVALID_ARG, "out overlaps beta");
  }
  if (gt.rms_w != nullptr) {
    if ((uintptr_t)gt.rms_w % es) return fail(GLA_ERR_INVALID_ARG, "rms_weight is misaligned");
    if (ranges_overlap(out, bytes, gt.rms_w, (size_t)d * es))
      return fail(GLA_ERR_INVALID_ARG, "out overlaps rms_weight");
    if (!std::isfinite(rms_eps) || !(rms_eps > 0.f))
      return fail(GLA_ERR_INVALID_ARG, "rms_eps must be finite and > 0");
  }
  return GLA_OK;
}

// Bytes of the saved state of a call: the reduced (S, z) of every (batch,
// head, temporal block), d*d + d fp32 each.
size_t saved_state_bytes(int64_t B, int64_t H, int64_t T, int64_t F, int64_t d) {
  const int64_t nb = F > 0 ? T / F : 1;
  return (size_t)(B * H * nb) * (size_t)gla::kPartialStride(d) * sizeof(float);
}

// The saved state buffer: 256-byte aligned (as a workspace), apart from
// every tensor of the call.
gla_status check_saved(const void *saved, size_t saved_bytes, size_t tensor_bytes,
                       std::initializer_list<const void *> tensors) {
  if (((uintptr_t)saved & 255) != 0)
    return fail(GLA_ERR_INVALID_ARG, "saved state must be 256-byte aligned");
  for (const void *t : tensors)
    if (t != nullptr && ranges_overlap(saved, saved_bytes, t, tensor_bytes))
      return fail(GLA_ERR_INVALID_ARG, "saved state overlaps a tensor");
  return GLA_OK;
}

// Enqueues every stage of the operator on `stream`, with workspace `ws`.
// With `apply == false` only the state is computed (gla_state, cache-only
// block steps).
// The table used is returned in *tab_used (for the gradient kernels) when
// not null; may_alloc: the call may allocate the library's cached table and
// reduce counters.  With one temporal block on the matrix-core path the
// reduce runs in the state kernel's last workgroups (two launches per call).
// states_dst: where the reduced states go ([units][d*d + d] fp32), the
// workspace when null.
gla_status run_plan(const Plan &P, const void *q, const void *k, const void *v, const void *g,
                    void *out, void *ws, hipStream_t stream, bool apply,
                    const Cache &cache = Cache(), const Gates &gates = Gates(),
                    bool may_alloc = true, const float2 **tab_used = nullptr,
                    float *states_dst = nullptr) {
  char *base = (char *)ws;
  float *part = (float *)(base + P.off_part);
  float *states = states_dst != nullptr ? states_dst : (float *)(base + P.off_state);
  uint16_t *frags = P.mfma ? (uint16_t *)(base + P.off_frag) : nullptr;

  const float2 *tab = nullptr;
  gla_status st = rope_table_for(P, (float2 *)(base + P.off_tab), stream, may_alloc, &tab);
  if (st != GLA_OK) return st;
  if (tab_used != nullptr) *tab_used = tab;
  gla::FusedReduce fz;
  // (the last workgroup addresses a unit's C partials with 32-bit offsets)
  if (P.mfma && P.nb == 1 && P.units <= kMaxCounterUnits &&
      P.C * gla::kPartialStride(P.d) * 4 < ((int64_t)1 << 31)) {
    st = reduce_counters(stream, may_alloc, &fz.cnt);
    if (st != GLA_OK) return st;
    fz.states = states;
    fz.frags = apply ? frags : nullptr;
    fz.S_in = cache.S_in;
    fz.z_in = cache.z_in;
    fz.S_out = cache.S_out;
    fz.z_out = cache.z_out;
  }
  st = timed_launch(1, stream, "state kernel", [&] {
    return P.mfma ? gla::launch_state_mfma(P, k, v, gates.beta, tab, part, fz, stream)
                  : gla::launch_state_generic(P, k, v, gates.beta, tab, part, stream);
  });
  if (st != GLA_OK) return st;
  if (fz.cnt == nullptr) st = timed_launch(2, stream, "reduce kernel", [&] {
    return gla::launch_reduce(P, part, states, apply ? frags : nullptr, cache.S_in, cache.z_in,
                              cache.S_out, cache.z_out, stream);
  });
  if (st != GLA_OK) return st;
  if (!apply) return GLA_OK;
  return timed_launch(3, stream, "apply kernel", [&] {
    return P.mfma ? gla::launch_apply_mfma(P, q, g, states, frags, tab, gates.rms_w, out, stream)
                  : gla::launch_apply_generic(P, q, g, states, tab, gates.rms_w, out, stream);
  });
}

// Token-causal call: table, chunk partials, range prefixes, tile kernel.
gla_status run_causal(const Plan &P, const void *q, const void *k, const void *v, const void *g,
                      void *out, void *ws, hipStream_t stream) {
  char *base = (char *)ws;
  float *part = (float *)(base + P.off_part);
  float *states = (float *)(base + P.off_state);
  const float2 *tab = nullptr;
  gla_status st = rope_table_for(P, (float2 *)(base + P.off_tab), stream, true, &tab);
  if (st != GLA_OK) return st;
  st = timed_launch(1, stream, "state kernel", [&] {
    return P.mfma ? gla::launch_state_mfma(P, k, v, nullptr, tab, part, gla::FusedReduce(),
                                           stream)
                  : gla::launch_state_generic(P, k, v, nullptr, tab, part, stream);
  });
  if (st != GLA_OK) return st;
  st = timed_launch(2, stream, "range prefix kernel",
                    [&] { return gla::launch_range_prefix(P, part, states, stream); });
  if (st != GLA_OK) return st;
  return timed_launch(5, stream, "causal tile kernel", [&] {
    return P.mfma ? gla::launch_causal_mfma(P, q, k, v, g, states, tab, out, stream)
                  : gla::launch_causal_generic(P, q, k, v, g, states, tab, out, stream);
  });
}

gla_status forward_impl(const void *q, const void *k, const void *v, const void *g, void *out,
                        int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                        int64_t F, float theta, float eps, gla_dtype dtype, void *ws,
                        size_t ws_bytes, bool own_ws, hipStream_t stream,
                        const Step *step = nullptr, const Gates *gates = nullptr,
                        float rms_eps = 0.f, bool scratch = false, float *saved = nullptr) {
  g_last_error[0] = '\0';
  gla_status st = check_sizes(B, H, T, Hs, Ws, d, F, dtype);
  if (st != GLA_OK) return st;
  if (!std::isfinite(theta)) return fail(GLA_ERR_INVALID_ARG, "rope_theta must be finite");
  if (!std::isfinite(eps) || eps < 0.f)
    return fail(GLA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  const size_t bytes = (size_t)(B * T * Hs * Ws * H * d) * (dtype == GLA_BF16 ? 2 : 4);
  const bool apply = out != nullptr || step == nullptr;
  if (step != nullptr) {
    st = check_step(q, k, v, g, out, bytes, *step, B * H, d, T);
    if (st != GLA_OK) return st;
  } else {
    st = check_pointers(q, k, v, g, out, bytes);
    if (st != GLA_OK) return st;
  }
  if (gates != nullptr) {
    st = check_gates(*gates, out, bytes, B * T * Hs * Ws * H, d, dtype, rms_eps);
    if (st != GLA_OK) return st;
  }
  if (!own_ws && !scratch && (ws == nullptr || ((uintptr_t)ws & 255) != 0))
    return fail(GLA_ERR_INVALID_ARG, "workspace must be a non-null, 256-byte aligned pointer");
  if (saved != nullptr) {
    st = check_saved(saved, saved_state_bytes(B, H, T, F, d), bytes, {q, k, v, g, out});
    if (st != GLA_OK) return st;
  }
  int cus = 0;
  st = device_cus(&cus);
  if (st != GLA_OK) return st;
  const bool aligned16 = (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)g |
                          (uintptr_t)out) & 15) == 0;
  Plan P;
  st = make_plan(B, H, T, Hs, Ws, d, F, dtype, theta, eps, cus, aligned16, &P);
  if (st != GLA_OK) return st;
  P.rms_eps = rms_eps;
  const Gates no_gates;
  const Gates &gt = gates != nullptr ? *gates : no_gates;
  Cache cache;
  if (step != nullptr) {
    P.t0 = step->t0;
    cache.S_in = step->S_io;
    cache.z_in = step->z_io;
    if (step->update) {
      cache.S_out = step->S_io;
      cache.z_out = step->z_io;
    }
  }
  if (scratch) {
    // the library's static scratch array of this device: no allocation
    if (P.total_bytes > gla::kNoAllocScratchBytes)
      return fail(GLA_ERR_UNSUPPORTED,
                  "this call needs %zu bytes of scratch; gla_forward_noalloc has %zu per device "
                  "(use gla_forward_ws with a larger workspace)",
                  P.total_bytes, gla::kNoAllocScratchBytes);
    void *mem = nullptr;
    hipError_t e = gla::noalloc_scratch(&mem);
    if (e != hipSuccess) return hip_fail(e, "scratch address (hipGetSymbolAddress)");
    return run_plan(P, q, k, v, g, out, mem, stream, apply, cache, gt, false);
  }
  if (!own_ws) {
    if (ws_bytes < P.total_bytes)
      return fail(GLA_ERR_INVALID_ARG, "workspace too small: %zu bytes given, %zu needed", ws_bytes,
                  P.total_bytes);
    return run_plan(P, q, k, v, g, out, ws, stream, apply, cache, gt, true, nullptr, saved);
  }
  void *mem = nullptr;
  hipError_t e = hipMallocAsync(&mem, P.total_bytes, stream);
  if (e != hipSuccess || mem == nullptr) {
    (void)hipGetLastError();
    return fail(GLA_ERR_ALLOC, "hipMallocAsync of %zu workspace bytes failed: %s", P.total_bytes,
                hipGetErrorString(e));
  }
  st = run_plan(P, q, k, v, g, out, mem, stream, apply, cache, gt, true, nullptr, saved);
  e = hipFreeAsync(mem, stream);
  if (st == GLA_OK && e != hipSuccess) return hip_fail(e, "hipFreeAsync");
  return st;
}

// Gradients; with `saved` (the states a gla_forward_train call kept) the
// state stage is not re-run.
gla_status backward_impl(const void *q, const void *k, const void *v, const void *g,
                         const void *dout, void *dq, void *dk, void *dv, void *dg, int64_t B,
                         int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                         int64_t frames_per_block, float rope_theta, float eps, gla_dtype dtype,
                         void *workspace, size_t workspace_bytes, hipStream_t stream,
                         const float *saved) {
  g_last_error[0] = '\0';
  const int64_t F = frames_per_block;
  gla_status st = check_sizes(B, H, T, Hs, Ws, d, F, dtype);
  if (st != GLA_OK) return st;
  if (!std::isfinite(rope_theta)) return fail(GLA_ERR_INVALID_ARG, "rope_theta must be finite");
  if (!std::isfinite(eps) || eps < 0.f)
    return fail(GLA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  const void *ins[5] = {q, k, v, g, dout};
  const void *outs[4] = {dq, dk, dv, dg};
  const char *in_names[5] = {"q", "k", "v", "g", "dout"};
  const char *out_names[4] = {"dq", "dk", "dv", "dg"};
  for (int i = 0; i < 5; ++i)
    if (!ins[i]) return fail(GLA_ERR_INVALID_ARG, "null tensor pointer (%s)", in_names[i]);
  for (int i = 0; i < 4; ++i)
    if (!outs[i]) return fail(GLA_ERR_INVALID_ARG, "null tensor pointer (%s)", out_names[i]);
  const size_t bytes = (size_t)(B * T * Hs * Ws * H * d) * (dtype == GLA_BF16 ? 2 : 4);
  for (int o = 0; o < 4; ++o) {
    for (int i = 0; i < 5; ++i)
      if (ranges_overlap(outs[o], bytes, ins[i], bytes))
        return fail(GLA_ERR_INVALID_ARG, "%s overlaps input %s", out_names[o], in_names[i]);
    for (int o2 = o + 1; o2 < 4; ++o2)
      if (ranges_overlap(outs[o], bytes, outs[o2], bytes))
        return fail(GLA_ERR_INVALID_ARG, "%s overlaps %s", out_names[o], out_names[o2]);
  }
  if (workspace != nullptr && ((uintptr_t)workspace & 255) != 0)
    return fail(GLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (saved != nullptr) {
    st = check_saved(saved, saved_state_bytes(B, H, T, F, d), bytes,
                     {q, k, v, g, dout, dq, dk, dv, dg});
    if (st != GLA_OK) return st;
  }
  int cus = 0;
  st = device_cus(&cus);
  if (st != GLA_OK) return st;
  // (the matrix-core kernels move 16-byte pieces of q, k and v and 8-byte
  // pieces of every tensor)
  uintptr_t all = 0;
  for (const void *t : ins) all |= (uintptr_t)t;
  for (const void *t : outs) all |= (uintptr_t)t;
  const bool aligned16 = (all & 15) == 0;
  Plan P;
  st = make_plan(B, H, T, Hs, Ws, d, F, dtype, rope_theta, eps, cus, aligned16, &P);
  if (st != GLA_OK) return st;
  if (workspace != nullptr && workspace_bytes < P.bwd_total_bytes)
    return fail(GLA_ERR_INVALID_ARG, "workspace too small: %zu bytes given, %zu needed",
                workspace_bytes, P.bwd_total_bytes);
  void *mem = workspace;
  if (mem == nullptr) {
    hipError_t e = hipMallocAsync(&mem, P.bwd_total_bytes, stream);
    if (e != hipSuccess || mem == nullptr) {
      (void)hipGetLastError();
      return fail(GLA_ERR_ALLOC, "hipMallocAsync of %zu workspace bytes failed", P.bwd_total_bytes);
    }
  }
  // the forward state of the call (re-run, or the saved one), then the
  // gradient kernels
  char *base = (char *)mem;
  const float2 *tab = nullptr;
  const float *states = saved;
  if (saved != nullptr) {
    st = rope_table_for(P, (float2 *)(base + P.off_tab), stream, true, &tab);
  } else {
    st = run_plan(P, nullptr, k, v, nullptr, nullptr, mem, stream, false, Cache(), Gates(), true,
                  &tab);
    states = (const float *)(base + P.off_state);
  }
  if (st == GLA_OK) {
    st = timed_launch(4, stream, "gradient kernels", [&] {
      return gla::launch_backward(P, q, k, v, g, dout, states, tab,
                                  (float *)(base + P.off_bpart), (float *)(base + P.off_grad),
                                  (float2 *)(base + P.off_dd),
                                  dq, dk, dv, dg, stream);
    });
  }
  if (workspace == nullptr) {
    hipError_t e = hipFreeAsync(mem, stream);
    if (st == GLA_OK && e != hipSuccess) return hip_fail(e, "hipFreeAsync");
  }
  return st;
}

}  // namespace

// ===================================================================== C ABI
extern "C" {

gla_status gla_forward(const void *q, const void *k, const void *v, const void *g, void *out,
                       int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                       float rope_theta, float eps, gla_dtype dtype, hipStream_t stream) {
  return forward_impl(q, k, v, g, out, B, H, T, Hs, Ws, d, 0, rope_theta, eps, dtype, nullptr, 0,
                      true, stream);
}

gla_status gla_block_causal_forward(const void *q, const void *k, const void *v, const void *g,
                                    void *out, int64_t B, int64_t H, int64_t T, int64_t Hs,
                                    int64_t Ws, int64_t d, int64_t frames_per_block,
                                    float rope_theta, float eps, gla_dtype dtype,
                                    hipStream_t stream) {
  if (frames_per_block < 1) {
    g_last_error[0] = '\0';
    return fail(GLA_ERR_INVALID_ARG, "frames_per_block must be >= 1 (got %lld)",
                (long long)frames_per_block);
  }
  return forward_impl(q, k, v, g, out, B, H, T, Hs, Ws, d, frames_per_block, rope_theta, eps,
                      dtype, nullptr, 0, true, stream);
}

gla_status gla_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws,
                               int64_t d, int64_t frames_per_block, gla_dtype dtype,
                               size_t *bytes) {
  g_last_error[0] = '\0';
  if (!bytes) return fail(GLA_ERR_INVALID_ARG, "bytes must not be null");
  gla_status st = check_sizes(B, H, T, Hs, Ws, d, frames_per_block, dtype);
  if (st != GLA_OK) return st;
  int cus = 0;
  st = device_cus(&cus);
  if (st != GLA_OK) return st;
  // the larger of the two kernel families' needs (unaligned tensors fall
  // back to the vector kernels, whose chunking differs)
  Plan P, Pv;
  st = make_plan(B, H, T, Hs, Ws, d, frames_per_block, dtype, 10000.f, 0.f, cus, true, &P);
  if (st != GLA_OK) return st;
  st = make_plan(B, H, T, Hs, Ws, d, frames_per_block, dtype, 10000.f, 0.f, cus, false, &Pv);
  if (st != GLA_OK) return st;
  *bytes = std::max(P.total_bytes, Pv.total_bytes);
  return GLA_OK;
}

gla_status gla_forward_ws(const void *q, const void *k, const void *v, const void *g, void *out,
                          int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                          int64_t frames_per_block, float rope_theta, float eps, gla_dtype dtype,
                          void *workspace, size_t workspace_bytes, hipStream_t stream) {
  return forward_impl(q, k, v, g, out, B, H, T, Hs, Ws, d, frames_per_block, rope_theta, eps,
                      dtype, workspace, workspace_bytes, false, stream);
}

gla_status gla_forward_noalloc(const void *q, const void *k, const void *v, const void *g,
                               void *out, int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws,
                               int64_t d, int64_t frames_per_block, float rope_theta, float eps,
                               gla_dtype dtype, hipStream_t stream) {
  return forward_impl(q, k, v, g, out, B, H, T, Hs, Ws, d, frames_per_block, rope_theta, eps,
                      dtype, nullptr, 0, false, stream, nullptr, nullptr, 0.f, true);
}

gla_status gla_state(const void *k, const void *v, float *S_out, float *z_out, int64_t B,
                     int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                     int64_t frames_per_block, float rope_theta, gla_dtype dtype,
                     hipStream_t stream) {
  g_last_error[0] = '\0';
  gla_status st = check_sizes(B, H, T, Hs, Ws, d, frames_per_block, dtype);
  if (st != GLA_OK) return st;
  if (!k || !v || !S_out || !z_out) return fail(GLA_ERR_INVALID_ARG, "null pointer");
  if (!std::isfinite(rope_theta)) return fail(GLA_ERR_INVALID_ARG, "rope_theta must be finite");
  int cus = 0;
  st = device_cus(&cus);
  if (st != GLA_OK) return st;
  const bool aligned16 = (((uintptr_t)k | (uintptr_t)v) & 15) == 0;
  Plan P;
  st = make_plan(B, H, T, Hs, Ws, d, frames_per_block, dtype, rope_theta, 0.f, cus, aligned16,
                 &P);
  if (st != GLA_OK) return st;
  void *mem = nullptr;
  hipError_t e = hipMallocAsync(&mem, P.total_bytes, stream);
  if (e != hipSuccess || mem == nullptr) {
    (void)hipGetLastError();
    return fail(GLA_ERR_ALLOC, "hipMallocAsync of %zu workspace bytes failed", P.total_bytes);
  }
  st = run_plan(P, nullptr, k, v, nullptr, nullptr, mem, stream, false);
  if (st == GLA_OK) {
    // states are [units][d*d + d]; unpack to S [units][d][d] and z [units][d]
    const float *states = (const float *)((char *)mem + P.off_state);
    const size_t stride = (size_t)gla::kPartialStride(d) * sizeof(float);
    e = hipMemcpy2DAsync(S_out, (size_t)d * d * sizeof(float), states, stride,
                         (size_t)d * d * sizeof(float), (size_t)P.units, hipMemcpyDeviceToDevice,
                         stream);
    if (e == hipSuccess)
      e = hipMemcpy2DAsync(z_out, (size_t)d * sizeof(float), states + d * d, stride,
                           (size_t)d * sizeof(float), (size_t)P.units, hipMemcpyDeviceToDevice,
                           stream);
    if (e != hipSuccess) st = hip_fail(e, "state export copy");
  }
  e = hipFreeAsync(mem, stream);
  if (st == GLA_OK && e != hipSuccess) return hip_fail(e, "hipFreeAsync");
  return st;
}

gla_status gla_block_step(const void *q, const void *k, const void *v, const void *g, void *out,
                          float *S_io, float *z_io, int64_t B, int64_t H, int64_t Tb, int64_t Hs,
                          int64_t Ws, int64_t d, int64_t t_offset, int update, float rope_theta,
                          float eps, gla_dtype dtype, void *workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  Step s;
  s.t0 = t_offset;
  s.S_io = S_io;
  s.z_io = z_io;
  s.update = update != 0;
  return forward_impl(q, k, v, g, out, B, H, Tb, Hs, Ws, d, 0, rope_theta, eps, dtype, workspace,
                      workspace_bytes, workspace == nullptr, stream, &s);
}

gla_status gla_gated_forward(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, const void *rms_weight, void *out, int64_t B,
                             int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                             int64_t frames_per_block, float rope_theta, float eps, float rms_eps,
                             gla_dtype dtype, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  Gates gt;
  gt.beta = beta;
  gt.rms_w = rms_weight;
  return forward_impl(q, k, v, g, out, B, H, T, Hs, Ws, d, frames_per_block, rope_theta, eps,
                      dtype, workspace, workspace_bytes, workspace == nullptr, stream, nullptr, &gt,
                      rms_eps);
}

gla_status gla_backward(const void *q, const void *k, const void *v, const void *g,
                        const void *dout, void *dq, void *dk, void *dv, void *dg, int64_t B,
                        int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                        int64_t frames_per_block, float rope_theta, float eps, gla_dtype dtype,
                        void *workspace, size_t workspace_bytes, hipStream_t stream) {
  return backward_impl(q, k, v, g, dout, dq, dk, dv, dg, B, H, T, Hs, Ws, d, frames_per_block,
                       rope_theta, eps, dtype, workspace, workspace_bytes, stream, nullptr);
}

gla_status gla_saved_state_bytes(int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws,
                                 int64_t d, int64_t frames_per_block, size_t *bytes) {
  g_last_error[0] = '\0';
  if (!bytes) return fail(GLA_ERR_INVALID_ARG, "bytes must not be null");
  gla_status st = check_sizes(B, H, T, Hs, Ws, d, frames_per_block, GLA_F32);
  if (st != GLA_OK) return st;
  *bytes = saved_state_bytes(B, H, T, frames_per_block, d);
  return GLA_OK;
}

gla_status gla_forward_train(const void *q, const void *k, const void *v, const void *g,
                             void *out, int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws,
                             int64_t d, int64_t frames_per_block, float rope_theta, float eps,
                             gla_dtype dtype, float *saved, void *workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (saved == nullptr) {
    g_last_error[0] = '\0';
    return fail(GLA_ERR_INVALID_ARG, "saved must not be null");
  }
  return forward_impl(q, k, v, g, out, B, H, T, Hs, Ws, d, frames_per_block, rope_theta, eps,
                      dtype, workspace, workspace_bytes, workspace == nullptr, stream, nullptr,
                      nullptr, 0.f, false, saved);
}

gla_status gla_backward_saved(const void *q, const void *k, const void *v, const void *g,
                              const void *dout, void *dq, void *dk, void *dv, void *dg,
                              const float *saved, int64_t B, int64_t H, int64_t T, int64_t Hs,
                              int64_t Ws, int64_t d, int64_t frames_per_block, float rope_theta,
                              float eps, gla_dtype dtype, void *workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  if (saved == nullptr) {
    g_last_error[0] = '\0';
    return fail(GLA_ERR_INVALID_ARG, "saved must not be null");
  }
  return backward_impl(q, k, v, g, dout, dq, dk, dv, dg, B, H, T, Hs, Ws, d, frames_per_block,
                       rope_theta, eps, dtype, workspace, workspace_bytes, stream, saved);
}

gla_status gla_token_causal_forward(const void *q, const void *k, const void *v, const void *g,
                                    void *out, int64_t B, int64_t H, int64_t T, int64_t Hs,
                                    int64_t Ws, int64_t d, float rope_theta, float eps,
                                    gla_dtype dtype, void *workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  g_last_error[0] = '\0';
  gla_status st = check_sizes(B, H, T, Hs, Ws, d, 0, dtype);
  if (st != GLA_OK) return st;
  if (!std::isfinite(rope_theta)) return fail(GLA_ERR_INVALID_ARG, "rope_theta must be finite");
  if (!std::isfinite(eps) || eps < 0.f)
    return fail(GLA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  const size_t bytes = (size_t)(B * T * Hs * Ws * H * d) * (dtype == GLA_BF16 ? 2 : 4);
  st = check_pointers(q, k, v, g, out, bytes);
  if (st != GLA_OK) return st;
  if (workspace != nullptr && ((uintptr_t)workspace & 255) != 0)
    return fail(GLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  int cus = 0;
  st = device_cus(&cus);
  if (st != GLA_OK) return st;
  const bool aligned16 = (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)g |
                          (uintptr_t)out) & 15) == 0;
  Plan P;
  st = make_causal_plan(B, H, T, Hs, Ws, d, dtype, rope_theta, eps, cus, aligned16, &P);
  if (st != GLA_OK) return st;
  if (workspace != nullptr) {
    if (workspace_bytes < P.total_bytes)
      return fail(GLA_ERR_INVALID_ARG, "workspace too small: %zu bytes given, %zu needed",
                  workspace_bytes, P.total_bytes);
    return run_causal(P, q, k, v, g, out, workspace, stream);
  }
  void *mem = nullptr;
  hipError_t e = hipMallocAsync(&mem, P.total_bytes, stream);
  if (e != hipSuccess || mem == nullptr) {
    (void)hipGetLastError();
    return fail(GLA_ERR_ALLOC, "hipMallocAsync of %zu workspace bytes failed", P.total_bytes);
  }
  st = run_causal(P, q, k, v, g, out, mem, stream);
  e = hipFreeAsync(mem, stream);
  if (st == GLA_OK && e != hipSuccess) return hip_fail(e, "hipFreeAsync");
  return st;
}

gla_status gla_token_causal_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t Hs,
                                            int64_t Ws, int64_t d, gla_dtype dtype,
                                            size_t *bytes) {
  g_last_error[0] = '\0';
  if (!bytes) return fail(GLA_ERR_INVALID_ARG, "bytes must not be null");
  gla_status st = check_sizes(B, H, T, Hs, Ws, d, 0, dtype);
  if (st != GLA_OK) return st;
  int cus = 0;
  st = device_cus(&cus);
  if (st != GLA_OK) return st;
  Plan P, Pv;
  st = make_causal_plan(B, H, T, Hs, Ws, d, dtype, 10000.f, 0.f, cus, true, &P);
  if (st != GLA_OK) return st;
  st = make_causal_plan(B, H, T, Hs, Ws, d, dtype, 10000.f, 0.f, cus, false, &Pv);
  if (st != GLA_OK) return st;
  *bytes = std::max(P.total_bytes, Pv.total_bytes);
  return GLA_OK;
}

gla_status gla_backward_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws,
                                        int64_t d, int64_t frames_per_block, gla_dtype dtype,
                                        size_t *bytes) {
  g_last_error[0] = '\0';
  if (!bytes) return fail(GLA_ERR_INVALID_ARG, "bytes must not be null");
  gla_status st = check_sizes(B, H, T, Hs, Ws, d, frames_per_block, dtype);
  if (st != GLA_OK) return st;
  int cus = 0;
  st = device_cus(&cus);
  if (st != GLA_OK) return st;
  Plan P, Pv;
  st = make_plan(B, H, T, Hs, Ws, d, frames_per_block, dtype, 10000.f, 0.f, cus, true, &P);
  if (st != GLA_OK) return st;
  st = make_plan(B, H, T, Hs, Ws, d, frames_per_block, dtype, 10000.f, 0.f, cus, false, &Pv);
  if (st != GLA_OK) return st;
  *bytes = std::max(P.bwd_total_bytes, Pv.bwd_total_bytes);
  return GLA_OK;
}

const char *gla_status_string(gla_status status) {
  switch (status) {
    case GLA_OK: return "success";
    case GLA_ERR_INVALID_ARG: return "invalid argument";
    case GLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case GLA_ERR_ALLOC: return "workspace allocation failed";
    case GLA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *gla_last_error(void) { return g_last_error; }

gla_status gla_profile_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  prof_clear_locked();
  g_prof_on = enable != 0;
  return GLA_OK;
}

gla_status gla_profile_read(int64_t launches[GLA_NUM_STAGES], double total_ms[GLA_NUM_STAGES]) {
  g_last_error[0] = '\0';
  if (!launches || !total_ms) return fail(GLA_ERR_INVALID_ARG, "null output array");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (int s = 0; s < GLA_NUM_STAGES; ++s) {
    launches[s] = 0;
    total_ms[s] = 0.0;
  }
  for (auto &r : g_prof) {
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    launches[r.stage] += 1;
    total_ms[r.stage] += ms;
  }
  return GLA_OK;
}

const char *gla_stage_name(int stage) {
  if (stage < 0 || stage >= GLA_NUM_STAGES) return "";
  return kStageNames[stage];
}

int gla_uses_matrix_cores(int64_t T, int64_t Hs, int64_t Ws, int64_t d, gla_dtype dtype) {
  Plan P;
  if (make_plan(1, 1, T, Hs, Ws, d, 0, dtype, 10000.f, 0.f, 1, true, &P) != GLA_OK) return -1;
  return P.mfma ? 1 : 0;
}

}  // extern "C"
