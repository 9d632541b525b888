/*
 * gla.h - C ABI of libgla.so, the gated ReLU linear-attention token mixer on
 * AMD MI355X (CDNA4, gfx950).
 *
 * The operator (per batch b and head h; phi = ReLU; RoPE = 3D rotary
 * embedding over the (t, h, w) latent grid):
 *
 *   S   = sum_n RoPE_n(phi(k_n))^T v_n          d x d, rows = key feature
 *   z   = sum_n phi(k_n)                         d
 *   o_i = (RoPE_i(phi(q_i)) S) / (phi(q_i) . z + eps)  *  sigmoid(g_i)
 *
 * Sources: "SANA-Video 2.0: Hybrid Linear Attention with Attention Residuals
 * for Efficient Video Generation" (arXiv 2607.21553), Section 2, paragraph
 * "Gated linear attention", Eq. (1) (the +eps denominator and the sigmoid
 * output gate g); "SANA-Video: Efficient Video Generation with Block Linear
 * Diffusion Transformer" (paper notes), Section 3.2 "Linear Attention with
 * RoPE" (ReLU feature map, RoPE applied after ReLU and only in the
 * numerator, tensors laid out (B, N, H, D)) and Section 3.4 "Block Linear
 * Attention with Constant-Memory KV Cache" (the running sums of phi(K)^T V
 * and phi(K) carried across temporal blocks).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  q, k, v, g and out are dense [B, N, H, d] arrays (d fastest),
 *   N = T * Hs * Ws, tokens in t-major order: token n sits at
 *   t = n / (Hs*Ws), h = (n / Ws) % Hs, w = n % Ws.
 * Element type.  GLA_BF16: every tensor is bfloat16 (raw 16-bit storage);
 *   GLA_F32: every tensor is float.  Arithmetic is fp32 in both cases
 *   (bf16 matrix-core products accumulate in fp32); bf16 outputs are rounded
 *   to nearest-even once, at the store.
 * Positions and RoPE.  d is split (d/4, 3d/8, 3d/8) over (t, h, w); on each
 *   axis the adjacent feature pairs (2i, 2i+1) of that axis' slice rotate by
 *   pos_axis * rope_theta^(-2i/d_axis).  rope_theta <= 0 disables the
 *   rotation.  Positions are the integer grid indices starting at 0.
 * Supported sizes.  B, H, T, Hs, Ws >= 1; 16 <= d <= 128 with d % 16 == 0.
 *   bf16 with d = 64 or d = 128 and 16-byte-aligned tensors runs on the
 *   matrix-core kernels; every other supported case (fp32, other d,
 *   misaligned tensors, grids whose table slices exceed the kernels' LDS)
 *   runs on the vector kernels.
 * Memory.  Every tensor pointer is device memory owned by the caller; the
 *   library neither frees nor keeps any of them.  out may not overlap an
 *   input.
 * Streams.  All work is enqueued on `stream` (NULL = the null stream) with
 *   no host synchronisation; GLA_OK means "enqueued".  Errors raised by a
 *   kernel at run time surface at the caller's next synchronisation.
 * Errors.  Arguments are validated on the host before any HIP call, and
 *   the dynamic-LDS attributes of all the library's kernels are set on a
 *   device before the library's first launch there: a call that returns
 *   GLA_ERR_INVALID_ARG, GLA_ERR_UNSUPPORTED or GLA_ERR_ALLOC has enqueued
 *   nothing.  GLA_ERR_HIP means that the HIP runtime refused a call or a
 *   launch; when it refuses a later launch of a call, earlier kernels of
 *   that call may already be enqueued, and the call's outputs (for
 *   gla_block_step with update also the cache, for gla_forward_train also
 *   the saved state) are then unspecified.
 *   gla_last_error() returns a description of the last failure on the
 *   calling thread.  No C++ exception crosses this interface.
 * Library memory.  On each device the library keeps, until the process
 *   ends: the RoPE (cos, sin) table of every (T, Hs, Ws, d, rope_theta,
 *   t_offset) it has met, up to 256 of them (T*d/8 + 3*(Hs + Ws)*d/16
 *   entries of 8 bytes each, computed on the calling stream by a shape's
 *   first call), and a set of 256 KiB of counters for each stream it has run
 *   on, up to 64 streams (zeroed on that stream by its first call).  Any
 *   entry point may allocate these at first use; gla_forward_noalloc and
 *   calls made during stream capture never do (they compute the table into
 *   their workspace and run the reduce as a kernel of its own, with bitwise
 *   the same results).
 * Determinism.  For identical inputs, shapes and device, results are
 *   bitwise identical run to run (fixed-order reductions, no float atomics).
 */
#ifndef GLA_H
#define GLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

typedef enum {
  GLA_OK = 0,
  GLA_ERR_INVALID_ARG = 1, /* a null pointer, a bad size, overlapping out */
  GLA_ERR_UNSUPPORTED = 2, /* valid arguments the library cannot run */
  GLA_ERR_ALLOC = 3,       /* workspace allocation failed */
  GLA_ERR_HIP = 4          /* a HIP runtime call or a launch failed */
} gla_status;

typedef enum { GLA_BF16 = 0, GLA_F32 = 1 } gla_dtype;

/*
 * Non-causal operator ("SANA-Video 2.0" Eq. (1) without beta, RMSNorm and
 * W_o; "SANA-Video" Section 3.2).  Every token reads the state and
 * normaliser of all N tokens of its (batch, head).
 * The workspace is taken stream-ordered on `stream` (hipMallocAsync) and
 * released the same way; GLA_ERR_ALLOC if that fails.
 */
gla_status gla_forward(const void *q, const void *k, const void *v, const void *g, void *out,
                       int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                       float rope_theta, float eps, gla_dtype dtype, hipStream_t stream);

/*
 * Block-causal operator ("SANA-Video" Section 3.4): the T latent frames form
 * T / frames_per_block temporal blocks of frames_per_block * Hs * Ws
 * consecutive tokens.  A token of block b reads the state and normaliser
 * summed over every token of blocks 0..b (its own block included, so
 * attention within a block is bidirectional).  Positions stay absolute.
 * frames_per_block must divide T; frames_per_block == T gives gla_forward.
 */
gla_status gla_block_causal_forward(const void *q, const void *k, const void *v, const void *g,
                                    void *out, int64_t B, int64_t H, int64_t T, int64_t Hs,
                                    int64_t Ws, int64_t d, int64_t frames_per_block,
                                    float rope_theta, float eps, gla_dtype dtype,
                                    hipStream_t stream);

/*
 * Workspace size in bytes for one call with these sizes on the current
 * device (frames_per_block = 0: non-causal).  The size depends on the
 * device's compute-unit count.  Writes *bytes; GLA_ERR_INVALID_ARG on bad
 * sizes.
 */
gla_status gla_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws,
                               int64_t d, int64_t frames_per_block, gla_dtype dtype,
                               size_t *bytes);

/*
 * Either operator with a caller-owned workspace (device memory, at least
 * gla_workspace_bytes() bytes, 256-byte aligned); frames_per_block = 0 is
 * the non-causal operator.  Allocates no per-call memory (only the library
 * memory described above, at first use).  Calls that share a workspace must
 * be ordered on one stream.
 */
gla_status gla_forward_ws(const void *q, const void *k, const void *v, const void *g, void *out,
                          int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                          int64_t frames_per_block, float rope_theta, float eps, gla_dtype dtype,
                          void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * gla_forward_ws without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and errors as gla_forward_ws (frames_per_block = 0:
 * non-causal), bitwise identical to it.  The kernels use a static scratch
 * array of 64 MiB that the library holds on each device it runs on until
 * the process ends; a call whose workspace (gla_workspace_bytes) exceeds it
 * returns GLA_ERR_UNSUPPORTED before enqueueing anything.  Every call on a
 * device shares that device's array (each call fully rewrites what it
 * reads, so nothing carries over between calls): calls that overlap in time
 * on one device race, so order them on one stream.
 */
gla_status gla_forward_noalloc(const void *q, const void *k, const void *v, const void *g,
                               void *out, int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws,
                               int64_t d, int64_t frames_per_block, float rope_theta, float eps,
                               gla_dtype dtype, hipStream_t stream);

/*
 * Diagnostic export of the state and normaliser ("SANA-Video" Section 3.2
 * steps 3-4, Section 3.4 cache): S_out [B, H, nb, d, d] and z_out
 * [B, H, nb, d] as float (device memory), nb = T / frames_per_block (1 when
 * frames_per_block = 0).  Block b holds the sums over blocks 0..b.  These
 * are the fp32 values the output stage reads (before any bf16 rounding).
 */
gla_status gla_state(const void *k, const void *v, float *S_out, float *z_out, int64_t B,
                     int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                     int64_t frames_per_block, float rope_theta, gla_dtype dtype,
                     hipStream_t stream);

/*
 * The gated mixer of "SANA-Video 2.0" Section 2, Eq. (1), short of the
 * output projection W_o: the operator above plus
 *   - the write gate beta ([B, N, H], the tensors' element type; NULL: 1):
 *       S = sum_n beta_n RoPE_n(phi(k_n))^T v_n   (z keeps the plain phi(k));
 *   - the RMSNorm of y_i = num_i / den_i over its d features, before the
 *     output gate (rms_weight [d], the tensors' type; NULL: no RMSNorm):
 *       o_i = y_i / sqrt(mean_e y_i[e]^2 + rms_eps) * rms_weight * sigmoid(g_i).
 * beta is used as given (any activation that produces it happens upstream);
 * the RMSNorm weight is shared by the heads.  rms_eps must be finite and
 * > 0 when rms_weight is given.  frames_per_block as gla_forward_ws (0:
 * non-causal).  workspace: NULL (stream-ordered allocation, like
 * gla_forward) or at least gla_workspace_bytes() bytes, 256-byte aligned.
 * With beta and rms_weight both NULL this is gla_forward_ws.
 */
gla_status gla_gated_forward(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, const void *rms_weight, void *out, int64_t B,
                             int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                             int64_t frames_per_block, float rope_theta, float eps, float rms_eps,
                             gla_dtype dtype, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * One step of the streaming block-causal mode ("SANA-Video" Section 3.4
 * and its Algorithm 1, the constant-memory cache): one temporal block of
 * Tb latent frames (q, k, v, g, out are [B, Tb*Hs*Ws, H, d]) whose first
 * frame sits at absolute temporal position t_offset, read against a
 * caller-owned cache of the sums over every earlier block:
 *   S_io [B, H, d, d] float (rows = key feature), z_io [B, H, d] float,
 *   device memory, 4-byte aligned.
 * With S_blk, z_blk the block's own state and normaliser, the block attends
 * to itself and to the cache:
 *   out = (RoPE(phi(q)) (S_io + S_blk)) / (phi(q) . (z_io + z_blk) + eps)
 *         * sigmoid(g)
 * and, when update != 0, the cache then takes the block's sums in place:
 *   S_io += S_blk, z_io += z_blk.
 * Feeding the blocks of a grid in order (t_offset = 0, Tb, 2 Tb, ...) with
 * update = 1 from a zeroed cache reproduces gla_block_causal_forward with
 * frames_per_block = Tb; the cache costs 4 (d*d + d) bytes per (batch,
 * head) whatever the video length.
 * out == NULL (q and g may then be NULL) only updates the cache, as after
 * the last denoising step of a block; out == NULL with update == 0 is
 * GLA_ERR_INVALID_ARG.  The cache may not overlap any tensor.
 * workspace: NULL (taken stream-ordered on `stream`, like gla_forward) or
 * at least gla_workspace_bytes(B, H, Tb, Hs, Ws, d, 0, dtype) bytes of
 * device memory, 256-byte aligned (then no per-call memory is allocated).
 */
gla_status gla_block_step(const void *q, const void *k, const void *v, const void *g, void *out,
                          float *S_io, float *z_io, int64_t B, int64_t H, int64_t Tb, int64_t Hs,
                          int64_t Ws, int64_t d, int64_t t_offset, int update, float rope_theta,
                          float eps, gla_dtype dtype, void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * Gradients of the non-causal or block-causal operator (frames_per_block = 0
 * or its block size): with the loss L = sum over every element of
 * dout * out, writes dq = dL/dq, dk, dv and dg ([B, N, H, d], the tensors'
 * element type, device memory; none may overlap another or an input).
 * By the chain rule through the definition above ("SANA-Video 2.0" Eq. (1),
 * "SANA-Video" Sections 3.2 and 3.4); the derivative of ReLU at 0 is taken
 * as 0, and in block-causal mode a block's keys and values receive the
 * gradients of every later block that reads them.  The call re-runs the
 * state stage, then the gradient kernels: on the matrix cores for bf16 with
 * d = 64 or 128 and 16-byte aligned tensors (bf16 hi + lo operands, fp32
 * accumulation), else fp32 arithmetic on the vector units.
 * workspace: NULL (taken stream-ordered on `stream`) or at least
 * gla_backward_workspace_bytes() bytes of device memory, 256-byte aligned.
 */
gla_status gla_backward(const void *q, const void *k, const void *v, const void *g,
                        const void *dout, void *dq, void *dk, void *dv, void *dg, int64_t B,
                        int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                        int64_t frames_per_block, float rope_theta, float eps, gla_dtype dtype,
                        void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace of gla_backward with these sizes on the current device. */
gla_status gla_backward_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws,
                                        int64_t d, int64_t frames_per_block, gla_dtype dtype,
                                        size_t *bytes);

/*
 * The training pair: a forward that keeps its state, and gradients that take
 * it instead of re-running the state stage (the same chain rule as
 * gla_backward; S and z are the sums of "SANA-Video 2.0" Eq. (1) and the
 * "SANA-Video" notes page, Section 3.2, per temporal block in block-causal
 * mode as in its Section 3.4).
 *
 * saved: caller-owned device memory of gla_saved_state_bytes() bytes,
 * 256-byte aligned, overlapping no tensor of the call.  Layout: one record
 * of d*d + d fp32 per (batch, head, temporal block), in that order, b
 * slowest: S row-major [p][e] (feature p of the rotated key, e of the
 * value), then z [p]; in block-causal mode a block's record holds the sums
 * over that block and every earlier one (what the block's outputs read).
 *
 * gla_forward_train: gla_forward_ws (workspace may be NULL: taken
 * stream-ordered on `stream`), which also writes the record of every
 * (batch, head, block) into `saved`.
 * gla_backward_saved: gla_backward with the records of a gla_forward_train
 * call on the same k, v, sizes, frames_per_block and rope_theta (nothing
 * checks that they match: other contents give the gradients of another
 * state); enqueues the gradient kernels only.
 * Both return GLA_ERR_INVALID_ARG for a null, misaligned or overlapping
 * `saved`, before any launch.
 */
gla_status gla_saved_state_bytes(int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                                 int64_t frames_per_block, size_t *bytes);
gla_status gla_forward_train(const void *q, const void *k, const void *v, const void *g, void *out,
                             int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t d,
                             int64_t frames_per_block, float rope_theta, float eps,
                             gla_dtype dtype, float *saved, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);
gla_status gla_backward_saved(const void *q, const void *k, const void *v, const void *g,
                              const void *dout, void *dq, void *dk, void *dv, void *dg,
                              const float *saved, int64_t B, int64_t H, int64_t T, int64_t Hs,
                              int64_t Ws, int64_t d, int64_t frames_per_block, float rope_theta,
                              float eps, gla_dtype dtype, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * Token-causal form ("SANA-Video" notes page, Section 3.4: the causal
 * linear-attention output of token i, the form behind the constant-memory
 * cache): token i of a (batch, head) attends to tokens 0..i of the t-major
 * flattened grid, itself included:
 *   S_i = sum_{j<=i} RoPE_j(phi(k_j))^T v_j,   z_i = sum_{j<=i} phi(k_j)
 *   out_i = (RoPE_i(phi(q_i)) S_i) / (phi(q_i) . z_i + eps) * sigmoid(g_i)
 * with the RoPE, eps and gate of gla_forward.  Tensors, layout, dtype,
 * alignment, ownership and errors as gla_forward.  Computed chunkwise: a
 * state stage over chunks of tokens, an exclusive prefix over the chunks,
 * then per range of tokens a tile kernel that adds each tile's own
 * (lower-triangular) part to the carried sums; the result does not depend on
 * the decomposition beyond rounding.
 * workspace: NULL (taken stream-ordered on `stream`) or at least
 * gla_token_causal_workspace_bytes() bytes of device memory, 256-byte
 * aligned (then no per-call memory is allocated).
 */
gla_status gla_token_causal_forward(const void *q, const void *k, const void *v, const void *g,
                                    void *out, int64_t B, int64_t H, int64_t T, int64_t Hs,
                                    int64_t Ws, int64_t d, float rope_theta, float eps,
                                    gla_dtype dtype, void *workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* Workspace of gla_token_causal_forward with these sizes on the current device. */
gla_status gla_token_causal_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t Hs,
                                            int64_t Ws, int64_t d, gla_dtype dtype,
                                            size_t *bytes);

/* Static description of a status code. */
const char *gla_status_string(gla_status status);

/* Description of the last failure on the calling thread ("" if none). */
const char *gla_last_error(void);

/*
 * Stage timing.  While enabled, every launch the library makes is bracketed
 * by HIP events recorded on the launch stream.  gla_profile_read() waits for
 * the recorded events and returns, per stage, the number of launches and
 * their summed duration in milliseconds.  Stages: 0 rope table, 1 state
 * partials, 2 reduce/prefix, 3 apply, 4 gradient kernels (gla_backward),
 * 5 token-causal tile kernel (gla_token_causal_forward).  Enabling (or
 * disabling) clears the record.  Meant for one thread at a time.
 */
#define GLA_NUM_STAGES 6
gla_status gla_profile_enable(int enable);
gla_status gla_profile_read(int64_t launches[GLA_NUM_STAGES], double total_ms[GLA_NUM_STAGES]);
const char *gla_stage_name(int stage);

/* Which kernels a call with these sizes would run: 1 the matrix-core
 * kernels (bf16, d = 64 or 128, and a latent grid whose spatial RoPE rows
 * fit in LDS), 0 the vector kernels, -1 invalid sizes. */
int gla_uses_matrix_cores(int64_t T, int64_t Hs, int64_t Ws, int64_t d, gla_dtype dtype);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H */
