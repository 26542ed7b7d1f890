/*
 * lingen_mate.h -- C ABI of the MI355X (gfx950) MATE token mixer library.
 *
 * MATE is LinGen's linear-complexity replacement for DiT self-attention
 * (page "Towards High-Resolution Minute-Length Text-to-Video Generation with
 * Linear Computational Complexity", English abstract).  It has two branches
 * over a T x H x W video-latent token tensor:
 *
 *   MA  Rotary Major Scan (four token orders used in turn by layer) followed
 *       by a bidirectional Mamba2 selective-SSM scan, optionally preceded by
 *       review tokens that seed the scan state (abstract; page
 *       "视频生成模子太贵太慢如何办？", section 要领：线性复杂度的 MATE 模块;
 *       page "LinGen：基于Mamba机制的线性复杂度高清长视频生成框架",
 *       section 关键算法创新 > Rotary Major Scan).
 *   TE  TEmporal Swin Attention: softmax attention inside small fixed 3D
 *       windows, the window grid shifted by half a window on odd layers
 *       (same pages, sections 要领 and 关键算法创新 > TESA).
 *
 * and y = y_MA + y_TE.  lingen_mate_fwd takes the projected tensors (x, dt,
 * B, C for the scan and q, k, v for the attention) and returns the mixed
 * tokens; lingen_mate_block_fwd (at the end of this header) adds the steps
 * and projections of the whole block around it.
 *
 * The scan uses Mamba2's scalar-A recurrence (Dao & Gu 2024): per head, with
 * state h in R^{P x N},
 *     h <- exp(dt_c * A) * h + dt_c * (x_c outer B_c),   y_c = h C_c + D x_c,
 * run once along the scan order and once along the reversed order, the two
 * outputs summed (so the skip term appears as 2 D x).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Canonical token order is (t, h, w) row-major: c = (t*H + h)*W + w,
 *   L = T*H*W tokens per batch element.
 * - Tensor pointers marked "device" are HIP device pointers owned by the
 *   caller; the library never allocates, frees or retains them.  Inputs are
 *   read only.  Outputs must not alias inputs.  All device pointers must be
 *   16-byte aligned.
 * - Layouts (contiguous, row-major, batch outermost):
 *     x        [batch, L, Hs, P]   dtype
 *     dt       [batch, L, Hs]      fp32, > 0 (already through softplus)
 *     A        [Hs]                fp32, <= 0
 *     B, C     [batch, L, G, N]    dtype (G groups; head h uses group
 *                                  h / (Hs/G), so G = 1 shares them by all heads)
 *     D        [Hs]                fp32
 *     q, k, v  [batch, L, Ha, d]   dtype
 *     y        [batch, L, Hs*P]    dtype  (head i owns columns i*P..i*P+P-1)
 *   "dtype" is shape->dtype: LINGEN_F32 or LINGEN_BF16.
 * - Every call validates its arguments on the host before it touches the GPU
 *   and returns a negative lingen_status on failure, with nothing enqueued.
 *   Device work is enqueued on `stream` and the call returns without waiting;
 *   a launch failure is reported as LINGEN_ERR_HIP.  The only state the
 *   library keeps is a per-device cache of the compute-unit count (it sizes
 *   the persistent attention grid) and, for lingen_mate_block_fwd, one
 *   rocBLAS handle per device; concurrent calls on different streams are
 *   safe if they use different outputs and workspaces.
 */
#ifndef LINGEN_MATE_H
#define LINGEN_MATE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LINGEN_OK = 0,
  LINGEN_ERR_NULL = -1,        /* a required pointer is NULL                       */
  LINGEN_ERR_SHAPE = -2,       /* sizes inconsistent or out of range               */
  LINGEN_ERR_DTYPE = -3,       /* dtype code unknown                               */
  LINGEN_ERR_ALIGN = -4,       /* a device pointer is not 16-byte aligned          */
  LINGEN_ERR_WORKSPACE = -5,   /* workspace smaller than lingen_mate_workspace_bytes */
  LINGEN_ERR_HIP = -6,         /* a HIP call or kernel launch failed               */
  LINGEN_ERR_UNSUPPORTED = -7, /* valid shape, but no compiled kernel for it       */
  LINGEN_ERR_SCRATCH = -8      /* shape needs more workspace than the fixed scratch
                                  array of lingen_mate_fwd_noalloc holds          */
} lingen_status;

typedef enum { LINGEN_F32 = 0, LINGEN_BF16 = 1 } lingen_dtype;

typedef struct {
  int32_t batch, T, H, W;          /* token grid; L = T*H*W                        */
  int32_t ssd_heads, headdim;      /* Hs, P                                        */
  int32_t d_state, ngroups, chunk; /* N, G (must divide Hs), Q (must divide L)    */
  int32_t attn_heads, attn_headdim;/* Ha, d; Ha*d must equal Hs*P                  */
  int32_t win_t, win_h, win_w;     /* TESA window; must divide T, H, W             */
  int32_t dtype;                   /* lingen_dtype of x, B, C, q, k, v, y          */
  int32_t n_review;                /* 0 (no review tokens) or rgrid_t*rgrid_h*rgrid_w */
  int32_t rpool_t, rpool_h, rpool_w;  /* review pooling block; divides T, H, W     */
  int32_t rgrid_t, rgrid_h, rgrid_w;  /* review points per axis; divides the pooled grid */
} lingen_mate_shape;

/* Compiled kernel families (anything else returns LINGEN_ERR_UNSUPPORTED):
 *   scan:      (dtype, P, N, Q) in { (F32, 32, 16, 16), (BF16, 64, 64, 64),
 *                                    (BF16, 64, 128, 128) }
 *   attention: (dtype, d, win_t*win_h*win_w) in { (F32, 32, 32), (BF16, 64, 256),
 *                                                 (BF16, 64, 27) }
 * Odd window sizes (the 3x3x3 example of the TESA section) shift by the
 * floored half window, 1 per axis of 3, the grid offset moving forward:
 * along an axis of length n the shifted cut points are s, s+w, s+2w, ...
 */

/* Human-readable name of a status code (static string, never NULL). */
const char* lingen_status_str(int status);

/* Host-only check of a shape against every rule above.  Touches no GPU. */
int lingen_mate_validate(const lingen_mate_shape* shape);

/* Bytes of device workspace that lingen_mate_fwd, lingen_ma_fwd and
 * lingen_ssd_chunk_states need for `shape` (written to *bytes).  Host only.
 * The workspace holds the per-chunk scan states of both directions, the
 * chunk decays and, with review tokens, the pooled review tokens and their
 * state.  Its contents on entry are ignored. */
int lingen_mate_workspace_bytes(const lingen_mate_shape* shape, size_t* bytes);

/* Rotary Major Scan index maps on the host (page "LinGen：基于Mamba机制的
 * 线性复杂度高清长视频生成框架", section 关键算法创新 > Rotary Major Scan).
 * mode 0: W fastest, then H, then T   (spatial row-major)
 * mode 1: H fastest, then W, then T   (spatial column-major)
 * mode 2: T fastest, then W, then H   (temporal row-major)
 * mode 3: T fastest, then H, then W   (temporal column-major)
 * perm_host[s] = canonical index of scan position s; inv_host[c] = scan
 * position of canonical token c.  Both arrays are caller-owned host memory of
 * T*H*W int32; either may be NULL to skip it.  Errors: LINGEN_ERR_SHAPE for a
 * mode outside 0..3 or a non-positive or too large (>= 2^31 tokens) grid. */
int lingen_rms_index(int32_t mode, int32_t T, int32_t H, int32_t W,
                     int32_t* perm_host, int32_t* inv_host);

/* The same map computed on the GPU by the device function the scan kernels
 * use for their loads and stores: perm_dev[s] = canonical index (device,
 * T*H*W int32). */
int lingen_rms_index_device(int32_t mode, int32_t T, int32_t H, int32_t W,
                            int32_t* perm_dev, hipStream_t stream);

/* Scan-order copy of a token tensor: dst row s = src row perm[s], rows of
 * row_bytes bytes (a multiple of 16), batch 1.  The scan kernels never make
 * this copy (they address src through the map directly); it exists to
 * measure and test the gather on its own.  src, dst: device, T*H*W*row_bytes. */
int lingen_rms_gather(const void* src, int64_t row_bytes, int32_t mode,
                      int32_t T, int32_t H, int32_t W, void* dst, hipStream_t stream);

/* Scan states at chunk boundaries for RMS mode `mode` (both directions,
 * including the review-token state when shape->n_review > 0):
 *   h_fwd[b, c, i, p, n] = forward state before the first token of chunk c,
 *   h_bwd[b, c, i, p, n] = backward state before the last token of chunk c
 *                          (i.e. after absorbing every later chunk),
 * chunks counted along the scan order, fp32, [batch, L/Q, Hs, P, N], device.
 * Needs the workspace of lingen_mate_workspace_bytes. */
int lingen_ssd_chunk_states(const void* x, const float* dt, const float* A, const void* B,
                            int32_t mode, const lingen_mate_shape* shape,
                            float* h_fwd, float* h_bwd,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* MA branch alone: y_ma = bidirectional scan along RMS order `mode` (0..3),
 * with review tokens if shape->n_review > 0.  y_ma: device, layout of y. */
int lingen_ma_fwd(const void* x, const float* dt, const float* A, const void* B,
                  const void* C, const float* D, int32_t mode,
                  const lingen_mate_shape* shape, void* y_ma,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* MA branch with a parameter set per scan direction (the reading in which
 * the two directions of the bidirectional Mamba2 block keep weights of their
 * own; lingen_ma_fwd and lingen_mate_fwd share one set between them):
 *   y_ma = scan(x_f, dt_f, A_f, B_f, C_f, D_f along the order of `mode`)
 *        + scan(x_b, dt_b, A_b, B_b, C_b, D_b along the reversed order),
 * each scan carrying its own skip D x (so y_ma holds D_f x_f + D_b x_b).
 * Layouts, dtypes and workspace as lingen_ma_fwd, for both sets.  With
 * review tokens (shape->n_review > 0; page "视频生成模子太贵太慢如何办？",
 * section 要领) each direction pools its review tokens from its own x, dt,
 * B and scans them with its own A, and starts from the state they leave.
 * With bf16 storage the forward scan's result reaches the sum with about 16
 * significant bits (kept as two bf16 halves in the workspace) and the sum
 * is rounded once. */
int lingen_ma_fwd_dirs(const void* x_f, const float* dt_f, const float* A_f, const void* B_f,
                       const void* C_f, const float* D_f,
                       const void* x_b, const float* dt_b, const float* A_b, const void* B_b,
                       const void* C_b, const float* D_b,
                       int32_t mode, const lingen_mate_shape* shape, void* y_ma,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* TE branch alone: y_te = windowed softmax attention with the window grid
 * shifted by (win_t/2, win_h/2, win_w/2) if `shifted` != 0; border windows are
 * cut, not wrapped.  Scale 1/sqrt(d).  y_te: device, layout of y. */
int lingen_te_fwd(const void* q, const void* k, const void* v, int32_t shifted,
                  const lingen_mate_shape* shape, void* y_te, hipStream_t stream);

/* TE branch with an explicit window-grid offset and either reading of a
 * shifted partition (page "LinGen：基于Mamba机制的线性复杂度高清长视频生成框架",
 * section 关键算法创新 > TESA says only that plain and shifted windows alternate):
 *   shift_t, shift_h, shift_w  grid offset per axis, 0 <= shift < window
 *                              (lingen_te_fwd uses window/2 or 0);
 *   masked = 1                 the border pieces cut off by the offset are
 *                              windows of their own (Swin's masked roll; what
 *                              lingen_te_fwd and lingen_mate_fwd compute);
 *   masked = 0                 cyclic windows: the tokens that roll past the
 *                              end join the last window of that axis, so every
 *                              window holds win_t*win_h*win_w tokens.
 * Other arguments and errors as lingen_te_fwd, plus LINGEN_ERR_SHAPE for an
 * offset outside [0, window) or masked not 0 or 1. */
int lingen_te_fwd_shift(const void* q, const void* k, const void* v,
                        int32_t shift_t, int32_t shift_h, int32_t shift_w, int32_t masked,
                        const lingen_mate_shape* shape, void* y_te, hipStream_t stream);

/* Backward pass of the TE branch: the gradients of y_te =
 * lingen_te_fwd_shift(q, k, v, shift, masked) for an upstream gradient d_out,
 *     dv = P^T d_out,  dS = P * (d_out v^T - rowsum(d_out * y_te)),
 *     dq = dS k / sqrt(d),  dk = dS^T q / sqrt(d)      (per window and head),
 * P being the softmax weights of a window (the chain rule through the
 * attention of page "LinGen：基于Mamba机制的线性复杂度高清长视频生成框架",
 * section 关键算法创新 > TESA, which training the model needs).  The
 * forward output is recomputed, not passed in.
 *   q, k, v, d_out:  device, [batch, L, Ha, d] dtype (the forward's inputs and
 *                    the gradient of its output);
 *   dq, dk, dv:      device, [batch, L, Ha, d] dtype, written in full; they
 *                    must not alias the inputs or each other.
 * Offsets and masking as lingen_te_fwd_shift.  Compiled for the forward's
 * three families: BF16 with d = 64 and 256-token windows (MFMA tiles), BF16
 * with d = 64 and 3x3x3-token windows, FP32 with d = 32 and 32-token windows
 * (fp32 loops); other valid shapes return LINGEN_ERR_UNSUPPORTED.  Errors as
 * lingen_te_fwd_shift. */
int lingen_te_bwd(const void* q, const void* k, const void* v, const void* d_out,
                  int32_t shift_t, int32_t shift_h, int32_t shift_w, int32_t masked,
                  const lingen_mate_shape* shape, void* dq, void* dk, void* dv,
                  hipStream_t stream);

/* The same forward and backward with the row statistics saved instead of
 * formed twice (memory traded for time, as a training step keeps
 * activations for its backward pass; the backward itself is the chain rule
 * through the attention of page "LinGen：基于Mamba机制的线性复杂度高清长视频生成框架",
 * section 关键算法创新 > TESA, as for lingen_te_bwd):
 *   lingen_te_fwd_saved writes y_te exactly as lingen_te_fwd_shift does (the
 *   same kernel, bit for bit) and, per query token and head, the base-2 log
 *   of its softmax denominator,
 *       lse[b, l, h] = log2 sum_j exp(q_l . k_j / sqrt(d))
 *   over the keys j of l's window (masked pairs excluded), [batch, L, Ha]
 *   fp32, device, caller-owned, overwritten;
 *   lingen_te_bwd_saved takes that y_te as o and that lse and forms
 *   D_l = sum_e d_out[l, e] o[l, e] from them instead of recomputing the
 *   forward inside every window first; the gradients are lingen_te_bwd's up
 *   to the rounding of o to the storage type.  The caller must pass the
 *   backward the q, k, v, offsets and masking its saved forward ran with.
 * Supported: BF16 with d = 64 and 256-token windows, for the forward with
 * an even head count (its kernel takes two heads per item); other valid
 * shapes return LINGEN_ERR_UNSUPPORTED.  Other arguments and errors as
 * lingen_te_fwd_shift and lingen_te_bwd. */
int lingen_te_fwd_saved(const void* q, const void* k, const void* v,
                        int32_t shift_t, int32_t shift_h, int32_t shift_w, int32_t masked,
                        const lingen_mate_shape* shape, void* y_te, float* lse,
                        hipStream_t stream);
int lingen_te_bwd_saved(const void* q, const void* k, const void* v, const void* o,
                        const void* d_out, const float* lse,
                        int32_t shift_t, int32_t shift_h, int32_t shift_w, int32_t masked,
                        const lingen_mate_shape* shape, void* dq, void* dk, void* dv,
                        hipStream_t stream);

/* The mixer: y = MA(mode = layer_idx mod 4) + TE(shifted = layer_idx odd).
 * layer_idx >= 0.  y: device, [batch, L, Hs*P] dtype; it is also used as the
 * staging buffer of the MA branch, so its contents on entry are ignored. */
int lingen_mate_fwd(const void* x, const float* dt, const float* A, const void* B,
                    const void* C, const float* D,
                    const void* q, const void* k, const void* v,
                    int32_t layer_idx, const lingen_mate_shape* shape, void* y,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* lingen_mate_fwd that also records six caller-created HIP events on
 * `stream` at the stage boundaries of the call, for timing each stage:
 *   events[0] start                     events[3] after the inter-chunk state pass
 *   events[1] after review tokens       events[4] after the chunk outputs (MA done)
 *   events[2] after the chunk states    events[5] after windowed attention (y done)
 * (events[1] follows events[0] at once when there are no review tokens).
 * Same arguments, results and errors as lingen_mate_fwd, plus LINGEN_ERR_NULL
 * for a NULL array or event and LINGEN_ERR_SHAPE for batch != 1.  The events
 * stay owned by the caller. */
int lingen_mate_fwd_events(const void* x, const float* dt, const float* A, const void* B,
                           const void* C, const float* D,
                           const void* q, const void* k, const void* v,
                           int32_t layer_idx, const lingen_mate_shape* shape, void* y,
                           void* workspace, size_t workspace_bytes, hipStream_t stream,
                           hipEvent_t* events);

/* Bytes of the device scratch array behind lingen_mate_fwd_noalloc: one
 * copy per GPU the library runs on, held until the process ends. */
#define LINGEN_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/* lingen_mate_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The workspace is a file-scope device array of LINGEN_NOALLOC_SCRATCH_BYTES
 * (256 MiB) per GPU instead of a caller-provided buffer; the call allocates
 * and frees nothing, and the caller still passes inputs and the output y.
 * Shapes whose lingen_mate_workspace_bytes exceeds that size (with the
 * 512p-like dimensions, more than about 32k tokens) return
 * LINGEN_ERR_SCRATCH before anything is enqueued; every 16,384-token shape
 * fits.  Every call on one GPU shares that GPU's array, which keeps the last
 * call's contents (the mixer writes all of it that it reads, so nothing
 * carries over): calls that overlap on one GPU, on different streams or from
 * different threads, race on it and must be serialised by the caller.  The
 * first call on a device looks up the array's device address (the HIP
 * runtime loads the library's code object for that device if it has not yet
 * done so).  Arguments, results and other errors as lingen_mate_fwd. */
int lingen_mate_fwd_noalloc(const void* x, const float* dt, const float* A, const void* B,
                            const void* C, const float* D,
                            const void* q, const void* k, const void* v,
                            int32_t layer_idx, const lingen_mate_shape* shape, void* y,
                            hipStream_t stream);

/* Dense softmax attention over all L tokens of each sequence, per head:
 *     o_i = sum_j softmax_j(q_i . k_j / sqrt(d)) v_j,   j = 0 .. L-1,
 * with no mask and no bias.  This is the quadratic self-attention of the DiT
 * baseline that MATE replaces (abstract of the first page above: linear
 * complexity in place of DiT self-attention; page "视频生成模子太贵太慢如何办？",
 * section 评估: latency and FLOPs against the attention model), provided so
 * that the two mixers can be timed at the same L, heads and head size.  It is
 * not used by lingen_mate_fwd.
 *   q, k, v, o: device, [batch, L, heads, head_dim], dtype; o must not alias
 *               the inputs.
 *   dtype:      LINGEN_F32 or LINGEN_BF16 (LINGEN_ERR_DTYPE otherwise).
 * Compiled for LINGEN_BF16 with head_dim 64 (fp32 accumulation and softmax);
 * other valid combinations return LINGEN_ERR_UNSUPPORTED.  batch, L or heads
 * equal to 0 is a no-op that does not look at the pointers; negative sizes,
 * batch or heads above 65535 and more than 2^40 elements per tensor give
 * LINGEN_ERR_SHAPE. */
int lingen_dense_attn_fwd(const void* q, const void* k, const void* v, void* o,
                          int32_t batch, int32_t L, int32_t heads, int32_t head_dim,
                          int32_t dtype, hipStream_t stream);

/* Backward pass of the MA branch: the gradients of sum(dy * y_ma) for y_ma =
 * lingen_ma_fwd(x, dt, A, B, C, D, mode), with review tokens when
 * shape->n_review > 0 (the shared-parameter bidirectional scan; [SSD]
 * recurrence, page "视频生成模子太贵太慢如何办？", section 要领：线性复杂度的 MATE
 * 模块, whose review tokens seed both directions), with respect to every
 * input:
 *   dx:  [batch, L, Hs, P] fp32      ddt: [batch, L, Hs] fp32
 *   dB, dC: [batch, L, G, N] fp32 (summed over the heads of each group)
 *   dA, dD: [Hs] fp32 (summed over tokens and batch elements)
 * all device, caller-owned, overwritten.  dy has the layout and dtype of y.
 * The gradients are assembled from the library's scan kernels run on dy
 * with other token weights (the chunk-state pass of dy against C with the
 * token weights e^{dt A}, i.e. the states of dy e^{dt A} / dt: the adjoint
 * states; the output kernel in its transposed form over those states for
 * (M_f^T + M_b^T) dy / dt, behind dx) and a per-chunk MFMA kernel for the
 * crossing sums behind ddt and dA and for dB and dC; see the source for the
 * derivation.  With review tokens the adjoint that reaches the review state
 * (the sum of the two directions' initial-state adjoints, the final carries
 * of the adjoint state pass) is walked back through the review tokens' scan
 * and each pooled token's gradient is spread over its pooling block (dx,
 * ddt, dB, dA gain these shares; dC and dD do not: the review tokens'
 * outputs are discarded).
 * Supported: the three compiled scan families (BF16, 64, 64, 64) and
 * (BF16, 64, 128, 128) (MFMA tiles), and (F32, 32, 16, 16) (fp32 loops);
 * anything else that passes lingen_mate_validate returns
 * LINGEN_ERR_UNSUPPORTED.
 * workspace: device, lingen_ma_bwd_workspace_bytes (two scan workspaces,
 * whose bf16 chunk states the kernels read, plus the crossing sums, the
 * transposed outputs and, with review tokens, their gradients).
 * Errors: those of lingen_mate_validate; LINGEN_ERR_UNSUPPORTED as above;
 * LINGEN_ERR_SHAPE for mode outside 0..3; LINGEN_ERR_NULL / _ALIGN for a
 * pointer; LINGEN_ERR_WORKSPACE. */
int lingen_ma_bwd_workspace_bytes(const lingen_mate_shape* shape, size_t* bytes);
int lingen_ma_bwd(const void* x, const float* dt, const float* A, const void* B, const void* C,
                  const float* D, const void* dy, int32_t mode, const lingen_mate_shape* shape,
                  float* dx, float* ddt, float* dA, float* dB, float* dC, float* dD,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The same backward pass with the forward scan states saved by the forward
 * instead of computed again (memory traded for time, as a training step
 * keeps activations for its backward pass): lingen_ma_fwd_saved computes
 * y_ma exactly as lingen_ma_fwd does and leaves, per batch element, the
 * chunk states of both scan directions (and, with review tokens, the pooled
 * review tokens) in `saved`; lingen_ma_bwd_saved then reads them in place
 * of its first chunk-state pass (a chunk-state launch and a two-direction
 * state pass per batch element).  The kernels and their order are those of
 * lingen_ma_fwd and lingen_ma_bwd: y_ma (no atomic sums) and dx equal
 * theirs bit for bit, the other gradients up to the order in which their
 * floating-point atomic sums land.
 *   saved:  device, caller-owned, lingen_ma_saved_bytes (per batch
 *           element, the scan workspace lingen_ma_fwd runs in: mostly its
 *           chunk states, 2 * (L / chunk) * Hs * P * N storage elements);
 *           written by lingen_ma_fwd_saved, read by
 *           lingen_ma_bwd_saved, which must be given the same x, dt, A, B,
 *           mode and shape (nothing checks that it was).
 *   workspace of lingen_ma_bwd_saved: lingen_ma_bwd_saved_workspace_bytes
 *           (lingen_ma_bwd's without its first scan workspace).
 * Other arguments, supported families and errors: those of lingen_ma_fwd
 * and lingen_ma_bwd; LINGEN_ERR_WORKSPACE also when saved_bytes is below
 * lingen_ma_saved_bytes. */
int lingen_ma_saved_bytes(const lingen_mate_shape* shape, size_t* bytes);
int lingen_ma_fwd_saved(const void* x, const float* dt, const float* A, const void* B, const void* C,
                        const float* D, int32_t mode, const lingen_mate_shape* shape, void* y_ma,
                        void* saved, size_t saved_bytes, hipStream_t stream);
int lingen_ma_bwd_saved_workspace_bytes(const lingen_mate_shape* shape, size_t* bytes);
int lingen_ma_bwd_saved(const void* x, const float* dt, const float* A, const void* B, const void* C,
                        const float* D, const void* dy, const void* saved, size_t saved_bytes,
                        int32_t mode, const lingen_mate_shape* shape, float* dx, float* ddt, float* dA,
                        float* dB, float* dC, float* dD, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* ----------------------------------------------------------------------------
 * Steps around the scan.  The MA branch is a bidirectional Mamba2 block (page
 * "视频生成模子太贵太慢如何办？", section 要领：线性复杂度的 MATE 模块); these two
 * calls carry out the elementwise steps of that block either side of the
 * scan, in the layout of the Mamba-2 architecture (Dao & Gu 2024, section 7:
 * a short depthwise causal convolution with SiLU on the x, B, C channels and
 * a softplus on dt before the scan, a SiLU(z) gate with a grouped RMS norm
 * after it).  Where the pages leave the step open, the readings taken are:
 * the convolution is causal along the order the scan visits the tokens (so
 * each direction of the scan convolves along its own order, with its own
 * weights), and dt is shared by both directions.
 * ------------------------------------------------------------------------- */

/* Before the scan, for RMS order `mode` (0..3):
 *   x_f | B_f | C_f = silu(conv_f(xbc)) along the scan order of `mode`,
 *   x_b | B_b | C_b = silu(conv_b(xbc)) along the reversed order,
 *   dt[b, l, i]     = softplus(dt_raw[b, l, i] + dt_bias[i]),
 * where for the token at scan position s (taps before the first position
 * are zero), channel c and K = conv_k taps,
 *   conv(u)[order[s], c] = bias[c] + sum_{k<K} w[c, k] u[order[s-K+1+k], c].
 *   xbc:          device, [batch, L, Hs*P + 2*G*N], shape->dtype, canonical
 *                 token order; channels x (Hs*P, head-major) then B (G*N)
 *                 then C (G*N).
 *   dt_raw:       device, [batch, L, Hs] fp32.      dt_bias: device, [Hs] fp32.
 *   conv_w_f/_b:  device, [Hs*P + 2*G*N, K] fp32.   conv_b_f/_b: device,
 *                 [Hs*P + 2*G*N] fp32 (forward / backward direction).
 *   x_f, x_b:     device outputs, layout of x;  B_f, C_f, B_b, C_b: layout
 *                 of B;  dt: device output, layout of dt.  These are the
 *                 inputs lingen_ma_fwd_dirs takes.
 * The shape must pass lingen_mate_validate.  Errors: those of
 * lingen_mate_validate; LINGEN_ERR_SHAPE for mode outside 0..3, conv_k
 * outside 1..4, or Hs*P or G*N not a multiple of 16 bytes of elements;
 * LINGEN_ERR_NULL / _ALIGN for a pointer. */
int lingen_ma_prep(const void* xbc, const float* dt_raw, const float* conv_w_f,
                   const float* conv_b_f, const float* conv_w_b, const float* conv_b_b,
                   const float* dt_bias, int32_t conv_k, int32_t mode,
                   const lingen_mate_shape* shape, void* x_f, void* B_f, void* C_f,
                   void* x_b, void* B_b, void* C_b, float* dt, hipStream_t stream);

/* lingen_ma_prep followed by lingen_ma_fwd_dirs in one pass per direction:
 * the convolution, SiLU and softplus are taken inside the scan kernels, on
 * the rows the scan reads (each chunk also reads the conv_k - 1 positions
 * before it), and none of x_f .. C_b or dt is written to memory.  Results
 * equal those of the two calls: every value is formed with the same
 * operations in the same order.
 *   xbc, dt_raw, dt_bias, conv_w_f/_b, conv_b_f/_b, conv_k, mode: as
 *                 lingen_ma_prep.   A_f, D_f, A_b, D_b: as lingen_ma_fwd_dirs
 *                 (the dt of both directions is softplus(dt_raw + dt_bias)).
 *   y_ma:         device output, layout of y.
 *   workspace:    device, lingen_mate_workspace_bytes(shape) bytes.
 * It reads xBC twice per direction instead of writing and reading the six
 * convolved tensors, but forms the convolution in both scan kernels of each
 * direction; lingen_mate_block_fwd takes the two calls, the faster form on
 * MI355X at the benchmark workloads.
 * Errors: those of lingen_ma_prep and lingen_ma_fwd_dirs;
 * LINGEN_ERR_UNSUPPORTED for fp32 storage or review tokens
 * (shape->n_review > 0), which take the two calls instead. */
int lingen_ma_fwd_dirs_conv(const void* xbc, const float* dt_raw, const float* dt_bias,
                            int32_t conv_k, const float* conv_w_f, const float* conv_b_f,
                            const float* A_f, const float* D_f, const float* conv_w_b,
                            const float* conv_b_b, const float* A_b, const float* D_b,
                            int32_t mode, const lingen_mate_shape* shape, void* y_ma,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* After the scan: for every row r of `rows` and channel c of `dim`,
 *   g[r, c]   = y[r, c] * silu(z[r, c]),
 *   out[r, c] = g[r, c] / sqrt(mean_{c' in group(c)} g[r, c']^2 + eps) * weight[c],
 * the groups being `group` consecutive channels.
 *   y, z, out: device, [rows, dim], dtype (LINGEN_F32 or LINGEN_BF16); the
 *              arithmetic is fp32, out rounded once.  out may not alias y, z.
 *   weight:    device, [dim] fp32.
 * rows = 0 is a no-op that does not look at the pointers.  Errors:
 * LINGEN_ERR_DTYPE; LINGEN_ERR_SHAPE for rows < 0 or >= 2^31, dim < 1,
 * group < 1, group not dividing dim, group not a multiple of 16 bytes of
 * elements (8 bf16, 4 fp32), dim above 8192 (bf16) / 4096 (fp32), or eps < 0;
 * LINGEN_ERR_NULL / _ALIGN for a pointer. */
int lingen_gated_rmsnorm(const void* y, const void* z, const float* weight, float eps,
                         int64_t rows, int32_t dim, int32_t group, int32_t dtype,
                         void* out, hipStream_t stream);

/* ----------------------------------------------------------------------------
 * The whole MATE block: the mixer with the projections around both branches
 * (page "视频生成模子太贵太慢如何办？", section 要领：线性复杂度的 MATE 模块: an MA
 * branch and a TE branch replace the block's self-attention).  Readings where
 * the pages are silent: the MA branch is laid out as a Mamba-2 block (Dao &
 * Gu 2024, section 7) with one input projection per product (z, xBC, dt),
 * the convolution of lingen_ma_prep, the per-direction scan of
 * lingen_ma_fwd_dirs, the gated norm of lingen_gated_rmsnorm with one norm
 * group per B/C group, and an output projection; the TE branch projects q,
 * k, v, attends as lingen_te_fwd and projects its output; the block returns
 * the sum of the two projected outputs.  The projections carry no bias.
 * ------------------------------------------------------------------------- */

/* Weights of one block, all device pointers owned by the caller, 16-byte
 * aligned.  Projection matrices are row-major [out, in] in the shape dtype
 * (y = u W^T); Dm = d_model, d = Hs*P = Ha*d_head, Ch = d + 2*G*N. */
typedef struct {
  const void* w_z;          /* [d, Dm]  gate z                                   */
  const void* w_xbc;        /* [Ch, Dm] x, B, C channels                         */
  const void* w_dt;         /* [Hs, Dm] dt_raw (product kept in fp32)            */
  const float* conv_w_f;    /* [Ch, K] fp32, forward direction                   */
  const float* conv_b_f;    /* [Ch]                                              */
  const float* conv_w_b;    /* [Ch, K] fp32, backward direction                  */
  const float* conv_b_b;    /* [Ch]                                              */
  const float* dt_bias;     /* [Hs]                                              */
  const float* A_f;         /* [Hs] <= 0, forward scan                           */
  const float* D_f;         /* [Hs]                                              */
  const float* A_b;         /* [Hs] <= 0, backward scan                          */
  const float* D_b;         /* [Hs]                                              */
  const float* norm_w;      /* [d] gated-norm weight                             */
  const void* w_out_ma;     /* [Dm, d] MA output projection                      */
  const void* w_q;          /* [d, Dm]                                           */
  const void* w_k;          /* [d, Dm]                                           */
  const void* w_v;          /* [d, Dm]                                           */
  const void* w_o;          /* [Dm, d] TE output projection                      */
} lingen_mate_block_weights;

/* Workspace size of lingen_mate_block_fwd for `shape` and `d_model`.
 * Errors as lingen_mate_block_fwd's shape checks; LINGEN_ERR_NULL for a NULL
 * `bytes`. */
int lingen_mate_block_workspace_bytes(const lingen_mate_shape* shape, int32_t d_model,
                                      size_t* bytes);

/* out = MA(u) + TE(u) for u [batch, L, d_model] (canonical token order,
 * shape dtype), RMS mode = layer_idx mod 4 and shifted windows on odd
 * layer_idx as in lingen_mate_fwd; conv_k taps (1..4); norm_eps >= 0.
 * Review tokens (shape->n_review > 0) enter the MA branch as in
 * lingen_ma_fwd_dirs, pooled from each direction's scan inputs (after the
 * convolution).
 *   out:       device, [batch, L, d_model], shape dtype; must not alias u.
 *   workspace: device, at least lingen_mate_block_workspace_bytes bytes,
 *              16-byte aligned; its contents on return are unspecified.
 * The projections run as rocBLAS GEMMs (fp32 accumulation) on `stream`; the
 * library keeps one rocBLAS handle per device for them, created at the first
 * call on that device, and serialises its use with a lock.  Intermediates
 * (z, xBC, q, k, v, the scan output and the normed output) are stored in the
 * shape dtype; dt_raw and dt in fp32.
 * Errors, all found before anything is enqueued: those of
 * lingen_mate_validate; LINGEN_ERR_SHAPE for d_model outside 1..65536,
 * batch*L of 2^31 or more, layer_idx < 0, conv_k outside 1..4, eps < 0, or
 * d, G*N or d/G not a multiple of 16 bytes of elements or d above 8192
 * (bf16) / 4096 (fp32); LINGEN_ERR_NULL / _ALIGN for a pointer (weights
 * included);
 * LINGEN_ERR_WORKSPACE.  A failing rocBLAS call is reported as
 * LINGEN_ERR_HIP, with the earlier steps already enqueued. */
int lingen_mate_block_fwd(const void* u, const lingen_mate_block_weights* w, int32_t d_model,
                          int32_t conv_k, float norm_eps, int32_t layer_idx,
                          const lingen_mate_shape* shape, void* out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LINGEN_MATE_H */
