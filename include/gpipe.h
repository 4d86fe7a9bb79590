/*
 * gpipe.h - one GPipe pipeline cell's training step on an AMD Instinct MI355X.
 *
 * Source of the method: the GPipe technical review page (zzz0906.github.io,
 * "GPipe：微批次流水线并行的大规模模型训练 — 深度技术评审"), section "GPipe algorithm in
 * detail".  A model is a sequence of L layers; GPipe cuts it into K contiguous
 * cells ("minimal interface design"), splits each mini-batch of N into M
 * micro-batches, runs the forward pass keeping only the cells' boundary
 * activations, re-computes each micro-batch's forward during the backward pass
 * (re-materialization), sums the micro-batch gradients and applies them in one
 * synchronous update ("pipeline execution flow", phases 1-3).
 *
 * This library runs one cell of L/K identical pre-LN Transformer layers
 * (LayerNorm, multi-head attention, GeLU FFN) on one GPU.
 *
 * Conventions for every entry point
 *  - Plain C types only.  Device pointers are HIP device addresses (for
 *    example from torch tensors on a ROCm device); the library never allocates
 *    or frees device memory and never keeps a pointer beyond what is stated.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Device work is only
 *    enqueued on it; calls return without waiting, so buffers must stay alive
 *    until the caller has synchronised the stream.
 *  - Errors are return codes.  On any error no device work has been enqueued
 *    and no output has been written, except GPIPE_ERR_DEVICE (a HIP launch
 *    failed part-way; outputs are then undefined).
 *  - Activations (x, target, y, dx) are row-major [N, S, D], token-major;
 *    their element type is the cell's precision (float32, or bf16 stored as
 *    uint16), and they must be 16-byte aligned.
 */
#ifndef GPIPE_H
#define GPIPE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gpipe_cell gpipe_cell; /* opaque; host-side metadata only */

typedef enum {
  GPIPE_OK = 0,
  GPIPE_ERR_INVALID = 1,     /* an argument is out of range or misaligned      */
  GPIPE_ERR_OOM = 2,         /* the plan does not fit the device's free memory */
  GPIPE_ERR_DEVICE = 3,      /* a HIP call failed                              */
  GPIPE_ERR_UNSUPPORTED = 4, /* a shape outside what the kernels implement     */
  GPIPE_ERR_STATE = 5        /* e.g. step before bind                          */
} gpipe_status;

typedef enum {
  GPIPE_FP32 = 0, /* everything in float32                                        */
  GPIPE_BF16 = 1  /* bf16 activations and weight copy; fp32 accumulation, master
                     weights, gradients, optimizer state and normalisation stats */
} gpipe_precision;

/* Per-layer tensors, in their order inside the flat parameter vector (layer
 * major: all tensors of layer 0, then layer 1, ...).  Matrices are
 * [out_features, in_features] row-major, y = x W^T + b.  w_qkv rows 0..D-1
 * produce q, D..2D-1 k, 2D..3D-1 v; head h owns columns h*D/H .. (h+1)*D/H-1. */
typedef enum {
  GPIPE_LN1_G = 0, GPIPE_LN1_B, GPIPE_W_QKV, GPIPE_B_QKV, GPIPE_W_O, GPIPE_B_O,
  GPIPE_LN2_G, GPIPE_LN2_B, GPIPE_W_1, GPIPE_B_1, GPIPE_W_2, GPIPE_B_2,
  GPIPE_N_TENSORS
} gpipe_tensor;

/* Saved activations of one layer for one micro-batch of T = (N/M)*S tokens
 * (what re-materialization rebuilds; "preliminaries 5").  Element type is the
 * cell's precision except the LayerNorm statistics (float32 pairs mean, rstd). */
typedef enum {
  GPIPE_SAVED_X = 0, /* layer input [T, D] (layer 0: the caller's x)          */
  GPIPE_SAVED_H1,    /* LN1 output [T, D]                                     */
  GPIPE_SAVED_ST1,   /* LN1 (mean, rstd) [T, 2] float32                       */
  GPIPE_SAVED_QKV,   /* [T, 3D]                                               */
  GPIPE_SAVED_P,     /* softmax [N/M, H, S, ldS], ldS = S rounded up to 8; in
                      * bf16 cells with head dim 64 or 128 (fused attention)
                      * instead the base-2 log-sum-exp of every query row,
                      * float32 [N/M, H, S]: lse2 = log2 sum_k 2^(x_k),
                      * x = (q . k) * log2(e) / sqrt(head dim)                 */
  GPIPE_SAVED_CTX,   /* attention output before the projection [T, D]         */
  GPIPE_SAVED_X1,    /* residual after attention [T, D]                        */
  GPIPE_SAVED_H2,    /* LN2 output [T, D]                                     */
  GPIPE_SAVED_ST2,   /* LN2 (mean, rstd) [T, 2] float32                       */
  GPIPE_SAVED_U,     /* FFN pre-activation [T, F]                             */
  GPIPE_SAVED_G,     /* GeLU(u) [T, F]                                        */
  GPIPE_N_SAVED
} gpipe_saved;

/* ---------------------------------------------------------------------------
 * Convolutional cells with micro-batch BatchNorm ("algorithm / BatchNorm
 * handling": during training each micro-batch is normalised with its own
 * statistics, and moving averages over the whole mini-batch are kept for
 * evaluation).  A conv cell is `blocks` residual blocks
 *     a = conv3x3(x, W1); r = ReLU(BN1(a)); z = conv3x3(r, W2); y = x + BN2(z)
 * (pad 1, stride 1, no conv bias, BN eps 1e-5, biased variance), activations
 * NHWC [N, H, W, C].  The same entry points as for Transformer cells apply
 * (param_count, param_offset with gpipe_conv_tensor, bind, sync_lowp,
 * workspace_bytes, saved_offset with gpipe_conv_saved, step, apply_update,
 * gemm_plan); the step additionally updates the moving averages bound with
 * gpipe_cell_bind_running once, after its forward phase, from the pooled
 * micro-batch moments (mean = mean of the micro-batch means; variance = mean
 * of (var_m + mu_m^2) minus mean^2, made unbiased with n/(n-1), n = N*H*W):
 *     running <- momentum * running + (1 - momentum) * statistic.
 * The re-materialized forward never touches them.
 * ------------------------------------------------------------------------- */
typedef enum {
  GPIPE_CONV_W1 = 0, /* [C_out, 3, 3, C_in] */
  GPIPE_CONV_BN1_G, GPIPE_CONV_BN1_B,
  GPIPE_CONV_W2,
  GPIPE_CONV_BN2_G, GPIPE_CONV_BN2_B,
  GPIPE_CONV_N_TENSORS
} gpipe_conv_tensor;

/* Saved tensors of one block for one micro-batch of P = (N/M)*H*W pixels.
 * Micro-batch BatchNorm makes the cell's gradients small remainders of
 * near-cancellations, so a bf16 conv cell keeps its forward activations exact
 * to about 2^-17: x and r as split pairs of bf16, [P, 2C] with hi = bf16(v) in
 * channels 0..C-1 and lo = bf16(v - hi) in channels C..2C-1 (v ~ hi + lo; the
 * forward convolutions take them as 2C-channel inputs with the weights
 * repeated over both halves), a and z in float32; only the backward's
 * operands are bf16.  In fp32 cells x and r are float32 [P, C]. */
typedef enum {
  GPIPE_CONV_SAVED_X = 0, /* block input (block 0: the caller's x, not saved) */
  GPIPE_CONV_SAVED_A,     /* conv1 output [P, C] float32 */
  GPIPE_CONV_SAVED_ST1,   /* BN1 (mean[C], rstd[C]) float32 */
  GPIPE_CONV_SAVED_R,     /* ReLU(BN1(a)) */
  GPIPE_CONV_SAVED_Z,     /* conv2 output [P, C] float32 */
  GPIPE_CONV_SAVED_ST2,   /* BN2 (mean[C], rstd[C]) float32 */
  GPIPE_CONV_N_SAVED
} gpipe_conv_saved;

/* Creates a conv cell.  Requirements: blocks, height, width > 0; channels a
 * positive multiple of 8; 0 <= bn_momentum < 1.  Errors as for
 * gpipe_cell_create. */
gpipe_status gpipe_conv_cell_create(int blocks, int channels, int height, int width,
                                    float bn_momentum, gpipe_precision prec, gpipe_cell **out);

/* Binds the moving averages of a conv cell: float32 [blocks][2 BNs][mean[C], var[C]],
 * 16-byte aligned, owned and initialised by the caller (for example mean 0,
 * var 1).  Required before gpipe_cell_step on a conv cell.
 * Errors: GPIPE_ERR_INVALID for a Transformer cell or a misaligned pointer. */
gpipe_status gpipe_cell_bind_running(gpipe_cell *cell, float *running);

/* Creates a cell of `layers` (= L/K) identical pre-LN Transformer layers:
 * x1 = x + MHA(LN1(x)), y = x1 + W2 GeLU(W1 LN2(x1) + b1) + b2, attention
 * scale 1/sqrt(d_model/heads), causal mask if `causal`, LayerNorm eps 1e-5,
 * exact-erf GeLU.  Requirements: all sizes > 0; d_model, d_ff and
 * d_model/heads multiples of 8; d_model <= 8192; seq <= 4096.
 * Errors: GPIPE_ERR_INVALID for a non-positive size or heads not dividing
 * d_model; GPIPE_ERR_UNSUPPORTED for the other requirements.  *out is set
 * only on success; free it with gpipe_cell_destroy. */
gpipe_status gpipe_cell_create(int layers, int d_model, int heads, int d_ff, int seq, int causal,
                               gpipe_precision prec, gpipe_cell **out);

gpipe_status gpipe_cell_destroy(gpipe_cell *cell); /* NULL is accepted */

/* Number of parameters P of the cell (= layers * (4D^2 + 2DF + 9D + F)). */
gpipe_status gpipe_cell_param_count(const gpipe_cell *cell, size_t *n_params);

/* Element offset and element count of tensor `tensor` of layer `layer` in the
 * flat parameter vector (and in the gradient and optimizer-state vectors,
 * which share the layout). */
gpipe_status gpipe_cell_param_offset(const gpipe_cell *cell, int layer, int tensor,
                                     size_t *offset, size_t *count);

/* Hands the cell its parameter state; the caller owns all four buffers and
 * keeps them alive while the cell is used.  Each holds P elements:
 *   master  float32 weights (read by fp32 cells, updated by gpipe_apply_update)
 *   w_lowp  bf16 copy of master used by bf16 cells' GEMMs (NULL for fp32 cells;
 *           required for bf16 cells; the caller initialises it, the update
 *           rewrites it)
 *   grad    float32 gradient accumulator (written by gpipe_cell_step)
 *   ms      float32 RMSProp mean-square state, zero-initialised by the caller
 * This is the "~12 bytes per parameter" optimizer footprint of the pages'
 * preliminaries section 2 (fp32: 12 B; bf16 adds the 2 B copy).
 * All four must be 16-byte aligned. */
gpipe_status gpipe_cell_bind(gpipe_cell *cell, float *master, void *w_lowp, float *grad,
                             float *ms);

/* Writes w_lowp <- bf16(master) (round to nearest even) for a bf16 cell, so
 * the copy the GEMMs read starts equal to the master weights; a no-op for
 * fp32 cells.  Errors: GPIPE_ERR_STATE if not bound. */
gpipe_status gpipe_cell_sync_lowp(gpipe_cell *cell, void *stream);

/* Exact device workspace needed by gpipe_cell_step(N, M, remat): one
 * micro-batch's saved activations of all layers when remat != 0 (the pages'
 * O(N + L/K * N/M) activation bound, "preliminaries 5": the boundary tensors
 * are the caller's x / y), all M micro-batches' when remat == 0, plus one
 * layer's backward transients and the reduction partials.
 * It also tells whether that fits: GPIPE_ERR_OOM when the plan -- plus the
 * parameter state (12 B/param for fp32 cells, 14 for bf16) while the cell is
 * not bound yet -- exceeds the free memory of the current device
 * (hipMemGetInfo); *bytes still receives the plan then, so the caller can
 * report the bytes it would need.  Query before allocating the workspace: a
 * query made while that workspace is allocated counts it as used.  Without a
 * visible device only the plan is reported.  Nothing is enqueued either way.
 * GPIPE_ERR_INVALID unless N > 0, M > 0 and N % M == 0.
 * (gpipe_cell_step allocates nothing, so it has no OOM of its own: it takes
 * the workspace the caller allocated after this query.) */
gpipe_status gpipe_cell_workspace_bytes(const gpipe_cell *cell, int N, int M, int remat,
                                        size_t *bytes);

/* Byte offset inside the workspace of saved tensor `which` of layer `layer`
 * for micro-batch `micro`, as laid out for gpipe_cell_step(N, M, remat).
 * With remat != 0 only one micro-batch set exists (micro must be 0); it is
 * the re-materialization's scratch, whose layer slots the step assigns as its
 * schedule needs (their contents when the step ends are unspecified).  For
 * GPIPE_SAVED_X of layer 0 (the caller's x) it returns GPIPE_ERR_INVALID.
 * Meant for inspection and tests. */
gpipe_status gpipe_cell_saved_offset(const gpipe_cell *cell, int N, int M, int remat, int micro,
                                     int layer, int which, size_t *offset, size_t *bytes);

/* One training step of the cell, phases 1 and 2 of "pipeline execution flow":
 *  - split x [N, S, D] into M micro-batches of N/M sequences (views);
 *  - forward phase: run every micro-batch through the cell, writing its
 *    boundary output into y; with remat != 0 the layer intermediates are
 *    dropped (overwritten by the next micro-batch);
 *  - backward phase, micro-batches m = 0 .. M-1 in order: with remat != 0
 *    rebuild the intermediates by re-running the forward (bitwise identical
 *    to the forward phase), take the loss against target, backpropagate,
 *    and accumulate the parameter gradients in float32: micro-batch 0 stores
 *    into grad, the others add.
 * Loss: loss = sum((y - target)^2) / (N*S*D), gradient 2(y - target)/(N*S*D)
 * for every micro-batch, so the summed gradients are the full mini-batch's.
 * Outputs: y [N,S,D]; dx [N,S,D] (gradient w.r.t. x; NULL to skip); *loss_dev
 * (a float32 on the device); grad (the bound accumulator).  x, target, y and
 * dx must not overlap the workspace.  The workspace (ws_bytes >=
 * gpipe_cell_workspace_bytes) is owned by the caller; its contents on entry
 * are ignored.  Errors: GPIPE_ERR_STATE if not bound; GPIPE_ERR_INVALID for
 * bad N/M, misaligned pointers or too small a workspace.
 * Streams: all work is enqueued behind what the caller has enqueued on
 * `stream` and the call returns after enqueueing; synchronising `stream`
 * covers the whole step.  A Transformer cell also uses two streams of its
 * own (created at its first step, default priority, on the device current
 * then; a later step on another device returns GPIPE_ERR_STATE).  With
 * remat != 0, bf16, head dim 64 or 128 and at least two layers, the forward
 * phase runs groups of consecutive micro-batches (one launch per layer for the
 * whole group) alternately on `stream` and the cell's streams; the second
 * stream then runs the weight-gradient GEMMs of the backward phase and the
 * third re-materializes micro-batch m+1 layer by layer while micro-batch m's
 * backward frees the saved set's layer slots.  Events order them against `stream` both ways, the
 * weight gradients still accumulate the micro-batches in order and the step
 * is bitwise reproducible.  A cell must not run two steps at once. */
gpipe_status gpipe_cell_step(gpipe_cell *cell, const void *x, const void *target, void *y,
                             void *dx, int N, int M, int remat, void *workspace, size_t ws_bytes,
                             void *stream, float *loss_dev);

/* The two phases of gpipe_cell_step as separate calls, for cells chained on
 * one device ("minimal interface design": a model is cut into K cells of
 * contiguous layers and communication sits only at the cell boundaries; cell
 * k's output is cell k+1's input, and in the backward pass the gradient with
 * respect to cell k+1's input is the output gradient of cell k).
 *
 * gpipe_cell_forward: phase 1 of "pipeline execution flow" -- every
 * micro-batch through the cell, y [N, S, D] (NHWC for conv cells) written,
 * with remat != 0 nothing else kept; conv cells also update the moving
 * averages as the step does.
 *
 * gpipe_cell_backward: phase 2 with the output gradient dy [N, S, D] handed
 * down by the cell above instead of a loss: for m = 0 .. M-1 in order,
 * re-materialize micro-batch m (remat != 0), backpropagate dy's rows of m,
 * accumulate the parameter gradients in float32 into the bound grad
 * (micro-batch 0 stores, the others add) and write dx [N, S, D] (NULL to
 * skip).  dy and dx have the cell's activation type (bf16 cells hand bf16
 * gradients across the boundary).  With remat == 0 the saved activations are
 * those gpipe_cell_forward left in the workspace, so both calls must get the
 * same workspace, x, N and M, with no other step of the cell in between; with
 * remat != 0 the workspace's contents on entry are ignored.
 *
 * gpipe_cell_step(x, target) equals gpipe_cell_forward followed by the
 * backward against the loss's gradient; a stack of cells c_0 .. c_{K-1} takes
 * forward(c_k, x_k, x_{k+1}) for k < K-1, step(c_{K-1}, x_{K-1}, target) and
 * then backward(c_k, x_k, dy = dx_{k+1}, dx_k) for k = K-2 .. 0, which is one
 * step of the whole stack.  Workspace, alignment, stream and error rules as
 * for gpipe_cell_step; GPIPE_ERR_INVALID also for a null dy. */
gpipe_status gpipe_cell_forward(gpipe_cell *cell, const void *x, void *y, int N, int M, int remat,
                                void *workspace, size_t ws_bytes, void *stream);
gpipe_status gpipe_cell_backward(gpipe_cell *cell, const void *x, const void *dy, void *dx, int N,
                                 int M, int remat, void *workspace, size_t ws_bytes, void *stream);

/* Size of the library's own device scratch used by gpipe_cell_step_noalloc:
 * one array per device, held from the first such call on that device until
 * the process ends. */
#define GPIPE_SCRATCH_BYTES ((size_t)64 << 20)

/* gpipe_cell_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The workspace is the library's static scratch of GPIPE_SCRATCH_BYTES on the
 * device current at the call (its address is looked up once per device), and
 * every launch goes to `stream` alone: no stream, event or memory is created,
 * and nothing is allocated or freed (role timing is not applied).  The caller
 * still provides x, target, y, dx (NULL to skip) and loss_dev; arguments,
 * results and the bound state are those of gpipe_cell_step, bitwise.  The
 * scratch's contents on entry are ignored (nothing in it has to start at
 * zero).  All calls on one device share its scratch and leave the last call's
 * contents there, so calls whose work overlaps on one GPU (other streams,
 * other threads, other cells) race: a caller must order them, for example on
 * one stream.  Transformer cells only.
 * Errors: GPIPE_ERR_OOM (no work enqueued) when gpipe_cell_workspace_bytes(N,
 * M, remat) exceeds GPIPE_SCRATCH_BYTES; GPIPE_ERR_UNSUPPORTED for a conv
 * cell; otherwise as gpipe_cell_step. */
gpipe_status gpipe_cell_step_noalloc(gpipe_cell *cell, const void *x, const void *target, void *y,
                                     void *dx, int N, int M, int remat, void *stream,
                                     float *loss_dev);

/* Phase 3, the single synchronous update: RMSProp over all P parameters,
 *   ms <- decay*ms + (1-decay)*grad^2;  master <- master - lr*grad/(sqrt(ms)+eps)
 * and, for bf16 cells, w_lowp <- bf16(master) (round to nearest even).
 * grad is read, not cleared.  Errors: GPIPE_ERR_STATE if not bound;
 * GPIPE_ERR_INVALID if decay is outside [0, 1) or lr/eps are negative or
 * not finite. */
gpipe_status gpipe_apply_update(gpipe_cell *cell, float lr, float decay, float eps, void *stream);

/* gpipe_cell_step followed by gpipe_apply_update(lr, decay, eps): the same
 * work and the same results, bit for bit, in one call.  The update stays the
 * pages' single synchronous one -- every parameter moves once, after the
 * gradients of all M micro-batches are summed -- but on a Transformer cell
 * each layer's update is enqueued as soon as that layer's gradients are
 * complete (after the last micro-batch's backward of the layer and its
 * weight gradients), on the cell's second stream, beside the backward of the
 * layers below it; the call's work on `stream` still ends after every
 * update.  A conv cell runs the two calls one after the other.
 * Errors: those of gpipe_cell_step and of gpipe_apply_update (checked before
 * any work is enqueued). */
gpipe_status gpipe_cell_step_update(gpipe_cell *cell, const void *x, const void *target, void *y,
                                    void *dx, int N, int M, int remat, void *workspace,
                                    size_t workspace_bytes, void *stream, float *loss_dev,
                                    float lr, float decay, float eps);

/* Stability options for deep stacks ("training stability challenges of deep
 * models": sharp predictions and exploding gradients, fixed by scaling the
 * feed-forward initialisation down with the depth and by clipping the
 * activations in front of a softmax that exceed a threshold).
 *
 * gpipe_cell_set_logit_clip: with threshold > 0 every attention score
 * s = q.k / sqrt(d_model/heads) is clipped to [-threshold, threshold] before
 * the softmax, in the forward, re-materialized and backward passes alike; a
 * clipped score (|s| > threshold) passes no gradient back to q and k.  The
 * attention softmax is the cell's only softmax.  0 switches clipping off (the
 * default).  Takes effect at the next step; host side only.
 * Errors: GPIPE_ERR_INVALID for a negative or non-finite threshold or a conv
 * cell.
 *
 * gpipe_cell_scale_ffn_init: divides the FFN matrices w_1 and w_2 of every
 * layer of the bound master weights by total_layers -- the depth L of the
 * whole stack the cell belongs to, not the cell's L/K -- with correctly
 * rounded float32 division, and rewrites their bf16 copy in bf16 cells.  Meant
 * right after the caller has written the initial weights; enqueued on
 * `stream`.  Errors: GPIPE_ERR_STATE if not bound; GPIPE_ERR_INVALID for
 * total_layers < 1 or a conv cell. */
gpipe_status gpipe_cell_set_logit_clip(gpipe_cell *cell, float threshold);
gpipe_status gpipe_cell_scale_ffn_init(gpipe_cell *cell, int total_layers, void *stream);

/* The cell partition of "minimal interface design": split L layers with
 * estimated costs costs[0..L-1] (finite, >= 0) into K contiguous non-empty
 * cells minimising the variance of the cells' summed costs.  Writes
 * bounds[0..K] (bounds[0] = 0, bounds[K] = L, cell k = layers
 * bounds[k] .. bounds[k+1]-1) and the variance (1/K) sum_k (C_k - mean)^2.
 * Exact minimum by dynamic programming over prefix sums, O(K L^2); among
 * equal minima the lexicographically smallest bounds.  Host only.
 * Errors: GPIPE_ERR_INVALID if L < 1, K < 1, K > L or a cost is negative or
 * not finite. */
gpipe_status gpipe_partition(const double *costs, int L, int K, int *bounds, double *variance);

/* Kernel roles of a step, for gpipe_cell_profile.  One role is one kind of
 * launch (e.g. the FFN up-projection GEMM of the forward and re-materialized
 * passes); its launches all have the same shape within a step. */
typedef enum {
  GPIPE_ROLE_LN1_FWD = 0, GPIPE_ROLE_QKV_FWD, GPIPE_ROLE_SCORES_FWD, GPIPE_ROLE_SOFTMAX_FWD,
  GPIPE_ROLE_PV_FWD, GPIPE_ROLE_OUT_FWD, GPIPE_ROLE_LN2_FWD, GPIPE_ROLE_FFN1_FWD,
  GPIPE_ROLE_FFN2_FWD, GPIPE_ROLE_MSE, GPIPE_ROLE_FFN2_DGRAD, GPIPE_ROLE_FFN2_WGRAD,
  GPIPE_ROLE_FFN1_DGRAD, GPIPE_ROLE_FFN1_WGRAD, GPIPE_ROLE_LN2_BWD, GPIPE_ROLE_OUT_DGRAD,
  GPIPE_ROLE_OUT_WGRAD, GPIPE_ROLE_DP, GPIPE_ROLE_DV, GPIPE_ROLE_SOFTMAX_BWD, GPIPE_ROLE_DQ,
  GPIPE_ROLE_DK, GPIPE_ROLE_QKV_DGRAD, GPIPE_ROLE_QKV_WGRAD, GPIPE_ROLE_LN1_BWD,
  GPIPE_ROLE_BIAS_GRAD, GPIPE_ROLE_NORM_GRAD, GPIPE_ROLE_LOSS_REDUCE, GPIPE_ROLE_RMSPROP,
  /* convolutional cells */
  GPIPE_ROLE_CONV_FWD, GPIPE_ROLE_CONV_DGRAD, GPIPE_ROLE_CONV_WGRAD, GPIPE_ROLE_IM2COL,
  GPIPE_ROLE_COL2IM, GPIPE_ROLE_BN_STATS, GPIPE_ROLE_BN_APPLY, GPIPE_ROLE_BN_BWD,
  GPIPE_ROLE_BN_RUNNING,
  /* fused attention (bf16, head dim 64 or 128): ATTN_FWD the forward, ATTN_DQ
   * the backward (dQ per query block and dK, dV per key block, in one
   * launch); ATTN_DELTA and ATTN_DKDV are no longer launched (kept so that
   * the later roles keep their values) */
  GPIPE_ROLE_ATTN_FWD, GPIPE_ROLE_ATTN_DELTA, GPIPE_ROLE_ATTN_DKDV, GPIPE_ROLE_ATTN_DQ,
  /* conv cells in bf16 with channels a multiple of 64: implicit-GEMM
   * convolution (the 3 x 3 neighbourhood gathered by the GEMM's loads) and the
   * input gradient as the convolution of dz with tap-flipped weights; the
   * weight gradient with the neighbourhood gathered along the pixels (when a
   * micro-batch's pixel count is a multiple of 64 below 2^21) */
  GPIPE_ROLE_CONV_FWD_IMPLICIT, GPIPE_ROLE_CONV_DGRAD_IMPLICIT, GPIPE_ROLE_CONV_WGRAD_IMPLICIT,
  GPIPE_N_ROLES
} gpipe_role;

/* Event timing of selected kernel roles.  With bit r of role_mask set, every
 * later launch of role r by gpipe_cell_step / forward / backward /
 * gpipe_apply_update, on whichever of the step's streams it runs, is timed
 * by two HIP events: a GEMM role's events are recorded in its own dispatch
 * (the span of its kernels), any other role's on its stream right before and
 * after the launch.  With several streams a launch's span may share the CUs
 * with other kernels: it is the time the launch took in the step.  Calling
 * it again (any mask, 0 switches timing off) discards what was recorded.  The
 * cell creates the events it needs and destroys them in gpipe_cell_destroy.
 * gpipe_cell_step_noalloc never times.
 * Errors: GPIPE_ERR_DEVICE if events cannot be created. */
gpipe_status gpipe_cell_profile(gpipe_cell *cell, unsigned long long role_mask);

/* gpipe_cell_profile timing only every `every`-th launch of each selected
 * role (the first, the every+1-th, ...; counted per role from this call), so
 * that the events' own cost (each timed launch delays the next kernel of its
 * stream by several microseconds) stays a fraction of it; every = 1 is
 * gpipe_cell_profile.  gpipe_cell_profile_read then reports the timed
 * launches only.
 * Errors: GPIPE_ERR_INVALID for a null cell or every < 1. */
gpipe_status gpipe_cell_profile_sampled(gpipe_cell *cell, unsigned long long role_mask,
                                        int every);

/* Total milliseconds and number of launches of `role` recorded since the last
 * gpipe_cell_profile call; waits for the recorded events to complete. */
gpipe_status gpipe_cell_profile_read(gpipe_cell *cell, int role, double *total_ms,
                                     long long *launches);

/* The GEMM plan a role uses in gpipe_cell_step(N, M) of this cell: macro
 * tile rows / columns and the number of k-splits (a split GEMM launches a
 * second kernel that sums the splits in order).  For roles that are not
 * GEMMs all three are 0.  Inspection only; host side, no device work.
 * Errors: GPIPE_ERR_INVALID for bad N/M or role. */
gpipe_status gpipe_cell_gemm_plan(const gpipe_cell *cell, int N, int M, int role, int *tile_m,
                                  int *tile_n, int *splits);

/* How the forward phase of gpipe_cell_step(N, M, remat) on a Transformer cell
 * is launched: on `lanes` streams (1: the caller's stream alone), `group`
 * consecutive micro-batches per launch (the last group takes the remaining
 * M mod group), and the bytes of split-K partials each lane owns in the
 * workspace, which hold the largest split product of any launch of that lane.
 * Micro-batches share a launch only where every forward product sums over k
 * in the same order as for one micro-batch, so the forward phase's boundary
 * outputs are bitwise those the re-materialization reproduces.  Inspection
 * only; host side, no device work.  Errors: GPIPE_ERR_INVALID for a conv cell
 * or bad N/M. */
gpipe_status gpipe_cell_forward_plan(const gpipe_cell *cell, int N, int M, int remat, int *lanes,
                                     int *group, size_t *lane_partial_bytes);

/* Static string naming a status code. */
const char *gpipe_status_string(gpipe_status status);

#ifdef __cplusplus
}
#endif

#endif /* GPIPE_H */
