// Host-callable launchers of the cell's HIP kernels (internal to the library).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gp {

// ---------------------------------------------------------------- GEMM
// LAY_CONV: the A operand is the 3 x 3 im2col matrix of an NHWC image that is
// never materialised: row p, column tap*C + c reads pixel p shifted by the
// tap's (dh, dw), or zero outside the image (A only, k-tiles within one tap).
// LAY_CONV_MN: the B operand is that matrix with the pixels along k
// (B(k, n) = im2col[k][n], n = tap*C + c), for the convolution's weight
// gradient; the k extent (pixels) must stay below 2^21.
enum { LAY_K = 0, LAY_MN = 1, LAY_CONV = 2, LAY_CONV_MN = 3 };

enum {
  EPI_STORE = 0,       // C(act) = alpha * acc
  EPI_BIAS = 1,        // C(act) = acc + bias[n]
  EPI_BIAS_RESID = 2,  // C(act) = acc + bias[n] + R(act)[m, n]
  EPI_BIAS_GELU = 3,   // U(act) = acc + bias[n] (unless U is null);  C(act) = gelu(U)
  EPI_GELU_BWD = 4,    // C(act) = acc * gelu'(U(act)[m, n])
  EPI_STORE_F32 = 5,   // C(f32) = alpha * acc
  EPI_ACC_F32 = 6,     // C(f32) = (beta ? C : 0) + acc
};

// Causal structure of the attention products (rows i, keys j, j <= i kept):
//   SKIP_UPPER:  output tiles entirely above the diagonal are not computed
//   K_UPTO_M:    reduction over k < (tile's last row + 1)   (P.V, dS.K)
//   K_FROM_M:    reduction over k >= tile's first row       (P^T.dC, dS^T.Q)
// The masked entries of P and dS are stored as exact zeros, so the partial
// k-tiles these modes keep contribute nothing extra.
enum { CAUSAL_NONE = 0, CAUSAL_SKIP_UPPER = 1, CAUSAL_K_UPTO_M = 2, CAUSAL_K_FROM_M = 3 };

struct GemmParams {
  int M, N, K;
  const void* A; int64_t lda, sAb, sAh;   // element strides; batch z -> (z / hdiv, z % hdiv)
  const void* B; int64_t ldb, sBb, sBh;
  void* C; int64_t ldc, sCb, sCh;
  int hdiv;
  int causal;
  const float* bias;
  const void* R; int64_t ldr;
  void* U; int64_t ldu;
  float alpha;
  int beta;
  float* P;     // split-K partials [splits][M][N] (f32), required when the plan splits
  int kchunk;   // split-K: k extent of one split (set by gemm())
  int conv_h, conv_w, conv_c;  // image geometry of a LAY_CONV operand
  int conv_ld;  // pixel stride of a LAY_CONV_MN image in elements (0: conv_c)
  // Optional (weight-gradient roles, where gemm_rowsum_parts() > 0): partial
  // sums of A over k, rowsum[t * M + m] for tile column t, written (beta = 0)
  // or added (beta = 1) like C; summed over t they
  // give the row sums (each tile column adds up its own share of the k-tiles).
  float* rowsum;
};

// Macro tile and split-K chosen for one GEMM launch.
struct GemmPlan {
  int cfg;      // tile configuration (gemm_impl.hpp), -1 for the fp32 kernel
  int splits;   // k-splits reduced in a fixed order by a second kernel
  int kchunk;
};
GemmPlan plan_gemm(int role, bool bf16, int M, int N, int K, int batch);
// bf16 GEMM with a given plan (the planner's choice is gemm(); this form lets
// a benchmark compare tile configurations).  The partial buffer g.P must hold
// splits * M * N floats when the plan splits.
hipError_t gemm_with_plan(int role, const GemmPlan& plan, const GemmParams& g, int batch, hipStream_t s);
// Number of partial row-sum vectors (GemmParams::rowsum) the bf16 launch of
// this role and shape writes, 0 where it cannot: the bias gradient of a
// weight-gradient product, from the tiles of the output gradient in LDS.
int gemm_rowsum_parts(int role, const GemmParams& g, int batch);
int gemm_cfg_bm(int cfg);
int gemm_cfg_bn(int cfg);
// Floats of split-K partials the launch needs (0 if it does not split).
size_t gemm_partial_floats(int role, bool bf16, int M, int N, int K, int batch);

// role: a gpipe_role of a GEMM launch; it fixes the operand layouts and the
// epilogue (see gemm.hip) and names the kernel instance in profiles.
hipError_t gemm(bool bf16, int role, const GemmParams& g, int batch, hipStream_t s);

// Role timing inside the dispatch.  When start / stop are set (host side, by
// the step driver's role timing), the next GEMM launch records them in its
// own dispatch packets -- start at the beginning of its first kernel, stop
// at the end of its last -- and clears them, so the measured interval is the
// kernels' execution, not the enqueue around it.  Per host thread.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& launch_events();
// An event the next launch through launch_k() (or a GEMM's last kernel) records
// when its kernel ends, in that kernel's own dispatch packet -- no packet of
// its own on the stream, which would hold back the stream's next kernel by a
// few microseconds -- and clears.  Set only right before a call whose last
// kernel should take it; the caller records it on the stream if it is still
// pending afterwards.
hipEvent_t& next_done_event();
template <typename K, typename... A>
hipError_t launch_k(K kernel, dim3 grid, dim3 block, uint32_t smem, hipStream_t s, A... args) {
  hipEvent_t& d = next_done_event();
  if (d) {
    const hipEvent_t e = d;
    d = nullptr;
    hipExtLaunchKernelGGL(kernel, grid, block, smem, s, nullptr, e, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, smem, s, args...);
  }
  return hipGetLastError();
}
// true for the roles whose launch is a gemm() call (they take the events)
bool gemm_role(int role);

// ---------------------------------------------------------------- row kernels
// LayerNorm forward over rows of length D: y(act) = gamma*(x-mu)*rstd + beta, stats[2*row] = (mu, rstd).
hipError_t layernorm_fwd(bool bf16, const void* x, void* y, float* stats, const float* gamma,
                         const float* beta, int rows, int d, float eps, hipStream_t s);

// LayerNorm backward.  dh: f32 [rows, d] gradient w.r.t. the LN output; x: act input;
// res_in: f32 residual gradient added to dx; writes dx_f32 (may alias res_in) and dx_act;
// per-block partial sums of dgamma and dbeta written (beta = 0) or added (beta = 1) to
// part[nblk][2][d]; returns nblk via *nblk (at most 256 whatever the row count).
hipError_t layernorm_bwd(bool bf16, const float* dh, const void* x, const float* stats,
                         const float* gamma, const float* res_in, float* dx_f32, void* dx_act,
                         float* part, int rows, int d, int beta, int* nblk, hipStream_t s);
int layernorm_bwd_blocks(int rows, int d);

// Softmax forward of scores (f32, already scaled) into P(act); rows of length n, row pitch ld,
// optional causal mask (key j > row index i within its [n x n] block); masked entries -> 0.
// clip > 0: the scores are clipped to [-clip, clip] first (logit clipping).
hipError_t softmax_fwd(bool bf16, const float* scores, void* p, int64_t rows, int n, int64_t ld,
                       int causal, float clip, hipStream_t s);
// Softmax backward: dS(act) = scale * P * (dP - rowsum(P*dP)); masked entries -> 0.  With
// keep_in_ds, ds holds the clip's keep mask on entry (clip_keep) and clipped entries get 0.
hipError_t softmax_bwd(bool bf16, const void* p, const float* dp, void* ds, int64_t rows, int n,
                       int64_t ld, int causal, float scale, int keep_in_ds, hipStream_t s);
// keep(act) = 1 where |scores| <= clip, else 0 (same row layout as softmax_fwd).
hipError_t clip_keep(bool bf16, const float* scores, void* keep, int64_t rows, int n, int64_t ld,
                     int causal, float clip, hipStream_t s);
// w[i] = w[i] / d over n floats (correctly rounded fp32 division).
hipError_t div_scalar(float* w, int64_t n, float d, hipStream_t s);

// MSE: r = y - t over `count` elements; dy = 2 r / denom into dy_f32 and dy_act;
// per-block partial sums of r^2 / denom into part[nblk].
hipError_t mse_fwd_bwd(bool bf16, const void* y, const void* t, float* dy_f32, void* dy_act,
                       float* part, int64_t count, float inv_denom, int* nblk, hipStream_t s);
int mse_blocks(int64_t count);
// The output gradient handed down by the cell above: dy (act, count a multiple
// of 8) into dy_f32 and its act copy dy_act.
hipError_t grad_in(bool bf16, const void* dy, float* dy_f32, void* dy_act, int64_t count, hipStream_t s);

// Column sums: part[chunk][c] = sum over the rows of chunk of x[r, c] (x is f32 or act).
hipError_t colsum_partial(int xtype, const void* x, int64_t ld, int rows, int cols, float* part,
                          int* nchunk, hipStream_t s);
int colsum_chunks(int rows);
// out[c] = (beta ? out[c] : 0) + sum_p part[p * stride + c], p = 0 .. nparts-1 in order;
// acc (optional) receives the same sum the same way under acc_beta.
hipError_t sum_partials(const float* part, int nparts, int64_t stride, int cols, float* out,
                        int beta, hipStream_t s, float* acc = nullptr, int acc_beta = 0);
// Several such sums (beta 0, no acc) in one launch, each bitwise what
// sum_partials computes; jobs of fewer than 32 columns are launched one by one.
struct SumJob {
  const float* part;
  float* out;
  int64_t stride;
  int nparts, cols;
};
constexpr int kSumJobsMax = 64;  // per launch (the jobs travel in the kernel arguments)
hipError_t sum_partials_batch(const SumJob* jobs, int njobs, hipStream_t s);

// RMSProp over n parameters; writes the bf16 copy when w_lowp is non-null.
hipError_t rmsprop(float* w, const float* g, float* ms, void* w_lowp, int64_t n, float lr,
                   float decay, float eps, hipStream_t s, int max_blocks = 0);

// ---------------------------------------------------------------- conv cell
// Storage of a conv-cell activation: float32 [P][C], bf16 [P][C], or a split
// pair of bf16 [P][2C] (hi = bf16(v) in channels 0 .. C-1, lo = bf16(v - hi)
// in C .. 2C-1; v ~ hi + lo to about 2^-17 relative).
enum { SK_F32 = 0, SK_BF16 = 1, SK_SPLIT = 2 };
// col [B*H*W, 9*C] from x [B, H, W, ldx] (its first C channels; pad 1); column (kh*3 + kw)*C + c.
hipError_t im2col(bool bf16, const void* x, int ldx, void* col, int B, int H, int W, int C,
                  hipStream_t s);
// dx = res (optional) + adjoint of im2col applied to dcol (f32); writes f32 and (optional) act.
hipError_t col2im(bool bf16, const float* dcol, const float* res, float* dx_f32, void* dx_act,
                  int B, int H, int W, int C, hipStream_t s);
int bn_chunks(int64_t rows);
// Per-channel statistics over `rows` rows: stats = (mean[C], rstd[C]); rec (optional) = (mean, biased var).
hipError_t bn_stats(bool bf16, const void* x, int64_t rows, int C, float eps, float* part,
                    float* stats, float* rec, hipStream_t s);
// From float32 a:  mode 0: out = relu(bn(a));  mode 1: out = res + bn(a); res and out
// stored as the given SK_* kinds (mode 0: out f32 or split; mode 1: res/out f32/f32,
// bf16/split, split/split, split/bf16 or bf16/bf16; res may be out).
hipError_t bn_apply(int mode, const float* a, const float* stats, const float* gamma,
                    const float* beta, const void* res, int res_kind, void* out, int out_kind,
                    int64_t rows, int C, hipStream_t s);
// Backward of bn over float32 a (mask: dy is multiplied by [r > 0], r stored f32 or split);
// sums = (sum dy*xhat, sum dy) of this batch (part: [chunks][2C] scratch), also stored
// (grad_beta = 0) or added into grad [2C] (the gain and shift gradients); da = input gradient
// stored as da_kind (f32 or bf16).
hipError_t bn_bwd(int da_kind, int mask, const float* dy_src, const void* r, int r_kind,
                  const float* a, const float* stats, const float* gamma, float* part, float* sums,
                  float* grad, int grad_beta, void* da, int64_t rows, int C, int* nchunk,
                  hipStream_t s);
// Moving averages from the M micro-batches' recorded moments.
hipError_t bn_running(const float* rec, int M, int nbn, int C, int64_t n_total, float momentum,
                      float* running, hipStream_t s);
// [C][9][2C] weights repeating [C][9][C] over both halves of a split input (bf16).
hipError_t conv_dup_weights(const void* src, void* dst, int C, hipStream_t s);

// ---------------------------------------------------------------- fused attention
// bf16 cells with head dim 64 or 128.  qkv [B*S][3D], ctx/dctx [B*S][D],
// lse2/delta [B*H][S] float32, dqkv [B*S][3D].
bool flash_ok(bool bf16, int dh);
// clip > 0: logit clipping, every score q.k/sqrt(dh) limited to [-clip, clip]
// before the softmax; in the backward a clipped score passes no gradient.
hipError_t flash_fwd(const void* qkv, void* ctx, float* lse2, int B, int H, int S, int D,
                     int causal, float clip, hipStream_t s);
// dQ, dK and dV in one launch (each block computes the row sums rowsum(dctx * ctx) it needs)
hipError_t flash_bwd(const void* qkv, const void* ctx, const void* dctx, const float* lse2,
                     void* dqkv, int B, int H, int S, int D, int causal, float clip, hipStream_t s);

// Tap-flipped, transposed 3 x 3 weights: dst[c][t][o] = src[o][8 - t][c] (bf16, C x C x 9);
// the input gradient of a convolution is the convolution of its output gradient with them.
hipError_t conv_flip_weights(const void* src, void* dst, int C, hipStream_t s);

// dst = bf16(src), n elements.
hipError_t to_bf16(const float* src, void* dst, int64_t n, hipStream_t s);

enum { XT_F32 = 0, XT_BF16 = 2 };

}  // namespace gp
