// Memory-bound kernels of the cell step: LayerNorm, softmax, MSE, column sums,
// RMSProp.  Every reduction has a fixed combination order (no float atomics),
// so a step is bitwise reproducible and re-materialization rebuilds exactly
// the activations of the forward phase.
//
// Rows are processed in chunks of 8 elements (one 16-byte bf16 vector or two
// float4), so row lengths must be multiples of 8.
#include "common.hpp"
#include "kernels.hpp"

namespace gp {

// ------------------------------------------------------------ LayerNorm forward
// One wave per row; lane owns chunks lane, lane+64, ... (NV of them).
template <typename T, int NV>
__global__ __launch_bounds__(256) void ln_fwd_kernel(const T* __restrict__ x, T* __restrict__ y,
                                                     float* __restrict__ stats,
                                                     const float* __restrict__ gamma,
                                                     const float* __restrict__ beta, int rows,
                                                     int d, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int nch = d >> 3;
  const T* xr = x + int64_t(row) * d;
  // the gain and shift are loaded with the row, so the output needs no
  // second memory round trip after the two reductions
  float v[NV][8], gm[NV][8], bt[NV][8];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      load8<T>(xr + c * 8, v[i]);
      load8<float>(gamma + c * 8, gm[i]);
      load8<float>(beta + c * 8, bt[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[i][e];
    }
  }
  const float mu = wave_sum(s) / float(d);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = v[i][e] - mu;
        q += t * t;
      }
    }
  }
  const float var = wave_sum(q) / float(d);
  const float rstd = 1.0f / sqrtf(var + eps);
  T* yr = y + int64_t(row) * d;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (v[i][e] - mu) * rstd * gm[i][e] + bt[i][e];
      store8<T>(yr + c * 8, o);
    }
  }
  if (lane == 0) {
    stats[2 * row] = mu;
    stats[2 * row + 1] = rstd;
  }
}

template <typename T>
static hipError_t ln_fwd_t(const void* x, void* y, float* stats, const float* g, const float* b,
                           int rows, int d, float eps, hipStream_t s) {
  const int nch = d / 8;
  dim3 grid((rows + 3) / 4), blk(256);
  const T* xp = static_cast<const T*>(x);
  T* yp = static_cast<T*>(y);
  if (nch <= 64) hipLaunchKernelGGL((ln_fwd_kernel<T, 1>), grid, blk, 0, s, xp, yp, stats, g, b, rows, d, eps);
  else if (nch <= 128) hipLaunchKernelGGL((ln_fwd_kernel<T, 2>), grid, blk, 0, s, xp, yp, stats, g, b, rows, d, eps);
  else if (nch <= 256) hipLaunchKernelGGL((ln_fwd_kernel<T, 4>), grid, blk, 0, s, xp, yp, stats, g, b, rows, d, eps);
  else if (nch <= 512) hipLaunchKernelGGL((ln_fwd_kernel<T, 8>), grid, blk, 0, s, xp, yp, stats, g, b, rows, d, eps);
  else if (nch <= 1024) hipLaunchKernelGGL((ln_fwd_kernel<T, 16>), grid, blk, 0, s, xp, yp, stats, g, b, rows, d, eps);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t layernorm_fwd(bool bf16, const void* x, void* y, float* stats, const float* gamma,
                         const float* beta, int rows, int d, float eps, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  return bf16 ? ln_fwd_t<bf16_t>(x, y, stats, gamma, beta, rows, d, eps, s)
              : ln_fwd_t<float>(x, y, stats, gamma, beta, rows, d, eps, s);
}

// ------------------------------------------------------------ LayerNorm backward
// A block of 256 threads takes chunks of kLnRows consecutive rows (chunk
// blockIdx.x, then every gridDim.x-th); thread owns chunks tid, tid+256, ...
// of every row, so it also owns those columns' dgamma/dbeta partial sums,
// which it writes (beta = 0) or adds to the block's partial row (beta = 1)
// once.  The grid is capped, so the partial rows do not grow with the rows.
constexpr int kLnRows = 8;
constexpr int kLnMaxBlocks = 256;

template <typename T, int NVB>
__global__ __launch_bounds__(256) void ln_bwd_kernel(const float* __restrict__ dh,
                                                     const T* __restrict__ x,
                                                     const float* __restrict__ stats,
                                                     const float* __restrict__ gamma,
                                                     const float* res_in, float* dx_f32,
                                                     T* __restrict__ dx_act,
                                                     float* __restrict__ part, int rows, int d,
                                                     int beta) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int nch = d >> 3;
  float pg[NVB][8], pb[NVB][8];
#pragma unroll
  for (int i = 0; i < NVB; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) pg[i][e] = pb[i][e] = 0.f;
  for (int r0 = blockIdx.x * kLnRows; r0 < rows; r0 += gridDim.x * kLnRows)
  for (int row = r0, r1 = min(rows, r0 + kLnRows); row < r1; ++row) {
    const float mu = stats[2 * row], rstd = stats[2 * row + 1];
    float xh[NVB][8], dxh[NVB][8];
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int i = 0; i < NVB; ++i) {
      const int c = tid + 256 * i;
      if (c < nch) {
        float xv[8], gv[8];
        load8<T>(x + int64_t(row) * d + c * 8, xv);
        load8<float>(dh + int64_t(row) * d + c * 8, gv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xh[i][e] = (xv[e] - mu) * rstd;
          dxh[i][e] = gv[e] * gamma[c * 8 + e];
          sa += dxh[i][e];
          sb += dxh[i][e] * xh[i][e];
          pg[i][e] += gv[e] * xh[i][e];
          pb[i][e] += gv[e];
        }
      }
    }
    const float ma = block_sum(sa, red) / float(d);
    const float mb = block_sum(sb, red) / float(d);
#pragma unroll
    for (int i = 0; i < NVB; ++i) {
      const int c = tid + 256 * i;
      if (c < nch) {
        float rv[8], o[8];
        load8<float>(res_in + int64_t(row) * d + c * 8, rv);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = rv[e] + rstd * (dxh[i][e] - ma - xh[i][e] * mb);
        store8<float>(dx_f32 + int64_t(row) * d + c * 8, o);
        store8<T>(dx_act + int64_t(row) * d + c * 8, o);
      }
    }
  }
  float* pgo = part + int64_t(blockIdx.x) * 2 * d;
#pragma unroll
  for (int i = 0; i < NVB; ++i) {
    const int c = tid + 256 * i;
    if (c < nch) {
      if (beta) {
        float og[8], ob[8];
        load8<float>(pgo + c * 8, og);
        load8<float>(pgo + d + c * 8, ob);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pg[i][e] += og[e];
          pb[i][e] += ob[e];
        }
      }
      store8<float>(pgo + c * 8, pg[i]);
      store8<float>(pgo + d + c * 8, pb[i]);
    }
  }
}

// One wave per row, four rows per block at a time (rows of up to 4096): the
// row's two reductions are wave butterflies.  Block b takes row groups b,
// b + gridDim.x, ...; each wave sums its rows' dgamma / dbeta terms in
// registers, the four waves' sums are added in wave order through LDS and
// written (beta = 0) or added (beta = 1) to the block's partial row once.
constexpr int kLnWaveRows = 4;

template <typename T, int NV>
__global__ __launch_bounds__(256) void ln_bwd_wave_kernel(const float* __restrict__ dh,
                                                          const T* __restrict__ x,
                                                          const float* __restrict__ stats,
                                                          const float* __restrict__ gamma,
                                                          const float* res_in, float* dx_f32,
                                                          T* __restrict__ dx_act,
                                                          float* __restrict__ part, int rows,
                                                          int d, int beta) {
  extern __shared__ float lds[];  // [4][d]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nch = d >> 3;
  float* out = part + int64_t(blockIdx.x) * 2 * d;
  // the block's partial row, to be added to (beta), is loaded before the rows
  // (its own memory round trip overlaps theirs)
  constexpr int CPT = (NV * 64 + 255) / 256;  // chunks per thread in the fold
  float prev[2][CPT][8];
  if (beta)
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = threadIdx.x + 256 * j;
        if (c < nch) load8<float>(out + half * d + c * 8, prev[half][j]);
      }
  float pg[NV][8], pb[NV][8];
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) pg[i][e] = pb[i][e] = 0.f;
  for (int row = blockIdx.x * kLnWaveRows + w; row < rows; row += gridDim.x * kLnWaveRows) {
    const float mu = stats[2 * row], rstd = stats[2 * row + 1];
    // the residual gradient is loaded with the other inputs (no second
    // memory round trip after the reductions)
    float xh[NV][8], dxh[NV][8], rv[NV][8];
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = lane + 64 * i;
      if (c < nch) {
        float xv[8], gv[8], gm[8];
        load8<T>(x + int64_t(row) * d + c * 8, xv);
        load8<float>(dh + int64_t(row) * d + c * 8, gv);
        load8<float>(gamma + c * 8, gm);
        load8<float>(res_in + int64_t(row) * d + c * 8, rv[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xh[i][e] = (xv[e] - mu) * rstd;
          dxh[i][e] = gv[e] * gm[e];
          sa += dxh[i][e];
          sb += dxh[i][e] * xh[i][e];
          pg[i][e] += gv[e] * xh[i][e];
          pb[i][e] += gv[e];
        }
      }
    }
    const float ma = wave_sum(sa) / float(d);
    const float mb = wave_sum(sb) / float(d);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = lane + 64 * i;
      if (c < nch) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = rv[i][e] + rstd * (dxh[i][e] - ma - xh[i][e] * mb);
        store8<float>(dx_f32 + int64_t(row) * d + c * 8, o);
        store8<T>(dx_act + int64_t(row) * d + c * 8, o);
      }
    }
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = lane + 64 * i;
      if (c < nch) store8<float>(lds + w * d + c * 8, half ? pb[i] : pg[i]);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = threadIdx.x + 256 * j;
      if (c >= nch) continue;
      float s[8], v[8];
      load8<float>(lds + c * 8, s);
#pragma unroll
      for (int r = 1; r < kLnWaveRows; ++r) {
        load8<float>(lds + r * d + c * 8, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += v[e];
      }
      if (beta) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += prev[half][j][e];
      }
      store8<float>(out + half * d + c * 8, s);
    }
    __syncthreads();
  }
}

int layernorm_bwd_blocks(int rows, int d) {
  const int per = (d / 8 <= 512) ? kLnWaveRows : kLnRows;
  return std::min((rows + per - 1) / per, kLnMaxBlocks);
}

template <typename T>
static hipError_t ln_bwd_t(const float* dh, const void* x, const float* stats, const float* gamma,
                           const float* res_in, float* dx_f32, void* dx_act, float* part,
                           int rows, int d, int beta, hipStream_t s) {
  const int nch = d / 8;
  dim3 grid(layernorm_bwd_blocks(rows, d)), blk(256);
  const T* xp = static_cast<const T*>(x);
  T* op = static_cast<T*>(dx_act);
  const size_t sh = size_t(kLnWaveRows) * d * 4;
#define GP_LNW(NV) launch_k((ln_bwd_wave_kernel<T, NV>), grid, blk, sh, s, dh, xp, stats, gamma, res_in, dx_f32, op, part, rows, d, beta)
  if (nch <= 64) GP_LNW(1);
  else if (nch <= 128) GP_LNW(2);
  else if (nch <= 256) GP_LNW(4);
  else if (nch <= 512) GP_LNW(8);
#undef GP_LNW
  else if (nch <= 256) launch_k((ln_bwd_kernel<T, 1>), grid, blk, 0, s, dh, xp, stats, gamma, res_in, dx_f32, op, part, rows, d, beta);
  else if (nch <= 512) launch_k((ln_bwd_kernel<T, 2>), grid, blk, 0, s, dh, xp, stats, gamma, res_in, dx_f32, op, part, rows, d, beta);
  else if (nch <= 1024) launch_k((ln_bwd_kernel<T, 4>), grid, blk, 0, s, dh, xp, stats, gamma, res_in, dx_f32, op, part, rows, d, beta);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t layernorm_bwd(bool bf16, const float* dh, const void* x, const float* stats,
                         const float* gamma, const float* res_in, float* dx_f32, void* dx_act,
                         float* part, int rows, int d, int beta, int* nblk, hipStream_t s) {
  *nblk = layernorm_bwd_blocks(rows, d);
  if (rows == 0) return hipSuccess;
  return bf16 ? ln_bwd_t<bf16_t>(dh, x, stats, gamma, res_in, dx_f32, dx_act, part, rows, d, beta, s)
              : ln_bwd_t<float>(dh, x, stats, gamma, res_in, dx_f32, dx_act, part, rows, d, beta, s);
}

// ------------------------------------------------------------ softmax
// One wave per row of length n (row pitch ld >= n rounded up to 8); rows are
// grouped in [n x n] blocks, so the query index of a row is row % n.  Causal
// rows keep keys j <= i; the other entries of P, and the row padding, are
// written as zeros.
// clip > 0: every score is first clipped to [-clip, clip] (logit clipping).
template <typename T, int NV>
__global__ __launch_bounds__(256) void softmax_fwd_kernel(const float* __restrict__ sc,
                                                          T* __restrict__ p, int64_t rows, int n,
                                                          int64_t ld, int causal, float clip) {
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int valid = causal ? int(row % n) + 1 : n;
  const int nch = (n + 7) >> 3;  // the last chunk may run into the row padding
  const float* sr = sc + row * ld;
  float v[NV][8];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c < nch && c * 8 < valid) {
      load8<float>(sr + c * 8, v[i]);
      if (clip > 0.f)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] = fminf(fmaxf(v[i][e], -clip), clip);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (c * 8 + e >= valid) v[i][e] = -INFINITY;
        mx = fmaxf(mx, v[i][e]);
      }
    }
  }
  mx = wave_max(mx);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c < nch && c * 8 < valid) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[i][e] = (c * 8 + e < valid) ? expf(v[i][e] - mx) : 0.f;
        sum += v[i][e];
      }
    }
  }
  const float inv = 1.0f / wave_sum(sum);
  T* pr = p + row * ld;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      float o[8];
      const bool live = c * 8 < valid;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = live ? v[i][e] * inv : 0.f;
      store8<T>(pr + c * 8, o);
    }
  }
}

// keep_in_ds: ds holds on entry the clip's keep mask (clip_keep_kernel: 1 where
// the score passed the clip unchanged, 0 where it was clipped); a clipped
// score gets no gradient.  Each thread reads its own chunk of the mask
// before it overwrites it with dS.
template <typename T, int NV>
__global__ __launch_bounds__(256) void softmax_bwd_kernel(const T* __restrict__ p,
                                                          const float* __restrict__ dp,
                                                          T* ds, int64_t rows, int n,
                                                          int64_t ld, int causal, float scale,
                                                          int keep_in_ds) {
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int valid = causal ? int(row % n) + 1 : n;
  const int nch = (n + 7) >> 3;  // the last chunk may run into the row padding
  float pv[NV][8], gv[NV][8];
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c < nch && c * 8 < valid) {
      load8<T>(p + row * ld + c * 8, pv[i]);
      load8<float>(dp + row * ld + c * 8, gv[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (c * 8 + e >= valid) pv[i][e] = gv[i][e] = 0.f;
        r += pv[i][e] * gv[i][e];
      }
    }
  }
  r = wave_sum(r);
  T* dr = ds + row * ld;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      float o[8], kv[8];
      const bool live = c * 8 < valid;
      if (keep_in_ds && live) load8<T>(dr + c * 8, kv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[e] = live ? scale * pv[i][e] * (gv[i][e] - r) : 0.f;
        if (keep_in_ds && live && kv[e] == 0.f) o[e] = 0.f;
      }
      store8<T>(dr + c * 8, o);
    }
  }
}

// The logit clip's keep mask of scores sc: 1 where |s| <= clip, else 0 (the
// causal mask's and the padding's entries are written as 0 too).
template <typename T, int NV>
__global__ __launch_bounds__(256) void clip_keep_kernel(const float* __restrict__ sc,
                                                        T* __restrict__ keep, int64_t rows, int n,
                                                        int64_t ld, int causal, float clip) {
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int valid = causal ? int(row % n) + 1 : n;
  const int nch = (n + 7) >> 3;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, o[8];
      if (c * 8 < valid) load8<float>(sc + row * ld + c * 8, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (c * 8 + e < valid && fabsf(v[e]) <= clip) ? 1.f : 0.f;
      store8<T>(keep + row * ld + c * 8, o);
    }
  }
}

#define GP_SOFTMAX_DISPATCH(KERNEL, T, ...)                                                    \
  do {                                                                                         \
    const int nch_ = (n + 7) / 8;                                                              \
    dim3 grid_((unsigned)((rows + 3) / 4)), blk_(256);                                         \
    if (nch_ <= 64) hipLaunchKernelGGL((KERNEL<T, 1>), grid_, blk_, 0, s, __VA_ARGS__);        \
    else if (nch_ <= 128) hipLaunchKernelGGL((KERNEL<T, 2>), grid_, blk_, 0, s, __VA_ARGS__);  \
    else if (nch_ <= 256) hipLaunchKernelGGL((KERNEL<T, 4>), grid_, blk_, 0, s, __VA_ARGS__);  \
    else if (nch_ <= 512) hipLaunchKernelGGL((KERNEL<T, 8>), grid_, blk_, 0, s, __VA_ARGS__);  \
    else return hipErrorInvalidValue;                                                          \
  } while (0)

hipError_t softmax_fwd(bool bf16, const float* scores, void* p, int64_t rows, int n, int64_t ld,
                       int causal, float clip, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (bf16) GP_SOFTMAX_DISPATCH(softmax_fwd_kernel, bf16_t, scores, static_cast<bf16_t*>(p), rows, n, ld, causal, clip);
  else GP_SOFTMAX_DISPATCH(softmax_fwd_kernel, float, scores, static_cast<float*>(p), rows, n, ld, causal, clip);
  return hipGetLastError();
}

hipError_t softmax_bwd(bool bf16, const void* p, const float* dp, void* ds, int64_t rows, int n,
                       int64_t ld, int causal, float scale, int keep_in_ds, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (bf16) GP_SOFTMAX_DISPATCH(softmax_bwd_kernel, bf16_t, static_cast<const bf16_t*>(p), dp, static_cast<bf16_t*>(ds), rows, n, ld, causal, scale, keep_in_ds);
  else GP_SOFTMAX_DISPATCH(softmax_bwd_kernel, float, static_cast<const float*>(p), dp, static_cast<float*>(ds), rows, n, ld, causal, scale, keep_in_ds);
  return hipGetLastError();
}

hipError_t clip_keep(bool bf16, const float* scores, void* keep, int64_t rows, int n, int64_t ld,
                     int causal, float clip, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (bf16) GP_SOFTMAX_DISPATCH(clip_keep_kernel, bf16_t, scores, static_cast<bf16_t*>(keep), rows, n, ld, causal, clip);
  else GP_SOFTMAX_DISPATCH(clip_keep_kernel, float, scores, static_cast<float*>(keep), rows, n, ld, causal, clip);
  return hipGetLastError();
}

// ------------------------------------------------------------ w /= d (IEEE division)
__global__ __launch_bounds__(256) void div_scalar_kernel(float* __restrict__ w, int64_t n, float d) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
    w[i] = w[i] / d;
}

hipError_t div_scalar(float* w, int64_t n, float d, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int blocks = int(std::min<int64_t>((n + 255) / 256, 4096));
  hipLaunchKernelGGL(div_scalar_kernel, dim3(blocks), dim3(256), 0, s, w, n, d);
  return hipGetLastError();
}

// ------------------------------------------------------------ output gradient from the cell above
// dy (act, `count` elements, a multiple of 8) -> the backward's residual-stream
// gradient dy_f32 and its act copy dy_act, 8 elements per thread.
template <typename T>
__global__ __launch_bounds__(256) void grad_in_kernel(const T* __restrict__ dy, float* __restrict__ dy_f32,
                                                      T* __restrict__ dy_act, int64_t nch) {
  for (int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x; c < nch; c += int64_t(gridDim.x) * 256) {
    float v[8];
    load8<T>(dy + c * 8, v);
    store8<float>(dy_f32 + c * 8, v);
    store8<T>(dy_act + c * 8, v);
  }
}

hipError_t grad_in(bool bf16, const void* dy, float* dy_f32, void* dy_act, int64_t count, hipStream_t s) {
  const int64_t nch = count / 8;
  if (nch == 0) return hipSuccess;
  const int blocks = int(std::min<int64_t>((nch + 255) / 256, 2048));
  if (bf16)
    hipLaunchKernelGGL(grad_in_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s, static_cast<const bf16_t*>(dy),
                       dy_f32, static_cast<bf16_t*>(dy_act), nch);
  else
    hipLaunchKernelGGL(grad_in_kernel<float>, dim3(blocks), dim3(256), 0, s, static_cast<const float*>(dy),
                       dy_f32, static_cast<float*>(dy_act), nch);
  return hipGetLastError();
}

// ------------------------------------------------------------ MSE
constexpr int kMseBlocks = 256;
int mse_blocks(int64_t count) {
  const int64_t chunks = count / 8;
  return int(chunks < kMseBlocks * 256 ? (chunks + 255) / 256 : kMseBlocks);
}

template <typename T>
__global__ __launch_bounds__(256) void mse_kernel(const T* __restrict__ y, const T* __restrict__ t,
                                                  float* __restrict__ dy_f32, T* __restrict__ dy_act,
                                                  float* __restrict__ part, int64_t nch,
                                                  float inv_denom, float two_inv_denom) {
  __shared__ float red[4];
  float acc = 0.f;
  for (int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x; c < nch; c += int64_t(gridDim.x) * 256) {
    float yv[8], tv[8], o[8];
    load8<T>(y + c * 8, yv);
    load8<T>(t + c * 8, tv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float r = yv[e] - tv[e];
      acc += r * r;
      o[e] = two_inv_denom * r;
    }
    store8<float>(dy_f32 + c * 8, o);
    store8<T>(dy_act + c * 8, o);
  }
  const float tot = block_sum(acc, red);
  if (threadIdx.x == 0) part[blockIdx.x] = tot * inv_denom;
}

hipError_t mse_fwd_bwd(bool bf16, const void* y, const void* t, float* dy_f32, void* dy_act,
                       float* part, int64_t count, float inv_denom, int* nblk, hipStream_t s) {
  *nblk = mse_blocks(count);
  if (count == 0) return hipSuccess;
  const float k = 2.0f * inv_denom;
  if (bf16)
    launch_k(mse_kernel<bf16_t>, dim3(*nblk), dim3(256), 0, s, static_cast<const bf16_t*>(y),
                       static_cast<const bf16_t*>(t), dy_f32, static_cast<bf16_t*>(dy_act), part, count / 8, inv_denom, k);
  else
    launch_k(mse_kernel<float>, dim3(*nblk), dim3(256), 0, s, static_cast<const float*>(y),
                       static_cast<const float*>(t), dy_f32, static_cast<float*>(dy_act), part, count / 8, inv_denom, k);
  return hipGetLastError();
}

// ------------------------------------------------------------ column sums
// A block covers 256 columns x kColRows rows: thread (g, c) sums 8 consecutive
// columns over rows g, g+8, ... of the chunk; the 8 row groups are then added
// in order through LDS.  Columns must be a multiple of 8.
constexpr int kColRows = 32;
int colsum_chunks(int rows) { return (rows + kColRows - 1) / kColRows; }

template <typename T>
__global__ __launch_bounds__(256) void colsum_kernel(const T* __restrict__ x, int64_t ld, int rows,
                                                     int cols, float* __restrict__ part) {
  __shared__ float red[8][257];
  const int cg = threadIdx.x & 31, rg = threadIdx.x >> 5;
  const int c0 = blockIdx.x * 256 + cg * 8;
  const int r0 = blockIdx.y * kColRows, r1 = min(rows, r0 + kColRows);
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c0 < cols) {
    for (int r = r0 + rg; r < r1; r += 8) {
      float v[8];
      load8<T>(x + int64_t(r) * ld + c0, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += v[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][cg * 8 + e] = s[e];
  __syncthreads();
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c < cols) {
    float t = red[0][threadIdx.x];
#pragma unroll
    for (int g = 1; g < 8; ++g) t += red[g][threadIdx.x];
    part[int64_t(blockIdx.y) * cols + c] = t;
  }
}

hipError_t colsum_partial(int xtype, const void* x, int64_t ld, int rows, int cols, float* part,
                          int* nchunk, hipStream_t s) {
  *nchunk = colsum_chunks(rows);
  if (rows == 0 || cols == 0) return hipSuccess;
  dim3 grid((cols + 255) / 256, *nchunk);
  if (xtype == XT_BF16)
    hipLaunchKernelGGL(colsum_kernel<bf16_t>, grid, dim3(256), 0, s, static_cast<const bf16_t*>(x), ld, rows, cols, part);
  else
    hipLaunchKernelGGL(colsum_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(x), ld, rows, cols, part);
  return hipGetLastError();
}

// out[c] (+)= sum_p part[p * stride + c].  CW columns per block, 256/CW
// threads per column each summing every (256/CW)-th part, then a fixed-order
// combination in LDS.
template <int CW>
__device__ __forceinline__ void sum_partials_block(const float* __restrict__ part, int nparts,
                                                   int64_t stride, int cols, float* __restrict__ out,
                                                   int beta, float* __restrict__ acc, int acc_beta) {
  constexpr int G = 256 / CW;
  __shared__ float red[256];
  const int cl = threadIdx.x % CW, pg = threadIdx.x / CW;
  const int c = blockIdx.x * CW + cl;
  float s = 0.f;
  if (c < cols) {
#pragma unroll 8
    for (int p = pg; p < nparts; p += G) s += part[int64_t(p) * stride + c];
  }
  red[threadIdx.x] = s;
  __syncthreads();
  // tree over the G groups of this column, fixed pairing
  for (int h = G / 2; h > 0; h >>= 1) {
    if (pg < h) red[pg * CW + cl] += red[(pg + h) * CW + cl];
    __syncthreads();
  }
  if (pg == 0 && c < cols) {
    out[c] = beta ? out[c] + red[cl] : red[cl];
    if (acc) acc[c] = acc_beta ? acc[c] + red[cl] : red[cl];
  }
}

template <int CW>
__global__ __launch_bounds__(256) void sum_partials_kernel(const float* __restrict__ part, int nparts,
                                                           int64_t stride, int cols,
                                                           float* __restrict__ out, int beta,
                                                           float* __restrict__ acc,
                                                           int acc_beta) {
  sum_partials_block<CW>(part, nparts, stride, cols, out, beta, acc, acc_beta);
}

struct SumJobs {
  SumJob j[kSumJobsMax];
};
// job blockIdx.y, its columns along x (blocks past a job's columns store nothing)
__global__ __launch_bounds__(256) void sum_partials_batch_kernel(SumJobs jobs) {
  const SumJob& jb = jobs.j[blockIdx.y];
  sum_partials_block<32>(jb.part, jb.nparts, jb.stride, jb.cols, jb.out, 0, nullptr, 0);
}

hipError_t sum_partials_batch(const SumJob* jobs, int njobs, hipStream_t s) {
  SumJobs b;
  int n = 0, xmax = 0;
  auto flush = [&]() -> hipError_t {
    if (!n) return hipSuccess;
    hipLaunchKernelGGL(sum_partials_batch_kernel, dim3(xmax, n), dim3(256), 0, s, b);
    n = xmax = 0;
    return hipGetLastError();
  };
  for (int i = 0; i < njobs; ++i) {
    const SumJob& jb = jobs[i];
    if (jb.cols == 0) continue;
    if (jb.cols < 32) {
      const hipError_t e = sum_partials(jb.part, jb.nparts, jb.stride, jb.cols, jb.out, 0, s);
      if (e != hipSuccess) return e;
      continue;
    }
    b.j[n++] = jb;
    xmax = std::max(xmax, (jb.cols + 31) / 32);
    if (n == kSumJobsMax) {
      const hipError_t e = flush();
      if (e != hipSuccess) return e;
    }
  }
  return flush();
}

hipError_t sum_partials(const float* part, int nparts, int64_t stride, int cols, float* out,
                        int beta, hipStream_t s, float* acc, int acc_beta) {
  if (cols == 0) return hipSuccess;
  if (cols >= 32)
    hipLaunchKernelGGL(sum_partials_kernel<32>, dim3((cols + 31) / 32), dim3(256), 0, s, part,
                       nparts, stride, cols, out, beta, acc, acc_beta);
  else
    hipLaunchKernelGGL(sum_partials_kernel<1>, dim3(cols), dim3(256), 0, s, part, nparts, stride,
                       cols, out, beta, acc, acc_beta);
  return hipGetLastError();
}

// ------------------------------------------------------------ RMSProp
__global__ __launch_bounds__(256) void rmsprop_kernel(float* __restrict__ w, const float* __restrict__ g,
                                                      float* __restrict__ ms, bf16_t* __restrict__ wl,
                                                      int64_t n, float lr, float decay, float eps) {
  const float keep = decay, mix = 1.0f - decay;
  const int64_t n4 = n / 4;
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n4; i += stride) {
    float4 wv = reinterpret_cast<float4*>(w)[i];
    const float4 gv = reinterpret_cast<const float4*>(g)[i];
    float4 mv = reinterpret_cast<float4*>(ms)[i];
    mv.x = keep * mv.x + mix * gv.x * gv.x;
    mv.y = keep * mv.y + mix * gv.y * gv.y;
    mv.z = keep * mv.z + mix * gv.z * gv.z;
    mv.w = keep * mv.w + mix * gv.w * gv.w;
    wv.x -= lr * gv.x / (sqrtf(mv.x) + eps);
    wv.y -= lr * gv.y / (sqrtf(mv.y) + eps);
    wv.z -= lr * gv.z / (sqrtf(mv.z) + eps);
    wv.w -= lr * gv.w / (sqrtf(mv.w) + eps);
    reinterpret_cast<float4*>(ms)[i] = mv;
    reinterpret_cast<float4*>(w)[i] = wv;
    if (wl) {
      uint2 o;
      o.x = f2bf2(wv.x, wv.y);
      o.y = f2bf2(wv.z, wv.w);
      reinterpret_cast<uint2*>(wl)[i] = o;
    }
  }
  // tail (n % 4 elements)
  for (int64_t i = n4 * 4 + int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) {
    const float gv = g[i];
    const float mv = keep * ms[i] + mix * gv * gv;
    const float wv = w[i] - lr * gv / (sqrtf(mv) + eps);
    ms[i] = mv;
    w[i] = wv;
    if (wl) wl[i] = f2bf(wv);
  }
}

hipError_t rmsprop(float* w, const float* g, float* ms, void* w_lowp, int64_t n, float lr,
                   float decay, float eps, hipStream_t s, int max_blocks) {
  if (n == 0) return hipSuccess;
  // one thread per group of four parameters: measured on 403 M parameters,
  // 1.58 ms (5.6 TB/s) against 1.91 ms with the grid capped at 8192 blocks
  // (a grid-stride loop); unrolling, the hardware reciprocal and
  // non-temporal accesses did not help
  const int64_t n4 = (n + 3) / 4;
  const int64_t want = (n4 + 255) / 256;
  // (max_blocks > 0: at most that many blocks, each looping over the groups;
  // the same per-element arithmetic)
  const int64_t cap = max_blocks > 0 ? max_blocks : (int64_t(1) << 30);
  const int blocks = int(want < cap ? want : cap);
  hipLaunchKernelGGL(rmsprop_kernel, dim3(blocks), dim3(256), 0, s, w, g, ms,
                     static_cast<bf16_t*>(w_lowp), n, lr, decay, eps);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void to_bf16_kernel(const float* __restrict__ src,
                                                      bf16_t* __restrict__ dst, int64_t n) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) dst[i] = f2bf(src[i]);
}

hipError_t to_bf16(const float* src, void* dst, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  const int blocks = int(want < 256 * 32 ? want : 256 * 32);
  hipLaunchKernelGGL(to_bf16_kernel, dim3(blocks), dim3(256), 0, s, src, static_cast<bf16_t*>(dst), n);
  return hipGetLastError();
}

}  // namespace gp
