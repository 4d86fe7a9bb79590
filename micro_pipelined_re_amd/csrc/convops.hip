// Kernels of the convolutional cell with micro-batch BatchNorm (GPipe
// technical review page, "GPipe algorithm in detail / BatchNorm handling":
// each micro-batch normalises with its own statistics; moving averages over
// the mini-batch are kept for evaluation).
//
// Activations are NHWC [B, H, W, C]; a 3x3 convolution (pad 1, stride 1) is
// a GEMM over the im2col matrix [B*H*W, 9*C] (column (kh*3 + kw)*C + c).
// Channels are processed in chunks of 8 (C must be a multiple of 8).  Every
// reduction has a fixed order, so re-materialization is bitwise.
#include "common.hpp"
#include "kernels.hpp"

namespace gp {

// ------------------------------------------------------------ activation storage
// Eight channels c0 .. c0+7 of pixel p of a tensor of C channels, stored as
// SK_F32 (float [P][C]), SK_BF16 ([P][C] bf16) or SK_SPLIT: a pair of bf16
// values per element, hi = bf16(v) in channels 0 .. C-1 and lo = bf16(v - hi)
// in channels C .. 2C-1 of a [P][2C] tensor, v ~ hi + lo to about 2^-17
// relative (v - hi is exact in float32).  A convolution over the [P][2C]
// tensor with the weights repeated over both halves is the convolution of
// hi + lo.
template <int K>
__device__ __forceinline__ void ld8k(const void* base, int64_t p, int C, int c0, float* v) {
  if constexpr (K == SK_F32) {
    load8<float>(static_cast<const float*>(base) + p * C + c0, v);
  } else if constexpr (K == SK_BF16) {
    load8<bf16_t>(static_cast<const bf16_t*>(base) + p * C + c0, v);
  } else {
    const bf16_t* b = static_cast<const bf16_t*>(base) + p * 2 * C + c0;
    float lo[8];
    load8<bf16_t>(b, v);
    load8<bf16_t>(b + C, lo);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] += lo[e];
  }
}

template <int K>
__device__ __forceinline__ void st8k(void* base, int64_t p, int C, int c0, const float* v) {
  if constexpr (K == SK_F32) {
    store8<float>(static_cast<float*>(base) + p * C + c0, v);
  } else if constexpr (K == SK_BF16) {
    store8<bf16_t>(static_cast<bf16_t*>(base) + p * C + c0, v);
  } else {
    bf16_t* b = static_cast<bf16_t*>(base) + p * 2 * C + c0;
    float hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hi[e] = bf2f(f2bf(v[e]));
      lo[e] = v[e] - hi[e];
    }
    store8<bf16_t>(b, hi);
    store8<bf16_t>(b + C, lo);
  }
}

// ------------------------------------------------------------ im2col / col2im
template <typename T, typename I>
__global__ __launch_bounds__(256) void im2col_kernel(const T* __restrict__ x, T* __restrict__ col,
                                                     int B, int H, int W, int C, int ldx) {
  // one 8-element chunk per thread, copied as raw 16-byte words (no
  // conversion); I is the index type (32-bit whenever the count fits)
  constexpr int WORDS = sizeof(T) * 8 / 16;
  const I cc8 = I(C >> 3);
  const I total = I(B) * H * W * 9 * cc8;
  const I i = I(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total) return;
  const I cc = i % cc8;
  const I rest = i / cc8;
  const int tap = int(rest % 9);
  const I p = rest / 9;
  const int w = int(p % W), h = int((p / W) % H);
  const I b = p / (I(W) * H);
  const int hs = h + tap / 3 - 1, ws = w + tap % 3 - 1;
  uint4 v[WORDS];
#pragma unroll
  for (int k = 0; k < WORDS; ++k) v[k] = make_uint4(0, 0, 0, 0);
  if (hs >= 0 && hs < H && ws >= 0 && ws < W) {
    const uint4* src = reinterpret_cast<const uint4*>(x + ((int64_t(b) * H + hs) * W + ws) * ldx + cc * 8);
#pragma unroll
    for (int k = 0; k < WORDS; ++k) v[k] = src[k];
  }
  uint4* dst = reinterpret_cast<uint4*>(col + int64_t(p) * 9 * C + tap * C + cc * 8);
#pragma unroll
  for (int k = 0; k < WORDS; ++k) dst[k] = v[k];
}

hipError_t im2col(bool bf16, const void* x, int ldx, void* col, int B, int H, int W, int C,
                  hipStream_t s) {
  const int64_t total = int64_t(B) * H * W * 9 * (C / 8);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const bool small = total < (int64_t(1) << 31);
#define GP_IM2COL(T, I) hipLaunchKernelGGL((im2col_kernel<T, I>), dim3(unsigned(blocks)), dim3(256), 0, s, \
                                           static_cast<const T*>(x), static_cast<T*>(col), B, H, W, C, ldx)
  if (bf16) {
    if (small) GP_IM2COL(bf16_t, uint32_t);
    else GP_IM2COL(bf16_t, uint64_t);
  } else {
    if (small) GP_IM2COL(float, uint32_t);
    else GP_IM2COL(float, uint64_t);
  }
#undef GP_IM2COL
  return hipGetLastError();
}

// dx[p] = res[p] + sum over the nine taps t of dcol[p - offset(t)][t] (the
// pixels whose tap t reads p), taps in order 0..8.
template <typename T>
__global__ __launch_bounds__(256) void col2im_kernel(const float* __restrict__ dcol,
                                                     const float* res,  // may alias dx_f32
                                                     float* dx_f32,
                                                     T* __restrict__ dx_act, int B, int H, int W,
                                                     int C) {
  const int cc8 = C >> 3;
  const int64_t total = int64_t(B) * H * W * cc8;
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < total; i += stride) {
    const int cc = int(i % cc8);
    const int64_t p = i / cc8;
    const int w = int(p % W), h = int((p / W) % H), b = int(p / (int64_t(W) * H));
    float acc[8];
    if (res) load8<float>(res + p * C + cc * 8, acc);
    else
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int tap = 0; tap < 9; ++tap) {
      const int hs = h - (tap / 3 - 1), ws = w - (tap % 3 - 1);
      if (hs < 0 || hs >= H || ws < 0 || ws >= W) continue;
      float v[8];
      load8<float>(dcol + ((int64_t(b) * H + hs) * W + ws) * 9 * C + tap * C + cc * 8, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += v[e];
    }
    store8<float>(dx_f32 + p * C + cc * 8, acc);
    if (dx_act) store8<T>(dx_act + p * C + cc * 8, acc);
  }
}

hipError_t col2im(bool bf16, const float* dcol, const float* res, float* dx_f32, void* dx_act,
                  int B, int H, int W, int C, hipStream_t s) {
  const int64_t total = int64_t(B) * H * W * (C / 8);
  if (total == 0) return hipSuccess;
  const int64_t want = (total + 255) / 256;
  const int blocks = int(want < 16384 ? want : 16384);
  if (bf16)
    hipLaunchKernelGGL(col2im_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s, dcol, res, dx_f32,
                       static_cast<bf16_t*>(dx_act), B, H, W, C);
  else
    hipLaunchKernelGGL(col2im_kernel<float>, dim3(blocks), dim3(256), 0, s, dcol, res, dx_f32,
                       static_cast<float*>(dx_act), B, H, W, C);
  return hipGetLastError();
}

// ------------------------------------------------------------ BatchNorm statistics
// One pass over the input.  A block covers 256 channels x kBnRows rows (a
// chunk); thread (rg, cg) holds rows rg, rg+8, ... of the chunk for channels
// cg*8 .. cg*8+7 in registers.  Per chunk it writes the channel sums and the
// sums of squared deviations from the chunk's own mean (M2); the finalize
// merges the chunks with the exact pairwise formula
//   mean = sum_k S_k / n,   M2 = sum_k (M2_k + n_k (S_k/n_k - mean)^2),
// in a fixed order, so the result is reproducible bit for bit.
constexpr int kBnRows = 32;
constexpr int kBnRowsPerThread = kBnRows / 8;
int bn_chunks(int64_t rows) { return int((rows + kBnRows - 1) / kBnRows); }

template <typename T>
__global__ __launch_bounds__(256) void bn_moments_kernel(const T* __restrict__ x,
                                                         float* __restrict__ part, int64_t rows,
                                                         int C) {
  __shared__ float red[8][257];
  __shared__ float mean_k[256];
  const int cg = threadIdx.x & 31, rg = threadIdx.x >> 5;
  const int c0 = blockIdx.x * 256 + cg * 8;
  const int64_t r0 = int64_t(blockIdx.y) * kBnRows;
  const int nk = int(r0 + kBnRows < rows ? kBnRows : rows - r0);
  float v[kBnRowsPerThread][8];
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const bool cok = c0 < C;
#pragma unroll
  for (int i = 0; i < kBnRowsPerThread; ++i) {
    const int r = rg + 8 * i;
    if (cok && r < nk) {
      load8<T>(x + (r0 + r) * C + c0, v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += v[i][e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][cg * 8 + e] = s[e];
  __syncthreads();
  const int c = blockIdx.x * 256 + threadIdx.x;
  float sum = red[0][threadIdx.x];
#pragma unroll
  for (int g = 1; g < 8; ++g) sum += red[g][threadIdx.x];
  mean_k[threadIdx.x] = sum / float(nk);
  __syncthreads();
  float q[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kBnRowsPerThread; ++i) {
    const int r = rg + 8 * i;
    if (cok && r < nk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[i][e] - mean_k[cg * 8 + e];
        q[e] += d * d;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][cg * 8 + e] = q[e];
  __syncthreads();
  if (c < C) {
    float m2 = red[0][threadIdx.x];
#pragma unroll
    for (int g = 1; g < 8; ++g) m2 += red[g][threadIdx.x];
    part[int64_t(blockIdx.y) * 2 * C + c] = sum;
    part[int64_t(blockIdx.y) * 2 * C + C + c] = m2;
  }
}

// Block: 2 channels x 128 chunk groups; each group adds every 128th chunk,
// the groups are then combined by a fixed tree.  stats = (mean, rstd); rec
// (optional) = (mean, biased variance).  (With 8 channels x 32 groups a
// 256-channel merge ran on 32 workgroups: 10.4 us for 512 chunks.)
constexpr int kMergeCh = 2, kMergeGroups = 128;

__device__ __forceinline__ float merge_tree(float v, float (*red)[kMergeCh + 1], int g, int cl) {
  red[g][cl] = v;
  __syncthreads();
#pragma unroll
  for (int h = kMergeGroups / 2; h > 0; h >>= 1) {
    if (g < h) red[g][cl] += red[g + h][cl];
    __syncthreads();
  }
  const float t = red[0][cl];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(256) void bn_merge_kernel(const float* __restrict__ part, int nchunk,
                                                       int64_t rows, int C, float eps,
                                                       float* __restrict__ stats,
                                                       float* __restrict__ rec) {
  __shared__ float red[kMergeGroups][kMergeCh + 1];
  const int cl = threadIdx.x % kMergeCh, g = threadIdx.x / kMergeCh;
  const int c = blockIdx.x * kMergeCh + cl;
  const bool ok = c < C;
  float s = 0.f;
  if (ok) {
#pragma unroll 8
    for (int k = g; k < nchunk; k += kMergeGroups) s += part[int64_t(k) * 2 * C + c];
  }
  const float mean = merge_tree(s, red, g, cl) / float(rows);
  float m2 = 0.f;
  if (ok) {
#pragma unroll 8
    for (int k = g; k < nchunk; k += kMergeGroups) {
      const float nk = float(int64_t(k) * kBnRows + kBnRows <= rows ? kBnRows
                                                                    : rows - int64_t(k) * kBnRows);
      const float d = part[int64_t(k) * 2 * C + c] / nk - mean;
      m2 += part[int64_t(k) * 2 * C + C + c] + nk * d * d;
    }
  }
  const float var = merge_tree(m2, red, g, cl) / float(rows);
  if (g == 0 && ok) {
    stats[c] = mean;
    stats[C + c] = 1.0f / sqrtf(var + eps);
    if (rec) {
      rec[c] = mean;
      rec[C + c] = var;
    }
  }
}

// stats: [2][C] = (mean, rstd).  rec (optional): [2][C] = (mean, biased var).
// part: [bn_chunks(rows)][2C] scratch.
hipError_t bn_stats(bool bf16, const void* x, int64_t rows, int C, float eps, float* part,
                    float* stats, float* rec, hipStream_t s) {
  if (rows == 0 || C == 0) return hipSuccess;
  const int nch = bn_chunks(rows);
  const dim3 grid((C + 255) / 256, nch);
  if (bf16)
    hipLaunchKernelGGL(bn_moments_kernel<bf16_t>, grid, dim3(256), 0, s,
                       static_cast<const bf16_t*>(x), part, rows, C);
  else
    hipLaunchKernelGGL(bn_moments_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(x), part, rows, C);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bn_merge_kernel, dim3((C + kMergeCh - 1) / kMergeCh), dim3(256), 0, s, part, nch,
                     rows, C, eps, stats, rec);
  return hipGetLastError();
}

// ------------------------------------------------------------ BatchNorm apply
// y = gamma * (a - mean) * rstd + beta from the float32 input a;  MODE 0:
// out = max(y, 0);  MODE 1: out = res + y.  res and out are stored as KR / KO
// (they may be the same tensor: each thread reads its elements of res before
// it writes them).
template <int MODE, int KR, int KO>
__global__ __launch_bounds__(256) void bn_apply_kernel(const float* __restrict__ a,
                                                       const float* __restrict__ stats,
                                                       const float* __restrict__ gamma,
                                                       const float* __restrict__ beta,
                                                       const void* res, void* out, int64_t rows,
                                                       int C) {
  const int cc8 = C >> 3;
  const int64_t total = rows * cc8;
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < total; i += stride) {
    const int c0 = int(i % cc8) * 8;
    const int64_t p = i / cc8;
    float v[8], o[8], rv[8];
    load8<float>(a + p * C + c0, v);
    if constexpr (MODE == 1) ld8k<KR>(res, p, C, c0, rv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = c0 + e;
      const float y = gamma[c] * (v[e] - stats[c]) * stats[C + c] + beta[c];
      o[e] = MODE == 0 ? fmaxf(y, 0.f) : rv[e] + y;
    }
    st8k<KO>(out, p, C, c0, o);
  }
}

hipError_t bn_apply(int mode, const float* a, const float* stats, const float* gamma,
                    const float* beta, const void* res, int res_kind, void* out, int out_kind,
                    int64_t rows, int C, hipStream_t s) {
  const int64_t total = rows * (C / 8);
  if (total == 0) return hipSuccess;
  const int64_t want = (total + 255) / 256;
  const int blocks = int(want < 16384 ? want : 16384);
#define GP_BN_APPLY(M, KR, KO)                                                                 \
  hipLaunchKernelGGL((bn_apply_kernel<M, KR, KO>), dim3(blocks), dim3(256), 0, s, a, stats,   \
                     gamma, beta, res, out, rows, C)
  if (mode == 0) {
    if (out_kind == SK_F32) GP_BN_APPLY(0, SK_F32, SK_F32);
    else if (out_kind == SK_SPLIT) GP_BN_APPLY(0, SK_F32, SK_SPLIT);
    else return hipErrorInvalidValue;
  } else {
    if (res_kind == SK_F32 && out_kind == SK_F32) GP_BN_APPLY(1, SK_F32, SK_F32);
    else if (res_kind == SK_BF16 && out_kind == SK_SPLIT) GP_BN_APPLY(1, SK_BF16, SK_SPLIT);
    else if (res_kind == SK_SPLIT && out_kind == SK_SPLIT) GP_BN_APPLY(1, SK_SPLIT, SK_SPLIT);
    else if (res_kind == SK_SPLIT && out_kind == SK_BF16) GP_BN_APPLY(1, SK_SPLIT, SK_BF16);
    else if (res_kind == SK_BF16 && out_kind == SK_BF16) GP_BN_APPLY(1, SK_BF16, SK_BF16);
    else return hipErrorInvalidValue;
  }
#undef GP_BN_APPLY
  return hipGetLastError();
}

// ------------------------------------------------------------ BatchNorm backward
// dy = dy_src (MASK: times [r > 0], r the ReLU output stored as KR; of a split
// r the hi half decides), xhat = (a - mean) * rstd with a float32.
// part[chunk][0:C] = sum dy*xhat, part[chunk][C:2C] = sum dy (gamma, beta order).
template <int KR>
__device__ __forceinline__ void relu_mask8(const void* r, int64_t row, int C, int c0, float* g) {
  float rv[8];
  ld8k<KR == SK_SPLIT ? SK_BF16 : KR>(r, row * (KR == SK_SPLIT ? 2 : 1), C, c0, rv);
#pragma unroll
  for (int e = 0; e < 8; ++e) g[e] = rv[e] > 0.f ? g[e] : 0.f;
}

template <int KR, int MASK>
__global__ __launch_bounds__(256) void bn_bwd_partial_kernel(const float* __restrict__ dy_src,
                                                             const void* __restrict__ r,
                                                             const float* __restrict__ a,
                                                             const float* __restrict__ stats,
                                                             float* __restrict__ part,
                                                             int64_t rows, int C) {
  __shared__ float red[2][8][257];
  const int cg = threadIdx.x & 31, rg = threadIdx.x >> 5;
  const int c0 = blockIdx.x * 256 + cg * 8;
  const int64_t r0 = int64_t(blockIdx.y) * kBnRows;
  const int64_t r1 = r0 + kBnRows < rows ? r0 + kBnRows : rows;
  float sg[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, sb[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c0 < C) {
    float mu[8], rs[8];
    load8<float>(stats + c0, mu);
    load8<float>(stats + C + c0, rs);
    for (int64_t row = r0 + rg; row < r1; row += 8) {
      float g[8], av[8];
      load8<float>(dy_src + row * C + c0, g);
      load8<float>(a + row * C + c0, av);
      if (MASK) relu_mask8<KR>(r, row, C, c0, g);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sg[e] += g[e] * (av[e] - mu[e]) * rs[e];
        sb[e] += g[e];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[0][rg][cg * 8 + e] = sg[e];
    red[1][rg][cg * 8 + e] = sb[e];
  }
  __syncthreads();
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c < C) {
    float tg = red[0][0][threadIdx.x], tb = red[1][0][threadIdx.x];
#pragma unroll
    for (int g = 1; g < 8; ++g) {
      tg += red[0][g][threadIdx.x];
      tb += red[1][g][threadIdx.x];
    }
    part[int64_t(blockIdx.y) * 2 * C + c] = tg;
    part[int64_t(blockIdx.y) * 2 * C + C + c] = tb;
  }
}

// da (stored as KD) = gamma * rstd * (dy - sum(dy)/n - xhat * sum(dy*xhat)/n);
// sums = [2][C] as in the partials.
template <int KD, int KR, int MASK>
__global__ __launch_bounds__(256) void bn_bwd_apply_kernel(const float* __restrict__ dy_src,
                                                           const void* __restrict__ r,
                                                           const float* __restrict__ a,
                                                           const float* __restrict__ stats,
                                                           const float* __restrict__ gamma,
                                                           const float* __restrict__ sums,
                                                           void* __restrict__ da, int64_t rows,
                                                           int C, float inv_n) {
  const int cc8 = C >> 3;
  const int64_t total = rows * cc8;
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < total; i += stride) {
    const int c0 = int(i % cc8) * 8;
    const int64_t row = i / cc8;
    const int64_t off = row * C + c0;
    float g[8], av[8], o[8];
    load8<float>(dy_src + off, g);
    load8<float>(a + off, av);
    if (MASK) relu_mask8<KR>(r, row, C, c0, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = c0 + e;
      const float rs = stats[C + c];
      const float xh = (av[e] - stats[c]) * rs;
      o[e] = gamma[c] * rs * (g[e] - sums[C + c] * inv_n - xh * sums[c] * inv_n);
    }
    st8k<KD>(da, row, C, c0, o);
  }
}

hipError_t bn_bwd(int da_kind, int mask, const float* dy_src, const void* r, int r_kind,
                  const float* a, const float* stats, const float* gamma, float* part, float* sums,
                  float* grad, int grad_beta, void* da, int64_t rows, int C, int* nchunk,
                  hipStream_t s) {
  *nchunk = bn_chunks(rows);
  if (rows == 0 || C == 0) return hipSuccess;
  if ((da_kind != SK_F32 && da_kind != SK_BF16) || (mask && r_kind != SK_F32 && r_kind != SK_SPLIT))
    return hipErrorInvalidValue;
  dim3 grid((C + 255) / 256, *nchunk);
#define GP_BN_BWD_P(KR, MK)                                                                   \
  hipLaunchKernelGGL((bn_bwd_partial_kernel<KR, MK>), grid, dim3(256), 0, s, dy_src, r, a,   \
                     stats, part, rows, C)
  if (!mask) GP_BN_BWD_P(SK_F32, 0);
  else if (r_kind == SK_F32) GP_BN_BWD_P(SK_F32, 1);
  else GP_BN_BWD_P(SK_SPLIT, 1);
#undef GP_BN_BWD_P
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = sum_partials(part, *nchunk, 2 * C, 2 * C, sums, 0, s, grad, grad_beta);
  if (e != hipSuccess) return e;
  const int64_t total = rows * (C / 8);
  const int64_t want = (total + 255) / 256;
  const int blocks = int(want < 16384 ? want : 16384);
  const float inv_n = float(1.0 / double(rows));
#define GP_BN_BWD_A(KD, KR, MK)                                                              \
  launch_k((bn_bwd_apply_kernel<KD, KR, MK>), dim3(blocks), dim3(256), 0, s, dy_src, r, a,    \
           stats, gamma, sums, da, rows, C, inv_n)
  if (da_kind == SK_F32) {
    if (!mask) GP_BN_BWD_A(SK_F32, SK_F32, 0);
    else if (r_kind == SK_F32) GP_BN_BWD_A(SK_F32, SK_F32, 1);
    else GP_BN_BWD_A(SK_F32, SK_SPLIT, 1);
  } else {
    if (!mask) GP_BN_BWD_A(SK_BF16, SK_F32, 0);
    else if (r_kind == SK_F32) GP_BN_BWD_A(SK_BF16, SK_F32, 1);
    else GP_BN_BWD_A(SK_BF16, SK_SPLIT, 1);
  }
#undef GP_BN_BWD_A
  return hipGetLastError();
}

// ------------------------------------------------------------ flipped weights
// dst[c][t][o] = src[o][8 - t][c]: the input gradient of y = conv3x3(x, W) is
// conv3x3(dy, dst) (the taps mirrored through the centre, in and out swapped).
__global__ __launch_bounds__(256) void conv_flip_kernel(const bf16_t* __restrict__ src,
                                                        bf16_t* __restrict__ dst, int C) {
  const int64_t n = int64_t(9) * C * C;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const int o = int(i % C);
    const int t = int((i / C) % 9);
    const int c = int(i / (int64_t(9) * C));
    dst[i] = src[(int64_t(o) * 9 + (8 - t)) * C + c];
  }
}

hipError_t conv_flip_weights(const void* src, void* dst, int C, hipStream_t s) {
  const int64_t n = int64_t(9) * C * C;
  if (n == 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  const int blocks = int(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(conv_flip_kernel, dim3(blocks), dim3(256), 0, s,
                     static_cast<const bf16_t*>(src), static_cast<bf16_t*>(dst), C);
  return hipGetLastError();
}

// ------------------------------------------------------------ repeated weights
// dst[o][t][c'] = src[o][t][c' mod C], c' < 2C: the weights of a convolution
// over a split [P][2C] tensor (its hi and lo halves meet the same weights).
__global__ __launch_bounds__(256) void conv_dup_kernel(const bf16_t* __restrict__ src,
                                                       bf16_t* __restrict__ dst, int C) {
  const int64_t n = int64_t(9) * C * C;  // in 8-element chunks of the source: n / 8
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n / 8; i += int64_t(gridDim.x) * 256) {
    const int64_t e = i * 8;
    const int64_t ot = e / C;  // o * 9 + t
    const int c = int(e - ot * C);
    const uint4 v = *reinterpret_cast<const uint4*>(src + e);
    bf16_t* d = dst + ot * 2 * C + c;
    *reinterpret_cast<uint4*>(d) = v;
    *reinterpret_cast<uint4*>(d + C) = v;
  }
}

hipError_t conv_dup_weights(const void* src, void* dst, int C, hipStream_t s) {
  const int64_t n = int64_t(9) * C * C / 8;
  if (n == 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  const int blocks = int(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(conv_dup_kernel, dim3(blocks), dim3(256), 0, s,
                     static_cast<const bf16_t*>(src), static_cast<bf16_t*>(dst), C);
  return hipGetLastError();
}

// ------------------------------------------------------------ moving averages
// rec: [M][nbn][2][C] = per micro-batch (mean, biased var); running: [nbn][2][C].
// Pooled over the M equal micro-batches in order:
//   mu = mean_m mu_m,  var = mean_m(var_m + mu_m^2) - mu^2,  unbiased * n/(n-1).
__global__ __launch_bounds__(256) void bn_running_kernel(const float* __restrict__ rec, int M,
                                                         int nbn, int C, float n_total,
                                                         float momentum,
                                                         float* __restrict__ running) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= nbn * C) return;
  const int j = i / C, c = i % C;
  double mu = 0.0, sq = 0.0;
  for (int m = 0; m < M; ++m) {
    const float* r = rec + (int64_t(m) * nbn + j) * 2 * C;
    mu += r[c];
    sq += double(r[C + c]) + double(r[c]) * double(r[c]);
  }
  mu /= M;
  const double var = sq / M - mu * mu;
  const double unbiased = n_total > 1.f ? var * n_total / (n_total - 1.0) : var;
  float* run = running + int64_t(j) * 2 * C;
  run[c] = float(momentum * run[c] + (1.0 - momentum) * mu);
  run[C + c] = float(momentum * run[C + c] + (1.0 - momentum) * unbiased);
}

hipError_t bn_running(const float* rec, int M, int nbn, int C, int64_t n_total, float momentum,
                      float* running, hipStream_t s) {
  if (nbn * C == 0) return hipSuccess;
  hipLaunchKernelGGL(bn_running_kernel, dim3((nbn * C + 255) / 256), dim3(256), 0, s, rec, M, nbn,
                     C, float(n_total), momentum, running);
  return hipGetLastError();
}

}  // namespace gp
