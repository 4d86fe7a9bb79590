// Device-side helpers shared by the cell kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gp {

typedef uint16_t bf16_t;  // bf16 storage: the upper half of an IEEE fp32

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN): v_cvt_pk_bf16_f32,
// two values per instruction.
typedef float float2v_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v_t{lo, hi}), bf16x2v_t));
}
__device__ __forceinline__ bf16_t f2bf(float f) { return bf16_t(f2bf2(f, 0.0f) & 0xffffu); }

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f2bf(v); }

// Reductions over the 64 lanes of a wave; every lane gets the same result
// and the combination order is fixed, so the result is reproducible.  Inside
// each row of 16 lanes: DPP steps pairing lanes l ^ 1, l ^ 2, then the
// mirror within 8 and within 16 lanes (after the first two steps a quad holds
// one value, so the mirrors pair whole quads and halves); every pairing adds
// the same two operands on both lanes.  The four row results are then read
// into scalars and combined as (r0 + r1) + (r2 + r3).  No LDS round trips.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// erf(x) by Abramowitz & Stegun, Handbook of Mathematical Functions,
// formula 7.1.26: erf(|x|) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5))))
// exp(-x^2), t = 1 / (1 + p |x|), |error| <= 1.5e-7 -- below the bf16
// rounding of the activations it feeds.  Branch-free (one reciprocal, one
// exponential; the library erff evaluates two branches in a divergent wave,
// ~40 instructions).  *ex2 receives exp(-x^2).
__device__ __forceinline__ float erf_as(float x, float* ex2) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.0f));
  const float e = __builtin_amdgcn_exp2f((ax * ax) * -1.4426950408889634f);
  float p = fmaf(t, 1.061405429f, -1.453152027f);
  p = fmaf(t, p, 1.421413741f);
  p = fmaf(t, p, -0.284496736f);
  p = fmaf(t, p, 0.254829592f);
  *ex2 = e;
  return copysignf(fmaf(-(p * t), e, 1.0f), x);
}

// GeLU, exact form u * Phi(u), and its derivative Phi(u) + u * phi(u), with
// Phi(u) = (1 + erf(u / sqrt 2)) / 2 and phi(u) = exp(-u^2 / 2) / sqrt(2 pi).
__device__ __forceinline__ float gelu_f(float u) {
  float e;
  return 0.5f * u * (1.0f + erf_as(u * 0.70710678118654752f, &e));
}
__device__ __forceinline__ float gelu_grad_f(float u) {
  float e;  // exp(-(u / sqrt 2)^2) = exp(-u^2 / 2)
  const float cdf = 0.5f * (1.0f + erf_as(u * 0.70710678118654752f, &e));
  return cdf + u * (e * 0.39894228040143268f);
}

// ------------------------------------------------------------ 8-element chunks
template <typename T> __device__ __forceinline__ void load8(const T* p, float* v);
template <> __device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <> __device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float* v) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <typename T> __device__ __forceinline__ void store8(T* p, const float* v);
template <> __device__ __forceinline__ void store8<float>(float* p, const float* v) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
template <> __device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float* v) {
  uint4 a;
  a.x = f2bf2(v[0], v[1]);
  a.y = f2bf2(v[2], v[3]);
  a.z = f2bf2(v[4], v[5]);
  a.w = f2bf2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = a;
}

// Sum over the 256 threads of a block, fixed order; every thread gets the result.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

}  // namespace gp
