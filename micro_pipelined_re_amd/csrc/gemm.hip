// LDS-staged MFMA GEMM for the cell's contractions (gfx950).
//
//   C[z] (M x N) = epilogue( sum_k A[z](m, k) * B[z](k, n) )
//
// Operand layouts in global memory:
//   A: LAY_K  -> A(m, k) = A[m * lda + k]   (k contiguous)
//      LAY_MN -> A(m, k) = A[k * lda + m]   (m contiguous)
//   B: LAY_K  -> B(k, n) = B[n * ldb + k]   (k contiguous)
//      LAY_MN -> B(k, n) = B[k * ldb + n]   (n contiguous)
// Forward linears are (A=K, B=K), input-gradient products (A=K, B=MN) and
// weight-gradient products, which reduce over tokens, (A=MN, B=MN).
//
// Both tiles are written to LDS k-contiguous (an m-contiguous operand is
// transposed in registers on its way in), so every MFMA fragment is one
// 16-byte LDS read.  Two LDS buffers: tile k+1 is fetched from HBM into
// registers while tile k is multiplied, one barrier per k-tile.
//
// bf16: v_mfma_f32_16x16x32_bf16, fp32 accumulate.  fp32: v_mfma_f32_16x16x4_f32.
// A lane feeds an MFMA with elements at k = 8*(lane/16)+e (bf16) or, over four
// consecutive instructions, k = 4*(lane/16)+s (fp32); A and B use the same
// lane->k assignment, which is all the contraction needs.
// Accumulator layout (16x16 block): lane l holds column l%16, rows 4*(l/16)+v.
#include "../../include/gpipe.h"
#include "common.hpp"
#include "kernels.hpp"

namespace gp {

template <typename T> struct Tile;
template <> struct Tile<bf16_t> {
  static constexpr int BM = 128, BN = 128, BK = 32, WM = 2, WN = 2;
  static constexpr int VEC = 8;   // elements per 16-byte vector
  static constexpr int PAD = 8;   // LDS row padding (elements)
};
template <> struct Tile<float> {
  static constexpr int BM = 64, BN = 64, BK = 16, WM = 2, WN = 2;
  static constexpr int VEC = 4;
  static constexpr int PAD = 4;
};

constexpr int kThreads = 256;

template <typename T> __device__ __forceinline__ T elem_of(const uint4& v, int e);
template <> __device__ __forceinline__ bf16_t elem_of<bf16_t>(const uint4& v, int e) {
  const uint32_t w = (e < 2) ? v.x : (e < 4) ? v.y : (e < 6) ? v.z : v.w;
  return bf16_t((e & 1) ? (w >> 16) : (w & 0xffffu));
}
template <> __device__ __forceinline__ float elem_of<float>(const uint4& v, int e) {
  const uint32_t w = (e == 0) ? v.x : (e == 1) ? v.y : (e == 2) ? v.z : v.w;
  return __uint_as_float(w);
}

template <typename T> __device__ __forceinline__ void set_elem(uint4& v, int e, T x);
template <> __device__ __forceinline__ void set_elem<bf16_t>(uint4& v, int e, bf16_t x) {
  uint32_t* w = reinterpret_cast<uint32_t*>(&v) + (e >> 1);
  *w = (e & 1) ? ((*w & 0xffffu) | (uint32_t(x) << 16)) : ((*w & 0xffff0000u) | x);
}
template <> __device__ __forceinline__ void set_elem<float>(uint4& v, int e, float x) {
  reinterpret_cast<uint32_t*>(&v)[e] = __float_as_uint(x);
}

// Loads one [ROWS x BK] tile of an operand into registers and stores it to LDS
// as s[row][k] (row pitch BK + PAD).  rows_total / kend bound the valid region;
// everything outside is zero.
template <typename T, int LAY, int ROWS>
struct TileLoader {
  using Tl = Tile<T>;
  static constexpr int BK = Tl::BK, VEC = Tl::VEC, LDP = Tl::BK + Tl::PAD;
  // k-contiguous: chunks of VEC consecutive k in one row
  static constexpr int CPR = BK / VEC;
  static constexpr int NCH = ROWS * CPR;
  // m-contiguous: blocks of KB consecutive k times VEC consecutive rows
  static constexpr int KB = 4;
  static constexpr int NBLK = (BK / KB) * (ROWS / VEC);
  static constexpr int PER = (LAY == LAY_K) ? (NCH + kThreads - 1) / kThreads
                                            : (NBLK + kThreads - 1) / kThreads;
  static constexpr int NV = (LAY == LAY_K) ? 1 : KB;
  uint4 v[PER][NV];

  __device__ __forceinline__ void load(const T* __restrict__ p, int64_t ld, int row0,
                                       int rows_total, int k0, int kend, int tid) {
    if constexpr (LAY == LAY_K) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int c = tid + i * kThreads;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (c < NCH) {
          const int r = c / CPR, kc = (c % CPR) * VEC;
          const int gr = row0 + r, gk = k0 + kc;
          if (gr < rows_total && gk < kend) {
            const T* src = p + int64_t(gr) * ld + gk;
            if (gk + VEC <= kend) {
              x = *reinterpret_cast<const uint4*>(src);
            } else {
              for (int e = 0; e < VEC; ++e)
                if (gk + e < kend) set_elem<T>(x, e, src[e]);
            }
          }
        }
        v[i][0] = x;
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int b = tid + i * kThreads;
        const int kq = b / (ROWS / VEC), mc = b % (ROWS / VEC);
        const int gm = row0 + mc * VEC;
#pragma unroll
        for (int r = 0; r < KB; ++r) {
          uint4 x = make_uint4(0, 0, 0, 0);
          const int gk = k0 + kq * KB + r;
          if (b < NBLK && gk < kend && gm < rows_total) {
            const T* src = p + int64_t(gk) * ld + gm;
            if (gm + VEC <= rows_total) {
              x = *reinterpret_cast<const uint4*>(src);
            } else {
              for (int e = 0; e < VEC; ++e)
                if (gm + e < rows_total) set_elem<T>(x, e, src[e]);
            }
          }
          v[i][r] = x;
        }
      }
    }
  }

  __device__ __forceinline__ void store(T* s, int tid) const {
    if constexpr (LAY == LAY_K) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int c = tid + i * kThreads;
        if (c < NCH) {
          const int r = c / CPR, kc = (c % CPR) * VEC;
          *reinterpret_cast<uint4*>(s + r * LDP + kc) = v[i][0];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int b = tid + i * kThreads;
        if (b < NBLK) {
          const int kq = b / (ROWS / VEC), mc = b % (ROWS / VEC);
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            T* dst = s + (mc * VEC + e) * LDP + kq * KB;
            if constexpr (sizeof(T) == 2) {
              uint2 w;
              w.x = uint32_t(elem_of<T>(v[i][0], e)) | (uint32_t(elem_of<T>(v[i][1], e)) << 16);
              w.y = uint32_t(elem_of<T>(v[i][2], e)) | (uint32_t(elem_of<T>(v[i][3], e)) << 16);
              *reinterpret_cast<uint2*>(dst) = w;
            } else {
              uint4 w;
              w.x = __float_as_uint(elem_of<T>(v[i][0], e));
              w.y = __float_as_uint(elem_of<T>(v[i][1], e));
              w.z = __float_as_uint(elem_of<T>(v[i][2], e));
              w.w = __float_as_uint(elem_of<T>(v[i][3], e));
              *reinterpret_cast<uint4*>(dst) = w;
            }
          }
        }
      }
    }
  }
};

// ROLE only names the instance (one kernel symbol per role of the step).
template <typename T, int LA, int LB, int EPI, int ROLE>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmParams g) {
  using Tl = Tile<T>;
  constexpr int BM = Tl::BM, BN = Tl::BN, BK = Tl::BK, LDP = Tl::BK + Tl::PAD;
  constexpr int WTM = BM / Tl::WM, WTN = BN / Tl::WN;  // wave tile
  constexpr int FM = WTM / 16, FN = WTN / 16;           // 16x16 blocks per wave
  __shared__ __attribute__((aligned(16))) T As[2][BM * LDP];
  __shared__ __attribute__((aligned(16))) T Bs[2][BN * LDP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles_n = (g.N + BN - 1) / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int z = blockIdx.z, zb = z / g.hdiv, zh = z % g.hdiv;

  // causal structure of the attention products (see kernels.hpp)
  if (g.causal == CAUSAL_SKIP_UPPER && n0 > m0 + BM - 1) return;
  int kbeg = 0, kend = g.K;
  if (g.causal == CAUSAL_K_UPTO_M) kend = min(g.K, m0 + BM);
  if (g.causal == CAUSAL_K_FROM_M) kbeg = (m0 / BK) * BK;

  const T* A = static_cast<const T*>(g.A) + zb * g.sAb + zh * g.sAh;
  const T* B = static_cast<const T*>(g.B) + zb * g.sBb + zh * g.sBh;

  TileLoader<T, LA, BM> la;
  TileLoader<T, LB, BN> lb;
  floatx4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int wm0 = (wave / Tl::WN) * WTM, wn0 = (wave % Tl::WN) * WTN;
  const int nkt = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

  if (nkt > 0) {
    la.load(A, g.lda, m0, g.M, kbeg, kend, tid);
    lb.load(B, g.ldb, n0, g.N, kbeg, kend, tid);
    la.store(As[0], tid);
    lb.store(Bs[0], tid);
  }
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nkt) {
      la.load(A, g.lda, m0, g.M, kbeg + (kt + 1) * BK, kend, tid);
      lb.load(B, g.ldb, n0, g.N, kbeg + (kt + 1) * BK, kend, tid);
    }
    const T* as = As[cur];
    const T* bs = Bs[cur];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int ks = 0; ks < BK; ks += 32) {
        bf16x8_t af[FM], bfr[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[i] = *reinterpret_cast<const bf16x8_t*>(as + (wm0 + i * 16 + (lane & 15)) * LDP + ks + (lane >> 4) * 8);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8_t*>(bs + (wn0 + j * 16 + (lane & 15)) * LDP + ks + (lane >> 4) * 8);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < BK; ks += 16) {
        floatx4_t af[FM], bfr[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[i] = *reinterpret_cast<const floatx4_t*>(as + (wm0 + i * 16 + (lane & 15)) * LDP + ks + (lane >> 4) * 4);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfr[j] = *reinterpret_cast<const floatx4_t*>(bs + (wn0 + j * 16 + (lane & 15)) * LDP + ks + (lane >> 4) * 4);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][s], bfr[j][s], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < nkt) {
      la.store(As[cur ^ 1], tid);
      lb.store(Bs[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // epilogue
  const int64_t coff = zb * g.sCb + zh * g.sCh;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn0 + j * 16 + (lane & 15);
      if (col >= g.N) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + wm0 + i * 16 + (lane >> 4) * 4 + v;
        if (row >= g.M) continue;
        const float a = acc[i][j][v];
        const int64_t ci = coff + int64_t(row) * g.ldc + col;
        if constexpr (EPI == EPI_STORE) {
          static_cast<T*>(g.C)[ci] = from_f<T>(g.alpha * a);
        } else if constexpr (EPI == EPI_BIAS) {
          static_cast<T*>(g.C)[ci] = from_f<T>(a + g.bias[col]);
        } else if constexpr (EPI == EPI_BIAS_RESID) {
          const float r = to_f<T>(static_cast<const T*>(g.R)[int64_t(row) * g.ldr + col]);
          static_cast<T*>(g.C)[ci] = from_f<T>(a + g.bias[col] + r);
        } else if constexpr (EPI == EPI_BIAS_GELU) {
          const float u = a + g.bias[col];
          static_cast<T*>(g.U)[int64_t(row) * g.ldu + col] = from_f<T>(u);
          static_cast<T*>(g.C)[ci] = from_f<T>(gelu_f(u));
        } else if constexpr (EPI == EPI_GELU_BWD) {
          const float u = to_f<T>(static_cast<const T*>(g.U)[int64_t(row) * g.ldu + col]);
          static_cast<T*>(g.C)[ci] = from_f<T>(a * gelu_grad_f(u));
        } else if constexpr (EPI == EPI_STORE_F32) {
          static_cast<float*>(g.C)[ci] = g.alpha * a;
        } else if constexpr (EPI == EPI_ACC_F32) {
          float* c = static_cast<float*>(g.C) + ci;
          *c = g.beta ? (*c + a) : a;
        }
      }
    }
  }
}

template <typename T, int LA, int LB, int EPI, int ROLE>
static hipError_t launch(const GemmParams& g, int batch, hipStream_t s) {
  using Tl = Tile<T>;
  const int tiles = ((g.M + Tl::BM - 1) / Tl::BM) * ((g.N + Tl::BN - 1) / Tl::BN);
  if (tiles == 0 || batch == 0) return hipSuccess;
  dim3 grid(tiles, 1, batch);
  hipLaunchKernelGGL((gemm_kernel<T, LA, LB, EPI, ROLE>), grid, dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

// Operand layouts and epilogue of every GEMM role of the step.
//   forward linears          C = A W^T (+ epilogue)          A: K, B: K
//   input-gradient products  dA = dC W                      A: K, B: MN
//   weight gradients         G (+)= dC^T A  (over tokens)    A: MN, B: MN
template <typename T>
static hipError_t dispatch(int role, const GemmParams& g, int batch, hipStream_t s) {
#define GP_ROLE(R, LA_, LB_, EPI_) \
  case R: return launch<T, LA_, LB_, EPI_, R>(g, batch, s);
  switch (role) {
    GP_ROLE(GPIPE_ROLE_QKV_FWD, LAY_K, LAY_K, EPI_BIAS)
    GP_ROLE(GPIPE_ROLE_SCORES_FWD, LAY_K, LAY_K, EPI_STORE_F32)
    GP_ROLE(GPIPE_ROLE_PV_FWD, LAY_K, LAY_MN, EPI_STORE)
    GP_ROLE(GPIPE_ROLE_OUT_FWD, LAY_K, LAY_K, EPI_BIAS_RESID)
    GP_ROLE(GPIPE_ROLE_FFN1_FWD, LAY_K, LAY_K, EPI_BIAS_GELU)
    GP_ROLE(GPIPE_ROLE_FFN2_FWD, LAY_K, LAY_K, EPI_BIAS_RESID)
    GP_ROLE(GPIPE_ROLE_FFN2_DGRAD, LAY_K, LAY_MN, EPI_GELU_BWD)
    GP_ROLE(GPIPE_ROLE_FFN2_WGRAD, LAY_MN, LAY_MN, EPI_ACC_F32)
    GP_ROLE(GPIPE_ROLE_FFN1_DGRAD, LAY_K, LAY_MN, EPI_STORE_F32)
    GP_ROLE(GPIPE_ROLE_FFN1_WGRAD, LAY_MN, LAY_MN, EPI_ACC_F32)
    GP_ROLE(GPIPE_ROLE_OUT_DGRAD, LAY_K, LAY_MN, EPI_STORE)
    GP_ROLE(GPIPE_ROLE_OUT_WGRAD, LAY_MN, LAY_MN, EPI_ACC_F32)
    GP_ROLE(GPIPE_ROLE_DP, LAY_K, LAY_K, EPI_STORE_F32)
    GP_ROLE(GPIPE_ROLE_DV, LAY_MN, LAY_MN, EPI_STORE)
    GP_ROLE(GPIPE_ROLE_DQ, LAY_K, LAY_MN, EPI_STORE)
    GP_ROLE(GPIPE_ROLE_DK, LAY_MN, LAY_MN, EPI_STORE)
    GP_ROLE(GPIPE_ROLE_QKV_DGRAD, LAY_K, LAY_MN, EPI_STORE_F32)
    GP_ROLE(GPIPE_ROLE_QKV_WGRAD, LAY_MN, LAY_MN, EPI_ACC_F32)
    default: return hipErrorInvalidValue;
  }
#undef GP_ROLE
}

hipError_t gemm(bool bf16, int role, const GemmParams& g, int batch, hipStream_t s) {
  return bf16 ? dispatch<bf16_t>(role, g, batch, s) : dispatch<float>(role, g, batch, s);
}

int gemm_tile_m(bool bf16) { return bf16 ? Tile<bf16_t>::BM : Tile<float>::BM; }

}  // namespace gp
