// MFMA GEMM kernels of the cell (gfx950).  Included by the gemm_*.hip files,
// each of which instantiates the roles it serves.
//
//   C[z] (M x N) = epilogue( sum_k A[z](m, k) * B[z](k, n) )
//
// Operand layouts in global memory:
//   A: LAY_K  -> A(m, k) = A[m * lda + k]   (k contiguous)
//      LAY_MN -> A(m, k) = A[k * lda + m]   (m contiguous)
//   B: LAY_K  -> B(k, n) = B[n * ldb + k]   (k contiguous)
//      LAY_MN -> B(k, n) = B[k * ldb + n]   (n contiguous)
//
// Register-staged bf16 kernel, used when k is not a multiple of 64 (the
// direct-to-LDS kernel of gemm_dma.hpp takes the rest): 256 threads (4 waves,
// 2 x 2), macro tile BM x BN x 64, each
// wave a (BM/2) x (BN/2) block of v_mfma_f32_16x16x32_bf16 accumulators.
// Both operands sit in LDS k-contiguous, 64 bf16 per row without padding;
// the eight 16-byte chunks of a row are XOR-swizzled by the row index, which
// makes the MFMA fragment reads (16 consecutive rows, one chunk) and the
// tile writes conflict-free.  An m-contiguous operand is loaded as 8 x 8
// blocks (8 k-rows of 8 elements) and transposed in registers before its
// 16-byte LDS writes.  Two LDS buffers: tile k+1 is fetched into registers
// while tile k is multiplied; one barrier per k-tile.
//
// A lane feeds an MFMA with elements k = 8*(lane/16) + e (bf16) or, over four
// consecutive instructions, k = 4*(lane/16) + s (fp32); A and B use the same
// lane->k assignment, which is all the contraction needs.
// Accumulator layout (16x16 block): lane l holds column l%16, rows 4*(l/16)+v.
#pragma once
#include "../../include/gpipe.h"
#include <hip/hip_ext.h>

#include "common.hpp"
#include "kernels.hpp"

namespace gp {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- helpers
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
__device__ __forceinline__ uint32_t dword_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Epilogue of one accumulator element (row, col) of batch offset coff.
template <typename T, int EPI>
__device__ __forceinline__ void epi_store(const GemmParams& g, int row, int col, float a,
                                          int64_t coff) {
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
    if (g.U) static_cast<T*>(g.U)[int64_t(row) * g.ldu + col] = from_f<T>(u);
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

// Causal k-range and tile skipping (see kernels.hpp).  Returns false if the
// tile is skipped entirely.
__device__ __forceinline__ bool causal_range(const GemmParams& g, int m0, int n0, int BM, int BK,
                                             int* kbeg, int* kend) {
  if (g.causal == CAUSAL_SKIP_UPPER && n0 > m0 + BM - 1) return false;
  *kbeg = 0;
  *kend = g.K;
  if (g.causal == CAUSAL_K_UPTO_M) *kend = min(g.K, m0 + BM);
  if (g.causal == CAUSAL_K_FROM_M) *kbeg = (m0 / BK) * BK;
  return true;
}

// Tile index of this workgroup.  Workgroups are dealt to the 8 XCDs round
// robin; renumber so each XCD gets a contiguous range of tiles, walked with
// the m-tile fastest, which keeps the operand panels a range shares in that
// XCD's L2.
// Workgroups are dealt to the eight XCDs round-robin (XCD = bid % 8), and
// each XCD has its own L2.  Each XCD is given one rectangle of the tile grid:
// tiles_m / a row tiles by tiles_n / (8 / a) column tiles, with a in
// {1, 2, 4, 8} chosen to minimise the operand rows it touches,
// (tiles_m / a) * bm + (tiles_n * a / 8) * bn; inside it, tm runs fastest.
// Grids that do not split evenly keep the plain order.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int bm, int bn, int* tm,
                                        int* tn) {
  int best = 0, cost = 0;
  for (int a = 1; a <= 8; a *= 2) {
    const int b = 8 / a;
    if (tiles_m % a || tiles_n % b) continue;
    const int c = (tiles_m / a) * bm + (tiles_n / b) * bn;
    if (!best || c < cost) {
      best = a;
      cost = c;
    }
  }
  if (!best) {
    *tm = bid % tiles_m;
    *tn = bid / tiles_m;
    return;
  }
  const int xcd = bid % 8, j = bid / 8;
  const int rm = tiles_m / best, rn = tiles_n / (8 / best);
  // Within the region, column-major over bands of gm tile rows (the last band
  // may be shorter), so that the 32 workgroups an XCD runs at once share few
  // operand panels: 8 x 4 tiles of 128 x 256, 4 x 8 of 256 x 128 (an A panel
  // of BM rows against a B panel of BN columns, both K deep).
  const int gm = min(bm > bn ? 4 : 8, rm);
  const int full = rm / gm, jb = full * gm * rn;
  int r, c;
  if (j < jb) {
    const int band = j / (gm * rn), q = j % (gm * rn);
    r = band * gm + q % gm;
    c = q / gm;
  } else {
    const int h = rm - full * gm, q = j - jb;
    r = full * gm + q % h;
    c = q / h;
  }
  *tm = (xcd / (8 / best)) * rm + r;
  *tn = (xcd % (8 / best)) * rn + c;
}

// Tile and k-split of a workgroup.  Workgroups go to the 8 XCDs round-robin
// by linear id (x fastest).  Unsplit, or split with a tile count that is a
// multiple of 8 (every split of a tile then shares its XCD), tile_of places
// the tiles.  Otherwise the linear ids are renumbered so that each XCD holds
// one contiguous run of (split, tile) pairs, split-major: the tiles of a
// split, which read the same k-range of A (and of a gathered B), share one L2.
__device__ __forceinline__ void grid_tile(int tiles_m, int tiles_n, int bm, int bn, int* tm,
                                          int* tn, int* split) {
  const int tiles = tiles_m * tiles_n;
  if (gridDim.y == 1 || tiles % 8 == 0) {
    tile_of(blockIdx.x, tiles_m, tiles_n, bm, bn, tm, tn);
    *split = blockIdx.y;
    return;
  }
  const int n = tiles * int(gridDim.y);
  const int lin = int(blockIdx.y) * tiles + int(blockIdx.x);
  const int xcd = lin % 8, i = lin / 8;
  const int v = xcd * (n / 8) + min(xcd, n % 8) + i;  // XCD xcd owns (n - xcd + 7) / 8 ids
  *split = v / tiles;
  const int t = v % tiles;
  *tm = t % tiles_m;
  *tn = t / tiles_m;
}

// ---------------------------------------------------------------- bf16 kernel
template <int BM_, int BN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  // waves per SIMD the register allocation must allow, and LDS stages of the
  // direct-to-LDS kernel (256 x 128: 3 x 48 KB; 128 x 128: 2 x 32 KB, two
  // workgroups per CU; 64 x 64: 3 x 16 KB, three per CU)
  static constexpr int OCC = (BM * BN >= 256 * 128) ? 1 : (BM * BN >= 128 * 128) ? 2 : 3;
  static constexpr int STAGES = (BM * BN == 128 * 128) ? 2 : 3;
  static constexpr int WTM = BM / 2, WTN = BN / 2;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
};

// element offset of (row, 8-element chunk) in a swizzled [rows][64] bf16 tile
__device__ __forceinline__ int swz_off(int row, int chunk) {
  return row * 64 + ((chunk ^ (row & 7)) << 3);
}

template <int ROWS, int LAY>
struct Bf16Loader {
  static constexpr int BK = 64;
  // k-contiguous: 8 chunks of 8 bf16 per row
  static constexpr int NCH = ROWS * 8;
  // m-contiguous: blocks of KB k-rows x 8 elements (KB = 8 when that still
  // gives every thread a block, else 4)
  static constexpr int KB = ((BK / 8) * (ROWS / 8) >= kThreads) ? 8 : 4;
  static constexpr int NBLK = (BK / KB) * (ROWS / 8);
  static constexpr int PER = (LAY == LAY_K) ? NCH / kThreads : (NBLK + kThreads - 1) / kThreads;
  static constexpr int NV = (LAY == LAY_K) ? 1 : KB;
  uint4 v[PER][NV];

  __device__ __forceinline__ void load(const bf16_t* __restrict__ p, int64_t ld, int row0,
                                       int rows_total, int k0, int kend, int tid) {
    if constexpr (LAY == LAY_K) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int c = tid + i * kThreads;
        const int r = c >> 3, kc = (c & 7) * 8;
        const int gr = row0 + r, gk = k0 + kc;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (gr < rows_total && gk < kend) {
          const bf16_t* src = p + int64_t(gr) * ld + gk;
          if (gk + 8 <= kend) {
            x = *reinterpret_cast<const uint4*>(src);
          } else {
            for (int e = 0; e < 8; ++e)
              if (gk + e < kend) set_elem<bf16_t>(x, e, src[e]);
          }
        }
        v[i][0] = x;
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int b = tid + i * kThreads;
        const int kq = b / (ROWS / 8), mc = b % (ROWS / 8);
        const int gm = row0 + mc * 8;
#pragma unroll
        for (int r = 0; r < KB; ++r) {
          uint4 x = make_uint4(0, 0, 0, 0);
          const int gk = k0 + kq * KB + r;
          if (b < NBLK && gk < kend && gm < rows_total) {
            const bf16_t* src = p + int64_t(gk) * ld + gm;
            if (gm + 8 <= rows_total) {
              x = *reinterpret_cast<const uint4*>(src);
            } else {
              for (int e = 0; e < 8; ++e)
                if (gm + e < rows_total) set_elem<bf16_t>(x, e, src[e]);
            }
          }
          v[i][r] = x;
        }
      }
    }
  }

  __device__ __forceinline__ void store(bf16_t* s, int tid) const {
    if constexpr (LAY == LAY_K) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int c = tid + i * kThreads;
        *reinterpret_cast<uint4*>(s + swz_off(c >> 3, c & 7)) = v[i][0];
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int b = tid + i * kThreads;
        if (b < NBLK) {
          const int kq = b / (ROWS / 8), mc = b % (ROWS / 8);
          // transpose the KB x 8 block: output row e gets element e of the KB k-rows
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            uint32_t w[KB / 2];
#pragma unroll
            for (int j = 0; j < KB / 2; ++j) {
              const uint32_t lo = dword_of(v[i][2 * j], e >> 1);
              const uint32_t hi = dword_of(v[i][2 * j + 1], e >> 1);
              w[j] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
            if constexpr (KB == 8) {
              *reinterpret_cast<uint4*>(s + swz_off(mc * 8 + e, kq)) = make_uint4(w[0], w[1], w[2], w[3]);
            } else {
              // half a 16-byte chunk: chunk kq/2, half kq%2
              *reinterpret_cast<uint2*>(s + swz_off(mc * 8 + e, kq >> 1) + (kq & 1) * 4) = make_uint2(w[0], w[1]);
            }
          }
        }
      }
    }
  }
};

template <class C, int LA, int LB, int EPI, int ROLE>
__global__ __launch_bounds__(kThreads, C::OCC) void gemm_bf16_kernel(GemmParams g) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, FM = C::FM, FN = C::FN;
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * BK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, BM, BN, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int z = blockIdx.z, zb = z / g.hdiv, zh = z % g.hdiv;
  int kbeg, kend;
  if (!causal_range(g, m0, n0, BM, BK, &kbeg, &kend)) return;
  // split-K: this workgroup's share of the k range
  const int split = blockIdx.y;
  if (gridDim.y > 1) {
    kbeg = max(kbeg, split * g.kchunk);
    kend = min(kend, (split + 1) * g.kchunk);
  }

  const bf16_t* A = static_cast<const bf16_t*>(g.A) + zb * g.sAb + zh * g.sAh;
  const bf16_t* B = static_cast<const bf16_t*>(g.B) + zb * g.sBb + zh * g.sBh;
  Bf16Loader<BM, LA> la;
  Bf16Loader<BN, LB> lb;
  floatx4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int wm0 = (wave >> 1) * C::WTM, wn0 = (wave & 1) * C::WTN;
  const int nkt = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  const int lrow = lane & 15, lchunk = lane >> 4;
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
    const bf16_t* as = As[cur];
    const bf16_t* bs = Bs[cur];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(as + swz_off(wm0 + i * 16 + lrow, ks * 4 + lchunk));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(bs + swz_off(wn0 + j * 16 + lrow, ks * 4 + lchunk));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nkt) {
      la.store(As[cur ^ 1], tid);
      lb.store(Bs[cur ^ 1], tid);
    }
    __syncthreads();
  }

  if (gridDim.y > 1) {
    // split-K: raw fp32 partial sums; the reduce kernel applies the epilogue
    float* P = g.P + int64_t(split) * g.M * g.N;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn0 + j * 16 + (lane & 15);
        if (col >= g.N) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = m0 + wm0 + i * 16 + (lane >> 4) * 4 + v;
          if (row < g.M) P[int64_t(row) * g.N + col] = acc[i][j][v];
        }
      }
    return;
  }
  const int64_t coff = zb * g.sCb + zh * g.sCh;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn0 + j * 16 + (lane & 15);
      if (col >= g.N) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + wm0 + i * 16 + (lane >> 4) * 4 + v;
        if (row < g.M) epi_store<bf16_t, EPI>(g, row, col, acc[i][j][v], coff);
      }
    }
}

// Sum of the split-K partials in split order, then the role's epilogue.
template <typename T, int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmParams g, int splits) {
  const int64_t n = int64_t(g.M) * g.N;
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < n; e += stride) {
    float s = 0.f;
    for (int p = 0; p < splits; ++p) s += g.P[int64_t(p) * n + e];
    const int row = int(e / g.N), col = int(e % g.N);
    epi_store<T, EPI>(g, row, col, s, 0);
  }
}

// ---------------------------------------------------------------- fp32 kernel
// 64 x 64 x 16 tiles, rows padded by 4 floats in LDS.
template <int LAY, int ROWS>
struct F32Loader {
  static constexpr int BK = 16, LDP = 20;
  static constexpr int CPR = BK / 4, NCH = ROWS * CPR;            // k-contiguous
  static constexpr int NBLK = (BK / 4) * (ROWS / 4);               // m-contiguous 4 x 4 blocks
  static constexpr int PER = ((LAY == LAY_K ? NCH : NBLK) + kThreads - 1) / kThreads;
  static constexpr int NV = (LAY == LAY_K) ? 1 : 4;
  uint4 v[PER][NV];

  __device__ __forceinline__ void load(const float* __restrict__ p, int64_t ld, int row0,
                                       int rows_total, int k0, int kend, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * kThreads;
      if constexpr (LAY == LAY_K) {
        uint4 x = make_uint4(0, 0, 0, 0);
        if (c < NCH) {
          const int r = c / CPR, kc = (c % CPR) * 4;
          const int gr = row0 + r, gk = k0 + kc;
          if (gr < rows_total && gk < kend) {
            const float* src = p + int64_t(gr) * ld + gk;
            if (gk + 4 <= kend) x = *reinterpret_cast<const uint4*>(src);
            else
              for (int e = 0; e < 4; ++e)
                if (gk + e < kend) set_elem<float>(x, e, src[e]);
          }
        }
        v[i][0] = x;
      } else {
        const int kq = c / (ROWS / 4), mc = c % (ROWS / 4);
        const int gm = row0 + mc * 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          uint4 x = make_uint4(0, 0, 0, 0);
          const int gk = k0 + kq * 4 + r;
          if (c < NBLK && gk < kend && gm < rows_total) {
            const float* src = p + int64_t(gk) * ld + gm;
            if (gm + 4 <= rows_total) x = *reinterpret_cast<const uint4*>(src);
            else
              for (int e = 0; e < 4; ++e)
                if (gm + e < rows_total) set_elem<float>(x, e, src[e]);
          }
          v[i][r] = x;
        }
      }
    }
  }

  __device__ __forceinline__ void store(float* s, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * kThreads;
      if constexpr (LAY == LAY_K) {
        if (c < NCH) {
          const int r = c / CPR, kc = (c % CPR) * 4;
          *reinterpret_cast<uint4*>(s + r * LDP + kc) = v[i][0];
        }
      } else {
        if (c < NBLK) {
          const int kq = c / (ROWS / 4), mc = c % (ROWS / 4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            *reinterpret_cast<uint4*>(s + (mc * 4 + e) * LDP + kq * 4) =
                make_uint4(dword_of(v[i][0], e), dword_of(v[i][1], e), dword_of(v[i][2], e),
                           dword_of(v[i][3], e));
        }
      }
    }
  }
};

template <int LA, int LB, int EPI, int ROLE>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmParams g) {
  constexpr int BM = 64, BN = 64, BK = 16, LDP = 20, FM = 2, FN = 2, WT = 32;
  __shared__ __attribute__((aligned(16))) float As[2][BM * LDP];
  __shared__ __attribute__((aligned(16))) float Bs[2][BN * LDP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, BM, BN, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int z = blockIdx.z, zb = z / g.hdiv, zh = z % g.hdiv;
  int kbeg, kend;
  if (!causal_range(g, m0, n0, BM, BK, &kbeg, &kend)) return;
  const float* A = static_cast<const float*>(g.A) + zb * g.sAb + zh * g.sAh;
  const float* B = static_cast<const float*>(g.B) + zb * g.sBb + zh * g.sBh;
  F32Loader<LA, BM> la;
  F32Loader<LB, BN> lb;
  floatx4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  const int wm0 = (wave >> 1) * WT, wn0 = (wave & 1) * WT;
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
    floatx4_t af[FM], bfr[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
      af[i] = *reinterpret_cast<const floatx4_t*>(As[cur] + (wm0 + i * 16 + (lane & 15)) * LDP + (lane >> 4) * 4);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      bfr[j] = *reinterpret_cast<const floatx4_t*>(Bs[cur] + (wn0 + j * 16 + (lane & 15)) * LDP + (lane >> 4) * 4);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][s], bfr[j][s], acc[i][j], 0, 0, 0);
    if (kt + 1 < nkt) {
      la.store(As[cur ^ 1], tid);
      lb.store(Bs[cur ^ 1], tid);
    }
    __syncthreads();
  }
  const int64_t coff = zb * g.sCb + zh * g.sCh;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn0 + j * 16 + (lane & 15);
      if (col >= g.N) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + wm0 + i * 16 + (lane >> 4) * 4 + v;
        if (row < g.M) epi_store<float, EPI>(g, row, col, acc[i][j][v], coff);
      }
    }
}

// ---------------------------------------------------------------- launch helpers
// Tile configurations of the bf16 kernel (index = GemmPlan::cfg).
// Tile configurations (GemmPlan::cfg): macro tile, k-tile depth and LDS
// stages of the direct-to-LDS kernel.
enum {
  CFG_256x128_K64 = 0,   // specialised waves: 3 stages x 48 KB, one workgroup per CU
  CFG_128x256_K64 = 1,
  CFG_128x128_K64 = 2,   // 2 stages x 32 KB, two workgroups per CU
  CFG_128x128_SPEC = 3,  // specialised waves: 4 stages x 32 KB, one workgroup per CU
  CFG_64x64_K64 = 4,     // 3 stages x 16 KB
  CFG_N
};
constexpr int kCfgBM[CFG_N] = {256, 128, 128, 128, 64};
constexpr int kCfgBN[CFG_N] = {128, 256, 128, 128, 64};

// Launches one instance (defined in gemm_dma.hpp).
template <class DC, class RC, int LA, int LB, int EPI, int ROLE>
hipError_t launch_bf16(int path, const GemmParams& g, int batch, int splits, hipStream_t s);

// Operand layouts and epilogue of every GEMM role of the step.
//   forward linears          C = A W^T (+ epilogue)          A: K,  B: K
//   input-gradient products  dA = dC W                      A: K,  B: MN
//   weight gradients         G (+)= dC^T A  (over tokens)    A: MN, B: MN
template <int ROLE> struct RoleSpec;
#define GP_SPEC(R, LA_, LB_, EPI_)                                        \
  template <> struct RoleSpec<R> {                                        \
    static constexpr int LA = LA_, LB = LB_, EPI = EPI_;                  \
  };
GP_SPEC(GPIPE_ROLE_QKV_FWD, LAY_K, LAY_K, EPI_BIAS)
GP_SPEC(GPIPE_ROLE_SCORES_FWD, LAY_K, LAY_K, EPI_STORE_F32)
GP_SPEC(GPIPE_ROLE_PV_FWD, LAY_K, LAY_MN, EPI_STORE)
GP_SPEC(GPIPE_ROLE_OUT_FWD, LAY_K, LAY_K, EPI_BIAS_RESID)
GP_SPEC(GPIPE_ROLE_FFN1_FWD, LAY_K, LAY_K, EPI_BIAS_GELU)
GP_SPEC(GPIPE_ROLE_FFN2_FWD, LAY_K, LAY_K, EPI_BIAS_RESID)
GP_SPEC(GPIPE_ROLE_FFN2_DGRAD, LAY_K, LAY_MN, EPI_GELU_BWD)
GP_SPEC(GPIPE_ROLE_FFN2_WGRAD, LAY_MN, LAY_MN, EPI_ACC_F32)
GP_SPEC(GPIPE_ROLE_FFN1_DGRAD, LAY_K, LAY_MN, EPI_STORE_F32)
GP_SPEC(GPIPE_ROLE_FFN1_WGRAD, LAY_MN, LAY_MN, EPI_ACC_F32)
GP_SPEC(GPIPE_ROLE_OUT_DGRAD, LAY_K, LAY_MN, EPI_STORE)
GP_SPEC(GPIPE_ROLE_OUT_WGRAD, LAY_MN, LAY_MN, EPI_ACC_F32)
GP_SPEC(GPIPE_ROLE_DP, LAY_K, LAY_K, EPI_STORE_F32)
GP_SPEC(GPIPE_ROLE_DV, LAY_MN, LAY_MN, EPI_STORE)
GP_SPEC(GPIPE_ROLE_DQ, LAY_K, LAY_MN, EPI_STORE)
GP_SPEC(GPIPE_ROLE_DK, LAY_MN, LAY_MN, EPI_STORE)
GP_SPEC(GPIPE_ROLE_QKV_DGRAD, LAY_K, LAY_MN, EPI_STORE_F32)
GP_SPEC(GPIPE_ROLE_QKV_WGRAD, LAY_MN, LAY_MN, EPI_ACC_F32)
// 3x3 convolutions as GEMMs over the im2col matrix [P, 9C]:
//   forward  a = col W^T (f32: the BatchNorm input);  input gradient dcol = da W (f32);
//   weight gradient G (+)= da^T col
GP_SPEC(GPIPE_ROLE_CONV_FWD, LAY_K, LAY_K, EPI_STORE_F32)
GP_SPEC(GPIPE_ROLE_CONV_DGRAD, LAY_K, LAY_MN, EPI_STORE_F32)
GP_SPEC(GPIPE_ROLE_CONV_WGRAD, LAY_MN, LAY_MN, EPI_ACC_F32)
// implicit GEMM: a = im2col(x) W^T with the column matrix gathered by the loads;
// the input gradient (+)= im2col(dz) Wflip^T, Wflip the tap-flipped transposed weights
GP_SPEC(GPIPE_ROLE_CONV_FWD_IMPLICIT, LAY_CONV, LAY_K, EPI_STORE_F32)
GP_SPEC(GPIPE_ROLE_CONV_DGRAD_IMPLICIT, LAY_CONV, LAY_K, EPI_ACC_F32)
// and the weight gradient G (+)= da^T im2col(x), the column matrix gathered along k
GP_SPEC(GPIPE_ROLE_CONV_WGRAD_IMPLICIT, LAY_MN, LAY_CONV_MN, EPI_ACC_F32)
#undef GP_SPEC

template <int BM, int BN, int BK, int ST, int OCC> struct DCfg;
// DCfg is defined in gemm_dma.hpp; the register-staged fallback uses 128 x 128
// for the big configurations and 64 x 64 for the small one.
template <int ROLE>
hipError_t launch_role(int path, int cfg, const GemmParams& g, int batch, int splits, hipStream_t s) {
  using R = RoleSpec<ROLE>;
  using RB = Cfg<128, 128>;
  if constexpr (R::LA == LAY_CONV) {
    // three tile configurations for the gathered operand
    if (cfg == CFG_128x128_SPEC)
      return launch_bf16<DCfg<128, 128, 64, 4, 1>, RB, R::LA, R::LB, R::EPI, ROLE>(path, g, batch,
                                                                                  splits, s);
    if (cfg == CFG_128x256_K64)
      return launch_bf16<DCfg<128, 256, 64, 3, 1>, RB, R::LA, R::LB, R::EPI, ROLE>(path, g, batch,
                                                                                  splits, s);
    if (cfg != CFG_128x128_K64) return hipErrorInvalidValue;
    return launch_bf16<DCfg<128, 128, 64, 2, 2>, RB, R::LA, R::LB, R::EPI, ROLE>(path, g, batch,
                                                                                splits, s);
  } else if constexpr (R::LB == LAY_CONV_MN) {
    // the specialised-wave tile configurations for the gathered B operand
    switch (cfg) {
      case CFG_256x128_K64: return launch_bf16<DCfg<256, 128, 64, 3, 1>, RB, R::LA, R::LB, R::EPI, ROLE>(path, g, batch, splits, s);
      case CFG_128x128_SPEC: return launch_bf16<DCfg<128, 128, 64, 4, 1>, RB, R::LA, R::LB, R::EPI, ROLE>(path, g, batch, splits, s);
    }
    return hipErrorInvalidValue;
  } else {
  switch (cfg) {
    case CFG_256x128_K64: return launch_bf16<DCfg<256, 128, 64, 3, 1>, RB, R::LA, R::LB, R::EPI, ROLE>(path, g, batch, splits, s);
    case CFG_128x256_K64: return launch_bf16<DCfg<128, 256, 64, 3, 1>, RB, R::LA, R::LB, R::EPI, ROLE>(path, g, batch, splits, s);
    case CFG_128x128_K64: return launch_bf16<DCfg<128, 128, 64, 2, 2>, RB, R::LA, R::LB, R::EPI, ROLE>(path, g, batch, splits, s);
    case CFG_128x128_SPEC: return launch_bf16<DCfg<128, 128, 64, 4, 1>, RB, R::LA, R::LB, R::EPI, ROLE>(path, g, batch, splits, s);
    case CFG_64x64_K64: return launch_bf16<DCfg<64, 64, 64, 3, 3>, Cfg<64, 64>, R::LA, R::LB, R::EPI, ROLE>(path, g, batch, splits, s);
  }
  return hipErrorInvalidValue;
  }
}

// Per-file group launchers (gemm_fwd.hip, gemm_dgrad.hip, gemm_wgrad.hip,
// gemm_attn.hip, gemm_f32.hip).
hipError_t gemm_group_fwd(int role, int path, int cfg, const GemmParams& g, int batch, int splits, hipStream_t s);
hipError_t gemm_group_dgrad(int role, int path, int cfg, const GemmParams& g, int batch, int splits, hipStream_t s);
hipError_t gemm_group_wgrad(int role, int path, int cfg, const GemmParams& g, int batch, int splits, hipStream_t s);
hipError_t gemm_group_attn(int role, int path, int cfg, const GemmParams& g, int batch, int splits, hipStream_t s);
hipError_t gemm_group_f32(int role, const GemmParams& g, int batch, hipStream_t s);

// Launches a kernel; `first` / `last`: it is the first / last kernel of its
// GEMM launch, which then records the pending role-timing events
// (launch_events()) in its dispatch and clears them.
template <typename K, typename... A>
hipError_t launch_timed(K kernel, dim3 grid, dim3 block, uint32_t smem, hipStream_t s, bool first,
                        bool last, A... args) {
  LaunchEvents& le = launch_events();
  hipEvent_t e0 = first ? le.start : nullptr, e1 = last ? le.stop : nullptr;
  if (first) le.start = nullptr;
  if (last) le.stop = nullptr;
  // the pending end event (next_done_event) goes to the last kernel's dispatch
  // unless role timing holds its stop slot; then it is recorded after it
  hipEvent_t done = nullptr;
  if (last) {
    done = next_done_event();
    next_done_event() = nullptr;
    if (!e1) {
      e1 = done;
      done = nullptr;
    }
  }
  if (e0 || e1)
    hipExtLaunchKernelGGL(kernel, grid, block, smem, s, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, smem, s, args...);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess && done) err = hipEventRecord(done, s);
  return err;
}

// A GEMM launch with nothing to compute still takes the pending events:
// both are recorded on the stream (an empty interval).
inline hipError_t launch_nothing(hipStream_t s) {
  LaunchEvents& le = launch_events();
  hipError_t e = hipSuccess;
  if (le.start) e = hipEventRecord(le.start, s);
  if (le.stop && e == hipSuccess) e = hipEventRecord(le.stop, s);
  if (next_done_event() && e == hipSuccess) e = hipEventRecord(next_done_event(), s);
  le.start = le.stop = nullptr;
  next_done_event() = nullptr;
  return e;
}

template <int LA, int LB, int EPI, int ROLE>
hipError_t launch_f32(const GemmParams& g, int batch, hipStream_t s) {
  const int tiles = ((g.M + 63) / 64) * ((g.N + 63) / 64);
  if (tiles == 0 || batch == 0) return launch_nothing(s);
  return launch_timed((gemm_f32_kernel<LA, LB, EPI, ROLE>), dim3(tiles, 1, batch), dim3(kThreads),
                      0, s, true, true, g);
}

}  // namespace gp
