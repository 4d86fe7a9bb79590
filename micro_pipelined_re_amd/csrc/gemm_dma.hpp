// bf16 GEMM with HBM -> LDS direct loads (gfx950 global_load_lds_dwordx4).
//
// No staging registers: each wave's load instruction writes 64 x 16 bytes to
// a contiguous kilobyte of LDS (lane l at +16*l), and the global address each
// lane fetches is chosen so that the kilobyte holds the tile in its swizzled
// layout.  S LDS stages keep S-1 k-tiles in flight.
//
// Tile layouts in LDS (k-tile depth BK = 64 or 32):
//   k-contiguous operand  [rows][BK]: rows of BK/8 16-byte chunks; chunk c of
//       row r stored at position c ^ (r & 7) (BK 64) or c ^ ((r >> 2) & 3)
//       (BK 32); MFMA fragments are one ds_read_b128 (16 rows x one chunk).
//       Measured with the LDS bank-conflict counter on gfx950, the plain
//       c ^ (r & 7) reads without conflicts where c ^ ((r ^ r>>3) & 7)
//       spends a quarter of its LDS cycles in conflicts.
//   m-contiguous operand  [64 k][R]: rows of R elements in 32-byte granules,
//       granule q of k-row r stored at q ^ f(r), f(r) = (r & 3) | (r>>3 & 1) << 2
//       (R >= 128) or (r>>1 & 1) | (r>>3 & 1) << 1 (R = 64), which the LDS
//       bank-conflict counter shows conflict-free for the fragment reads (a
//       plain r & 7 conflicts half of the time); fragments are two
//       ds_read_b64_tr_b16: within a group of 16
//       lanes, lane s points at (k0 + s/4, m0 + 4*(s%4)) and lane i receives
//       the four k-rows k0..k0+3 of column m0 + i.
// Rows past the operand's extent are read from its last row (valid memory;
// those results are never stored).  k must be a multiple of 64.
#pragma once
#include <type_traits>

#include "gemm_impl.hpp"

namespace gp {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

__device__ __forceinline__ void dma16(const void* g, bf16_t* lds_block) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds_block, 16, 0, 0);
}

// Workgroup barrier without a memory fence: the waves have already waited for
// their own LDS loads (vmcnt), and a fence would also drain the loads of the
// younger k-tiles still in flight.  The asm's memory clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// Barrier after ordinary LDS writes: s_barrier alone does not wait for a
// wave's outstanding LDS operations, so drain them (lgkmcnt) first.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

#define LPT_CHECK(lpt, stages) ((lpt) * ((stages) - 2) < 64)

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// granule swizzle of an m-contiguous tile with R elements per k-row
template <int R>
__device__ __forceinline__ int mn_swz(int k) {
  // one fragment read touches k-rows {0..3, 8..11, 16..19, 24..27} (+ 32 ks);
  // these map to distinct 32-byte granule slots within each half wave
  if constexpr (R >= 128) return (k & 3) | (((k >> 3) & 1) << 2);
  else return ((k >> 1) & 1) | (((k >> 3) & 1) << 1);
}
template <int R>
__device__ __forceinline__ int mn_off(int k, int m) {
  return k * R + (((m >> 4) ^ mn_swz<R>(k)) << 4) + (m & 15);
}

// element offset of (row, 16-byte chunk) in a swizzled k-contiguous tile
template <int BK>
__device__ __forceinline__ int kswz_off(int row, int chunk) {
  if constexpr (BK == 64) return row * 64 + ((chunk ^ (row & 7)) << 3);
  else return row * 32 + ((chunk ^ ((row >> 2) & 3)) << 3);
}

// All-zero source for the loads of padding pixels of a LAY_CONV operand.
static __device__ __attribute__((aligned(16))) bf16_t g_conv_zero[8];

// A operand gathered from an NHWC image (LAY_CONV): the tile is stored like a
// k-contiguous one; each load instruction's lane owns one pixel row and one
// 16-byte chunk, and its source moves with the k-tile's tap.
template <int ROWS, int BK>
struct DmaConvOperand {
  static_assert(BK == 64, "conv operands use 64-deep k-tiles");
  static constexpr int ELEMS = ROWS * BK;
  static constexpr int KB_PER_STAGE = ELEMS * 2 / 1024;
  static constexpr int PER_WAVE = KB_PER_STAGE / 4;
  int pix[PER_WAVE];     // pixel index (row of the operand, clamped into range)
  short hh[PER_WAVE], ww[PER_WAVE];
  short coff[PER_WAVE];  // element offset of the lane's chunk inside the k-tile
  int H, W, C, kbeg;

  __device__ __forceinline__ void init(const GemmParams& g, int row0, int rows_total, int kb,
                                       int wave, int lane) {
    H = g.conv_h;
    W = g.conv_w;
    C = g.conv_c;
    kbeg = kb;
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q) {
      const int blk = q * 4 + wave;
      const int r = blk * 8 + lane / 8;       // 8 rows of 8 chunks per kilobyte
      const int p = lane % 8;
      const int c = p ^ (r & 7);
      const int gr = min(row0 + r, rows_total - 1);
      pix[q] = gr;
      ww[q] = short(gr % W);
      hh[q] = short((gr / W) % H);
      coff[q] = short(c * 8);
    }
  }

  __device__ __forceinline__ void issue(const bf16_t* img, int kt, bf16_t* stage, int wave) const {
    const int k0 = kbeg + kt * BK;
    const int tap = k0 / C, c0 = k0 - tap * C;
    const int dh = tap / 3 - 1, dw = tap - (tap / 3) * 3 - 1;
    const int shift = dh * W + dw;
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q) {
      const int hs = hh[q] + dh, ws = ww[q] + dw;
      const bool in = unsigned(hs) < unsigned(H) && unsigned(ws) < unsigned(W);
      const bf16_t* src = in ? img + int64_t(pix[q] + shift) * C + c0 + coff[q] : g_conv_zero;
      dma16(src, stage + (q * 4 + wave) * 512);
    }
  }

  __device__ __forceinline__ bf16x8_t frag(const bf16_t* stage, int row16, int lane, int ks) const {
    const int r = row16 + (lane & 15);
    return *reinterpret_cast<const bf16x8_t*>(stage + kswz_off<BK>(r, ks * 4 + (lane >> 4)));
  }
};

template <int ROWS, int BK, int LAY>
struct DmaOperand {
  static constexpr int ELEMS = ROWS * BK;          // per stage
  static constexpr int KB_PER_STAGE = ELEMS * 2 / 1024;
  static constexpr int PER_WAVE = KB_PER_STAGE / 4;  // load instructions per wave per stage
  static_assert(PER_WAVE >= 1 && KB_PER_STAGE % 4 == 0, "tile too small for four waves");
  int64_t off[PER_WAVE];  // element offsets of this lane's source (at k-tile 0)
  int64_t kstep;          // element step per k-tile

  __device__ __forceinline__ void init(int64_t ld, int row0, int rows_total, int kbeg, int wave,
                                       int lane) {
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q) {
      const int blk = q * 4 + wave;  // kilobyte of the stage this instruction fills
      if constexpr (LAY == LAY_K) {
        constexpr int CPR = BK / 8;          // chunks per row
        constexpr int RPK = 1024 / (BK * 2); // rows per kilobyte
        const int r = blk * RPK + lane / CPR;
        const int p = lane % CPR;
        const int c = (BK == 64) ? (p ^ (r & 7)) : (p ^ ((r >> 2) & 3));
        const int gr = min(row0 + r, rows_total - 1);
        off[q] = int64_t(gr) * ld + kbeg + c * 8;
      } else {
        const int byte = blk * 1024 + lane * 16;
        const int kr = byte / (ROWS * 2);
        const int within = byte % (ROWS * 2);
        const int p = within >> 5, h = (within >> 4) & 1;
        const int m = ((p ^ mn_swz<ROWS>(kr)) << 4) + h * 8;
        const int gm = min(row0 + m, rows_total - 8);
        off[q] = int64_t(kbeg + kr) * ld + gm;
      }
    }
    kstep = (LAY == LAY_K) ? BK : int64_t(BK) * ld;
  }

  __device__ __forceinline__ void issue(const bf16_t* base, int kt, bf16_t* stage, int wave) const {
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q) dma16(base + off[q] + kt * kstep, stage + (q * 4 + wave) * 512);
  }

  // MFMA fragment (8 bf16, k = ks*32 + 8*(lane/16) + e) of tile rows row16 .. row16+15
  __device__ __forceinline__ bf16x8_t frag(const bf16_t* stage, int row16, int lane, int ks) const {
    if constexpr (LAY == LAY_K) {
      const int r = row16 + (lane & 15);
      return *reinterpret_cast<const bf16x8_t*>(stage + kswz_off<BK>(r, ks * 4 + (lane >> 4)));
    } else {
      const int s = lane & 15, g = lane >> 4;
      const int k0 = ks * 32 + g * 8 + (s >> 2);
      const int m = row16 + 4 * (s & 3);
      const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_short4_t*)(stage + mn_off<ROWS>(k0, m)));
      const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_short4_t*)(stage + mn_off<ROWS>(k0 + 4, m)));
      typedef short short8_t __attribute__((ext_vector_type(8)));
      const short8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return __builtin_bit_cast(bf16x8_t, v);
    }
  }
};

// B operand gathered from an NHWC image with the pixels along k
// (LAY_CONV_MN): stored like an m-contiguous tile.  Each load's lane owns
// eight columns (channels c..c+7 of one tap) and one k-row.  The columns fix
// the tap; the pixel of a k-row moves by 64 per k-tile, and its (h, w) are
// carried along: found once by two divisions (products with rounded
// reciprocals, exact for pixel indices below 2^21: the rounded quotient of
// (p + 0.5) / W lies within 2^-23 relative of the true one, which is at
// least 0.5 / W away from an integer), then advanced by (64 / W) mod H rows
// and 64 mod W columns with one carry each.  issue() must be called for the
// k-tiles 0, 1, 2, ... in order.
template <int ROWS, int BK>
struct DmaConvMnOperand : DmaOperand<ROWS, BK, LAY_MN> {
  static_assert(BK == 64, "conv operands use 64-deep k-tiles");
  static constexpr int PER_WAVE = DmaOperand<ROWS, BK, LAY_MN>::PER_WAVE;
  int src[PER_WAVE];               // element offset of the shifted pixel's channels
  int h[PER_WAVE], w[PER_WAVE];    // image row and column of the k-row's pixel
  int hlo[PER_WAVE], wlo[PER_WAVE];        // the tap's pixel is inside the image
  unsigned hcnt[PER_WAVE], wcnt[PER_WAVE];  // iff h - hlo < hcnt and w - wlo < wcnt
  int H, W, step, dh64, dw64;

  __device__ __forceinline__ void init(const GemmParams& g, int col0, int cols_total, int kb,
                                       int wave, int lane) {
    H = g.conv_h;
    W = g.conv_w;
    const int C = g.conv_c;
    const int LD = g.conv_ld ? g.conv_ld : C;  // the image's pixel stride
    step = BK * LD;
    dh64 = (BK / W) % H;
    dw64 = BK % W;
    const float inv_w = 1.0f / float(W), inv_h = 1.0f / float(H);
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q) {
      const int blk = q * 4 + wave;
      const int byte = blk * 1024 + lane * 16;
      const int r = byte / (ROWS * 2);
      const int within = byte % (ROWS * 2);
      const int gq = within >> 5, hf = (within >> 4) & 1;
      const int m = ((gq ^ mn_swz<ROWS>(r)) << 4) + hf * 8;
      const int gn = min(col0 + m, cols_total - 8);
      const int tap = gn / C;
      const int dh = tap / 3 - 1, dw = tap - (tap / 3) * 3 - 1;
      const int p = kb + r;
      const int pw = int((float(p) + 0.5f) * inv_w);  // p / W
      const int ph = int((float(pw) + 0.5f) * inv_h);  // (p / W) / H
      w[q] = p - pw * W;
      h[q] = pw - ph * H;
      src[q] = (p + dh * W + dw) * LD + (gn - tap * C);
      hlo[q] = dh < 0 ? 1 : 0;
      wlo[q] = dw < 0 ? 1 : 0;
      hcnt[q] = unsigned(H - (dh != 0 ? 1 : 0));
      wcnt[q] = unsigned(W - (dw != 0 ? 1 : 0));
    }
  }

  __device__ __forceinline__ void issue(const bf16_t* img, int, bf16_t* stage, int wave) {
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q) {
      // (both tests evaluated: a select, no branch)
      const bool in = (unsigned(h[q] - hlo[q]) < hcnt[q]) & (unsigned(w[q] - wlo[q]) < wcnt[q]);
      dma16(in ? img + src[q] : g_conv_zero, stage + (q * 4 + wave) * 512);
      src[q] += step;
      w[q] += dw64;
      const int carry = w[q] >= W ? 1 : 0;
      w[q] -= carry * W;
      h[q] += dh64 + carry;
      if (h[q] >= H) h[q] -= H;
    }
  }
};

// Waits until at most n (<= MAXN) younger k-tiles of LPT loads each are in flight.
template <int LPT, int MAXN>
__device__ __forceinline__ void wait_tiles(int n) {
  if (n >= MAXN) {
    wait_vmcnt<MAXN * LPT>();
  } else if constexpr (MAXN > 0) {
    wait_tiles<LPT, MAXN - 1>(n);
  }
}

// Tile configuration of the direct-to-LDS kernel.
template <int BM_, int BN_, int BK_, int STAGES_, int OCC_>
struct DCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, OCC = OCC_;
  static constexpr int WTM = BM / 2, WTN = BN / 2;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
};

// Epilogue of eight consecutive columns (col .. col+7) of one row, all in range.
template <int EPI>
__device__ __forceinline__ void epi_store8(const GemmParams& g, int row, int col, const float* a,
                                           int64_t coff, float* P) {
  if (P) {  // split-K partial sums
    float* dst = P + int64_t(row) * g.N + col;
    reinterpret_cast<float4*>(dst)[0] = make_float4(a[0], a[1], a[2], a[3]);
    reinterpret_cast<float4*>(dst)[1] = make_float4(a[4], a[5], a[6], a[7]);
    return;
  }
  const int64_t ci = coff + int64_t(row) * g.ldc + col;
  float o[8];
  if constexpr (EPI == EPI_STORE_F32 || EPI == EPI_ACC_F32) {
    float* dst = static_cast<float*>(g.C) + ci;
    if (EPI == EPI_ACC_F32 && g.beta) {
      const float4 c0 = reinterpret_cast<const float4*>(dst)[0];
      const float4 c1 = reinterpret_cast<const float4*>(dst)[1];
      o[0] = c0.x + a[0]; o[1] = c0.y + a[1]; o[2] = c0.z + a[2]; o[3] = c0.w + a[3];
      o[4] = c1.x + a[4]; o[5] = c1.y + a[5]; o[6] = c1.z + a[6]; o[7] = c1.w + a[7];
    } else {
      const float k = (EPI == EPI_STORE_F32) ? g.alpha : 1.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = k * a[e];
    }
    reinterpret_cast<float4*>(dst)[0] = make_float4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<float4*>(dst)[1] = make_float4(o[4], o[5], o[6], o[7]);
    return;
  } else {
    auto ld8 = [](const bf16_t* p, float* v) {
      const uint4 u = *reinterpret_cast<const uint4*>(p);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    };
    auto st8 = [](bf16_t* p, const float* v) {
      uint4 u;
      u.x = f2bf2(v[0], v[1]);
      u.y = f2bf2(v[2], v[3]);
      u.z = f2bf2(v[4], v[5]);
      u.w = f2bf2(v[6], v[7]);
      *reinterpret_cast<uint4*>(p) = u;
    };
    float b[8];
    if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_RESID || EPI == EPI_BIAS_GELU) {
      const float4 b0 = reinterpret_cast<const float4*>(g.bias + col)[0];
      const float4 b1 = reinterpret_cast<const float4*>(g.bias + col)[1];
      b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w;
      b[4] = b1.x; b[5] = b1.y; b[6] = b1.z; b[7] = b1.w;
    }
    if constexpr (EPI == EPI_STORE) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = g.alpha * a[e];
    } else if constexpr (EPI == EPI_BIAS) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = a[e] + b[e];
    } else if constexpr (EPI == EPI_BIAS_RESID) {
      float r[8];
      ld8(static_cast<const bf16_t*>(g.R) + int64_t(row) * g.ldr + col, r);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = a[e] + b[e] + r[e];
    } else if constexpr (EPI == EPI_BIAS_GELU) {
      float u[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        u[e] = a[e] + b[e];
        o[e] = gelu_f(u[e]);
      }
      if (g.U) st8(static_cast<bf16_t*>(g.U) + int64_t(row) * g.ldu + col, u);
    } else if constexpr (EPI == EPI_GELU_BWD) {
      float u[8];
      ld8(static_cast<const bf16_t*>(g.U) + int64_t(row) * g.ldu + col, u);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = a[e] * gelu_grad_f(u[e]);
    }
    st8(static_cast<bf16_t*>(g.C) + ci, o);
  }
}

template <class C, int LA, int LB, int EPI, int ROLE>
__global__ __launch_bounds__(kThreads, C::OCC) void gemm_dma_kernel(GemmParams g) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, STAGES = C::STAGES, FM = C::FM, FN = C::FN;
  using OA = typename std::conditional<LA == LAY_CONV, DmaConvOperand<BM, BK>,
                                       DmaOperand<BM, BK, LA>>::type;
  using OB = typename std::conditional<LB == LAY_CONV_MN, DmaConvMnOperand<BN, BK>,
                                       DmaOperand<BN, BK, LB>>::type;
  static_assert(LPT_CHECK(OA::PER_WAVE + OB::PER_WAVE, STAGES), "vmcnt range");
  constexpr int LPT = OA::PER_WAVE + OB::PER_WAVE;  // load instructions per wave per k-tile
  // pipeline stages; after the k loop the same memory holds the fp32 tile
  constexpr int PIPE = STAGES * (BM + BN) * BK * 2, TP = BN + 4;  // TP: tile row pitch (floats)
  constexpr int SMEM = (PIPE > BM * TP * 4) ? PIPE : BM * TP * 4;
  __shared__ __attribute__((aligned(1024))) bf16_t smem[SMEM / 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, BM, BN, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int z = blockIdx.z, zb = z / g.hdiv, zh = z % g.hdiv;
  int kbeg, kend;
  if (!causal_range(g, m0, n0, BM, BK, &kbeg, &kend)) return;
  const int split = blockIdx.y;
  if (gridDim.y > 1) {
    kbeg = max(kbeg, split * g.kchunk);
    kend = min(kend, (split + 1) * g.kchunk);
  }
  const bf16_t* A = static_cast<const bf16_t*>(g.A) + zb * g.sAb + zh * g.sAh;
  const bf16_t* B = static_cast<const bf16_t*>(g.B) + zb * g.sBb + zh * g.sBh;
  OA oa;
  OB ob;
  if constexpr (LA == LAY_CONV) oa.init(g, m0, g.M, kbeg, wave, lane);
  else oa.init(g.lda, m0, g.M, kbeg, wave, lane);
  if constexpr (LB == LAY_CONV_MN) ob.init(g, n0, g.N, kbeg, wave, lane);
  else ob.init(g.ldb, n0, g.N, kbeg, wave, lane);
  auto sa = [&](int st) { return smem + st * (BM + BN) * BK; };
  auto sb = [&](int st) { return smem + st * (BM + BN) * BK + BM * BK; };

  floatx4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  const int wm0 = (wave >> 1) * C::WTM, wn0 = (wave & 1) * C::WTN;
  const int nkt = kend > kbeg ? (kend - kbeg) / BK : 0;

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nkt) {
      oa.issue(A, s, sa(s), wave);
      ob.issue(B, s, sb(s), wave);
    }
  int st = 0;
  for (int kt = 0; kt < nkt; ++kt) {
    // tile kt must have landed; up to STAGES-2 younger tiles may still be in flight
    wait_tiles<LPT, STAGES - 2>(min(STAGES - 2, nkt - 1 - kt));
    barrier_nofence();
    if (kt + STAGES - 1 < nkt) {
      const int ns = (st + STAGES - 1) % STAGES;
      oa.issue(A, kt + STAGES - 1, sa(ns), wave);
      ob.issue(B, kt + STAGES - 1, sb(ns), wave);
    }
    const bf16_t* as = sa(st);
    const bf16_t* bs = sb(st);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = oa.frag(as, wm0 + i * 16, lane, ks);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = ob.frag(bs, wn0 + j * 16, lane, ks);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    st = (st + 1 == STAGES) ? 0 : st + 1;
  }

  // Epilogue through LDS: each wave writes its accumulators into a [BM][BN+4]
  // fp32 tile (conflict-free: the four row groups of a write land 16 banks
  // apart), then each thread takes 8 consecutive columns of a row and does
  // 16-byte loads and stores.
  barrier_lds();
  float* tile = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        tile[(wm0 + i * 16 + (lane >> 4) * 4 + v) * TP + wn0 + j * 16 + (lane & 15)] = acc[i][j][v];
  barrier_lds();
  float* P = gridDim.y > 1 ? g.P + int64_t(split) * g.M * g.N : nullptr;
  const int64_t coff = zb * g.sCb + zh * g.sCh;
  constexpr int CH = BN / 8;  // 8-column chunks per row
  for (int idx = tid; idx < BM * CH; idx += kThreads) {
    const int r = idx / CH, c = (idx % CH) * 8;
    const int row = m0 + r, col = n0 + c;
    if (row >= g.M || col >= g.N) continue;
    const float4 t0 = *reinterpret_cast<const float4*>(tile + r * TP + c);
    const float4 t1 = *reinterpret_cast<const float4*>(tile + r * TP + c + 4);
    const float a[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
    if (col + 8 <= g.N) {
      epi_store8<EPI>(g, row, col, a, coff, P);
    } else {
      for (int e = 0; e < 8 && col + e < g.N; ++e) {
        if (P) P[int64_t(row) * g.N + col + e] = a[e];
        else epi_store<bf16_t, EPI>(g, row, col + e, a[e], coff);
      }
    }
  }
}

// One workgroup per CU, 8 waves in two roles.  Waves 0-3 only read LDS and
// issue MFMAs (2 x 2 grid, each a (BM/2) x (BN/2) block); waves 4-7 only
// issue the direct-to-LDS loads.  A wave issues in order, and a load
// instruction waits for the CU's texture unit: issued from the MFMA waves, the
// loads of one k-tile stalled the MFMAs behind them for about 60% of the
// k-tile's MFMA time on gfx950, so the loads live in waves of their own.
// Three LDS stages: after barrier j of the k loop the stage of tile j is free
// (its last fragments were read before the barrier) and the loader waves
// refill it with tile j + 3; before barrier j they wait for tile j + 1.
// MFMA waves keep the B fragments of both k-steps of a tile in registers and
// stream the A fragments (A row block i of the next k-step is read as soon as
// its MFMAs of the current one are issued), which fits in 256 VGPRs; the
// scheduling hints interleave one LDS read with a few MFMAs.  LDS is dynamic
// (set at launch) so that the register budget is that of two waves per SIMD.
constexpr int kSpecThreads = 512;

// acc + the sum of a fragment's 8 bf16 values (pairs through the bf16 dot
// product with (1, 1)), in a fixed order
__device__ __forceinline__ float frag_sum(const bf16x8_t& v, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const bf16x2_t p = {v[e], v[e + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(p, one, acc, false);
  }
  return acc;
}

template <class C>
constexpr int spec_smem_bytes() {
  constexpr int pipe = C::STAGES * (C::BM + C::BN) * 64 * 2, tile = C::BM * (C::BN + 4) * 4;
  return pipe > tile ? pipe : tile;
}

template <class C, int LA, int LB, int EPI, int ROLE>
__global__ __launch_bounds__(kSpecThreads, 1) void gemm_spec_kernel(GemmParams g) {
  constexpr int BM = C::BM, BN = C::BN, BK = 64, FM = C::FM, FN = C::FN, S = C::STAGES;
  static_assert(C::BK == 64 && S >= 3 && S <= 5, "specialised kernel: 64-deep k-tiles, 3-5 stages");
  // (A may be the gathered column matrix of a 3x3 convolution)
  using OA = typename std::conditional<LA == LAY_CONV, DmaConvOperand<BM, BK>,
                                       DmaOperand<BM, BK, LA>>::type;
  using OB = typename std::conditional<LB == LAY_CONV_MN, DmaConvMnOperand<BN, BK>,
                                       DmaOperand<BN, BK, LB>>::type;
  constexpr int LPT = OA::PER_WAVE + OB::PER_WAVE;  // loads per loader wave per k-tile
  static_assert(LPT * (S - 1) < 64, "vmcnt range");
  constexpr int RA = LA == LAY_MN ? 2 : 1, RB = LB == LAY_MN || LB == LAY_CONV_MN ? 2 : 1;  // LDS reads per fragment
  constexpr int STAGE = (BM + BN) * BK, TP = BN + 4;
  // Weight gradients can also sum A over k (the bias gradient).  The loader
  // waves do it from the LDS tiles they loaded, with the MFMA fragment reads
  // (lane l: 8 k-values of row l % 16) and bf16 dot products against (1, 1);
  // each wave owns MB blocks of 16 rows.  Tile column tn sums its share of
  // the k-tiles (the tile columns of one tile row see the same A) and writes
  // partial sums for its rows; a second pass adds up the tile columns.
  constexpr bool RS = EPI == EPI_ACC_F32 && LA == LAY_MN;
  constexpr int MB = BM / 64;
  extern __shared__ __attribute__((aligned(1024))) bf16_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, cw = wave & 3;
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  int tm, tn, split;
  grid_tile(tiles_m, tiles_n, BM, BN, &tm, &tn, &split);
  const int m0 = tm * BM, n0 = tn * BN;
  const int z = blockIdx.z, zb = z / g.hdiv, zh = z % g.hdiv;
  int kbeg, kend;
  if (!causal_range(g, m0, n0, BM, BK, &kbeg, &kend)) return;
  if (gridDim.y > 1) {
    kbeg = max(kbeg, split * g.kchunk);
    kend = min(kend, (split + 1) * g.kchunk);
  }
  const int nkt = kend > kbeg ? (kend - kbeg) / BK : 0;
  auto sa = [&](int st) { return smem + st * STAGE; };
  auto sb = [&](int st) { return smem + st * STAGE + BM * BK; };

  floatx4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  const int wm0 = (cw >> 1) * C::WTM, wn0 = (cw & 1) * C::WTN;

  if (wave >= 4) {
    // ---- loader waves
    const bf16_t* A = static_cast<const bf16_t*>(g.A) + zb * g.sAb + zh * g.sAh;
    const bf16_t* B = static_cast<const bf16_t*>(g.B) + zb * g.sBb + zh * g.sBh;
    OA oa;
    OB ob;
    if constexpr (LA == LAY_CONV) oa.init(g, m0, g.M, kbeg, cw, lane);
    else oa.init(g.lda, m0, g.M, kbeg, cw, lane);
    if constexpr (LB == LAY_CONV_MN) ob.init(g, n0, g.N, kbeg, cw, lane);
    else ob.init(g.ldb, n0, g.N, kbeg, cw, lane);
    const int pre = min(S, nkt);
    for (int t = 0; t < pre; ++t) {
      oa.issue(A, t, sa(t), cw);
      ob.issue(B, t, sb(t), cw);
    }
    wait_tiles<LPT, S - 1>(pre - 1);  // tile 0 has landed
    barrier_nofence();
    // row sums (RS): tile t is in LDS from barrier t-1 (the prologue barrier
    // for t = 0) until barrier t; this wave's reads end before it arrives there
    const bool do_rs = RS && g.rowsum;
    const int rs_per = (nkt + tiles_n - 1) / tiles_n;
    const int rs_lo = tn * rs_per, rs_hi = min(nkt, rs_lo + rs_per);  // this tile column's k-tiles
    float rsum[MB];
#pragma unroll
    for (int j = 0; j < MB; ++j) rsum[j] = 0.f;
    auto add_rows = [&](int st) {
#pragma unroll
      for (int j = 0; j < MB; ++j)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) rsum[j] = frag_sum(oa.frag(sa(st), (cw * MB + j) * 16, lane, ks), rsum[j]);
      // the sums exist before the next barrier, so the reads behind them have
      // completed (an lgkmcnt(0) there would also wait for the loads in flight)
#pragma unroll
      for (int j = 0; j < MB; ++j) asm volatile("" ::"v"(rsum[j]));
    };
    if (do_rs && rs_lo <= 0 && 0 < rs_hi) add_rows(0);
    for (int kt = 0; kt < nkt; ++kt) {
      wait_tiles<LPT, S - 2>(min(S - 2, nkt - 2 - kt));  // tile kt + 1 has landed
      barrier_nofence();
      if (do_rs && rs_lo <= kt + 1 && kt + 1 < rs_hi) add_rows((kt + 1) % S);
      // after barrier kt every wave is done with tile kt's stage: refill it
      if (kt + S < nkt) {
        const int st = kt % S;
        oa.issue(A, kt + S, sa(st), cw);
        ob.issue(B, kt + S, sb(st), cw);
      }
    }
    wait_vmcnt<0>();
    if (do_rs) {
      // the four lane groups hold disjoint k-values of the same rows
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        float v = rsum[j];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        const int row = m0 + (cw * MB + j) * 16 + lane;
        if (lane < 16 && row < g.M) {
          float* dst = g.rowsum + int64_t(tn) * g.M + row;
          *dst = g.beta ? *dst + v : v;
        }
      }
    }
  } else {
    // ---- MFMA waves
    OA oa;  // fragment addressing only
    OB ob;
    bf16x8_t fa[FM], fb0[FN], fb1[FN];
    barrier_nofence();
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = oa.frag(sa(0), wm0 + i * 16, lane, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb0[j] = ob.frag(sb(0), wn0 + j * 16, lane, 0);
    constexpr int REST = FM * FN - 1 - FN * RB;
    constexpr int PER_A = REST / FM;
    int s_cur = 0;
    for (int kt = 0; kt < nkt; ++kt) {
      const int s_nxt = s_cur == S - 1 ? 0 : s_cur + 1;
      {  // k-step 0 of tile kt; read k-step 1
        const bf16_t* as = sa(s_cur);
        const bf16_t* bs = sb(s_cur);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb1[j] = ob.frag(bs, wn0 + j * 16, lane, 1);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb0[j], acc[i][j], 0, 0, 0);
          fa[i] = oa.frag(as, wm0 + i * 16, lane, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
        for (int q = 0; q < FN * RB; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
#pragma unroll
        for (int q = 0; q < FM; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x100, RA, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, PER_A, 0);
        }
      }
      // tile kt + 1 has landed; every wave is done reading tile kt's stage
      barrier_lds();
      {  // k-step 1 of tile kt; read k-step 0 of tile kt + 1
        const bf16_t* as = sa(s_nxt);
        const bf16_t* bs = sb(s_nxt);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb0[j] = ob.frag(bs, wn0 + j * 16, lane, 0);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb1[j], acc[i][j], 0, 0, 0);
          fa[i] = oa.frag(as, wm0 + i * 16, lane, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
        for (int q = 0; q < FN * RB; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
#pragma unroll
        for (int q = 0; q < FM; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x100, RA, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, PER_A, 0);
        }
      }
      s_cur = s_nxt;
    }
  }

  // Epilogue through LDS (every load has landed: the loader waves drained
  // theirs before this barrier), then all 8 waves store.
  float* P = gridDim.y > 1 ? g.P + int64_t(split) * g.M * g.N : nullptr;
  const int64_t coff = zb * g.sCb + zh * g.sCh;
  constexpr int CH = BN / 8;
  // Accumulating weight gradients: every old output chunk of this thread is
  // loaded before the first store (a load placed after a store to the output
  // may alias it, so each would wait a full round trip): 2 us less per launch.
  // (The other epilogues keep their per-chunk loads: issuing theirs up front
  // made them 1-5 us slower.)
  constexpr bool kPre = EPI == EPI_ACC_F32;
  constexpr int NPRE = kPre ? BM * CH / kSpecThreads : 1;
  static_assert(!kPre || BM * CH % kSpecThreads == 0, "whole chunks per thread");
  float4 pre[NPRE][2];
  if (kPre && g.beta && !P)
#pragma unroll
    for (int j = 0; j < NPRE; ++j) {
      const int idx = tid + j * kSpecThreads;
      const int row = m0 + idx / CH, col = n0 + (idx % CH) * 8;
      if (row < g.M && col + 8 <= g.N) {
        const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(g.C) + coff +
                                                            int64_t(row) * g.ldc + col);
        pre[j][0] = src[0];
        pre[j][1] = src[1];
      }
    }
  barrier_lds();
  float* tile = reinterpret_cast<float*>(smem);
  if (wave < 4) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          tile[(wm0 + i * 16 + (lane >> 4) * 4 + v) * TP + wn0 + j * 16 + (lane & 15)] = acc[i][j][v];
  }
  barrier_lds();
  if constexpr (kPre) {
    if (g.beta && !P) {
#pragma unroll
      for (int j = 0; j < NPRE; ++j) {
        const int idx = tid + j * kSpecThreads;
        const int r = idx / CH, c = (idx % CH) * 8;
        const int row = m0 + r, col = n0 + c;
        if (row >= g.M || col >= g.N) continue;
        const float4 t0 = *reinterpret_cast<const float4*>(tile + r * TP + c);
        const float4 t1 = *reinterpret_cast<const float4*>(tile + r * TP + c + 4);
        if (col + 8 <= g.N) {
          float4* dst = reinterpret_cast<float4*>(static_cast<float*>(g.C) + coff +
                                                  int64_t(row) * g.ldc + col);
          dst[0] = make_float4(pre[j][0].x + t0.x, pre[j][0].y + t0.y, pre[j][0].z + t0.z,
                               pre[j][0].w + t0.w);
          dst[1] = make_float4(pre[j][1].x + t1.x, pre[j][1].y + t1.y, pre[j][1].z + t1.z,
                               pre[j][1].w + t1.w);
        } else {
          const float a[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
          for (int e = 0; e < 8 && col + e < g.N; ++e) epi_store<bf16_t, EPI>(g, row, col + e, a[e], coff);
        }
      }
      return;
    }
  }
  for (int idx = tid; idx < BM * CH; idx += kSpecThreads) {
    const int r = idx / CH, c = (idx % CH) * 8;
    const int row = m0 + r, col = n0 + c;
    if (row >= g.M || col >= g.N) continue;
    const float4 t0 = *reinterpret_cast<const float4*>(tile + r * TP + c);
    const float4 t1 = *reinterpret_cast<const float4*>(tile + r * TP + c + 4);
    const float a[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
    if (col + 8 <= g.N) {
      epi_store8<EPI>(g, row, col, a, coff, P);
    } else {
      for (int e = 0; e < 8 && col + e < g.N; ++e) {
        if (P) P[int64_t(row) * g.N + col + e] = a[e];
        else epi_store<bf16_t, EPI>(g, row, col + e, a[e], coff);
      }
    }
  }
}

// path 0: direct-to-LDS kernel with configuration DC (the specialised-wave
// kernel for the one-workgroup-per-CU 3-stage configurations); path 1:
// register-staged kernel with tile RC (for k not a multiple of 64).
// Split-K sum, eight consecutive columns per thread with 16-byte accesses:
// the partials are added in split order (0 + p0 + p1 + ..., as the
// per-element kernel does) and the role's epilogue is applied.  For outputs
// whose rows are multiples of 8 elements (with 16-byte aligned pointers).
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce8_kernel(GemmParams g, int splits) {
  const int cpr = g.N / 8;  // 8-column chunks per row
  const int64_t n = int64_t(g.M) * g.N, nch = int64_t(g.M) * cpr;
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x; c < nch; c += stride) {
    const int row = int(c / cpr), col = int(c % cpr) * 8;
    const int64_t e = int64_t(row) * g.N + col;
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < splits; ++p) {
      const float4* src = reinterpret_cast<const float4*>(g.P + int64_t(p) * n + e);
      const float4 v0 = src[0], v1 = src[1];
      a[0] += v0.x; a[1] += v0.y; a[2] += v0.z; a[3] += v0.w;
      a[4] += v1.x; a[5] += v1.y; a[6] += v1.z; a[7] += v1.w;
    }
    epi_store8<EPI>(g, row, col, a, 0, nullptr);
  }
}

inline bool aligned16_ptr(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <class DC, class RC, int LA, int LB, int EPI, int ROLE>
hipError_t launch_bf16(int path, const GemmParams& g, int batch, int splits, hipStream_t s) {
  const int bm = path == 0 ? DC::BM : RC::BM, bn = path == 0 ? DC::BN : RC::BN;
  const int tiles = ((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn);
  if (tiles == 0 || batch == 0) return launch_nothing(s);
  const dim3 grid(tiles, splits, batch);
  const bool one = splits == 1;  // the product is the whole launch
  hipError_t e;
  if ((LA == LAY_CONV || LB == LAY_CONV_MN) && path != 0) {
    return hipErrorInvalidValue;  // the gathered operands exist only on the direct-to-LDS path
  } else if (path == 0) {
    if constexpr (DC::OCC == 1 && DC::BK == 64 && DC::STAGES >= 3) {
      constexpr int smem = spec_smem_bytes<DC>();
      static const hipError_t attr = hipFuncSetAttribute(
          reinterpret_cast<const void*>(&gemm_spec_kernel<DC, LA, LB, EPI, ROLE>),
          hipFuncAttributeMaxDynamicSharedMemorySize, smem);
      if (attr != hipSuccess) return attr;
      e = launch_timed((gemm_spec_kernel<DC, LA, LB, EPI, ROLE>), grid, dim3(kSpecThreads), smem, s,
                       true, one, g);
    } else {
      e = launch_timed((gemm_dma_kernel<DC, LA, LB, EPI, ROLE>), grid, dim3(kThreads), 0, s, true, one, g);
    }
  } else {
    e = launch_timed((gemm_bf16_kernel<RC, LA, LB, EPI, ROLE>), grid, dim3(kThreads), 0, s, true, one, g);
  }
  if (e != hipSuccess || one) return e;
  const int64_t n = int64_t(g.M) * g.N;
  const bool vec = g.N % 8 == 0 && g.ldc % 8 == 0 && g.ldr % 8 == 0 && g.ldu % 8 == 0 &&
                   aligned16_ptr(g.C) && aligned16_ptr(g.P) && (!g.R || aligned16_ptr(g.R)) &&
                   (!g.U || aligned16_ptr(g.U)) && (!g.bias || aligned16_ptr(g.bias));
  if (vec) {
    const int64_t want = (n / 8 + 255) / 256;
    const int blocks = int(want < (int64_t(1) << 30) ? want : (int64_t(1) << 30));
    return launch_timed((splitk_reduce8_kernel<EPI>), dim3(blocks), dim3(256), 0, s, false, true,
                        g, splits);
  }
  const int64_t want = (n + 255) / 256;
  const int blocks = int(want < 4096 ? want : 4096);
  return launch_timed((splitk_reduce_kernel<bf16_t, EPI>), dim3(blocks), dim3(256), 0, s, false,
                      true, g, splits);
}

}  // namespace gp
