// Fused causal / full multi-head attention for bf16 cells (head dim 64 or 128).
//
// Forward, per (sequence, head) and block of 64 queries: stream the key/value
// blocks through LDS, keep the running row maximum and row sum of the
// softmax in registers, and accumulate the output; only the log-sum-exp of
// every query row is saved.  Backward recomputes the probabilities from it:
// one kernel per key block accumulates dK and dV over the query blocks, one
// per query block accumulates dQ over the key blocks, so every sum has a
// fixed order (no atomics) and the result is reproducible.
//
// Scores live in base 2: x = (q . k) * scale * log2(e), p = 2^(x - lse2).
//
// MFMA v_mfma_f32_16x16x32_bf16: A lane l holds row l%16, k 8*(l/16)+e;
// B lane l holds k 8*(l/16)+e of column l%16; C lane l holds rows
// 4*(l/16)+v of column l%16.  A product whose k index runs over keys
// (P.V, dS.K) or queries (P^T.dO, dS^T.Q) takes its A operand straight from
// the C registers of the score product, with k slot 8g+e of lane group g
// standing for row 16*t0 + 4g + e (e < 4) or 16*t1 + 4g + e - 4 (e >= 4) of
// the two 16-row score tiles t0, t1; the B operand is read with the same
// permutation by two transposing LDS reads.
//
// LDS tiles [64 rows][DH] bf16 in 32-byte granules: granule G of row r sits
// at G ^ f(r), f(r) = r & 7 (DH 128) or (r >> 1) & 3 (DH 64).  Both the
// 16-byte row reads and the transposing reads of 16 consecutive rows then
// touch distinct banks within each half wave.
#include "common.hpp"
#include "kernels.hpp"

namespace gp {
namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

constexpr int kBlk = 64;  // queries or keys per block
constexpr float kLog2e = 1.4426950408889634f;

template <int DH>
__device__ __forceinline__ int toff(int r, int col) {
  constexpr int NG = DH / 16;
  const int f = (DH >= 128) ? (r & 7) : ((r >> 1) & 3);
  return r * DH + ((((col >> 4) ^ f) & (NG - 1)) << 4) + (col & 15);
}

__device__ __forceinline__ floatx4_t mfma(bf16x8_t a, bf16x8_t b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 bf16 of row r, columns c8*8 .. c8*8+7 of an LDS tile
template <int DH>
__device__ __forceinline__ bf16x8_t frag_row(const bf16_t* t, int r, int c8) {
  return *reinterpret_cast<const bf16x8_t*>(t + toff<DH>(r, c8 * 8));
}

// B operand over permuted rows: lane group g gets rows rlo+4g .. +3 (slots
// 0-3) and rhi+4g .. +3 (slots 4-7) of column m0 + lane%16.
template <int DH>
__device__ __forceinline__ bf16x8_t frag_tr(const bf16_t* t, int rlo, int rhi, int m0, int lane) {
  const int s = lane & 15, g = lane >> 4;
  const int col = m0 + 4 * (s & 3);
  const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4_t*)(t + toff<DH>(rlo + 4 * g + (s >> 2), col)));
  const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4_t*)(t + toff<DH>(rhi + 4 * g + (s >> 2), col)));
  const short8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// bf16x8 from 8 floats (round to nearest even)
__device__ __forceinline__ bf16x8_t pack8(const float* v) {
  short8_t s;
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = short(f2bf(v[e]));
  return __builtin_bit_cast(bf16x8_t, s);
}

// A 64 x DH tile of a [rows][ld] bf16 matrix, staged through registers.
// Rows >= nrows read as zeros.
template <int DH>
struct TileLoad {
  static constexpr int CPR = DH / 8;                 // 16-byte chunks per row
  static constexpr int PER = kBlk * CPR / 256;       // per thread
  uint4 v[PER];
  __device__ __forceinline__ void load(const bf16_t* base, int64_t ld, int r0, int nrows) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int cid = threadIdx.x + 256 * i;
      const int r = cid / CPR, c = cid % CPR;
      v[i] = make_uint4(0, 0, 0, 0);
      if (r0 + r < nrows) v[i] = *reinterpret_cast<const uint4*>(base + int64_t(r0 + r) * ld + c * 8);
    }
  }
  __device__ __forceinline__ void store(bf16_t* t) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int cid = threadIdx.x + 256 * i;
      const int r = cid / CPR, c = cid % CPR;
      *reinterpret_cast<uint4*>(t + toff<DH>(r, c * 8)) = v[i];
    }
  }
};

// 8 bf16 of global row `row` (zeros past nrows), columns c0 .. c0+7
__device__ __forceinline__ bf16x8_t gfrag(const bf16_t* base, int64_t ld, int row, int nrows, int c0) {
  if (row >= nrows) return __builtin_bit_cast(bf16x8_t, short8_t{0, 0, 0, 0, 0, 0, 0, 0});
  return *reinterpret_cast<const bf16x8_t*>(base + int64_t(row) * ld + c0);
}

// ------------------------------------------------------------------ forward
// grid (query blocks, B*H); qkv [B*S][3D], ctx [B*S][D], lse2 [B*H][S].
template <int DH>
__global__ __launch_bounds__(256) void flash_fwd_kernel(const bf16_t* __restrict__ qkv,
                                                        bf16_t* __restrict__ ctx,
                                                        float* __restrict__ lse2, int S, int H,
                                                        int D, int causal, float sl2) {
  constexpr int KS = DH / 32;   // k steps over the head dimension
  constexpr int DT = DH / 16;   // 16-column output tiles
  __shared__ __attribute__((aligned(16))) bf16_t kt[2][kBlk * DH];
  __shared__ __attribute__((aligned(16))) bf16_t vt[2][kBlk * DH];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, ln = lane & 15;
  const int nqb = (S + kBlk - 1) / kBlk;
  const int qb = nqb - 1 - int(blockIdx.x);  // longest causal rows first
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int64_t ld = 3 * int64_t(D);
  const bf16_t* Qg = qkv + int64_t(b) * S * ld + h * DH;
  const bf16_t* Kg = Qg + D;
  const bf16_t* Vg = Qg + 2 * D;
  const int q = qb * kBlk + w * 16 + ln;  // this lane's query (column of S^T)
  bf16x8_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = gfrag(Qg, ld, q, S, ks * 32 + 8 * g);

  floatx4_t o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int nkb = causal ? min(qb + 1, (S + kBlk - 1) / kBlk) : (S + kBlk - 1) / kBlk;
  TileLoad<DH> lk, lv;
  lk.load(Kg, ld, 0, S);
  lv.load(Vg, ld, 0, S);
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    lk.store(kt[buf]);
    lv.store(vt[buf]);
    __syncthreads();
    if (kb + 1 < nkb) {
      lk.load(Kg, ld, (kb + 1) * kBlk, S);
      lv.load(Vg, ld, (kb + 1) * kBlk, S);
    }
    // S^T tile t: keys 16t + 4g + v, query q
    floatx4_t st[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      st[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        st[t] = mfma(frag_row<DH>(kt[buf], t * 16 + ln, ks * 4 + g), qf[ks], st[t]);
    }
    const int k0 = kb * kBlk;
    const bool full = (k0 + kBlk <= S) && (!causal || k0 + kBlk - 1 <= qb * kBlk);
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float x = st[t][v] * sl2;
        if (!full) {
          const int key = k0 + t * 16 + 4 * g + v;
          if (key >= S || (causal && key > q)) x = -INFINITY;
        }
        st[t][v] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float ls = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float p = exp2f(st[t][v] - m_new);
        st[t][v] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    l_run = l_run * alpha + ls;
    m_run = m_new;
    // rescale the output rows (queries 4g+v of this wave) by their alpha
    float av[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) av[v] = __shfl(alpha, 4 * g + v, 64);
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) o[i][v] *= av[v];
    // O += P V over two 32-key halves
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const float pv[8] = {st[2 * k2][0], st[2 * k2][1], st[2 * k2][2], st[2 * k2][3],
                           st[2 * k2 + 1][0], st[2 * k2 + 1][1], st[2 * k2 + 1][2], st[2 * k2 + 1][3]};
      const bf16x8_t pa = pack8(pv);
#pragma unroll
      for (int i = 0; i < DT; ++i)
        o[i] = mfma(pa, frag_tr<DH>(vt[buf], 32 * k2, 32 * k2 + 16, i * 16, lane), o[i]);
    }
  }
  // normalise and store: lane holds rows (queries) 4g+v, column i*16 + ln
  float lv4[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) lv4[v] = 1.0f / __shfl(l_run, 4 * g + v, 64);
  bf16_t* Cg = ctx + int64_t(b) * S * D + h * DH;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int qr = qb * kBlk + w * 16 + 4 * g + v;
    if (qr < S)
#pragma unroll
      for (int i = 0; i < DT; ++i) Cg[int64_t(qr) * D + i * 16 + ln] = f2bf(o[i][v] * lv4[v]);
  }
  if (g == 0 && q < S) lse2[int64_t(bh) * S + q] = m_run + log2f(l_run);
}

// ------------------------------------------------------------------ backward
// delta[bh][s] = sum_d dO[s][h*DH + d] * O[s][h*DH + d]
template <int DH>
__global__ __launch_bounds__(256) void flash_delta_kernel(const bf16_t* __restrict__ dctx,
                                                          const bf16_t* __restrict__ ctx,
                                                          float* __restrict__ delta, int S, int H,
                                                          int D, int rows) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // (token, head)
  if (i >= rows) return;
  const int t = i / H, h = i % H;
  const int b = t / S, s = t % S;
  const bf16_t* a = dctx + int64_t(t) * D + h * DH;
  const bf16_t* c = ctx + int64_t(t) * D + h * DH;
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < DH; k += 8) {
    float x[8], y[8];
    load8<bf16_t>(a + k, x);
    load8<bf16_t>(c + k, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += x[e] * y[e];
  }
  delta[(int64_t(b) * H + h) * S + s] = acc;
}

// dK, dV for one key block: grid (key blocks, B*H)
template <int DH>
__global__ __launch_bounds__(256) void flash_dkdv_kernel(
    const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ dctx,
    const float* __restrict__ lse2, const float* __restrict__ delta, bf16_t* __restrict__ dqkv,
    int S, int H, int D, int causal, float sl2, float scale) {
  constexpr int KS = DH / 32;
  constexpr int DT = DH / 16;
  __shared__ __attribute__((aligned(16))) bf16_t qt[2][kBlk * DH];
  __shared__ __attribute__((aligned(16))) bf16_t ot[2][kBlk * DH];  // dO
  __shared__ float ls_s[2][kBlk], dl_s[2][kBlk];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, ln = lane & 15;
  const int nb = (S + kBlk - 1) / kBlk;
  const int kbk = int(blockIdx.x);
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int64_t ld = 3 * int64_t(D);
  const bf16_t* Qg = qkv + int64_t(b) * S * ld + h * DH;
  const bf16_t* Kg = Qg + D;
  const bf16_t* Vg = Qg + 2 * D;
  const bf16_t* Og = dctx + int64_t(b) * S * D + h * DH;
  const float* Lg = lse2 + int64_t(bh) * S;
  const float* Dg = delta + int64_t(bh) * S;
  const int key = kbk * kBlk + w * 16 + ln;  // this lane's key (column of S)
  bf16x8_t kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = gfrag(Kg, ld, key, S, ks * 32 + 8 * g);
    vf[ks] = gfrag(Vg, ld, key, S, ks * 32 + 8 * g);
  }
  floatx4_t dk[DT], dv[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) dk[i] = dv[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  const int q_first = causal ? kbk : 0;
  TileLoad<DH> lq, lo;
  float lsv = 0.f, dlv = 0.f;
  auto load_blk = [&](int qb) {
    lq.load(Qg, ld, qb * kBlk, S);
    lo.load(Og, D, qb * kBlk, S);
    if (threadIdx.x < kBlk) {
      const int qq = qb * kBlk + threadIdx.x;
      lsv = qq < S ? Lg[qq] : INFINITY;
      dlv = qq < S ? Dg[qq] : 0.f;
    }
  };
  load_blk(q_first);
  for (int qb = q_first; qb < nb; ++qb) {
    const int buf = (qb - q_first) & 1;
    lq.store(qt[buf]);
    lo.store(ot[buf]);
    if (threadIdx.x < kBlk) {
      ls_s[buf][threadIdx.x] = lsv;
      dl_s[buf][threadIdx.x] = dlv;
    }
    __syncthreads();
    if (qb + 1 < nb) load_blk(qb + 1);
    // S and dP tiles t: rows (queries) 16t + 4g + v, column (key) `key`
    floatx4_t sp[4], dp[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sp[t] = dp[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sp[t] = mfma(frag_row<DH>(qt[buf], t * 16 + ln, ks * 4 + g), kf[ks], sp[t]);
        dp[t] = mfma(frag_row<DH>(ot[buf], t * 16 + ln, ks * 4 + g), vf[ks], dp[t]);
      }
    }
    const int q0 = qb * kBlk;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = t * 16 + 4 * g + v;
        const int qq = q0 + r;
        float p = exp2f(sp[t][v] * sl2 - ls_s[buf][r]);
        if (key >= S || (causal && key > qq)) p = 0.f;
        sp[t][v] = p;                                   // P
        dp[t][v] = p * (dp[t][v] - dl_s[buf][r]);       // dS (unscaled)
      }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const float pv[8] = {sp[2 * k2][0], sp[2 * k2][1], sp[2 * k2][2], sp[2 * k2][3],
                           sp[2 * k2 + 1][0], sp[2 * k2 + 1][1], sp[2 * k2 + 1][2], sp[2 * k2 + 1][3]};
      const float sv[8] = {dp[2 * k2][0], dp[2 * k2][1], dp[2 * k2][2], dp[2 * k2][3],
                           dp[2 * k2 + 1][0], dp[2 * k2 + 1][1], dp[2 * k2 + 1][2], dp[2 * k2 + 1][3]};
      const bf16x8_t pa = pack8(pv), sa = pack8(sv);
#pragma unroll
      for (int i = 0; i < DT; ++i) {
        dv[i] = mfma(pa, frag_tr<DH>(ot[buf], 32 * k2, 32 * k2 + 16, i * 16, lane), dv[i]);
        dk[i] = mfma(sa, frag_tr<DH>(qt[buf], 32 * k2, 32 * k2 + 16, i * 16, lane), dk[i]);
      }
    }
  }
  // lane holds rows (keys) 4g+v of this wave, column i*16 + ln
  bf16_t* dKg = dqkv + int64_t(b) * S * ld + D + h * DH;
  bf16_t* dVg = dKg + D;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int kr = kbk * kBlk + w * 16 + 4 * g + v;
    if (kr < S)
#pragma unroll
      for (int i = 0; i < DT; ++i) {
        dKg[int64_t(kr) * ld + i * 16 + ln] = f2bf(dk[i][v] * scale);
        dVg[int64_t(kr) * ld + i * 16 + ln] = f2bf(dv[i][v]);
      }
  }
}

// dQ for one query block: grid (query blocks, B*H)
template <int DH>
__global__ __launch_bounds__(256) void flash_dq_kernel(
    const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ dctx,
    const float* __restrict__ lse2, const float* __restrict__ delta, bf16_t* __restrict__ dqkv,
    int S, int H, int D, int causal, float sl2, float scale) {
  constexpr int KS = DH / 32;
  constexpr int DT = DH / 16;
  __shared__ __attribute__((aligned(16))) bf16_t kt[2][kBlk * DH];
  __shared__ __attribute__((aligned(16))) bf16_t vt[2][kBlk * DH];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, ln = lane & 15;
  const int nb = (S + kBlk - 1) / kBlk;
  const int qb = nb - 1 - int(blockIdx.x);
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int64_t ld = 3 * int64_t(D);
  const bf16_t* Qg = qkv + int64_t(b) * S * ld + h * DH;
  const bf16_t* Kg = Qg + D;
  const bf16_t* Vg = Qg + 2 * D;
  const bf16_t* Og = dctx + int64_t(b) * S * D + h * DH;
  const int q = qb * kBlk + w * 16 + ln;  // this lane's query (column of S^T)
  bf16x8_t qf[KS], of[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = gfrag(Qg, ld, q, S, ks * 32 + 8 * g);
    of[ks] = gfrag(Og, D, q, S, ks * 32 + 8 * g);
  }
  const float lq = q < S ? lse2[int64_t(bh) * S + q] : INFINITY;
  const float dq_ = q < S ? delta[int64_t(bh) * S + q] : 0.f;
  floatx4_t acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  const int nkb = causal ? min(qb + 1, nb) : nb;
  TileLoad<DH> lk, lv;
  lk.load(Kg, ld, 0, S);
  lv.load(Vg, ld, 0, S);
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    lk.store(kt[buf]);
    lv.store(vt[buf]);
    __syncthreads();
    if (kb + 1 < nkb) {
      lk.load(Kg, ld, (kb + 1) * kBlk, S);
      lv.load(Vg, ld, (kb + 1) * kBlk, S);
    }
    // S^T and dP^T tiles t: rows (keys) 16t + 4g + v, column (query) q
    floatx4_t st[4], dpt[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      st[t] = dpt[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        st[t] = mfma(frag_row<DH>(kt[buf], t * 16 + ln, ks * 4 + g), qf[ks], st[t]);
        dpt[t] = mfma(frag_row<DH>(vt[buf], t * 16 + ln, ks * 4 + g), of[ks], dpt[t]);
      }
    }
    const int k0 = kb * kBlk;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key = k0 + t * 16 + 4 * g + v;
        float p = exp2f(st[t][v] * sl2 - lq);
        if (key >= S || (causal && key > q)) p = 0.f;
        st[t][v] = p * (dpt[t][v] - dq_);   // dS^T (unscaled)
      }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const float sv[8] = {st[2 * k2][0], st[2 * k2][1], st[2 * k2][2], st[2 * k2][3],
                           st[2 * k2 + 1][0], st[2 * k2 + 1][1], st[2 * k2 + 1][2], st[2 * k2 + 1][3]};
      const bf16x8_t sa = pack8(sv);
#pragma unroll
      for (int i = 0; i < DT; ++i)
        acc[i] = mfma(sa, frag_tr<DH>(kt[buf], 32 * k2, 32 * k2 + 16, i * 16, lane), acc[i]);
    }
  }
  bf16_t* dQg = dqkv + int64_t(b) * S * ld + h * DH;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int qr = qb * kBlk + w * 16 + 4 * g + v;
    if (qr < S)
#pragma unroll
      for (int i = 0; i < DT; ++i) dQg[int64_t(qr) * ld + i * 16 + ln] = f2bf(acc[i][v] * scale);
  }
}

}  // namespace

bool flash_ok(bool bf16, int dh) { return bf16 && (dh == 64 || dh == 128); }

hipError_t flash_fwd(const void* qkv, void* ctx, float* lse2, int B, int H, int S, int D,
                     int causal, hipStream_t s) {
  const int dh = D / H;
  const float sl2 = kLog2e / sqrtf(float(dh));
  const dim3 grid((S + kBlk - 1) / kBlk, B * H);
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  const bf16_t* q = static_cast<const bf16_t*>(qkv);
  bf16_t* c = static_cast<bf16_t*>(ctx);
  if (dh == 128)
    hipLaunchKernelGGL(flash_fwd_kernel<128>, grid, dim3(256), 0, s, q, c, lse2, S, H, D, causal, sl2);
  else if (dh == 64)
    hipLaunchKernelGGL(flash_fwd_kernel<64>, grid, dim3(256), 0, s, q, c, lse2, S, H, D, causal, sl2);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t flash_bwd(const void* qkv, const void* ctx, const void* dctx, const float* lse2,
                     float* delta, void* dqkv, int B, int H, int S, int D, int causal,
                     hipStream_t s, int stage) {
  const int dh = D / H;
  const float scale = 1.0f / sqrtf(float(dh));
  const float sl2 = kLog2e * scale;
  const dim3 grid((S + kBlk - 1) / kBlk, B * H);
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  const bf16_t* q = static_cast<const bf16_t*>(qkv);
  const bf16_t* o = static_cast<const bf16_t*>(ctx);
  const bf16_t* dO = static_cast<const bf16_t*>(dctx);
  bf16_t* dq = static_cast<bf16_t*>(dqkv);
  const int rows = B * S * H;
  if (dh != 128 && dh != 64) return hipErrorInvalidValue;
  if (stage == 0) {
    if (dh == 128)
      hipLaunchKernelGGL(flash_delta_kernel<128>, dim3((rows + 255) / 256), dim3(256), 0, s, dO, o,
                         delta, S, H, D, rows);
    else
      hipLaunchKernelGGL(flash_delta_kernel<64>, dim3((rows + 255) / 256), dim3(256), 0, s, dO, o,
                         delta, S, H, D, rows);
  } else if (stage == 1) {
    if (dh == 128)
      hipLaunchKernelGGL(flash_dkdv_kernel<128>, grid, dim3(256), 0, s, q, dO, lse2, delta, dq, S, H,
                         D, causal, sl2, scale);
    else
      hipLaunchKernelGGL(flash_dkdv_kernel<64>, grid, dim3(256), 0, s, q, dO, lse2, delta, dq, S, H,
                         D, causal, sl2, scale);
  } else {
    if (dh == 128)
      hipLaunchKernelGGL(flash_dq_kernel<128>, grid, dim3(256), 0, s, q, dO, lse2, delta, dq, S, H, D,
                         causal, sl2, scale);
    else
      hipLaunchKernelGGL(flash_dq_kernel<64>, grid, dim3(256), 0, s, q, dO, lse2, delta, dq, S, H, D,
                         causal, sl2, scale);
  }
  return hipGetLastError();
}

}  // namespace gp
