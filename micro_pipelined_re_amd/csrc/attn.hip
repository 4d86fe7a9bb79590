// Fused causal / full multi-head attention for bf16 cells (head dim 64 or 128).
//
// Forward, per (sequence, head) and block of 64 queries: stream the key/value
// blocks through LDS, keep the running row maximum and row sum of the
// softmax in registers, and accumulate the output (two wave groups, each
// over half of the key blocks, combined at the end); only the log-sum-exp of
// every query row is saved.  Backward recomputes the probabilities from it:
// one kernel per query block accumulates dQ over the key blocks (and first
// computes the rows' sums of dO * O), then one kernel per key block
// accumulates dK and dV over the query blocks, so every sum has a fixed
// order (no atomics) and the result is reproducible.
//
// Scores live in base 2: x = (q . k) * scale * log2(e), p = 2^(x - lse2).
// With logit clipping (CLIP) the raw product q . k is first limited to
// [-craw, craw], craw = threshold / scale, and in the backward a clipped
// score passes no gradient (d clip(s)/ds = 0 for |s| > threshold).
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

// bf16x8 from 8 floats, round to nearest even (v_cvt_pk_bf16_f32 per pair)
__device__ __forceinline__ bf16x8_t pack8(const float* v) {
  typedef float float2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  bf16x8_t r;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const bf16x2v h = __builtin_convertvector((float2v{v[e], v[e + 1]}), bf16x2v);
    r[e] = h[0];
    r[e + 1] = h[1];
  }
  return r;
}

// 2^x without the library's range reduction (one v_exp_f32): the arguments
// here are at most 0 and results below the fp32 normal range only scale
// probabilities that are negligible next to the row's largest one (1).
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

// This thread's 16-byte chunks of a 64 x DH tile of a [rows][ld] bf16
// matrix, held in registers (256 threads of one wave group: chunk t + 256 i
// is column chunk (t + 256 i) % CPR of row (t + 256 i) / CPR).  Rows at or
// past nrows read row nrows - 1: the loads need no branch, so the compiler
// keeps an exact count of the loads in flight and does not wait for them
// before their first use (rows past the sequence carry a zero probability
// wherever these values enter).
template <int DH>
struct TileRows {
  static constexpr int CPR = DH / 8;                 // 16-byte chunks per row
  static constexpr int PER = kBlk * CPR / 256;       // per thread
  uint4 v[PER];
  __device__ __forceinline__ void load(const bf16_t* base, int64_t ld, int r0, int nrows, int t) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int cid = t + 256 * i;
      const int r = min(r0 + cid / CPR, nrows - 1), c = cid % CPR;
      v[i] = *reinterpret_cast<const uint4*>(base + int64_t(r) * ld + c * 8);
    }
  }
};

// An integer the optimizer cannot look into (an empty asm that may change it).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Per-lane byte offsets of the fragment reads inside a 64 x DH tile.  With
// them every read in a loop is tile + offset + constant: the compiler then
// still knows which LDS variable the read touches (it follows only a few
// address steps), so a read of one buffer does not wait for the loads
// streaming into the other.  row[ks]: frag_row(t * 16 + ln, ks * 4 + g) at
// row[ks] + 32 t DH bytes.  tr[i]: the transposing reads of frag_tr(rlo,
// rhi, 16 i) at tr[i] + 2 rlo DH and tr[i] + 2 rhi DH bytes (rlo, rhi
// multiples of 8, where the swizzle of a row repeats).
template <int DH>
struct FragOffsets {
  static constexpr int KS = DH / 32, DT = DH / 16;
  int row[KS], tr[DT];
  __device__ __forceinline__ void init(int lane) {
    const int g = lane >> 4, s = lane & 15;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) row[ks] = opaque(2 * toff<DH>(s, (ks * 4 + g) * 8));
#pragma unroll
    for (int i = 0; i < DT; ++i) tr[i] = opaque(2 * toff<DH>(4 * g + (s >> 2), i * 16 + 4 * (s & 3)));
  }
};

template <int DH>
__device__ __forceinline__ bf16x8_t frag_row_at(const bf16_t* tile, int off, int t) {
  return *reinterpret_cast<const bf16x8_t*>(reinterpret_cast<const char*>(tile) + off + 32 * t * DH);
}

template <int DH>
__device__ __forceinline__ bf16x8_t frag_tr_at(const bf16_t* tile, int off, int rlo, int rhi) {
  const char* p = reinterpret_cast<const char*>(tile) + off;
  const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p + 2 * rlo * DH));
  const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p + 2 * rhi * DH));
  const short8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// s_waitcnt vmcnt(0), the other counters left alone (gfx9 encoding).  Loads
// guarded by a branch leave the compiler unsure how many are in flight, so
// its first use of a register loaded before a loop waits for every load,
// the loop's own prefetch of the next block included; waiting once for the
// loads issued before the loop clears them from that count.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// A wave group's share of a 64 x DH tile of a [rows][ld] bf16 matrix loaded
// straight into LDS (global_load_lds_dwordx4, no registers in between).
// Instruction i of group wave wl fills 1 KB of the tile: its 64 lanes write
// consecutive 16-byte chunks, i.e. RPI whole rows, lane l chunk position
// l % CPR of row l / CPR.  Each lane fetches the chunk of global columns
// that the tile's granule swizzle places at that position.  Rows at or past
// nrows read row nrows - 1 (valid memory): keys past the sequence get a
// masked score and a zero probability, so their finite values never count.
template <int DH>
struct TileDma {
  static constexpr int CPR = DH / 8;           // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;         // rows per instruction
  static constexpr int IPW = kBlk / RPI / 4;   // instructions per wave and tile
  static constexpr int NG = DH / 16;           // 32-byte granules per row
  int row[IPW], col[IPW];
  uint32_t off[IPW];  // byte offset of the lane's chunk from the tile's first row
  int64_t ld;         // row stride (elements) of the matrices this loader reads
  __device__ __forceinline__ void init(int wl, int lane, int64_t ld_) {
    ld = ld_;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int r = (wl * IPW + i) * RPI + lane / CPR, pc = lane % CPR;
      const int f = (DH >= 128) ? (r & 7) : ((r >> 1) & 3);
      row[i] = r;
      col[i] = ((((pc >> 1) ^ f) & (NG - 1)) << 4) + (pc & 1) * 8;
      off[i] = uint32_t(r * int(ld_) + col[i]) * 2u;
    }
  }
  // rows r0 .. r0+63 of base (row stride ld); wl must be wave-uniform (the
  // LDS address of a load is)
  __device__ __forceinline__ void load(const bf16_t* base, int r0, int nrows, bf16_t* tile,
                                       int wl) const {
    if (r0 + kBlk <= nrows) {
      const char* b0 = reinterpret_cast<const char*>(base + int64_t(r0) * ld);
#pragma unroll
      for (int i = 0; i < IPW; ++i)
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(b0 + off[i]),
                                         (lds_void_t*)(tile + (wl * IPW + i) * 512), 16, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int r = min(r0 + row[i], nrows - 1);
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(base + int64_t(r) * ld + col[i]),
                                         (lds_void_t*)(tile + (wl * IPW + i) * 512), 16, 0, 0);
      }
    }
  }
};

// 8 bf16 of global row `row` (zeros past nrows), columns c0 .. c0+7
__device__ __forceinline__ bf16x8_t gfrag(const bf16_t* base, int64_t ld, int row, int nrows, int c0) {
  if (row >= nrows) return __builtin_bit_cast(bf16x8_t, short8_t{0, 0, 0, 0, 0, 0, 0, 0});
  return *reinterpret_cast<const bf16x8_t*>(base + int64_t(row) * ld + c0);
}

// Every kernel below runs 8 waves in two groups of 4 that split the blocks
// of its sequential loop: group 0 takes blocks 0, 2, 4, ... of the range,
// group 1 blocks 1, 3, 5, ...  Each group keeps its own partial result in
// registers; at the end group 1 hands its partial to group 0 through LDS
// and group 0 combines the two (group 0's + group 1's, in that order).  With
// one (sequence, head, 64-row block) per workgroup a single group would give
// each SIMD one wave with every latency of its dependent chain exposed; two
// groups double the waves per SIMD and halve the chain.  Both groups run the
// same number of iterations (a group without a block in the last one only
// joins the barrier), so every barrier is reached by all 512 threads.
constexpr int kGroups = 2;

// LDS of the kernels (static, declared in each kernel): two tile buffers,
// each [group][2 tiles] bf16, and for the dK/dV blocks two [group][2][64]
// float row-statistics buffers.  Each buffer is a variable of its own (see
// FragOffsets).
template <int DH>
constexpr int attn_tile_elems() { return kBlk * DH; }

// ------------------------------------------------------------------ forward
// grid (B*H, query blocks); qkv [B*S][3D], ctx [B*S][D], lse2 [B*H][S].
//
// The key/value tiles go straight from memory into LDS, one block ahead:
// while a group computes on one buffer, its next tiles stream into the
// other.  The two buffers are separate LDS variables and the loop body is
// written out once per buffer, so the compiler can see that the reads of
// one buffer do not depend on the loads into the other (with one array and
// a computed buffer index it waits for every load before the first read).
template <int DH, bool CLIP>
__global__ __launch_bounds__(512) void flash_fwd_kernel(const bf16_t* __restrict__ qkv,
                                                        bf16_t* __restrict__ ctx,
                                                        float* __restrict__ lse2, int S, int H,
                                                        int D, int causal, float sl2, float craw) {
  constexpr int KS = DH / 32;   // k steps over the head dimension
  constexpr int DT = DH / 16;   // 16-column output tiles
  constexpr int TE = attn_tile_elems<DH>();
  // [group][K, V] tiles of buffer 0 and of buffer 1
  __shared__ __attribute__((aligned(16))) bf16_t buf0[kGroups * 2 * TE];
  __shared__ __attribute__((aligned(16))) bf16_t buf1[kGroups * 2 * TE];
  const int lane = threadIdx.x & 63, g = lane >> 4, ln = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int grp = w >> 2, wl = w & 3;
  const int nqb = (S + kBlk - 1) / kBlk;
  const int qb = nqb - 1 - int(blockIdx.y);  // longest causal rows first
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int64_t ld = 3 * int64_t(D);
  const bf16_t* Qg = qkv + int64_t(b) * S * ld + h * DH;
  const bf16_t* Kg = Qg + D;
  const bf16_t* Vg = Qg + 2 * D;
  const int q = qb * kBlk + wl * 16 + ln;  // this lane's query (column of S^T)
  const int nkb = causal ? min(qb + 1, (S + kBlk - 1) / kBlk) : (S + kBlk - 1) / kBlk;
  const int iters = (nkb + kGroups - 1) / kGroups;
  // the first key/value tiles are requested before the queries, so the two
  // memory round trips overlap
  TileDma<DH> dm;
  dm.init(wl, lane, ld);
  if (grp < nkb) {
    dm.load(Kg, grp * kBlk, S, buf0 + grp * 2 * TE, wl);
    dm.load(Vg, grp * kBlk, S, buf0 + grp * 2 * TE + TE, wl);
  }
  bf16x8_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = gfrag(Qg, ld, q, S, ks * 32 + 8 * g);

  floatx4_t o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  // iteration `it` on this group's tiles in `cur`, the next ones into `nxt`
  auto step = [&](int it, bf16_t* cur, bf16_t* nxt) __attribute__((always_inline)) {
    const int kb = kGroups * it + grp;
    const bf16_t* kt = cur;
    const bf16_t* vt = cur + TE;
    // this wave's share of the tiles has landed; after the barrier every
    // share has, and every wave is done with the other buffer
    wait_vm_all();
    __syncthreads();
    const bool more = kb + kGroups < nkb;
    if (kb >= nkb) return;
    // S^T tile t: keys 16t + 4g + v, query q.  Every LDS read of the block
    // is issued before the first MFMA (otherwise each MFMA waits for its own
    // read's round trip), and before the next tiles are requested: the
    // transposing reads carry no alias information, so one issued after the
    // request would wait for it.
    floatx4_t st[4];
    bf16x8_t kfr[4][KS], vfr[DT], vfr1[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) vfr[i] = frag_tr<DH>(vt, 0, 16, i * 16, lane);
#pragma unroll
    for (int i = 0; i < DT; ++i) vfr1[i] = frag_tr<DH>(vt, 32, 48, i * 16, lane);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kfr[t][ks] = frag_row<DH>(kt, t * 16 + ln, ks * 4 + g);
    if (more) {
      dm.load(Kg, (kb + kGroups) * kBlk, S, nxt, wl);
      dm.load(Vg, (kb + kGroups) * kBlk, S, nxt + TE, wl);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) st[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int t = 0; t < 4; ++t) st[t] = mfma(kfr[t][ks], qf[ks], st[t]);
    if constexpr (CLIP)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) st[t][v] = fminf(fmaxf(st[t][v], -craw), craw);
    const int k0 = kb * kBlk;
    const bool full = (k0 + kBlk <= S) && (!causal || k0 + kBlk - 1 <= qb * kBlk);
    if (!full)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int key = k0 + t * 16 + 4 * g + v;
          if (key >= S || (causal && key > q)) st[t][v] = -INFINITY;
        }
    // the maximum of the raw scores times the (positive) scale is the
    // maximum of the scaled scores
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) mx = fmaxf(mx, st[t][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // every visited block holds an unmasked key of every row (its first key
    // is below S and, causally, at most the row's query), so m_new is finite
    const float m_new = fmaxf(m_run, mx * sl2);
    const float alpha = exp2_raw(m_run - m_new);
    float ls = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float p = exp2_raw(fmaf(st[t][v], sl2, -m_new));
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
    // O += P V over the two 32-key halves
    const float pv0[8] = {st[0][0], st[0][1], st[0][2], st[0][3], st[1][0], st[1][1], st[1][2], st[1][3]};
    const float pv1[8] = {st[2][0], st[2][1], st[2][2], st[2][3], st[3][0], st[3][1], st[3][2], st[3][3]};
    const bf16x8_t pa0 = pack8(pv0), pa1 = pack8(pv1);
#pragma unroll
    for (int i = 0; i < DT; ++i) o[i] = mfma(pa0, vfr[i], o[i]);
#pragma unroll
    for (int i = 0; i < DT; ++i) o[i] = mfma(pa1, vfr1[i], o[i]);
  };
  for (int it = 0; it < iters; it += 2) {
    step(it, buf0 + grp * 2 * TE, buf1 + grp * 2 * TE);
    if (it + 1 < iters) step(it + 1, buf1 + grp * 2 * TE, buf0 + grp * 2 * TE);
  }
  // combine the groups: per wave slot [DT*4][64] group 1's output, then
  // m[group][16], l[group][16] of the wave's 16 queries
  __syncthreads();
  float* slot = reinterpret_cast<float*>(buf0) + wl * (DT * 256 + 64);
  float* stat = slot + DT * 256;
  if (grp == 1)
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) slot[(i * 4 + v) * 64 + lane] = o[i][v];
  if (g == 0) {
    stat[grp * 16 + ln] = m_run;
    stat[32 + grp * 16 + ln] = l_run;
  }
  __syncthreads();
  if (grp != 0) return;
  // rows (queries) 4g+v: the weights of the two partial outputs
  float f0[4], f1[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = 4 * g + v;
    const float a = stat[r], c = stat[16 + r];
    const float mm = fmaxf(a, c);
    const float e0 = exp2f(a - mm), e1 = exp2f(c - mm);
    const float inv = 1.0f / (stat[32 + r] * e0 + stat[48 + r] * e1);
    f0[v] = e0 * inv;
    f1[v] = e1 * inv;
  }
  bf16_t* Cg = ctx + int64_t(b) * S * D + h * DH;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int qr = qb * kBlk + wl * 16 + 4 * g + v;
    if (qr < S)
#pragma unroll
      for (int i = 0; i < DT; ++i)
        Cg[int64_t(qr) * D + i * 16 + ln] =
            f2bf(o[i][v] * f0[v] + slot[(i * 4 + v) * 64 + lane] * f1[v]);
  }
  if (g == 0 && q < S) {
    const float a = stat[ln], c = stat[16 + ln];
    const float mm = fmaxf(a, c);
    lse2[int64_t(bh) * S + q] = mm + log2f(stat[32 + ln] * exp2f(a - mm) + stat[48 + ln] * exp2f(c - mm));
  }
}

// ------------------------------------------------------------------ backward
// The tiles a block's loop visits go straight from memory into LDS, one
// block ahead, into the buffer the group is not reading (as in the forward);
// the loop body is written out once per buffer.

// dK, dV for key block kbk of (sequence, head) bh; the groups split the
// query blocks, and each computes the row sums delta = rowsum(dO * O) of the
// query blocks it visits from dO and O rows it holds in registers.
template <int DH, bool CLIP>
__device__ __forceinline__ void flash_dkdv_body(
    const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ ctx,
    const bf16_t* __restrict__ dctx, const float* __restrict__ lse2, bf16_t* __restrict__ dqkv,
    int S, int H, int D, int causal, float sl2, float scale, float craw, int bh, int kbk,
    bf16_t* buf0, bf16_t* buf1, float* sta0, float* sta1) {
  constexpr int KS = DH / 32;
  constexpr int DT = DH / 16;
  constexpr int TE = attn_tile_elems<DH>();
  const int lane = threadIdx.x & 63, g = lane >> 4, ln = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int grp = w >> 2, wl = w & 3, gt = threadIdx.x & 255;
  const int nb = (S + kBlk - 1) / kBlk;
  const int b = bh / H, h = bh % H;
  const int64_t ld = 3 * int64_t(D);
  const bf16_t* Qg = qkv + int64_t(b) * S * ld + h * DH;
  const bf16_t* Kg = Qg + D;
  const bf16_t* Vg = Qg + 2 * D;
  const bf16_t* Og = dctx + int64_t(b) * S * D + h * DH;
  const float* Lg = lse2 + int64_t(bh) * S;
  const bf16_t* Cg = ctx + int64_t(b) * S * D + h * DH;
  const int key = kbk * kBlk + wl * 16 + ln;  // this lane's key (column of S)
  const int q_first = causal ? kbk : 0;
  const int nqb = nb - q_first;
  const int iters = (nqb + kGroups - 1) / kGroups;
  TileDma<DH> dmq, dmo;  // Q (row stride 3D) and dO (row stride D) tiles
  dmq.init(wl, lane, ld);
  dmo.init(wl, lane, D);
  TileRows<DH> ro, rc;  // dO and O rows of a query block (for delta)
  float lsv = 0.f;      // lse of row gt of the block (wave 0 of each group)
  // requests query block qb: Q and dO tiles into `tiles`, dO, O rows and the
  // block's lse values into registers
  auto request = [&](int qb, bf16_t* tiles) __attribute__((always_inline)) {
    dmq.load(Qg, qb * kBlk, S, tiles, wl);
    dmo.load(Og, qb * kBlk, S, tiles + TE, wl);
    ro.load(Og, D, qb * kBlk, S, gt);
    rc.load(Cg, D, qb * kBlk, S, gt);
    if (wl == 0) lsv = Lg[min(qb * kBlk + gt, S - 1)];
  };
  if (grp < nqb) request(q_first + grp, buf0 + grp * 2 * TE);
  bf16x8_t kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = gfrag(Kg, ld, key, S, ks * 32 + 8 * g);
    vf[ks] = gfrag(Vg, ld, key, S, ks * 32 + 8 * g);
  }
  FragOffsets<DH> fo;
  fo.init(lane);
  floatx4_t dk[DT], dv[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) dk[i] = dv[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  auto step = [&](int it, bf16_t* cur, bf16_t* nxt, float* ls_s) __attribute__((always_inline)) {
    const int qi = kGroups * it + grp;  // index into this key block's query blocks
    const bool have = qi < nqb;
    const int qb = q_first + qi;
    const bf16_t* qt = cur;
    const bf16_t* ot = cur + TE;
    float* dl_s = ls_s + kBlk;
    wait_vm_all();  // this wave's requests for the block have landed
    if (have) {
      if (wl == 0) ls_s[gt] = qb * kBlk + gt < S ? lsv : INFINITY;
      // delta = rowsum(dO * O) of the block's rows: chunk i of this thread is
      // 8 columns of row (gt + 256 i) / CPR, the CPR consecutive threads of a
      // row add their dot products in a fixed butterfly
      constexpr int CPR = TileRows<DH>::CPR;
#pragma unroll
      for (int i = 0; i < TileRows<DH>::PER; ++i) {
        const uint32_t av[4] = {ro.v[i].x, ro.v[i].y, ro.v[i].z, ro.v[i].w};
        const uint32_t cv[4] = {rc.v[i].x, rc.v[i].y, rc.v[i].z, rc.v[i].w};
        float dsum = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dsum = fmaf(__uint_as_float(av[e] << 16), __uint_as_float(cv[e] << 16), dsum);
          dsum = fmaf(__uint_as_float(av[e] & 0xffff0000u), __uint_as_float(cv[e] & 0xffff0000u), dsum);
        }
#pragma unroll
        for (int m = CPR / 2; m > 0; m >>= 1) dsum += __shfl_xor(dsum, m, 64);
        if (gt % CPR == 0) dl_s[(gt + 256 * i) / CPR] = dsum;
      }
    }
    __syncthreads();
    if (qi + kGroups < nqb) request(qb + kGroups, nxt);
    if (!have) return;
    // S and dP tiles t: rows (queries) 16t + 4g + v, column (key) `key`
    floatx4_t sp[4], dp[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sp[t] = dp[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sp[t] = mfma(frag_row_at<DH>(qt, fo.row[ks], t), kf[ks], sp[t]);
        dp[t] = mfma(frag_row_at<DH>(ot, fo.row[ks], t), vf[ks], dp[t]);
      }
    }
    const int q0 = qb * kBlk;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = t * 16 + 4 * g + v;
        const int qq = q0 + r;
        const float s0 = sp[t][v];
        float p = exp2_raw(fmaf(CLIP ? fminf(fmaxf(s0, -craw), craw) : s0, sl2, -ls_s[r]));
        if (key >= S || (causal && key > qq)) p = 0.f;
        sp[t][v] = p;                                   // P
        dp[t][v] = p * (dp[t][v] - dl_s[r]);            // dS (unscaled)
        if (CLIP && !(fabsf(s0) <= craw)) dp[t][v] = 0.f;
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
        dv[i] = mfma(pa, frag_tr_at<DH>(ot, fo.tr[i], 32 * k2, 32 * k2 + 16), dv[i]);
        dk[i] = mfma(sa, frag_tr_at<DH>(qt, fo.tr[i], 32 * k2, 32 * k2 + 16), dk[i]);
      }
    }
  };
  for (int it = 0; it < iters; it += 2) {
    step(it, buf0 + grp * 2 * TE, buf1 + grp * 2 * TE, sta0 + grp * 2 * kBlk);
    if (it + 1 < iters) step(it + 1, buf1 + grp * 2 * TE, buf0 + grp * 2 * TE, sta1 + grp * 2 * kBlk);
  }
  // combine: group 1's dK, dV through LDS (per wave [2][DT*4][64]), added to group 0's
  __syncthreads();
  float* slot = reinterpret_cast<float*>(buf0) + wl * (2 * DT * 256);
  if (grp == 1)
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        slot[(i * 4 + v) * 64 + lane] = dk[i][v];
        slot[DT * 256 + (i * 4 + v) * 64 + lane] = dv[i][v];
      }
  __syncthreads();
  if (grp != 0) return;
  // lane holds rows (keys) 4g+v of this wave, column i*16 + ln
  bf16_t* dKg = dqkv + int64_t(b) * S * ld + D + h * DH;
  bf16_t* dVg = dKg + D;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int kr = kbk * kBlk + wl * 16 + 4 * g + v;
    if (kr < S)
#pragma unroll
      for (int i = 0; i < DT; ++i) {
        const float k1 = slot[(i * 4 + v) * 64 + lane], v1 = slot[DT * 256 + (i * 4 + v) * 64 + lane];
        dKg[int64_t(kr) * ld + i * 16 + ln] = f2bf((dk[i][v] + k1) * scale);
        dVg[int64_t(kr) * ld + i * 16 + ln] = f2bf(dv[i][v] + v1);
      }
  }
}

// dQ for query block qb of (sequence, head) bh; the groups split the key
// blocks.  Each computes the block's row sums delta = rowsum(dO * O) itself.
template <int DH, bool CLIP>
__device__ __forceinline__ void flash_dq_body(
    const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ ctx,
    const bf16_t* __restrict__ dctx, const float* __restrict__ lse2, bf16_t* __restrict__ dqkv,
    int S, int H, int D, int causal, float sl2, float scale, float craw, int bh, int qb,
    bf16_t* buf0, bf16_t* buf1) {
  constexpr int KS = DH / 32;
  constexpr int DT = DH / 16;
  constexpr int TE = attn_tile_elems<DH>();
  const int lane = threadIdx.x & 63, g = lane >> 4, ln = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int grp = w >> 2, wl = w & 3;
  const int nb = (S + kBlk - 1) / kBlk;
  const int b = bh / H, h = bh % H;
  const int64_t ld = 3 * int64_t(D);
  const bf16_t* Qg = qkv + int64_t(b) * S * ld + h * DH;
  const bf16_t* Kg = Qg + D;
  const bf16_t* Vg = Qg + 2 * D;
  const bf16_t* Og = dctx + int64_t(b) * S * D + h * DH;
  const int q = qb * kBlk + wl * 16 + ln;  // this lane's query (column of S^T)
  const int nkb = causal ? min(qb + 1, nb) : nb;
  const int iters = (nkb + kGroups - 1) / kGroups;
  TileDma<DH> dm;
  dm.init(wl, lane, ld);
  if (grp < nkb) {
    dm.load(Kg, grp * kBlk, S, buf0 + grp * 2 * TE, wl);
    dm.load(Vg, grp * kBlk, S, buf0 + grp * 2 * TE + TE, wl);
  }
  bf16x8_t qf[KS], of[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = gfrag(Qg, ld, q, S, ks * 32 + 8 * g);
    of[ks] = gfrag(Og, D, q, S, ks * 32 + 8 * g);
  }
  const float lq = q < S ? lse2[int64_t(bh) * S + q] : INFINITY;
  float dq_ = 0.f;  // delta of query q: each lane a 32-column share, the four lane groups added
  {
    const bf16_t* Cg = ctx + int64_t(b) * S * D + h * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8_t o = gfrag(Cg, D, q, S, ks * 32 + 8 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) dq_ = fmaf(float(of[ks][e]), float(o[e]), dq_);
    }
    dq_ += __shfl_xor(dq_, 16, 64);
    dq_ += __shfl_xor(dq_, 32, 64);
  }
  FragOffsets<DH> fo;
  fo.init(lane);
  floatx4_t acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  auto step = [&](int it, bf16_t* cur, bf16_t* nxt) __attribute__((always_inline)) {
    const int kb = kGroups * it + grp;
    const bf16_t* kt = cur;
    const bf16_t* vt = cur + TE;
    wait_vm_all();  // this wave's share of the tiles has landed
    __syncthreads();
    if (kb + kGroups < nkb) {
      dm.load(Kg, (kb + kGroups) * kBlk, S, nxt, wl);
      dm.load(Vg, (kb + kGroups) * kBlk, S, nxt + TE, wl);
    }
    if (kb >= nkb) return;
    // S^T and dP^T tiles t: rows (keys) 16t + 4g + v, column (query) q
    floatx4_t st[4], dpt[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      st[t] = dpt[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        st[t] = mfma(frag_row_at<DH>(kt, fo.row[ks], t), qf[ks], st[t]);
        dpt[t] = mfma(frag_row_at<DH>(vt, fo.row[ks], t), of[ks], dpt[t]);
      }
    }
    const int k0 = kb * kBlk;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key = k0 + t * 16 + 4 * g + v;
        const float s0 = st[t][v];
        float p = exp2_raw(fmaf(CLIP ? fminf(fmaxf(s0, -craw), craw) : s0, sl2, -lq));
        if (key >= S || (causal && key > q)) p = 0.f;
        st[t][v] = p * (dpt[t][v] - dq_);   // dS^T (unscaled)
        if (CLIP && !(fabsf(s0) <= craw)) st[t][v] = 0.f;
      }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const float sv[8] = {st[2 * k2][0], st[2 * k2][1], st[2 * k2][2], st[2 * k2][3],
                           st[2 * k2 + 1][0], st[2 * k2 + 1][1], st[2 * k2 + 1][2], st[2 * k2 + 1][3]};
      const bf16x8_t sa = pack8(sv);
#pragma unroll
      for (int i = 0; i < DT; ++i)
        acc[i] = mfma(sa, frag_tr_at<DH>(kt, fo.tr[i], 32 * k2, 32 * k2 + 16), acc[i]);
    }
  };
  for (int it = 0; it < iters; it += 2) {
    step(it, buf0 + grp * 2 * TE, buf1 + grp * 2 * TE);
    if (it + 1 < iters) step(it + 1, buf1 + grp * 2 * TE, buf0 + grp * 2 * TE);
  }
  // combine: group 1's dQ through LDS (per wave [DT*4][64]), added to group 0's
  __syncthreads();
  float* slot = reinterpret_cast<float*>(buf0) + wl * (DT * 256);
  if (grp == 1)
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) slot[(i * 4 + v) * 64 + lane] = acc[i][v];
  __syncthreads();
  if (grp != 0) return;
  bf16_t* dQg = dqkv + int64_t(b) * S * ld + h * DH;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int qr = qb * kBlk + wl * 16 + 4 * g + v;
    if (qr < S)
#pragma unroll
      for (int i = 0; i < DT; ++i)
        dQg[int64_t(qr) * ld + i * 16 + ln] = f2bf((acc[i][v] + slot[(i * 4 + v) * 64 + lane]) * scale);
  }
}

// The backward of the attention in one launch: grid (B*H, 2 * blocks); y <
// blocks: dQ of query block blocks-1-y (longest causal rows first), else dK /
// dV of key block y-blocks (key block 0, the longest, first).  The dQ and the
// dK/dV blocks are independent, so a CU that finishes a short one takes the
// next.
template <int DH, bool CLIP>
__global__ __launch_bounds__(512) void flash_bwd_kernel(
    const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ ctx,
    const bf16_t* __restrict__ dctx, const float* __restrict__ lse2, bf16_t* __restrict__ dqkv,
    int S, int H, int D, int causal, float sl2, float scale, float craw) {
  constexpr int TE = attn_tile_elems<DH>();
  __shared__ __attribute__((aligned(16))) bf16_t buf0[kGroups * 2 * TE];
  __shared__ __attribute__((aligned(16))) bf16_t buf1[kGroups * 2 * TE];
  __shared__ float sta0[kGroups * 2 * kBlk];  // [group][lse, delta][64]
  __shared__ float sta1[kGroups * 2 * kBlk];
  const int nb = (S + kBlk - 1) / kBlk;
  const int y = int(blockIdx.y), bh = int(blockIdx.x);
  if (y < nb)
    flash_dq_body<DH, CLIP>(qkv, ctx, dctx, lse2, dqkv, S, H, D, causal, sl2, scale, craw, bh,
                            nb - 1 - y, buf0, buf1);
  else
    flash_dkdv_body<DH, CLIP>(qkv, ctx, dctx, lse2, dqkv, S, H, D, causal, sl2, scale, craw, bh,
                              y - nb, buf0, buf1, sta0, sta1);
}

// The clip threshold in units of the raw product q . k (INFINITY: no clipping).
float raw_clip(float clip, float scale) { return clip > 0.f ? clip / scale : INFINITY; }

}  // namespace

bool flash_ok(bool bf16, int dh) { return bf16 && (dh == 64 || dh == 128); }

hipError_t flash_fwd(const void* qkv, void* ctx, float* lse2, int B, int H, int S, int D,
                     int causal, float clip, hipStream_t s) {
  const int dh = D / H;
  const float scale = 1.0f / sqrtf(float(dh));
  const float sl2 = kLog2e / sqrtf(float(dh));
  const float craw = raw_clip(clip, scale);
  // (sequence, head) along x: workgroups go to the XCDs round-robin by linear
  // id, so with B*H a multiple of 8 every block of one (sequence, head) --
  // which all read the same keys and values -- shares one XCD's L2
  const dim3 grid(B * H, (S + kBlk - 1) / kBlk);
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  const bf16_t* q = static_cast<const bf16_t*>(qkv);
  bf16_t* c = static_cast<bf16_t*>(ctx);
  if (dh != 128 && dh != 64) return hipErrorInvalidValue;
  // (the forward kernel's LDS is static)
  const bool cl = craw < INFINITY;
  if (dh == 128 && cl)
    hipLaunchKernelGGL((flash_fwd_kernel<128, true>), grid, dim3(512), 0, s, q, c, lse2, S, H, D, causal, sl2, craw);
  else if (dh == 128)
    hipLaunchKernelGGL((flash_fwd_kernel<128, false>), grid, dim3(512), 0, s, q, c, lse2, S, H, D, causal, sl2, craw);
  else if (cl)
    hipLaunchKernelGGL((flash_fwd_kernel<64, true>), grid, dim3(512), 0, s, q, c, lse2, S, H, D, causal, sl2, craw);
  else
    hipLaunchKernelGGL((flash_fwd_kernel<64, false>), grid, dim3(512), 0, s, q, c, lse2, S, H, D, causal, sl2, craw);
  return hipGetLastError();
}

hipError_t flash_bwd(const void* qkv, const void* ctx, const void* dctx, const float* lse2,
                     void* dqkv, int B, int H, int S, int D, int causal, float clip, hipStream_t s) {
  const int dh = D / H;
  const float scale = 1.0f / sqrtf(float(dh));
  const float sl2 = kLog2e * scale;
  const float craw = raw_clip(clip, scale);
  const int nb = (S + kBlk - 1) / kBlk;
  if (B * H == 0 || nb == 0) return hipSuccess;
  const bf16_t* q = static_cast<const bf16_t*>(qkv);
  const bf16_t* o = static_cast<const bf16_t*>(ctx);
  const bf16_t* dO = static_cast<const bf16_t*>(dctx);
  bf16_t* dq = static_cast<bf16_t*>(dqkv);
  if (dh != 128 && dh != 64) return hipErrorInvalidValue;
  // (the kernel's LDS is static)
  // (sequence, head) along x: workgroups go to the XCDs round-robin by linear
  // id, so with B*H a multiple of 8 every block of one (sequence, head) --
  // which all read the same keys and values -- shares one XCD's L2
  const dim3 grid(B * H, 2 * nb);
  const bool cl = craw < INFINITY;
  if (dh == 128 && cl)
    launch_k((flash_bwd_kernel<128, true>), grid, dim3(512), 0, s, q, o, dO, lse2, dq, S, H, D, causal, sl2, scale, craw);
  else if (dh == 128)
    launch_k((flash_bwd_kernel<128, false>), grid, dim3(512), 0, s, q, o, dO, lse2, dq, S, H, D, causal, sl2, scale, craw);
  else if (cl)
    launch_k((flash_bwd_kernel<64, true>), grid, dim3(512), 0, s, q, o, dO, lse2, dq, S, H, D, causal, sl2, scale, craw);
  else
    launch_k((flash_bwd_kernel<64, false>), grid, dim3(512), 0, s, q, o, dO, lse2, dq, S, H, D, causal, sl2, scale, craw);
  return hipGetLastError();
}

}  // namespace gp
