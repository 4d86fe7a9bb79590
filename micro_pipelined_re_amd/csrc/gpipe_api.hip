// C-ABI of the GPipe cell library: cell metadata, the activation-workspace
// plan, the partition, and the step / update drivers that enqueue the kernels.
//
// Schedule (GPipe technical review page, "GPipe algorithm in detail / pipeline
// execution flow"): forward phase over the M micro-batches keeping only the
// boundary output, backward phase re-materializing each micro-batch's
// intermediates and accumulating float32 gradients, then one update.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <limits>
#include <mutex>
#include <new>
#include <vector>

#include "cell.hpp"

using namespace gp;


namespace {

// ----------------------------------------------------------------- workspace plan
// Byte layout of the workspace for one (N, M, remat):
//   sets:   remat ? 1 : M micro-batch sets; each set holds, for every layer,
//           the saved tensors of gpipe_saved (layer 0 has no X slot)
//   yre:    output of the re-materialized forward [T, D] (remat only)
//   scores: float32 [B*H, S, ldS]  (forward scores, backward dP; unfused
//           attention only)
//   ds:     act [B*H, S, ldS] (unfused attention only)
//   spare:  one more layer slot after the set (pipelined backward phase: the
//           next micro-batch's first layer is re-materialized there while the
//           current one's backward still holds every slot of the set)
//   r0, r1, dm: float32 [T, D]   (residual-stream gradients, LN input grads)
//   a0, a1: act [T, D], two copies each;  dctx: act [T, D]
//   du: act [T, F];  dqkv: act [T, 3D], two copies each (the weight-gradient
//           stream reads them: the input-gradient chain writes one copy while
//           the other's readers may still run)
//   colpart: float32 [colsum chunks, max(3D, F)] (bias gradients summed by
//            column sums: fp32 cells, or shapes the weight-gradient kernel
//            does not sum)
//   gpart:   per layer, float32 block partial sums that stay in place for the
//            whole backward phase: LN1 and LN2 [LN blocks][2D] (gain, shift)
//            and, where the weight-gradient kernel sums the bias gradient,
//            its partial rows [parts][rows] for b_qkv, b_o, b_1, b_2.  Micro-
//            batch 0 writes them, the others add; after the last micro-batch
//            one fixed-order pass per tensor reduces them into G.
//   msepart: float32 [M, mse blocks]
enum { GPS_LN1, GPS_LN2, GPS_BQKV, GPS_BO, GPS_B1, GPS_B2, GPS_N };

// Parameters of a weight-gradient product G[M][N] (+)= A^T-product over K
// tokens; make_plan and mm_wgrad build them the same way, so the plan's
// partial-row counts are the launches' counts.
GemmParams wgrad_params(int M, int N, int K, const void* A, int64_t lda, const void* B,
                        int64_t ldb, float* C, int64_t ldc, int beta);

struct Plan {
  int N, M, B, T, ldS;
  bool flash;  // fused attention kernels
  size_t eb;
  size_t saved_off[GPIPE_N_SAVED];  // inside one layer's slot
  size_t saved_bytes[GPIPE_N_SAVED];
  size_t layer_bytes, set_bytes;
  int nsets;
  bool spare;  // a spare layer slot after set 0 (slot index L)
  size_t yre, scores, ds, r0, r1, dm, a0[2], a1[2], dctx, du[2], dqkv[2], colpart, gpart, msepart,
      splitk, splitk2, splitk3;
  size_t colpart_floats;
  // gpart slots (GPS_*): offset inside a layer's block, partial rows, row length
  size_t gp_off[GPS_N], gp_layer;
  int gp_parts[GPS_N], gp_cols[GPS_N];
  int mse_nblk;
  // forward phase with re-materialization (overlapped_forward): lanes and
  // micro-batches per launch; 1 / 1 when that phase runs one micro-batch at
  // a time on the caller's stream
  int fwd_lanes, fwd_group;
  size_t total;
};

// The forward products of one layer over `rows` tokens.
void forward_shapes(const gpipe_cell* c, int rows, int out[4][4]) {
  const int D = c->D, F = c->F;
  const int s[4][4] = {{GPIPE_ROLE_QKV_FWD, rows, 3 * D, D}, {GPIPE_ROLE_OUT_FWD, rows, D, D},
                       {GPIPE_ROLE_FFN1_FWD, rows, F, D}, {GPIPE_ROLE_FFN2_FWD, rows, D, F}};
  memcpy(out, s, sizeof(s));
}

// True when every forward product sums over k the same way at `a` and at `b`
// rows: the same k-splits of the same depth (an unsplit product accumulates
// each output in increasing k with the same MFMA instruction whatever the
// tile, and split partials are summed in split order), so each row's result
// does not depend on how many rows share the launch.
bool same_k_order(const gpipe_cell* c, int a, int b) {
  int sa[4][4], sb[4][4];
  forward_shapes(c, a, sa);
  forward_shapes(c, b, sb);
  const bool bf = c->prec == GPIPE_BF16;
  for (int i = 0; i < 4; ++i) {
    const GemmPlan pa = plan_gemm(sa[i][0], bf, sa[i][1], sa[i][2], sa[i][3], 1);
    const GemmPlan pb = plan_gemm(sb[i][0], bf, sb[i][1], sb[i][2], sb[i][3], 1);
    const bool ua = pa.splits <= 1, ub = pb.splits <= 1;
    if (ua != ub || (!ua && (pa.splits != pb.splits || pa.kchunk != pb.kchunk))) return false;
  }
  return true;
}

// Micro-batches per launch (G) and lanes of the forward phase with
// re-materialization: two lanes of up to four micro-batches, about 4096
// tokens, per launch (each lane takes G layer slots of the set), provided
// the grouped launches -- G micro-batches, and the M mod G of the last group
// -- sum every product in the same k order as one micro-batch (so the
// boundary outputs are bitwise those the re-materialization reproduces);
// else one micro-batch per launch on up to three lanes.  Two lanes of four
// 1024-token micro-batches ran the 8-layer 2048-wide step in 156.4 ms
// against 158.8 (three lanes of one), 157.4 (one lane of eight) and 159.9
// (three lanes of two) -- A/B on one box.
void forward_groups(const gpipe_cell* c, int M, int T, int* lanes, int* group) {
  const int L = c->L;
  int G = std::min({L / 2, std::max(1, 4096 / std::max(T, 1)), M});
  for (; G >= 2; --G) {
    if (int64_t(G) * T > std::numeric_limits<int>::max()) continue;
    if (same_k_order(c, T, G * T) && (M % G == 0 || same_k_order(c, T, (M % G) * T))) break;
  }
  *lanes = G >= 2 ? 2 : std::min(L, 3);
  *group = std::max(G, 1);
}

bool make_plan(const gpipe_cell* c, int N, int M, int remat, Plan* p) {
  if (N <= 0 || M <= 0 || N % M) return false;
  p->N = N;
  p->M = M;
  p->B = N / M;
  const size_t S = c->S, D = c->D, F = c->F, H = c->H;
  const size_t B = p->B;
  const size_t T = B * S;
  if (T > size_t(std::numeric_limits<int>::max())) return false;
  p->T = int(T);
  p->ldS = int(align_up(S, 8));
  const size_t eb = c->prec == GPIPE_BF16 ? 2 : 4;
  p->eb = eb;
  const size_t pbytes = B * H * S * size_t(p->ldS);
  p->flash = flash_ok(c->prec == GPIPE_BF16, c->D / c->H);
  // fused attention keeps the row log-sum-exp instead of the probabilities
  const size_t p_saved = p->flash ? B * H * S * 4 : pbytes * eb;
  const size_t sizes[GPIPE_N_SAVED] = {
      T * D * eb, T * D * eb, T * 2 * 4, T * 3 * D * eb, p_saved, T * D * eb,
      T * D * eb, T * D * eb, T * 2 * 4, T * F * eb, T * F * eb};
  size_t off = 0;
  for (int i = 0; i < GPIPE_N_SAVED; ++i) {
    p->saved_off[i] = off;
    p->saved_bytes[i] = sizes[i];
    off += align_up(sizes[i], kAlign);
  }
  p->layer_bytes = off;
  // layer 0 has no X slot: the set is L layer slots minus one X slot
  p->set_bytes = size_t(c->L) * p->layer_bytes;
  p->nsets = remat ? 1 : M;
  // the backward phase is pipelined (transformer_run) with re-materialization,
  // fused attention and two or more layers
  p->spare = remat && p->flash && c->L >= 2;
  size_t o = size_t(p->nsets) * p->set_bytes + (p->spare ? p->layer_bytes : 0);
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes, kAlign);
    return at;
  };
  p->yre = take(remat ? T * D * eb : 0);
  // unfused attention: scores / dP (f32) and dS
  p->scores = take(p->flash ? 0 : pbytes * 4);
  p->ds = take(p->flash ? 0 : pbytes * eb);
  p->r0 = take(T * D * 4);
  p->r1 = take(T * D * 4);
  p->dm = take(T * D * 4);
  for (int k = 0; k < 2; ++k) {
    p->a0[k] = take(T * D * eb);
    p->a1[k] = take(T * D * eb);
    p->du[k] = take(T * F * eb);
    p->dqkv[k] = take(T * 3 * D * eb);
  }
  p->dctx = take(T * D * eb);
  p->colpart_floats = size_t(colsum_chunks(int(T))) * std::max(3 * D, F);
  p->colpart = take(p->colpart_floats * 4);
  {
    const int Ti = int(T), Di = c->D, Fi = c->F;
    const int nbl = layernorm_bwd_blocks(Ti, Di);
    // role, rows M, columns N, lda, ldb (= ldc) of the four weight gradients
    const int wg[4][5] = {{GPIPE_ROLE_QKV_WGRAD, 3 * Di, Di, 3 * Di, Di},
                          {GPIPE_ROLE_OUT_WGRAD, Di, Di, Di, Di},
                          {GPIPE_ROLE_FFN1_WGRAD, Fi, Di, Fi, Di},
                          {GPIPE_ROLE_FFN2_WGRAD, Di, Fi, Di, Fi}};
    size_t lo = 0;
    for (int k = 0; k < GPS_N; ++k) {
      int parts = 0, cols = 0;
      if (k <= GPS_LN2) {
        parts = nbl;
        cols = 2 * Di;
      } else if (c->prec == GPIPE_BF16) {
        const int* r = wg[k - GPS_BQKV];
        const GemmParams g = wgrad_params(r[1], r[2], Ti, nullptr, r[3], nullptr, r[4], nullptr, r[4], 0);
        parts = gemm_rowsum_parts(r[0], g, 1);
        cols = r[1];
      }
      p->gp_off[k] = lo;
      p->gp_parts[k] = parts;
      p->gp_cols[k] = parts ? cols : 0;
      lo += align_up(size_t(parts) * cols * 4, kAlign);
    }
    p->gp_layer = lo;
    p->gpart = take(size_t(c->L) * lo);
  }
  p->mse_nblk = mse_blocks(int64_t(T) * int64_t(D));
  p->msepart = take(size_t(M) * size_t(p->mse_nblk) * 4);
  // split-K partials of the largest split GEMM of a layer (none for fp32 cells)
  const bool bf = c->prec == GPIPE_BF16;
  const int Ti = int(T), Di = c->D, Fi = c->F;
  const int shapes[][4] = {{GPIPE_ROLE_QKV_FWD, Ti, 3 * Di, Di}, {GPIPE_ROLE_OUT_FWD, Ti, Di, Di},
                           {GPIPE_ROLE_FFN1_FWD, Ti, Fi, Di},     {GPIPE_ROLE_FFN2_FWD, Ti, Di, Fi},
                           {GPIPE_ROLE_FFN2_DGRAD, Ti, Fi, Di},   {GPIPE_ROLE_FFN1_DGRAD, Ti, Di, Fi},
                           {GPIPE_ROLE_OUT_DGRAD, Ti, Di, Di},    {GPIPE_ROLE_QKV_DGRAD, Ti, Di, 3 * Di}};
  size_t sk = 0;
  for (const auto& r : shapes) sk = std::max(sk, gemm_partial_floats(r[0], bf, r[1], r[2], r[3], 1));
  p->fwd_lanes = p->fwd_group = 1;
  if (remat && p->flash && c->L >= 2) forward_groups(c, M, Ti, &p->fwd_lanes, &p->fwd_group);
  // the grouped forward launches (G micro-batches, and the last group's M mod
  // G) take their lane's partials too
  for (const int g : {p->fwd_group, M % p->fwd_group}) {
    if (g < 2) continue;
    int fs[4][4];
    forward_shapes(c, g * Ti, fs);
    for (const auto& r : fs) sk = std::max(sk, gemm_partial_floats(r[0], bf, r[1], r[2], r[3], 1));
  }
  p->splitk = take(sk * 4);
  // the forward phase's second lane (overlapped_forward) has its own partials
  p->splitk2 = take(sk * 4);
  // and its third lane (used with re-materialization by bf16 cells with
  // fused attention and at least three layers; laid out whenever the cell
  // could use it, like the second lane's, so that the two workspaces differ
  // by the saved sets only)
  p->splitk3 = take(p->flash && c->L >= 3 ? sk * 4 : 0);
  p->total = o;
  return true;
}

// Offset of a saved tensor of (set, layer).  Layer 0's X slot exists in the
// layout but is never used (its input is the caller's x).
inline size_t saved_at(const Plan& p, int set, int layer, int which) {
  return size_t(set) * p.set_bytes + size_t(layer) * p.layer_bytes + p.saved_off[which];
}

inline size_t gpart_at(const Plan& p, int layer, int slot) {
  return p.gpart + size_t(layer) * p.gp_layer + p.gp_off[slot];
}

struct Ctx {
  const gpipe_cell* c;
  gpipe_cell* prof;  // non-null when some role is being timed
  const Plan* p;
  char* ws;
  hipStream_t s;
  bool bf16;
  size_t splitk;     // workspace offset of this stream's split-K partials
  const void* wmat(int layer, int t) const {
    const size_t off = size_t(layer) * c->per_layer + c->rel_off[t];
    if (bf16) return static_cast<const uint16_t*>(c->w_lowp) + off;
    return c->master + off;
  }
  const float* wf32(int layer, int t) const {
    return c->master + size_t(layer) * c->per_layer + c->rel_off[t];
  }
  float* grad(int layer, int t) const {
    return c->grad + size_t(layer) * c->per_layer + c->rel_off[t];
  }
  void* at(size_t off) const { return ws + off; }
  void* act(const void* base, size_t elems) const {
    return const_cast<char*>(static_cast<const char*>(base)) + elems * p->eb;
  }
};

GemmParams gp0() {
  GemmParams g;
  memset(&g, 0, sizeof(g));
  g.hdiv = 1;
  g.alpha = 1.0f;
  return g;
}

// Plain 2-D product, no batching.
hipError_t mm(const Ctx& x, int role, int M, int N, int K, const void* A, int64_t lda,
              const void* B, int64_t ldb, void* C, int64_t ldc, const float* bias = nullptr,
              const void* R = nullptr, int64_t ldr = 0, void* U = nullptr, int64_t ldu = 0,
              int beta = 0) {
  GemmParams g = gp0();
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda;
  g.B = B; g.ldb = ldb;
  g.C = C; g.ldc = ldc;
  g.bias = bias; g.R = R; g.ldr = ldr; g.U = U; g.ldu = ldu; g.beta = beta;
  g.P = static_cast<float*>(x.at(x.splitk));
  return gemm(x.bf16, role, g, 1, x.s);
}

GemmParams wgrad_params(int M, int N, int K, const void* A, int64_t lda, const void* B,
                        int64_t ldb, float* C, int64_t ldc, int beta) {
  GemmParams g = gp0();
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda;
  g.B = B; g.ldb = ldb;
  g.C = C; g.ldc = ldc;
  g.beta = beta;
  return g;
}

// Weight gradient G (+)= A^T-product over tokens.  Where the plan gives the
// layer's bias a gpart slot (bf16 cells, shapes the specialised kernel
// takes), the same kernel also sums A over tokens into that slot's partial
// rows (written for micro-batch 0, added for the others; reduced into G
// after the backward phase) and *fused is set; otherwise the caller sums the
// bias gradient.
hipError_t mm_wgrad(const Ctx& x, int role, int layer, int slot, int M, int N, int K,
                    const void* A, int64_t lda, const void* B, int64_t ldb, float* C,
                    int64_t ldc, int beta, bool* fused) {
  GemmParams g = wgrad_params(M, N, K, A, lda, B, ldb, C, ldc, beta);
  g.P = static_cast<float*>(x.at(x.splitk));
  const int parts = x.bf16 ? gemm_rowsum_parts(role, g, 1) : 0;
  *fused = parts > 0 && parts == x.p->gp_parts[slot] && M == x.p->gp_cols[slot];
  if (*fused) g.rowsum = static_cast<float*>(x.at(gpart_at(*x.p, layer, slot)));
  return gemm(x.bf16, role, g, 1, x.s);
}

// Batched over (sequence b, head h) of one micro-batch.
struct Bat {
  const void* ptr;
  int64_t ld, sb, sh;
};
hipError_t bmm(const Ctx& x, int role, int M, int N, int K, Bat A, Bat B, Bat C,
               int causal, float alpha) {
  GemmParams g = gp0();
  g.M = M; g.N = N; g.K = K;
  g.A = A.ptr; g.lda = A.ld; g.sAb = A.sb; g.sAh = A.sh;
  g.B = B.ptr; g.ldb = B.ld; g.sBb = B.sb; g.sBh = B.sh;
  g.C = const_cast<void*>(C.ptr); g.ldc = C.ld; g.sCb = C.sb; g.sCh = C.sh;
  g.hdiv = x.c->H;
  g.causal = causal;
  g.alpha = alpha;
  return gemm(x.bf16, role, g, x.p->B * x.c->H, x.s);
}

// Column sums of x [T, cols] added (beta) or stored into out[cols].
hipError_t colsum_into(const Ctx& x, int xtype, const void* src, int64_t ld, int cols, float* out,
                       int beta) {
  int nch = 0;
  float* part = static_cast<float*>(x.at(x.p->colpart));
  hipError_t e = colsum_partial(xtype, src, ld, x.p->T, cols, part, &nch, x.s);
  if (e != hipSuccess) return e;
  return sum_partials(part, nch, cols, cols, out, beta, x.s);
}

// Forward of layer l for one micro-batch: input xin, saved tensors in `set`,
// output xout (all act [T, D]).
// (slot: the layer slot of `set` that receives the intermediates; l: the
// layer whose weights are applied -- the same except in the forward phase's
// one-slot scratch)
// (keep_u: store the FFN pre-activation u, which only the backward reads)
// (end_event: recorded when the layer's last kernel ends, in its dispatch)
gpipe_status layer_forward(const Ctx& x, int set, int slot, int l, const void* xin, void* xout,
                           bool keep_u = true, hipEvent_t end_event = nullptr) {
  const gpipe_cell* c = x.c;
  const Plan& p = *x.p;
  const int T = p.T, D = c->D, F = c->F, S = c->S, H = c->H, dh = D / H;
  const int64_t ldS = p.ldS;
  void* h1 = x.at(saved_at(p, set, slot, GPIPE_SAVED_H1));
  float* st1 = static_cast<float*>(x.at(saved_at(p, set, slot, GPIPE_SAVED_ST1)));
  void* qkv = x.at(saved_at(p, set, slot, GPIPE_SAVED_QKV));
  void* P = x.at(saved_at(p, set, slot, GPIPE_SAVED_P));
  void* ctx = x.at(saved_at(p, set, slot, GPIPE_SAVED_CTX));
  void* x1 = x.at(saved_at(p, set, slot, GPIPE_SAVED_X1));
  void* h2 = x.at(saved_at(p, set, slot, GPIPE_SAVED_H2));
  float* st2 = static_cast<float*>(x.at(saved_at(p, set, slot, GPIPE_SAVED_ST2)));
  void* u = x.at(saved_at(p, set, slot, GPIPE_SAVED_U));
  void* g = x.at(saved_at(p, set, slot, GPIPE_SAVED_G));
  float* scores = static_cast<float*>(x.at(p.scores));

  GP_RUN(x, GPIPE_ROLE_LN1_FWD, layernorm_fwd(x.bf16, xin, h1, st1, x.wf32(l, GPIPE_LN1_G), x.wf32(l, GPIPE_LN1_B), T, D,
                         c->ln_eps, x.s));
  GP_RUN(x, GPIPE_ROLE_QKV_FWD, mm(x, GPIPE_ROLE_QKV_FWD, T, 3 * D, D, h1, D, x.wmat(l, GPIPE_W_QKV), D, qkv, 3 * D,
              x.wf32(l, GPIPE_B_QKV)));
  const int64_t sq = int64_t(S) * 3 * D;       // per-sequence stride inside qkv
  const int64_t sp = int64_t(H) * S * ldS;     // per-sequence stride inside P / scores
  const float scale = 1.0f / sqrtf(float(dh));
  Bat Q{qkv, 3 * D, sq, dh}, K{x.act(qkv, D), 3 * D, sq, dh}, V{x.act(qkv, 2 * D), 3 * D, sq, dh};
  Bat SC{scores, ldS, sp, int64_t(S) * ldS};
  Bat PP{P, ldS, sp, int64_t(S) * ldS};
  Bat CX{ctx, D, int64_t(S) * D, dh};
  if (p.flash) {
    GP_RUN(x, GPIPE_ROLE_ATTN_FWD, flash_fwd(qkv, ctx, static_cast<float*>(P), p.B, H, S, D,
                                             c->causal, c->logit_clip, x.s));
  } else {
    GP_RUN(x, GPIPE_ROLE_SCORES_FWD, bmm(x, GPIPE_ROLE_SCORES_FWD, S, S, dh, Q, K, SC,
                 c->causal ? CAUSAL_SKIP_UPPER : CAUSAL_NONE, scale));
    GP_RUN(x, GPIPE_ROLE_SOFTMAX_FWD, softmax_fwd(x.bf16, scores, P, int64_t(p.B) * H * S, S, ldS, c->causal,
                                                  c->logit_clip, x.s));
    GP_RUN(x, GPIPE_ROLE_PV_FWD, bmm(x, GPIPE_ROLE_PV_FWD, S, dh, S, PP, V, CX,
                 c->causal ? CAUSAL_K_UPTO_M : CAUSAL_NONE, 1.0f));
  }
  GP_RUN(x, GPIPE_ROLE_OUT_FWD, mm(x, GPIPE_ROLE_OUT_FWD, T, D, D, ctx, D, x.wmat(l, GPIPE_W_O), D, x1, D,
              x.wf32(l, GPIPE_B_O), xin, D));
  GP_RUN(x, GPIPE_ROLE_LN2_FWD, layernorm_fwd(x.bf16, x1, h2, st2, x.wf32(l, GPIPE_LN2_G), x.wf32(l, GPIPE_LN2_B), T, D,
                         c->ln_eps, x.s));
  GP_RUN(x, GPIPE_ROLE_FFN1_FWD, mm(x, GPIPE_ROLE_FFN1_FWD, T, F, D, h2, D, x.wmat(l, GPIPE_W_1), D, g, F,
              x.wf32(l, GPIPE_B_1), nullptr, 0, keep_u ? u : nullptr, F));
  next_done_event() = end_event;
  GP_RUN(x, GPIPE_ROLE_FFN2_FWD, mm(x, GPIPE_ROLE_FFN2_FWD, T, D, F, g, F, x.wmat(l, GPIPE_W_2), F, xout, D,
              x.wf32(l, GPIPE_B_2), x1, D));
  if (end_event && next_done_event() == end_event) {
    next_done_event() = nullptr;
    GP_CHECK(hipEventRecord(end_event, x.s));
  }
  return GPIPE_OK;
}

gpipe_status cell_forward(const Ctx& x, int set, const void* xin, void* yout) {
  const int L = x.c->L;
  for (int l = 0; l < L; ++l) {
    const void* in = l == 0 ? xin : x.at(saved_at(*x.p, set, l, GPIPE_SAVED_X));
    void* out = l == L - 1 ? yout : x.at(saved_at(*x.p, set, l + 1, GPIPE_SAVED_X));
    gpipe_status st = layer_forward(x, set, l, l, in, out);
    if (st != GPIPE_OK) return st;
  }
  return GPIPE_OK;
}

// Layout of one layer slot for g micro-batches at once (every per-row tensor
// g times longer), with the slot stride `stride`.
bool group_plan(const gpipe_cell* c, const Plan& p, int g, size_t stride, Plan* q) {
  Plan t;
  if (!make_plan(c, g * p.B, 1, 1, &t) || t.layer_bytes > stride) return false;
  *q = p;
  q->B = t.B;
  q->T = t.T;
  for (int i = 0; i < GPIPE_N_SAVED; ++i) {
    q->saved_off[i] = t.saved_off[i];
    q->saved_bytes[i] = t.saved_bytes[i];
  }
  q->layer_bytes = stride;
  return true;
}

// The forward phase with re-materialization keeps nothing but the boundary
// output, so a micro-batch needs only one layer's intermediates, reused layer
// after layer (the layer's output overwrites its input, which is last read by
// the out-projection's residual add).  The micro-batches are independent: they
// run in groups of G consecutive ones (rows contiguous in x and y) per launch,
// group i on lane i mod K -- the caller's stream and the cell's others, the
// lanes after the first with their own split-K partials -- in that lane's
// share of the saved set, so each stream's kernels fill the CUs and launch
// gaps the others leave; the set is free until the backward phase
// re-materializes into it, after the streams join.  Role timing covers these
// launches too (each one's own span, which may share the CUs with the other
// streams' kernels).  G and K come from the plan (forward_groups).
gpipe_status overlapped_forward(const Ctx& cx, Streams& ss, const void* x, void* y, int M,
                                size_t mb) {
  const Plan& p = *cx.p;
  const int L = cx.c->L;
  const int K = p.fwd_lanes, G = p.fwd_group;
  // a group's rows are contiguous in x and y, and its intermediates take
  // lane k's share of the set: [k, k+1) x the full group's slot size
  Plan pg[2];
  {
    Plan t;
    if (!make_plan(cx.c, G * p.B, 1, 1, &t) || size_t(K) * t.layer_bytes > p.set_bytes ||
        !group_plan(cx.c, p, G, t.layer_bytes, &pg[0]) ||
        !group_plan(cx.c, p, M % G ? M % G : G, t.layer_bytes, &pg[1]))
      return GPIPE_ERR_INVALID;
  }
  Ctx lane[3] = {cx, cx, cx};
  lane[1].s = ss.s2;
  lane[1].splitk = p.splitk2;
  lane[2].s = ss.s3;
  lane[2].splitk = p.splitk3;
  // the inputs and weights exist
  if ((K >= 2 && !ss.fork()) || (K == 3 && !ss.fork3())) return GPIPE_ERR_DEVICE;
  // K groups are enqueued layer by layer, alternating the streams, so that
  // all always have work queued (enqueueing a whole group per stream let each
  // run dry while the host fed the others)
  const int ng = (M + G - 1) / G;
  for (int g0 = 0; g0 < ng; g0 += K)
    for (int l = 0; l < L; ++l)
      for (int gi = g0; gi < std::min(ng, g0 + K); ++gi) {
        const int k = gi % K, m = gi * G;
        Ctx z = lane[k];
        z.p = m + G > M ? &pg[1] : &pg[0];
        void* xs = z.at(saved_at(*z.p, 0, k, GPIPE_SAVED_X));
        const void* in = l == 0 ? cx.act(x, m * mb) : xs;
        void* out = l == L - 1 ? cx.act(y, m * mb) : xs;
        // (nothing of the layer but its output is read again)
        gpipe_status st = layer_forward(z, 0, k, l, in, out, false);
        if (st != GPIPE_OK) return st;
      }
  return (K < 2 || ss.join_all()) && (K < 3 || ss.join3()) ? GPIPE_OK : GPIPE_ERR_DEVICE;
}

// The four gradients of a layer's backward that weight gradients read.
struct Transients {
  Transient a0, a1, du, dqkv;
};

// Backward of layer l (its saved tensors in layer slot `slot` of `set`).  On
// entry r0 (f32) / the current a0 copy (act) hold the gradient w.r.t. the
// layer output; on exit they hold the gradient w.r.t. its input (the next a0
// copy, or dx_out when given, receives the act copy).
gpipe_status layer_backward(const Ctx& x, Streams& ss, Transients& tb, int set, int slot, int l,
                            const void* xin, int beta, void* dx_out, hipEvent_t* s1_done = nullptr) {
  Ctx w = x;  // the weight gradients' context: the second stream
  w.s = ss.s2;
  const gpipe_cell* c = x.c;
  const Plan& p = *x.p;
  const int T = p.T, D = c->D, F = c->F, S = c->S, H = c->H, dh = D / H;
  const int64_t ldS = p.ldS;
  const bool bf = x.bf16;
  const int xt_act = bf ? XT_BF16 : XT_F32;
  void* h1 = x.at(saved_at(p, set, slot, GPIPE_SAVED_H1));
  const float* st1 = static_cast<const float*>(x.at(saved_at(p, set, slot, GPIPE_SAVED_ST1)));
  void* qkv = x.at(saved_at(p, set, slot, GPIPE_SAVED_QKV));
  void* P = x.at(saved_at(p, set, slot, GPIPE_SAVED_P));
  void* ctx = x.at(saved_at(p, set, slot, GPIPE_SAVED_CTX));
  void* x1 = x.at(saved_at(p, set, slot, GPIPE_SAVED_X1));
  void* h2 = x.at(saved_at(p, set, slot, GPIPE_SAVED_H2));
  const float* st2 = static_cast<const float*>(x.at(saved_at(p, set, slot, GPIPE_SAVED_ST2)));
  void* u = x.at(saved_at(p, set, slot, GPIPE_SAVED_U));
  void* g = x.at(saved_at(p, set, slot, GPIPE_SAVED_G));
  float* r0 = static_cast<float*>(x.at(p.r0));
  float* r1 = static_cast<float*>(x.at(p.r1));
  float* dm = static_cast<float*>(x.at(p.dm));
  void* a0 = x.at(tb.a0.off[tb.a0.cur]);
  void* dctx = x.at(p.dctx);
  void* a1 = nullptr;
  void* du = nullptr;
  void* dqkv = nullptr;
  float* dP = static_cast<float*>(x.at(p.scores));
  void* dS = x.at(p.ds);
  float* ln1part = static_cast<float*>(x.at(gpart_at(p, l, GPS_LN1)));
  float* ln2part = static_cast<float*>(x.at(gpart_at(p, l, GPS_LN2)));

  // FFN: y = x1 + g W2^T + b2,  g = gelu(u),  u = h2 W1^T + b1
  // (bias gradients: from the weight-gradient kernel where it sums them --
  // over the bf16 copy of the output gradient it reads -- else summed here)
  // The weight gradients are handed to the second stream in two batches per
  // layer, each after the input-gradient kernel that produces the last of
  // their operands, whose dispatch records the hand-off event (an event
  // recorded as a packet of its own delays the caller's next launch by a few
  // microseconds); the two batches keep the weight gradients in the same
  // order on the second stream.
  bool fused = false;
  if (!tb.du.next(&ss)) return GPIPE_ERR_DEVICE;
  du = x.at(tb.du.off[tb.du.cur]);
  ss.fork_begin();
  GP_RUN(x, GPIPE_ROLE_FFN2_DGRAD, mm(x, GPIPE_ROLE_FFN2_DGRAD, T, F, D, a0, D, x.wmat(l, GPIPE_W_2), F, du, F,
              nullptr, nullptr, 0, u, F));
  if (!ss.fork_end()) return GPIPE_ERR_DEVICE;  // a0, g and du exist
  // (the events after the weight gradients are recorded in their dispatches)
  hipEvent_t ev = ss.mark_begin();
  GP_RUN(w, GPIPE_ROLE_FFN2_WGRAD, mm_wgrad(w, GPIPE_ROLE_FFN2_WGRAD, l, GPS_B2, D, F, T, a0, D, g, F,
              x.grad(l, GPIPE_W_2), F, beta, &fused));
  if (!tb.a0.read_by_s2_at(&ss, tb.a0.cur, ev)) return GPIPE_ERR_DEVICE;
  if (!fused) GP_RUN(x, GPIPE_ROLE_BIAS_GRAD, colsum_into(x, XT_F32, r0, D, D, x.grad(l, GPIPE_B_2), beta));
  ev = ss.mark_begin();
  GP_RUN(w, GPIPE_ROLE_FFN1_WGRAD, mm_wgrad(w, GPIPE_ROLE_FFN1_WGRAD, l, GPS_B1, F, D, T, du, F, h2, D,
              x.grad(l, GPIPE_W_1), D, beta, &fused));
  if (!tb.du.read_by_s2_at(&ss, tb.du.cur, ev)) return GPIPE_ERR_DEVICE;
  GP_RUN(x, GPIPE_ROLE_FFN1_DGRAD, mm(x, GPIPE_ROLE_FFN1_DGRAD, T, D, F, du, F, x.wmat(l, GPIPE_W_1), D, dm, D));
  if (!fused) GP_RUN(x, GPIPE_ROLE_BIAS_GRAD, colsum_into(x, xt_act, du, F, F, x.grad(l, GPIPE_B_1), beta));
  int nblk = 0;
  if (!tb.a1.next(&ss)) return GPIPE_ERR_DEVICE;
  a1 = x.at(tb.a1.off[tb.a1.cur]);
  GP_RUN(x, GPIPE_ROLE_LN2_BWD, layernorm_bwd(bf, dm, x1, st2, x.wf32(l, GPIPE_LN2_G), r0, r1, a1, ln2part, T, D,
                         beta, &nblk, x.s));

  // attention: x1 = x + ctx Wo^T + bo
  GP_RUN(x, GPIPE_ROLE_OUT_DGRAD, mm(x, GPIPE_ROLE_OUT_DGRAD, T, D, D, a1, D, x.wmat(l, GPIPE_W_O), D, dctx, D));
  if (!tb.dqkv.next(&ss)) return GPIPE_ERR_DEVICE;
  dqkv = x.at(tb.dqkv.off[tb.dqkv.cur]);
  const int64_t sq = int64_t(S) * 3 * D;
  const int64_t sp = int64_t(H) * S * ldS;
  const int64_t sd = int64_t(S) * D;
  const float scale = 1.0f / sqrtf(float(dh));
  Bat Q{qkv, 3 * D, sq, dh}, K{x.act(qkv, D), 3 * D, sq, dh}, V{x.act(qkv, 2 * D), 3 * D, sq, dh};
  Bat dQ{dqkv, 3 * D, sq, dh}, dK{x.act(dqkv, D), 3 * D, sq, dh}, dV{x.act(dqkv, 2 * D), 3 * D, sq, dh};
  Bat PP{P, ldS, sp, int64_t(S) * ldS}, DP{dP, ldS, sp, int64_t(S) * ldS}, DS{dS, ldS, sp, int64_t(S) * ldS};
  Bat DC{dctx, D, sd, dh};
  const int cz = c->causal;
  if (p.flash) {
    const float* lse2 = static_cast<const float*>(P);
    // dQ, dK and dV in one launch
    ss.fork_begin();
    GP_RUN(x, GPIPE_ROLE_ATTN_DQ, flash_bwd(qkv, ctx, dctx, lse2, dqkv, p.B, H, S, D, cz,
                                            c->logit_clip, x.s));
  } else {
    const bool clip = c->logit_clip > 0.f;
    if (clip) {
      // the clip's keep mask from the recomputed scores, into dS's buffer
      // (softmax_bwd reads it there before writing dS); then dP takes the
      // scores' buffer
      Bat SC{dP, ldS, sp, int64_t(S) * ldS};
      GP_RUN(x, GPIPE_ROLE_SCORES_FWD, bmm(x, GPIPE_ROLE_SCORES_FWD, S, S, dh, Q, K, SC,
                   cz ? CAUSAL_SKIP_UPPER : CAUSAL_NONE, scale));
      GP_CHECK(clip_keep(bf, dP, dS, int64_t(p.B) * H * S, S, ldS, cz, c->logit_clip, x.s));
    }
    GP_RUN(x, GPIPE_ROLE_DP, bmm(x, GPIPE_ROLE_DP, S, S, dh, DC, V, DP,
                 cz ? CAUSAL_SKIP_UPPER : CAUSAL_NONE, 1.0f));
    GP_RUN(x, GPIPE_ROLE_DV, bmm(x, GPIPE_ROLE_DV, S, dh, S, PP, DC, dV,
                 cz ? CAUSAL_K_FROM_M : CAUSAL_NONE, 1.0f));
    GP_RUN(x, GPIPE_ROLE_SOFTMAX_BWD, softmax_bwd(bf, P, dP, dS, int64_t(p.B) * H * S, S, ldS, cz, scale,
                                                  clip ? 1 : 0, x.s));
    GP_RUN(x, GPIPE_ROLE_DQ, bmm(x, GPIPE_ROLE_DQ, S, dh, S, DS, K, dQ,
                 cz ? CAUSAL_K_UPTO_M : CAUSAL_NONE, 1.0f));
    ss.fork_begin();
    GP_RUN(x, GPIPE_ROLE_DK, bmm(x, GPIPE_ROLE_DK, S, dh, S, DS, Q, dK,
                 cz ? CAUSAL_K_FROM_M : CAUSAL_NONE, 1.0f));
  }

  // qkv = h1 Wqkv^T + bqkv,  h1 = LN1(x)
  if (!ss.fork_end()) return GPIPE_ERR_DEVICE;  // a1 and dqkv exist
  ev = ss.mark_begin();
  GP_RUN(w, GPIPE_ROLE_OUT_WGRAD, mm_wgrad(w, GPIPE_ROLE_OUT_WGRAD, l, GPS_BO, D, D, T, a1, D, ctx, D,
              x.grad(l, GPIPE_W_O), D, beta, &fused));
  if (!tb.a1.read_by_s2_at(&ss, tb.a1.cur, ev)) return GPIPE_ERR_DEVICE;
  if (!fused) GP_RUN(x, GPIPE_ROLE_BIAS_GRAD, colsum_into(x, XT_F32, r1, D, D, x.grad(l, GPIPE_B_O), beta));
  ev = ss.mark_begin();
  GP_RUN(w, GPIPE_ROLE_QKV_WGRAD, mm_wgrad(w, GPIPE_ROLE_QKV_WGRAD, l, GPS_BQKV, 3 * D, D, T, dqkv, 3 * D, h1,
              D, x.grad(l, GPIPE_W_QKV), D, beta, &fused));
  if (!tb.dqkv.read_by_s2_at(&ss, tb.dqkv.cur, ev)) return GPIPE_ERR_DEVICE;
  GP_RUN(x, GPIPE_ROLE_QKV_DGRAD, mm(x, GPIPE_ROLE_QKV_DGRAD, T, D, 3 * D, dqkv, 3 * D, x.wmat(l, GPIPE_W_QKV), D,
              dm, D));
  if (!fused)
    GP_RUN(x, GPIPE_ROLE_BIAS_GRAD, colsum_into(x, xt_act, dqkv, 3 * D, 3 * D, x.grad(l, GPIPE_B_QKV), beta));
  void* a0_in = dx_out;  // the gradient w.r.t. the layer input (act)
  if (!a0_in) {
    if (!tb.a0.next(&ss)) return GPIPE_ERR_DEVICE;
    a0_in = x.at(tb.a0.off[tb.a0.cur]);
  }
  // (s1_done: an event the LayerNorm backward, the layer's last kernel on the
  // caller's stream, records in its dispatch)
  if (s1_done && !ss.single) next_done_event() = *s1_done = ss.next();
  GP_RUN(x, GPIPE_ROLE_LN1_BWD, layernorm_bwd(bf, dm, xin, st1, x.wf32(l, GPIPE_LN1_G), r1, r0, a0_in,
                         ln1part, T, D, beta, &nblk, x.s));
  if (s1_done && *s1_done && next_done_event() == *s1_done) {
    next_done_event() = nullptr;
    GP_CHECK(hipEventRecord(*s1_done, x.s));
  }
  return GPIPE_OK;
}

// After the backward phase: reduce each layer's in-place partial sums (LN
// gains and shifts -- adjacent in the parameter layout, so one pass over 2D
// columns -- and the biases the weight-gradient kernels summed) into G.
gpipe_status reduce_gparts(const Ctx& x, int l_begin = 0, int l_end = -1) {
  const Plan& p = *x.p;
  const int grad_of[GPS_N] = {GPIPE_LN1_G, GPIPE_LN2_G, GPIPE_B_QKV, GPIPE_B_O, GPIPE_B_1, GPIPE_B_2};
  if (l_end < 0) l_end = x.c->L;
  // (all of them in one launch: each is its own row of the grid)
  std::vector<SumJob> jobs;
  for (int l = l_begin; l < l_end; ++l)
    for (int k = 0; k < GPS_N; ++k) {
      if (!p.gp_parts[k]) continue;
      const int cols = p.gp_cols[k];
      jobs.push_back(SumJob{static_cast<const float*>(x.at(gpart_at(p, l, k))), x.grad(l, grad_of[k]),
                            cols, p.gp_parts[k], cols});
    }
  GP_RUN(x, GPIPE_ROLE_NORM_GRAD, sum_partials_batch(jobs.data(), int(jobs.size()), x.s));
  return GPIPE_OK;
}

// The allocation-free step's workspace: one array per device, resident while
// the process lives.  In host code `scratch` names a host-side stand-in, not
// device memory, so the host only ever uses the device address that
// hipGetSymbolAddress returns for it, looked up once per device with that
// device current (each device holds its own copy at its own address).
__device__ __align__(256) static unsigned char scratch[GPIPE_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

gpipe_status scratch_of_current_device(void** out) {
  int dev = -1;
  GP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return GPIPE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return GPIPE_ERR_DEVICE;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GPIPE_OK;
}

// What one call of the Transformer cell's driver does: the forward phase
// (PH_FWD), the backward phase (PH_BWD) or both (the step).  The backward's
// output gradient comes from the loss against `target`, or is `dy`, handed
// down by the cell above.  `single`: every launch on the caller's stream, no
// stream or event of the cell's own (and no role timing).
enum { PH_FWD = 1, PH_BWD = 2 };
struct StepIO {
  int phases = 0;
  const void* x = nullptr;
  const void* target = nullptr;
  const void* dy = nullptr;
  void* y = nullptr;
  void* dx = nullptr;
  float* loss_dev = nullptr;
  int N = 0, M = 0, remat = 0;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  hipStream_t s = nullptr;
  bool single = false;
  // the RMSProp update follows the step (gpipe_cell_step_update)
  bool update = false;
  float lr = 0.f, decay = 0.f, eps = 0.f;
};

// RMSProp over layer l's parameters (contiguous in master, grad, ms and the
// bf16 copy), as gpipe_apply_update does over all of them.  It runs beside
// the backward of the layers below, so its grid is capped at one workgroup
// per CU (each looping over its share): 140.0-140.1 ms/step against
// 140.2-140.3 uncapped, 140.4-140.7 at 128 workgroups and ~143 at 64 (three
// A/B rounds on one box).
hipError_t rmsprop_layer(const gpipe_cell* c, int l, float lr, float decay, float eps, hipStream_t s) {
  const size_t off = size_t(l) * c->per_layer;
  void* wl = c->prec == GPIPE_BF16 ? static_cast<void*>(static_cast<uint16_t*>(c->w_lowp) + off) : nullptr;
  return rmsprop(c->master + off, c->grad + off, c->ms + off, wl, int64_t(c->per_layer), lr, decay, eps, s,
                 256);
}

gpipe_status transformer_run(gpipe_cell* c, const StepIO& io) {
  Plan p;
  if (!make_plan(c, io.N, io.M, io.remat, &p)) return GPIPE_ERR_INVALID;
  const bool fwd = io.phases & PH_FWD, bwd = io.phases & PH_BWD;
  const int M = io.M, remat = io.remat;
  const void* x = io.x;
  if (!x || !io.ws || io.ws_bytes < p.total) return GPIPE_ERR_INVALID;
  if (fwd && !io.y) return GPIPE_ERR_INVALID;
  // the backward's output gradient: the loss (needs y, target, loss_dev) or dy
  if (bwd && (io.target ? (!io.y || !io.loss_dev || io.dy) : !io.dy)) return GPIPE_ERR_INVALID;
  if (!aligned16(x) || (io.y && !aligned16(io.y)) || (io.target && !aligned16(io.target)) ||
      (io.dy && !aligned16(io.dy)) || (io.dx && !aligned16(io.dx)) || !aligned16(io.ws))
    return GPIPE_ERR_INVALID;
  if (!io.single) {
    const gpipe_status st = ensure_streams(c);
    if (st != GPIPE_OK) return st;
  }
  Ctx cx{c, (c->prof_mask && !io.single) ? c : nullptr, &p, io.ws, io.s, c->prec == GPIPE_BF16,
         p.splitk};
  next_done_event() = nullptr;  // (nothing pending from an earlier call that failed)
  Streams ss{c, cx.s, io.single ? cx.s : c->aux, io.single ? cx.s : c->aux2, io.single};
  const size_t mb = size_t(p.T) * c->D;  // elements per micro-batch
  const float inv_denom = float(1.0 / (double(io.N) * c->S * c->D));
  float* msepart = static_cast<float*>(cx.at(p.msepart));
  const int L = c->L;
  // several streams (the grouped forward, the pipelined re-materialization)
  // where the fused attention and two or more layers make them pay
  const bool lanes = remat && p.flash && L >= 2 && !io.single;

  // phase 1: forward, boundary output only (intermediates are overwritten)
  if (fwd) {
    if (lanes) {
      gpipe_status st = overlapped_forward(cx, ss, x, io.y, M, mb);
      if (st != GPIPE_OK) return st;
    } else {
      for (int m = 0; m < M; ++m) {
        const int set = remat ? 0 : m;
        gpipe_status st = cell_forward(cx, set, cx.act(x, m * mb), cx.act(io.y, m * mb));
        if (st != GPIPE_OK) return st;
      }
    }
  }
  if (!bwd) return GPIPE_OK;
  // phase 2: backward with re-materialization and float32 accumulation.
  // With fused attention the re-materialization of micro-batch m+1 runs on
  // the third stream during the backward of micro-batch m, in the saved set
  // and one spare layer slot: the backward frees the layer slots from the top
  // down and the re-materialization fills them from the bottom up.  Micro-batch
  // m+1 puts layer 0 in the spare slot as soon as micro-batch m's backward
  // starts (after its loss, which reads the re-materialized output), and layer
  // j >= 1 in the slot that layer L-j of micro-batch m held, enqueued after
  // that slot's backward and weight gradients; so its last layer can start
  // after micro-batch m's layer 1 and is done about when layer 0 is.  The slot
  // micro-batch m's layer 0 frees is the next spare.  A layer's output goes to
  // its own slot's X tensor (the next layer's input), the top layer's to the
  // re-materialized output.  Micro-batch 0 re-materializes on the caller's
  // stream before its backward.
  const bool piped = lanes;
  // layer-wise update (gpipe_cell_step_update), where every layer's parameter
  // range starts 16-byte aligned (RMSProp takes four parameters per thread)
  const bool upd = io.update && c->per_layer % 4 == 0;
  if (piped && !p.spare) return GPIPE_ERR_STATE;
  std::vector<int> cur(L), nxt(L);  // layer -> slot, this micro-batch and the next
  for (int l = 0; l < L; ++l) cur[l] = l;
  int spare = L;
  Ctx cr = cx;  // the re-materialization's context on the third stream
  cr.s = ss.s3;
  cr.splitk = p.splitk2;
  // (the third stream's re-materialization of a micro-batch ends with its top
  // layer's last kernel, which records remat_done in its dispatch; the caller's
  // stream waits for that event before the micro-batch's backward)
  hipEvent_t remat_done = nullptr;
  auto remat_layer = [&](const Ctx& z, const std::vector<int>& sl, int m, int j) {
    const void* in = j == 0 ? cx.act(x, m * mb) : z.at(saved_at(p, 0, sl[j - 1], GPIPE_SAVED_X));
    void* out = j == L - 1 ? z.at(p.yre) : z.at(saved_at(p, 0, sl[j], GPIPE_SAVED_X));
    hipEvent_t end = nullptr;
    if (j == L - 1 && z.s != cx.s && !ss.single) end = remat_done = ss.next();
    return layer_forward(z, 0, sl[j], j, in, out, true, end);
  };
  Transients tb;
  for (int k = 0; k < 2; ++k) {
    tb.a0.off[k] = p.a0[k];
    tb.a1.off[k] = p.a1[k];
    tb.du.off[k] = p.du[k];
    tb.dqkv.off[k] = p.dqkv[k];
  }
  for (int m = 0; m < M; ++m) {
    const int set = remat ? 0 : m;
    const void* xm = cx.act(x, m * mb);
    const void* ym = io.y ? cx.act(io.y, m * mb) : nullptr;
    // unpipelined, the re-materialization below overwrites the saved
    // activations the previous micro-batch's weight gradients read
    // (pipelined, the third stream's forks order those reads, and the
    // transients the weight gradients read wait per copy)
    if (m > 0 && !piped && !ss.join_all()) return GPIPE_ERR_DEVICE;
    if (piped) {
      if (m == 0) {
        for (int j = 0; j < L; ++j) {
          gpipe_status st = remat_layer(cx, cur, 0, j);
          if (st != GPIPE_OK) return st;
        }
      } else if (remat_done ? !ss.join(remat_done) : !ss.join3()) {
        return GPIPE_ERR_DEVICE;  // (this micro-batch's re-materialization is done)
      }
      ym = cx.at(p.yre);
    } else if (remat) {
      void* yre = cx.at(p.yre);
      gpipe_status st = cell_forward(cx, set, xm, yre);
      if (st != GPIPE_OK) return st;
      ym = yre;
    }
    if (!tb.a0.next(&ss)) return GPIPE_ERR_DEVICE;
    void* a0 = cx.at(tb.a0.off[tb.a0.cur]);  // the loss gradient's act copy
    // (the loss kernel records loss_done in its dispatch: the next micro-batch's
    // first layer, re-materialized on the third stream, waits for it)
    hipEvent_t loss_done = nullptr;
    if (piped && m + 1 < M && !ss.single) next_done_event() = loss_done = ss.next();
    if (io.target) {
      int nblk = 0;
      GP_RUN(cx, GPIPE_ROLE_MSE, mse_fwd_bwd(cx.bf16, ym, cx.act(io.target, m * mb),
                                             static_cast<float*>(cx.at(p.r0)), a0,
                                             msepart + size_t(m) * p.mse_nblk, int64_t(mb),
                                             inv_denom, &nblk, cx.s));
    } else {
      GP_CHECK(grad_in(cx.bf16, cx.act(io.dy, m * mb), static_cast<float*>(cx.at(p.r0)), a0,
                       int64_t(mb), cx.s));
    }
    if (loss_done && next_done_event() == loss_done) {
      next_done_event() = nullptr;
      GP_CHECK(hipEventRecord(loss_done, cx.s));
    }
    if (piped && m + 1 < M) {
      // the spare slot (micro-batch m-1's layer 0, whose backward and weight
      // gradients are enqueued before this point) takes micro-batch m+1's
      // layer 0 (the last work on the second stream is micro-batch m-1's
      // layer-0 QKV weight gradient, whose event tb.dqkv holds; none yet for
      // micro-batch 0)
      if (!ss.fork3_after(loss_done, tb.dqkv.read[tb.dqkv.cur])) return GPIPE_ERR_DEVICE;
      nxt[0] = spare;
      gpipe_status st = remat_layer(cr, nxt, m + 1, 0);
      if (st != GPIPE_OK) return st;
    }
    for (int l = L - 1; l >= 0; --l) {
      // (the layer's input: the output of layer l-1, in that layer's slot when
      // pipelined, else in this layer's X tensor)
      const void* xin = l == 0 ? xm
                        : piped ? cx.at(saved_at(p, set, cur[l - 1], GPIPE_SAVED_X))
                                : cx.at(saved_at(p, set, l, GPIPE_SAVED_X));
      void* dxo = (l == 0 && io.dx) ? cx.act(io.dx, m * mb) : nullptr;
      const bool refill = piped && m + 1 < M && l >= 1;
      // (layer-wise update: after the last micro-batch's backward of layer l
      // nothing reads its parameters or writes its gradients but the weight
      // gradients already enqueued on the second stream)
      const bool upd_l = upd && m == M - 1;
      hipEvent_t s1_done = nullptr;
      gpipe_status st = layer_backward(cx, ss, tb, set, piped ? cur[l] : l, l, xin, m > 0 ? 1 : 0, dxo,
                                       refill || upd_l ? &s1_done : nullptr);
      if (st != GPIPE_OK) return st;
      if (upd_l) {
        // on the third stream (idle in the last micro-batch: nothing is left to
        // re-materialize), after this layer's backward on the caller's stream
        // (s1_done) and its weight gradients on the second (the event after the
        // last of them, the QKV one)
        if (!ss.fork3_after(s1_done, tb.dqkv.read[tb.dqkv.cur])) return GPIPE_ERR_DEVICE;
        Ctx w = cx;
        w.s = ss.s3;
        st = reduce_gparts(w, l, l + 1);
        if (st != GPIPE_OK) return st;
        GP_RUN(w, GPIPE_ROLE_RMSPROP, rmsprop_layer(c, l, io.lr, io.decay, io.eps, w.s));
      }
      if (refill) {
        // layer l's slot is free once its backward (s1) and weight gradients (s2)
        // are done
        // (the weight gradients' last event: after the layer's QKV weight
        // gradient, the last launch on s2)
        if (!ss.fork3_after(s1_done, tb.dqkv.read[tb.dqkv.cur])) return GPIPE_ERR_DEVICE;
        const int j = L - l;
        nxt[j] = cur[l];
        st = remat_layer(cr, nxt, m + 1, j);
        if (st != GPIPE_OK) return st;
      }
    }
    if (piped && m + 1 < M) {
      spare = cur[0];
      cur.swap(nxt);
    }
  }
  // the weight gradients (and their bias partial sums; with the layer-wise
  // update, on the third stream, the updates) are complete
  if (!ss.join_all() || (upd && !ss.join3())) return GPIPE_ERR_DEVICE;
  if (!upd) {
    gpipe_status st = reduce_gparts(cx);
    if (st != GPIPE_OK) return st;
    if (io.update)
      GP_RUN(cx, GPIPE_ROLE_RMSPROP,
             rmsprop(c->master, c->grad, c->ms, c->prec == GPIPE_BF16 ? c->w_lowp : nullptr,
                     int64_t(c->n_params), io.lr, io.decay, io.eps, cx.s));
  }
  if (io.target)
    GP_RUN(cx, GPIPE_ROLE_LOSS_REDUCE, sum_partials(msepart, M * p.mse_nblk, 1, 1, io.loss_dev, 0, cx.s));
  return GPIPE_OK;
}

}  // namespace

extern "C" {

const char* gpipe_status_string(gpipe_status s) {
  switch (s) {
    case GPIPE_OK: return "ok";
    case GPIPE_ERR_INVALID: return "invalid argument";
    case GPIPE_ERR_OOM: return "out of device memory";
    case GPIPE_ERR_DEVICE: return "HIP device error";
    case GPIPE_ERR_UNSUPPORTED: return "unsupported shape";
    case GPIPE_ERR_STATE: return "invalid state";
  }
  return "unknown status";
}

gpipe_status gpipe_cell_create(int layers, int d_model, int heads, int d_ff, int seq, int causal,
                               gpipe_precision prec, gpipe_cell** out) {
  if (!out) return GPIPE_ERR_INVALID;
  if (layers <= 0 || d_model <= 0 || heads <= 0 || d_ff <= 0 || seq <= 0) return GPIPE_ERR_INVALID;
  if (d_model % heads) return GPIPE_ERR_INVALID;
  if (prec != GPIPE_FP32 && prec != GPIPE_BF16) return GPIPE_ERR_INVALID;
  const int dh = d_model / heads;
  if (d_model % 8 || d_ff % 8 || dh % 8 || d_model > 8192 || seq > 4096)
    return GPIPE_ERR_UNSUPPORTED;
  gpipe_cell* c = new (std::nothrow) gpipe_cell();
  if (!c) return GPIPE_ERR_INVALID;
  c->kind = CELL_TRANSFORMER;
  c->L = layers; c->D = d_model; c->H = heads; c->F = d_ff; c->S = seq;
  c->causal = causal ? 1 : 0;
  c->prec = prec;
  c->ln_eps = 1e-5f;
  const size_t D = d_model, F = d_ff;
  const size_t cnt[GPIPE_N_TENSORS] = {D, D, 3 * D * D, 3 * D, D * D, D, D, D, F * D, F, D * F, D};
  size_t off = 0;
  for (int t = 0; t < GPIPE_N_TENSORS; ++t) {
    c->rel_off[t] = off;
    c->count[t] = cnt[t];
    off += cnt[t];
  }
  c->per_layer = off;
  c->n_params = off * size_t(layers);
  *out = c;
  return GPIPE_OK;
}

gpipe_status gpipe_conv_cell_create(int blocks, int channels, int height, int width,
                                    float bn_momentum, gpipe_precision prec, gpipe_cell** out) {
  if (!out) return GPIPE_ERR_INVALID;
  if (blocks <= 0 || channels <= 0 || height <= 0 || width <= 0) return GPIPE_ERR_INVALID;
  if (!(bn_momentum >= 0.f && bn_momentum < 1.f)) return GPIPE_ERR_INVALID;
  if (prec != GPIPE_FP32 && prec != GPIPE_BF16) return GPIPE_ERR_INVALID;
  if (channels % 8 || channels > 8192 || size_t(height) * width > (size_t(1) << 24))
    return GPIPE_ERR_UNSUPPORTED;
  gpipe_cell* c = new (std::nothrow) gpipe_cell();
  if (!c) return GPIPE_ERR_INVALID;
  c->kind = CELL_CONV;
  c->L = blocks;
  c->C = channels;
  c->Hc = height;
  c->Wc = width;
  c->bn_momentum = bn_momentum;
  c->bn_eps = 1e-5f;
  c->prec = prec;
  conv_cell_init(c);
  *out = c;
  return GPIPE_OK;
}

gpipe_status gpipe_cell_bind_running(gpipe_cell* c, float* running) {
  if (!c || !running || c->kind != CELL_CONV || !aligned16(running)) return GPIPE_ERR_INVALID;
  c->running = running;
  return GPIPE_OK;
}

gpipe_status gpipe_cell_destroy(gpipe_cell* c) {
  if (c) {
    for (hipEvent_t e : c->prof_events) (void)hipEventDestroy(e);
    for (hipEvent_t e : c->sync_events) (void)hipEventDestroy(e);
    if (c->aux) (void)hipStreamDestroy(c->aux);
    if (c->aux2) (void)hipStreamDestroy(c->aux2);
  }
  delete c;
  return GPIPE_OK;
}

gpipe_status gpipe_cell_param_count(const gpipe_cell* c, size_t* n) {
  if (!c || !n) return GPIPE_ERR_INVALID;
  *n = c->n_params;
  return GPIPE_OK;
}

gpipe_status gpipe_cell_param_offset(const gpipe_cell* c, int layer, int tensor, size_t* offset,
                                     size_t* count) {
  if (!c || !offset || !count || layer < 0 || layer >= c->L || tensor < 0 ||
      tensor >= (c->kind == CELL_CONV ? int(GPIPE_CONV_N_TENSORS) : int(GPIPE_N_TENSORS)))
    return GPIPE_ERR_INVALID;
  *offset = size_t(layer) * c->per_layer + c->rel_off[tensor];
  *count = c->count[tensor];
  return GPIPE_OK;
}

gpipe_status gpipe_cell_bind(gpipe_cell* c, float* master, void* w_lowp, float* grad, float* ms) {
  if (!c || !master || !grad || !ms) return GPIPE_ERR_INVALID;
  if ((c->prec == GPIPE_BF16) != (w_lowp != nullptr)) return GPIPE_ERR_INVALID;
  if (!aligned16(master) || !aligned16(grad) || !aligned16(ms) || (w_lowp && !aligned16(w_lowp)))
    return GPIPE_ERR_INVALID;
  c->master = master;
  c->w_lowp = w_lowp;
  c->grad = grad;
  c->ms = ms;
  c->bound = true;
  return GPIPE_OK;
}

gpipe_status gpipe_cell_sync_lowp(gpipe_cell* c, void* stream) {
  if (!c) return GPIPE_ERR_INVALID;
  if (!c->bound) return GPIPE_ERR_STATE;
  if (c->prec != GPIPE_BF16) return GPIPE_OK;
  GP_CHECK(to_bf16(c->master, c->w_lowp, int64_t(c->n_params), static_cast<hipStream_t>(stream)));
  return GPIPE_OK;
}

gpipe_status gpipe_cell_workspace_bytes(const gpipe_cell* c, int N, int M, int remat, size_t* bytes) {
  if (!c || !bytes) return GPIPE_ERR_INVALID;
  size_t plan = 0;
  if (c->kind == CELL_CONV) {
    if (!conv_workspace_bytes(c, N, M, remat, &plan)) return GPIPE_ERR_INVALID;
  } else {
    Plan p;
    if (!make_plan(c, N, M, remat, &p)) return GPIPE_ERR_INVALID;
    plan = p.total;
  }
  *bytes = plan;
  // The fit: the plan, plus the parameter state while the cell is unbound
  // (it must be allocated too), against the free memory of the current
  // device.  Without a device (a host-only process) there is nothing to
  // compare with and the plan is only reported.
  size_t free_b = 0, total_b = 0;
  if (hipMemGetInfo(&free_b, &total_b) != hipSuccess) {
    (void)hipGetLastError();
    return GPIPE_OK;
  }
  const size_t state = c->bound ? 0 : c->n_params * (c->prec == GPIPE_BF16 ? 14 : 12);
  return plan + state > free_b ? GPIPE_ERR_OOM : GPIPE_OK;
}

gpipe_status gpipe_cell_saved_offset(const gpipe_cell* c, int N, int M, int remat, int micro,
                                     int layer, int which, size_t* offset, size_t* bytes) {
  if (!c || !offset || !bytes) return GPIPE_ERR_INVALID;
  if (c->kind == CELL_CONV)
    return conv_saved_offset(c, N, M, remat, micro, layer, which, offset, bytes) ? GPIPE_OK
                                                                                 : GPIPE_ERR_INVALID;
  Plan p;
  if (!make_plan(c, N, M, remat, &p)) return GPIPE_ERR_INVALID;
  if (micro < 0 || micro >= p.nsets || layer < 0 || layer >= c->L || which < 0 ||
      which >= GPIPE_N_SAVED || (layer == 0 && which == GPIPE_SAVED_X))
    return GPIPE_ERR_INVALID;
  *offset = saved_at(p, micro, layer, which);
  *bytes = p.saved_bytes[which];
  return GPIPE_OK;
}

gpipe_status gpipe_cell_step(gpipe_cell* c, const void* x, const void* target, void* y, void* dx,
                             int N, int M, int remat, void* workspace, size_t ws_bytes,
                             void* stream, float* loss_dev) {
  if (!c) return GPIPE_ERR_INVALID;
  if (!c->bound) return GPIPE_ERR_STATE;
  if (c->kind == CELL_CONV)
    return conv_cell_step(c, x, target, y, dx, N, M, remat, workspace, ws_bytes,
                          static_cast<hipStream_t>(stream), loss_dev);
  StepIO io;
  io.phases = PH_FWD | PH_BWD;
  io.x = x; io.target = target; io.y = y; io.dx = dx; io.loss_dev = loss_dev;
  io.N = N; io.M = M; io.remat = remat;
  io.ws = static_cast<char*>(workspace); io.ws_bytes = ws_bytes;
  io.s = static_cast<hipStream_t>(stream);
  return transformer_run(c, io);
}

static bool update_args_ok(float lr, float decay, float eps) {
  return decay >= 0.f && decay < 1.f && lr >= 0.f && eps >= 0.f && isfinite(lr) && isfinite(eps);
}

gpipe_status gpipe_cell_step_update(gpipe_cell* c, const void* x, const void* target, void* y,
                                    void* dx, int N, int M, int remat, void* workspace,
                                    size_t ws_bytes, void* stream, float* loss_dev, float lr,
                                    float decay, float eps) {
  if (!c) return GPIPE_ERR_INVALID;
  if (!c->bound) return GPIPE_ERR_STATE;
  if (!update_args_ok(lr, decay, eps)) return GPIPE_ERR_INVALID;
  if (c->kind == CELL_CONV) {
    const gpipe_status st = gpipe_cell_step(c, x, target, y, dx, N, M, remat, workspace, ws_bytes,
                                            stream, loss_dev);
    return st != GPIPE_OK ? st : gpipe_apply_update(c, lr, decay, eps, stream);
  }
  StepIO io;
  io.phases = PH_FWD | PH_BWD;
  io.x = x; io.target = target; io.y = y; io.dx = dx; io.loss_dev = loss_dev;
  io.N = N; io.M = M; io.remat = remat;
  io.ws = static_cast<char*>(workspace); io.ws_bytes = ws_bytes;
  io.s = static_cast<hipStream_t>(stream);
  io.update = true;
  io.lr = lr; io.decay = decay; io.eps = eps;
  return transformer_run(c, io);
}

gpipe_status gpipe_cell_forward(gpipe_cell* c, const void* x, void* y, int N, int M, int remat,
                                void* workspace, size_t ws_bytes, void* stream) {
  if (!c) return GPIPE_ERR_INVALID;
  if (!c->bound) return GPIPE_ERR_STATE;
  if (c->kind == CELL_CONV)
    return conv_cell_run(c, 1, x, nullptr, nullptr, y, nullptr, N, M, remat, workspace, ws_bytes,
                         static_cast<hipStream_t>(stream), nullptr);
  StepIO io;
  io.phases = PH_FWD;
  io.x = x; io.y = y;
  io.N = N; io.M = M; io.remat = remat;
  io.ws = static_cast<char*>(workspace); io.ws_bytes = ws_bytes;
  io.s = static_cast<hipStream_t>(stream);
  return transformer_run(c, io);
}

gpipe_status gpipe_cell_backward(gpipe_cell* c, const void* x, const void* dy, void* dx, int N,
                                 int M, int remat, void* workspace, size_t ws_bytes, void* stream) {
  if (!c) return GPIPE_ERR_INVALID;
  if (!c->bound) return GPIPE_ERR_STATE;
  if (!dy) return GPIPE_ERR_INVALID;
  if (c->kind == CELL_CONV)
    return conv_cell_run(c, 2, x, nullptr, dy, nullptr, dx, N, M, remat, workspace, ws_bytes,
                         static_cast<hipStream_t>(stream), nullptr);
  StepIO io;
  io.phases = PH_BWD;
  io.x = x; io.dy = dy; io.dx = dx;
  io.N = N; io.M = M; io.remat = remat;
  io.ws = static_cast<char*>(workspace); io.ws_bytes = ws_bytes;
  io.s = static_cast<hipStream_t>(stream);
  return transformer_run(c, io);
}

gpipe_status gpipe_cell_step_noalloc(gpipe_cell* c, const void* x, const void* target, void* y,
                                     void* dx, int N, int M, int remat, void* stream,
                                     float* loss_dev) {
  if (!c) return GPIPE_ERR_INVALID;
  if (!c->bound) return GPIPE_ERR_STATE;
  if (c->kind == CELL_CONV) return GPIPE_ERR_UNSUPPORTED;
  Plan p;
  if (!make_plan(c, N, M, remat, &p)) return GPIPE_ERR_INVALID;
  if (p.total > GPIPE_SCRATCH_BYTES) return GPIPE_ERR_OOM;
  void* ws = nullptr;
  {
    const gpipe_status st = scratch_of_current_device(&ws);
    if (st != GPIPE_OK) return st;
  }
  StepIO io;
  io.phases = PH_FWD | PH_BWD;
  io.x = x; io.target = target; io.y = y; io.dx = dx; io.loss_dev = loss_dev;
  io.N = N; io.M = M; io.remat = remat;
  io.ws = static_cast<char*>(ws); io.ws_bytes = GPIPE_SCRATCH_BYTES;
  io.s = static_cast<hipStream_t>(stream);
  io.single = true;
  return transformer_run(c, io);
}

gpipe_status gpipe_cell_set_logit_clip(gpipe_cell* c, float threshold) {
  if (!c || c->kind != CELL_TRANSFORMER || !(threshold >= 0.f) || !isfinite(threshold))
    return GPIPE_ERR_INVALID;
  c->logit_clip = threshold;
  return GPIPE_OK;
}

gpipe_status gpipe_cell_scale_ffn_init(gpipe_cell* c, int total_layers, void* stream) {
  if (!c || c->kind != CELL_TRANSFORMER || total_layers < 1) return GPIPE_ERR_INVALID;
  if (!c->bound) return GPIPE_ERR_STATE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  for (int l = 0; l < c->L; ++l)
    for (const int t : {GPIPE_W_1, GPIPE_W_2}) {
      const size_t off = size_t(l) * c->per_layer + c->rel_off[t];
      GP_CHECK(div_scalar(c->master + off, int64_t(c->count[t]), float(total_layers), s));
      if (c->prec == GPIPE_BF16)
        GP_CHECK(to_bf16(c->master + off, static_cast<uint16_t*>(c->w_lowp) + off,
                         int64_t(c->count[t]), s));
    }
  return GPIPE_OK;
}

gpipe_status gpipe_apply_update(gpipe_cell* c, float lr, float decay, float eps, void* stream) {
  if (!c) return GPIPE_ERR_INVALID;
  if (!c->bound) return GPIPE_ERR_STATE;
  if (!update_args_ok(lr, decay, eps)) return GPIPE_ERR_INVALID;
  Ctx cx{c, c->prof_mask ? c : nullptr, nullptr, nullptr, static_cast<hipStream_t>(stream),
         c->prec == GPIPE_BF16, 0};
  GP_RUN(cx, GPIPE_ROLE_RMSPROP,
         rmsprop(c->master, c->grad, c->ms, c->prec == GPIPE_BF16 ? c->w_lowp : nullptr,
                 int64_t(c->n_params), lr, decay, eps, cx.s));
  return GPIPE_OK;
}

gpipe_status gpipe_cell_profile_sampled(gpipe_cell* c, unsigned long long role_mask, int every) {
  if (!c || every < 1) return GPIPE_ERR_INVALID;
  c->prof_mask = role_mask;
  c->prof_every = every;
  c->prof_seen.assign(GPIPE_N_ROLES, 0);
  c->prof_roles.clear();
  return GPIPE_OK;
}

gpipe_status gpipe_cell_profile(gpipe_cell* c, unsigned long long role_mask) {
  return gpipe_cell_profile_sampled(c, role_mask, 1);
}

gpipe_status gpipe_cell_profile_read(gpipe_cell* c, int role, double* total_ms, long long* launches) {
  if (!c || !total_ms || !launches || role < 0 || role >= GPIPE_N_ROLES) return GPIPE_ERR_INVALID;
  double t = 0.0;
  long long n = 0;
  for (size_t i = 0; i < c->prof_roles.size(); ++i) {
    if (c->prof_roles[i] != role) continue;
    float ms = 0.f;
    if (hipEventSynchronize(c->prof_events[2 * i + 1]) != hipSuccess) return GPIPE_ERR_DEVICE;
    if (hipEventElapsedTime(&ms, c->prof_events[2 * i], c->prof_events[2 * i + 1]) != hipSuccess)
      return GPIPE_ERR_DEVICE;
    t += ms;
    ++n;
  }
  *total_ms = t;
  *launches = n;
  return GPIPE_OK;
}

gpipe_status gpipe_cell_forward_plan(const gpipe_cell* c, int N, int M, int remat, int* lanes,
                                     int* group, size_t* lane_partial_bytes) {
  if (!c || !lanes || !group || !lane_partial_bytes || c->kind != CELL_TRANSFORMER)
    return GPIPE_ERR_INVALID;
  Plan p;
  if (!make_plan(c, N, M, remat, &p)) return GPIPE_ERR_INVALID;
  *lanes = p.fwd_lanes;
  *group = p.fwd_group;
  *lane_partial_bytes = p.splitk2 - p.splitk;
  return GPIPE_OK;
}

gpipe_status gpipe_cell_gemm_plan(const gpipe_cell* c, int N, int M, int role, int* tile_m,
                                  int* tile_n, int* splits) {
  if (!c || !tile_m || !tile_n || !splits || role < 0 || role >= GPIPE_N_ROLES)
    return GPIPE_ERR_INVALID;
  if (c->kind == CELL_CONV) return conv_gemm_plan(c, N, M, role, tile_m, tile_n, splits);
  Plan p;
  if (!make_plan(c, N, M, 1, &p)) return GPIPE_ERR_INVALID;
  const int T = p.T, D = c->D, F = c->F, S = c->S, dh = c->D / c->H, bh = p.B * c->H;
  int mnk[4] = {0, 0, 0, 0};  // M, N, K, batch
  switch (role) {
    case GPIPE_ROLE_QKV_FWD: mnk[0] = T; mnk[1] = 3 * D; mnk[2] = D; break;
    case GPIPE_ROLE_OUT_FWD: mnk[0] = T; mnk[1] = D; mnk[2] = D; break;
    case GPIPE_ROLE_FFN1_FWD: mnk[0] = T; mnk[1] = F; mnk[2] = D; break;
    case GPIPE_ROLE_FFN2_FWD: mnk[0] = T; mnk[1] = D; mnk[2] = F; break;
    case GPIPE_ROLE_FFN2_DGRAD: mnk[0] = T; mnk[1] = F; mnk[2] = D; break;
    case GPIPE_ROLE_FFN1_DGRAD: mnk[0] = T; mnk[1] = D; mnk[2] = F; break;
    case GPIPE_ROLE_OUT_DGRAD: mnk[0] = T; mnk[1] = D; mnk[2] = D; break;
    case GPIPE_ROLE_QKV_DGRAD: mnk[0] = T; mnk[1] = D; mnk[2] = 3 * D; break;
    case GPIPE_ROLE_FFN2_WGRAD: mnk[0] = D; mnk[1] = F; mnk[2] = T; break;
    case GPIPE_ROLE_FFN1_WGRAD: mnk[0] = F; mnk[1] = D; mnk[2] = T; break;
    case GPIPE_ROLE_OUT_WGRAD: mnk[0] = D; mnk[1] = D; mnk[2] = T; break;
    case GPIPE_ROLE_QKV_WGRAD: mnk[0] = 3 * D; mnk[1] = D; mnk[2] = T; break;
    case GPIPE_ROLE_SCORES_FWD: case GPIPE_ROLE_DP: mnk[0] = S; mnk[1] = S; mnk[2] = dh; break;
    case GPIPE_ROLE_PV_FWD: case GPIPE_ROLE_DV: case GPIPE_ROLE_DQ: case GPIPE_ROLE_DK:
      mnk[0] = S; mnk[1] = dh; mnk[2] = S; break;
    default:
      *tile_m = *tile_n = *splits = 0;
      return GPIPE_OK;
  }
  const bool attn = role == GPIPE_ROLE_SCORES_FWD || role == GPIPE_ROLE_DP || role == GPIPE_ROLE_PV_FWD ||
                    role == GPIPE_ROLE_DV || role == GPIPE_ROLE_DQ || role == GPIPE_ROLE_DK;
  const GemmPlan g = plan_gemm(role, c->prec == GPIPE_BF16, mnk[0], mnk[1], mnk[2], attn ? bh : 1);
  if (g.cfg < 0) {  // fp32 kernel
    *tile_m = *tile_n = 64;
  } else {
    *tile_m = gemm_cfg_bm(g.cfg);
    *tile_n = gemm_cfg_bn(g.cfg);
  }
  *splits = g.splits;
  return GPIPE_OK;
}

gpipe_status gpipe_partition(const double* costs, int L, int K, int* bounds, double* variance) {
  if (!costs || !bounds || L < 1 || K < 1 || K > L) return GPIPE_ERR_INVALID;
  for (int i = 0; i < L; ++i)
    if (!(costs[i] >= 0.0) || !isfinite(costs[i])) return GPIPE_ERR_INVALID;
  // Minimising the variance of the K cell sums C_k is minimising sum_k C_k^2
  // (their total is fixed).  g[k][i]: least sum of squares splitting layers
  // i..L-1 into k non-empty cells; the cuts are then read from the front,
  // always taking the earliest optimal cut, which gives the
  // lexicographically smallest bounds among the optima.
  std::vector<double> pre(L + 1, 0.0);
  for (int i = 0; i < L; ++i) pre[i + 1] = pre[i] + costs[i];
  const double inf = std::numeric_limits<double>::infinity();
  std::vector<double> g(size_t(K + 1) * (L + 1), inf);
  auto G = [&](int k, int i) -> double& { return g[size_t(k) * (L + 1) + i]; };
  G(0, L) = 0.0;
  for (int k = 1; k <= K; ++k)
    for (int i = 0; i <= L - k; ++i) {
      double best = inf;
      for (int j = i + 1; j <= L - (k - 1); ++j) {
        const double cj = pre[j] - pre[i];
        const double v = cj * cj + G(k - 1, j);
        if (v < best) best = v;
      }
      G(k, i) = best;
    }
  bounds[0] = 0;
  int i = 0;
  for (int k = K; k >= 1; --k) {
    int pick = -1;
    for (int j = i + 1; j <= L - (k - 1); ++j) {
      const double cj = pre[j] - pre[i];
      if (cj * cj + G(k - 1, j) == G(k, i)) {
        pick = j;
        break;
      }
    }
    if (pick < 0) return GPIPE_ERR_INVALID;  // unreachable for finite costs
    bounds[K - k + 1] = pick;
    i = pick;
  }
  if (variance) {
    const double mean = pre[L] / K;
    double v = 0.0;
    for (int k = 0; k < K; ++k) {
      const double ck = pre[bounds[k + 1]] - pre[bounds[k]] - mean;
      v += ck * ck;
    }
    *variance = v / K;
  }
  return GPIPE_OK;
}

}  // extern "C"
