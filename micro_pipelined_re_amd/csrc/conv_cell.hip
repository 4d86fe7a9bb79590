// Driver of the convolutional cell with micro-batch BatchNorm.
//
// Schedule (GPipe technical review page, "GPipe algorithm in detail"):
// forward phase over the M micro-batches keeping the boundary output, each
// micro-batch normalised with its own BatchNorm statistics ("BatchNorm
// handling"), whose moments are recorded; the moving averages are updated
// once from them; backward phase re-materializing each micro-batch and
// accumulating float32 gradients; the update is gpipe_apply_update.
#include "cell.hpp"

namespace gp {
namespace {

// Storage.  Micro-batch BatchNorm makes this cell's gradients the small
// remainder of near-cancellations: a relative rounding of 2^-9 in any forward
// activation (block output, conv output, ReLU output) moves dx and the weight
// gradients by 2-5% (measured on the float64 oracle at the 64- and
// 256-channel shapes), while the same rounding of the backward's gradients
// moves them by 0.1-0.4%.  So bf16 cells keep the forward exact to float32
// level: the convolution outputs a and z (the BatchNorm inputs) in float32,
// the block outputs and ReLU outputs -- the convolutions' input operands -- as
// split bf16 pairs [P][2C] (SK_SPLIT: hi + lo), convolved with the weights
// repeated over both halves; the backward's operands (dz, da) stay bf16, and
// the weight gradients read the hi halves.  Every saved tensor is then 4 bytes
// per element in both precisions.
//
// Byte layout of a conv-cell workspace for one (N, M, remat):
//   sets:  remat ? 1 : M micro-batch sets, each L blocks of the saved tensors
//          of gpipe_conv_saved (block 0 has no X slot in use)
//   yre:   output of the re-materialized forward [P, C] (act; remat only)
//   col:   im2col matrix (act): [P, 9 Cin] for the explicit forward (Cin = 2C
//          for split inputs), [P, 9C] for the explicit weight gradient
//   dcol:  [P, 9C] input-gradient columns (f32, explicit path)
//   wflip: tap-flipped transposed weights [L][2][C][9][C] (implicit path)
//   wdup:  weights repeated over split inputs [L][2][C][9][2C] (bf16 cells)
//   r0:    residual-stream gradient [P, C] (f32);  r1: ReLU-input gradient (f32)
//   dz:    BN input gradient [P, C] (act, GEMM operand), kDzCopies copies
//          used in turn (the weight gradients on the second stream read the
//          two of a block while the input-gradient chain writes the next)
//   part, sums: BN reduction partials;  rec: forward-phase moments [M][2L][2][C]
//   msepart, splitk
// Copies of dz: a block's two BatchNorm backwards each write one, so with four
// the copy written was last read by the weight gradients of the block two
// above, which have long finished.
constexpr int kDzCopies = 4;

struct CPlan {
  int N, M, B;
  bool implicit;  // bf16, channels a multiple of 64: implicit-GEMM convolutions
  bool implicit_wgrad;  // and the weight gradient too: pixels a multiple of 64, below 2^21
  int64_t P;  // pixels per micro-batch
  size_t eb;
  size_t saved_off[GPIPE_CONV_N_SAVED], saved_bytes[GPIPE_CONV_N_SAVED];
  size_t block_bytes, set_bytes;
  int nsets;
  size_t yre, col, dcol, r0, r1, dz[4], part, sums, rec, msepart, splitk, wflip, wdup;
  bool split;  // bf16 cells: split forward activations (see above)
  // forward-phase lanes (see conv_cell_step): count, and the BN / split-K
  // partials of lanes 1 and 2 (lane 0 uses part and splitk)
  int lanes;
  size_t lane_part[3], lane_splitk[3];
  // pipelined backward (see conv_cell_step): with re-materialization and the
  // implicit weight gradient on at least two blocks; wsplitk: the split-K
  // partials of the weight gradients on the second stream
  bool piped;
  size_t wsplitk;
  int mse_nblk;
  size_t total;
};

bool make_cplan(const gpipe_cell* c, int N, int M, int remat, CPlan* p) {
  if (N <= 0 || M <= 0 || N % M) return false;
  p->N = N;
  p->M = M;
  p->B = N / M;
  const size_t C = c->C;
  const size_t P = size_t(p->B) * c->Hc * c->Wc;
  if (P * 9 * C > size_t(1) << 40) return false;
  p->P = int64_t(P);
  const size_t eb = c->prec == GPIPE_BF16 ? 2 : 4;
  p->eb = eb;
  p->split = c->prec == GPIPE_BF16;
  // x, r: f32 [P][C] or split [P][2C] bf16; a, z: f32 -- 4 bytes per element
  const size_t sizes[GPIPE_CONV_N_SAVED] = {P * C * 4, P * C * 4, 2 * C * 4,
                                            P * C * 4, P * C * 4, 2 * C * 4};
  size_t off = 0;
  for (int i = 0; i < GPIPE_CONV_N_SAVED; ++i) {
    p->saved_off[i] = off;
    p->saved_bytes[i] = sizes[i];
    off += align_up(sizes[i], kAlign);
  }
  p->block_bytes = off;
  p->set_bytes = size_t(c->L) * off;
  p->nsets = remat ? 1 : M;
  p->implicit = c->prec == GPIPE_BF16 && C % 64 == 0;
  p->implicit_wgrad = p->implicit && P % 64 == 0 && P < (size_t(1) << 21) &&
                      (P + 64) * C < (size_t(1) << 31);
  p->piped = remat && p->implicit_wgrad && c->L >= 2;
  // pipelined, one spare block slot after the set (block index L): the next
  // micro-batch's block 0 is re-materialized there (conv_cell_run)
  size_t o = size_t(p->nsets) * p->set_bytes + (p->piped ? p->block_bytes : 0);
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes, kAlign);
    return at;
  };
  const size_t cin = p->split ? 2 * C : C;  // channels of a forward convolution's input
  p->yre = take(remat ? P * C * eb : 0);
  p->col = take(!p->implicit ? P * 9 * cin * eb : p->implicit_wgrad ? 0 : P * 9 * C * eb);
  p->dcol = take(p->implicit ? 0 : P * 9 * C * 4);
  p->wflip = take(p->implicit ? size_t(c->L) * 2 * 9 * C * C * 2 : 0);
  p->wdup = take(p->split ? size_t(c->L) * 2 * 9 * C * cin * 2 : 0);
  p->r0 = take(P * C * 4);
  p->r1 = take(P * C * 4);
  for (int k = 0; k < kDzCopies; ++k) p->dz[k] = take(P * C * eb);
  p->part = take(size_t(bn_chunks(int64_t(P))) * 2 * C * 4);
  p->sums = take(2 * C * 4);
  p->rec = take(size_t(M) * 2 * c->L * 2 * C * 4);
  p->mse_nblk = mse_blocks(int64_t(P * C));
  p->msepart = take(size_t(M) * p->mse_nblk * 4);
  const bool bf = c->prec == GPIPE_BF16;
  const int Pi = int(P), Ci = int(C);
  const int Ki = int(9 * cin);  // k extent of a forward convolution of a split input
  const size_t skf = std::max({gemm_partial_floats(GPIPE_ROLE_CONV_FWD, bf, Pi, Ci, 9 * Ci, 1),
                               gemm_partial_floats(GPIPE_ROLE_CONV_FWD, bf, Pi, Ci, Ki, 1),
                               gemm_partial_floats(GPIPE_ROLE_CONV_FWD_IMPLICIT, bf, Pi, Ci, 9 * Ci, 1),
                               gemm_partial_floats(GPIPE_ROLE_CONV_FWD_IMPLICIT, bf, Pi, Ci, Ki, 1)});
  const size_t sk = std::max({skf,
                              gemm_partial_floats(GPIPE_ROLE_CONV_DGRAD, bf, Pi, 9 * Ci, Ci, 1),
                              gemm_partial_floats(GPIPE_ROLE_CONV_WGRAD, bf, Ci, 9 * Ci, Pi, 1),
                              gemm_partial_floats(GPIPE_ROLE_CONV_DGRAD_IMPLICIT, bf, Pi, Ci, 9 * Ci, 1),
                              gemm_partial_floats(GPIPE_ROLE_CONV_WGRAD_IMPLICIT, bf, Ci, 9 * Ci, Pi, 1)});
  p->splitk = take(sk * 4);
  // lanes of the forward phase: implicit convolutions and at least two
  // blocks (their partials are laid out with or without re-materialization,
  // so that the two workspaces differ by the saved sets only)
  p->lanes = p->implicit && c->L >= 2 ? std::min(3, c->L) : 1;
  p->lane_part[0] = p->part;
  p->lane_splitk[0] = p->splitk;
  for (int k = 1; k < 3; ++k) {
    p->lane_part[k] = take(k < p->lanes ? size_t(bn_chunks(int64_t(P))) * 2 * C * 4 : 0);
    p->lane_splitk[k] = take(k < p->lanes ? skf * 4 : 0);
  }
  p->wsplitk = take(p->implicit_wgrad && c->L >= 2
                        ? gemm_partial_floats(GPIPE_ROLE_CONV_WGRAD_IMPLICIT, bf, Ci, 9 * Ci, Pi, 1) * 4
                        : 0);
  p->total = o;
  return true;
}

inline size_t csaved_at(const CPlan& p, int set, int block, int which) {
  return size_t(set) * p.set_bytes + size_t(block) * p.block_bytes + p.saved_off[which];
}

struct CCtx {
  const gpipe_cell* c;
  gpipe_cell* prof;
  const CPlan* p;
  char* ws;
  hipStream_t s;
  bool bf16;
  size_t part, splitk;  // workspace offsets of this stream's BN and split-K partials
  const void* wmat(int block, int t) const {
    const size_t off = size_t(block) * c->per_layer + c->rel_off[t];
    if (bf16) return static_cast<const uint16_t*>(c->w_lowp) + off;
    return c->master + off;
  }
  const float* wf32(int block, int t) const {
    return c->master + size_t(block) * c->per_layer + c->rel_off[t];
  }
  float* grad(int block, int t) const {
    return c->grad + size_t(block) * c->per_layer + c->rel_off[t];
  }
  void* at(size_t off) const { return ws + off; }
  float* f(size_t off) const { return reinterpret_cast<float*>(ws + off); }
  void* act(const void* base, size_t elems) const {
    return const_cast<char*>(static_cast<const char*>(base)) + elems * p->eb;
  }
  // tap-flipped transposed weights of conv `which` (0: W1, 1: W2) of block l
  const void* flipped(int block, int which) const {
    const size_t n = size_t(9) * c->C * c->C;
    return ws + p->wflip + (size_t(block) * 2 + which) * n * 2;
  }
  // the same convolution's weights repeated over a split input's halves
  const void* dup(int block, int which) const {
    const size_t n = size_t(9) * c->C * 2 * c->C;
    return ws + p->wdup + (size_t(block) * 2 + which) * n * 2;
  }
  // storage of the caller's activations and of the block boundaries / ReLU outputs
  int act_kind() const { return bf16 ? SK_BF16 : SK_F32; }
  int xs_kind() const { return p->split ? SK_SPLIT : SK_F32; }
};

hipError_t cmm(const CCtx& x, int role, int M, int N, int K, const void* A, int64_t lda,
               const void* B, int64_t ldb, void* C, int64_t ldc, int beta = 0) {
  GemmParams g;
  memset(&g, 0, sizeof(g));
  g.hdiv = 1;
  g.alpha = 1.0f;
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda;
  g.B = B; g.ldb = ldb;
  g.C = C; g.ldc = ldc;
  g.beta = beta;
  g.P = x.f(x.splitk);
  return gemm(x.bf16, role, g, 1, x.s);
}

// Implicit-GEMM convolution of an NHWC image [P, cin] with [C][9 cin] weights
// (k-contiguous): out[P, C] f32 (beta: accumulate).
hipError_t cconv(const CCtx& x, int role, const void* img, int cin, const void* w, void* out,
                 int beta) {
  GemmParams g;
  memset(&g, 0, sizeof(g));
  const int C = x.c->C;
  g.hdiv = 1;
  g.alpha = 1.0f;
  g.M = int(x.p->P); g.N = C; g.K = 9 * cin;
  g.A = img; g.lda = cin;
  g.B = w; g.ldb = 9 * cin;
  g.C = out; g.ldc = C;
  g.beta = beta;
  g.conv_h = x.c->Hc; g.conv_w = x.c->Wc; g.conv_c = cin;
  g.P = x.f(x.splitk);
  return gemm(true, role, g, 1, x.s);
}

// Weight gradient of a convolution: grad (+)= dz^T im2col(img), [C][9C] f32,
// img the first C channels of an image of pixel stride img_ld (the hi half of
// a split activation).
gpipe_status cwgrad(const CCtx& x, const void* img, int img_ld, const void* dz, float* grad,
                    int beta) {
  const gpipe_cell* c = x.c;
  const int C = c->C;
  const int P = int(x.p->P);
  if (!x.p->implicit_wgrad) {
    void* col = x.at(x.p->col);
    GP_RUN(x, GPIPE_ROLE_IM2COL, im2col(x.bf16, img, img_ld, col, x.p->B, c->Hc, c->Wc, C, x.s));
    GP_RUN(x, GPIPE_ROLE_CONV_WGRAD,
           cmm(x, GPIPE_ROLE_CONV_WGRAD, C, 9 * C, P, dz, C, col, 9 * C, grad, 9 * C, beta));
    return GPIPE_OK;
  }
  GemmParams g;
  memset(&g, 0, sizeof(g));
  g.hdiv = 1;
  g.alpha = 1.0f;
  g.M = C; g.N = 9 * C; g.K = P;
  g.A = dz; g.lda = C;
  g.B = img; g.ldb = 9 * C;
  g.C = grad; g.ldc = 9 * C;
  g.beta = beta;
  g.conv_h = c->Hc; g.conv_w = c->Wc; g.conv_c = C;
  g.conv_ld = img_ld;
  g.P = x.f(x.splitk);
  GP_RUN(x, GPIPE_ROLE_CONV_WGRAD_IMPLICIT, gemm(true, GPIPE_ROLE_CONV_WGRAD_IMPLICIT, g, 1, x.s));
  return GPIPE_OK;
}

// One block forward of one micro-batch; rec (nullable) receives the BN
// moments [2][2][C] of this block (forward phase only).
// (slot: the block slot of `set` that receives the saved tensors; l: the
// block whose weights apply -- the same except in the forward phase's lanes)
gpipe_status block_forward(const CCtx& x, int set, int slot, int l, const void* xin, void* xout,
                           float* rec) {
  const gpipe_cell* c = x.c;
  const CPlan& p = *x.p;
  const int C = c->C, B = p.B, H = c->Hc, W = c->Wc;
  const int64_t P = p.P;
  void* a = x.at(csaved_at(p, set, slot, GPIPE_CONV_SAVED_A));
  float* st1 = x.f(csaved_at(p, set, slot, GPIPE_CONV_SAVED_ST1));
  void* r = x.at(csaved_at(p, set, slot, GPIPE_CONV_SAVED_R));
  void* z = x.at(csaved_at(p, set, slot, GPIPE_CONV_SAVED_Z));
  float* st2 = x.f(csaved_at(p, set, slot, GPIPE_CONV_SAVED_ST2));
  float* part = x.f(x.part);
  // block 0 reads the caller's x, the last block writes the caller's y (or
  // the re-materialized output), both in the cell's activation type; the
  // boundaries between blocks and the ReLU outputs are split in bf16 cells
  const int in_kind = l == 0 ? x.act_kind() : x.xs_kind();
  const int out_kind = l == c->L - 1 ? x.act_kind() : x.xs_kind();
  const int r_kind = x.xs_kind();
  // conv(img, W_which): a split image meets the repeated weights over 2C channels
  auto conv = [&](const void* img, int kind, int which, float* out) -> gpipe_status {
    const int cin = kind == SK_SPLIT ? 2 * C : C;
    const void* w = kind == SK_SPLIT ? x.dup(l, which)
                                     : x.wmat(l, which == 0 ? GPIPE_CONV_W1 : GPIPE_CONV_W2);
    if (p.implicit) {
      GP_RUN(x, GPIPE_ROLE_CONV_FWD_IMPLICIT,
             cconv(x, GPIPE_ROLE_CONV_FWD_IMPLICIT, img, cin, w, out, 0));
    } else {
      void* col = x.at(p.col);
      GP_RUN(x, GPIPE_ROLE_IM2COL, im2col(x.bf16, img, cin, col, B, H, W, cin, x.s));
      GP_RUN(x, GPIPE_ROLE_CONV_FWD, cmm(x, GPIPE_ROLE_CONV_FWD, int(P), C, 9 * cin, col, 9 * cin,
                                         w, 9 * cin, out, C));
    }
    return GPIPE_OK;
  };
  {
    const gpipe_status st = conv(xin, in_kind, 0, static_cast<float*>(a));
    if (st != GPIPE_OK) return st;
  }
  GP_RUN(x, GPIPE_ROLE_BN_STATS, bn_stats(false, a, P, C, c->bn_eps, part, st1, rec, x.s));
  GP_RUN(x, GPIPE_ROLE_BN_APPLY, bn_apply(0, static_cast<const float*>(a), st1,
                                          x.wf32(l, GPIPE_CONV_BN1_G), x.wf32(l, GPIPE_CONV_BN1_B),
                                          nullptr, SK_F32, r, r_kind, P, C, x.s));
  {
    const gpipe_status st = conv(r, r_kind, 1, static_cast<float*>(z));
    if (st != GPIPE_OK) return st;
  }
  GP_RUN(x, GPIPE_ROLE_BN_STATS,
         bn_stats(false, z, P, C, c->bn_eps, part, st2, rec ? rec + 2 * C : nullptr, x.s));
  GP_RUN(x, GPIPE_ROLE_BN_APPLY, bn_apply(1, static_cast<const float*>(z), st2,
                                          x.wf32(l, GPIPE_CONV_BN2_G), x.wf32(l, GPIPE_CONV_BN2_B),
                                          xin, in_kind, xout, out_kind, P, C, x.s));
  return GPIPE_OK;
}

gpipe_status cell_forward(const CCtx& x, int set, const void* xin, void* yout, float* rec) {
  const int L = x.c->L, C = x.c->C;
  for (int l = 0; l < L; ++l) {
    const void* in = l == 0 ? xin : x.at(csaved_at(*x.p, set, l, GPIPE_CONV_SAVED_X));
    void* out = l == L - 1 ? yout : x.at(csaved_at(*x.p, set, l + 1, GPIPE_CONV_SAVED_X));
    gpipe_status st = block_forward(x, set, l, l, in, out, rec ? rec + size_t(l) * 4 * C : nullptr);
    if (st != GPIPE_OK) return st;
  }
  return GPIPE_OK;
}

// Backward of block l (saved tensors in `slot` of `set`).  On entry r0 holds
// the gradient w.r.t. the block output (f32); on exit the gradient w.r.t.
// its input (r0, and dx_out when given).  With streams (ss) the two weight
// gradients run on the second stream, handed over together after BN1's
// backward (one hand-off event, recorded in the dispatch of that backward's
// last kernel): W2's reads the copy of dz that BN2's backward
// wrote, W1's the copy BN1's wrote, and each BatchNorm backward writes the
// other copy than the last one, waiting only for that copy's readers.
gpipe_status block_backward(const CCtx& x, Streams* ss, Transient* tdz, int set, int slot, int l,
                            const void* xin, int beta, void* dx_out, hipEvent_t* s1_done = nullptr) {
  const gpipe_cell* c = x.c;
  const CPlan& p = *x.p;
  const int C = c->C, B = p.B, H = c->Hc, W = c->Wc;
  const int64_t P = p.P;
  const float* a = x.f(csaved_at(p, set, slot, GPIPE_CONV_SAVED_A));
  const float* st1 = x.f(csaved_at(p, set, slot, GPIPE_CONV_SAVED_ST1));
  const void* r = x.at(csaved_at(p, set, slot, GPIPE_CONV_SAVED_R));
  const float* z = x.f(csaved_at(p, set, slot, GPIPE_CONV_SAVED_Z));
  // pixel strides of the weight gradients' images: the hi halves of split ones
  const int r_ld = x.xs_kind() == SK_SPLIT ? 2 * C : C;
  const int x_ld = (l == 0 || x.xs_kind() != SK_SPLIT) ? C : 2 * C;
  const float* st2 = x.f(csaved_at(p, set, slot, GPIPE_CONV_SAVED_ST2));
  CCtx w = x;  // the weight gradients' context
  if (ss) {
    w.s = ss->s2;
    w.splitk = p.wsplitk;
  }
  float* dcol = x.f(p.dcol);
  float* r0 = x.f(p.r0);
  float* r1 = x.f(p.r1);
  float* part = x.f(p.part);
  float* sums = x.f(p.sums);
  int nch = 0;
  // y = x + BN2(z) (the gain and shift gradients, adjacent, accumulate in the same pass)
  if (!tdz->next(ss)) return GPIPE_ERR_DEVICE;
  const int k2 = tdz->cur;
  void* dz2 = x.at(tdz->off[k2]);
  GP_RUN(x, GPIPE_ROLE_BN_BWD, bn_bwd(x.act_kind(), 0, r0, nullptr, SK_F32, z, st2,
                                      x.wf32(l, GPIPE_CONV_BN2_G), part, sums,
                                      x.grad(l, GPIPE_CONV_BN2_G), beta, dz2, P, C, &nch, x.s));
  // z = conv(r, W2)
  if (p.implicit) {
    GP_RUN(x, GPIPE_ROLE_CONV_DGRAD_IMPLICIT,
           cconv(x, GPIPE_ROLE_CONV_DGRAD_IMPLICIT, dz2, C, x.flipped(l, 1), r1, 0));
  } else {
    GP_RUN(x, GPIPE_ROLE_CONV_DGRAD, cmm(x, GPIPE_ROLE_CONV_DGRAD, int(P), 9 * C, C, dz2, C,
                                         x.wmat(l, GPIPE_CONV_W2), 9 * C, dcol, 9 * C));
    GP_RUN(x, GPIPE_ROLE_COL2IM, col2im(x.bf16, dcol, nullptr, r1, nullptr, B, H, W, C, x.s));
  }
  // r = ReLU(BN1(a))
  if (!tdz->next(ss)) return GPIPE_ERR_DEVICE;
  const int k1 = tdz->cur;
  void* dz1 = x.at(tdz->off[k1]);
  // (the hand-off events are recorded in the dispatches of the kernels they
  // follow: BN1's backward on the caller's stream, the weight gradients)
  if (ss) ss->fork_begin();
  GP_RUN(x, GPIPE_ROLE_BN_BWD, bn_bwd(x.act_kind(), 1, r1, r, x.xs_kind(), a, st1,
                                      x.wf32(l, GPIPE_CONV_BN1_G), part, sums,
                                      x.grad(l, GPIPE_CONV_BN1_G), beta, dz1, P, C, &nch, x.s));
  // the weight gradients of W2 and W1 (in that order on the second stream)
  if (ss && !ss->fork_end()) return GPIPE_ERR_DEVICE;
  {
    hipEvent_t ev = ss ? ss->mark_begin() : nullptr;
    gpipe_status st = cwgrad(w, r, r_ld, dz2, x.grad(l, GPIPE_CONV_W2), beta);
    if (st != GPIPE_OK) return st;
    if (!tdz->read_by_s2_at(ss, k2, ev)) return GPIPE_ERR_DEVICE;
    ev = ss ? ss->mark_begin() : nullptr;
    st = cwgrad(w, xin, x_ld, dz1, x.grad(l, GPIPE_CONV_W1), beta);
    if (st != GPIPE_OK) return st;
    if (!tdz->read_by_s2_at(ss, k1, ev)) return GPIPE_ERR_DEVICE;
  }
  // a = conv(x, W1); the residual gradient r0 is added in col2im (in place)
  // (s1_done: an event the implicit input-gradient convolution, then the
  // block's last kernel on the caller's stream, records in its dispatch)
  const bool tail = s1_done && ss && !ss->single && p.implicit && !dx_out;
  if (tail) next_done_event() = *s1_done = ss->next();
  if (p.implicit) {
    // the residual gradient already in r0 gets the convolution's input gradient added
    GP_RUN(x, GPIPE_ROLE_CONV_DGRAD_IMPLICIT,
           cconv(x, GPIPE_ROLE_CONV_DGRAD_IMPLICIT, dz1, C, x.flipped(l, 0), r0, 1));
    if (dx_out) GP_CHECK(to_bf16(r0, dx_out, P * C, x.s));
  } else {
    GP_RUN(x, GPIPE_ROLE_CONV_DGRAD, cmm(x, GPIPE_ROLE_CONV_DGRAD, int(P), 9 * C, C, dz1, C,
                                         x.wmat(l, GPIPE_CONV_W1), 9 * C, dcol, 9 * C));
    GP_RUN(x, GPIPE_ROLE_COL2IM, col2im(x.bf16, dcol, r0, r0, dx_out, B, H, W, C, x.s));
  }
  if (tail && next_done_event() == *s1_done) {
    next_done_event() = nullptr;
    GP_CHECK(hipEventRecord(*s1_done, x.s));
  }
  return GPIPE_OK;
}

}  // namespace

gpipe_status conv_cell_init(gpipe_cell* c) {
  const size_t C = c->C;
  const size_t cnt[GPIPE_CONV_N_TENSORS] = {9 * C * C, C, C, 9 * C * C, C, C};
  size_t off = 0;
  for (int t = 0; t < GPIPE_CONV_N_TENSORS; ++t) {
    c->rel_off[t] = off;
    c->count[t] = cnt[t];
    off += cnt[t];
  }
  c->per_layer = off;
  c->n_params = off * size_t(c->L);
  return GPIPE_OK;
}

bool conv_workspace_bytes(const gpipe_cell* c, int N, int M, int remat, size_t* bytes) {
  CPlan p;
  if (!make_cplan(c, N, M, remat, &p)) return false;
  *bytes = p.total;
  return true;
}

bool conv_saved_offset(const gpipe_cell* c, int N, int M, int remat, int micro, int block,
                       int which, size_t* offset, size_t* bytes) {
  CPlan p;
  if (!make_cplan(c, N, M, remat, &p)) return false;
  if (micro < 0 || micro >= p.nsets || block < 0 || block >= c->L || which < 0 ||
      which >= GPIPE_CONV_N_SAVED || (block == 0 && which == GPIPE_CONV_SAVED_X))
    return false;
  *offset = csaved_at(p, micro, block, which);
  *bytes = p.saved_bytes[which];
  return true;
}

gpipe_status conv_gemm_plan(const gpipe_cell* c, int N, int M, int role, int* tile_m, int* tile_n,
                            int* splits) {
  CPlan p;
  if (!make_cplan(c, N, M, 1, &p)) return GPIPE_ERR_INVALID;
  const int P = int(p.P), C = c->C;
  const int cin = p.split ? 2 * C : C;  // a forward convolution's input channels (blocks > 0)
  int m = 0, n = 0, k = 0;
  switch (role) {
    case GPIPE_ROLE_CONV_FWD: m = P; n = C; k = 9 * cin; break;
    case GPIPE_ROLE_CONV_DGRAD: m = P; n = 9 * C; k = C; break;
    case GPIPE_ROLE_CONV_WGRAD: case GPIPE_ROLE_CONV_WGRAD_IMPLICIT: m = C; n = 9 * C; k = P; break;
    case GPIPE_ROLE_CONV_FWD_IMPLICIT: m = P; n = C; k = 9 * cin; break;
    case GPIPE_ROLE_CONV_DGRAD_IMPLICIT: m = P; n = C; k = 9 * C; break;
    default:
      *tile_m = *tile_n = *splits = 0;
      return GPIPE_OK;
  }
  const GemmPlan g = plan_gemm(role, c->prec == GPIPE_BF16, m, n, k, 1);
  *tile_m = g.cfg < 0 ? 64 : gemm_cfg_bm(g.cfg);
  *tile_n = g.cfg < 0 ? 64 : gemm_cfg_bn(g.cfg);
  *splits = g.splits;
  return GPIPE_OK;
}

gpipe_status conv_cell_step(gpipe_cell* c, const void* x, const void* target, void* y, void* dx,
                            int N, int M, int remat, void* workspace, size_t ws_bytes,
                            hipStream_t stream, float* loss_dev) {
  return conv_cell_run(c, 3, x, target, nullptr, y, dx, N, M, remat, workspace, ws_bytes, stream,
                       loss_dev);
}

gpipe_status conv_cell_run(gpipe_cell* c, int phases, const void* x, const void* target,
                           const void* dy, void* y, void* dx, int N, int M, int remat,
                           void* workspace, size_t ws_bytes, hipStream_t stream, float* loss_dev) {
  CPlan p;
  if (!make_cplan(c, N, M, remat, &p)) return GPIPE_ERR_INVALID;
  if (!c->running) return GPIPE_ERR_STATE;
  const bool fwd = phases & 1, bwd = phases & 2;
  if (!x || !workspace || ws_bytes < p.total || (fwd && !y)) return GPIPE_ERR_INVALID;
  // the backward's output gradient: the loss (needs y, target, loss_dev) or dy
  if (bwd && (target ? (!y || !loss_dev || dy) : !dy)) return GPIPE_ERR_INVALID;
  if (!aligned16(x) || (target && !aligned16(target)) || (y && !aligned16(y)) ||
      (dy && !aligned16(dy)) || (dx && !aligned16(dx)) || !aligned16(workspace))
    return GPIPE_ERR_INVALID;
  CCtx cx{c, c->prof_mask ? c : nullptr, &p, static_cast<char*>(workspace), stream,
          c->prec == GPIPE_BF16, p.part, p.splitk};
  next_done_event() = nullptr;  // (nothing pending from an earlier call that failed)
  const size_t mb = size_t(p.P) * c->C;
  const float inv_denom = float(1.0 / (double(N) * c->Hc * c->Wc * c->C));
  float* rec = cx.f(p.rec);
  float* msepart = cx.f(p.msepart);
  const size_t rec_mb = size_t(2) * c->L * 2 * c->C;
  // the weights repeated over split inputs, for every forward and
  // re-materialized convolution of the call
  if (p.split && (fwd || remat))
    for (int l = 0; l < c->L; ++l) {
      GP_CHECK(conv_dup_weights(cx.wmat(l, GPIPE_CONV_W1), const_cast<void*>(cx.dup(l, 0)), c->C,
                                stream));
      GP_CHECK(conv_dup_weights(cx.wmat(l, GPIPE_CONV_W2), const_cast<void*>(cx.dup(l, 1)), c->C,
                                stream));
    }
  // the tap-flipped weights of the input gradients, once per backward phase
  if (p.implicit && bwd)
    for (int l = 0; l < c->L; ++l) {
      GP_CHECK(conv_flip_weights(cx.wmat(l, GPIPE_CONV_W1), const_cast<void*>(cx.flipped(l, 0)),
                                 c->C, stream));
      GP_CHECK(conv_flip_weights(cx.wmat(l, GPIPE_CONV_W2), const_cast<void*>(cx.flipped(l, 1)),
                                 c->C, stream));
    }
  // phase 1: forward; each micro-batch normalised with its own statistics.
  // With re-materialization only the boundary output is kept, so a
  // micro-batch needs one block's saved tensors, reused block after block
  // (the block's output overwrites its input, last read by the residual add
  // of its final BatchNorm apply).  The micro-batches are independent:
  // micro-batch m runs on lane m mod K (up to 3 streams: the caller's and the
  // cell's two) in block slot m mod K of set 0, with its own BN and split-K
  // partials, enqueued block by block so that every stream has work queued.
  // Role timing covers every stream (a launch's time is its own span, which
  // may share the CUs with the other streams' kernels).
  if (fwd && remat && p.lanes > 1) {
    {
      const gpipe_status st = ensure_streams(c);
      if (st != GPIPE_OK) return st;
    }
    Streams ss{c, stream, c->aux, c->aux2};
    const int K = p.lanes;
    CCtx lane[3] = {cx, cx, cx};
    for (int k = 0; k < 3; ++k) {
      lane[k].part = p.lane_part[k];
      lane[k].splitk = p.lane_splitk[k];
    }
    lane[1].s = ss.s2;
    lane[2].s = ss.s3;
    // (the flipped weights, inputs and weights exist)
    if (!ss.fork() || (K == 3 && !ss.fork3())) return GPIPE_ERR_DEVICE;
    for (int m0 = 0; m0 < M; m0 += K)
      for (int l = 0; l < c->L; ++l)
        for (int m = m0; m < std::min(M, m0 + K); ++m) {
          const int k = m % K;
          void* xs = cx.at(csaved_at(p, 0, k, GPIPE_CONV_SAVED_X));
          const void* in = l == 0 ? cx.act(x, m * mb) : xs;
          void* out = l == c->L - 1 ? cx.act(y, m * mb) : xs;
          gpipe_status st = block_forward(lane[k], 0, k, l, in, out,
                                          rec + m * rec_mb + size_t(l) * 4 * c->C);
          if (st != GPIPE_OK) return st;
        }
    if (!ss.join_all() || (K == 3 && !ss.join3())) return GPIPE_ERR_DEVICE;
  } else if (fwd) {
    for (int m = 0; m < M; ++m) {
      gpipe_status st = cell_forward(cx, remat ? 0 : m, cx.act(x, m * mb), cx.act(y, m * mb),
                                     rec + m * rec_mb);
      if (st != GPIPE_OK) return st;
    }
  }
  // the moving averages, once per step, from the forward phase's moments
  if (fwd)
    GP_RUN(cx, GPIPE_ROLE_BN_RUNNING, bn_running(rec, M, 2 * c->L, c->C,
                                                int64_t(N) * c->Hc * c->Wc, c->bn_momentum,
                                                c->running, stream));
  if (!bwd) return GPIPE_OK;
  // phase 2: re-materialize and backpropagate each micro-batch.  Pipelined
  // (p.piped): the weight gradients run on the second stream, and micro-batch
  // m+1 re-materializes on the third while micro-batch m's backward frees the
  // saved set's block slots, from the top block down: m+1 puts block 0 in a
  // spare slot as soon as m's backward starts (after its loss, which reads
  // the re-materialized output) and block j >= 1 in the slot m's block L-j
  // held, each enqueued after that slot's backward and weight gradients (the
  // slot m's block 0 frees is the next spare); a block's output goes to its
  // own slot's X tensor (the next block's input), the top block's to the
  // re-materialized output.  Micro-batch 0 re-materializes on the caller's
  // stream.
  const int L = c->L;
  std::vector<int> slots(L), next_slots(L);  // block -> slot, this / next micro-batch
  for (int j = 0; j < L; ++j) slots[j] = j;
  int spare = L;  // the slot the next micro-batch's block 0 takes
  Streams ss{c, stream, c->aux, c->aux2};
  CCtx cr = cx;  // the re-materialization's context on the third stream
  if (p.piped) {
    const gpipe_status st = ensure_streams(c);
    if (st != GPIPE_OK) return st;
    ss = Streams{c, stream, c->aux, c->aux2};
    cr.s = ss.s3;
    cr.part = p.lane_part[1];
    cr.splitk = p.lane_splitk[1];
  }
  auto remat_block = [&](const CCtx& z, int m, int j, const std::vector<int>& sl) {
    const void* in = j == 0 ? cx.act(x, m * mb) : z.at(csaved_at(p, 0, sl[j - 1], GPIPE_CONV_SAVED_X));
    void* out = j == L - 1 ? z.at(p.yre) : z.at(csaved_at(p, 0, sl[j], GPIPE_CONV_SAVED_X));
    return block_forward(z, 0, sl[j], j, in, out, nullptr);
  };
  Transient tdz;  // the BatchNorm input gradients the weight gradients read
  tdz.n = kDzCopies;
  for (int k = 0; k < kDzCopies; ++k) tdz.off[k] = p.dz[k];
  Streams* sp = p.piped ? &ss : nullptr;
  for (int m = 0; m < M; ++m) {
    const int set = remat ? 0 : m;
    const void* xm = cx.act(x, m * mb);
    const void* ym = y ? cx.act(y, m * mb) : nullptr;
    if (p.piped) {
      // this micro-batch's re-materialization is done (the third stream's
      // forks ordered it after the previous micro-batch's weight gradients
      // read their slots; dz waits per copy)
      if (m > 0 && !ss.join3()) return GPIPE_ERR_DEVICE;
      if (m == 0)
        for (int j = 0; j < L; ++j) {
          gpipe_status st = remat_block(cx, 0, j, slots);
          if (st != GPIPE_OK) return st;
        }
      ym = cx.at(p.yre);
    } else if (remat) {
      gpipe_status st = cell_forward(cx, set, xm, cx.at(p.yre), nullptr);
      if (st != GPIPE_OK) return st;
      ym = cx.at(p.yre);
    }
    // (the loss gradient's act copy goes to the next dz copy; the backward reads r0)
    if (!tdz.next(sp)) return GPIPE_ERR_DEVICE;
    if (target) {
      int nblk = 0;
      GP_RUN(cx, GPIPE_ROLE_MSE, mse_fwd_bwd(cx.bf16, ym, cx.act(target, m * mb), cx.f(p.r0),
                                             cx.at(tdz.off[tdz.cur]), msepart + size_t(m) * p.mse_nblk,
                                             int64_t(mb), inv_denom, &nblk, stream));
    } else {
      GP_CHECK(grad_in(cx.bf16, cx.act(dy, m * mb), cx.f(p.r0), cx.at(tdz.off[tdz.cur]), int64_t(mb),
                       stream));
    }
    const bool next = p.piped && m + 1 < M;
    if (next) {
      // the spare slot (micro-batch m-1's block 0, whose backward and weight
      // gradients are enqueued before this point) takes micro-batch m+1's block 0
      next_slots[0] = spare;
      if (!ss.fork3()) return GPIPE_ERR_DEVICE;
      gpipe_status st = remat_block(cr, m + 1, 0, next_slots);
      if (st != GPIPE_OK) return st;
    }
    for (int l = L - 1; l >= 0; --l) {
      const void* xin = l == 0 ? xm
                        : p.piped ? cx.at(csaved_at(p, set, slots[l - 1], GPIPE_CONV_SAVED_X))
                                  : cx.at(csaved_at(p, set, l, GPIPE_CONV_SAVED_X));
      void* dxo = (l == 0 && dx) ? cx.act(dx, m * mb) : nullptr;
      hipEvent_t s1_done = nullptr;
      gpipe_status st = block_backward(cx, sp, &tdz, set, slots[l], l,
                                       xin, m > 0 ? 1 : 0, dxo, next && l >= 1 ? &s1_done : nullptr);
      if (st != GPIPE_OK) return st;
      if (next && l >= 1) {
        // block l's slot is free once its backward (s1) and weight gradients
        // (s2) are done (the latter end with W1's, whose event is the dz copy's)
        const int j = L - l;
        next_slots[j] = slots[l];
        if (!ss.fork3_after(s1_done, tdz.read[tdz.cur])) return GPIPE_ERR_DEVICE;
        st = remat_block(cr, m + 1, j, next_slots);
        if (st != GPIPE_OK) return st;
      }
    }
    if (next) {
      spare = slots[0];  // freed by this micro-batch's block 0
      slots.swap(next_slots);
    }
  }
  // the weight gradients are complete
  if (p.piped && !ss.join_all()) return GPIPE_ERR_DEVICE;
  if (target)
    GP_RUN(cx, GPIPE_ROLE_LOSS_REDUCE, sum_partials(msepart, M * p.mse_nblk, 1, 1, loss_dev, 0, stream));
  return GPIPE_OK;
}

}  // namespace gp
