// Internal: the cell handle and helpers shared by the Transformer-cell and
// conv-cell drivers.
#pragma once
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/gpipe.h"
#include "kernels.hpp"

enum { CELL_TRANSFORMER = 0, CELL_CONV = 1 };

struct gpipe_cell {
  int kind;  // CELL_TRANSFORMER or CELL_CONV
  // Transformer cell: L layers of width D, H heads, FFN width F, sequence S.
  // Conv cell: L blocks of C channels on H x W images (in Hc, Wc).
  int L, D, H, F, S, causal;
  int C, Hc, Wc;
  float bn_momentum, bn_eps;
  float* running;  // conv cells: moving averages [L][2][2][C]
  gpipe_precision prec;
  float ln_eps;
  float logit_clip = 0.f;  // attention logit clipping threshold (0: off)
  size_t n_params;
  size_t per_layer;
  size_t rel_off[GPIPE_N_TENSORS];  // offsets inside one layer / block
  size_t count[GPIPE_N_TENSORS];
  float* master;
  void* w_lowp;
  float* grad;
  float* ms;
  bool bound;
  // Transformer cells: the second stream of the backward phase (the weight
  // gradients), the third (the next micro-batch's re-materialization) and
  // the ring of events ordering them against the caller's stream; created at
  // the first step, on the device current then.
  hipStream_t aux = nullptr, aux2 = nullptr;
  int aux_device = -1;
  std::vector<hipEvent_t> sync_events;
  size_t sync_next = 0;
  // event timing of selected kernel roles (gpipe_cell_profile)
  unsigned long long prof_mask = 0;
  int prof_every = 1;                    // time every prof_every-th launch of a role
  std::vector<long long> prof_seen;      // launches of each role since the profile call
  std::vector<hipEvent_t> prof_events;  // pool, pairs (start, end), reused
  std::vector<int> prof_roles;          // role of each recorded pair
};

namespace gp {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define GP_CHECK(expr)                              \
  do {                                              \
    if ((expr) != hipSuccess) return GPIPE_ERR_DEVICE; \
  } while (0)

// Next (start, end) event pair of the cell's pool for a launch of `role`.
inline bool prof_pair(gpipe_cell* c, int role, hipEvent_t* e0, hipEvent_t* e1) {
  const size_t k = 2 * c->prof_roles.size();
  while (c->prof_events.size() < k + 2) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return false;
    c->prof_events.push_back(e);
  }
  *e0 = c->prof_events[k];
  *e1 = c->prof_events[k + 1];
  c->prof_roles.push_back(role);
  return true;
}

// Whether this launch of a timed role is one of the sampled ones (every
// prof_every-th launch of the role, counting from the first).
inline bool prof_take(gpipe_cell* c, int role) {
  if (c->prof_every <= 1) return true;
  if (c->prof_seen.size() <= size_t(role)) c->prof_seen.resize(role + 1, 0);
  return c->prof_seen[role]++ % c->prof_every == 0;
}

// Launches `expr`; when `role` is being timed (and this launch is sampled), a
// GEMM role's launch records two events in its own dispatch
// (launch_events()), any other role is bracketed by two events recorded on
// the context's stream.
#define GP_RUN(ctx, role, expr)                                                         \
  do {                                                                                 \
    hipEvent_t e0_ = nullptr, e1_ = nullptr;                                           \
    const bool in_launch_ = gemm_role(role);                                           \
    if ((ctx).prof && (((ctx).prof->prof_mask >> (role)) & 1ull) &&                   \
        prof_take((ctx).prof, (role))) {                                               \
      if (!prof_pair((ctx).prof, (role), &e0_, &e1_)) return GPIPE_ERR_DEVICE;          \
      if (in_launch_)                                                                  \
        launch_events() = LaunchEvents{e0_, e1_};                                      \
      else if (hipEventRecord(e0_, (ctx).s) != hipSuccess)                             \
        return GPIPE_ERR_DEVICE;                                                       \
    }                                                                                  \
    if ((expr) != hipSuccess) return GPIPE_ERR_DEVICE;                                 \
    if (e1_ && in_launch_ && (launch_events().start || launch_events().stop)) {        \
      launch_events() = LaunchEvents{};                                                \
      return GPIPE_ERR_STATE; /* a GEMM launch path did not take the events */         \
    }                                                                                  \
    if (e1_ && !in_launch_ && hipEventRecord(e1_, (ctx).s) != hipSuccess)              \
      return GPIPE_ERR_DEVICE;                                                         \
  } while (0)

// Conv-cell driver (conv_cell.hip).
gpipe_status conv_cell_init(gpipe_cell* c);
bool conv_workspace_bytes(const gpipe_cell* c, int N, int M, int remat, size_t* bytes);
bool conv_saved_offset(const gpipe_cell* c, int N, int M, int remat, int micro, int block, int which,
                       size_t* offset, size_t* bytes);
gpipe_status conv_cell_step(gpipe_cell* c, const void* x, const void* target, void* y, void* dx,
                            int N, int M, int remat, void* workspace, size_t ws_bytes,
                            hipStream_t stream, float* loss_dev);
// phases: 1 the forward phase (and the moving averages), 2 the backward
// phase, 3 both; the backward's output gradient is the loss against target,
// or dy when target is null.
gpipe_status conv_cell_run(gpipe_cell* c, int phases, const void* x, const void* target,
                           const void* dy, void* y, void* dx, int N, int M, int remat,
                           void* workspace, size_t ws_bytes, hipStream_t stream, float* loss_dev);
gpipe_status conv_gemm_plan(const gpipe_cell* c, int N, int M, int role, int* tile_m, int* tile_n,
                            int* splits);

// Ordering of a step's streams: s1 is the caller's, s2 and s3 the cell's own.
// A fork makes s2 (fork3: s3) wait for everything enqueued so far on s1 (and
// s2); mark records an event after the work enqueued so far on s2; a join
// makes s1 wait for such an event (join3: for s3's work so far).  In the
// Transformer cell's backward phase the weight gradients, which feed nothing
// in the input-gradient chain, run on s2 in issue order (so every gradient
// still sums the micro-batches in order 0 .. M-1) and s1 joins before it
// overwrites a buffer a weight gradient reads.
// With `single` set all three are the caller's stream and every ordering
// call is a no-op (the stream's own order covers it; no event is used).
struct Streams {
  gpipe_cell* c;
  hipStream_t s1, s2, s3;
  bool single = false;
  hipEvent_t next() { return c->sync_events[c->sync_next++ % c->sync_events.size()]; }
  // s2 waits for the work enqueued so far on s1
  bool fork() {
    if (single) return true;
    const hipEvent_t e = next();
    return hipEventRecord(e, s1) == hipSuccess && hipStreamWaitEvent(s2, e, 0) == hipSuccess;
  }
  // event recorded on s2 after the work enqueued so far on it
  bool mark(hipEvent_t* out) {
    if (single) {
      *out = nullptr;
      return true;
    }
    *out = next();
    return hipEventRecord(*out, s2) == hipSuccess;
  }
  // s1 waits for an event of s2 (nullptr: nothing to wait for).  A ring
  // event recorded again since only makes the wait longer, never shorter.
  bool join(hipEvent_t e) { return !e || hipStreamWaitEvent(s1, e, 0) == hipSuccess; }
  bool join_all() {
    hipEvent_t e;
    return mark(&e) && join(e);
  }
  // s3 waits for the work enqueued so far on s1 and on s2
  bool fork3() {
    if (single) return true;
    const hipEvent_t e1 = next(), e2 = next();
    return hipEventRecord(e1, s1) == hipSuccess && hipEventRecord(e2, s2) == hipSuccess &&
           hipStreamWaitEvent(s3, e1, 0) == hipSuccess && hipStreamWaitEvent(s3, e2, 0) == hipSuccess;
  }
  // fork() with its event recorded in the dispatch of the next kernel launched
  // on s1 (next_done_event: no packet of its own on s1): fork_begin right
  // before the call whose last kernel ends the work s2 waits for, fork_end
  // after it (it records the event on s1 if no launch took it)
  hipEvent_t pending = nullptr;
  void fork_begin() {
    if (single) return;
    pending = next();
    next_done_event() = pending;
  }
  bool fork_end() {
    if (single) return true;
    const hipEvent_t e = pending;
    pending = nullptr;
    if (next_done_event() == e) {
      next_done_event() = nullptr;
      if (hipEventRecord(e, s1) != hipSuccess) return false;
    }
    return hipStreamWaitEvent(s2, e, 0) == hipSuccess;
  }
  // mark() with the event recorded in the dispatch of the next kernel launched
  // on s2: mark_begin right before that launch (null in single mode),
  // mark_end after it
  hipEvent_t mark_begin() {
    if (single) return nullptr;
    const hipEvent_t e = next();
    next_done_event() = e;
    return e;
  }
  bool mark_end(hipEvent_t e) {
    if (!e || next_done_event() != e) return true;
    next_done_event() = nullptr;
    return hipEventRecord(e, s2) == hipSuccess;
  }
  // fork3 where the work enqueued so far on s1 ends at event e1 and that on s2
  // at e2 (events recorded in kernels' dispatches; a null one is recorded now)
  bool fork3_after(hipEvent_t e1, hipEvent_t e2) {
    if (single) return true;
    if (!e1) {
      e1 = next();
      if (hipEventRecord(e1, s1) != hipSuccess) return false;
    }
    if (!e2) {
      e2 = next();
      if (hipEventRecord(e2, s2) != hipSuccess) return false;
    }
    return hipStreamWaitEvent(s3, e1, 0) == hipSuccess && hipStreamWaitEvent(s3, e2, 0) == hipSuccess;
  }
  // s1 waits for the work enqueued so far on s3
  bool join3() {
    if (single) return true;
    const hipEvent_t e = next();
    return hipEventRecord(e, s3) == hipSuccess && hipStreamWaitEvent(s1, e, 0) == hipSuccess;
  }
};

// A transient gradient of a backward phase that weight gradients on the
// second stream read: n copies (2 to 4) used in turn (workspace offsets),
// each with the event recorded after the last weight gradient that read it.
// The input-gradient chain writes the copy after the one just written,
// waiting only for that copy's readers -- from n writes earlier -- instead of
// for the weight-gradient stream to catch up.
struct Transient {
  static constexpr int kMax = 4;
  size_t off[kMax];
  hipEvent_t read[kMax] = {nullptr, nullptr, nullptr, nullptr};
  int n = 2, cur = 0;
  // switches to the next copy, once its last readers are done (ss null: one
  // stream, nothing to wait for)
  bool next(Streams* ss) {
    cur = cur + 1 == n ? 0 : cur + 1;
    if (ss && !ss->join(read[cur])) return false;
    read[cur] = nullptr;
    return true;
  }
  // the weight gradients enqueued so far on the second stream read copy k
  bool read_by_s2(Streams* ss, int k) { return !ss || ss->mark(&read[k]); }
  // the same, with e the event the last of them recorded (Streams::mark_begin)
  bool read_by_s2_at(Streams* ss, int k, hipEvent_t e) {
    if (!ss || !ss->mark_end(e)) return !ss;
    read[k] = e;
    return true;
  }
};

// Creates the cell's two streams and the event ring at its first step.
inline gpipe_status ensure_streams(gpipe_cell* c) {
  int dev = -1;
  GP_CHECK(hipGetDevice(&dev));
  if (c->aux) return dev == c->aux_device ? GPIPE_OK : GPIPE_ERR_STATE;
  GP_CHECK(hipStreamCreateWithFlags(&c->aux, hipStreamNonBlocking));
  GP_CHECK(hipStreamCreateWithFlags(&c->aux2, hipStreamNonBlocking));
  c->aux_device = dev;
  // (a ring: an event is recorded again ~20 layers of the backward phase
  // later, well after its last wait)
  for (int i = 0; i < 256; ++i) {
    hipEvent_t e;
    GP_CHECK(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    c->sync_events.push_back(e);
  }
  return GPIPE_OK;
}

}  // namespace gp
