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

// Launches `expr`; when `role` is being timed, a GEMM role's launch records
// two events in its own dispatch (launch_events()), any other role is
// bracketed by two events recorded on the context's stream.
#define GP_RUN(ctx, role, expr)                                                         \
  do {                                                                                 \
    hipEvent_t e0_ = nullptr, e1_ = nullptr;                                           \
    const bool in_launch_ = gemm_role(role);                                           \
    if ((ctx).prof && (((ctx).prof->prof_mask >> (role)) & 1ull)) {                   \
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
gpipe_status conv_gemm_plan(const gpipe_cell* c, int N, int M, int role, int* tile_m, int* tile_n,
                            int* splits);

}  // namespace gp
