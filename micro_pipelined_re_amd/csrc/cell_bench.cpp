// Native driver of the cell step through the C-ABI, without Python: creates
// a cell, fills its weights and a mini-batch with seeded normal draws (bf16
// values of N(0, 0.02^2) weights, N(0, 1) activations; LayerNorm gamma 1,
// beta 0, biases 0), runs `warmup` + `steps` steps (step + RMSProp update)
// and prints the mean step time.  Used to profile the kernels (for instance
// HBM traffic counters) outside an interpreter.
//
//   cell_bench [L D H F S causal N M steps warmup]   (default: 8 2048 16 8192 512 1 64 32 2 1)
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "../../include/gpipe.h"

#define HIP_OK(x)                                                                \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      std::fprintf(stderr, "%s:%d %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      return 1;                                                                  \
    }                                                                            \
  } while (0)
#define GP_OK(x)                                                                       \
  do {                                                                                 \
    gpipe_status s_ = (x);                                                             \
    if (s_ != GPIPE_OK) {                                                              \
      std::fprintf(stderr, "%s:%d %s\n", __FILE__, __LINE__, gpipe_status_string(s_)); \
      return 1;                                                                        \
    }                                                                                  \
  } while (0)

static uint16_t bf16_of(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

static float f32_of_bf16(uint16_t h) {
  const uint32_t u = uint32_t(h) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

int main(int argc, char** argv) {
  int a[10] = {8, 2048, 16, 8192, 512, 1, 64, 32, 2, 1};
  for (int i = 1; i < argc && i <= 10; ++i) a[i - 1] = std::atoi(argv[i]);
  const int L = a[0], D = a[1], H = a[2], F = a[3], S = a[4], causal = a[5], N = a[6], M = a[7];
  const int steps = a[8], warmup = a[9];
  gpipe_cell* cell = nullptr;
  GP_OK(gpipe_cell_create(L, D, H, F, S, causal, GPIPE_BF16, &cell));
  size_t n = 0;
  GP_OK(gpipe_cell_param_count(cell, &n));
  std::printf("[cell_bench] L=%d D=%d H=%d F=%d S=%d causal=%d N=%d M=%d params=%zu\n", L, D, H, F, S,
              causal, N, M, n);
  std::fflush(stdout);

  std::mt19937_64 rng(0);
  std::normal_distribution<float> nd(0.f, 1.f);
  std::vector<float> w(n, 0.f);
  for (int l = 0; l < L; ++l)
    for (int t = 0; t < GPIPE_N_TENSORS; ++t) {
      size_t off = 0, cnt = 0;
      GP_OK(gpipe_cell_param_offset(cell, l, t, &off, &cnt));
      const bool matrix = t == GPIPE_W_QKV || t == GPIPE_W_O || t == GPIPE_W_1 || t == GPIPE_W_2;
      const bool gamma = t == GPIPE_LN1_G || t == GPIPE_LN2_G;
      for (size_t i = 0; i < cnt; ++i)
        w[off + i] = matrix ? f32_of_bf16(bf16_of(0.02f * nd(rng))) : (gamma ? 1.f : 0.f);
    }
  const size_t act = size_t(N) * S * D;
  std::vector<uint16_t> xh(act), th(act);
  for (auto& v : xh) v = bf16_of(nd(rng));
  for (auto& v : th) v = bf16_of(nd(rng));

  float *master, *grad, *ms, *loss;
  void *lowp, *x, *t, *y, *dx, *ws;
  size_t ws_bytes = 0;
  GP_OK(gpipe_cell_workspace_bytes(cell, N, M, 1, &ws_bytes));
  HIP_OK(hipMalloc(&master, n * 4));
  HIP_OK(hipMalloc(&grad, n * 4));
  HIP_OK(hipMalloc(&ms, n * 4));
  HIP_OK(hipMalloc(&lowp, n * 2));
  HIP_OK(hipMalloc(&loss, 4));
  HIP_OK(hipMalloc(&x, act * 2));
  HIP_OK(hipMalloc(&t, act * 2));
  HIP_OK(hipMalloc(&y, act * 2));
  HIP_OK(hipMalloc(&dx, act * 2));
  HIP_OK(hipMalloc(&ws, ws_bytes));
  HIP_OK(hipMemcpy(master, w.data(), n * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(ms, 0, n * 4));
  HIP_OK(hipMemcpy(x, xh.data(), act * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(t, th.data(), act * 2, hipMemcpyHostToDevice));
  GP_OK(gpipe_cell_bind(cell, master, lowp, grad, ms));
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  GP_OK(gpipe_cell_sync_lowp(cell, s));   // float32 -> bf16 copy: a plain streaming kernel
  HIP_OK(hipStreamSynchronize(s));

  auto step = [&]() -> gpipe_status {
    gpipe_status st = gpipe_cell_step(cell, x, t, y, dx, N, M, 1, ws, ws_bytes, s, loss);
    if (st != GPIPE_OK) return st;
    return gpipe_apply_update(cell, 1e-3f, 0.9f, 1e-8f, s);
  };
  for (int i = 0; i < warmup; ++i) GP_OK(step());
  HIP_OK(hipStreamSynchronize(s));
  hipEvent_t e0, e1;
  HIP_OK(hipEventCreate(&e0));
  HIP_OK(hipEventCreate(&e1));
  HIP_OK(hipEventRecord(e0, s));
  for (int i = 0; i < steps; ++i) GP_OK(step());
  HIP_OK(hipEventRecord(e1, s));
  HIP_OK(hipEventSynchronize(e1));
  float ms_tot = 0.f;
  HIP_OK(hipEventElapsedTime(&ms_tot, e0, e1));
  float loss_h = 0.f;
  HIP_OK(hipMemcpy(&loss_h, loss, 4, hipMemcpyDeviceToHost));
  const double per = steps ? ms_tot / steps : 0.0;
  std::printf("[cell_bench] %d steps: %.3f ms/step, %.1f tokens/s, loss %.6f\n", steps, per,
              per > 0 ? double(N) * S / (per * 1e-3) : 0.0, loss_h);
  GP_OK(gpipe_cell_destroy(cell));
  HIP_OK(hipStreamDestroy(s));
  for (void* p : {(void*)master, (void*)grad, (void*)ms, lowp, (void*)loss, x, t, y, dx, ws})
    HIP_OK(hipFree(p));
  return std::isfinite(loss_h) ? 0 : 1;
}
