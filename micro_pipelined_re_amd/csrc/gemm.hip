// Host side of the cell's GEMMs: per-role choice of macro tile and split-K,
// and dispatch to the kernel instances (gemm_fwd/dgrad/wgrad/attn/f32.hip).
#include <math.h>

#include <algorithm>

#include "gemm_dma.hpp"

namespace gp {

namespace {

bool is_attention(int role) {
  return role == GPIPE_ROLE_SCORES_FWD || role == GPIPE_ROLE_PV_FWD || role == GPIPE_ROLE_DP ||
         role == GPIPE_ROLE_DV || role == GPIPE_ROLE_DQ || role == GPIPE_ROLE_DK;
}
bool is_wgrad(int role) {
  return role == GPIPE_ROLE_FFN2_WGRAD || role == GPIPE_ROLE_FFN1_WGRAD ||
         role == GPIPE_ROLE_OUT_WGRAD || role == GPIPE_ROLE_QKV_WGRAD;
}
bool is_conv(int role) {
  return role == GPIPE_ROLE_CONV_FWD || role == GPIPE_ROLE_CONV_DGRAD ||
         role == GPIPE_ROLE_CONV_WGRAD || role == GPIPE_ROLE_CONV_FWD_IMPLICIT ||
         role == GPIPE_ROLE_CONV_DGRAD_IMPLICIT || role == GPIPE_ROLE_CONV_WGRAD_IMPLICIT;
}
// B operand k-contiguous (the weight of a forward linear layer)
bool b_k_contiguous(int role) {
  return role == GPIPE_ROLE_QKV_FWD || role == GPIPE_ROLE_OUT_FWD || role == GPIPE_ROLE_FFN1_FWD ||
         role == GPIPE_ROLE_FFN2_FWD;
}
int group_of(int role) {
  switch (role) {
    case GPIPE_ROLE_QKV_FWD: case GPIPE_ROLE_OUT_FWD: case GPIPE_ROLE_FFN1_FWD:
    case GPIPE_ROLE_FFN2_FWD: return 0;
    case GPIPE_ROLE_FFN2_DGRAD: case GPIPE_ROLE_FFN1_DGRAD: case GPIPE_ROLE_OUT_DGRAD:
    case GPIPE_ROLE_QKV_DGRAD: return 1;
    case GPIPE_ROLE_CONV_FWD: case GPIPE_ROLE_CONV_FWD_IMPLICIT: return 0;
    case GPIPE_ROLE_CONV_DGRAD: case GPIPE_ROLE_CONV_DGRAD_IMPLICIT: return 1;
    case GPIPE_ROLE_CONV_WGRAD: case GPIPE_ROLE_CONV_WGRAD_IMPLICIT: return 2;
  }
  return is_wgrad(role) ? 2 : is_attention(role) ? 3 : -1;
}

// The direct-to-LDS kernel reads whole 64-deep k-tiles and 8-element chunks
// of m-contiguous operands without masking: k must be a multiple of 64 and
// an m-contiguous operand's extent a multiple of 8 (its rows past the extent
// are then read from valid memory and never stored).
// Its epilogue writes 8 consecutive columns with 16-byte accesses, so the
// output's leading dimensions must be multiples of 8 as well.
bool dma_ok(int role, const GemmParams& g) {
  if (g.K % 64 || g.M < 8 || g.N < 8 || g.N % 8 || g.ldc % 8 || g.ldr % 8 || g.ldu % 8) return false;
  const bool a_mn = role == GPIPE_ROLE_FFN2_WGRAD || role == GPIPE_ROLE_FFN1_WGRAD ||
                    role == GPIPE_ROLE_OUT_WGRAD || role == GPIPE_ROLE_QKV_WGRAD ||
                    role == GPIPE_ROLE_DV || role == GPIPE_ROLE_DK || role == GPIPE_ROLE_CONV_WGRAD ||
                    role == GPIPE_ROLE_CONV_WGRAD_IMPLICIT;
  const bool b_mn = role != GPIPE_ROLE_QKV_FWD && role != GPIPE_ROLE_SCORES_FWD &&
                    role != GPIPE_ROLE_OUT_FWD && role != GPIPE_ROLE_FFN1_FWD &&
                    role != GPIPE_ROLE_FFN2_FWD && role != GPIPE_ROLE_DP &&
                    role != GPIPE_ROLE_CONV_FWD && role != GPIPE_ROLE_CONV_FWD_IMPLICIT &&
                    role != GPIPE_ROLE_CONV_DGRAD_IMPLICIT;
  const bool conv = role == GPIPE_ROLE_CONV_FWD_IMPLICIT || role == GPIPE_ROLE_CONV_DGRAD_IMPLICIT;
  // a gathered operand needs every 64-deep k-tile inside one tap
  if (conv && (g.conv_c % 64 || g.K != 9 * g.conv_c)) return false;
  // gathered along k: eight-column chunks inside one tap, pixel indices below
  // 2^21, element offsets within 32 bits
  if (role == GPIPE_ROLE_CONV_WGRAD_IMPLICIT &&
      (g.conv_c % 8 || g.N != 9 * g.conv_c || g.K >= (1 << 21) || g.conv_h < 1 || g.conv_w < 1 ||
       g.K % (g.conv_h * g.conv_w) || (g.conv_ld && (g.conv_ld < g.conv_c || g.conv_ld % 8)) ||
       int64_t(g.K + 64) * (g.conv_ld ? g.conv_ld : g.conv_c) >= (int64_t(1) << 31)))
    return false;
  if (a_mn && g.M % 8) return false;
  if (b_mn && g.N % 8) return false;
  return true;
}

constexpr int kCUs = 256;

}  // namespace

// Tile and split choice, from per-role timings on MI355X with random
// operands and A/B runs of the whole step.  The linear layers' products
// (forward, input gradient, weight gradient) take the specialised-wave
// kernel: 256 x 128 tiles (128 x 256 for outputs wider than tall where both
// operands are k-contiguous, and for weight gradients wider than tall) when
// the output has at least 192 of them -- at least 64 for the backward's
// products -- else 128 x 128 tiles, unsplit.  The input gradients run on the
// backward's critical stream beside the weight gradients and the next
// re-materialization: with 64 big tiles for its 1024 x 2048 outputs (the
// FFN1, QKV and out-projection input gradients) instead of 128 tiles of
// 128 x 128 the 8-layer 2048-wide step ran 146.0 ms against 149.5 (both A/B
// runs on one box); big tiles for the 64- and 128-tile forward outputs as
// well ran 146.7, for the forward products alone 148.5, and the input
// gradients in 128 x 256 tiles 148.0.  Then 128 x 256 tiles for the 2048 x
// 8192 FFN2 weight gradient with 256 x 128 tiles for the 2048 x 2048
// out-projection one (128 instead of 256 tiles of 128 x 128) ran 143.8-144.1
// against 144.9-145.0, and 147.8-147.9 against 149.6-149.7 on a slower box
// (three A/B rounds each); either change alone gained 0.3 ms or less.  The
// backward's long input gradients (K >= 4096) split in two over k ran the
// step 0.3 ms slower, in four 6 ms slower: the step is bound by the CUs'
// work, not by the critical stream's latency.  The step runs these products beside other
// streams' work (the forward lanes, the weight gradients, the next
// re-materialization), which fills the CUs a small grid leaves idle, so what
// pays alone does not in the step: the 1024 x 2048 x 8192 down-projection
// split in two took 49 us alone against ~60 us unsplit, yet the step ran
// 166.0 ms with the split and 162.1 ms without; 128 x 64 tiles for the 1024
// x 2048 outputs at k = 2048 (256 tiles instead of 64) took 21.0 against
// 24.6 us in the step's own timing, yet the step ran 161.6 ms with them and
// 160.6 ms without (A/B on one box each); the input-gradient products of
// the backward's critical stream split in two (FFN1 1024 x 2048 x 8192, and
// with it QKV 1024 x 2048 x 6144) ran the step in 160.1 and 162.8 ms
// against 160.1 unsplit.  Against 128 x 128 tiles with two
// workgroups per CU the specialised kernel ran 5-37% faster on every role of
// the 2048-wide layer.  Weight gradients never split (their fp32 partials
// would double the accumulator traffic).  The attention products (K = 128 or
// 512, 32 batches) take 64 x 64 tiles; the explicit convolutions and small
// products 128 x 128 tiles of the two-workgroup kernel, where split-K pays
// only when the output has fewer tiles than CUs: it then aims at about two
// workgroups per CU with splits at least 512 deep.  The implicit
// convolutions take 128 x 128 specialised tiles (the weight gradient split
// to about one workgroup per CU).
GemmPlan plan_gemm(int role, bool bf16, int M, int N, int K, int batch) {
  GemmPlan p{is_attention(role) ? CFG_64x64_K64 : CFG_128x128_K64, 1, K};
  if (!bf16) {
    p.cfg = -1;
    return p;
  }
  auto split_of = [&](int want, int min_depth) {
    int s = std::min(want, std::min(8, K / min_depth));
    while (s > 1) {
      const int kc = ((K + s - 1) / s + 63) / 64 * 64;
      if ((s - 1) * kc < K) break;
      --s;
    }
    if (s > 1) {
      p.splits = s;
      p.kchunk = ((K + s - 1) / s + 63) / 64 * 64;
    }
  };
  const bool linear = group_of(role) >= 0 && group_of(role) <= 2 && !is_conv(role);
  if (linear && batch == 1 && K >= 512) {
    const int cfg = ((b_k_contiguous(role) || is_wgrad(role)) && N > M) ? CFG_128x256_K64
                                                                         : CFG_256x128_K64;
    const long tiles = long((M + kCfgBM[cfg] - 1) / kCfgBM[cfg]) * ((N + kCfgBN[cfg] - 1) / kCfgBN[cfg]);
    if (tiles >= 192 || (tiles >= 64 && group_of(role) != 0)) {
      p.cfg = cfg;
      return p;
    }
    const long t128 = long((M + 127) / 128) * ((N + 127) / 128);
    if (t128 >= 64) {
      // fewer big tiles than 3/4 of the CUs: 128 x 128 tiles
      p.cfg = CFG_128x128_SPEC;
      return p;
    }
  }
  // implicit-GEMM convolutions with at least 192 tiles of 128 x 128: the
  // specialised-wave kernel with the gathered-operand loader.  The forward
  // convolution (the forward phase's lanes and the re-materialization) takes
  // 128 x 256 tiles where they cover the output channels, so one launch
  // holds about half the CUs and leaves the rest to the caller's stream.
  if ((role == GPIPE_ROLE_CONV_FWD_IMPLICIT || role == GPIPE_ROLE_CONV_DGRAD_IMPLICIT) &&
      batch == 1 && long((M + 127) / 128) * ((N + 127) / 128) >= 192) {
    p.cfg = role == GPIPE_ROLE_CONV_FWD_IMPLICIT && N % 256 == 0 ? CFG_128x256_K64 : CFG_128x128_SPEC;
    return p;
  }
  // the weight gradient with the gathered column matrix: C x 9C outputs
  // reduced over every pixel of the micro-batch, split to about one
  // workgroup per CU
  if (role == GPIPE_ROLE_CONV_WGRAD_IMPLICIT) {
    p.cfg = CFG_128x128_SPEC;
    const long tiles = long((M + 127) / 128) * ((N + 127) / 128) * batch;
    if (tiles < kCUs && K >= 1024) split_of(int(std::max(1L, kCUs / tiles)), 512);
    return p;
  }
  // (the convolution's weight gradient is small -- C x 9C -- and reduces over
  // every pixel of the micro-batch, so it does split)
  const bool can_split = !is_attention(role) && (!is_wgrad(role) || role == GPIPE_ROLE_CONV_WGRAD) &&
                         batch == 1;
  const int bm = kCfgBM[p.cfg], bn = kCfgBN[p.cfg];
  const long tiles = long((M + bm - 1) / bm) * ((N + bn - 1) / bn) * batch;
  if (can_split && tiles < kCUs && K >= 1024) split_of(int((2 * kCUs + tiles - 1) / tiles), 512);
  return p;
}

LaunchEvents& launch_events() {
  static thread_local LaunchEvents e;
  return e;
}

hipEvent_t& next_done_event() {
  static thread_local hipEvent_t e = nullptr;
  return e;
}

bool gemm_role(int role) { return group_of(role) >= 0; }

int gemm_cfg_bm(int cfg) { return kCfgBM[cfg]; }
int gemm_cfg_bn(int cfg) { return kCfgBN[cfg]; }

size_t gemm_partial_floats(int role, bool bf16, int M, int N, int K, int batch) {
  const GemmPlan p = plan_gemm(role, bf16, M, N, K, batch);
  return p.splits > 1 ? size_t(p.splits) * M * N : 0;
}

hipError_t gemm(bool bf16, int role, const GemmParams& g0, int batch, hipStream_t s) {
  if (!bf16) return gemm_group_f32(role, g0, batch, s);
  return gemm_with_plan(role, plan_gemm(role, true, g0.M, g0.N, g0.K, batch), g0, batch, s);
}

namespace {
bool spec_cfg(int cfg) {
  return cfg == CFG_256x128_K64 || cfg == CFG_128x256_K64 || cfg == CFG_128x128_SPEC;
}
}  // namespace

int gemm_rowsum_parts(int role, const GemmParams& g, int batch) {
  if (!is_wgrad(role) || batch != 1) return 0;
  const GemmPlan p = plan_gemm(role, true, g.M, g.N, g.K, batch);
  if (!(spec_cfg(p.cfg) && p.splits == 1 && dma_ok(role, g))) return 0;
  return (g.N + kCfgBN[p.cfg] - 1) / kCfgBN[p.cfg];
}

hipError_t gemm_with_plan(int role, const GemmPlan& p, const GemmParams& g0, int batch, hipStream_t s) {
  if (p.cfg < 0 || p.cfg >= CFG_N || p.splits < 1) return hipErrorInvalidValue;
  GemmParams g = g0;
  g.kchunk = p.kchunk;
  if (p.splits > 1 && !g.P) return hipErrorInvalidValue;
  const int path = dma_ok(role, g) ? 0 : 1;
  // row sums come only from the specialised kernel of a weight gradient, unsplit
  if (g.rowsum && !(is_wgrad(role) && batch == 1 && spec_cfg(p.cfg) && p.splits == 1 && path == 0))
    return hipErrorInvalidValue;
  int cfg = p.cfg;
  switch (group_of(role)) {
    case 0: return gemm_group_fwd(role, path, cfg, g, batch, p.splits, s);
    case 1: return gemm_group_dgrad(role, path, cfg, g, batch, p.splits, s);
    case 2: return gemm_group_wgrad(role, path, cfg, g, batch, p.splits, s);
    case 3: return gemm_group_attn(role, path, cfg, g, batch, p.splits, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gp
