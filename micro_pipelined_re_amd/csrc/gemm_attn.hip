// Instances of the bf16 GEMM for the attn roles of the step.
#include "gemm_dma.hpp"

namespace gp {

hipError_t gemm_group_attn(int role, int path, int cfg, const GemmParams& g, int batch, int splits, hipStream_t s) {
  switch (role) {
    case GPIPE_ROLE_SCORES_FWD: return launch_role<GPIPE_ROLE_SCORES_FWD>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_PV_FWD: return launch_role<GPIPE_ROLE_PV_FWD>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_DP: return launch_role<GPIPE_ROLE_DP>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_DV: return launch_role<GPIPE_ROLE_DV>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_DQ: return launch_role<GPIPE_ROLE_DQ>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_DK: return launch_role<GPIPE_ROLE_DK>(path, cfg, g, batch, splits, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gp
