// Instances of the bf16 GEMM for the wgrad roles of the step.
#include "gemm_dma.hpp"

namespace gp {

hipError_t gemm_group_wgrad(int role, int path, int cfg, const GemmParams& g, int batch, int splits, hipStream_t s) {
  switch (role) {
    case GPIPE_ROLE_FFN2_WGRAD: return launch_role<GPIPE_ROLE_FFN2_WGRAD>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_FFN1_WGRAD: return launch_role<GPIPE_ROLE_FFN1_WGRAD>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_OUT_WGRAD: return launch_role<GPIPE_ROLE_OUT_WGRAD>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_QKV_WGRAD: return launch_role<GPIPE_ROLE_QKV_WGRAD>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_CONV_WGRAD: return launch_role<GPIPE_ROLE_CONV_WGRAD>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_CONV_WGRAD_IMPLICIT:
      return launch_role<GPIPE_ROLE_CONV_WGRAD_IMPLICIT>(path, cfg, g, batch, splits, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gp
