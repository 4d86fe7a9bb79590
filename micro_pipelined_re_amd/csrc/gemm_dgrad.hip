// Instances of the bf16 GEMM for the dgrad roles of the step.
#include "gemm_dma.hpp"

namespace gp {

hipError_t gemm_group_dgrad(int role, int path, int cfg, const GemmParams& g, int batch, int splits, hipStream_t s) {
  switch (role) {
    case GPIPE_ROLE_FFN2_DGRAD: return launch_role<GPIPE_ROLE_FFN2_DGRAD>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_FFN1_DGRAD: return launch_role<GPIPE_ROLE_FFN1_DGRAD>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_OUT_DGRAD: return launch_role<GPIPE_ROLE_OUT_DGRAD>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_QKV_DGRAD: return launch_role<GPIPE_ROLE_QKV_DGRAD>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_CONV_DGRAD: return launch_role<GPIPE_ROLE_CONV_DGRAD>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_CONV_DGRAD_IMPLICIT:
      return launch_role<GPIPE_ROLE_CONV_DGRAD_IMPLICIT>(path, cfg, g, batch, splits, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gp
