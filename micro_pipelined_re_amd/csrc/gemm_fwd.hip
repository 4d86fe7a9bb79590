// Instances of the bf16 GEMM for the fwd roles of the step.
#include "gemm_dma.hpp"

namespace gp {

hipError_t gemm_group_fwd(int role, int path, int cfg, const GemmParams& g, int batch, int splits, hipStream_t s) {
  switch (role) {
    case GPIPE_ROLE_QKV_FWD: return launch_role<GPIPE_ROLE_QKV_FWD>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_OUT_FWD: return launch_role<GPIPE_ROLE_OUT_FWD>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_FFN1_FWD: return launch_role<GPIPE_ROLE_FFN1_FWD>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_FFN2_FWD: return launch_role<GPIPE_ROLE_FFN2_FWD>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_CONV_FWD: return launch_role<GPIPE_ROLE_CONV_FWD>(path, cfg, g, batch, splits, s);
    case GPIPE_ROLE_CONV_FWD_IMPLICIT:
      return launch_role<GPIPE_ROLE_CONV_FWD_IMPLICIT>(path, cfg, g, batch, splits, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gp
