// Instances of the fp32 GEMM (fp32 cells) for every role of the step.
#include "gemm_impl.hpp"

namespace gp {

hipError_t gemm_group_f32(int role, const GemmParams& g, int batch, hipStream_t s) {
  switch (role) {
    case GPIPE_ROLE_QKV_FWD: return launch_f32<RoleSpec<GPIPE_ROLE_QKV_FWD>::LA, RoleSpec<GPIPE_ROLE_QKV_FWD>::LB, RoleSpec<GPIPE_ROLE_QKV_FWD>::EPI, GPIPE_ROLE_QKV_FWD>(g, batch, s);
    case GPIPE_ROLE_SCORES_FWD: return launch_f32<RoleSpec<GPIPE_ROLE_SCORES_FWD>::LA, RoleSpec<GPIPE_ROLE_SCORES_FWD>::LB, RoleSpec<GPIPE_ROLE_SCORES_FWD>::EPI, GPIPE_ROLE_SCORES_FWD>(g, batch, s);
    case GPIPE_ROLE_PV_FWD: return launch_f32<RoleSpec<GPIPE_ROLE_PV_FWD>::LA, RoleSpec<GPIPE_ROLE_PV_FWD>::LB, RoleSpec<GPIPE_ROLE_PV_FWD>::EPI, GPIPE_ROLE_PV_FWD>(g, batch, s);
    case GPIPE_ROLE_OUT_FWD: return launch_f32<RoleSpec<GPIPE_ROLE_OUT_FWD>::LA, RoleSpec<GPIPE_ROLE_OUT_FWD>::LB, RoleSpec<GPIPE_ROLE_OUT_FWD>::EPI, GPIPE_ROLE_OUT_FWD>(g, batch, s);
    case GPIPE_ROLE_FFN1_FWD: return launch_f32<RoleSpec<GPIPE_ROLE_FFN1_FWD>::LA, RoleSpec<GPIPE_ROLE_FFN1_FWD>::LB, RoleSpec<GPIPE_ROLE_FFN1_FWD>::EPI, GPIPE_ROLE_FFN1_FWD>(g, batch, s);
    case GPIPE_ROLE_FFN2_FWD: return launch_f32<RoleSpec<GPIPE_ROLE_FFN2_FWD>::LA, RoleSpec<GPIPE_ROLE_FFN2_FWD>::LB, RoleSpec<GPIPE_ROLE_FFN2_FWD>::EPI, GPIPE_ROLE_FFN2_FWD>(g, batch, s);
    case GPIPE_ROLE_FFN2_DGRAD: return launch_f32<RoleSpec<GPIPE_ROLE_FFN2_DGRAD>::LA, RoleSpec<GPIPE_ROLE_FFN2_DGRAD>::LB, RoleSpec<GPIPE_ROLE_FFN2_DGRAD>::EPI, GPIPE_ROLE_FFN2_DGRAD>(g, batch, s);
    case GPIPE_ROLE_FFN2_WGRAD: return launch_f32<RoleSpec<GPIPE_ROLE_FFN2_WGRAD>::LA, RoleSpec<GPIPE_ROLE_FFN2_WGRAD>::LB, RoleSpec<GPIPE_ROLE_FFN2_WGRAD>::EPI, GPIPE_ROLE_FFN2_WGRAD>(g, batch, s);
    case GPIPE_ROLE_FFN1_DGRAD: return launch_f32<RoleSpec<GPIPE_ROLE_FFN1_DGRAD>::LA, RoleSpec<GPIPE_ROLE_FFN1_DGRAD>::LB, RoleSpec<GPIPE_ROLE_FFN1_DGRAD>::EPI, GPIPE_ROLE_FFN1_DGRAD>(g, batch, s);
    case GPIPE_ROLE_FFN1_WGRAD: return launch_f32<RoleSpec<GPIPE_ROLE_FFN1_WGRAD>::LA, RoleSpec<GPIPE_ROLE_FFN1_WGRAD>::LB, RoleSpec<GPIPE_ROLE_FFN1_WGRAD>::EPI, GPIPE_ROLE_FFN1_WGRAD>(g, batch, s);
    case GPIPE_ROLE_OUT_DGRAD: return launch_f32<RoleSpec<GPIPE_ROLE_OUT_DGRAD>::LA, RoleSpec<GPIPE_ROLE_OUT_DGRAD>::LB, RoleSpec<GPIPE_ROLE_OUT_DGRAD>::EPI, GPIPE_ROLE_OUT_DGRAD>(g, batch, s);
    case GPIPE_ROLE_OUT_WGRAD: return launch_f32<RoleSpec<GPIPE_ROLE_OUT_WGRAD>::LA, RoleSpec<GPIPE_ROLE_OUT_WGRAD>::LB, RoleSpec<GPIPE_ROLE_OUT_WGRAD>::EPI, GPIPE_ROLE_OUT_WGRAD>(g, batch, s);
    case GPIPE_ROLE_DP: return launch_f32<RoleSpec<GPIPE_ROLE_DP>::LA, RoleSpec<GPIPE_ROLE_DP>::LB, RoleSpec<GPIPE_ROLE_DP>::EPI, GPIPE_ROLE_DP>(g, batch, s);
    case GPIPE_ROLE_DV: return launch_f32<RoleSpec<GPIPE_ROLE_DV>::LA, RoleSpec<GPIPE_ROLE_DV>::LB, RoleSpec<GPIPE_ROLE_DV>::EPI, GPIPE_ROLE_DV>(g, batch, s);
    case GPIPE_ROLE_DQ: return launch_f32<RoleSpec<GPIPE_ROLE_DQ>::LA, RoleSpec<GPIPE_ROLE_DQ>::LB, RoleSpec<GPIPE_ROLE_DQ>::EPI, GPIPE_ROLE_DQ>(g, batch, s);
    case GPIPE_ROLE_DK: return launch_f32<RoleSpec<GPIPE_ROLE_DK>::LA, RoleSpec<GPIPE_ROLE_DK>::LB, RoleSpec<GPIPE_ROLE_DK>::EPI, GPIPE_ROLE_DK>(g, batch, s);
    case GPIPE_ROLE_QKV_DGRAD: return launch_f32<RoleSpec<GPIPE_ROLE_QKV_DGRAD>::LA, RoleSpec<GPIPE_ROLE_QKV_DGRAD>::LB, RoleSpec<GPIPE_ROLE_QKV_DGRAD>::EPI, GPIPE_ROLE_QKV_DGRAD>(g, batch, s);
    case GPIPE_ROLE_QKV_WGRAD: return launch_f32<RoleSpec<GPIPE_ROLE_QKV_WGRAD>::LA, RoleSpec<GPIPE_ROLE_QKV_WGRAD>::LB, RoleSpec<GPIPE_ROLE_QKV_WGRAD>::EPI, GPIPE_ROLE_QKV_WGRAD>(g, batch, s);
    case GPIPE_ROLE_CONV_FWD: return launch_f32<RoleSpec<GPIPE_ROLE_CONV_FWD>::LA, RoleSpec<GPIPE_ROLE_CONV_FWD>::LB, RoleSpec<GPIPE_ROLE_CONV_FWD>::EPI, GPIPE_ROLE_CONV_FWD>(g, batch, s);
    case GPIPE_ROLE_CONV_DGRAD: return launch_f32<RoleSpec<GPIPE_ROLE_CONV_DGRAD>::LA, RoleSpec<GPIPE_ROLE_CONV_DGRAD>::LB, RoleSpec<GPIPE_ROLE_CONV_DGRAD>::EPI, GPIPE_ROLE_CONV_DGRAD>(g, batch, s);
    case GPIPE_ROLE_CONV_WGRAD: return launch_f32<RoleSpec<GPIPE_ROLE_CONV_WGRAD>::LA, RoleSpec<GPIPE_ROLE_CONV_WGRAD>::LB, RoleSpec<GPIPE_ROLE_CONV_WGRAD>::EPI, GPIPE_ROLE_CONV_WGRAD>(g, batch, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gp
