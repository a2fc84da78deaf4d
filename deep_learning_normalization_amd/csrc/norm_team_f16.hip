// norm_team_f16.hip -- the team kernels for fp16 storage, every access width.
#include "norm_team_menu.hpp"

namespace dln {

norm_status_t launch_team_fwd_f16(const Plan &p, const FwdArgs &a, hipStream_t s) {
  return team_fwd_any<f16_t, f16_t>(p, a, s);
}

norm_status_t launch_team_bwd_f16(const Plan &p, const BwdArgs &a, hipStream_t s) {
  return team_bwd_any<f16_t, f16_t>(p, a, s);
}

} // namespace dln
