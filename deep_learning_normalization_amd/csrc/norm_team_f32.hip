// norm_team_f32.hip -- the team kernels for fp32 storage, every access width.
#include "norm_team_menu.hpp"

namespace dln {

norm_status_t launch_team_fwd_f32(const Plan &p, const FwdArgs &a, hipStream_t s) {
  return team_fwd_any<float, float>(p, a, s);
}

norm_status_t launch_team_bwd_f32(const Plan &p, const BwdArgs &a, hipStream_t s) {
  return team_bwd_any<float, float>(p, a, s);
}

} // namespace dln
