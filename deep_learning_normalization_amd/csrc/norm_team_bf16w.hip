// norm_team_bf16w.hip -- the team kernels for bf16 activations with fp32 weights, every access width.
#include "norm_team_menu.hpp"

namespace dln {

norm_status_t launch_team_fwd_bf16w(const Plan &p, const FwdArgs &a, hipStream_t s) {
  return team_fwd_any<bf16_bits, float>(p, a, s);
}

norm_status_t launch_team_bwd_bf16w(const Plan &p, const BwdArgs &a, hipStream_t s) {
  return team_bwd_any<bf16_bits, float>(p, a, s);
}

} // namespace dln
