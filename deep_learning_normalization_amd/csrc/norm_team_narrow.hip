// norm_team_narrow.hip -- the team kernels with 8- and 4-byte accesses.
//
// A row of N elements starts at byte N * sizeof(T) * row from the tensor base. When N is not a
// multiple of the 16-byte vector (8 bf16, 4 fp32) or a pointer is only 8- or 4-byte aligned,
// 16-byte accesses would straddle rows or misalign; the widest whole-word access that divides
// both still streams every element once through coalesced loads and stores (64 lanes x 8 or 4
// bytes per instruction), instead of one element per lane.
//
// Shapes are the full-width menus with the accesses per thread multiplied by the width ratio
// (SC = 16-byte elements / elements per access), so a thread holds as many elements in
// registers as its full-width counterpart. Menu entries below are in full-width units (V) and
// launch V * SC accesses per thread; one row per team.
#include "norm_team_kernels.hpp"

namespace dln {
namespace {

#define DLN_WAVE_MENU_NARROW(X) X(1, 1, 256) X(2, 1, 256) X(4, 1, 256)
#define DLN_BLOCK_MENU_NARROW_FWD(X)                                                            \
  X(1, 1, 256) X(2, 1, 256) X(4, 1, 256) X(8, 1, 256) X(1, 1, 512) X(2, 1, 512) X(4, 1, 512)     \
      X(1, 1, 1024) X(2, 1, 1024)
#define DLN_BLOCK_MENU_NARROW_BWD(X)                                                            \
  X(1, 1, 256) X(2, 1, 256) X(4, 1, 256) X(1, 1, 512) X(2, 1, 512) X(1, 1, 1024)

template <typename T, typename TW, int EV>
norm_status_t fwd_narrow(const Plan &p, const FwdArgs &a, hipStream_t s) {
  constexpr int SC = full_epv<T>() / EV;
  const bool resid = a.r != nullptr;
  const int lb = p.lb;
  hipError_t e = hipErrorInvalidConfiguration;
  bool found = false;
  if (p.scheme == NORM_SCHEME_WAVE) {
#define X(V, R, L)                                                                              \
  if (!found && p.vpt == V * SC && p.rows == R && lb == L) {                                    \
    found = true;                                                                               \
    e = fwd_launch<T, TW, EV, V * SC, R, L, true>(p, a, resid, s);                              \
  }
    DLN_WAVE_MENU_NARROW(X)
#undef X
  } else {
#define X(V, R, L)                                                                              \
  if (!found && p.vpt == V * SC && p.rows == R && lb == L) {                                    \
    found = true;                                                                               \
    e = fwd_launch<T, TW, EV, V * SC, R, L, false>(p, a, resid, s);                             \
  }
    DLN_BLOCK_MENU_NARROW_FWD(X)
#undef X
  }
  if (!found) return NORM_ERR_UNSUPPORTED;
  return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

template <typename T, typename TW, int EV>
norm_status_t bwd_narrow(const Plan &p, const BwdArgs &a, hipStream_t s) {
  constexpr int SC = full_epv<T>() / EV;
  const int lb = p.lb;
  hipError_t e = hipErrorInvalidConfiguration;
  bool found = false;
  if (p.scheme == NORM_SCHEME_WAVE) {
#define X(V, R, L)                                                                              \
  if (!found && p.vpt == V * SC && p.rows == R && lb == L) {                                    \
    found = true;                                                                               \
    e = bwd_launch<T, TW, EV, V * SC, R, L, true>(p, a, s);                                     \
  }
    DLN_WAVE_MENU_NARROW(X)
#undef X
  } else {
#define X(V, R, L)                                                                              \
  if (!found && p.vpt == V * SC && p.rows == R && lb == L) {                                    \
    found = true;                                                                               \
    e = bwd_launch<T, TW, EV, V * SC, R, L, false>(p, a, s);                                    \
  }
    DLN_BLOCK_MENU_NARROW_BWD(X)
#undef X
  }
  if (!found) return NORM_ERR_UNSUPPORTED;
  return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

// bf16 activations: 8-byte (4 elements) or 4-byte (2 elements) accesses
template <typename TW>
norm_status_t fwd_bf16(const Plan &p, const FwdArgs &a, hipStream_t s) {
  if (p.epv == 4) return fwd_narrow<bf16_bits, TW, 4>(p, a, s);
  if (p.epv == 2) return fwd_narrow<bf16_bits, TW, 2>(p, a, s);
  return NORM_ERR_UNSUPPORTED;
}
template <typename TW>
norm_status_t bwd_bf16(const Plan &p, const BwdArgs &a, hipStream_t s) {
  if (p.epv == 4) return bwd_narrow<bf16_bits, TW, 4>(p, a, s);
  if (p.epv == 2) return bwd_narrow<bf16_bits, TW, 2>(p, a, s);
  return NORM_ERR_UNSUPPORTED;
}

} // namespace

norm_status_t launch_team_fwd_narrow(const Plan &p, norm_dtype_t dtype, const FwdArgs &a,
                                     hipStream_t s) {
  switch (dtype) {
  case NORM_F32: return p.epv == 2 ? fwd_narrow<float, float, 2>(p, a, s) : NORM_ERR_UNSUPPORTED;
  case NORM_BF16: return fwd_bf16<bf16_bits>(p, a, s);
  case NORM_BF16_F32W: return fwd_bf16<float>(p, a, s);
  default: return NORM_ERR_UNSUPPORTED;
  }
}

norm_status_t launch_team_bwd_narrow(const Plan &p, norm_dtype_t dtype, const BwdArgs &a,
                                     hipStream_t s) {
  switch (dtype) {
  case NORM_F32: return p.epv == 2 ? bwd_narrow<float, float, 2>(p, a, s) : NORM_ERR_UNSUPPORTED;
  case NORM_BF16: return bwd_bf16<bf16_bits>(p, a, s);
  case NORM_BF16_F32W: return bwd_bf16<float>(p, a, s);
  default: return NORM_ERR_UNSUPPORTED;
  }
}

} // namespace dln
