// norm_team_menu.hpp -- the compiled shapes of the team kernels and their dispatch by plan,
// for every access width: 16-byte and element-wise accesses, and 8- and 4-byte accesses for
// rows whose length or pointers rule out 16-byte ones. Each storage type's translation unit
// (norm_team_<type>.hip) instantiates them for its types only, so they compile in parallel.
//
// 8- and 4-byte shapes are the full-width menus with the accesses per thread multiplied by the
// width ratio (SC = 16-byte elements / elements per access), so a thread holds as many
// elements in registers as its full-width counterpart; their menu entries are in full-width
// units (V) and launch V * SC accesses per thread, one row per team.
#pragma once

#include "norm_team_kernels.hpp"

namespace dln {

// The menu of compiled shapes. Wave scheme: workgroups of 256 threads (4 one-wave teams).
// Block scheme: teams of up to LB threads. Entries are (VPT, ROWS, LB).
#define DLN_WAVE_MENU(X)                                                                        \
  X(1, 1, 256) X(1, 2, 256) X(1, 4, 256) X(2, 1, 256) X(2, 2, 256) X(2, 4, 256) X(4, 1, 256)       \
      X(4, 2, 256) X(8, 1, 256)
#define DLN_WAVE_MENU_SCALAR(X) X(1, 1, 256) X(2, 1, 256) X(4, 1, 256) X(8, 1, 256) X(16, 1, 256)
#define DLN_BLOCK_MENU(X)                                                                       \
  X(1, 1, 256) X(1, 2, 256) X(1, 4, 256) X(2, 1, 256) X(2, 2, 256) X(2, 4, 256) X(4, 1, 256)       \
      X(8, 1, 256) X(1, 1, 512) X(1, 2, 512) X(1, 4, 512) X(2, 1, 512) X(2, 2, 512) X(4, 1, 512)   \
          X(1, 1, 768) X(1, 2, 768) X(1, 1, 1024) X(1, 2, 1024) X(2, 1, 1024)
#define DLN_BLOCK_MENU_SCALAR(X) X(4, 1, 1024) X(8, 1, 1024)

template <typename T, typename TW>
norm_status_t team_fwd_typed(const Plan &p, const FwdArgs &a, hipStream_t s) {
  const bool resid = a.r != nullptr;
  const int lb = p.lb;
  hipError_t e = hipErrorInvalidConfiguration;
  bool found = false;
  if (p.scheme == NORM_SCHEME_WAVE) {
    if (p.vector) {
#define X(V, R, L)                                                                              \
  if (!found && p.vpt == V && p.rows == R && lb == L) {                                         \
    found = true;                                                                               \
    e = fwd_launch<T, TW, full_epv<T>(), V, R, L, true>(p, a, resid, s);                           \
  }
      DLN_WAVE_MENU(X)
#undef X
    } else {
#define X(V, R, L)                                                                              \
  if (!found && p.vpt == V && p.rows == R && lb == L) {                                         \
    found = true;                                                                               \
    e = fwd_launch<T, TW, 1, V, R, L, true>(p, a, resid, s);                                \
  }
      DLN_WAVE_MENU_SCALAR(X)
#undef X
    }
  } else {
    if (p.vector) {
#define X(V, R, L)                                                                              \
  if (!found && p.vpt == V && p.rows == R && lb == L) {                                         \
    found = true;                                                                               \
    e = fwd_launch<T, TW, full_epv<T>(), V, R, L, false>(p, a, resid, s);                          \
  }
      DLN_BLOCK_MENU(X)
#undef X
    } else {
#define X(V, R, L)                                                                              \
  if (!found && p.vpt == V && p.rows == R && lb == L) {                                         \
    found = true;                                                                               \
    e = fwd_launch<T, TW, 1, V, R, L, false>(p, a, resid, s);                               \
  }
      DLN_BLOCK_MENU_SCALAR(X)
#undef X
    }
  }
  if (!found) return NORM_ERR_UNSUPPORTED;
  return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

template <typename T, typename TW>
norm_status_t team_bwd_typed(const Plan &p, const BwdArgs &a, hipStream_t s) {
  const int lb = p.lb;
  hipError_t e = hipErrorInvalidConfiguration;
  bool found = false;
  if (p.scheme == NORM_SCHEME_WAVE) {
    if (p.vector) {
#define X(V, R, L)                                                                              \
  if (!found && p.vpt == V && p.rows == R && lb == L) {                                         \
    found = true;                                                                               \
    e = bwd_launch<T, TW, full_epv<T>(), V, R, L, true>(p, a, s);                                  \
  }
      DLN_WAVE_MENU(X)
#undef X
    } else {
#define X(V, R, L)                                                                              \
  if (!found && p.vpt == V && p.rows == R && lb == L) {                                         \
    found = true;                                                                               \
    e = bwd_launch<T, TW, 1, V, R, L, true>(p, a, s);                                       \
  }
      DLN_WAVE_MENU_SCALAR(X)
#undef X
    }
  } else {
    if (p.vector) {
#define X(V, R, L)                                                                              \
  if (!found && p.vpt == V && p.rows == R && lb == L) {                                         \
    found = true;                                                                               \
    e = bwd_launch<T, TW, full_epv<T>(), V, R, L, false>(p, a, s);                                 \
  }
      DLN_BLOCK_MENU(X)
#undef X
    } else {
#define X(V, R, L)                                                                              \
  if (!found && p.vpt == V && p.rows == R && lb == L) {                                         \
    found = true;                                                                               \
    e = bwd_launch<T, TW, 1, V, R, L, false>(p, a, s);                                      \
  }
      DLN_BLOCK_MENU_SCALAR(X)
#undef X
    }
  }
  if (!found) return NORM_ERR_UNSUPPORTED;
  return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

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

// 16-bit activations (bf16, fp16): 8-byte (4 elements) or 4-byte (2 elements) accesses
template <typename T, typename TW>
norm_status_t fwd_16(const Plan &p, const FwdArgs &a, hipStream_t s) {
  if (p.epv == 4) return fwd_narrow<T, TW, 4>(p, a, s);
  if (p.epv == 2) return fwd_narrow<T, TW, 2>(p, a, s);
  return NORM_ERR_UNSUPPORTED;
}
template <typename T, typename TW>
norm_status_t bwd_16(const Plan &p, const BwdArgs &a, hipStream_t s) {
  if (p.epv == 4) return bwd_narrow<T, TW, 4>(p, a, s);
  if (p.epv == 2) return bwd_narrow<T, TW, 2>(p, a, s);
  return NORM_ERR_UNSUPPORTED;
}

// Every access width of one storage combination (T activations, TW weights).
template <typename T, typename TW>
norm_status_t team_fwd_any(const Plan &p, const FwdArgs &a, hipStream_t s) {
  if (p.scale == 1) return team_fwd_typed<T, TW>(p, a, s);
  if constexpr (sizeof(T) == 2) return fwd_16<T, TW>(p, a, s);
  return p.epv == 2 ? fwd_narrow<T, TW, 2>(p, a, s) : NORM_ERR_UNSUPPORTED;
}

template <typename T, typename TW>
norm_status_t team_bwd_any(const Plan &p, const BwdArgs &a, hipStream_t s) {
  if (p.scale == 1) return team_bwd_typed<T, TW>(p, a, s);
  if constexpr (sizeof(T) == 2) return bwd_16<T, TW>(p, a, s);
  return p.epv == 2 ? bwd_narrow<T, TW, 2>(p, a, s) : NORM_ERR_UNSUPPORTED;
}

} // namespace dln
