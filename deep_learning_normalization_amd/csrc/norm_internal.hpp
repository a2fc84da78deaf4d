// norm_internal.hpp -- host-side types shared by the C ABI layer and the kernel launchers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "norm.h"
#include "norm_plan.hpp"

namespace dln {

// Launch parameter blocks (passed by value to kernels).
struct FwdArgs {
  const void *x;
  const void *r;      // residual or nullptr
  const void *w;
  const void *b;      // bias or nullptr
  void *y;
  void *h;            // residual output or nullptr
  float *mean;        // or nullptr
  float *rstd;        // or nullptr
  float *rowpart;     // split: [M][chunks][4]
  uint64_t *xpart;    // split exchange form: [M][chunks][kXchgWordsPerChunk] exchange words
  uint64_t *xerr;     // split exchange form: the workspace header's exchange-failure word
  int64_t xgroups;    // split exchange form: row groups
  uint32_t polls;     // split exchange form: polls before a row is given up
  uint32_t tag;       // split exchange form: this call's tag (never 0 or ~0)
  int32_t withhold;   // split exchange form, tests only: chunk 0 publishes nothing
  int64_t ldx, ldr, ldy, ldh; // elements between row starts of X, R, Y, H (N when contiguous)
  int64_t M;
  int32_t N;
  int32_t nacc;       // accesses per row (N / epv)
  int32_t period;     // wave/block at the full width, rows off 16-byte boundaries: the number
                      // of row phase classes P (1, 2, 4 or 8); 0 for aligned rows
  int32_t phase0;     // with period: elements by which row 0 starts past a 16-byte boundary
  int32_t dphase;     // with period: the same for the step from one row to the next
  int64_t chunks;     // split
  int32_t chunk_acc;  // split: accesses per chunk
  int32_t layernorm;  // 1 LayerNorm, 0 RMSNorm
  int32_t blocked;    // wave/block: contiguous row blocks per workgroup (else interleaved)
  float eps;
  float inv_n;        // 1 / N
};

struct BwdArgs {
  const void *x;
  const void *dy;
  const void *dh;     // or nullptr
  const void *w;
  const float *mean;  // or nullptr (recompute)
  const float *rstd;  // or nullptr (recompute)
  void *dx;
  void *dr;           // separate dR buffer or nullptr
  void *dw;           // split scheme with one row group: final dW written directly, else nullptr
  void *db;           // as dw, for dB
  float *colpart;     // [2][partials][N]
  int64_t *header;    // workspace header: magic, partials, N
  float *rowpart;     // split: [M][chunks][4]
  float *stats;       // split without saved stats: [2][M]
  uint64_t *xpart;    // split exchange form: [M][chunks][kXchgWordsPerChunk] exchange words,
                      // or nullptr when the two-pass form runs
  uint64_t *xerr;     // split exchange form: the workspace header's exchange-failure word
  uint32_t polls;     // split exchange form: polls before a row is given up
  uint32_t tag;       // split exchange form: this call's tag (never 0 or ~0)
  int32_t withhold;   // split exchange form, tests only: chunk 0 publishes nothing
  int64_t ldx, lddy, lddh, lddx, lddr; // elements between row starts (N when contiguous)
  int64_t M;
  int32_t N;
  int32_t nacc;
  int32_t period;     // as in FwdArgs
  int32_t phase0;
  int32_t dphase;
  int64_t chunks;
  int32_t chunk_acc;
  int64_t partials;
  int64_t row_groups;
  int64_t rows_per_group;
  int32_t layernorm;
  int32_t want_db;
  int32_t blocked;    // wave/block: contiguous row blocks per workgroup (else interleaved)
  float eps;
  float inv_n;
};

struct ReduceArgs {
  const int64_t *header; // written by the fused pass: magic, partials, N
  const float *colpart;  // [2][partials][N]
  void *dw;
  void *db;              // or nullptr
  int64_t max_partials;  // partial rows the workspace can hold
  int32_t N;
};

// Launchers (one translation unit per scheme family). Each returns NORM_OK or
// NORM_ERR_UNSUPPORTED / NORM_ERR_HIP.
norm_status_t launch_team_fwd(const Plan &p, norm_dtype_t dtype, const FwdArgs &a,
                              hipStream_t s);
norm_status_t launch_team_bwd(const Plan &p, norm_dtype_t dtype, const BwdArgs &a,
                              hipStream_t s);
// the team kernels of one storage combination, every access width (norm_team_<type>.hip)
#define DLN_TEAM_TYPE_LAUNCHERS(tag)                                                            \
  norm_status_t launch_team_fwd_##tag(const Plan &p, const FwdArgs &a, hipStream_t s);          \
  norm_status_t launch_team_bwd_##tag(const Plan &p, const BwdArgs &a, hipStream_t s);
DLN_TEAM_TYPE_LAUNCHERS(f32)
DLN_TEAM_TYPE_LAUNCHERS(bf16)
DLN_TEAM_TYPE_LAUNCHERS(bf16w)
DLN_TEAM_TYPE_LAUNCHERS(f16)
DLN_TEAM_TYPE_LAUNCHERS(f16w)
#undef DLN_TEAM_TYPE_LAUNCHERS
// rows of 1024-2048 full-width accesses: two sweeps per row, the second from the L2
norm_status_t launch_looped_bwd(const Plan &p, norm_dtype_t dtype, const BwdArgs &a,
                                hipStream_t s);
norm_status_t launch_split_fwd(const Plan &p, norm_dtype_t dtype, const FwdArgs &a,
                               hipStream_t s);
norm_status_t launch_split_bwd(const Plan &p, norm_dtype_t dtype, const BwdArgs &a,
                               hipStream_t s);
// the split scheme in one pass, chunk partials exchanged between the workgroups of a row;
// xsplit_ready: whether the device keeps its kernels resident as the plan assumes
bool xsplit_ready(norm_dtype_t dtype, bool layernorm, bool bwd);
// A fresh tag for one call of the exchange form: a process-wide counter from a random start,
// never 0 or ~0.
uint32_t next_exchange_tag();
norm_status_t launch_xsplit_fwd(const Plan &p, norm_dtype_t dtype, const FwdArgs &a,
                                hipStream_t s);
norm_status_t launch_xsplit_bwd(norm_dtype_t dtype, const BwdArgs &a, hipStream_t s);
norm_status_t launch_reduce(norm_dtype_t dtype, const ReduceArgs &a, hipStream_t s);
norm_status_t launch_zero(void *p, size_t bytes, hipStream_t s);

// Events armed by norm_set_launch_events for the calling thread's next entry point: start is
// attached to the first kernel that call launches, stop to every kernel (the last one wins), so
// the pair brackets exactly the GPU time of the call's kernels.
struct LaunchEvents {
  hipEvent_t start;
  hipEvent_t stop;
};
LaunchEvents &launch_events();

template <typename... P, typename Tup, size_t... I>
hipError_t launch_tuple(void (*k)(P...), dim3 grid, dim3 block, hipStream_t s, Tup &t,
                        std::index_sequence<I...>) {
  void *argv[sizeof...(P) + 1] = {static_cast<void *>(&std::get<I>(t))..., nullptr};
  LaunchEvents &ev = launch_events();
  if (ev.stop) {
    const hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void *>(k), grid, block, argv,
                                            0, s, ev.start, ev.stop, 0);
    ev.start = nullptr;
    return e;
  }
  return hipLaunchKernel(reinterpret_cast<const void *>(k), grid, block, argv, 0, s);
}

// Every kernel of the library is launched through here (no dynamic LDS).
template <typename... P, typename... A>
hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, hipStream_t s, A... a) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> t{static_cast<P>(a)...};
  return launch_tuple(k, grid, block, s, t, std::index_sequence_for<P...>{});
}

// First thread of the fused backward pass records the partial count for the reduction.
__device__ __forceinline__ void write_ws_header(int64_t *h, int64_t partials, int64_t N) {
  if (h && blockIdx.x == 0 && threadIdx.x == 0) {
    h[0] = kWsMagic;
    h[1] = partials;
    h[2] = N;
  }
}

} // namespace dln
