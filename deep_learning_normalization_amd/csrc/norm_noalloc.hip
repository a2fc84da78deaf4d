// norm_noalloc.hip -- norm_bwd for callers that cannot allocate: the workspace is a file-scope
// device array owned by the library instead of a caller buffer.
//
// The array lives in the code object's zero-initialised data, so every device the library runs
// on holds its own copy of kScratchBytes until the process ends. Host code never passes the
// array's name to a kernel (on the host that name is only a stand-in for the device symbol):
// the first call on a device, with that device current, asks the runtime for the array's device
// address with hipGetSymbolAddress and keeps it per device; every later call passes that
// address as the workspace of the ordinary backward.
//
// Nothing in the backward's workspace has to start at zero: its fused pass writes the header
// and every column-partial row before the column reduction reads them, and the split scheme's
// exchange words carry a per-call tag (under graph capture they are cleared by a kernel, as for
// any workspace). Every call on one device shares the array, so calls that overlap in time on
// one device (different streams or threads without ordering between them) race on it.
#include <atomic>
#include <mutex>

#include "norm_internal.hpp"

namespace dln {
namespace {

// 96 MiB: the looped LayerNorm backward of 16384-element bf16 rows (two workgroups per CU on up
// to 256 CUs) needs 64 MiB of column partials plus the header
constexpr size_t kScratchBytes = (size_t)96 << 20;
constexpr int kMaxScratchDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_scratch_once[kMaxScratchDevices];
std::atomic<void *> g_scratch_ptr[kMaxScratchDevices];

// The current device's address of `scratch` (looked up once per device, with it current).
norm_status_t device_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
    return NORM_ERR_HIP;
  std::call_once(g_scratch_once[dev], [dev] {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess)
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    else
      (void)hipGetLastError(); // leave no error for the caller's next check
  });
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) return NORM_ERR_HIP;
  *out = p;
  return NORM_OK;
}

} // namespace
} // namespace dln

extern "C" norm_status_t norm_bwd_noalloc(norm_kind_t kind, const void *X, const void *dY,
                                          const void *dH, const void *W, const float *mean,
                                          const float *rstd, float eps, int64_t M, int64_t N,
                                          norm_dtype_t dtype, void *dX, void *dR, void *dW,
                                          void *dB, norm_stream_t stream) {
  // the same checks as norm_bwd, minus the workspace (it comes from the scratch below)
  if (N <= 0) return NORM_ERR_INVALID_ARG;
  dln::BwdCheck c{kind, dtype, X,  dY, dH, W,  mean,    rstd, eps, M, N, dX, dR, dW, dB,
                  nullptr, 0,  1,  1,  N,  N,  N, N, N};
  norm_status_t st = dln::check_bwd(c);
  if (st != NORM_OK) return st;
  size_t need = 0;
  st = norm_workspace_size(kind, dtype, NORM_PASS_BWD, M, N, 0, &need);
  if (st != NORM_OK) return st;
  if (need > dln::kScratchBytes) return NORM_ERR_WORKSPACE;
  void *ws = nullptr;
  st = dln::device_scratch(&ws);
  if (st != NORM_OK) return st;
  return norm_bwd(kind, X, dY, dH, W, mean, rstd, eps, M, N, dtype, dX, dR, dW, dB, ws,
                  dln::kScratchBytes, stream);
}
