// norm_lazy_check.cpp -- argument checks of norm_fold_projection and norm_lazy_linear (host
// only, no device access): sizes, NULL pointers, overlaps and the layouts the product reads.
#include <cmath>
#include <cstdint>

#include "norm_lazy.hpp"

namespace dln {
namespace {

constexpr int64_t kMaxN = 2147483647; // a row length or output count fits a 32-bit int

bool valid_kind(int k) { return k == NORM_LAYERNORM || k == NORM_RMSNORM; }

// bytes per gamma / beta value
size_t weight_size(int d) { return d == NORM_BF16 ? 2 : 4; }

struct Span {
  const void *p;
  size_t n;
};

bool overlap(Span a, Span b) {
  if (!a.p || !b.p || !a.n || !b.n) return false;
  const uintptr_t x = (uintptr_t)a.p, y = (uintptr_t)b.p;
  return x < y + b.n && y < x + a.n;
}

// every output disjoint from every input and from every other output
bool disjoint(const Span *in, int nin, const Span *outs, int nout) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], in[j])) return false;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return false;
  }
  return true;
}

// a row stride of at least N that keeps (M - 1) * ld + N elements addressable
bool stride_ok(int64_t M, int64_t N, int64_t ld) {
  if (ld < N) return false;
  return M <= (INT64_MAX / 16) / ld;
}

// bytes an [M, N] tensor with row stride ld spans
size_t span(int64_t M, int64_t N, int64_t ld, size_t s) {
  return M > 0 ? ((size_t)(M - 1) * (size_t)ld + (size_t)N) * s : 0;
}

} // namespace

norm_status_t check_fold(const FoldCheck &c) {
  if (!valid_kind(c.kind) || (c.dtype != NORM_BF16 && c.dtype != NORM_BF16_F32W))
    return NORM_ERR_INVALID_ARG;
  if (!c.L || !c.gamma || !c.G || c.Nout <= 0 || c.K <= 0 || c.K > kMaxN)
    return NORM_ERR_INVALID_ARG;
  if (!stride_ok(c.Nout, c.K, c.ldl) || !stride_ok(c.Nout, c.K, c.ldg))
    return NORM_ERR_INVALID_ARG;
  const bool ln = c.kind == NORM_LAYERNORM;
  if (ln ? !c.s : c.beta != nullptr) return NORM_ERR_INVALID_ARG;
  if ((c.beta || c.c) && !c.t) return NORM_ERR_INVALID_ARG;
  const size_t ws = weight_size(c.dtype);
  const Span in[] = {{c.L, span(c.Nout, c.K, c.ldl, 2)}, {c.gamma, (size_t)c.K * ws},
                     {c.beta, (size_t)c.K * ws}, {c.c, (size_t)c.Nout * 4}};
  const Span out[] = {{c.G, span(c.Nout, c.K, c.ldg, 2)},
                      {ln ? c.s : nullptr, (size_t)c.Nout * 4}, {c.t, (size_t)c.Nout * 4}};
  if (!disjoint(in, 4, out, 3)) return NORM_ERR_INVALID_ARG;
  const void *ptrs[] = {c.L, c.G};
  if (common_align(ptrs, 2) < 2 || ((uintptr_t)c.gamma % ws) || ((uintptr_t)c.beta % ws) ||
      ((uintptr_t)c.c & 3u) || ((uintptr_t)c.s & 3u) || ((uintptr_t)c.t & 3u))
    return NORM_ERR_INVALID_ARG;
  return NORM_OK;
}

norm_status_t check_lazy(const LazyCheck &c) {
  if (!valid_kind(c.kind)) return NORM_ERR_INVALID_ARG;
  const bool ln = c.kind == NORM_LAYERNORM;
  if (c.M < 0 || c.K <= 0 || c.K > kMaxN || c.Nout <= 0 || c.Nout > kMaxN)
    return NORM_ERR_INVALID_ARG;
  if (!(c.eps >= 0.0f) || c.eps == INFINITY) return NORM_ERR_INVALID_ARG;
  if (c.M == 0) return NORM_OK; // nothing to read or write
  if (!c.X || !c.G || !c.Y) return NORM_ERR_INVALID_ARG;
  if (!stride_ok(c.M, c.K, c.ldx) || !stride_ok(c.Nout, c.K, c.ldg) ||
      !stride_ok(c.M, c.Nout, c.ldy))
    return NORM_ERR_INVALID_ARG;
  if (ln && !c.s) return NORM_ERR_INVALID_ARG;
  // given statistics: rstd, and the mean for LayerNorm; formed ones: optional outputs
  if (c.rstd_in ? (ln != (c.mean_in != nullptr) || c.mean_out || c.rstd_out)
                : (c.mean_in != nullptr))
    return NORM_ERR_INVALID_ARG;
  if (!ln && c.mean_out) return NORM_ERR_INVALID_ARG;
  const Span in[] = {{c.X, span(c.M, c.K, c.ldx, 2)}, {c.G, span(c.Nout, c.K, c.ldg, 2)},
                     {ln ? c.s : nullptr, (size_t)c.Nout * 4}, {c.t, (size_t)c.Nout * 4},
                     {c.mean_in, (size_t)c.M * 4}, {c.rstd_in, (size_t)c.M * 4}};
  const Span out[] = {{c.Y, span(c.M, c.Nout, c.ldy, 2)}, {c.mean_out, (size_t)c.M * 4},
                      {c.rstd_out, (size_t)c.M * 4}};
  if (!disjoint(in, 6, out, 3)) return NORM_ERR_INVALID_ARG;
  const void *f32p[] = {c.s, c.t, c.mean_in, c.rstd_in, c.mean_out, c.rstd_out};
  if (common_align(f32p, 6) < 4 || ((uintptr_t)c.Y & 1u)) return NORM_ERR_INVALID_ARG;
  // the product reads X and G in 16-byte chunks of 8 values
  const void *ptrs[] = {c.X, c.G};
  if (c.K % 8 || c.ldx % 8 || c.ldg % 8 || common_align(ptrs, 2) < 16)
    return NORM_ERR_UNSUPPORTED;
  return NORM_OK;
}

} // namespace dln
