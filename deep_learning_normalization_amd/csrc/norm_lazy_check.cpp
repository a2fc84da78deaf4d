// norm_lazy_check.cpp -- argument checks of the fused entry points, norm_fold_projection,
// norm_lazy_linear and norm_attention_fwd (host only, no device access): sizes, NULL pointers,
// overlaps and the layouts the kernels read.
#include <cmath>
#include <cstdint>

#include "norm_attn.hpp"
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
  // rows of a 256-row tile are addressed by 32-bit byte offsets from its first row
  if (c.ldx >= (1 << 23) || c.ldg >= (1 << 23)) return NORM_ERR_UNSUPPORTED;
  return NORM_OK;
}

norm_status_t check_attention(const AttnCheck &c) {
  const bool nonorm = (c.flags & NORM_ATTN_NO_NORM) != 0;
  if (c.flags & ~(uint32_t)(NORM_ATTN_CAUSAL | NORM_ATTN_NO_NORM)) return NORM_ERR_INVALID_ARG;
  if (!nonorm && !valid_kind(c.kind)) return NORM_ERR_INVALID_ARG;
  if (c.B < 0 || c.S < 0 || c.Hq <= 0 || c.Hk <= 0 || c.D <= 0 || c.Hq % c.Hk != 0)
    return NORM_ERR_INVALID_ARG;
  if (c.B > kMaxN || c.S > kMaxN || c.Hq > kMaxN || c.D > kMaxN || c.Hq > kMaxN / c.D)
    return NORM_ERR_INVALID_ARG;
  if (!(c.eps >= 0.0f) || c.eps == INFINITY) return NORM_ERR_INVALID_ARG;
  if (!(c.scale > 0.0f) || c.scale == INFINITY) return NORM_ERR_INVALID_ARG;
  if (nonorm ? (c.wq || c.bq || c.wk || c.bk) : (!c.wq || !c.wk)) return NORM_ERR_INVALID_ARG;
  if (!nonorm && c.kind == NORM_RMSNORM && (c.bq || c.bk)) return NORM_ERR_INVALID_ARG;
  if (c.B == 0 || c.S == 0) return NORM_OK; // nothing to read or write
  if (!c.Q || !c.K || !c.V || !c.O) return NORM_ERR_INVALID_ARG;
  const int64_t T = c.B * c.S; // tokens
  if (!stride_ok(T, c.Hq * c.D, c.ldq) || !stride_ok(T, c.Hk * c.D, c.ldk) ||
      !stride_ok(T, c.Hk * c.D, c.ldv) || !stride_ok(T, c.Hq * c.D, c.ldo))
    return NORM_ERR_INVALID_ARG;
  const size_t nd = (size_t)c.D * 2;
  const Span in[] = {{c.Q, span(T, c.Hq * c.D, c.ldq, 2)}, {c.K, span(T, c.Hk * c.D, c.ldk, 2)},
                     {c.V, span(T, c.Hk * c.D, c.ldv, 2)}, {c.wq, nd}, {c.bq, nd},
                     {c.wk, nd}, {c.bk, nd}};
  if (!c.workspace != !c.workspace_bytes) return NORM_ERR_INVALID_ARG;
  const Span out[] = {{c.O, span(T, c.Hq * c.D, c.ldo, 2)},
                      {c.lse, (size_t)c.B * (size_t)c.Hq * (size_t)c.S * 4},
                      {c.workspace, c.workspace_bytes}};
  if (!disjoint(in, 7, out, 3)) return NORM_ERR_INVALID_ARG;
  if ((uintptr_t)c.lse & 3u) return NORM_ERR_INVALID_ARG;
  // the kernel: head size 128, 16-byte loads and stores of 8 values, a grid of one workgroup
  // per 256 queries of each (batch, query head)
  if (c.D != kAttnD) return NORM_ERR_UNSUPPORTED;
  const void *ptrs[] = {c.Q, c.K, c.V, c.O, c.wq, c.bq, c.wk, c.bk, c.workspace};
  if (c.ldq % 8 || c.ldk % 8 || c.ldv % 8 || c.ldo % 8 || common_align(ptrs, 9) < 16)
    return NORM_ERR_UNSUPPORTED;
  // key and value rows are addressed by 32-bit byte offsets within a tile
  if (c.ldk >= (1 << 24) || c.ldv >= (1 << 24)) return NORM_ERR_UNSUPPORTED;
  const int64_t qblocks = (c.S + kAttnBQ - 1) / kAttnBQ;
  if (c.B * c.Hq > 0x7fffffffLL / qblocks) return NORM_ERR_UNSUPPORTED;
  return NORM_OK;
}

size_t attention_workspace_bytes(int64_t B, int64_t S, int64_t Hk, int64_t D) {
  if (B <= 0 || S <= 0 || Hk <= 0 || D <= 0 || B > kMaxN || S > kMaxN || Hk > kMaxN ||
      D > kMaxN)
    return 0;
  const int64_t keys = B * S; // < 2^62
  if (keys > INT64_MAX / 2 / D / Hk) return 0;
  return (size_t)(keys * Hk * D * 2);
}

} // namespace dln
