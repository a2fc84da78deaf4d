// norm_lazy.hpp -- a norm deferred into a following projection: the argument blocks of its
// two kernels (norm_lazy.hip), their launchers, and the entry points' argument checks
// (norm_lazy_check.cpp).
#pragma once

#include "norm_internal.hpp"

namespace dln {

// output rows and columns per workgroup of the projection product
constexpr int kLazyTile = 256;

struct FoldArgs {
  const uint16_t *l;  // [Nout, K] bf16, row stride ldl
  const void *gamma;  // [K] bf16 or fp32
  const void *beta;   // [K] or nullptr
  const float *c;     // [Nout] or nullptr
  uint16_t *g;        // [Nout, K] bf16 out, row stride ldg
  float *s;           // [Nout] out or nullptr
  float *t;           // [Nout] out or nullptr
  int64_t K, ldl, ldg;
};

struct LazyArgs {
  const uint16_t *x;  // [M, K] bf16, row stride ldx
  const uint16_t *g;  // [Nout, K] bf16, row stride ldg
  const float *s;     // [Nout] (LayerNorm)
  const float *t;     // [Nout] or nullptr
  const float *mean_in, *rstd_in;  // given statistics, or nullptr
  float *mean_out, *rstd_out;      // formed statistics to store, or nullptr
  uint16_t *y;        // [M, Nout] bf16, row stride ldy
  int64_t M, N, K;    // N = Nout
  int64_t ldx, ldg, ldy;
  int32_t tiles_m, tiles_n;
  float eps, inv_k;
  int32_t vec_store;  // Y 8-byte aligned with ldy a multiple of 4: four columns per store
};

norm_status_t launch_fold_projection(bool f32_weights, const FoldArgs &a, int64_t nout,
                                     hipStream_t s);
norm_status_t launch_lazy_linear(bool layernorm, const LazyArgs &a, hipStream_t s);

// norm_fold_projection and norm_lazy_linear (NORM_OK, NORM_ERR_INVALID_ARG, or
// NORM_ERR_UNSUPPORTED for a layout the product does not read).
struct FoldCheck {
  int kind, dtype;
  const void *L, *gamma, *beta;
  const float *c;
  int64_t Nout, K, ldl, ldg;
  const void *G;
  const float *s, *t;
};
norm_status_t check_fold(const FoldCheck &c);

struct LazyCheck {
  int kind;
  const void *X;
  int64_t ldx, M, K;
  float eps;
  const void *G;
  int64_t ldg, Nout;
  const float *s, *t, *mean_in, *rstd_in;
  const float *mean_out, *rstd_out;
  const void *Y;
  int64_t ldy;
};
norm_status_t check_lazy(const LazyCheck &c);

} // namespace dln
