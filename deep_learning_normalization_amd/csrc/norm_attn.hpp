// norm_attn.hpp -- attention over normalised queries and keys in one kernel: the argument block
// of the kernel (norm_attn.hip), its launcher, and the entry point's argument check
// (norm_attn_check.cpp).
#pragma once

#include "norm_internal.hpp"

namespace dln {

constexpr int kAttnD = 128;      // head dimension the kernel is built for
constexpr int kAttnBQ = 256;     // queries per workgroup
constexpr int kAttnBK = 64;      // keys per staged tile

// What happens to the query and key vectors before the scores.
enum AttnNorm { ATTN_LAYERNORM = 0, ATTN_RMSNORM = 1, ATTN_NO_NORM = 2 };

struct AttnArgs {
  const uint16_t *q, *k, *v;          // bf16: q [B][S][Hq][D], k and v [B][S][Hk][D]
  const uint16_t *wq, *bq, *wk, *bk;  // bf16 [D] each: gammas and (LayerNorm) betas, or nullptr
  uint16_t *o;                        // bf16 [B][S][Hq][D]
  float *lse;                         // [B][Hq][S] natural-log softmax normalisers, or nullptr
  int64_t ldq, ldk, ldv, ldo;         // elements from one token to the next
  int32_t B, S, Hq, Hk;
  int32_t qblocks;                    // ceil(S / kAttnBQ)
  float eps;
  float scale_log2;                   // the logit scale times log2(e)
};

norm_status_t launch_attention(int norm, bool causal, const AttnArgs &a, hipStream_t s);

// norm_attention_fwd's checks (NORM_OK, NORM_ERR_INVALID_ARG, or NORM_ERR_UNSUPPORTED for a
// head size or layout the kernel does not read).
struct AttnCheck {
  int kind;
  uint32_t flags;
  int64_t B, S, Hq, Hk, D;
  const void *Q, *K, *V;
  int64_t ldq, ldk, ldv;
  const void *wq, *bq, *wk, *bk;
  float eps, scale;
  const void *O;
  int64_t ldo;
  const float *lse;
};
norm_status_t check_attention(const AttnCheck &c);

} // namespace dln
