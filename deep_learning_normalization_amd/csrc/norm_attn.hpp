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
  float scale;                        // the logit scale
  float scale_log2;                   // the logit scale times log2(e)
};

// The keys normalised by a pass of their own into a dense [B * S][Hk][D] bf16 buffer.
struct KnormArgs {
  const uint16_t *k;                  // bf16 [B][S][Hk][D], token stride ldk
  const uint16_t *wk, *bk;            // bf16 [D]; bk nullptr: no beta
  uint16_t *out;                      // bf16 [B * S * Hk][D]
  int64_t nkeys;                      // B * S * Hk
  int64_t ldk;
  int32_t Hk;
  float eps;
};

// A call whose keys are each read by at least this many (query block, query head) pairs
// normalises them in a pass of its own when the caller gives a workspace.
constexpr int64_t kAttnKeyPassReuse = 8;

norm_status_t launch_key_norm(bool layernorm, const KnormArgs &a, hipStream_t s);
// keys_normed: a.k holds keys normalised by launch_key_norm (the queries are still normalised
// by the attention kernel).
norm_status_t launch_attention(int norm, bool keys_normed, bool causal, const AttnArgs &a,
                               hipStream_t s);

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
  const void *workspace;
  size_t workspace_bytes;
};

// Bytes of workspace the key-norm pass needs (0 for sizes past what it addresses).
size_t attention_workspace_bytes(int64_t B, int64_t S, int64_t Hk, int64_t D);
norm_status_t check_attention(const AttnCheck &c);

} // namespace dln
