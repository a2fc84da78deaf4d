// norm_plan.hpp -- host logic of the norm library that needs no GPU: the shape dispatcher
// (launch plans and workspace layout) and the argument checks. Compiles with any C++17
// compiler; no HIP header is included.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "norm.h"

namespace dln {

// A launch plan: which scheme and kernel shape a (kind, pass, M, N, dtype) call uses, and
// where its workspace regions live.
struct Plan {
  int scheme = NORM_SCHEME_BLOCK;
  int vector = 1;          // vector accesses of whole 32-bit words (1) or element-wise (0)
  int epv = 8;             // elements per access
  int64_t nacc = 0;        // accesses per row: N / epv; with phase classes the most any class
                           // needs, ceil((N + pe) / epv)
  int period = 0;          // wave/block at the full width, rows off 16-byte boundaries: row phase
                           // classes P (the grid is a multiple of P); 0 for aligned rows
  int scale = 1;           // full-width elements (16 bytes) / epv on the vector paths: 1, 2, 4
  int access_bytes = 16;   // bytes per access: 16, 8 or 4, or the element size
  int threads = 256;       // workgroup size
  int lb = 256;            // compiled workgroup-size bound of the kernel (>= threads)
  int team_threads = 256;  // threads sharing a row (64 for the wave scheme)
  int vpt = 1;             // accesses per thread per row (per chunk for split)
  int rows = 1;            // rows a team holds at once
  int row_order = 0;       // wave/block: 0 interleaved row groups, 1 contiguous blocks
  int64_t grid = 1;        // workgroups of the main (persistent) kernel
  int64_t chunks = 1;      // split: chunks per row
  int64_t chunk_elems = 0; // split: elements per chunk
  int64_t row_groups = 1;  // split backward: row groups
  int64_t rows_per_group = 0; // split backward: rows per group
  int64_t partials = 0;    // rows of fp32 column partials (backward)
  int xchg = 0;            // split: the single-pass exchange form may run (norm_xsplit.hip)
  int64_t xrow_groups = 0; // split exchange form: row groups (its grid is xrow_groups x chunks)
  // workspace layout (bytes from the workspace start; every region 256-byte aligned)
  size_t off_header = 0;   // kWsHeaderBytes at the workspace start (see below)
  size_t off_colpart = 0;  // [2][partials][N] fp32: dW partials then dB partials
  size_t off_rowpart = 0;  // split: [M][chunks][4] fp32 per-chunk row partials
  size_t off_stats = 0;    // split backward without saved stats: [M] mean then [M] rstd
  size_t off_xpart = 0;    // split exchange form: [M][chunks][kXchgWordsPerChunk] 64-bit words
  size_t ws_bytes = 0;
};

// Every workspace starts with this header of 64-bit words. The backward's fused pass writes
// words 0-2 (magic, partial rows, N) so that the column reduction (possibly a separate call)
// knows how many partial rows follow; word 3 is set by a split-scheme exchange wait that gave
// up, and read and cleared by norm_workspace_status.
constexpr size_t kWsHeaderBytes = 256;
constexpr int64_t kWsMagic = 0x4E4F524D50415254LL; // "NORMPART"
constexpr int kWsErrWord = 3;
constexpr uint64_t kXchgFailWord = 0x584348474641494CULL; // "XCHGFAIL"
// Largest compute-unit count of a gfx950 device: norm_workspace_bytes sizes for every count up
// to this one.
constexpr int kMaxCuCount = 256;

// Split exchange form: workgroups per CU its kernels are compiled to keep resident (their
// launch bounds), which bounds its grid, and the most chunks per row it exchanges.
constexpr int kXchgFwdPerCu = 3;    // weights in registers (fp32 beside 16-bit activations)
constexpr int kXchgFwdPerCuLds = 4; // weights in LDS (stored like the activations)
constexpr int kXchgBwdPerCu = 2;
constexpr int xchg_fwd_per_cu(norm_dtype_t d) {
  return (d == NORM_BF16_F32W || d == NORM_F16_F32W) ? kXchgFwdPerCu : kXchgFwdPerCuLds;
}
// 64-bit exchange words per (row, chunk): each partial value (at most three) is published as a
// pair of words, padded to eight (64 bytes).
constexpr int kXchgWordsPerChunk = 8;
constexpr int64_t kXchgPollsDefault = 1 << 19;
constexpr int64_t kXchgPollsMax = 1 << 24;
constexpr int64_t kXchgMaxChunks = 512;
// By default the single-pass split form runs only where a row gathers at most this many chunk
// partials (LayerNorm publishes three per chunk, RMSNorm one), forward and backward;
// NORM_TUNE_SPLIT_EXCHANGE = 1 lifts the limit.
constexpr int64_t kXchgAutoMaxPartialsFwd = 512;
constexpr int64_t kXchgAutoMaxPartialsBwd = 640;

struct Tuning {
  int scheme = NORM_SCHEME_AUTO;
  int grid_per_cu = -1;
  int rows = -1;
  int team_threads = -1;
  int64_t split_chunk = -1;
  int64_t row_groups = -1;
  int teams = -1;
  int row_order = -1;
  int xchg = -1;
  int64_t xchg_polls = -1;
  int xchg_withhold = -1;
  int unaligned = -1;
  int attn_key_pass = -1;
};

const Tuning &tuning();
norm_status_t set_tuning(norm_tune_t key, int64_t value);

// align: the largest power of two, up to 16, that divides the address of every tensor the call
// touches and (times the element size) every row stride (16 for buffers from an allocator; 1
// when unknown or odd). phase0 / dphase: when every [M, N] tensor of the call starts the same
// number of elements past a 16-byte boundary and its row stride moves the start by the same
// number (modulo 16 bytes), those two numbers in elements; else -1.
norm_status_t make_plan(norm_kind_t kind, norm_dtype_t dtype, norm_pass_t pass, int64_t M,
                        int64_t N, int residual, int align, int phase0, int dphase, int cu_count,
                        const Tuning &t, Plan *out);

// The common phase of a call's [M, N] tensors (pointers and row strides, nullptr entries
// ignored) in elements of elem_bytes: writes phase0 and dphase as make_plan takes them.
void common_phase(const void *const *ptrs, const int64_t *ld, int n, size_t elem_bytes,
                  int *phase0, int *dphase);

// Largest workspace any pointer alignment can need for this call on cu_count CUs.
norm_status_t workspace_bytes(norm_kind_t kind, norm_dtype_t dtype, norm_pass_t pass, int64_t M,
                              int64_t N, int residual, int cu_count, const Tuning &t,
                              size_t *bytes);
// The largest of workspace_bytes over every compute-unit count 1 .. kMaxCuCount.
norm_status_t workspace_bytes_any_device(norm_kind_t kind, norm_dtype_t dtype, norm_pass_t pass,
                                         int64_t M, int64_t N, int residual, const Tuning &t,
                                         size_t *bytes);

// Argument checks (no device access). They return NORM_OK or NORM_ERR_INVALID_ARG.
struct FwdCheck {
  int kind, dtype;
  const void *X, *R, *W, *B;
  float eps;
  int64_t M, N;
  void *Y, *H;
  float *mean, *rstd;
  void *ws;
  size_t ws_bytes;
  int64_t ldx, ldr, ldy, ldh; // row strides in elements (each >= N)
  int stats_only;             // the statistics pass alone: no W, B, Y; some output required
};
norm_status_t check_fwd(const FwdCheck &c);

struct BwdCheck {
  int kind, dtype;
  const void *X, *dY, *dH, *W;
  const float *mean, *rstd;
  float eps;
  int64_t M, N;
  void *dX, *dR, *dW, *dB;
  void *ws;
  size_t ws_bytes;
  int need_dx;  // stage 1 (fused pass) is part of the call
  int need_dw;  // stage 2 (column reduction) is part of the call
  int64_t ldx, lddy, lddh, lddx, lddr; // row strides in elements (each >= N)
};
norm_status_t check_bwd(const BwdCheck &c);

bool all_aligned16(const void *const *ptrs, int n);
// The largest power of two, at most 16, dividing every non-null pointer (16 if all are null).
int common_align(const void *const *ptrs, int n);
// align lowered to the largest power of two that also divides each row stride in bytes (the
// row starts of a strided tensor are aligned only that far)
int fold_stride_align(int align, const int64_t *ld, int n, size_t elem_bytes);
// bytes per element of the [M, N] tensors of a dtype
size_t act_elem_size(norm_dtype_t d);
// Alignment the weight-sized outputs (dW, dB) need for the vector stores of an access of epv
// elements.
size_t weight_align_need(norm_dtype_t d, int epv);

} // namespace dln
