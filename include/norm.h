/*
 * norm.h -- C ABI of the MI355X (gfx950) row-wise LayerNorm / RMSNorm library.
 *
 * What the operations compute. Sources are web pages; each is cited by its title.
 *   [P1] "PyTorch atinge desempenho SOTA em normalização com torch.compile" (matsubara.tec.br):
 *     para. 2 -- LayerNorm normalises each row with its mean and variance and applies the
 *                trainable weight (gamma) and bias (beta); RMSNorm divides by the root mean
 *                square instead and has no bias.
 *     para. 3 -- both forwards reduce along the contiguous dimension, then apply pointwise work.
 *     para. 7 -- the backward produces dX, dW and, for LayerNorm, dB.
 *     paras. 8-10 -- dX and the dW/dB column reductions are fused in one pass over the data,
 *                the column sums go through a workspace of per-block partial sums without
 *                atomics, and an extra reduction pass consolidates that workspace.
 *
 * For a row x of N values (in fp32 arithmetic; bf16 inputs are widened exactly):
 *   LayerNorm: mean = sum(x)/N, var = sum((x-mean)^2)/N (biased), rstd = 1/sqrt(var+eps),
 *              y = (x-mean)*rstd*W + B
 *   RMSNorm:   rstd = 1/sqrt(sum(x^2)/N + eps), y = x*rstd*W
 *   Backward, with g = dY*W and xhat the normalised row:
 *              LayerNorm dX = rstd*(g - mean(g) - xhat*mean(g*xhat)),
 *              RMSNorm   dX = rstd*(g - xhat*mean(g*xhat)),
 *              dW = sum over rows of dY*xhat, dB = sum over rows of dY.
 *   Residual variant (fused add in front of the norm): h = R + X rounded once to the storage
 *   dtype is stored in H, and the norm is applied to that stored h; its backward is the plain
 *   backward on H, plus an optional incoming gradient dH of h, and dR = dX.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers on the current HIP device. X, R, Y, H, dY, dH,
 *     dX, dR are row-major contiguous [M, N] (row stride N); W, B, dW, dB are [N]; mean and
 *     rstd are [M] fp32 whatever the dtype; the workspace is raw device memory.
 *   - dtype gives the storage types of the non-statistic tensors (norm_dtype_t: one type for
 *     all, or 16-bit activations with fp32 W, B, dW, dB); arithmetic is fp32, and each output
 *     is rounded once (round to nearest even).
 *   - The caller owns all memory. The library allocates nothing and keeps no state beyond a
 *     per-device cache of the compute-unit count and the tuning overrides below.
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL = the null stream).
 *     Nothing synchronises the host. Device faults surface at the caller's next sync.
 *   - Output buffers must not overlap input buffers (in place is rejected), except that dR
 *     may be the same pointer as dX.
 *   - Accesses are the widest of 16, 8 and 4 bytes (at least two elements) that divides the
 *     row length in bytes and that the alignment common to every tensor pointer allows. An
 *     access of E elements needs E * element size bytes; with fp32 W, B, dW, dB beside bf16
 *     or fp16 activations it needs min(16, 4 E) bytes, for the weights read with it. Rows of an odd
 *     number of elements, or pointers aligned to one element only, run on a slower
 *     element-wise path. Results are the same on every path up to rounding order.
 *   - Arguments are checked before anything is launched; a failed check returns an error and
 *     launches nothing. M == 0 returns NORM_OK with no launch. No C++ exception crosses the
 *     ABI and the library never aborts the process.
 *   - Results are bitwise reproducible run to run on one device (fixed reduction orders, no
 *     atomics). They can differ in the last bits between devices with different CU counts.
 */
#ifndef DLN_NORM_H
#define DLN_NORM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { NORM_LAYERNORM = 0, NORM_RMSNORM = 1 } norm_kind_t;

/*
 * Storage types. NORM_F32, NORM_BF16 and NORM_F16 (IEEE binary16): every tensor in that type.
 * NORM_BF16_F32W / NORM_F16_F32W: X, R, Y, H, dY, dH, dX, dR in bf16 / fp16 and W, B, dW, dB
 * in fp32, the mixed-precision layout in which the parameters keep fp32 master copies ([P2]
 * "Otimização de Performance de GPU: Maximizando Throughput para Treinamento e Inferência de
 * LLM", section on mixed-precision training, which trains in FP16 with FP32 master weights).
 * mean and rstd are fp32 always; all arithmetic is fp32; outputs are rounded to nearest even
 * (fp16 values beyond 65504 round to infinity).
 */
typedef enum {
  NORM_F32 = 0,
  NORM_BF16 = 1,
  NORM_BF16_F32W = 2,
  NORM_F16 = 3,      /* IEEE binary16 */
  NORM_F16_F32W = 4  /* fp16 activations, fp32 W, B, dW, dB */
} norm_dtype_t;

typedef enum {
  NORM_OK = 0,
  NORM_ERR_INVALID_ARG = 1, /* a pointer, size, eps, kind or dtype is not acceptable */
  NORM_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels handle */
  NORM_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than norm_workspace_size() */
  NORM_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  NORM_ERR_EXCHANGE = 5     /* norm_workspace_status only: a call on this workspace gave up
                               waiting for the partial sums of a long row and wrote NaN */
} norm_status_t;

/* Which pass a workspace size or plan is asked for. */
typedef enum {
  NORM_PASS_FWD = 0,
  NORM_PASS_BWD = 1,
  NORM_PASS_STATS = 2 /* norm_stats: the forward's statistics alone (workspace as the forward) */
} norm_pass_t;

/* Kernel scheme chosen for a shape. */
typedef enum {
  NORM_SCHEME_AUTO = -1, /* tuning value only: let the dispatcher choose */
  NORM_SCHEME_WAVE = 0,  /* one row per 64-lane wavefront, registers only (short rows) */
  NORM_SCHEME_BLOCK = 1, /* one row per team of waves, cross-wave sums through LDS */
  NORM_SCHEME_SPLIT = 2, /* one row over several workgroups (very long rows): a single pass
                            in which the row's workgroups exchange their chunk partials through
                            the workspace, each chunk held in registers throughout (16-byte
                            accesses, no residual input, up to 512 chunks, saved statistics
                            for the backward), else two passes, the second re-reading its
                            chunk */
  NORM_SCHEME_LOOP = 3   /* backward only: one row per workgroup in two sweeps, the second
                            from the L2 (rows of 1024-2048 16-byte accesses); forcing it
                            leaves the forward to the dispatcher */
} norm_scheme_t;

typedef void *norm_stream_t; /* a hipStream_t */

/*
 * Forward [P1 paras. 2-3].
 *   kind   LayerNorm or RMSNorm.
 *   X      [M, N] input. Required.
 *   R      [M, N] residual added to X before the norm, or NULL.
 *   W      [N] weight. Required.
 *   B      [N] bias. LayerNorm: optional (NULL means zero). RMSNorm: must be NULL.
 *   eps    added to the variance (LayerNorm) or mean square (RMSNorm) inside the square root;
 *          finite and >= 0.
 *   M, N   rows (>= 0) and row length (1 <= N <= 2^31 - 1).
 *   dtype  storage type of X, R, W, B, Y, H.
 *   Y      [M, N] output. Required.
 *   H      [M, N] output R + X (rounded to dtype). Required when R is given, else NULL.
 *   mean   [M] fp32 row means. LayerNorm: optional. RMSNorm: must be NULL.
 *   rstd   [M] fp32 row 1/sqrt(stat + eps). Optional.
 *   workspace, workspace_bytes: device scratch of at least
 *          norm_workspace_size(kind, dtype, NORM_PASS_FWD, M, N, R != NULL) bytes, 256-byte
 *          aligned; may be NULL when that size is 0. Calls that share a workspace must not
 *          overlap in time.
 * Returns NORM_OK once the kernels are queued.
 * Very long rows (the split scheme's single-pass form) are spread over workgroups that wait
 * for each other's partial sums. The form assumes that every workgroup of a row group gets a
 * compute unit while the others wait: the grid is sized to fit the device at once, but neither
 * HIP nor the hardware promises that workgroups are dispatched in order or that other work on
 * the device leaves room. So the wait is bounded (NORM_TUNE_EXCHANGE_POLLS): a wait that gives
 * up writes NaN into the call's outputs for the rows it could not finish and sets the
 * workspace's exchange-failure word, which norm_workspace_status reports; it never hangs.
 */
norm_status_t norm_fwd(norm_kind_t kind, const void *X, const void *R, const void *W,
                       const void *B, float eps, int64_t M, int64_t N, norm_dtype_t dtype,
                       void *Y, void *H, float *mean, float *rstd, void *workspace,
                       size_t workspace_bytes, norm_stream_t stream);

/*
 * Backward [P1 paras. 7-10]: dX fused with per-block dW/dB partial sums in one pass over
 * X and dY, then a column reduction of the partials into dW/dB.
 *   X      [M, N] the norm's input (for the residual variant: the stored H). Required.
 *   dY     [M, N] gradient of Y. Required.
 *   dH     [M, N] incoming gradient of the residual output H, added to dX; or NULL.
 *   W      [N] weight. Required.
 *   mean, rstd: the forward's [M] fp32 statistics. LayerNorm: both or neither; RMSNorm: mean
 *          must be NULL, rstd optional. When absent they are recomputed from X with eps.
 *   eps, M, N, dtype: as for norm_fwd.
 *   dX     [M, N] output. Required.
 *   dR     [M, N] output equal to dX (residual variant); NULL, dX itself, or a separate buffer.
 *   dW     [N] output. Required.
 *   dB     [N] output. LayerNorm: optional. RMSNorm: must be NULL.
 *   workspace: at least norm_workspace_size(kind, dtype, NORM_PASS_BWD, M, N, 0) bytes.
 * Very long rows with saved statistics take the split scheme's single-pass form, with the
 * bounded wait described at norm_fwd (a wait that gives up leaves NaN in dX, dW and dB).
 */
norm_status_t norm_bwd(norm_kind_t kind, const void *X, const void *dY, const void *dH,
                       const void *W, const float *mean, const float *rstd, float eps,
                       int64_t M, int64_t N, norm_dtype_t dtype, void *dX, void *dR, void *dW,
                       void *dB, void *workspace, size_t workspace_bytes, norm_stream_t stream);

/*
 * norm_bwd without a caller workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation). Arguments,
 * results and errors are those of norm_bwd; the workspace is the library's own device array of
 * 96 MiB per device (zero-initialised data of the code object, held by every device the library
 * runs on until the process ends), so the call allocates nothing and makes no allocating call.
 * A shape whose backward needs more than 96 MiB of workspace on the current device (see
 * norm_workspace_size) returns NORM_ERR_WORKSPACE and launches nothing. Every call on a device
 * shares that array: calls that overlap in time on one device (different streams, or threads
 * without ordering between their calls) race on it and must be serialised by the caller. An
 * exchange wait that gives up writes NaN as for norm_bwd; its failure word stays in the array,
 * which norm_workspace_status cannot read.
 */
norm_status_t norm_bwd_noalloc(norm_kind_t kind, const void *X, const void *dY, const void *dH,
                               const void *W, const float *mean, const float *rstd, float eps,
                               int64_t M, int64_t N, norm_dtype_t dtype, void *dX, void *dR,
                               void *dW, void *dB, norm_stream_t stream);

/*
 * Row strides for the _ex variants below: the number of elements between the starts of
 * consecutive rows of each [M, N] tensor, so a tensor may be a row-strided view (for example
 * the query rows inside a fused query/key/value buffer). 0 means N (contiguous rows); any other
 * value must be >= N, and rows must not overlap one another or any other tensor of the call
 * (overlap is judged on the span (M - 1) * stride + N). Forward: x (X), r (R), y (Y), h (H).
 * Backward: x (its X), dy, dh, dx, dr; dR may alias dX only with the same stride.
 * Accesses are sized by the alignment common to the pointers and to every stride in bytes.
 */
typedef struct {
  int64_t x, r, y, h;
  int64_t dy, dh, dx, dr;
} norm_row_strides_t;

/*
 * The forward's statistics pass alone [P1 paras. 2-3, 6]: mean (LayerNorm) and rstd per row,
 * and H = R + X when R is given, without normalising (no W, B or Y; about half the forward's
 * HBM traffic). The statistics a consumer needs to apply the norm later, for example in the
 * epilogue of a following matrix product ([P3] "Towards Free Normalization", items 3-4 and
 * 9-10). Very long rows use the split scheme's per-chunk statistics over several workgroups
 * and one combine per row.
 *   Arguments as for norm_fwd; at least one of mean, rstd and H must be given; row_strides
 *   may be NULL (contiguous). Workspace: norm_workspace_size(..., NORM_PASS_FWD, ...).
 */
norm_status_t norm_stats(norm_kind_t kind, const void *X, const void *R, float eps, int64_t M,
                         int64_t N, norm_dtype_t dtype, void *H, float *mean, float *rstd,
                         void *workspace, size_t workspace_bytes,
                         const norm_row_strides_t *row_strides, norm_stream_t stream);

/* norm_fwd, norm_bwd and norm_bwd_fused with row strides (row_strides NULL: contiguous, the
 * same as the calls above). Everything else is as documented there. */
norm_status_t norm_fwd_ex(norm_kind_t kind, const void *X, const void *R, const void *W,
                          const void *B, float eps, int64_t M, int64_t N, norm_dtype_t dtype,
                          void *Y, void *H, float *mean, float *rstd, void *workspace,
                          size_t workspace_bytes, const norm_row_strides_t *row_strides,
                          norm_stream_t stream);
norm_status_t norm_bwd_ex(norm_kind_t kind, const void *X, const void *dY, const void *dH,
                          const void *W, const float *mean, const float *rstd, float eps,
                          int64_t M, int64_t N, norm_dtype_t dtype, void *dX, void *dR,
                          void *dW, void *dB, void *workspace, size_t workspace_bytes,
                          const norm_row_strides_t *row_strides, norm_stream_t stream);
norm_status_t norm_bwd_fused_ex(norm_kind_t kind, const void *X, const void *dY, const void *dH,
                                const void *W, const float *mean, const float *rstd, float eps,
                                int64_t M, int64_t N, norm_dtype_t dtype, void *dX, void *dR,
                                void *workspace, size_t workspace_bytes,
                                const norm_row_strides_t *row_strides, norm_stream_t stream);

/*
 * The two stages of norm_bwd, for callers that want them apart (for example to time the
 * fused pass alone, or to reduce the dW/dB partials later). norm_bwd_fused writes dX (and dR)
 * and leaves fp32 column partials in the workspace; norm_bwd_reduce turns those partials into
 * dW (and dB). Both must get the same kind, M, N, dtype, workspace and stream, with nothing
 * writing the workspace in between. Arguments as for norm_bwd.
 */
norm_status_t norm_bwd_fused(norm_kind_t kind, const void *X, const void *dY, const void *dH,
                             const void *W, const float *mean, const float *rstd, float eps,
                             int64_t M, int64_t N, norm_dtype_t dtype, void *dX, void *dR,
                             void *workspace, size_t workspace_bytes, norm_stream_t stream);

norm_status_t norm_bwd_reduce(norm_kind_t kind, int64_t M, int64_t N, norm_dtype_t dtype,
                              void *dW, void *dB, void *workspace, size_t workspace_bytes,
                              norm_stream_t stream);

/*
 * Workspace layout. A call that needs a workspace uses its first 256 bytes as a header of
 * 64-bit words: 0 a magic value, 1 the number of column-partial rows and 2 N (all three written
 * by the backward's fused pass for its column reduction), 3 the exchange-failure word (below).
 * The rest holds fp32 partial sums and, for very long rows, the exchange words of the split
 * scheme's single pass, which carry a tag of the call that wrote them (words of earlier calls,
 * or memory the workspace held before, never pass for this call's). The workspace's contents
 * need no initialisation and are not meaningful to the caller.
 *
 * Workspace bytes for a call, host only (no device needed) [P1 paras. 9-10: the workspace of
 * per-block partial sums of the split reduction]: the largest size the dispatcher's plan for
 * (kind, pass, M, N, dtype, residual) takes on any gfx950 device (1 to 256 compute units, the
 * plan's grid depends on the count) and any pointer alignment, under the current tuning
 * overrides. pass: NORM_PASS_FWD, NORM_PASS_BWD or NORM_PASS_STATS; residual: nonzero when R is
 * given. A workspace of this size, 256-byte aligned, is enough for the call on any gfx950
 * device. Returns SIZE_MAX for arguments no call accepts (kind, dtype or pass unknown, M < 0,
 * N <= 0, N >= 2^31) or a shape no kernel handles. It evaluates the plan for every compute-unit
 * count (about 0.1 ms on the host): size the workspace once per shape.
 */
size_t norm_workspace_bytes(norm_kind_t kind, int pass, int64_t M, int64_t N,
                            norm_dtype_t dtype, int residual);

/*
 * Workspace bytes a call needs on the CURRENT device (the size depends on its compute-unit
 * count), at most norm_workspace_bytes(). pass: NORM_PASS_FWD or NORM_PASS_BWD; residual:
 * nonzero when R is given. Writes the size to *bytes. Returns NORM_ERR_HIP if no device can be
 * queried.
 */
norm_status_t norm_workspace_size(norm_kind_t kind, norm_dtype_t dtype, norm_pass_t pass,
                                  int64_t M, int64_t N, int residual, size_t *bytes);

/*
 * Whether a call on this workspace gave up an exchange wait ([P1] para. 9's workspace reduction,
 * spread over workgroups that wait for each other's partial sums; see norm_fwd). A wait that
 * gives up writes NaN into its rows' outputs and sets the header's exchange-failure word; this
 * query waits for `stream` to finish (it synchronises the host), reads that word, clears it and
 * returns NORM_ERR_EXCHANGE if it was set, else NORM_OK. The word stays set until queried, so one
 * query covers every call on the workspace since the previous query. workspace_bytes below the
 * 256-byte header (including 0) returns NORM_OK: such a workspace belongs to no call that waits.
 * NORM_ERR_WORKSPACE for a NULL or unaligned workspace of 256 bytes or more, NORM_ERR_HIP if a
 * copy or the synchronisation fails. Not for use inside a captured HIP graph.
 */
norm_status_t norm_workspace_status(void *workspace, size_t workspace_bytes,
                                    norm_stream_t stream);

/* Description of the launch plan for a shape, for tests and tuning. */
typedef struct {
  int32_t scheme;         /* norm_scheme_t */
  int32_t access_bytes;   /* bytes per access: 16, 8 or 4, or the element size (element-wise) */
  int32_t elems_per_access;
  int32_t threads;        /* threads per workgroup */
  int32_t team_threads;   /* threads that share one row (64 for the wave scheme) */
  int32_t accesses_per_thread; /* per row (wave/block) or per chunk (split) */
  int32_t rows_per_iter;  /* rows a team holds at once */
  int32_t row_order;      /* wave/block: 0 interleaved row groups, 1 contiguous blocks */
  int64_t grid;           /* workgroups of the main kernel */
  int64_t chunks;         /* split scheme: chunks per row (1 otherwise) */
  int64_t chunk_elems;    /* split scheme: elements per chunk (N otherwise) */
  int64_t row_groups;     /* split backward: row groups sharing a column partial */
  int64_t partials;       /* rows of fp32 column partials in the backward workspace */
  uint64_t workspace_bytes;
  int64_t exchange_row_groups; /* split scheme: row groups of the single-pass exchange form
                                  when it applies (the backward's also needs the saved
                                  statistics), else 0 */
  int32_t phase_classes;  /* wave/block with 16-byte accesses to rows off 16-byte boundaries:
                             the row phase classes (1, 2, 4 or 8), each workgroup taking the
                             rows of one; 0 for aligned rows (NORM_TUNE_UNALIGNED) */
  int32_t reserved;
} norm_plan_t;

/*
 * The plan the dispatcher picks for a shape on a device with cu_count compute units. align is
 * the largest power of two, up to 16, that divides the address of every tensor of the call
 * (16 for buffers straight from an allocator; values above 16 count as 16; 0 or 1 when
 * unknown). Rows are taken as contiguous, so a row starts N elements after the previous one,
 * and below 16 the tensors' phases as unknown (a call whose tensors share one phase can take
 * 16-byte accesses over row phase classes where this plan shows narrower ones). Pure host
 * logic: needs no GPU.
 */
norm_status_t norm_plan(norm_kind_t kind, norm_dtype_t dtype, norm_pass_t pass, int64_t M,
                        int64_t N, int residual, int align, int cu_count, norm_plan_t *out);

/* Tuning overrides (process-wide; for tests and offline tuning; not thread-safe with
 * concurrent calls). Value -1 restores the default. */
typedef enum {
  NORM_TUNE_SCHEME = 0,         /* norm_scheme_t to force */
  NORM_TUNE_GRID_PER_CU = 1,    /* workgroups per compute unit for persistent kernels */
  NORM_TUNE_ROWS_PER_ITER = 2,  /* rows a team holds at once: 1, 2 or 4 */
  NORM_TUNE_TEAM_THREADS = 3,   /* threads per row team (multiple of 64); ignored where a team
                                   of that size cannot hold the row */
  NORM_TUNE_SPLIT_CHUNK = 4,    /* split scheme: elements per chunk */
  NORM_TUNE_ROW_GROUPS = 5,     /* split backward: number of row groups (the single-pass form
                                   takes at most this many, and never more than fit) */
  NORM_TUNE_TEAMS_PER_WG = 6,   /* block scheme: row teams per workgroup (their dW/dB partials
                                   are merged in LDS, so fewer partial rows are written) */
  NORM_TUNE_ROW_ORDER = 7,      /* wave/block schemes: 0 = row groups interleaved across the
                                   workgroups, 1 = each workgroup takes a contiguous block */
  NORM_TUNE_SPLIT_EXCHANGE = 8, /* split scheme: 1 = the single-pass exchange form wherever it
                                   applies, 0 = always the two-pass form, -1 (default) = the
                                   single-pass form where it applies and a row gathers at
                                   most 512 chunk partials forward, 640 backward (LayerNorm
                                   three per chunk, RMSNorm one) */
  NORM_TUNE_EXCHANGE_POLLS = 9, /* single-pass split form: polls of a row's exchange words
                                   before a workgroup gives up on the row and writes NaN for
                                   it and for its later rows (1 .. 2^24; default 2^19, about a
                                   second) */
  NORM_TUNE_EXCHANGE_WITHHOLD = 10, /* for tests of that bounded wait only: 1 = chunk 0 never
                                       publishes its partials, so every row gives up */
  NORM_TUNE_UNALIGNED = 11,     /* wave/block schemes, rows off 16-byte boundaries (their
                                   length, stride or start) with every [M, N] tensor at one
                                   phase: -1 (default) or 1, 16-byte accesses over row phase
                                   classes in place of 8-byte, 4-byte and element-wise ones;
                                   0 never */
  NORM_TUNE_ATTN_KEY_PASS = 12  /* norm_attention_fwd with a large enough workspace: 1 = the
                                   key pass always, 0 = never (the key norm deferred into the
                                   attention kernel), -1 (default) = when each key is read by
                                   at least 8 (query block, query head) pairs */
} norm_tune_t;

norm_status_t norm_set_tuning(norm_tune_t key, int64_t value);

/*
 * A norm whose output feeds a linear projection, with the normalisation deferred past the
 * matrix product ([P3] "Towards Free Normalization: Fusing Normalization into GEMM and
 * Attention Kernels", items 3-4 and 9-10; the page names "Lazy Pre-Norm" without giving its
 * algebra, so the form below is this library's reading). For X [M, K], the norm's gamma and
 * beta [K], a projection L [Nout, K] (row j gives output column j) and its bias c [Nout]:
 *     out = Norm(X) L^T + c
 *         = rstd * (X G^T - mean * s) + t          (row-wise rstd and mean, column-wise s, t)
 * with G = L * gamma (gamma folded into each row of L, rounded once to bf16), s[j] = sum_k
 * G[j,k] and t[j] = sum_k beta[k] L[j,k] + c[j]. The product then reads the raw X: it tiles
 * both of its dimensions freely, and the per-row statistics enter only its epilogue (the tiling
 * conflict between a row-wise norm and a 2-D tiled product that the page's item 9 describes).
 * RMSNorm has no mean and no beta: out = rstd * (X G^T) + t.
 *
 * norm_fold_projection: G, s and t from L, gamma, beta and c, once per projection weight.
 *   dtype   NORM_BF16 (gamma, beta bf16) or NORM_BF16_F32W (gamma, beta fp32); L and G bf16.
 *   L       [Nout, K] row stride ldl (elements); gamma [K]; beta [K] or NULL (LayerNorm only);
 *           c [Nout] fp32 or NULL.
 *   G       [Nout, K] bf16 out, row stride ldg: G[j,k] = bf16(L[j,k] * gamma[k]) (the fp32
 *           product, rounded to nearest even).
 *   s       [Nout] fp32 out, the sums of G's rows as stored (LayerNorm: required; RMSNorm:
 *           NULL or ignored).
 *   t       [Nout] fp32 out, or NULL when there is neither beta nor c.
 *   One workgroup per row of G; the sums are formed in a fixed order (the same bits on every
 *   call). G must not overlap L.
 *
 * norm_lazy_linear: Y = out above, rounded once to bf16.
 *   X       [M, K] bf16, row stride ldx; G [Nout, K] bf16, row stride ldg (from the fold).
 *   s, t    from the fold (t may be NULL: zero).
 *   Statistics: with rstd_in given, mean_in (LayerNorm) and rstd_in [M] fp32 are used as they
 *           are (for example from norm_stats or a forward). With rstd_in NULL the product
 *           forms them itself from the X tiles it reads anyway, in fp32 (sums shifted by the
 *           row's first element; var = E[(x-x0)^2] - E[x-x0]^2, clamped at 0; rstd =
 *           1/sqrt(var + eps)) and, when mean_out / rstd_out are given, stores them [M] fp32.
 *   Y       [M, Nout] bf16 out, row stride ldy.
 *   Requirements: K a multiple of 8; ldx and ldg multiples of 8 and below 2^23 (rows of a
 *   256-row tile are addressed by 32-bit byte offsets); X and G 16-byte aligned (the product
 *   reads 16-byte chunks of 8 values); ldy >= Nout. Otherwise NORM_ERR_UNSUPPORTED (layout)
 *   or NORM_ERR_INVALID_ARG (sizes, NULL pointers, eps). M == 0: NORM_OK once the sizes and
 *   eps pass, nothing launched and no pointer read. Y must not overlap X, G, s, t or the
 *   statistics.
 *   The product runs on the matrix cores (bf16 inputs, fp32 accumulation) in 256 x 256 output
 *   tiles; Y is written four columns (8 bytes) at a time where Y is 8-byte aligned and ldy a
 *   multiple of 4, else one value at a time.
 */
norm_status_t norm_fold_projection(norm_kind_t kind, norm_dtype_t dtype, const void *L,
                                   int64_t ldl, const void *gamma, const void *beta,
                                   const float *c, int64_t Nout, int64_t K, void *G, int64_t ldg,
                                   float *s, float *t, norm_stream_t stream);
norm_status_t norm_lazy_linear(norm_kind_t kind, const void *X, int64_t ldx, int64_t M,
                               int64_t K, float eps, const void *G, int64_t ldg, int64_t Nout,
                               const float *s, const float *t, const float *mean_in,
                               const float *rstd_in, float *mean_out, float *rstd_out, void *Y,
                               int64_t ldy, norm_stream_t stream);

/*
 * Attention over normalised queries and keys, in one kernel (web page "Towards Free
 * Normalization: Fusing Normalization into GEMM and Attention Kernels", item 5: several norms
 * fused around an attention kernel; the page gives no formulas, so the form below is this
 * library's reading, QK-norm). Per batch b and query head h, with g = Hq / Hk query heads per
 * key/value head (head h reads key/value head h / g):
 *     q'_i = Norm_q(Q[b, i, h, :]),   k'_j = Norm_k(K[b, j, h / g, :])
 *     O[b, i, h, :] = sum_j softmax_j(scale * q'_i . k'_j) V[b, j, h / g, :]
 *     lse[b, h, i]  = ln sum_j exp(scale * q'_i . k'_j)
 * over the keys j visible to query i: all S, or j <= i with NORM_ATTN_CAUSAL. Norm_q and Norm_k
 * are the row norm of `kind` along the head dimension D (LayerNorm: (x - mean) * rstd * gamma
 * + beta; RMSNorm: x * rstd * gamma; rstd = 1 / sqrt(var or mean square + eps)), with gamma
 * wq, wk and beta bq, bk of D entries shared by all heads. With NORM_ATTN_NO_NORM the queries
 * and keys are used as given (kind is ignored; the four vectors must be NULL): the attention
 * half of the same computation done in two passes.
 *   Q       [B, S, Hq, D] bf16: element (b, s, h, d) at (b * S + s) * ldq + h * D + d.
 *   K, V    [B, S, Hk, D] bf16 with token strides ldk, ldv.
 *   wq, wk  [D] bf16 gammas; bq, bk [D] bf16 betas or NULL (zero; LayerNorm only).
 *   eps     added inside the square root, >= 0 and finite. scale > 0 and finite (usually
 *           1 / sqrt(D)).
 *   O       [B, S, Hq, D] bf16 out, token stride ldo; must not overlap any input.
 *   lse     [B, Hq, S] fp32 out, or NULL.
 *   workspace  device memory the call may use, or NULL (then workspace_bytes must be 0); it
 *           must not overlap any argument. Each key vector is read by every query block of
 *           every query head of its group. When that is at least 8 (query block, head) pairs
 *           and workspace_bytes >= norm_attention_workspace_bytes(B, S, Hk, D), the keys are
 *           normalised once, by a pass of their own into the workspace, and the attention
 *           kernel reads them from there; the queries are always normalised inside the
 *           attention kernel, which never stores them. Otherwise the key norm is deferred into
 *           the attention kernel: the key gamma is folded into each query, the keys are
 *           staged as given (LayerNorm: centred) and each key's rstd scales its scores.
 *   Numerics: scores and O accumulate in fp32 on the matrix cores, the softmax weights enter
 *   the second product as bf16, O is rounded once to bf16 (nearest even). With the key pass
 *   the normalised queries and keys are each rounded once to bf16 (as two separate norm passes
 *   would store them); with the deferred key norm the normalised queries times the key gamma
 *   are rounded once to bf16 and the keys enter the product exactly (LayerNorm: centred,
 *   rounded once to bf16).
 *   Requirements: D == 128; ldq, ldk, ldv, ldo multiples of 8 and at least Hq * D (Hk * D for
 *   K and V); ldk and ldv below 2^24; Q, K, V, O, the norm vectors and the workspace 16-byte aligned. Otherwise NORM_ERR_UNSUPPORTED
 *   (head size, alignment) or NORM_ERR_INVALID_ARG (sizes, Hq not a multiple of Hk, NULL
 *   pointers, eps, scale, flags, overlaps). B == 0 or S == 0: NORM_OK once the rest passes,
 *   nothing launched and no pointer read. The call allocates nothing.
 */
#define NORM_ATTN_CAUSAL 1u
#define NORM_ATTN_NO_NORM 2u
norm_status_t norm_attention_fwd(norm_kind_t kind, uint32_t flags, int64_t B, int64_t S,
                                 int64_t Hq, int64_t Hk, int64_t D, const void *Q, int64_t ldq,
                                 const void *K, int64_t ldk, const void *V, int64_t ldv,
                                 const void *wq, const void *bq, const void *wk, const void *bk,
                                 float eps, float scale, void *O, int64_t ldo, float *lse,
                                 void *workspace, size_t workspace_bytes,
                                 norm_stream_t stream);
/* Workspace bytes for norm_attention_fwd's key pass: B * S * Hk * D * 2 (0 for sizes it does
 * not address). Host only. */
size_t norm_attention_workspace_bytes(int64_t B, int64_t S, int64_t Hk, int64_t D);

/*
 * Kernel timing for profilers and benchmarks. Arms two HIP events (hipEvent_t, created by the
 * caller on the device of the stream that will be used) for the calling thread's next call of
 * norm_fwd, norm_bwd, norm_bwd_fused, norm_bwd_reduce or norm_attention_fwd: `start_event` takes the start
 * timestamp of the first kernel that call launches and `stop_event` the end timestamp of its
 * last one (hipExtLaunchKernel; no extra packets are queued, so the stream runs as it would
 * without timing). hipEventElapsedTime of the pair is then the GPU time of that call's kernels.
 * The events are disarmed when that call returns, whatever its status; a call that launches no
 * kernel leaves them unrecorded. Both NULL disarms; exactly one NULL is NORM_ERR_INVALID_ARG
 * (and disarms). The library does not own the events.
 */
norm_status_t norm_set_launch_events(void *start_event, void *stop_event);

/* Static text for a status code. */
const char *norm_status_string(norm_status_t status);

/* Library version, major * 10000 + minor * 100 + patch. */
int norm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DLN_NORM_H */
