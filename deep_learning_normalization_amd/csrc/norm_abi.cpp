// norm_abi.cpp -- the extern "C" entry points declared in include/norm.h.
//
// Each call: check arguments (no device access), find the current device's compute-unit count
// (cached), build the launch plan, check the workspace, queue the kernels on the caller's
// stream. Nothing here allocates or synchronises.
#include <atomic>
#include <cstdint>
#include <new>

#include "norm_internal.hpp"
#include "norm_attn.hpp"
#include "norm_lazy.hpp"

namespace {

thread_local dln::LaunchEvents tl_events{nullptr, nullptr};

// Disarms the timing events when an entry point returns.
struct EventsDisarm {
  ~EventsDisarm() { tl_events = dln::LaunchEvents{nullptr, nullptr}; }
};

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

norm_status_t current_cu_count(int *cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return NORM_ERR_HIP;
  if (dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) {
      *cu = cached;
      return NORM_OK;
    }
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    return NORM_ERR_HIP;
  if (dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
  *cu = n;
  return NORM_OK;
}

float *ws_region(void *ws, size_t off) {
  return reinterpret_cast<float *>(static_cast<char *>(ws) + off);
}

// 64-bit word i of the workspace header
uint64_t *header_word(void *ws, int i) { return static_cast<uint64_t *>(ws) + i; }

norm_status_t ws_ok(const dln::Plan &p, const void *ws, size_t ws_bytes) {
  if (p.ws_bytes == 0) return NORM_OK;
  if (!ws || ws_bytes < p.ws_bytes || ((uintptr_t)ws & 15u)) return NORM_ERR_WORKSPACE;
  return NORM_OK;
}

// Row strides of one call in elements, each resolved (0 or no struct: N, contiguous rows).
struct Strides {
  int64_t x, r, y, h, dy, dh, dx, dr;
};

Strides resolve(const norm_row_strides_t *ld, int64_t N) {
  auto pick = [N](int64_t v) { return v ? v : N; };
  if (!ld) return Strides{N, N, N, N, N, N, N, N};
  return Strides{pick(ld->x),  pick(ld->r),  pick(ld->y),  pick(ld->h),
                 pick(ld->dy), pick(ld->dh), pick(ld->dx), pick(ld->dr)};
}

norm_status_t fwd_launch(norm_kind_t kind, const void *X, const void *R, const void *W,
                         const void *B, float eps, int64_t M, int64_t N, norm_dtype_t dtype,
                         void *Y, void *H, float *mean, float *rstd, void *workspace,
                         size_t workspace_bytes, const Strides &ld, norm_pass_t pass,
                         norm_stream_t stream);

// Plan, workspace check and argument block of the backward's fused pass.
norm_status_t bwd_setup(norm_kind_t kind, const void *X, const void *dY, const void *dH,
                        const void *W, const float *mean, const float *rstd, float eps,
                        int64_t M, int64_t N, norm_dtype_t dtype, void *dX, void *dR,
                        void *workspace, size_t workspace_bytes, const Strides &ld,
                        dln::Plan *plan, dln::BwdArgs *a) {
  int cu = 0;
  norm_status_t st = current_cu_count(&cu);
  if (st != NORM_OK) return st;
  const void *ptrs[] = {X, dY, dH, W, dX, dR};
  const int64_t lds[] = {ld.x, ld.dy, dH ? ld.dh : N, ld.dx, dR ? ld.dr : N};
  const int align = dln::fold_stride_align(dln::common_align(ptrs, 6), lds, 5,
                                           dln::act_elem_size(dtype));
  const void *acts[] = {X, dY, dH, dX, dR};
  int phase0 = -1, dphase = -1;
  dln::common_phase(acts, lds, 5, dln::act_elem_size(dtype), &phase0, &dphase);
  st = dln::make_plan(kind, dtype, NORM_PASS_BWD, M, N, 0, align, phase0, dphase, cu,
                      dln::tuning(), plan);
  if (st != NORM_OK) return st;
  st = ws_ok(*plan, workspace, workspace_bytes);
  if (st != NORM_OK) return st;
  dln::BwdArgs b{};
  b.x = X;
  b.dy = dY;
  b.dh = dH;
  b.w = W;
  b.mean = kind == NORM_LAYERNORM ? mean : nullptr;
  b.rstd = rstd;
  b.dx = dX;
  b.dr = (dR == dX) ? nullptr : dR;
  b.dw = nullptr;
  b.db = nullptr;
  b.colpart = ws_region(workspace, plan->off_colpart);
  b.header = reinterpret_cast<int64_t *>(static_cast<char *>(workspace) + plan->off_header);
  b.rowpart = plan->scheme == NORM_SCHEME_SPLIT ? ws_region(workspace, plan->off_rowpart) : nullptr;
  b.stats = plan->scheme == NORM_SCHEME_SPLIT ? ws_region(workspace, plan->off_stats) : nullptr;
  // the split scheme's single-pass exchange form needs the forward's statistics
  const bool xchg = plan->xchg && rstd && (kind != NORM_LAYERNORM || mean) &&
                    dln::xsplit_ready(dtype, kind == NORM_LAYERNORM, true);
  b.xpart = xchg ? reinterpret_cast<uint64_t *>(static_cast<char *>(workspace) + plan->off_xpart)
                 : nullptr;
  b.xerr = xchg ? header_word(workspace, dln::kWsErrWord) : nullptr;
  b.tag = xchg ? dln::next_exchange_tag() : 0u;
  b.polls = (uint32_t)(dln::tuning().xchg_polls > 0 ? dln::tuning().xchg_polls
                                                     : dln::kXchgPollsDefault);
  b.withhold = dln::tuning().xchg_withhold == 1 ? 1 : 0;
  b.ldx = ld.x;
  b.lddy = ld.dy;
  b.lddh = ld.dh;
  b.lddx = ld.dx;
  b.lddr = ld.dr;
  b.M = M;
  b.N = (int32_t)N;
  b.nacc = (int32_t)plan->nacc;
  b.period = plan->period;
  b.phase0 = phase0 < 0 ? 0 : phase0;
  b.dphase = dphase < 0 ? 0 : dphase;
  b.chunks = plan->chunks;
  b.chunk_acc = (int32_t)(plan->chunk_elems / plan->epv);
  b.partials = plan->partials;
  b.row_groups = xchg ? plan->xrow_groups : plan->row_groups;
  b.rows_per_group = plan->rows_per_group;
  b.layernorm = kind == NORM_LAYERNORM ? 1 : 0;
  b.want_db = 1;
  b.blocked = plan->row_order;
  b.eps = eps;
  b.inv_n = 1.0f / (float)N;
  *a = b;
  return NORM_OK;
}

norm_status_t run_fused(const dln::Plan &p, norm_dtype_t dtype, const dln::BwdArgs &a,
                        hipStream_t s) {
  if (p.scheme == NORM_SCHEME_SPLIT)
    return a.xpart ? dln::launch_xsplit_bwd(dtype, a, s) : dln::launch_split_bwd(p, dtype, a, s);
  if (p.scheme == NORM_SCHEME_LOOP) return dln::launch_looped_bwd(p, dtype, a, s);
  return dln::launch_team_bwd(p, dtype, a, s);
}

// Column reduction of the partials a fused pass left in `workspace` (its header says how many).
norm_status_t run_reduce(norm_dtype_t dtype, int64_t N, void *dW, void *dB, void *workspace,
                         size_t workspace_bytes, hipStream_t s) {
  const size_t row_pair = (size_t)2 * (size_t)N * 4;
  if (!workspace || ((uintptr_t)workspace & 15u) ||
      workspace_bytes < dln::kWsHeaderBytes + row_pair)
    return NORM_ERR_WORKSPACE;
  dln::ReduceArgs r{};
  r.header = static_cast<const int64_t *>(workspace);
  r.colpart = ws_region(workspace, dln::kWsHeaderBytes);
  r.dw = dW;
  r.db = dB;
  r.max_partials = (int64_t)((workspace_bytes - dln::kWsHeaderBytes) / row_pair);
  r.N = (int32_t)N;
  return dln::launch_reduce(dtype, r, s);
}

norm_status_t zero_outputs(int64_t N, norm_dtype_t dtype, void *dW, void *dB, hipStream_t s) {
  const size_t n = (size_t)N * ((dtype == NORM_BF16 || dtype == NORM_F16) ? 2 : 4); // dW, dB
  norm_status_t st = dln::launch_zero(dW, n, s);
  if (st == NORM_OK && dB) st = dln::launch_zero(dB, n, s);
  return st;
}

} // namespace

dln::LaunchEvents &dln::launch_events() { return tl_events; }

extern "C" {

norm_status_t norm_fwd(norm_kind_t kind, const void *X, const void *R, const void *W,
                       const void *B, float eps, int64_t M, int64_t N, norm_dtype_t dtype,
                       void *Y, void *H, float *mean, float *rstd, void *workspace,
                       size_t workspace_bytes, norm_stream_t stream) {
  return norm_fwd_ex(kind, X, R, W, B, eps, M, N, dtype, Y, H, mean, rstd, workspace,
                     workspace_bytes, nullptr, stream);
}

norm_status_t norm_fwd_ex(norm_kind_t kind, const void *X, const void *R, const void *W,
                          const void *B, float eps, int64_t M, int64_t N, norm_dtype_t dtype,
                          void *Y, void *H, float *mean, float *rstd, void *workspace,
                          size_t workspace_bytes, const norm_row_strides_t *row_strides,
                          norm_stream_t stream) {
  const EventsDisarm disarm;
  if (N <= 0) return NORM_ERR_INVALID_ARG;
  const Strides ld = resolve(row_strides, N);
  dln::FwdCheck c{kind, dtype, X, R, W, B, eps, M, N, Y, H, mean, rstd, workspace,
                  workspace_bytes, ld.x, ld.r, ld.y, ld.h, 0};
  norm_status_t st = dln::check_fwd(c);
  if (st != NORM_OK || M == 0) return st;
  return fwd_launch(kind, X, R, W, B, eps, M, N, dtype, Y, H, mean, rstd, workspace,
                    workspace_bytes, ld, NORM_PASS_FWD, stream);
}

norm_status_t norm_stats(norm_kind_t kind, const void *X, const void *R, float eps, int64_t M,
                         int64_t N, norm_dtype_t dtype, void *H, float *mean, float *rstd,
                         void *workspace, size_t workspace_bytes,
                         const norm_row_strides_t *row_strides, norm_stream_t stream) {
  const EventsDisarm disarm;
  if (N <= 0) return NORM_ERR_INVALID_ARG;
  const Strides ld = resolve(row_strides, N);
  dln::FwdCheck c{kind, dtype, X, R, nullptr, nullptr, eps, M, N, nullptr, H, mean, rstd,
                  workspace, workspace_bytes, ld.x, ld.r, ld.y, ld.h, 1};
  norm_status_t st = dln::check_fwd(c);
  if (st != NORM_OK || M == 0) return st;
  return fwd_launch(kind, X, R, nullptr, nullptr, eps, M, N, dtype, nullptr, H, mean, rstd,
                    workspace, workspace_bytes, ld, NORM_PASS_STATS, stream);
}

norm_status_t norm_fold_projection(norm_kind_t kind, norm_dtype_t dtype, const void *L,
                                   int64_t ldl, const void *gamma, const void *beta,
                                   const float *c, int64_t Nout, int64_t K, void *G, int64_t ldg,
                                   float *s, float *t, norm_stream_t stream) {
  const EventsDisarm disarm;
  const dln::FoldCheck fc{kind, dtype, L, gamma, beta, c, Nout, K, ldl, ldg, G, s, t};
  const norm_status_t st = dln::check_fold(fc);
  if (st != NORM_OK) return st;
  dln::FoldArgs a{};
  a.l = static_cast<const uint16_t *>(L);
  a.gamma = gamma;
  a.beta = beta;
  a.c = c;
  a.g = static_cast<uint16_t *>(G);
  a.s = kind == NORM_LAYERNORM ? s : nullptr;
  a.t = t;
  a.K = K;
  a.ldl = ldl;
  a.ldg = ldg;
  return dln::launch_fold_projection(dtype == NORM_BF16_F32W, a, Nout,
                                     static_cast<hipStream_t>(stream));
}

norm_status_t norm_lazy_linear(norm_kind_t kind, const void *X, int64_t ldx, int64_t M,
                               int64_t K, float eps, const void *G, int64_t ldg, int64_t Nout,
                               const float *s, const float *t, const float *mean_in,
                               const float *rstd_in, float *mean_out, float *rstd_out, void *Y,
                               int64_t ldy, norm_stream_t stream) {
  const EventsDisarm disarm;
  const dln::LazyCheck lc{kind, X, ldx, M, K, eps, G, ldg, Nout, s, t, mean_in, rstd_in,
                          mean_out, rstd_out, Y, ldy};
  const norm_status_t st = dln::check_lazy(lc);
  if (st != NORM_OK || M == 0) return st;
  dln::LazyArgs a{};
  a.x = static_cast<const uint16_t *>(X);
  a.g = static_cast<const uint16_t *>(G);
  a.s = s;
  a.t = t;
  a.mean_in = mean_in;
  a.rstd_in = rstd_in;
  a.mean_out = mean_out;
  a.rstd_out = rstd_out;
  a.y = static_cast<uint16_t *>(Y);
  a.M = M;
  a.N = Nout;
  a.K = K;
  a.ldx = ldx;
  a.ldg = ldg;
  a.ldy = ldy;
  const int64_t tm = (M + dln::kLazyTile - 1) / dln::kLazyTile;
  const int64_t tn = (Nout + dln::kLazyTile - 1) / dln::kLazyTile;
  if (tm > 0x7fffffff || tn > 0x7fffffff) return NORM_ERR_UNSUPPORTED;
  a.tiles_m = (int32_t)tm;
  a.tiles_n = (int32_t)tn;
  a.eps = eps;
  a.inv_k = 1.0f / (float)K;
  a.vec_store = ((uintptr_t)Y % 8 == 0 && ldy % 4 == 0) ? 1 : 0;
  return dln::launch_lazy_linear(kind == NORM_LAYERNORM, a, static_cast<hipStream_t>(stream));
}

norm_status_t norm_attention_fwd(norm_kind_t kind, uint32_t flags, int64_t B, int64_t S,
                                 int64_t Hq, int64_t Hk, int64_t D, const void *Q, int64_t ldq,
                                 const void *K, int64_t ldk, const void *V, int64_t ldv,
                                 const void *wq, const void *bq, const void *wk, const void *bk,
                                 float eps, float scale, void *O, int64_t ldo, float *lse,
                                 void *workspace, size_t workspace_bytes,
                                 norm_stream_t stream) {
  const EventsDisarm disarm;
  const dln::AttnCheck ac{kind, flags, B, S, Hq, Hk, D, Q, K, V, ldq, ldk, ldv,
                          wq, bq, wk, bk, eps, scale, O, ldo, lse, workspace, workspace_bytes};
  const norm_status_t st = dln::check_attention(ac);
  if (st != NORM_OK || B == 0 || S == 0) return st;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  dln::AttnArgs a{};
  a.q = static_cast<const uint16_t *>(Q);
  a.k = static_cast<const uint16_t *>(K);
  a.v = static_cast<const uint16_t *>(V);
  a.wq = static_cast<const uint16_t *>(wq);
  a.bq = static_cast<const uint16_t *>(bq);
  a.wk = static_cast<const uint16_t *>(wk);
  a.bk = static_cast<const uint16_t *>(bk);
  a.o = static_cast<uint16_t *>(O);
  a.lse = lse;
  a.ldq = ldq;
  a.ldk = ldk;
  a.ldv = ldv;
  a.ldo = ldo;
  a.B = (int32_t)B;
  a.S = (int32_t)S;
  a.Hq = (int32_t)Hq;
  a.Hk = (int32_t)Hk;
  a.qblocks = (int32_t)((S + dln::kAttnBQ - 1) / dln::kAttnBQ);
  a.eps = eps;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  const int norm = (flags & NORM_ATTN_NO_NORM) ? dln::ATTN_NO_NORM
                   : kind == NORM_LAYERNORM    ? dln::ATTN_LAYERNORM
                                               : dln::ATTN_RMSNORM;
  // keys read by many (query block, query head) pairs: normalise them once, into the
  // workspace, instead of in every query block
  const size_t kbytes = dln::attention_workspace_bytes(B, S, Hk, D);
  const int force = dln::tuning().attn_key_pass;
  const bool key_pass = norm != dln::ATTN_NO_NORM && workspace && kbytes &&
                        workspace_bytes >= kbytes && force != 0 &&
                        (force == 1 || (int64_t)a.qblocks * (Hq / Hk) >= dln::kAttnKeyPassReuse);
  if (key_pass) {
    dln::KnormArgs ka{};
    ka.k = a.k;
    ka.wk = a.wk;
    ka.bk = a.bk;
    ka.out = static_cast<uint16_t *>(workspace);
    ka.nkeys = B * S * Hk;
    ka.ldk = ldk;
    ka.Hk = (int32_t)Hk;
    ka.eps = eps;
    const norm_status_t ks = dln::launch_key_norm(norm == dln::ATTN_LAYERNORM, ka, hs);
    if (ks != NORM_OK) return ks;
    a.k = ka.out;
    a.ldk = Hk * D;
  }
  return dln::launch_attention(norm, key_pass, (flags & NORM_ATTN_CAUSAL) != 0, a, hs);
}

size_t norm_attention_workspace_bytes(int64_t B, int64_t S, int64_t Hk, int64_t D) {
  return dln::attention_workspace_bytes(B, S, Hk, D);
}

} // extern "C"

namespace {

// Plan and queue a checked forward (Y and W NULL: the statistics pass alone).
norm_status_t fwd_launch(norm_kind_t kind, const void *X, const void *R, const void *W,
                         const void *B, float eps, int64_t M, int64_t N, norm_dtype_t dtype,
                         void *Y, void *H, float *mean, float *rstd, void *workspace,
                         size_t workspace_bytes, const Strides &ld, norm_pass_t pass,
                         norm_stream_t stream) {
  norm_status_t st;
  int cu = 0;
  st = current_cu_count(&cu);
  if (st != NORM_OK) return st;
  const void *ptrs[] = {X, R, W, B, Y, H};
  const int64_t lds[] = {ld.x, R ? ld.r : N, ld.y, H ? ld.h : N};
  const int align = dln::fold_stride_align(dln::common_align(ptrs, 6), lds, 4,
                                           dln::act_elem_size(dtype));
  const void *acts[] = {X, R, Y, H};
  int phase0 = -1, dphase = -1;
  dln::common_phase(acts, lds, 4, dln::act_elem_size(dtype), &phase0, &dphase);
  dln::Plan p;
  st = dln::make_plan(kind, dtype, pass, M, N, R != nullptr, align, phase0, dphase, cu,
                      dln::tuning(), &p);
  if (st != NORM_OK) return st;
  st = ws_ok(p, workspace, workspace_bytes);
  if (st != NORM_OK) return st;
  dln::FwdArgs a{};
  a.x = X;
  a.r = R;
  a.w = W;
  a.b = kind == NORM_LAYERNORM ? B : nullptr;
  a.y = Y;
  a.h = H;
  a.mean = kind == NORM_LAYERNORM ? mean : nullptr;
  a.rstd = rstd;
  a.rowpart = p.scheme == NORM_SCHEME_SPLIT ? ws_region(workspace, p.off_rowpart) : nullptr;
  a.ldx = ld.x;
  a.ldr = ld.r;
  a.ldy = ld.y;
  a.ldh = ld.h;
  a.M = M;
  a.N = (int32_t)N;
  a.nacc = (int32_t)p.nacc;
  a.period = p.period;
  a.phase0 = phase0 < 0 ? 0 : phase0;
  a.dphase = dphase < 0 ? 0 : dphase;
  a.chunks = p.chunks;
  a.chunk_acc = (int32_t)(p.chunk_elems / p.epv);
  a.layernorm = kind == NORM_LAYERNORM ? 1 : 0;
  a.blocked = p.row_order;
  a.eps = eps;
  a.inv_n = 1.0f / (float)N;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.scheme == NORM_SCHEME_SPLIT) {
    // the single-pass exchange form where the plan allows it and Y is written
    if (p.xchg && Y && !R && dln::xsplit_ready(dtype, kind == NORM_LAYERNORM, false)) {
      a.xpart = reinterpret_cast<uint64_t *>(static_cast<char *>(workspace) + p.off_xpart);
      a.xerr = header_word(workspace, dln::kWsErrWord);
      a.tag = dln::next_exchange_tag();
      a.xgroups = p.xrow_groups;
      a.polls = (uint32_t)(dln::tuning().xchg_polls > 0 ? dln::tuning().xchg_polls
                                                         : dln::kXchgPollsDefault);
      a.withhold = dln::tuning().xchg_withhold == 1 ? 1 : 0;
      return dln::launch_xsplit_fwd(p, dtype, a, s);
    }
    return dln::launch_split_fwd(p, dtype, a, s);
  }
  return dln::launch_team_fwd(p, dtype, a, s);
}

} // namespace

extern "C" {

norm_status_t norm_bwd(norm_kind_t kind, const void *X, const void *dY, const void *dH,
                       const void *W, const float *mean, const float *rstd, float eps,
                       int64_t M, int64_t N, norm_dtype_t dtype, void *dX, void *dR, void *dW,
                       void *dB, void *workspace, size_t workspace_bytes, norm_stream_t stream) {
  return norm_bwd_ex(kind, X, dY, dH, W, mean, rstd, eps, M, N, dtype, dX, dR, dW, dB,
                     workspace, workspace_bytes, nullptr, stream);
}

norm_status_t norm_bwd_ex(norm_kind_t kind, const void *X, const void *dY, const void *dH,
                          const void *W, const float *mean, const float *rstd, float eps,
                          int64_t M, int64_t N, norm_dtype_t dtype, void *dX, void *dR,
                          void *dW, void *dB, void *workspace, size_t workspace_bytes,
                          const norm_row_strides_t *row_strides, norm_stream_t stream) {
  const EventsDisarm disarm;
  if (N <= 0) return NORM_ERR_INVALID_ARG;
  const Strides ld = resolve(row_strides, N);
  dln::BwdCheck c{kind,   dtype, X,  dY, dH,    W,     mean,     rstd,  eps,
                  M,      N,     dX, dR, dW,    dB,    workspace, workspace_bytes,
                  1,      1,     ld.x, ld.dy, ld.dh, ld.dx, ld.dr};
  norm_status_t st = dln::check_bwd(c);
  if (st != NORM_OK) return st;
  if (kind == NORM_RMSNORM) dB = nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M == 0) return zero_outputs(N, dtype, dW, dB, s); // empty column sums
  dln::Plan p;
  dln::BwdArgs a;
  st = bwd_setup(kind, X, dY, dH, W, mean, rstd, eps, M, N, dtype, dX, dR, workspace,
                 workspace_bytes, ld, &p, &a);
  if (st != NORM_OK) return st;
  // the split scheme with a single row group writes dW/dB itself, with no reduction pass
  // (its vector stores of dW and dB need the alignment of the weight loads of its width)
  const void *outs[] = {dW, dB};
  const bool direct = p.scheme == NORM_SCHEME_SPLIT && a.row_groups == 1 &&
                      (size_t)dln::common_align(outs, 2) >= dln::weight_align_need(dtype, p.epv);
  if (direct) {
    a.dw = dW;
    a.db = dB;
  }
  st = run_fused(p, dtype, a, s);
  if (st != NORM_OK || direct) return st;
  return run_reduce(dtype, N, dW, dB, workspace, workspace_bytes, s);
}

norm_status_t norm_bwd_fused(norm_kind_t kind, const void *X, const void *dY, const void *dH,
                             const void *W, const float *mean, const float *rstd, float eps,
                             int64_t M, int64_t N, norm_dtype_t dtype, void *dX, void *dR,
                             void *workspace, size_t workspace_bytes, norm_stream_t stream) {
  return norm_bwd_fused_ex(kind, X, dY, dH, W, mean, rstd, eps, M, N, dtype, dX, dR, workspace,
                           workspace_bytes, nullptr, stream);
}

norm_status_t norm_bwd_fused_ex(norm_kind_t kind, const void *X, const void *dY, const void *dH,
                                const void *W, const float *mean, const float *rstd, float eps,
                                int64_t M, int64_t N, norm_dtype_t dtype, void *dX, void *dR,
                                void *workspace, size_t workspace_bytes,
                                const norm_row_strides_t *row_strides, norm_stream_t stream) {
  const EventsDisarm disarm;
  if (N <= 0) return NORM_ERR_INVALID_ARG;
  const Strides ld = resolve(row_strides, N);
  dln::BwdCheck c{kind,   dtype, X,       dY,      dH,    W,     mean,      rstd,
                  eps,    M,     N,       dX,      dR,    nullptr, nullptr, workspace,
                  workspace_bytes, 1, 0,  ld.x,    ld.dy, ld.dh, ld.dx,     ld.dr};
  norm_status_t st = dln::check_bwd(c);
  if (st != NORM_OK || M == 0) return st;
  dln::Plan p;
  dln::BwdArgs a;
  st = bwd_setup(kind, X, dY, dH, W, mean, rstd, eps, M, N, dtype, dX, dR, workspace,
                 workspace_bytes, ld, &p, &a);
  if (st != NORM_OK) return st;
  return run_fused(p, dtype, a, static_cast<hipStream_t>(stream));
}

norm_status_t norm_bwd_reduce(norm_kind_t kind, int64_t M, int64_t N, norm_dtype_t dtype,
                              void *dW, void *dB, void *workspace, size_t workspace_bytes,
                              norm_stream_t stream) {
  const EventsDisarm disarm;
  dln::BwdCheck c{kind, dtype, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0.0f, M,
                  N, nullptr, nullptr, dW, dB, workspace, workspace_bytes, 0, 1,
                  N, N, N, N, N};
  norm_status_t st = dln::check_bwd(c);
  if (st != NORM_OK) return st;
  if (kind == NORM_RMSNORM) dB = nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M == 0) return zero_outputs(N, dtype, dW, dB, s);
  return run_reduce(dtype, N, dW, dB, workspace, workspace_bytes, s);
}

norm_status_t norm_workspace_size(norm_kind_t kind, norm_dtype_t dtype, norm_pass_t pass,
                                  int64_t M, int64_t N, int residual, size_t *bytes) {
  if (!bytes) return NORM_ERR_INVALID_ARG;
  if (M < 0 || N <= 0) return NORM_ERR_INVALID_ARG;
  int cu = 0;
  norm_status_t st = current_cu_count(&cu);
  if (st != NORM_OK) return st;
  return dln::workspace_bytes(kind, dtype, pass, M, N, residual, cu, dln::tuning(), bytes);
}

size_t norm_workspace_bytes(norm_kind_t kind, int pass, int64_t M, int64_t N,
                            norm_dtype_t dtype, int residual) {
  if (M < 0 || N <= 0) return SIZE_MAX;
  size_t b = 0;
  if (dln::workspace_bytes_any_device(kind, dtype, static_cast<norm_pass_t>(pass), M, N,
                                      residual, dln::tuning(), &b) != NORM_OK)
    return SIZE_MAX;
  return b;
}

norm_status_t norm_workspace_status(void *workspace, size_t workspace_bytes,
                                    norm_stream_t stream) {
  if (workspace_bytes < dln::kWsHeaderBytes) return NORM_OK;
  if (!workspace || ((uintptr_t)workspace & 15u)) return NORM_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint64_t *word = header_word(workspace, dln::kWsErrWord);
  uint64_t v = 0;
  if (hipMemcpyAsync(&v, word, sizeof v, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return NORM_ERR_HIP;
  if (v != dln::kXchgFailWord) return NORM_OK;
  const uint64_t zero = 0;
  if (hipMemcpyAsync(word, &zero, sizeof zero, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return NORM_ERR_HIP;
  return NORM_ERR_EXCHANGE;
}

norm_status_t norm_plan(norm_kind_t kind, norm_dtype_t dtype, norm_pass_t pass, int64_t M,
                        int64_t N, int residual, int align, int cu_count, norm_plan_t *out) {
  if (!out) return NORM_ERR_INVALID_ARG;
  dln::Plan p;
  norm_status_t st =
      dln::make_plan(kind, dtype, pass, M, N, residual, align, align >= 16 ? 0 : -1,
                     (int)((N * (int64_t)dln::act_elem_size(dtype)) % 16 /
                           (int64_t)dln::act_elem_size(dtype)),
                     cu_count, dln::tuning(), &p);
  if (st != NORM_OK) return st;
  norm_plan_t o{};
  o.scheme = p.scheme;
  o.access_bytes = p.access_bytes;
  o.elems_per_access = p.epv;
  o.threads = p.threads;
  o.team_threads = p.team_threads;
  o.accesses_per_thread = p.vpt;
  o.rows_per_iter = p.rows;
  o.row_order = p.row_order;
  o.grid = p.grid;
  o.chunks = p.chunks;
  o.chunk_elems = p.chunk_elems;
  o.row_groups = p.row_groups;
  o.partials = p.partials;
  o.workspace_bytes = p.ws_bytes;
  o.exchange_row_groups = p.xchg ? p.xrow_groups : 0;
  o.phase_classes = p.period;
  *out = o;
  return NORM_OK;
}

norm_status_t norm_set_tuning(norm_tune_t key, int64_t value) {
  return dln::set_tuning(key, value);
}

norm_status_t norm_set_launch_events(void *start_event, void *stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) {
    tl_events = dln::LaunchEvents{nullptr, nullptr};
    return NORM_ERR_INVALID_ARG;
  }
  tl_events = dln::LaunchEvents{static_cast<hipEvent_t>(start_event),
                                static_cast<hipEvent_t>(stop_event)};
  return NORM_OK;
}

const char *norm_status_string(norm_status_t status) {
  switch (status) {
  case NORM_OK: return "NORM_OK";
  case NORM_ERR_INVALID_ARG: return "NORM_ERR_INVALID_ARG: invalid argument";
  case NORM_ERR_UNSUPPORTED: return "NORM_ERR_UNSUPPORTED: shape or option not supported";
  case NORM_ERR_WORKSPACE: return "NORM_ERR_WORKSPACE: workspace missing or too small";
  case NORM_ERR_HIP: return "NORM_ERR_HIP: HIP runtime or launch failure";
  case NORM_ERR_EXCHANGE:
    return "NORM_ERR_EXCHANGE: a long-row call gave up waiting for partial sums (NaN outputs)";
  default: return "unknown norm status";
  }
}

int norm_version(void) { return 100; }

} // extern "C"
