// norm_split.hip -- split-row scheme for rows too long for one workgroup's registers.
//
// A row is cut into chunks of chunk_acc accesses; each chunk belongs to one workgroup.
//   forward : pass 1 writes per-chunk statistics (chunk mean, sum of squared deviations about
//             it and the sum of those deviations for LayerNorm; sum of squares for RMSNorm);
//             pass 2 combines the chunks of its row in a fixed order (the parallel-variance
//             combination: the row mean from the chunk means, the squared deviation as the
//             chunk sums plus count * (chunk mean - row mean)^2), re-reads its chunk and
//             writes the output.
//   backward: pass 1 walks a group of rows for one column chunk and writes, per (row, chunk),
//             the partial sums g*(x - mean), g and x - mean; pass 2 combines them per row,
//             re-reads the chunk, writes dX and accumulates the chunk's dW/dB column partials
//             over the group; the partials of the row groups are reduced afterwards (or
//             written directly when there is one group).
// Pass 2 re-reads what pass 1 read; its order is arranged so that the most recently read data
// comes back first (forward: block order reversed within each XCD; backward: same blocks,
// rows in descending order), which is what the L2 and the memory-side cache still hold.
//
// Method (web page "PyTorch atinge desempenho SOTA em normalização com torch.compile",
// matsubara.tec.br): para. 6 names very large shapes as a regression class; paras. 8-10 give
// the split reduction with a workspace of partial sums, without atomics, consolidated by an
// extra reduction pass. The page "Towards Free Normalization: Fusing Normalization into GEMM
// and Attention Kernels" (brifing.si), item 4, names spreading one row's norm over several
// thread blocks (multi-CTA).
#include "norm_device.hpp"
#include "norm_internal.hpp"

namespace dln {

constexpr int SPLIT_LB = 256;

// Bijection on [0, nb) that keeps b % 8 (the XCD a block is dispatched to) and reverses the
// order of the blocks within each XCD.
__device__ __forceinline__ int64_t reverse_within_xcd(int64_t b, int64_t nb) {
  const int64_t x = b & 7, i = b >> 3;
  const int64_t nx = (nb - x + 7) >> 3;
  return ((nx - 1 - i) << 3) + x;
}

// Per-(row, chunk) partials, RP floats each:
//   forward  LayerNorm: [0] chunk mean m_c, [1] sum (x - m_c)^2, [2] sum (x - m_c)
//            RMSNorm  : [0] sum x^2
//   backward LayerNorm: [0] sum g*(x - m), [1] sum g, [2] sum (x - m)   (m: the row's mean)
//            RMSNorm  : [0] sum g*x
constexpr int RP = 4;

// Combine the chunk statistics of one row (rp = rowpart + row * C * RP). LayerNorm returns the
// mean as shift + delta, with shift = chunk 0's mean: every chunk then contributes small,
// accurately representable terms (ln_chunk_terms), one team sum for both. All threads of the
// workgroup call it. The single-pass form (norm_xsplit.hip) combines in the same order with
// the same terms, so both forms give the same statistics bit for bit.
__device__ __forceinline__ void combine_row_stats(const float *rp, int64_t C, int32_t chunk_acc,
                                                  int32_t nacc, int E, int layernorm,
                                                  float inv_n, float eps, float *red, int &slot,
                                                  float &shift, float &delta, float &rstd) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, waves = blockDim.x >> 6;
  if (layernorm) {
    shift = rp[0];
    float ab[2] = {0.0f, 0.0f};
    for (int64_t c = tid; c < C; c += blockDim.x)
      ln_chunk_terms(split_chunk_elems(c, chunk_acc, nacc, E), rp[RP * c], rp[RP * c + 1],
                     rp[RP * c + 2], shift, ab[0], ab[1]);
    team_sum<2, SPLIT_LB / 64>(ab, red, slot, waves, 0, wave, lane);
    slot ^= 1;
    rstd = ln_combined_rstd(ab[0], ab[1], inv_n, eps, delta);
  } else {
    float q[1] = {0.0f};
    for (int64_t c = tid; c < C; c += blockDim.x) q[0] += rp[RP * c];
    team_sum<1, SPLIT_LB / 64>(q, red, slot, waves, 0, wave, lane);
    slot ^= 1;
    shift = 0.0f;
    delta = 0.0f;
    rstd = rsqrt_f32(q[0] * inv_n + eps);
  }
}

// ---- forward pass 1: chunk statistics ---------------------------------------------------

template <typename T, int EV, int VPT, bool RESID>
__global__ __launch_bounds__(SPLIT_LB) void split_stats_kernel(FwdArgs a) {
  using A = Acc<T, EV>;
  using raw = typename A::raw;
  constexpr int E = A::EPV;
  __shared__ __align__(16) float red[RED_FLOATS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, waves = blockDim.x >> 6;
  const int64_t C = a.chunks;
  const int64_t row = (int64_t)blockIdx.x / C;
  const int64_t c = (int64_t)blockIdx.x - row * C;
  const int64_t acc0 = c * a.chunk_acc;
  const int64_t left = (int64_t)a.nacc - acc0;
  const int nin = (int)(left < a.chunk_acc ? left : a.chunk_acc);
  const int64_t col0 = acc0 * E;
  const T *__restrict__ X = static_cast<const T *>(a.x) + row * a.ldx + col0;
  const T *__restrict__ Rr = RESID ? static_cast<const T *>(a.r) + row * a.ldr + col0 : nullptr;
  T *__restrict__ H = RESID ? static_cast<T *>(a.h) + row * a.ldh + col0 : nullptr;

  float x[VPT][E];
  {
    raw rx[VPT], rr[RESID ? VPT : 1];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int v = tid + k * SPLIT_LB;
      rx[k] = A::zero();
      if (RESID) rr[k] = A::zero();
      if (v < nin) {
        rx[k] = A::ld(X + (int64_t)v * E);
        if (RESID) rr[k] = A::ld(Rr + (int64_t)v * E);
      }
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      A::unpack(rx[k], x[k]);
      if (RESID) {
        float f[E];
        A::unpack(rr[k], f);
#pragma unroll
        for (int e = 0; e < E; ++e) f[e] += x[k][e];
        const raw hp = A::pack(f);
        A::unpack(hp, x[k]);
        const int v = tid + k * SPLIT_LB;
        if (v < nin) A::st(H + (int64_t)v * E, hp);
      }
    }
  }
  const float n_c = (float)(nin * E);
  float *out = a.rowpart + (row * C + c) * RP;
  int slot = 0;
  if (a.layernorm) {
    float s[1] = {0.0f};
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
      for (int e = 0; e < E; ++e) s[0] += x[k][e];
    team_sum<1, SPLIT_LB / 64>(s, red, slot, waves, 0, wave, lane);
    slot ^= 1;
    const float mc = s[0] / n_c;
    float qc[2] = {0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const bool in = tid + k * SPLIT_LB < nin;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float d = in ? x[k][e] - mc : 0.0f;
        qc[0] += d * d;
        qc[1] += d;
      }
    }
    team_sum<2, SPLIT_LB / 64>(qc, red, slot, waves, 0, wave, lane);
    if (tid == 0) {
      out[0] = mc;
      out[1] = qc[0];
      out[2] = qc[1];
    }
  } else {
    float q[1] = {0.0f};
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
      for (int e = 0; e < E; ++e) q[0] += x[k][e] * x[k][e];
    team_sum<1, SPLIT_LB / 64>(q, red, slot, waves, 0, wave, lane);
    if (tid == 0) out[0] = q[0];
  }
}

// ---- forward pass 2: combine, normalise the chunk ---------------------------------------

template <typename T, typename TW, int EV, int VPT>
__global__ __launch_bounds__(SPLIT_LB) void split_norm_kernel(FwdArgs a) {
  using A = Acc<T, EV>;
  using raw = typename A::raw;
  constexpr int E = A::EPV;
  __shared__ __align__(16) float red[RED_FLOATS];
  const int tid = threadIdx.x;
  const int64_t C = a.chunks;
  const int64_t b = reverse_within_xcd(blockIdx.x, gridDim.x);
  const int64_t row = b / C;
  const int64_t c = b - row * C;
  const int64_t acc0 = c * a.chunk_acc;
  const int64_t left = (int64_t)a.nacc - acc0;
  const int nin = (int)(left < a.chunk_acc ? left : a.chunk_acc);
  const int64_t col0 = acc0 * E;
  // the norm's input: the stored h for the residual variant, else X
  const T *__restrict__ S = static_cast<const T *>(a.r ? a.h : a.x) + row * (a.r ? a.ldh : a.ldx) +
                            col0;
  const TW *__restrict__ W = static_cast<const TW *>(a.w) + acc0 * E;
  const TW *__restrict__ Bb = a.b ? static_cast<const TW *>(a.b) + acc0 * E : nullptr;
  T *__restrict__ Y = static_cast<T *>(a.y) + row * a.ldy + col0;

  raw rx[VPT];
  WAcc<T, TW, EV> rw[VPT], rb[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int v = tid + k * SPLIT_LB;
    rx[k] = A::zero();
    rw[k].zero();
    rb[k].zero();
    if (v < nin) {
      rx[k] = A::ld_cached(S + (int64_t)v * E);
      rw[k].load(W + (int64_t)v * E);
      if (Bb) rb[k].load(Bb + (int64_t)v * E);
    }
  }
  int slot = 0;
  float shift, delta, rstd;
  combine_row_stats(a.rowpart + row * C * RP, C, a.chunk_acc, a.nacc, E, a.layernorm, a.inv_n,
                    a.eps, red, slot, shift, delta, rstd);
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int v = tid + k * SPLIT_LB;
    if (v < nin) {
      float xf[E], wf[E], bf[E], y[E];
      A::unpack(rx[k], xf);
      rw[k].get(wf);
      rb[k].get(bf);
#pragma unroll
      for (int e = 0; e < E; ++e) y[e] = ((xf[e] - shift) - delta) * rstd * wf[e] + bf[e];
      A::st(Y + (int64_t)v * E, A::pack(y));
    }
  }
  if (c == 0 && tid == 0) {
    if (a.mean) a.mean[row] = shift + delta;
    if (a.rstd) a.rstd[row] = rstd;
  }
}

// ---- statistics-only forward: combine the chunk statistics, write mean and rstd ------------

__global__ __launch_bounds__(SPLIT_LB) void split_stats_combine_kernel(FwdArgs a, int E) {
  __shared__ __align__(16) float red[RED_FLOATS];
  const int64_t row = blockIdx.x;
  int slot = 0;
  float shift, delta, rstd;
  combine_row_stats(a.rowpart + row * a.chunks * RP, a.chunks, a.chunk_acc, a.nacc, E,
                    a.layernorm, a.inv_n, a.eps, red, slot, shift, delta, rstd);
  if (threadIdx.x == 0) {
    if (a.mean) a.mean[row] = shift + delta;
    if (a.rstd) a.rstd[row] = rstd;
  }
}

// ---- backward: statistics when the forward's were not kept ------------------------------

__global__ __launch_bounds__(SPLIT_LB) void split_finalize_stats_kernel(BwdArgs a, int E) {
  __shared__ __align__(16) float red[RED_FLOATS];
  const int64_t row = blockIdx.x;
  int slot = 0;
  float shift, delta, rstd;
  combine_row_stats(a.rowpart + row * a.chunks * RP, a.chunks, a.chunk_acc, a.nacc, E,
                    a.layernorm, a.inv_n, a.eps, red, slot, shift, delta, rstd);
  if (threadIdx.x == 0) {
    a.stats[row] = shift + delta;
    a.stats[a.M + row] = rstd;
  }
}

// ---- backward pass 1: row partials ---------------------------------------------------------

// One workgroup per (row, chunk), like the forward's statistics pass: the whole grid streams X
// and dY once, with no loop-carried latency.
template <typename T, typename TW, int EV, int VPT, bool LN>
__global__ __launch_bounds__(SPLIT_LB) void split_bwd_partial_kernel(BwdArgs a) {
  using A = Acc<T, EV>;
  using raw = typename A::raw;
  constexpr int E = A::EPV;
  __shared__ __align__(16) float red[RED_FLOATS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, waves = blockDim.x >> 6;
  const int64_t C = a.chunks;
  const int64_t row = (int64_t)blockIdx.x / C;
  const int64_t c = (int64_t)blockIdx.x - row * C;
  const int64_t acc0 = c * a.chunk_acc;
  const int64_t left = (int64_t)a.nacc - acc0;
  const int nin = (int)(left < a.chunk_acc ? left : a.chunk_acc);
  const int64_t col0 = acc0 * E;
  const T *__restrict__ X = static_cast<const T *>(a.x) + row * a.ldx + col0;
  const T *__restrict__ DY = static_cast<const T *>(a.dy) + row * a.lddy + col0;
  const TW *__restrict__ W = static_cast<const TW *>(a.w) + acc0 * E;
  const float *mean_p = a.rstd ? a.mean : a.stats;

  raw rx[VPT], rdy[VPT];
  WAcc<T, TW, EV> rw[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int v = tid + k * SPLIT_LB;
    rx[k] = A::zero();
    rdy[k] = A::zero();
    rw[k].zero();
    if (v < nin) {
      rx[k] = A::ld(X + (int64_t)v * E);
      rdy[k] = A::ld(DY + (int64_t)v * E);
      rw[k].load(W + (int64_t)v * E);
    }
  }
  const float m = (LN && mean_p) ? mean_p[row] : 0.0f;
  constexpr int NV = LN ? 3 : 1;
  float sums[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) sums[i] = 0.0f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const bool in = tid + k * SPLIT_LB < nin;
    float xf[E], df[E], wf[E];
    A::unpack(rx[k], xf);
    A::unpack(rdy[k], df);
    rw[k].get(wf);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float d = in ? xf[e] - m : 0.0f;
      const float gg = df[e] * wf[e];
      sums[0] += gg * d;
      if constexpr (LN) {
        sums[1] += gg;
        sums[2] += d;
      }
    }
  }
  int slot = 0;
  team_sum<NV, SPLIT_LB / 64>(sums, red, slot, waves, 0, wave, lane);
  if (tid == 0) {
    float *out = a.rowpart + (row * C + c) * RP;
    out[0] = sums[0];
    if constexpr (LN) {
      out[1] = sums[1];
      out[2] = sums[2];
    }
  }
}

// ---- backward pass 2: dX and the column partials -------------------------------------------

// One workgroup per (row group, chunk). Rows are visited in descending order (the last rows
// pass 1 read come back first) and the next row group's X and dY are requested before the
// current one is combined and written.
template <typename T, typename TW, int EV, int VPT, int ROWS, bool LN>
__global__ __launch_bounds__(SPLIT_LB) void split_bwd_dx_kernel(BwdArgs a) {
  using A = Acc<T, EV>;
  using raw = typename A::raw;
  constexpr int E = A::EPV;
  __shared__ __align__(16) float red[RED_FLOATS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, waves = blockDim.x >> 6;
  const int64_t C = a.chunks;
  const int64_t g = (int64_t)blockIdx.x / C;
  const int64_t c = (int64_t)blockIdx.x - g * C;
  const int64_t acc0 = c * a.chunk_acc;
  const int64_t left = (int64_t)a.nacc - acc0;
  const int nin = (int)(left < a.chunk_acc ? left : a.chunk_acc);
  const int64_t N = a.N;
  const int64_t r_begin = g * a.rows_per_group;
  const int64_t r_end = r_begin + a.rows_per_group < a.M ? r_begin + a.rows_per_group : a.M;
  const T *__restrict__ X = static_cast<const T *>(a.x) + acc0 * E;
  const T *__restrict__ DY = static_cast<const T *>(a.dy) + acc0 * E;
  const T *__restrict__ DH = a.dh ? static_cast<const T *>(a.dh) + acc0 * E : nullptr;
  const TW *__restrict__ W = static_cast<const TW *>(a.w) + acc0 * E;
  T *__restrict__ DX = static_cast<T *>(a.dx) + acc0 * E;
  T *__restrict__ DR = a.dr ? static_cast<T *>(a.dr) + acc0 * E : nullptr;
  const float *mean_p = a.rstd ? a.mean : a.stats;
  const float *rstd_p = a.rstd ? a.rstd : a.stats + a.M;
  if (!a.dw) write_ws_header(a.header, a.row_groups, N);

  // the weight stays packed (half the registers for bf16), unpacked at use
  WAcc<T, TW, EV> rw[VPT];
  float accw[VPT][E], accb[LN ? VPT : 1][E];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int v = tid + k * SPLIT_LB;
    rw[k].zero();
    if (v < nin) rw[k].load(W + (int64_t)v * E);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      accw[k][e] = 0.0f;
      if constexpr (LN) accb[k][e] = 0.0f;
    }
  }
  const int64_t nrows = r_end > r_begin ? r_end - r_begin : 0;
  const int64_t iters = (nrows + ROWS - 1) / ROWS;
  // Prefetched with the next rows: X, dY, the row statistics, and the row partials of up to
  // RPF chunks per thread (the rest, for rows of more than RPF * 256 chunks, are read at use).
  constexpr int RPF = 2;
  constexpr int NQ = LN ? 3 : 1;
  raw px[ROWS][VPT], pdy[ROWS][VPT];
  float pm[ROWS], prs[ROWS], pq[ROWS][RPF][NQ];
  auto issue = [&](int64_t it) {
    const int64_t row0 = r_begin + it * ROWS;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const bool rv = it >= 0 && row0 + r < r_end;
      const int64_t rowc = rv ? row0 + r : r_end - 1;
      pm[r] = (LN && mean_p) ? mean_p[rowc] : 0.0f;
      prs[r] = rstd_p[rowc];
      const float *rp = a.rowpart + rowc * C * RP;
#pragma unroll
      for (int j = 0; j < RPF; ++j) {
        const int64_t cc = tid + (int64_t)j * SPLIT_LB;
#pragma unroll
        for (int q = 0; q < NQ; ++q) pq[r][j][q] = cc < C ? rp[RP * cc + q] : 0.0f;
      }
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int v = tid + k * SPLIT_LB;
        px[r][k] = A::zero();
        pdy[r][k] = A::zero();
        if (rv && v < nin) {
          px[r][k] = A::ld(X + (row0 + r) * a.ldx + (int64_t)v * E);
          pdy[r][k] = A::ld(DY + (row0 + r) * a.lddy + (int64_t)v * E);
        }
      }
    }
  };
  int slot = 0;
  issue(iters - 1);
#pragma unroll
  for (int k = 0; k < VPT; ++k) rw[k].settle();
  for (int64_t it = iters - 1; it >= 0; --it) {
    const int64_t row0 = r_begin + it * ROWS;
    raw rx[ROWS][VPT], rdy[ROWS][VPT];
    float m_r[ROWS], rs_r[ROWS];
    // combine the row partials of every chunk of these rows: this thread's chunks in
    // ascending order, then the team sum
    constexpr int NV = LN ? 3 * ROWS : ROWS;
    float sums[NV];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      m_r[r] = pm[r];
      rs_r[r] = prs[r];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < RPF; ++j) acc += pq[r][j][q];
        sums[q * ROWS + r] = acc;
      }
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        rx[r][k] = px[r][k];
        rdy[r][k] = pdy[r][k];
      }
    }
    issue(it - 1);
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const int64_t rowc = row0 + r < r_end ? row0 + r : r_end - 1;
      const float *rp = a.rowpart + rowc * C * RP;
      for (int64_t cc = tid + (int64_t)RPF * SPLIT_LB; cc < C; cc += SPLIT_LB) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) sums[q * ROWS + r] += rp[RP * cc + q];
      }
    }
    team_sum<NV, SPLIT_LB / 64>(sums, red, slot, waves, 0, wave, lane);
    slot ^= 1;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const int64_t row = row0 + r;
      const bool rv = row < r_end;
      const float m = m_r[r];
      const float rstd = rs_r[r];
      const float delta = LN ? sums[2 * ROWS + r] * a.inv_n : 0.0f;
      const float c1 = LN ? sums[ROWS + r] * a.inv_n : 0.0f;
      const float c2 = LN ? rstd * (sums[r] - delta * sums[ROWS + r]) * a.inv_n
                          : rstd * sums[r] * a.inv_n;
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int v = tid + k * SPLIT_LB;
        const bool in = rv && v < nin;
        float xf[E], df[E], wf[E], dx[E];
        A::unpack(rx[r][k], xf);
        A::unpack(rdy[r][k], df);
        rw[k].get(wf);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float xh = in ? ((xf[e] - m) - delta) * rstd : 0.0f;
          dx[e] = rstd * (df[e] * wf[e] - c1 - xh * c2);
          accw[k][e] += df[e] * xh;
          if constexpr (LN) accb[k][e] += df[e];
        }
        if (in) {
          const int64_t off = (int64_t)v * E;
          if (DH) {
            float hf[E];
            A::unpack(A::ld(DH + row * a.lddh + off), hf);
#pragma unroll
            for (int e = 0; e < E; ++e) dx[e] += hf[e];
          }
          const raw p = A::pack(dx);
          A::st(DX + row * a.lddx + off, p);
          if (DR) A::st(DR + row * a.lddr + off, p);
        }
      }
    }
  }
  // column partials of this (row group, chunk), or the final dW/dB when the caller asked for
  // them directly (only ever with a single row group)
  if (a.dw) {
    TW *dw = static_cast<TW *>(a.dw) + acc0 * E;
    TW *db = a.db ? static_cast<TW *>(a.db) + acc0 * E : nullptr;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int v = tid + k * SPLIT_LB;
      if (v < nin) {
        WAcc<T, TW, EV>::store(dw + (int64_t)v * E, accw[k]);
        if constexpr (LN)
          if (db) WAcc<T, TW, EV>::store(db + (int64_t)v * E, accb[k]);
      }
    }
  } else {
    float *pw = a.colpart + g * N + acc0 * E;
    float *pb = a.colpart + (a.row_groups + g) * N + acc0 * E;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int v = tid + k * SPLIT_LB;
      if (v < nin) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          pw[(int64_t)v * E + e] = accw[k][e];
          if constexpr (LN) pb[(int64_t)v * E + e] = accb[k][e];
        }
      }
    }
  }
}

// ---- launchers ---------------------------------------------------------------------------------

namespace {

#define DLN_SPLIT_FWD_MENU(X) X(1) X(2) X(4)
#define DLN_SPLIT_BWD_MENU(X) X(1, 1) X(1, 2) X(1, 4) X(2, 1) X(2, 2) X(2, 4) X(4, 1) X(4, 2)
#define DLN_SPLIT_SCALAR_VPT 8
// 8- and 4-byte accesses: the full-width chunk (4 accesses of 16 bytes per thread) in narrower
// accesses, one row at a time in the backward's second pass
#define DLN_SPLIT_NARROW_VPT_FULL 4

template <typename T, int EV, int V>
hipError_t split_stats_launch(const FwdArgs &a, bool resid, hipStream_t s) {
  const dim3 grid((unsigned)(a.M * a.chunks)), block(SPLIT_LB);
  return resid ? launch(split_stats_kernel<T, EV, V, true>, grid, block, s, a)
               : launch(split_stats_kernel<T, EV, V, false>, grid, block, s, a);
}

template <typename T, typename TW, int EV, int V>
hipError_t split_fwd_pair(const FwdArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)(a.M * a.chunks)), block(SPLIT_LB);
  hipError_t e = split_stats_launch<T, EV, V>(a, a.r != nullptr, s);
  if (e != hipSuccess) return e;
  if (!a.y) // statistics only: one combine per row, no second pass over X
    return launch(split_stats_combine_kernel, dim3((unsigned)a.M), block, s, a, EV);
  return launch(split_norm_kernel<T, TW, EV, V>, grid, block, s, a);
}

template <typename T, typename TW, int EV, int V, int R>
hipError_t split_bwd_pair(const Plan &p, const BwdArgs &a, hipStream_t s) {
  const dim3 grid1((unsigned)(a.M * a.chunks)), grid2((unsigned)p.grid), block(SPLIT_LB);
  hipError_t e;
  if (a.layernorm) {
    e = launch(split_bwd_partial_kernel<T, TW, EV, V, true>, grid1, block, s, a);
    if (e == hipSuccess)
      e = launch(split_bwd_dx_kernel<T, TW, EV, V, R, true>, grid2, block, s, a);
  } else {
    e = launch(split_bwd_partial_kernel<T, TW, EV, V, false>, grid1, block, s, a);
    if (e == hipSuccess)
      e = launch(split_bwd_dx_kernel<T, TW, EV, V, R, false>, grid2, block, s, a);
  }
  return e;
}

// The statistics pass of every width: hipErrorInvalidConfiguration when the plan's width and
// chunk have no kernel (reported as NORM_ERR_UNSUPPORTED by the callers).
template <typename T>
hipError_t split_stats_any(const Plan &p, const FwdArgs &a, bool resid, hipStream_t s,
                           bool *found) {
  constexpr int F = full_epv<T>();
  *found = true;
  if (p.epv == F) {
#define X(V)                                                                                    \
  if (p.vpt == V) return split_stats_launch<T, F, V>(a, resid, s);
    DLN_SPLIT_FWD_MENU(X)
#undef X
  } else if (p.epv == F / 2 && p.vpt == DLN_SPLIT_NARROW_VPT_FULL * 2) {
    return split_stats_launch<T, F / 2, DLN_SPLIT_NARROW_VPT_FULL * 2>(a, resid, s);
  } else if (p.epv == F / 4 && p.vpt == DLN_SPLIT_NARROW_VPT_FULL * 4) {
    if constexpr (F / 4 >= 2)
      return split_stats_launch<T, F / 4, DLN_SPLIT_NARROW_VPT_FULL * 4>(a, resid, s);
  } else if (p.epv == 1 && p.vpt == DLN_SPLIT_SCALAR_VPT) {
    return split_stats_launch<T, 1, DLN_SPLIT_SCALAR_VPT>(a, resid, s);
  }
  *found = false;
  return hipErrorInvalidConfiguration;
}

template <typename T, typename TW>
norm_status_t split_fwd_typed(const Plan &p, const FwdArgs &a, hipStream_t s) {
  constexpr int F = full_epv<T>();
  constexpr int NV = DLN_SPLIT_NARROW_VPT_FULL;
  hipError_t e = hipErrorInvalidConfiguration;
  bool found = true;
  if (p.epv == F) {
    found = false;
#define X(V)                                                                                    \
  if (!found && p.vpt == V) {                                                                   \
    found = true;                                                                               \
    e = split_fwd_pair<T, TW, F, V>(a, s);                                                      \
  }
    DLN_SPLIT_FWD_MENU(X)
#undef X
  } else if (p.epv == F / 2 && p.vpt == NV * 2) {
    e = split_fwd_pair<T, TW, F / 2, NV * 2>(a, s);
  } else if (p.epv == F / 4 && p.vpt == NV * 4) {
    if constexpr (F / 4 >= 2)
      e = split_fwd_pair<T, TW, F / 4, NV * 4>(a, s);
    else
      found = false;
  } else if (p.epv == 1 && p.vpt == DLN_SPLIT_SCALAR_VPT) {
    e = split_fwd_pair<T, TW, 1, DLN_SPLIT_SCALAR_VPT>(a, s);
  } else {
    found = false;
  }
  if (!found) return NORM_ERR_UNSUPPORTED;
  return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

template <typename T, typename TW>
norm_status_t split_bwd_typed(const Plan &p, const BwdArgs &a, hipStream_t s) {
  constexpr int F = full_epv<T>();
  constexpr int NV = DLN_SPLIT_NARROW_VPT_FULL;
  // statistics of the forward, when not supplied: chunk stats, then one combine per row
  if (a.rstd == nullptr) {
    FwdArgs f{};
    f.x = a.x;
    f.ldx = a.ldx;
    f.rowpart = a.rowpart;
    f.M = a.M;
    f.N = a.N;
    f.nacc = a.nacc;
    f.chunks = a.chunks;
    f.chunk_acc = a.chunk_acc;
    f.layernorm = a.layernorm;
    f.eps = a.eps;
    f.inv_n = a.inv_n;
    bool found = false;
    hipError_t e = split_stats_any<T>(p, f, false, s, &found);
    if (!found) return NORM_ERR_UNSUPPORTED;
    if (e == hipSuccess)
      e = launch(split_finalize_stats_kernel, dim3((unsigned)a.M), dim3(SPLIT_LB), s, a, p.epv);
    if (e != hipSuccess) return NORM_ERR_HIP;
  }
  bool found = true;
  hipError_t e = hipErrorInvalidConfiguration;
  if (p.epv == F) {
    found = false;
#define X(V, R)                                                                                 \
  if (!found && p.vpt == V && p.rows == R) {                                                    \
    found = true;                                                                               \
    e = split_bwd_pair<T, TW, F, V, R>(p, a, s);                                                \
  }
    DLN_SPLIT_BWD_MENU(X)
#undef X
  } else if (p.epv == F / 2 && p.vpt == NV * 2 && p.rows == 1) {
    e = split_bwd_pair<T, TW, F / 2, NV * 2, 1>(p, a, s);
  } else if (p.epv == F / 4 && p.vpt == NV * 4 && p.rows == 1) {
    if constexpr (F / 4 >= 2)
      e = split_bwd_pair<T, TW, F / 4, NV * 4, 1>(p, a, s);
    else
      found = false;
  } else if (p.epv == 1 && p.vpt == DLN_SPLIT_SCALAR_VPT && p.rows == 1) {
    e = split_bwd_pair<T, TW, 1, DLN_SPLIT_SCALAR_VPT, 1>(p, a, s);
  } else {
    found = false;
  }
  if (!found) return NORM_ERR_UNSUPPORTED;
  return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

} // namespace

norm_status_t launch_split_fwd(const Plan &p, norm_dtype_t dtype, const FwdArgs &a,
                               hipStream_t s) {
  switch (dtype) {
  case NORM_F32: return split_fwd_typed<float, float>(p, a, s);
  case NORM_BF16: return split_fwd_typed<bf16_bits, bf16_bits>(p, a, s);
  case NORM_BF16_F32W: return split_fwd_typed<bf16_bits, float>(p, a, s);
  case NORM_F16: return split_fwd_typed<f16_t, f16_t>(p, a, s);
  case NORM_F16_F32W: return split_fwd_typed<f16_t, float>(p, a, s);
  default: return NORM_ERR_UNSUPPORTED;
  }
}

norm_status_t launch_split_bwd(const Plan &p, norm_dtype_t dtype, const BwdArgs &a,
                               hipStream_t s) {
  switch (dtype) {
  case NORM_F32: return split_bwd_typed<float, float>(p, a, s);
  case NORM_BF16: return split_bwd_typed<bf16_bits, bf16_bits>(p, a, s);
  case NORM_BF16_F32W: return split_bwd_typed<bf16_bits, float>(p, a, s);
  case NORM_F16: return split_bwd_typed<f16_t, f16_t>(p, a, s);
  case NORM_F16_F32W: return split_bwd_typed<f16_t, float>(p, a, s);
  default: return NORM_ERR_UNSUPPORTED;
  }
}

} // namespace dln
