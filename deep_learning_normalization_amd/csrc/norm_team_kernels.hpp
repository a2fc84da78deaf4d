// norm_team_kernels.hpp -- row-resident forward and fused backward kernels (templates shared by
// the translation units that instantiate them for each access width).
//
// A "team" of threads owns one row at a time and keeps the whole row in registers:
//   wave scheme : a team is one 64-lane wavefront; sums stay inside the wavefront (DPP), no LDS
//                 and no barrier. Used for short rows.
//   block scheme: a team is several wavefronts; wavefront sums meet in LDS behind one barrier.
// Kernels are persistent: each workgroup walks row groups with a grid stride, so the weight
// (and bias) of a thread's columns are loaded once and, in the backward, the dW/dB column sums
// of all rows a workgroup visits accumulate in registers.
//
// Method (web page "PyTorch atinge desempenho SOTA em normalização com torch.compile",
// matsubara.tec.br):
//   para. 3  -- forward: reduction along the contiguous dimension, then pointwise work;
//   para. 5  -- short reduction dimensions are reduced without a loop, the row held on chip;
//   para. 7  -- backward gradients dX, dW, dB;
//   paras. 8-10 -- one fused pass produces dX and per-block partial column sums (no atomics;
//               several rows per block), and a second pass consolidates the partials;
//   para. 12 -- several rows in flight per team (the software-pipelining knob).
// Rows that do not start on 16-byte boundaries (an odd N, strides or pointers of that kind) keep
// 16-byte accesses (the PART instantiations, launched for such rows only, so the others compile
// without this code). With all activation tensors at one phase (the same address and stride
// modulo 16 bytes), row r starts pe(r) elements past a boundary, and pe(r) depends only on
// r mod P (P = 1, 2, 4 or 8 classes). Each workgroup takes the rows of one class, so its pe is
// fixed: access v of a row covers columns v * E - pe ... v * E - pe + E - 1, aligned in memory,
// except the first and the last access, which cover the row's first and last E columns (in
// bounds, possibly unaligned; they overlap their neighbours). Every lane loads, computes and
// stores all E columns of its access with its weights gathered once at those columns; a 0/1
// factor per element, fixed per lane for the workgroup, keeps the columns an edge access shares
// with its neighbour (and accesses past the row's end) out of the row sums and the dW / dB sums,
// and the shared columns are stored twice with the same value (the same instructions on the same
// inputs). So the rows take no branch and no element-wise access: measured on MI355X, a branch
// around loads or around values of loads in flight makes the compiler wait for every load in
// flight (LayerNorm 16384 x 4097 forward 240 us), and shifting the edge elements into an aligned
// grid costs the VALU time these kernels do not have (they run 60-75% VALU-busy).
// Memory: every [M, N] element moves through 16-byte coalesced accesses, exactly once per pass
// (web page "Otimização de Performance de GPU: Maximizando Throughput para Treinamento e
// Inferência de LLM", introl.com, sections on memory bandwidth and on kernel fusion), and all
// arithmetic is fp32 (same page, section on mixed precision).
#pragma once

#include "norm_device.hpp"
#include "norm_internal.hpp"

namespace dln {

// Partial column sums of the backward are merged across the teams of a workgroup through
// LDS in blocks of this many floats.
constexpr int MERGE_FLOATS = 4096;

struct TeamGeom {
  int tt;       // threads per team
  int team;     // team index in the workgroup
  int t;        // thread index in the team
  int teams;    // teams per workgroup
  int waves;    // wavefronts per team
  int wave0;    // first wavefront of this team in the workgroup
  int wave;     // this thread's wavefront in the workgroup
  int lane;
};

template <bool WAVE> __device__ __forceinline__ TeamGeom team_geom(int team_threads) {
  TeamGeom g;
  const int tid = threadIdx.x;
  g.tt = WAVE ? 64 : team_threads;
  g.team = tid / g.tt;
  g.t = tid - g.team * g.tt;
  g.teams = blockDim.x / g.tt;
  g.waves = g.tt >> 6;
  g.wave = tid >> 6;
  g.wave0 = g.team * g.waves;
  g.lane = tid & 63;
  return g;
}

// Row groups of this workgroup: first, first + step, ... below end. Interleaved: group g goes
// to workgroup g mod grid. Blocked: workgroup b takes the contiguous groups
// [b * per, (b + 1) * per), per = ceil(groups / grid), so its rows stream from one region.
struct GroupRange {
  int64_t first, step, end;
};
__device__ __forceinline__ GroupRange group_range(int64_t M, int64_t rows_per_group,
                                                  int blocked, int64_t bid, int64_t nb) {
  const int64_t groups = (M + rows_per_group - 1) / rows_per_group;
  if (!blocked) return GroupRange{bid, nb, groups};
  const int64_t per = (groups + nb - 1) / nb;
  const int64_t first = bid * per;
  return GroupRange{first, 1, first + per < groups ? first + per : groups};
}

// The rows a workgroup walks and where their accesses fall. Without PART: every row, accesses
// v * E ... v * E + E - 1 from the row start. With PART: the rows of class blockIdx.x mod P
// (row = cls + P * i for i < Mv), workgroup blockIdx.x / P of gridDim.x / P on them; their
// inner accesses start pe elements before their aligned block, nal accesses per row (see win).
template <int E, bool PART> struct RowPhase {
  int P = 1, cls = 0, pe = 0, nal = 0, lastn = E, n = 0;
  int64_t Mv = 0, bid = 0, nb = 1, m = 0;
  __device__ RowPhase(int nacc, int64_t M, int N, int period, int phase0, int dphase) {
    n = N;
    m = M;
    if constexpr (PART) {
      P = period;
      cls = (int)(blockIdx.x % (unsigned)P);
      bid = blockIdx.x / (unsigned)P;
      nb = gridDim.x / (unsigned)P;
      pe = (phase0 + cls * dphase) & (E - 1);
      nal = (N + pe + E - 1) / E;
      lastn = N + pe - (nal - 1) * E;
      Mv = M > cls ? (M - cls + P - 1) / P : 0;
    } else {
      (void)N, (void)period, (void)phase0, (void)dphase;
      nal = nacc;
      Mv = M;
      bid = blockIdx.x;
      nb = gridDim.x;
    }
  }
  __device__ int64_t row(int64_t i) const { return PART ? cls + (int64_t)P * i : i; }
  // a row of the tensor to load from for row index i of this workgroup, valid or not (PART
  // loads unconditionally: rows past the class's last read a real row, masked afterwards)
  __device__ int64_t load_row(int64_t i, bool valid) const {
    if (valid) return row(i);
    const int64_t r = row(Mv > 0 ? Mv - 1 : 0);
    return r < m ? r : m - 1;
  }
  // element offset, from the row's start, of the E columns access v loads and stores: v * E
  // without PART; with PART v * E - pe (aligned) for the inner accesses, 0 and N - E (N >= E)
  // for the first and the last
  __device__ int64_t win(int v) const {
    if constexpr (!PART) return (int64_t)v * E;
    // (arithmetic rather than a choice, which the compiler turns into a branch around the load)
    const int o = v * E - pe; // N < 2^31
    const int first = v == 0, last = v == nal - 1;
    return (int64_t)(o + first * pe + last * (n - E - o - first * pe));
  }
  // 1 for element e of access v if this access owns its column, 0 if the neighbouring access
  // owns it (the first access's last pe columns, the last access's first E - lastn) or v is past
  // the row's end
  __device__ float own(int v, int e) const {
    if constexpr (!PART) return 1.0f;
    const int olo = v == nal - 1 ? E - lastn : 0;
    const int ohi = v >= nal ? 0 : v == 0 ? E - pe : E;
    return (e >= olo && e < ohi) ? 1.0f : 0.0f;
  }
  // weights at access v's columns (once per workgroup; zero past the row's end)
  template <typename WA, typename TW> __device__ void gather(WA &w, const TW *p, int v) const {
    w.load_any(p + win(v < nal ? v : nal - 1));
    if (v >= nal) w.zero();
  }
};

// ---- forward ------------------------------------------------------------------------------

template <typename T, typename TW, int EV, int VPT, int ROWS, int LB, bool WAVE, bool RESID,
          bool PART = false>
__global__ __launch_bounds__(LB) void team_fwd_kernel(FwdArgs a, int team_threads) {
  using A = Acc<T, EV>;
  using raw = typename A::raw;
  constexpr int E = A::EPV;
  __shared__ __align__(16) float red[RED_FLOATS];
  const TeamGeom gm = team_geom<WAVE>(team_threads);
  const RowPhase<E, PART> ph(a.nacc, a.M, a.N, a.period, a.phase0, a.dphase);
  const int nacc = ph.nal;
  const int64_t M = ph.Mv; // rows walked below are indices among this workgroup's rows
  const T *__restrict__ X = static_cast<const T *>(a.x);
  const T *__restrict__ Rr = static_cast<const T *>(a.r);
  const TW *__restrict__ W = static_cast<const TW *>(a.w);
  const TW *__restrict__ Bb = static_cast<const TW *>(a.b);
  T *__restrict__ Y = static_cast<T *>(a.y);
  T *__restrict__ H = static_cast<T *>(a.h);

  float w[VPT][E], b[VPT][E];
  float own[PART ? VPT : 1][E]; // see RowPhase::own
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int v = gm.t + k * gm.tt;
    if constexpr (PART) {
#pragma unroll
      for (int e = 0; e < E; ++e) own[k][e] = ph.own(v, e);
    }
    WAcc<T, TW, EV> rw, rb;
    rw.zero();
    rb.zero();
    if constexpr (PART) { // the class's columns (once per workgroup)
      if (W) {
        ph.gather(rw, W, v);
        if (Bb) ph.gather(rb, Bb, v);
      }
    } else if (W && v < nacc) { // no weight: the statistics-only pass
      rw.load(W + (int64_t)v * E);
      if (Bb) rb.load(Bb + (int64_t)v * E);
    }
    rw.get(w[k]);
    rb.get(b[k]);
  }

  const int64_t rows_per_group = (int64_t)gm.teams * ROWS;
  // Software pipeline: the next row group's loads are issued before the current group is
  // reduced and written, so every wavefront keeps requests in flight across its barriers.
  raw px[ROWS][VPT], pr[ROWS][RESID ? VPT : 1];
  auto issue = [&](int64_t g, bool live) {
    const int64_t row0 = g * rows_per_group + (int64_t)gm.team * ROWS;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const bool rv = live && row0 + r < M;
      const int64_t row = ph.row(row0 + r);
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int v = gm.t + k * gm.tt;
        if constexpr (!PART) {
          px[r][k] = A::zero();
          if (RESID) pr[r][k] = A::zero();
        }
        if constexpr (PART) { // every slot loads (see RowPhase::load_row and own)
          const int64_t rl = ph.load_row(row0 + r, rv);
          const int64_t o = ph.win(v < nacc ? v : nacc - 1);
          px[r][k] = A::ld_once(X + rl * a.ldx + o);
          if (RESID) pr[r][k] = A::ld_once(Rr + rl * a.ldr + o);
        } else if (rv && v < nacc) {
          px[r][k] = A::ld_once(X + row * a.ldx + (int64_t)v * E);
          if (RESID) pr[r][k] = A::ld_once(Rr + row * a.ldr + (int64_t)v * E);
        }
      }
    }
  };
  int slot = 0;
  const GroupRange gr = group_range(M, rows_per_group, a.blocked, ph.bid, ph.nb);
  int64_t g = gr.first;
  issue(g, g < gr.end);
#pragma unroll
  for (int k = 0; k < VPT; ++k)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      settle(w[k][e]);
      settle(b[k][e]);
    }
  for (; g < gr.end; g += gr.step) {
    const int64_t row0 = g * rows_per_group + (int64_t)gm.team * ROWS;
    float x[ROWS][VPT][E];
    {
      raw rx[ROWS][VPT];
      raw rr[ROWS][RESID ? VPT : 1];
#pragma unroll
      for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
          rx[r][k] = px[r][k];
          if (RESID) rr[r][k] = pr[r][k];
        }
      issue(g + gr.step, g + gr.step < gr.end);
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const bool rv = row0 + r < M;
        const int64_t hbase = ph.row(row0 + r) * a.ldh;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
          A::unpack(rx[r][k], x[r][k]);
          if (RESID) {
            // h = R + X in fp32, rounded once to the storage type; the norm sees the rounded h
            float f[E];
            A::unpack(rr[r][k], f);
#pragma unroll
            for (int e = 0; e < E; ++e) f[e] += x[r][k][e];
            const raw hp = A::pack(f);
            A::unpack(hp, x[r][k]);
            const int v = gm.t + k * gm.tt;
            if (rv && v < nacc) A::st(H + hbase + ph.win(v), hp);
          }
        }
      }
    }

    // Statistics. LayerNorm: a first pass gives mean1; a second pass sums d = x - mean1 and
    // d^2. x - mean1 is exact for rows whose values sit near their mean, so sum(d)/N is an
    // accurate correction even when |mean| >> std and mean1 itself is off by many fp32 ulps of
    // the variance scale; the normalised value is formed as (x - mean1) - delta.
    float mean1[ROWS], delta[ROWS], rstd[ROWS];
    if (a.layernorm) {
      float s[ROWS];
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k)
#pragma unroll
          for (int e = 0; e < E; ++e) {
            if constexpr (PART) acc = __builtin_fmaf(x[r][k][e], own[k][e], acc);
            else acc += x[r][k][e];
          }
        s[r] = acc;
      }
      team_sum<ROWS, (WAVE ? 1 : LB / 64)>(s, red, slot, gm.waves, gm.wave0, gm.wave, gm.lane);
      slot ^= 1;
#pragma unroll
      for (int r = 0; r < ROWS; ++r) mean1[r] = mul_rn(s[r], a.inv_n);
      float qc[2 * ROWS];
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        float q = 0.0f, c = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
          const bool in = gm.t + k * gm.tt < nacc;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            float d;
            if constexpr (PART) d = (x[r][k][e] - mean1[r]) * own[k][e];
            else d = in ? x[r][k][e] - mean1[r] : 0.0f;
            q += d * d;
            c += d;
          }
        }
        qc[r] = q;
        qc[ROWS + r] = c;
      }
      team_sum<2 * ROWS, (WAVE ? 1 : LB / 64)>(qc, red, slot, gm.waves, gm.wave0, gm.wave, gm.lane);
      slot ^= 1;
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        delta[r] = qc[ROWS + r] * a.inv_n;
        const float var = clamp_var(qc[r] * a.inv_n - delta[r] * delta[r]);
        rstd[r] = rsqrt_f32(var + a.eps);
      }
    } else {
      float q[ROWS];
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k)
#pragma unroll
          for (int e = 0; e < E; ++e) {
            if constexpr (PART) acc += (x[r][k][e] * own[k][e]) * x[r][k][e];
            else acc += x[r][k][e] * x[r][k][e];
          }
        q[r] = acc;
      }
      team_sum<ROWS, (WAVE ? 1 : LB / 64)>(q, red, slot, gm.waves, gm.wave0, gm.wave, gm.lane);
      slot ^= 1;
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        mean1[r] = 0.0f;
        delta[r] = 0.0f;
        rstd[r] = rsqrt_f32(q[r] * a.inv_n + a.eps);
      }
    }

#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      if (row0 + r >= M) continue;
      const int64_t row = ph.row(row0 + r);
      const int64_t ybase = row * a.ldy;
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int v = gm.t + k * gm.tt;
        if (Y && v < nacc) { // no Y: the statistics-only pass
          float y[E];
#pragma unroll
          for (int e = 0; e < E; ++e)
            y[e] = ((x[r][k][e] - mean1[r]) - delta[r]) * rstd[r] * w[k][e] + b[k][e];
          A::st(Y + ybase + ph.win(v), A::pack(y));
        }
      }
      if (gm.t == 0) {
        if (a.mean) a.mean[row] = mean1[r] + delta[r];
        if (a.rstd) a.rstd[row] = rstd[r];
      }
    }
  }
}

// ---- backward -----------------------------------------------------------------------------

// Per element: unpack x, dY (and W once per row group), d = x - m, g = dY * W, the row sums;
// after the team sum, with per-row constants a = rstd, nd = -delta * rstd,
// B = -rstd * c2, C = -rstd * c1: xhat = d * a + nd, dX = g * a + (xhat * B + C), and the
// dW / dB column sums. d, g and dY stay in registers across the team sum when the thread holds
// at most 16 elements of the row group (KEEP; else they are formed again from the packed data).
//
// Software pipeline ([P1] para. 12, done with registers): the next row group's X, dY and
// saved statistics are requested before the current group is reduced and written.
//
// CLAMP (the RMSNorm kernels): every load is unconditional, from an address clamped into the
// tensor (rows past M read row M - 1, columns past the row's end its last access); rows past M
// are never stored or summed into dW / dB, and columns past the row's end are masked to zero
// where unpacked. Otherwise (LayerNorm) loads past the row's end or past M are skipped and the
// registers hold zeros. Both give the same results; they were measured on MI355X and each kind
// keeps the faster one (RMSNorm 32768 x 4096: 141.0 -> 135.7 us, residual 65536 x 7168: 518 ->
// 474 us with CLAMP; LayerNorm 16384 x 4096: 76.1 us without it, 81.5 us with it).
template <typename T, typename TW, int EV, int VPT, int ROWS, int LB, bool WAVE, bool LN,
          bool PART = false, bool CLAMP = !LN && !PART>
__global__ __launch_bounds__(LB) void team_bwd_kernel(BwdArgs a, int team_threads) {
  using A = Acc<T, EV>;
  using raw = typename A::raw;
  constexpr int E = A::EPV;
  constexpr int MAXW = WAVE ? 1 : LB / 64;
  constexpr bool KEEP = VPT * ROWS * E <= 16;
  __shared__ __align__(16) float red[RED_FLOATS];
  __shared__ float merge[MERGE_FLOATS];
  const TeamGeom gm = team_geom<WAVE>(team_threads);
  const RowPhase<E, PART> ph(a.nacc, a.M, a.N, a.period, a.phase0, a.dphase);
  const int nacc = ph.nal;
  const int64_t M = ph.Mv; // rows walked below are indices among this workgroup's rows
  const int64_t N = a.N;
  const T *__restrict__ X = static_cast<const T *>(a.x);
  const T *__restrict__ DY = static_cast<const T *>(a.dy);
  const T *__restrict__ DH = static_cast<const T *>(a.dh);
  const TW *__restrict__ W = static_cast<const TW *>(a.w);
  T *__restrict__ DX = static_cast<T *>(a.dx);
  T *__restrict__ DR = static_cast<T *>(a.dr);
  const bool have_stats = a.rstd != nullptr;
  write_ws_header(a.header, a.partials, N);

  // the weight stays in its storage format (half the registers for bf16), unpacked at use
  WAcc<T, TW, EV> rw[VPT];
  float accw[VPT][E], accb[LN ? VPT : 1][E];
  float own[PART ? VPT : 1][E]; // see RowPhase::own
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int v = gm.t + k * gm.tt;
    if constexpr (PART) {
#pragma unroll
      for (int e = 0; e < E; ++e) own[k][e] = ph.own(v, e);
    }
    rw[k].zero();
    if constexpr (PART) { // the class's columns (once per workgroup)
      ph.gather(rw[k], W, v);
    } else if (v < nacc) {
      rw[k].load(W + (int64_t)v * E);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      accw[k][e] = 0.0f;
      if constexpr (LN) accb[k][e] = 0.0f;
    }
  }

  const int64_t rows_per_group = (int64_t)gm.teams * ROWS;
  // X, dY and the saved statistics of row group g into one register set
  auto issue = [&](raw (&px)[ROWS][VPT], raw (&pdy)[ROWS][VPT], float (&pm)[ROWS],
                   float (&pr)[ROWS], int64_t g, bool live) {
    const int64_t row0 = g * rows_per_group + (int64_t)gm.team * ROWS;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const bool rv = live && row0 + r < M;
      const int64_t rowc = PART ? ph.load_row(row0 + r, rv) : (rv ? row0 + r : M - 1);
      pm[r] = 0.0f;
      pr[r] = 0.0f;
      if (have_stats) {
        if constexpr (LN) pm[r] = a.mean[rowc];
        pr[r] = a.rstd[rowc];
      }
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int v = gm.t + k * gm.tt;
        if constexpr (PART) { // every slot loads (see RowPhase::load_row and own)
          const int64_t o = ph.win(v < nacc ? v : nacc - 1);
          px[r][k] = A::ld_once(X + rowc * a.ldx + o);
          pdy[r][k] = A::ld_once(DY + rowc * a.lddy + o);
        } else if constexpr (CLAMP) {
          const int64_t off = (int64_t)(v < nacc ? v : nacc - 1) * E;
          px[r][k] = A::ld_once(X + rowc * a.ldx + off);
          pdy[r][k] = A::ld_once(DY + rowc * a.lddy + off);
        } else {
          px[r][k] = A::zero();
          pdy[r][k] = A::zero();
          if (rv && v < nacc) {
            px[r][k] = A::ld_once(X + rowc * a.ldx + (int64_t)v * E);
            pdy[r][k] = A::ld_once(DY + rowc * a.lddy + (int64_t)v * E);
          }
        }
      }
    }
  };
  // the raw access k of a set, zero for columns past the row's end (CLAMP loads hold the last
  // access there; the others already hold zeros)
  auto masked = [&](raw v, int k) {
    if constexpr (CLAMP) return gm.t + k * gm.tt < nacc ? v : A::zero();
    else return v;
  };
  int slot = 0;

  // One row group from its register set.
  auto process = [&](raw (&rx)[ROWS][VPT], raw (&rdy)[ROWS][VPT], const float (&sm)[ROWS],
                     const float (&sr)[ROWS], int64_t g) {
    const int64_t row0 = g * rows_per_group + (int64_t)gm.team * ROWS;
    // m: the row mean the forward saved (LayerNorm), or a first-pass mean when recomputing.
    // The reduction below also sums x - m, so the exact mean m + delta is used for xhat.
    float m[ROWS], rstd[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      m[r] = sm[r];
      rstd[r] = sr[r];
    }
    if (!have_stats) {
      // recompute the forward statistics from the register-resident rows
      if constexpr (LN) {
        float s[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          float acc = 0.0f;
#pragma unroll
          for (int k = 0; k < VPT; ++k) {
            float f[E];
            A::unpack(masked(rx[r][k], k), f);
#pragma unroll
            for (int e = 0; e < E; ++e) {
              if constexpr (PART) acc = __builtin_fmaf(f[e], own[k][e], acc);
              else acc += f[e];
            }
          }
          s[r] = acc;
        }
        team_sum<ROWS, MAXW>(s, red, slot, gm.waves, gm.wave0, gm.wave, gm.lane);
        slot ^= 1;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) m[r] = mul_rn(s[r], a.inv_n);
        float qc[2 * ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          float q = 0.0f, c = 0.0f;
#pragma unroll
          for (int k = 0; k < VPT; ++k) {
            if (gm.t + k * gm.tt < nacc) { // columns past the row end add nothing
              float f[E];
              A::unpack(masked(rx[r][k], k), f);
#pragma unroll
              for (int e = 0; e < E; ++e) {
                float d = f[e] - m[r];
                if constexpr (PART) d *= own[k][e];
                q = __builtin_fmaf(d, d, q);
                c += d;
              }
            }
          }
          qc[r] = q;
          qc[ROWS + r] = c;
        }
        team_sum<2 * ROWS, MAXW>(qc, red, slot, gm.waves, gm.wave0, gm.wave, gm.lane);
        slot ^= 1;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          const float dl = qc[ROWS + r] * a.inv_n;
          rstd[r] = rsqrt_f32(clamp_var(qc[r] * a.inv_n - dl * dl) + a.eps);
        }
      } else {
        float q[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          float acc = 0.0f;
#pragma unroll
          for (int k = 0; k < VPT; ++k) {
            float f[E];
            A::unpack(masked(rx[r][k], k), f);
#pragma unroll
            for (int e = 0; e < E; ++e) {
              if constexpr (PART) acc = __builtin_fmaf(f[e] * own[k][e], f[e], acc);
              else acc = __builtin_fmaf(f[e], f[e], acc);
            }
          }
          q[r] = acc;
        }
        team_sum<ROWS, MAXW>(q, red, slot, gm.waves, gm.wave0, gm.wave, gm.lane);
        slot ^= 1;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          m[r] = 0.0f;
          rstd[r] = rsqrt_f32(q[r] * a.inv_n + a.eps);
        }
      }
    }

    // One team sum per row group. With g = dY * W and d = x - m:
    //   LayerNorm: S0 = sum(g*d), S1 = sum(g), S2 = sum(d); delta = S2/N,
    //              c1 = S1/N, c2 = rstd * (S0 - delta*S1)/N  (= mean(g * xhat))
    //   RMSNorm  : S0 = sum(g*x), c2 = rstd * S0/N
    constexpr int NV = LN ? 3 * ROWS : ROWS;
    float sums[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) sums[i] = 0.0f;
    float kd[KEEP ? ROWS : 1][KEEP ? VPT : 1][E], kg[KEEP ? ROWS : 1][KEEP ? VPT : 1][E],
        kdy[KEEP ? ROWS : 1][KEEP ? VPT : 1][E];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      float wf[E];
      rw[k].get(wf);
      const bool in = gm.t + k * gm.tt < nacc;
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        float xf[E], df[E];
        A::unpack(masked(rx[r][k], k), xf);
        A::unpack(masked(rdy[r][k], k), df);
        float d[E], gg[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          d[e] = LN ? xf[e] - m[r] : xf[e];
          gg[e] = df[e] * wf[e];
          // columns past N hold x = dY = 0: g * d adds nothing there
          const float gs = PART ? gg[e] * own[k][e] : gg[e];
          sums[r] = __builtin_fmaf(gs, d[e], sums[r]);
          if constexpr (LN) sums[ROWS + r] += gs;
        }
        if constexpr (LN) {
          if constexpr (PART) {
#pragma unroll
            for (int e = 0; e < E; ++e)
              sums[2 * ROWS + r] = __builtin_fmaf(d[e], own[k][e], sums[2 * ROWS + r]);
          } else if (in) {
#pragma unroll
            for (int e = 0; e < E; ++e) sums[2 * ROWS + r] += d[e];
          }
        }
        if constexpr (KEEP) {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            kd[KEEP ? r : 0][KEEP ? k : 0][e] = d[e];
            kg[KEEP ? r : 0][KEEP ? k : 0][e] = gg[e];
            kdy[KEEP ? r : 0][KEEP ? k : 0][e] = df[e];
          }
        }
      }
    }
    team_sum<NV, MAXW>(sums, red, slot, gm.waves, gm.wave0, gm.wave, gm.lane);
    slot ^= 1;

#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      if (row0 + r >= M) continue; // rows past M add nothing to dW / dB and write nothing
      const int64_t row = ph.row(row0 + r);
      const float delta = LN ? sums[2 * ROWS + r] * a.inv_n : 0.0f;
      const float c1 = LN ? sums[ROWS + r] * a.inv_n : 0.0f;
      const float c2 =
          LN ? rstd[r] * (sums[r] - delta * sums[ROWS + r]) * a.inv_n : rstd[r] * sums[r] * a.inv_n;
      const float ra = rstd[r], nd = -delta * rstd[r];
      const float cB = -rstd[r] * c2, cC = -rstd[r] * c1;
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int v = gm.t + k * gm.tt;
        if (v >= nacc) continue; // columns past N: nothing to add or write
        float d[E], gg[E], df[E];
        if constexpr (KEEP) {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            d[e] = kd[KEEP ? r : 0][KEEP ? k : 0][e];
            gg[e] = kg[KEEP ? r : 0][KEEP ? k : 0][e];
            df[e] = kdy[KEEP ? r : 0][KEEP ? k : 0][e];
          }
        } else {
          float xf[E], wf[E];
          A::unpack(masked(rx[r][k], k), xf);
          A::unpack(masked(rdy[r][k], k), df);
          rw[k].get(wf);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            d[e] = LN ? xf[e] - m[r] : xf[e];
            gg[e] = df[e] * wf[e];
          }
        }
        float dx[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float xh = __builtin_fmaf(d[e], ra, nd);
          dx[e] = __builtin_fmaf(gg[e], ra, __builtin_fmaf(xh, cB, cC));
          const float dfs = PART ? df[e] * own[k][e] : df[e];
          accw[k][e] = __builtin_fmaf(dfs, xh, accw[k][e]);
          if constexpr (LN) accb[k][e] += dfs;
        }
        const int64_t off = ph.win(v);
        if (DH) {
          float hf[E];
          A::unpack(A::ld_once(DH + row * a.lddh + off), hf);
#pragma unroll
          for (int e = 0; e < E; ++e) dx[e] += hf[e];
        }
        const raw p = A::pack(dx);
        A::st(DX + row * a.lddx + off, p);
        if (DR) A::st(DR + row * a.lddr + off, p);
      }
    }
  };

  const GroupRange gr = group_range(M, rows_per_group, a.blocked, ph.bid, ph.nb);
  raw px[ROWS][VPT], pdy[ROWS][VPT];
  float pm[ROWS], pr[ROWS];
  int64_t g = gr.first;
  issue(px, pdy, pm, pr, g, g < gr.end);
#pragma unroll
  for (int k = 0; k < VPT; ++k) rw[k].settle();
  for (; g < gr.end; g += gr.step) {
    raw rx[ROWS][VPT], rdy[ROWS][VPT];
    float cm[ROWS], cr[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      cm[r] = pm[r];
      cr[r] = pr[r];
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        rx[r][k] = px[r][k];
        rdy[r][k] = pdy[r][k];
      }
    }
    issue(px, pdy, pm, pr, g + gr.step, g + gr.step < gr.end);
    process(rx, rdy, cm, cr, g);
  }

  // Column partials of this workgroup: sum over its teams (fixed order) and write one row
  // per quantity into the workspace.
  float *pw = a.colpart + (int64_t)blockIdx.x * N;
  float *pb = a.colpart + ((int64_t)a.partials + blockIdx.x) * N;
  if (gm.teams == 1) {
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int v = gm.t + k * gm.tt;
      if (v < nacc) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (PART && own[k][e] == 0.0f) continue; // the neighbouring access writes it
          pw[ph.win(v) + e] = accw[k][e];
          if constexpr (LN) pb[ph.win(v) + e] = accb[k][e];
        }
      }
    }
    return;
  }
  const int cols_per_block = MERGE_FLOATS / gm.teams;
  for (int q = 0; q < (LN ? 2 : 1); ++q) {
    float *dst = q == 0 ? pw : pb;
    for (int64_t c0 = 0; c0 < N; c0 += cols_per_block) {
      const int64_t c1 = c0 + cols_per_block < N ? c0 + cols_per_block : N;
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int v = gm.t + k * gm.tt;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int64_t col = ph.win(v) + e;
          if (v < nacc && col >= c0 && col < c1 && !(PART && own[k][e] == 0.0f))
            merge[gm.team * cols_per_block + (int)(col - c0)] =
                q == 0 ? accw[k][e] : accb[LN ? k : 0][e];
        }
      }
      __syncthreads();
      for (int64_t col = c0 + threadIdx.x; col < c1; col += blockDim.x) {
        float s = 0.0f;
        for (int tm = 0; tm < gm.teams; ++tm) s += merge[tm * cols_per_block + (int)(col - c0)];
        dst[col] = s;
      }
      __syncthreads();
    }
  }
}

// ---- launch helpers ---------------------------------------------------------------------------

template <typename T, typename TW, int EV, int VPT, int ROWS, int LB, bool WAVE>
hipError_t fwd_launch(const Plan &p, const FwdArgs &a, bool resid, hipStream_t s) {
  dim3 grid((unsigned)p.grid), block((unsigned)p.threads);
  if constexpr (EV == full_epv<T>()) { // rows in phase classes only at the full width
    if (a.period) {
      if (resid)
        return launch(team_fwd_kernel<T, TW, EV, VPT, ROWS, LB, WAVE, true, true>, grid, block,
                      s, a, p.team_threads);
      return launch(team_fwd_kernel<T, TW, EV, VPT, ROWS, LB, WAVE, false, true>, grid, block, s,
                    a, p.team_threads);
    }
  }
  if (resid)
    return launch(team_fwd_kernel<T, TW, EV, VPT, ROWS, LB, WAVE, true>, grid, block, s, a,
                  p.team_threads);
  return launch(team_fwd_kernel<T, TW, EV, VPT, ROWS, LB, WAVE, false>, grid, block, s, a,
                p.team_threads);
}

template <typename T, typename TW, int EV, int VPT, int ROWS, int LB, bool WAVE>
hipError_t bwd_launch(const Plan &p, const BwdArgs &a, hipStream_t s) {
  dim3 grid((unsigned)p.grid), block((unsigned)p.threads);
  if constexpr (EV == full_epv<T>()) {
    if (a.period) {
      if (a.layernorm)
        return launch(team_bwd_kernel<T, TW, EV, VPT, ROWS, LB, WAVE, true, true>, grid, block, s,
                      a, p.team_threads);
      return launch(team_bwd_kernel<T, TW, EV, VPT, ROWS, LB, WAVE, false, true>, grid, block, s,
                    a, p.team_threads);
    }
  }
  if (a.layernorm)
    return launch(team_bwd_kernel<T, TW, EV, VPT, ROWS, LB, WAVE, true>, grid, block, s, a,
                  p.team_threads);
  return launch(team_bwd_kernel<T, TW, EV, VPT, ROWS, LB, WAVE, false>, grid, block, s, a,
                p.team_threads);
}

} // namespace dln
