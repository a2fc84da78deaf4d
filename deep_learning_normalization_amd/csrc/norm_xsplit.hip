// norm_xsplit.hip -- the split-row scheme in a single pass over the data ("exchange" form).
//
// Rows too long for one workgroup are cut into chunks, as in norm_split.hip, but every chunk
// stays in its workgroup's registers from load to output: the workgroups that share a row swap
// their chunk partials through the workspace instead of re-reading the row in a second pass.
// X (and dY) cross HBM once, which is the traffic of the single-workgroup schemes.
//
//   grid      G row groups x C chunks. Workgroup (g, c) owns column chunk c (its weight and
//             bias stay in registers) and walks rows g, g + G, g + 2G, ...; it publishes row
//             r + G's partials before it waits for row r's, with row r + 2G's loads in flight.
//   exchange  per (row, chunk) eight 64-bit words: each fp32 partial goes out as a pair of
//             words, (tag, value) and (~tag, value), where tag is a 32-bit number drawn for the
//             call. A partial counts as published once both words of its pair carry this call's
//             tag (and its complement) around the same value, so words left by earlier calls
//             (other tags) or by whatever the memory held before (which would have to match 64
//             bits of pattern) never pass, and no call needs the words cleared first. Words are
//             written and read with relaxed atomics at agent scope, which the compiler makes
//             coherent across the XCDs' separate L2s; each pair validates itself, so no fence
//             orders anything. Tags come from a process-wide counter; a call captured into a
//             HIP graph replays with its tag fixed, so under capture the launcher clears the
//             words with a kernel first (no memset, so replays start clean).
//   progress  workgroup (g, c) only waits for the other C - 1 workgroups of row group g, whose
//             ids are adjacent to its own. The plan keeps the grid within what the device holds
//             at once (G * C <= resident workgroups), so on an otherwise idle device every
//             workgroup of a group is running while the others wait. Neither HIP nor the
//             hardware promises that (dispatch order is not guaranteed, and other work may hold
//             compute units), so the wait is bounded: after a set number of polls (2^19 by
//             default, a second or so) the workgroup gives up, writes NaN for the row, stops
//             waiting for later rows and sets the workspace header's exchange-failure word
//             (reported by norm_workspace_status): a broken assumption shows up as NaN outputs
//             and a status, never as a hang.
//
// Method (web page "PyTorch atinge desempenho SOTA em normalização com torch.compile",
// matsubara.tec.br): para. 6, very large shapes as a regression class; paras. 8-10, the split
// reduction with a workspace of partial sums and no atomics in the arithmetic. The page
// "Towards Free Normalization: Fusing Normalization into GEMM and Attention Kernels"
// (brifing.si), item 4: one row's norm spread over several thread blocks (multi-CTA). The
// chunk combination is the parallel-variance one: the row mean from the chunk means, the
// squared deviation from the chunk sums plus count * (chunk mean - row mean)^2.
#include <atomic>
#include <chrono>
#include <random>

#include "norm_device.hpp"
#include "norm_internal.hpp"

namespace dln {
namespace {

constexpr int XLB = 256;                // threads per workgroup
constexpr int XMAXCH = 2;               // chunks per thread in the exchange (C <= 512)
constexpr int kWordsPerChunk = kXchgWordsPerChunk;
static_assert(kXchgMaxChunks <= (int64_t)XLB * XMAXCH, "the plan admits more chunks than a "
                                                        "workgroup gathers");
static_assert(kWordsPerChunk >= 2 * 3, "a word pair for each of up to three partials");

// Partial q of a chunk: the word pair at 2q, 2q + 1.
__device__ __forceinline__ void publish(uint64_t *p, float v, uint32_t tag) {
  const uint64_t bits = (uint64_t)__builtin_bit_cast(unsigned, v);
  __hip_atomic_store(p, ((uint64_t)tag << 32) | bits, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(p + 1, ((uint64_t)(~tag) << 32) | bits, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t peek(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Whether the pair (a, b) was published by this call (tag): a carries the tag, b its
// complement, both the same value. Sets v to the value.
__device__ __forceinline__ int pair_valid(uint64_t a, uint64_t b, uint32_t tag, float &v) {
  v = __builtin_bit_cast(float, (unsigned)(a & 0xffffffffull));
  return (int)((uint32_t)(a >> 32) == tag) & (int)((uint32_t)(b >> 32) == ~tag) &
         (int)((uint32_t)a == (uint32_t)b);
}

// Wait until the NQ partials of every chunk of one row (xp: the row's words) are published and
// return this thread's chunks tid + XLB * j in v[j] (zeros past C), plus chunk 0's first
// partial in v0. Every thread of the workgroup calls it. Returns false, with NaN in every value,
// once a wait has given up after `polls` polls (`failed` then stays set and later calls return
// at once); the first give-up of a workgroup also sets the exchange-failure word `err`.
template <int NQ>
__device__ bool gather_row(const uint64_t *xp, int64_t C, unsigned polls, uint32_t tag,
                           uint64_t *err, float (&v)[XMAXCH][NQ], float &v0, bool &failed) {
  const int tid = threadIdx.x;
  if (!failed) {
    for (unsigned spin = 0;; ++spin) {
      int ok = pair_valid(peek(xp), peek(xp + 1), tag, v0);
#pragma unroll
      for (int j = 0; j < XMAXCH; ++j) {
        const int64_t cc = tid + (int64_t)j * XLB;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          v[j][q] = 0.0f;
          if (cc < C) {
            const uint64_t *w = xp + cc * kWordsPerChunk + 2 * q;
            ok &= pair_valid(peek(w), peek(w + 1), tag, v[j][q]);
          }
        }
      }
      if (__syncthreads_and(ok)) return true;
      if (spin + 1 >= polls) break;
      __builtin_amdgcn_s_sleep(4);
    }
    failed = true;
    if (tid == 0 && err)
      __hip_atomic_store(err, kXchgFailWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const float nan = __builtin_nanf("");
  v0 = nan;
#pragma unroll
  for (int j = 0; j < XMAXCH; ++j)
#pragma unroll
    for (int q = 0; q < NQ; ++q) v[j][q] = nan;
  return false;
}

// ---- forward -------------------------------------------------------------------------------

// Chunk partials (published as words 0..2):
//   LayerNorm: chunk mean m_c, sum (x - m_c)^2, sum (x - m_c)
//   RMSNorm  : sum x^2
// Two rows are in hand at a time: the partials of row r + G are published before the wait for
// row r's, so the wait overlaps the other workgroups' progress on row r; the inputs of row
// r + 2G are in flight meanwhile.
//
// The weight and bias of the chunk live in LDS when they are stored like the activations (16
// bytes per access; each thread reads only its own slots, so no barrier guards them): that
// frees 32 VGPRs and lets 4 workgroups share a CU. fp32 weights beside 16-bit activations
// (32 bytes per access) would need 64 KB of LDS per workgroup and stay in registers, 3 per CU.
template <typename T, typename TW, int EV> constexpr bool fwd_weights_in_lds() {
  return sizeof(WAcc<T, TW, EV>) <= 16;
}

template <typename T, typename TW, int EV, int VPT, bool LN>
__global__ __launch_bounds__(XLB, (fwd_weights_in_lds<T, TW, EV>() ? kXchgFwdPerCuLds
                                                                     : kXchgFwdPerCu))
void xsplit_fwd_kernel(FwdArgs a) {
  using A = Acc<T, EV>;
  using raw = typename A::raw;
  constexpr int E = A::EPV;
  constexpr int NQ = LN ? 3 : 1;
  __shared__ __align__(16) float red[RED_FLOATS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, waves = XLB / 64;
  const int64_t C = a.chunks, G = a.xgroups, M = a.M;
  const int64_t g = (int64_t)blockIdx.x / C;
  const int64_t c = (int64_t)blockIdx.x - g * C;
  const int64_t acc0 = c * a.chunk_acc;
  const int64_t left = (int64_t)a.nacc - acc0;
  const int nin = (int)(left < a.chunk_acc ? left : a.chunk_acc);
  const int64_t col0 = acc0 * E;
  const float n_c = (float)(nin * E);
  const T *__restrict__ X = static_cast<const T *>(a.x) + col0;
  T *__restrict__ Y = static_cast<T *>(a.y) + col0;
  const TW *__restrict__ W = static_cast<const TW *>(a.w) + col0;
  const TW *__restrict__ Bb = a.b ? static_cast<const TW *>(a.b) + col0 : nullptr;

  constexpr bool WL = fwd_weights_in_lds<T, TW, EV>();
  using WA = WAcc<T, TW, EV>;
  __shared__ WA lw[WL ? VPT : 1][WL ? XLB : 1], lb[WL ? VPT : 1][WL ? XLB : 1];
  WA rw[WL ? 1 : VPT], rb[WL ? 1 : VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int v = tid + k * XLB;
    WA w, b;
    w.zero();
    b.zero();
    if (v < nin) {
      w.load(W + (int64_t)v * E);
      if (Bb) b.load(Bb + (int64_t)v * E);
    }
    if constexpr (WL) {
      lw[k][tid] = w;
      lb[k][tid] = b;
    } else {
      rw[k] = w;
      rb[k] = b;
    }
  }
  raw px[VPT], ra[VPT], rn[VPT];
  auto issue = [&](int64_t row) {
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int v = tid + k * XLB;
      px[k] = A::zero();
      if (row < M && v < nin) px[k] = A::ld(X + row * a.ldx + (int64_t)v * E);
    }
  };
  int slot = 0;
  // this chunk's partials of one row (accesses past the chunk's end hold zeros), published
  auto publish_partials = [&](raw (&r)[VPT], int64_t row) {
    uint64_t *xc = a.xpart + (row * C + c) * kWordsPerChunk;
    if constexpr (LN) {
      float s[1] = {0.0f};
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        float xf[E];
        A::unpack(r[k], xf);
#pragma unroll
        for (int e = 0; e < E; ++e) s[0] += xf[e];
      }
      team_sum<1, XLB / 64>(s, red, slot, waves, 0, wave, lane);
      slot ^= 1;
#pragma unroll
      for (int k = 0; k < VPT; ++k) settle(r[k]);
      const float mc = s[0] / n_c;
      float qc[2] = {0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const bool in = tid + k * XLB < nin;
        float xf[E];
        A::unpack(r[k], xf);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float d = in ? xf[e] - mc : 0.0f;
          qc[0] += d * d;
          qc[1] += d;
        }
      }
      team_sum<2, XLB / 64>(qc, red, slot, waves, 0, wave, lane);
      slot ^= 1;
      if (tid == 0 && !(a.withhold && c == 0)) {
        publish(xc + 0, mc, a.tag);
        publish(xc + 2, qc[0], a.tag);
        publish(xc + 4, qc[1], a.tag);
      }
    } else {
      float q[1] = {0.0f};
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        float xf[E];
        A::unpack(r[k], xf);
#pragma unroll
        for (int e = 0; e < E; ++e) q[0] += xf[e] * xf[e];
      }
      team_sum<1, XLB / 64>(q, red, slot, waves, 0, wave, lane);
      slot ^= 1;
      if (tid == 0 && !(a.withhold && c == 0)) publish(xc, q[0], a.tag);
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) settle(r[k]);
  };

  issue(g); // g < M: the plan makes G at most M
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    if constexpr (!WL) {
      rw[k].settle();
      rb[k].settle();
    }
    ra[k] = px[k];
  }
  issue(g + G);
  publish_partials(ra, g);
  bool failed = false;
  for (int64_t row = g; row < M; row += G) {
    const int64_t next = row + G;
#pragma unroll
    for (int k = 0; k < VPT; ++k) rn[k] = px[k];
    issue(next + G);
    if (next < M) publish_partials(rn, next);

    // the row's statistics from every chunk's partials, in chunk order per thread, then the
    // team sum (a fixed order; the two-pass form combines in the same order with the same
    // terms, ln_chunk_terms, so both forms give the same bits)
    float pv[XMAXCH][NQ], m0;
    gather_row<NQ>(a.xpart + row * C * kWordsPerChunk, C, a.polls, a.tag, a.xerr, pv, m0,
                   failed);
#pragma unroll
    for (int k = 0; k < VPT; ++k) settle(ra[k]);
    float shift = 0.0f, delta = 0.0f, rstd;
    if constexpr (LN) {
      shift = m0;
      float ab[2] = {0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < XMAXCH; ++j) {
        const int64_t cc = tid + (int64_t)j * XLB;
        if (cc < C)
          ln_chunk_terms(split_chunk_elems(cc, a.chunk_acc, a.nacc, E), pv[j][0], pv[j][1],
                         pv[j][2], shift, ab[0], ab[1]);
      }
      team_sum<2, XLB / 64>(ab, red, slot, waves, 0, wave, lane);
      slot ^= 1;
      rstd = ln_combined_rstd(ab[0], ab[1], a.inv_n, a.eps, delta);
    } else {
      float q[1] = {0.0f};
#pragma unroll
      for (int j = 0; j < XMAXCH; ++j) q[0] += pv[j][0];
      team_sum<1, XLB / 64>(q, red, slot, waves, 0, wave, lane);
      slot ^= 1;
      rstd = rsqrt_f32(q[0] * a.inv_n + a.eps);
    }

    // normalise the chunk held in registers
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int v = tid + k * XLB;
      if (v < nin) {
        float xf[E], wf[E], bf[E], y[E];
        A::unpack(ra[k], xf);
        if constexpr (WL) {
          lw[k][tid].get(wf);
          lb[k][tid].get(bf);
        } else {
          rw[k].get(wf);
          rb[k].get(bf);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) y[e] = ((xf[e] - shift) - delta) * rstd * wf[e] + bf[e];
        A::st(Y + row * a.ldy + (int64_t)v * E, A::pack(y));
      }
    }
    if (c == 0 && tid == 0) {
      if (a.mean) a.mean[row] = shift + delta;
      if (a.rstd) a.rstd[row] = rstd;
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) ra[k] = rn[k];
  }
}

// ---- backward ------------------------------------------------------------------------------

// Chunk partials, around the row's saved mean m:
//   LayerNorm: sum g*(x - m), sum g, sum (x - m)    (g = dY * w)
//   RMSNorm  : sum g*x
// After the exchange each workgroup writes dX for its chunk from registers and keeps the
// chunk's dW (and dB) column sums over its rows; they are written once at the end as partial
// row g (or as the final dW/dB when there is one row group). Rows are pipelined as in the
// forward: row r + G's partials are published before the wait for row r's. The dB sums live
// in LDS (each thread owns one column of it, so no barrier guards them), which leaves the
// registers for three rows of X and dY.
template <typename T, typename TW, int EV, int VPT, bool LN>
__global__ __launch_bounds__(XLB, kXchgBwdPerCu) void xsplit_bwd_kernel(BwdArgs a) {
  using A = Acc<T, EV>;
  using raw = typename A::raw;
  constexpr int E = A::EPV;
  constexpr int NQ = LN ? 3 : 1;
  __shared__ __align__(16) float red[RED_FLOATS];
  // dB sums, 16-byte LDS accesses: elements 4h .. 4h + 3 of access k of thread t at
  // sdb[k * (E / 4) + h][t]
  static_assert(E % 4 == 0, "16-byte accesses of 2- or 4-byte elements");
  constexpr int E4 = E / 4;
  __shared__ float4 sdb[LN ? VPT * E4 : 1][XLB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, waves = XLB / 64;
  const int64_t C = a.chunks, G = a.row_groups, M = a.M;
  const int64_t g = (int64_t)blockIdx.x / C;
  const int64_t c = (int64_t)blockIdx.x - g * C;
  const int64_t acc0 = c * a.chunk_acc;
  const int64_t left = (int64_t)a.nacc - acc0;
  const int nin = (int)(left < a.chunk_acc ? left : a.chunk_acc);
  const int64_t col0 = acc0 * E;
  const int64_t N = a.N;
  const T *__restrict__ X = static_cast<const T *>(a.x) + col0;
  const T *__restrict__ DY = static_cast<const T *>(a.dy) + col0;
  const T *__restrict__ DH = a.dh ? static_cast<const T *>(a.dh) + col0 : nullptr;
  const TW *__restrict__ W = static_cast<const TW *>(a.w) + col0;
  T *__restrict__ DX = static_cast<T *>(a.dx) + col0;
  T *__restrict__ DR = a.dr ? static_cast<T *>(a.dr) + col0 : nullptr;
  if (!a.dw) write_ws_header(a.header, G, N);

  WAcc<T, TW, EV> rw[VPT];
  float accw[VPT][E];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int v = tid + k * XLB;
    rw[k].zero();
    if (v < nin) rw[k].load(W + (int64_t)v * E);
#pragma unroll
    for (int e = 0; e < E; ++e) accw[k][e] = 0.0f;
    if constexpr (LN) {
#pragma unroll
      for (int h = 0; h < E4; ++h) sdb[k * E4 + h][tid] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  }
  // px/pdy: in flight; xa/dya: the row being finished; xn/dyn: the next row (published)
  raw px[VPT], pdy[VPT], xa[VPT], dya[VPT], xn[VPT], dyn[VPT];
  float pm = 0.0f, prs = 0.0f, ma, rsa, mn, rsn;
  auto issue = [&](int64_t row) {
    const bool rv = row < M;
    const int64_t rowc = rv ? row : M - 1;
    pm = LN ? a.mean[rowc] : 0.0f;
    prs = a.rstd[rowc];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int v = tid + k * XLB;
      px[k] = A::zero();
      pdy[k] = A::zero();
      if (rv && v < nin) {
        px[k] = A::ld(X + row * a.ldx + (int64_t)v * E);
        pdy[k] = A::ld(DY + row * a.lddy + (int64_t)v * E);
      }
    }
  };
  int slot = 0;
  auto publish_partials = [&](raw (&rx)[VPT], raw (&rdy)[VPT], float m, int64_t row) {
    float sums[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) sums[q] = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const bool in = tid + k * XLB < nin;
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
    team_sum<NQ, XLB / 64>(sums, red, slot, waves, 0, wave, lane);
    slot ^= 1;
    if (tid == 0 && !(a.withhold && c == 0)) {
      uint64_t *xc = a.xpart + (row * C + c) * kWordsPerChunk;
#pragma unroll
      for (int q = 0; q < NQ; ++q) publish(xc + 2 * q, sums[q], a.tag);
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      settle(rx[k]);
      settle(rdy[k]);
    }
  };

  issue(g); // g < M: the plan makes G at most M
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    rw[k].settle();
    xa[k] = px[k];
    dya[k] = pdy[k];
  }
  ma = pm;
  rsa = prs;
  issue(g + G);
  publish_partials(xa, dya, ma, g);
  bool failed = false;
  for (int64_t row = g; row < M; row += G) {
    const int64_t next = row + G;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      xn[k] = px[k];
      dyn[k] = pdy[k];
    }
    mn = pm;
    rsn = prs;
    issue(next + G);
    if (next < M) publish_partials(xn, dyn, mn, next);

    float pv[XMAXCH][NQ], unused;
    gather_row<NQ>(a.xpart + row * C * kWordsPerChunk, C, a.polls, a.tag, a.xerr, pv, unused,
                   failed);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      settle(xa[k]);
      settle(dya[k]);
    }
    float tot[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < XMAXCH; ++j) s += pv[j][q];
      tot[q] = s;
    }
    team_sum<NQ, XLB / 64>(tot, red, slot, waves, 0, wave, lane);
    slot ^= 1;
    const float m = ma, rstd = rsa;
    const float delta = LN ? tot[2] * a.inv_n : 0.0f;
    const float c1 = LN ? tot[1] * a.inv_n : 0.0f;
    const float c2 = LN ? rstd * (tot[0] - delta * tot[1]) * a.inv_n : rstd * tot[0] * a.inv_n;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int v = tid + k * XLB;
      const bool in = v < nin;
      float xf[E], df[E], wf[E], dx[E];
      A::unpack(xa[k], xf);
      A::unpack(dya[k], df);
      rw[k].get(wf);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float xh = in ? ((xf[e] - m) - delta) * rstd : 0.0f;
        dx[e] = rstd * (df[e] * wf[e] - c1 - xh * c2);
        accw[k][e] += df[e] * xh;
      }
      if constexpr (LN) {
#pragma unroll
        for (int h = 0; h < E4; ++h) {
          float4 b = sdb[k * E4 + h][tid];
          b.x += df[4 * h];
          b.y += df[4 * h + 1];
          b.z += df[4 * h + 2];
          b.w += df[4 * h + 3];
          sdb[k * E4 + h][tid] = b;
        }
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
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      xa[k] = xn[k];
      dya[k] = dyn[k];
    }
    ma = mn;
    rsa = rsn;
  }
  // a wait that gave up poisons the column sums too (RMSNorm's dW does not depend on the
  // exchanged values and would otherwise come out finite)
  if (failed) {
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
#pragma unroll
      for (int e = 0; e < E; ++e) accw[k][e] = nan;
      if constexpr (LN) {
#pragma unroll
        for (int h = 0; h < E4; ++h) sdb[k * E4 + h][tid] = make_float4(nan, nan, nan, nan);
      }
    }
  }
  if (a.dw) {
    TW *dw = static_cast<TW *>(a.dw) + col0;
    TW *db = a.db ? static_cast<TW *>(a.db) + col0 : nullptr;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int v = tid + k * XLB;
      if (v < nin) {
        WAcc<T, TW, EV>::store(dw + (int64_t)v * E, accw[k]);
        if constexpr (LN) {
          float bsum[E];
#pragma unroll
          for (int h = 0; h < E4; ++h) {
            const float4 b = sdb[k * E4 + h][tid];
            bsum[4 * h] = b.x;
            bsum[4 * h + 1] = b.y;
            bsum[4 * h + 2] = b.z;
            bsum[4 * h + 3] = b.w;
          }
          if (db) WAcc<T, TW, EV>::store(db + (int64_t)v * E, bsum);
        }
      }
    }
  } else {
    float *pw = a.colpart + g * N + col0;
    float *pb = a.colpart + (G + g) * N + col0;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int v = tid + k * XLB;
      if (v < nin) {
#pragma unroll
        for (int e = 0; e < E; ++e) pw[(int64_t)v * E + e] = accw[k][e];
        if constexpr (LN) {
#pragma unroll
          for (int h = 0; h < E4; ++h) {
            const float4 b = sdb[k * E4 + h][tid];
            pb[(int64_t)v * E + 4 * h] = b.x;
            pb[(int64_t)v * E + 4 * h + 1] = b.y;
            pb[(int64_t)v * E + 4 * h + 2] = b.z;
            pb[(int64_t)v * E + 4 * h + 3] = b.w;
          }
        }
      }
    }
  }
}

// ---- launchers -------------------------------------------------------------------------------

// Clears n exchange words, with the same agent-scope stores that publish them; run only before
// a call captured into a HIP graph, whose replays reuse one tag. One kernel name per pass, so
// that profiles attribute it.
__device__ __forceinline__ void clear_n(uint64_t *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    __hip_atomic_store(p + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__global__ __launch_bounds__(256) void xclear_fwd_kernel(uint64_t *p, int64_t n) { clear_n(p, n); }
__global__ __launch_bounds__(256) void xclear_bwd_kernel(uint64_t *p, int64_t n) { clear_n(p, n); }

// Whether work queued on s now is being captured into a graph. A stream the runtime cannot
// answer for counts as captured (the clear is then merely redundant); the error that query
// leaves is consumed so that the caller's next error check does not see it.
bool capturing(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return true;
  }
  return cs != hipStreamCaptureStatusNone;
}

norm_status_t clear_words(uint64_t *words, int64_t M, int64_t C, bool bwd, hipStream_t s) {
  if (!capturing(s)) return NORM_OK; // eager calls: a fresh tag makes every old word stale
  const int64_t n = M * C * kWordsPerChunk;
  const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  const hipError_t e = launch(bwd ? xclear_bwd_kernel : xclear_fwd_kernel,
                              dim3((unsigned)blocks), dim3(256), s, words, n);
  return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

// Resident workgroups per CU of one kernel, asked of the runtime once per process (every
// device of a process is the same gfx950 part).
template <typename K> int resident_per_cu(K kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, XLB, 0) != hipSuccess) n = 0;
  return n;
}

template <typename T, typename TW, bool LN> int fwd_resident() {
  static const int n = resident_per_cu(xsplit_fwd_kernel<T, TW, full_epv<T>(), 4, LN>);
  return n;
}
template <typename T, typename TW, bool LN> int bwd_resident() {
  static const int n = resident_per_cu(xsplit_bwd_kernel<T, TW, full_epv<T>(), 4, LN>);
  return n;
}

template <typename T, typename TW>
norm_status_t xfwd_typed(const Plan &p, const FwdArgs &a, hipStream_t s) {
  constexpr int F = full_epv<T>();
  const int need = fwd_weights_in_lds<T, TW, F>() ? kXchgFwdPerCuLds : kXchgFwdPerCu;
  const int have = a.layernorm ? fwd_resident<T, TW, true>() : fwd_resident<T, TW, false>();
  if (have < need) return NORM_ERR_UNSUPPORTED;
  norm_status_t st = clear_words(a.xpart, a.M, a.chunks, false, s);
  if (st != NORM_OK) return st;
  const dim3 grid((unsigned)(a.xgroups * a.chunks)), block(XLB);
  const hipError_t e = a.layernorm
                           ? launch(xsplit_fwd_kernel<T, TW, F, 4, true>, grid, block, s, a)
                           : launch(xsplit_fwd_kernel<T, TW, F, 4, false>, grid, block, s, a);
  return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

template <typename T, typename TW>
norm_status_t xbwd_typed(const BwdArgs &a, hipStream_t s) {
  constexpr int F = full_epv<T>();
  const int need = (int)kXchgBwdPerCu;
  const int have = a.layernorm ? bwd_resident<T, TW, true>() : bwd_resident<T, TW, false>();
  if (have < need) return NORM_ERR_UNSUPPORTED;
  norm_status_t st = clear_words(a.xpart, a.M, a.chunks, true, s);
  if (st != NORM_OK) return st;
  const dim3 grid((unsigned)(a.row_groups * a.chunks)), block(XLB);
  const hipError_t e = a.layernorm
                           ? launch(xsplit_bwd_kernel<T, TW, F, 4, true>, grid, block, s, a)
                           : launch(xsplit_bwd_kernel<T, TW, F, 4, false>, grid, block, s, a);
  return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

} // namespace

uint32_t next_exchange_tag() {
  static std::atomic<uint32_t> counter{[] {
    std::random_device rd;
    return (uint32_t)rd() ^ (uint32_t)std::chrono::steady_clock::now().time_since_epoch().count();
  }()};
  for (;;) {
    const uint32_t t = counter.fetch_add(1, std::memory_order_relaxed);
    if (t != 0u && t != ~0u) return t;
  }
}

bool xsplit_ready(norm_dtype_t dtype, bool layernorm, bool bwd) {
  const int need = bwd ? (int)kXchgBwdPerCu : xchg_fwd_per_cu(dtype);
  int have = 0;
#define DLN_XR(T, TW)                                                                           \
  have = bwd ? (layernorm ? bwd_resident<T, TW, true>() : bwd_resident<T, TW, false>())          \
             : (layernorm ? fwd_resident<T, TW, true>() : fwd_resident<T, TW, false>());
  switch (dtype) {
  case NORM_F32: DLN_XR(float, float) break;
  case NORM_BF16: DLN_XR(bf16_bits, bf16_bits) break;
  case NORM_BF16_F32W: DLN_XR(bf16_bits, float) break;
  case NORM_F16: DLN_XR(f16_t, f16_t) break;
  case NORM_F16_F32W: DLN_XR(f16_t, float) break;
  default: return false;
  }
#undef DLN_XR
  return have >= need;
}

norm_status_t launch_xsplit_fwd(const Plan &p, norm_dtype_t dtype, const FwdArgs &a,
                                hipStream_t s) {
  switch (dtype) {
  case NORM_F32: return xfwd_typed<float, float>(p, a, s);
  case NORM_BF16: return xfwd_typed<bf16_bits, bf16_bits>(p, a, s);
  case NORM_BF16_F32W: return xfwd_typed<bf16_bits, float>(p, a, s);
  case NORM_F16: return xfwd_typed<f16_t, f16_t>(p, a, s);
  case NORM_F16_F32W: return xfwd_typed<f16_t, float>(p, a, s);
  default: return NORM_ERR_UNSUPPORTED;
  }
}

norm_status_t launch_xsplit_bwd(norm_dtype_t dtype, const BwdArgs &a, hipStream_t s) {
  switch (dtype) {
  case NORM_F32: return xbwd_typed<float, float>(a, s);
  case NORM_BF16: return xbwd_typed<bf16_bits, bf16_bits>(a, s);
  case NORM_BF16_F32W: return xbwd_typed<bf16_bits, float>(a, s);
  case NORM_F16: return xbwd_typed<f16_t, f16_t>(a, s);
  case NORM_F16_F32W: return xbwd_typed<f16_t, float>(a, s);
  default: return NORM_ERR_UNSUPPORTED;
  }
}

} // namespace dln
