// norm_looped.hip -- backward for rows too long for a team to hold X and dY in registers, but
// short enough that a row of X and dY stays in the L2 between two sweeps over it.
//
// One team (the whole workgroup) owns one row at a time. The row is covered by SEG segments of
// one access per thread. Sweep 1 streams X and dY from HBM and forms the row sums the backward
// needs; one team sum; sweep 2 reads X and dY again (from the L2, which holds the rows the 32
// CUs of an XCD have in flight: about 2 MB for 32 KB rows against 4 MB) and writes dX while
// accumulating the dW / dB column partials in registers. Registers hold only the weight and
// those accumulators across the row, about half of what the register-resident block backward
// holds per element, so a team covers twice the row at the same HBM traffic: X and dY read
// once from HBM, dX written once.
//
// Method (web page "PyTorch atinge desempenho SOTA em normalização com torch.compile",
// matsubara.tec.br): para. 5 -- reductions whose dimension is too large to hold on chip loop over
// it; para. 7 -- the backward's gradients dX, dW, dB; paras. 8-10 -- dX and per-block partial
// column sums from one fused pass, consolidated by a second pass over the partials.
#include <type_traits>

#include "norm_device.hpp"
#include "norm_internal.hpp"

namespace dln {

// Every sweep after the first must load the row again (from the L2): without this compiler
// barrier the loads of the same restrict-qualified addresses are merged with the first sweep's,
// which then holds the whole row in registers across the team sum.
__device__ __forceinline__ void reload_barrier() { asm volatile("" ::: "memory"); }

// DBL: the dB sums live in LDS instead of registers (each thread owns its own columns there, so
// no barrier guards them), which takes the four-segment LayerNorm kernel of 16-bit rows from 158
// to at most 128 VGPRs: two workgroups per CU (the bound's second argument is the wavefronts
// per SIMD it must leave room for).
template <typename T, typename TW, int EV, int SEG, int LB, bool LN, bool DBL = false>
__global__ __launch_bounds__(LB, DBL ? LB / 128 : 1) void looped_bwd_kernel(BwdArgs a) {
  using A = Acc<T, EV>;
  constexpr int E = A::EPV;
  constexpr int MAXW = LB / 64;
  static_assert(!DBL || (LN && E % 4 == 0), "dB in LDS: LayerNorm, whole float4 groups");
  constexpr int E4 = E / 4 > 0 ? E / 4 : 1;
  __shared__ __align__(16) float red[RED_FLOATS];
  // dB sums: elements 4h .. 4h + 3 of segment s of thread t at sdb[s * E4 + h][t]
  __shared__ __align__(16) float4 sdb[DBL ? SEG * E4 : 1][DBL ? LB : 1];
  const int t = threadIdx.x;
  const int tt = blockDim.x;
  const int waves = tt >> 6, wave = t >> 6, lane = t & 63;
  const int nacc = a.nacc;
  const int64_t M = a.M;
  const int64_t N = a.N;
  const T *__restrict__ X = static_cast<const T *>(a.x);
  const T *__restrict__ DY = static_cast<const T *>(a.dy);
  const T *__restrict__ DH = static_cast<const T *>(a.dh);
  const TW *__restrict__ W = static_cast<const TW *>(a.w);
  T *__restrict__ DX = static_cast<T *>(a.dx);
  T *__restrict__ DR = static_cast<T *>(a.dr);
  const bool have_stats = a.rstd != nullptr;
  write_ws_header(a.header, a.partials, N);

  WAcc<T, TW, EV> rw[SEG];
  float accw[SEG][E], accb[(LN && !DBL) ? SEG : 1][E];
#pragma unroll
  for (int s = 0; s < SEG; ++s) {
    const int v = t + s * tt;
    rw[s].zero();
    if (v < nacc) rw[s].load(W + (int64_t)v * E);
    rw[s].settle();
#pragma unroll
    for (int e = 0; e < E; ++e) {
      accw[s][e] = 0.0f;
      if constexpr (LN && !DBL) accb[s][e] = 0.0f;
    }
    if constexpr (DBL) {
#pragma unroll
      for (int h = 0; h < E4; ++h) sdb[s * E4 + h][t] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  }

  int slot = 0;
  for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
    // the row is uniform across the workgroup: scalar row pointers, 32-bit element offsets
    const T *xr = X + row * a.ldx;
    const T *dyr = DY + row * a.lddy;
    float m = 0.0f, rstd = 0.0f;
    if (have_stats) {
      if constexpr (LN) m = a.mean[row];
      rstd = a.rstd[row];
    } else if constexpr (LN) {
      // the forward's statistics, two sweeps: the mean, then the sums around it (as the
      // register-resident kernels form them)
      float s1[1] = {0.0f};
#pragma unroll
      for (int s = 0; s < SEG; ++s) {
        const int v = t + s * tt;
        if (v < nacc) {
          float f[E];
          A::unpack(A::ld(xr + v * E), f);
#pragma unroll
          for (int e = 0; e < E; ++e) s1[0] += f[e];
        }
      }
      team_sum<1, MAXW>(s1, red, slot, waves, 0, wave, lane);
      slot ^= 1;
      m = mul_rn(s1[0], a.inv_n);
      reload_barrier();
      float qc[2] = {0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < SEG; ++s) {
        const int v = t + s * tt;
        if (v < nacc) {
          float f[E];
          A::unpack(A::ld(xr + v * E), f);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float d = f[e] - m;
            qc[0] = __builtin_fmaf(d, d, qc[0]);
            qc[1] += d;
          }
        }
      }
      team_sum<2, MAXW>(qc, red, slot, waves, 0, wave, lane);
      slot ^= 1;
      const float dl = qc[1] * a.inv_n;
      rstd = rsqrt_f32(clamp_var(qc[0] * a.inv_n - dl * dl) + a.eps);
      reload_barrier();
    } else {
      float q[1] = {0.0f};
#pragma unroll
      for (int s = 0; s < SEG; ++s) {
        const int v = t + s * tt;
        if (v < nacc) {
          float f[E];
          A::unpack(A::ld(xr + v * E), f);
#pragma unroll
          for (int e = 0; e < E; ++e) q[0] = __builtin_fmaf(f[e], f[e], q[0]);
        }
      }
      team_sum<1, MAXW>(q, red, slot, waves, 0, wave, lane);
      slot ^= 1;
      rstd = rsqrt_f32(q[0] * a.inv_n + a.eps);
      reload_barrier();
    }

    // Sweep 1. With g = dY * W and d = x - m:
    //   LayerNorm: S0 = sum(g*d), S1 = sum(g), S2 = sum(d); delta = S2/N,
    //              c1 = S1/N, c2 = rstd * (S0 - delta*S1)/N  (= mean(g * xhat))
    //   RMSNorm  : S0 = sum(g*x), c2 = rstd * S0/N
    constexpr int NV = LN ? 3 : 1;
    float sums[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) sums[i] = 0.0f;
#pragma unroll
    for (int s = 0; s < SEG; ++s) {
      const int v = t + s * tt;
      if (v < nacc) {
        float xf[E], df[E], wf[E];
        A::unpack(A::ld(xr + v * E), xf);
        A::unpack(A::ld(dyr + v * E), df);
        rw[s].get(wf);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float d = LN ? xf[e] - m : xf[e];
          const float gg = df[e] * wf[e];
          sums[0] = __builtin_fmaf(gg, d, sums[0]);
          if constexpr (LN) {
            sums[1] += gg;
            sums[2] += d;
          }
        }
      }
    }
    team_sum<NV, MAXW>(sums, red, slot, waves, 0, wave, lane);
    slot ^= 1;
    const float delta = LN ? sums[2] * a.inv_n : 0.0f;
    const float c1 = LN ? sums[1] * a.inv_n : 0.0f;
    const float c2 = LN ? rstd * (sums[0] - delta * sums[1]) * a.inv_n : rstd * sums[0] * a.inv_n;
    const float ra = rstd, nd = -delta * rstd;
    const float cB = -rstd * c2, cC = -rstd * c1;
    reload_barrier();

    // Sweep 2: dX = rstd * (g - c1 - xhat * c2) (+ dH), and the column sums of dY * xhat, dY.
#pragma unroll
    for (int s = 0; s < SEG; ++s) {
      const int v = t + s * tt;
      if (v < nacc) {
        const int off = v * E;
        float xf[E], df[E], wf[E];
        A::unpack(A::ld_cached(xr + off), xf);
        A::unpack(A::ld_cached(dyr + off), df);
        rw[s].get(wf);
        float dx[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float d = LN ? xf[e] - m : xf[e];
          const float xh = __builtin_fmaf(d, ra, nd);
          dx[e] = __builtin_fmaf(df[e] * wf[e], ra, __builtin_fmaf(xh, cB, cC));
          accw[s][e] = __builtin_fmaf(df[e], xh, accw[s][e]);
          if constexpr (LN && !DBL) accb[s][e] += df[e];
        }
        if constexpr (DBL) {
#pragma unroll
          for (int h = 0; h < E4; ++h) {
            float4 b = sdb[s * E4 + h][t];
            b.x += df[4 * h];
            b.y += df[4 * h + 1];
            b.z += df[4 * h + 2];
            b.w += df[4 * h + 3];
            sdb[s * E4 + h][t] = b;
          }
        }
        if (DH) {
          float hf[E];
          A::unpack(A::ld(DH + row * a.lddh + off), hf);
#pragma unroll
          for (int e = 0; e < E; ++e) dx[e] += hf[e];
        }
        const typename A::raw p = A::pack(dx);
        A::st(DX + row * a.lddx + off, p);
        if (DR) A::st(DR + row * a.lddr + off, p);
      }
    }
  }

  // one partial row per quantity for this workgroup
  float *pw = a.colpart + (int64_t)blockIdx.x * N;
  float *pb = a.colpart + ((int64_t)a.partials + blockIdx.x) * N;
#pragma unroll
  for (int s = 0; s < SEG; ++s) {
    const int v = t + s * tt;
    if (v < nacc) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        pw[(int64_t)v * E + e] = accw[s][e];
        if constexpr (LN && !DBL) pb[(int64_t)v * E + e] = accb[s][e];
      }
      if constexpr (DBL) {
#pragma unroll
        for (int h = 0; h < E4; ++h) {
          const float4 b = sdb[s * E4 + h][t];
          pb[(int64_t)v * E + 4 * h] = b.x;
          pb[(int64_t)v * E + 4 * h + 1] = b.y;
          pb[(int64_t)v * E + 4 * h + 2] = b.z;
          pb[(int64_t)v * E + 4 * h + 3] = b.w;
        }
      }
    }
  }
}

namespace {

// Segments per row: 4 full-width (16-byte) accesses per thread, or 8 of 8 bytes; LayerNorm on
// 16-bit rows also has a kernel of 3 full-width segments. Workgroups of up to 512 threads. Two
// workgroups per CU are resident where a kernel takes at most 128 VGPRs (the compiler's report
// for gfx950: 16-byte kernels of fp32 rows 72-93, of RMSNorm on 16-bit rows 124, of LayerNorm
// on 16-bit rows 158 with four segments and 127 with three).
constexpr int kLoopedLB = 512;

template <typename T, typename TW, int EV>
norm_status_t looped_typed(const Plan &p, const BwdArgs &a, hipStream_t s) {
  constexpr int SEG = 4 * (full_epv<T>() / EV);
  constexpr bool kHas3 = EV == full_epv<T>() && sizeof(T) == 2;
  // 16-bit LayerNorm with four full-width segments keeps its dB sums in LDS (the fp16 kernel
  // spills 16 bytes per lane at the 128-VGPR bound, at no measured cost)
  constexpr bool kDbl = EV == full_epv<T>() && sizeof(T) == 2;
  const bool seg3 = kHas3 && a.layernorm && p.vpt == 3;
  if ((p.vpt != SEG && !seg3) || p.lb != kLoopedLB) return NORM_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)p.grid), block((unsigned)p.threads);
  hipError_t e;
  if constexpr (kHas3) {
    if (seg3) {
      e = launch(looped_bwd_kernel<T, TW, EV, 3, kLoopedLB, true>, grid, block, s, a);
      return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
    }
  }
  if constexpr (kDbl) {
    if (a.layernorm) {
      e = launch(looped_bwd_kernel<T, TW, EV, SEG, kLoopedLB, true, true>, grid, block, s, a);
      return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
    }
  }
  e = a.layernorm ? launch(looped_bwd_kernel<T, TW, EV, SEG, kLoopedLB, true>, grid, block, s, a)
                  : launch(looped_bwd_kernel<T, TW, EV, SEG, kLoopedLB, false>, grid, block, s, a);
  return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

template <typename T, typename TW>
norm_status_t looped_width(const Plan &p, const BwdArgs &a, hipStream_t s) {
  constexpr int F = full_epv<T>();
  if (p.epv == F) return looped_typed<T, TW, F>(p, a, s);
  if (p.epv == F / 2) return looped_typed<T, TW, F / 2>(p, a, s);
  return NORM_ERR_UNSUPPORTED; // 4-byte accesses would need 16 segments: they spill
}

} // namespace

norm_status_t launch_looped_bwd(const Plan &p, norm_dtype_t dtype, const BwdArgs &a,
                                hipStream_t s) {
  switch (dtype) {
  case NORM_F32: return looped_width<float, float>(p, a, s);
  case NORM_BF16: return looped_width<bf16_bits, bf16_bits>(p, a, s);
  case NORM_BF16_F32W: return looped_width<bf16_bits, float>(p, a, s);
  case NORM_F16: return looped_width<f16_t, f16_t>(p, a, s);
  case NORM_F16_F32W: return looped_width<f16_t, float>(p, a, s);
  default: return NORM_ERR_UNSUPPORTED;
  }
}

} // namespace dln
