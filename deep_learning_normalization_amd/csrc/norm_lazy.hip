// norm_lazy.hip -- a norm whose output feeds a linear projection, with the normalisation
// deferred to the projection's epilogue.
//
// Method (web page "Towards Free Normalization: Fusing Normalization into GEMM and Attention
// Kernels", brifing.si): items 3-4 -- the norm fused into the matrix product that consumes it
// ("Lazy Pre-Norm", named there without its algebra); items 9-10 -- a row-wise norm wants whole
// rows while a product tiles both of its dimensions, and forcing the norm's tiling on the
// product stops paying as rows grow. Reading taken here: Norm(X) L^T + c equals
// rstd * (X G^T - mean * s) + t with G = L * gamma, s = the row sums of G and t = L beta + c,
// so the product reads the raw X in its own 2-D tiling and each row's statistics enter only
// the epilogue. The statistics are given, or formed from the X tiles the product stages
// anyway: the workgroup that owns a row tile walks all K columns of those rows.
//
// The product: 128 x 128 output tiles, 256 threads (four wavefronts, 2 x 2, each 64 x 64 as
// 2 x 2 MFMA 32x32x16 bf16 blocks with fp32 accumulators), K in steps of 64 staged through
// double-buffered LDS. Global loads of step k+1 are in flight while step k multiplies.
#include "norm_device.hpp"
#include "norm_lazy.hpp"

namespace dln {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTM = 128, kTN = 128, kTK = 64;
constexpr int kThreads = 256;
// bf16 values per staged row: 64 + 8 of padding (144 bytes), so the rows that one 16-byte
// operand read of 32 lanes touches start on distinct LDS bank groups
constexpr int kLdsRow = kTK + 8;
// row tiles visited together: the column tiles of G they share stay in the L2
constexpr int kGroupM = 8;

// The hardware hands consecutive workgroup ids to the eight XCDs in turn. Renumber them so
// that each XCD works through one contiguous range of tiles (its own L2 then holds the rows of
// X and G that range shares), and walk that range in groups of kGroupM row tiles.
__device__ __forceinline__ void tile_of(int bid, int nwg, int tiles_m, int tiles_n, int &tm,
                                        int &tn) {
  if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);
  const int per_group = kGroupM * tiles_n;
  const int first_m = (bid / per_group) * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int r = bid % per_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

__device__ __forceinline__ float wval(uint16_t v) { return bf16_lo(v); }
__device__ __forceinline__ float wval(float v) { return v; }

template <bool LN, bool STATS_IN>
__global__ __launch_bounds__(kThreads, 2) void lazy_linear_kernel(LazyArgs a) {
  __shared__ __align__(16) uint16_t sa[2][kTM * kLdsRow];
  __shared__ __align__(16) uint16_t sb[2][kTN * kLdsRow];
  __shared__ float s_mean[kTM], s_rstd[kTM];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, a.tiles_m, a.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kTM, n0 = (int64_t)tn * kTN;
  const int64_t M = a.M, N = a.N, K = a.K;

  // Loader: thread t stages 16-byte chunk (t & 7) of rows (t >> 3) + 32q, q = 0..3, of both
  // operand tiles; 8 consecutive lanes cover one 128-byte row segment.
  const int lrow = t >> 3, lk = (t & 7) * 8;
  uint4 ra[4], rb[4];
  float sh[4], s1[4], s2[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t row = m0 + lrow + 32 * q;
    // LayerNorm sums are shifted by the row's first element (exact in fp32), which keeps the
    // one-pass variance free of cancellation for rows far from zero mean
    sh[q] = (LN && !STATS_IN && row < M) ? bf16_lo(a.x[row * a.ldx]) : 0.0f;
    s1[q] = 0.0f;
    s2[q] = 0.0f;
  }

  auto load = [&](int64_t k0) {
    const int64_t k = k0 + lk;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t row = m0 + lrow + 32 * q;
      ra[q] = (row < M && k < K) ? *reinterpret_cast<const uint4 *>(a.x + row * a.ldx + k)
                                 : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t col = n0 + lrow + 32 * q;
      rb[q] = (col < N && k < K) ? *reinterpret_cast<const uint4 *>(a.g + col * a.ldg + k)
                                 : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto stage = [&](int buf, int64_t k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<uint4 *>(&sa[buf][(lrow + 32 * q) * kLdsRow + lk]) = ra[q];
      *reinterpret_cast<uint4 *>(&sb[buf][(lrow + 32 * q) * kLdsRow + lk]) = rb[q];
    }
    if constexpr (!STATS_IN) {
      if (k0 + lk < K) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const unsigned w[4] = {ra[q].x, ra[q].y, ra[q].z, ra[q].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float d0 = bf16_lo(w[i]) - sh[q], d1 = bf16_hi(w[i]) - sh[q];
            s1[q] += d0;
            s1[q] += d1;
            s2[q] = __builtin_fmaf(d0, d0, s2[q]);
            s2[q] = __builtin_fmaf(d1, d1, s2[q]);
          }
        }
      }
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (int)((K + kTK - 1) / kTK);
  load(0);
  stage(0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load((int64_t)(kt + 1) * kTK);
    const uint16_t *pa = sa[buf] + (wm * 64 + (lane & 31)) * kLdsRow + (lane >> 5) * 8;
    const uint16_t *pb = sb[buf] + (wn * 64 + (lane & 31)) * kLdsRow + (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < kTK / 16; ++ks) {
      // MFMA operands: lane l supplies row (l & 31) of its 32-row block and the 8 values of K
      // at 8 * (l >> 5) within this 16-wide step, for A (rows of X) and B (rows of G) alike
      bf16x8_t fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = *reinterpret_cast<const bf16x8_t *>(pa + i * 32 * kLdsRow + ks * 16);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const bf16x8_t *>(pb + j * 32 * kLdsRow + ks * 16);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) stage(buf ^ 1, (int64_t)(kt + 1) * kTK);
    __syncthreads();
  }

  // Row statistics of the tile into LDS.
  if constexpr (STATS_IN) {
    if (t < kTM) {
      const int64_t row = m0 + t;
      s_mean[t] = (LN && row < M) ? a.mean_in[row] : 0.0f;
      s_rstd[t] = row < M ? a.rstd_in[row] : 0.0f;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // the 8 lanes of one row, in a fixed order
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) {
        s1[q] += __shfl_xor(s1[q], o);
        s2[q] += __shfl_xor(s2[q], o);
      }
    }
    if ((t & 7) == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = lrow + 32 * q;
        const int64_t row = m0 + r;
        float mean = 0.0f, rstd;
        if constexpr (LN) {
          const float d = s1[q] * a.inv_k;
          mean = sh[q] + d;
          rstd = rsqrt_f32(clamp_var(s2[q] * a.inv_k - d * d) + a.eps);
        } else {
          rstd = rsqrt_f32(s2[q] * a.inv_k + a.eps);
        }
        s_mean[r] = mean;
        s_rstd[r] = rstd;
        if (tn == 0 && row < M) {
          if (LN && a.mean_out) a.mean_out[row] = mean;
          if (a.rstd_out) a.rstd_out[row] = rstd;
        }
      }
    }
  }
  __syncthreads();

  // Epilogue: out = rstd * (acc - mean * s) + t, one RNE rounding to bf16. Accumulator r of
  // a 32x32 block holds row 8 * (r / 4) + 4 * (l / 32) + r % 4 and column l % 32.
  float sv[2], tv[2];
  int64_t col[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    col[j] = n0 + wn * 64 + j * 32 + (lane & 31);
    sv[j] = (LN && col[j] < N) ? a.s[col[j]] : 0.0f;
    tv[j] = (a.t && col[j] < N) ? a.t[col[j]] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      const int64_t row = m0 + rl;
      if (row >= M) continue;
      const float mean = s_mean[rl], rstd = s_rstd[rl];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (col[j] >= N) continue;
        const float p = LN ? acc[i][j][r] - mean * sv[j] : acc[i][j][r];
        const float v = __builtin_fmaf(rstd, p, tv[j]);
        a.y[row * a.ldy + col[j]] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
      }
    }
  }
}

// G = bf16(L * gamma) row by row, with s = the row sums of G as stored and t = L beta + c.
// One workgroup per row j; each thread sums its strided share, then the four wavefronts'
// sums are added in wave order (a fixed order: the same bits on every call).
template <typename TW>
__global__ __launch_bounds__(256) void fold_kernel(FoldArgs a) {
  __shared__ float red[8];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t j = blockIdx.x;
  const uint16_t *L = a.l + j * a.ldl;
  uint16_t *G = a.g + j * a.ldg;
  const TW *gam = static_cast<const TW *>(a.gamma);
  const TW *bet = static_cast<const TW *>(a.beta);
  float ss = 0.0f, tt = 0.0f;
  for (int64_t k = t; k < a.K; k += 256) {
    const float l = bf16_lo(L[k]);
    const unsigned gb = pack_bf16x2(l * wval(gam[k]), 0.0f) & 0xffffu;
    G[k] = (uint16_t)gb;
    ss += bf16_lo(gb);
    if (bet) tt = __builtin_fmaf(wval(bet[k]), l, tt);
  }
  ss = wave_sum(ss);
  tt = wave_sum(tt);
  if (lane == 0) {
    red[wave] = ss;
    red[4 + wave] = tt;
  }
  __syncthreads();
  if (t == 0) {
    if (a.s) a.s[j] = ((red[0] + red[1]) + red[2]) + red[3];
    if (a.t) a.t[j] = ((((red[4] + red[5]) + red[6]) + red[7])) + (a.c ? a.c[j] : 0.0f);
  }
}

} // namespace

norm_status_t launch_fold_projection(bool f32_weights, const FoldArgs &a, int64_t nout,
                                     hipStream_t s) {
  if (nout > 0x7fffffff) return NORM_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)nout), block(256);
  const hipError_t e = f32_weights ? launch(fold_kernel<float>, grid, block, s, a)
                                   : launch(fold_kernel<uint16_t>, grid, block, s, a);
  return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

norm_status_t launch_lazy_linear(bool layernorm, const LazyArgs &a, hipStream_t s) {
  const int64_t wg = (int64_t)a.tiles_m * a.tiles_n;
  // the grid's work-items must be countable in 32 bits
  if (wg <= 0 || wg > 0xffffffffLL / kThreads) return NORM_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)wg), block(kThreads);
  const bool given = a.rstd_in != nullptr;
  hipError_t e;
  if (layernorm)
    e = given ? launch(lazy_linear_kernel<true, true>, grid, block, s, a)
              : launch(lazy_linear_kernel<true, false>, grid, block, s, a);
  else
    e = given ? launch(lazy_linear_kernel<false, true>, grid, block, s, a)
              : launch(lazy_linear_kernel<false, false>, grid, block, s, a);
  return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

} // namespace dln
