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
// The product: 256 x 256 output tiles, 512 threads (eight wavefronts, 2 x 4, each 128 rows by
// 64 columns as 4 x 2 MFMA 32x32x16 bf16 blocks with fp32 accumulators), K in steps of 64
// staged through double-buffered LDS. Each wavefront reads the operands of the next 16-wide
// step from LDS while the current one multiplies; one barrier per 64-wide step; the global
// loads of a step are issued a full step before they are written to LDS.
#include "norm_device.hpp"
#include "norm_lazy.hpp"

namespace dln {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTM = kLazyTile, kTN = kLazyTile, kTK = 64;
constexpr int kThreads = 512;
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
__global__ __launch_bounds__(kThreads, 1) void lazy_linear_kernel(LazyArgs a) {
  __shared__ __align__(16) uint16_t sx[2][kTM * kLdsRow];
  __shared__ __align__(16) uint16_t sg[2][kTN * kLdsRow];
  __shared__ __align__(16) float s_mean[kTM], s_rstd[kTM], s_s[kTN], s_t[kTN];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, a.tiles_m, a.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kTM, n0 = (int64_t)tn * kTN;
  const int64_t M = a.M, N = a.N, K = a.K;

  // Loader: thread t stages 16-byte chunk (t & 7) of rows (t >> 3) + 64q, q = 0..3, of both
  // operand tiles; 8 consecutive lanes cover one 128-byte row segment. Rows past the end of X
  // or G read the last row instead (their products land in outputs that are not stored), and
  // a chunk past K reads the last chunk and is staged as zeros. Addresses are the tile's first
  // row plus a 32-bit byte offset per lane (row strides below 2^23 elements).
  const int lrow = t >> 3, lk = (t & 7) * 8;
  const char *xbase = reinterpret_cast<const char *>(a.x + m0 * a.ldx);
  const char *gbase = reinterpret_cast<const char *>(a.g + n0 * a.ldg);
  uint32_t xo[4], go[4];
  float sh[4], s1[4], s2[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t rx = min((int64_t)(lrow + 64 * q), M - 1 - m0);
    const int64_t rg = min((int64_t)(lrow + 64 * q), N - 1 - n0);
    xo[q] = (uint32_t)(rx * a.ldx * 2);
    go[q] = (uint32_t)(rg * a.ldg * 2);
    // LayerNorm sums are shifted by the row's first element (exact in fp32), which keeps the
    // one-pass variance free of cancellation for rows far from zero mean
    sh[q] = (LN && !STATS_IN) ? bf16_lo(*reinterpret_cast<const uint16_t *>(xbase + xo[q]))
                              : 0.0f;
    s1[q] = 0.0f;
    s2[q] = 0.0f;
  }

  uint4 rx[4], rg[4];
  auto gload = [&](int64_t k0) {
    const uint32_t c = (uint32_t)min((int64_t)lk, K - 8 - k0) * 2;
    const char *xk = xbase + k0 * 2, *gk = gbase + k0 * 2;
#pragma unroll
    for (int q = 0; q < 4; ++q) rx[q] = *reinterpret_cast<const uint4 *>(xk + (xo[q] + c));
#pragma unroll
    for (int q = 0; q < 4; ++q) rg[q] = *reinterpret_cast<const uint4 *>(gk + (go[q] + c));
  };
  auto stage = [&](int buf, int64_t k0) {
    // a chunk past K is staged as zeros (a mask, not a branch, around the loaded values)
    const bool in_k = k0 + lk < K;
    const unsigned keep = in_k ? ~0u : 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 vx = make_uint4(rx[q].x & keep, rx[q].y & keep, rx[q].z & keep, rx[q].w & keep);
      const uint4 vg = make_uint4(rg[q].x & keep, rg[q].y & keep, rg[q].z & keep, rg[q].w & keep);
      *reinterpret_cast<uint4 *>(&sx[buf][(lrow + 64 * q) * kLdsRow + lk]) = vx;
      *reinterpret_cast<uint4 *>(&sg[buf][(lrow + 64 * q) * kLdsRow + lk]) = vg;
    }
    if constexpr (!STATS_IN) {
      if (in_k) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const unsigned w[4] = {rx[q].x, rx[q].y, rx[q].z, rx[q].w};
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

  // acc[j][i]: the 32 x 32 block of G rows (output columns) j and X rows i of this wavefront,
  // computed as G X^T so that each lane holds one output row: register r of lane l is row
  // l % 32 of the block and column 8 * (r / 4) + 4 * (l / 32) + r % 4.
  f32x16_t acc[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

  // MFMA operands: lane l supplies row (l & 31) of its 32-row block and the 8 values of K at
  // 8 * (l >> 5) within the 16-wide step, for the A (rows of G) and B (rows of X) operands.
  bf16x8_t fx[2][4], fg[2][2];
  const int xrow = (wm * 128 + (lane & 31)) * kLdsRow + (lane >> 5) * 8;
  const int grow = (wn * 64 + (lane & 31)) * kLdsRow + (lane >> 5) * 8;
  auto frags = [&](int set, int buf, int ks) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fx[set][i] = *reinterpret_cast<const bf16x8_t *>(&sx[buf][xrow + i * 32 * kLdsRow + ks * 16]);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      fg[set][j] = *reinterpret_cast<const bf16x8_t *>(&sg[buf][grow + j * 32 * kLdsRow + ks * 16]);
  };
  auto mma = [&](int set) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fg[set][j], fx[set][i], acc[j][i],
                                                            0, 0, 0);
  };

  const int nk = (int)((K + kTK - 1) / kTK);
  gload(0);
  stage(0, 0);
  gload((int64_t)min(1, nk - 1) * kTK);
  __syncthreads();
  frags(0, 0, 0);
  // Every step but the last: step kt + 1 goes from registers into the other buffer (last read
  // before the previous barrier) and the loads of step kt + 2 are issued (the last step again
  // past the end: in bounds, never staged); the first operands of step kt + 1 are read while
  // the last 16-wide part of step kt multiplies. The last step runs outside the loop, so the
  // operands read at the end of an iteration are used on every path out of it.
  for (int kt = 0; kt + 1 < nk; ++kt) {
    const int b = kt & 1;
    frags(1, b, 1);
    mma(0);
    frags(0, b, 2);
    mma(1);
    frags(1, b, 3);
    mma(0);
    stage(b ^ 1, (int64_t)(kt + 1) * kTK);
    gload((int64_t)min(kt + 2, nk - 1) * kTK);
    __syncthreads();
    frags(0, b ^ 1, 0);
    mma(1);
  }
  {
    const int b = (nk - 1) & 1;
    frags(1, b, 1);
    mma(0);
    frags(0, b, 2);
    mma(1);
    frags(1, b, 3);
    mma(0);
    mma(1);
  }

  // Row statistics of the tile, and s and t of its columns, into LDS.
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
        const int r = lrow + 64 * q;
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
  if (t < kTN) {
    const int64_t col = n0 + t;
    s_s[t] = (LN && col < N) ? a.s[col] : 0.0f;
    s_t[t] = (a.t && col < N) ? a.t[col] : 0.0f;
  }
  __syncthreads();

  // Epilogue: out = rstd * (acc - mean * s) + t, one RNE rounding to bf16; four consecutive
  // columns of one row per store (8 bytes where Y's rows allow it).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = wm * 128 + i * 32 + (lane & 31);
    const int64_t row = m0 + rl;
    if (row >= M) continue;
    const float mean = s_mean[rl], rstd = s_rstd[rl];
    uint16_t *yrow = a.y + row * a.ldy;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int cl = wn * 64 + j * 32 + g * 8 + (lane >> 5) * 4;
        const int64_t col = n0 + cl;
        const float4 sv = *reinterpret_cast<const float4 *>(&s_s[cl]);
        const float4 tv = *reinterpret_cast<const float4 *>(&s_t[cl]);
        const float sc[4] = {sv.x, sv.y, sv.z, sv.w}, tc[4] = {tv.x, tv.y, tv.z, tv.w};
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float p = acc[j][i][g * 4 + c];
          v[c] = __builtin_fmaf(rstd, LN ? p - mean * sc[c] : p, tc[c]);
        }
        if (a.vec_store && col + 3 < N) {
          *reinterpret_cast<uint2 *>(yrow + col) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (col + c < N) yrow[col + c] = (uint16_t)(pack_bf16x2(v[c], 0.0f) & 0xffffu);
        }
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
