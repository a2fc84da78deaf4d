// norm_team.hip -- the column reduction of the backward's partials, a zero fill, and the
// team kernels' dispatch by storage type.
//
// The team kernels (norm_team_kernels.hpp) hold a row per team of threads in registers; each
// storage combination's shapes are instantiated in its own translation unit
// (norm_team_<type>.hip, from the menus in norm_team_menu.hpp).
#include "norm_team_kernels.hpp"

namespace dln {

// ---- column reduction ------------------------------------------------------------------------

// dW[j] (and dB[j]) = sum over p of colpart[q][p][j] (blockIdx.y: 0 = dW, 1 = dB) in a fixed
// order for a given partial count P, which comes from the header the fused pass wrote (a
// header that does not describe this workspace gives NaN outputs instead of reading past the
// partials). Few partial rows (P <= kNarrowP): every thread owns its columns and adds the P
// rows in ascending order. Otherwise a tile of columns is shared by slices of the partial
// rows: slice s adds rows s, s + S, ... in ascending order, then the S slice sums of a column
// are added in slice order. Workgroups stride over the column tiles, so the grid stays small
// for very long rows.
constexpr int64_t kNarrowP = 32;

template <typename T> __device__ __forceinline__ void store_col(void *dst, int64_t col, float t) {
  T *d = static_cast<T *>(dst);
  if constexpr (sizeof(T) == 4)
    d[col] = t;
  else if constexpr (__is_same(T, f16_t))
    d[col] = (f16_t)t;
  else
    d[col] = (T)(pack_bf16x2(t, 0.0f) & 0xffffu);
}

struct ColsumSrc {
  const float *src;
  int64_t P;
  bool valid;
};
__device__ __forceinline__ ColsumSrc colsum_src(const ReduceArgs &a) {
  const int64_t P = a.header[1];
  const bool valid =
      a.header[0] == kWsMagic && a.header[2] == a.N && P >= 1 && P <= a.max_partials;
  return ColsumSrc{a.colpart + (int64_t)blockIdx.y * (valid ? P : 0) * a.N, P, valid};
}

// Element-wise version (any N): wide tiles are 64 columns x 4 slices.
template <typename T>
__global__ __launch_bounds__(256) void colsum_kernel(ReduceArgs a) {
  __shared__ float part[4][64];
  const int64_t N = a.N;
  const ColsumSrc c = colsum_src(a);
  void *dst = blockIdx.y == 0 ? a.dw : a.db;
  if (!c.valid || c.P <= kNarrowP) {
    for (int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x; col < N;
         col += (int64_t)gridDim.x * 256) {
      float s = 0.0f;
      for (int64_t p = 0; c.valid && p < c.P; ++p) s += c.src[p * N + col];
      store_col<T>(dst, col, c.valid ? s : __builtin_nanf(""));
    }
    return;
  }
  const int lane = threadIdx.x & 63;
  const int slice = threadIdx.x >> 6;
  for (int64_t tile = blockIdx.x; tile * 64 < N; tile += gridDim.x) {
    const int64_t col = tile * 64 + lane;
    float s = 0.0f;
    if (col < N) {
      int64_t p = slice;
      for (; p + 12 < c.P; p += 16) {
        const float v0 = c.src[p * N + col];
        const float v1 = c.src[(p + 4) * N + col];
        const float v2 = c.src[(p + 8) * N + col];
        const float v3 = c.src[(p + 12) * N + col];
        s += v0;
        s += v1;
        s += v2;
        s += v3;
      }
      for (; p < c.P; p += 4) s += c.src[p * N + col];
    }
    part[slice][lane] = s;
    __syncthreads();
    if (slice == 0 && col < N)
      store_col<T>(dst, col, (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]));
    __syncthreads();
  }
}

// 16-byte version for N % 4 == 0 (every partial row is then 16-byte aligned): wide tiles are
// 32 columns (8 quads) x 32 slices.
template <typename T>
__global__ __launch_bounds__(256) void colsum4_kernel(ReduceArgs a) {
  __shared__ float part[32][33];
  const int64_t N = a.N;
  const ColsumSrc c = colsum_src(a);
  void *dst = blockIdx.y == 0 ? a.dw : a.db;
  if (!c.valid || c.P <= kNarrowP) {
    for (int64_t col0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; col0 < N;
         col0 += (int64_t)gridDim.x * 1024) {
      float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
      for (int64_t p = 0; c.valid && p < c.P; ++p) {
        const float4 v = *reinterpret_cast<const float4 *>(c.src + p * N + col0);
        s0 += v.x;
        s1 += v.y;
        s2 += v.z;
        s3 += v.w;
      }
      if (!c.valid) s0 = s1 = s2 = s3 = __builtin_nanf("");
      store_col<T>(dst, col0, s0);
      store_col<T>(dst, col0 + 1, s1);
      store_col<T>(dst, col0 + 2, s2);
      store_col<T>(dst, col0 + 3, s3);
    }
    return;
  }
  const int q = threadIdx.x & 7;
  const int slice = threadIdx.x >> 3;
  for (int64_t tile = blockIdx.x; tile * 32 < N; tile += gridDim.x) {
    const int64_t col0 = tile * 32 + q * 4;
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
    if (col0 < N) {
      int64_t p = slice;
      for (; p + 96 < c.P; p += 128) {
        const float4 v0 = *reinterpret_cast<const float4 *>(c.src + p * N + col0);
        const float4 v1 = *reinterpret_cast<const float4 *>(c.src + (p + 32) * N + col0);
        const float4 v2 = *reinterpret_cast<const float4 *>(c.src + (p + 64) * N + col0);
        const float4 v3 = *reinterpret_cast<const float4 *>(c.src + (p + 96) * N + col0);
        s0 += v0.x; s1 += v0.y; s2 += v0.z; s3 += v0.w;
        s0 += v1.x; s1 += v1.y; s2 += v1.z; s3 += v1.w;
        s0 += v2.x; s1 += v2.y; s2 += v2.z; s3 += v2.w;
        s0 += v3.x; s1 += v3.y; s2 += v3.z; s3 += v3.w;
      }
      for (; p < c.P; p += 32) {
        const float4 v = *reinterpret_cast<const float4 *>(c.src + p * N + col0);
        s0 += v.x; s1 += v.y; s2 += v.z; s3 += v.w;
      }
    }
    part[slice][q * 4 + 0] = s0;
    part[slice][q * 4 + 1] = s1;
    part[slice][q * 4 + 2] = s2;
    part[slice][q * 4 + 3] = s3;
    __syncthreads();
    if (threadIdx.x < 32) {
      const int64_t col = tile * 32 + threadIdx.x;
      float t = 0.0f;
      for (int sl = 0; sl < 32; ++sl) t += part[sl][threadIdx.x];
      if (col < N) store_col<T>(dst, col, t);
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void zero_kernel(unsigned char *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// ---- launchers ---------------------------------------------------------------------------------

norm_status_t launch_team_fwd(const Plan &p, norm_dtype_t dtype, const FwdArgs &a,
                              hipStream_t s) {
  switch (dtype) {
  case NORM_F32: return launch_team_fwd_f32(p, a, s);
  case NORM_BF16: return launch_team_fwd_bf16(p, a, s);
  case NORM_BF16_F32W: return launch_team_fwd_bf16w(p, a, s);
  case NORM_F16: return launch_team_fwd_f16(p, a, s);
  case NORM_F16_F32W: return launch_team_fwd_f16w(p, a, s);
  default: return NORM_ERR_UNSUPPORTED;
  }
}

norm_status_t launch_team_bwd(const Plan &p, norm_dtype_t dtype, const BwdArgs &a,
                              hipStream_t s) {
  switch (dtype) {
  case NORM_F32: return launch_team_bwd_f32(p, a, s);
  case NORM_BF16: return launch_team_bwd_bf16(p, a, s);
  case NORM_BF16_F32W: return launch_team_bwd_bf16w(p, a, s);
  case NORM_F16: return launch_team_bwd_f16(p, a, s);
  case NORM_F16_F32W: return launch_team_bwd_f16w(p, a, s);
  default: return NORM_ERR_UNSUPPORTED;
  }
}

norm_status_t launch_zero(void *p, size_t bytes, hipStream_t s) {
  if (!bytes) return NORM_OK;
  size_t blocks = (bytes + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  const hipError_t e = launch(zero_kernel, dim3((unsigned)blocks), dim3(256), s,
                              static_cast<unsigned char *>(p), bytes);
  return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

norm_status_t launch_reduce(norm_dtype_t dtype, const ReduceArgs &a, hipStream_t s) {
  // one workgroup per wide tile up to kReduceGrid workgroups per quantity; they stride beyond
  constexpr int64_t kReduceGrid = 2048;
  const unsigned q = a.db ? 2u : 1u;
  hipError_t e;
  if (a.N % 4 == 0) {
    const int64_t tiles = (a.N + 31) / 32;
    const dim3 grid((unsigned)(tiles < kReduceGrid ? tiles : kReduceGrid), q), block(256);
    // dW, dB are stored like W: bf16, fp16 or fp32
    e = dtype == NORM_BF16  ? launch(colsum4_kernel<bf16_bits>, grid, block, s, a)
        : dtype == NORM_F16 ? launch(colsum4_kernel<f16_t>, grid, block, s, a)
                            : launch(colsum4_kernel<float>, grid, block, s, a);
  } else {
    const int64_t tiles = (a.N + 63) / 64;
    const dim3 grid((unsigned)(tiles < kReduceGrid ? tiles : kReduceGrid), q), block(256);
    e = dtype == NORM_BF16  ? launch(colsum_kernel<bf16_bits>, grid, block, s, a)
        : dtype == NORM_F16 ? launch(colsum_kernel<f16_t>, grid, block, s, a)
                            : launch(colsum_kernel<float>, grid, block, s, a);
  }
  return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

} // namespace dln
