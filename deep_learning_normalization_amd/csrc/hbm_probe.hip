// hbm_probe.hip -- streaming probes of HBM bandwidth (read, write, copy, two reads and one
// write, two reads and two writes), the ceilings for the norm passes' stream mixes, and
// matrix-core and LDS read probes, the ceilings for the bf16 products.
//
// Each thread moves `U` 16-byte accesses per stream of one tile (256 threads x U accesses,
// consecutive threads on consecutive 16-byte words, so every wavefront access is 1 KiB
// contiguous); all of a tile's loads are issued before its first store. Stores are nontemporal,
// as in the norm kernels.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "hbm_probe.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <bool NT> __device__ __forceinline__ u32x4 load16(const u32x4 *p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int NIN, int NOUT, int U, bool NT>
__global__ __launch_bounds__(256) void probe_kernel(const u32x4 *__restrict__ a,
                                                    const u32x4 *__restrict__ b,
                                                    u32x4 *__restrict__ c, u32x4 *__restrict__ d,
                                                    int64_t nvec, int64_t ntiles, unsigned key) {
  constexpr int64_t TILE = 256 * U;
  unsigned acc = 0;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t base = tile * TILE + threadIdx.x;
    u32x4 va[U], vb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      va[u] = u32x4{0u, 0u, 0u, 0u};
      vb[u] = u32x4{0u, 0u, 0u, 0u};
      if (i < nvec) {
        if constexpr (NIN >= 1) va[u] = load16<NT>(a + i);
        if constexpr (NIN >= 2) vb[u] = load16<NT>(b + i);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      if (i >= nvec) continue;
      u32x4 r;
      if constexpr (NIN == 0) r = u32x4{key, (unsigned)i, key, (unsigned)i};
      else if constexpr (NIN == 1) r = va[u];
      else r = va[u] ^ vb[u];
      if constexpr (NOUT >= 1) __builtin_nontemporal_store(r, c + i);
      if constexpr (NOUT >= 2) __builtin_nontemporal_store(vb[u], d + i);
      if constexpr (NOUT == 0) acc ^= r.x ^ r.y ^ r.z ^ r.w;
    }
  }
  if constexpr (NOUT == 0) {
    if (acc == key) c[0] = u32x4{acc, acc, acc, acc}; // keeps the loads; practically never taken
  }
}

template <int NIN, int NOUT, int U, bool NT>
hipError_t launch(const void *in0, const void *in1, void *out0, void *out1, int64_t nvec,
                  int64_t grid, unsigned key, hipEvent_t e0, hipEvent_t e1, hipStream_t s) {
  const int64_t ntiles = (nvec + 256 * U - 1) / (256 * U);
  const int64_t g = grid > 0 ? (grid < ntiles ? grid : ntiles) : ntiles;
  const u32x4 *a = static_cast<const u32x4 *>(in0);
  const u32x4 *b = static_cast<const u32x4 *>(in1);
  u32x4 *c = static_cast<u32x4 *>(out0);
  u32x4 *d = static_cast<u32x4 *>(out1);
  void *args[] = {&a, &b, &c, &d, &nvec, const_cast<int64_t *>(&ntiles), &key};
  return hipExtLaunchKernel(reinterpret_cast<const void *>(probe_kernel<NIN, NOUT, U, NT>),
                            dim3((unsigned)g), dim3(256), args, 0, s, e0, e1, 0);
}

template <int NIN, int NOUT>
hipError_t by_shape(int unroll, int nt, const void *in0, const void *in1, void *out0, void *out1,
                    int64_t nvec, int64_t grid, unsigned key, hipEvent_t e0, hipEvent_t e1,
                    hipStream_t s) {
#define DLN_PROBE_U(U)                                                                         \
  return nt ? launch<NIN, NOUT, U, true>(in0, in1, out0, out1, nvec, grid, key, e0, e1, s)     \
            : launch<NIN, NOUT, U, false>(in0, in1, out0, out1, nvec, grid, key, e0, e1, s);
  switch (unroll) {
  case 1: DLN_PROBE_U(1)
  case 2: DLN_PROBE_U(2)
  case 4: DLN_PROBE_U(4)
  default: DLN_PROBE_U(8)
  }
#undef DLN_PROBE_U
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Every wavefront runs `iters` rounds of eight independent bf16 matrix operations on operands
// held in registers (no memory traffic), then stores one sum per lane so that none is dropped.
template <int SHAPE, int NT>
__global__ __launch_bounds__(NT) void mfma_probe_kernel(float *out, int iters) {
  const int t = threadIdx.x;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)((t + i) & 15);
    b[i] = (__bf16)(float)((t ^ i) & 15);
  }
  float s = 0.0f;
  if constexpr (SHAPE == 32) {
    f32x16_t acc[8] = {};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[u], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[u][r];
  } else {
    f32x4_t acc[8] = {};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[u], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) s += acc[u][r];
  }
  out[(int64_t)blockIdx.x * NT + t] = s;
}

template <int SHAPE, int NT>
hipError_t launch_mfma(float *out, int64_t grid, int iters, hipEvent_t e0, hipEvent_t e1,
                       hipStream_t s) {
  void *args[] = {&out, &iters};
  return hipExtLaunchKernel(reinterpret_cast<const void *>(mfma_probe_kernel<SHAPE, NT>),
                            dim3((unsigned)grid), dim3(NT), args, 0, s, e0, e1, 0);
}

// Every thread reads 16 bytes per access from a 64 KB LDS buffer (filled with a pattern
// first); the 64 lanes of an access read one contiguous KB (no bank conflicts), and successive
// accesses walk the buffer. The XOR of everything read goes to out[thread].
template <int NT>
__global__ __launch_bounds__(NT) void lds_probe_kernel(unsigned *out, int iters) {
  typedef unsigned u4 __attribute__((ext_vector_type(4)));
  __shared__ __align__(16) unsigned char buf[65536];
  const int t = threadIdx.x;
  for (int i = t; i < 65536 / 4; i += NT) reinterpret_cast<unsigned *>(buf)[i] = i * 2654435761u;
  __syncthreads();
  const int lane = t & 63, wave = t >> 6;
  unsigned acc = 0;
  int base = (wave * 1024) & 65535;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int off = (base + u * 1024 + lane * 16) & 65520;
      const u4 v = *reinterpret_cast<const u4 *>(buf + off);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    base = (base + 8192) & 65535;
  }
  out[(int64_t)blockIdx.x * NT + t] = acc;
}

} // namespace

extern "C" int lds_probe(int waves_per_simd, int64_t grid, int iters, unsigned *out,
                         void *start_event, void *stop_event, void *stream) {
  if ((waves_per_simd != 1 && waves_per_simd != 2 && waves_per_simd != 4) || grid <= 0 ||
      grid > 0x7fffffff / 1024 || iters <= 0 || !out)
    return -1;
  if ((start_event == nullptr) != (stop_event == nullptr)) return -1;
  hipEvent_t e0 = static_cast<hipEvent_t>(start_event), e1 = static_cast<hipEvent_t>(stop_event);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void *args[] = {&out, &iters};
  const void *k = waves_per_simd == 1 ? reinterpret_cast<const void *>(lds_probe_kernel<256>)
                  : waves_per_simd == 2 ? reinterpret_cast<const void *>(lds_probe_kernel<512>)
                                        : reinterpret_cast<const void *>(lds_probe_kernel<1024>);
  const hipError_t e = hipExtLaunchKernel(k, dim3((unsigned)grid), dim3(256 * waves_per_simd),
                                          args, 0, s, e0, e1, 0);
  return e == hipSuccess ? 0 : -2;
}

extern "C" int mfma_probe(int shape, int waves_per_simd, int64_t grid, int iters, float *out,
                          void *start_event, void *stop_event, void *stream) {
  if ((shape != 32 && shape != 16) || (waves_per_simd != 1 && waves_per_simd != 2)) return -1;
  if (grid <= 0 || grid > 0x7fffffff / 512 || iters <= 0 || !out) return -1;
  if ((start_event == nullptr) != (stop_event == nullptr)) return -1;
  hipEvent_t e0 = static_cast<hipEvent_t>(start_event), e1 = static_cast<hipEvent_t>(stop_event);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (shape == 32)
    e = waves_per_simd == 1 ? launch_mfma<32, 256>(out, grid, iters, e0, e1, s)
                            : launch_mfma<32, 512>(out, grid, iters, e0, e1, s);
  else
    e = waves_per_simd == 1 ? launch_mfma<16, 256>(out, grid, iters, e0, e1, s)
                            : launch_mfma<16, 512>(out, grid, iters, e0, e1, s);
  return e == hipSuccess ? 0 : -2;
}

extern "C" int hbm_probe(int nin, int nout, const void *in0, const void *in1, void *out0,
                         void *out1, size_t bytes, int unroll, int nt_loads, int64_t grid,
                         uint32_t key, void *start_event, void *stop_event, void *stream) {
  if (bytes == 0 || bytes % 16 || grid < 0 || (nt_loads != 0 && nt_loads != 1)) return -1;
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) return -1;
  if ((start_event == nullptr) != (stop_event == nullptr)) return -1;
  const bool shape_ok = (nin == 1 && nout == 0) || (nin == 0 && nout == 1) ||
                        (nin == 1 && nout == 1) || (nin == 2 && nout == 1) ||
                        (nin == 2 && nout == 2);
  if (!shape_ok) return -1;
  const void *ins[] = {in0, in1};
  void *outs[] = {out0, out1};
  for (int i = 0; i < nin; ++i)
    if (!ins[i] || !aligned16(ins[i])) return -1;
  if (!out0 || !aligned16(out0)) return -1; // the read probe's sink, or the first output
  if (nout == 2 && (!out1 || !aligned16(out1))) return -1;
  (void)outs;
  const int64_t nvec = (int64_t)(bytes / 16);
  hipEvent_t e0 = static_cast<hipEvent_t>(start_event), e1 = static_cast<hipEvent_t>(stop_event);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (nin == 1 && nout == 0)
    e = by_shape<1, 0>(unroll, nt_loads, in0, in1, out0, out1, nvec, grid, key, e0, e1, s);
  else if (nin == 0)
    e = by_shape<0, 1>(unroll, nt_loads, in0, in1, out0, out1, nvec, grid, key, e0, e1, s);
  else if (nin == 1)
    e = by_shape<1, 1>(unroll, nt_loads, in0, in1, out0, out1, nvec, grid, key, e0, e1, s);
  else if (nout == 1)
    e = by_shape<2, 1>(unroll, nt_loads, in0, in1, out0, out1, nvec, grid, key, e0, e1, s);
  else
    e = by_shape<2, 2>(unroll, nt_loads, in0, in1, out0, out1, nvec, grid, key, e0, e1, s);
  return e == hipSuccess ? 0 : -2;
}
