// norm_device.hpp -- device building blocks for the gfx950 norm kernels: 16-byte accesses with
// fp32 unpack/pack, wavefront sums over DPP, and team sums through LDS.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dln {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// bf16 tensors are carried as their raw 16-bit patterns; fp16 tensors as the compiler's
// binary16 type (conversions to and from fp32 are the hardware's, round to nearest even).
typedef uint16_t bf16_bits;
typedef _Float16 f16_t;

// Input loads and output stores of the streamed [M, N] tensors. Each element is touched once
// per pass, so stores bypass the caches' allocate-on-write (nontemporal). ld_stream loads stay
// ordinary: the looped and split schemes re-read their chunks and want them cached.
#ifndef DLN_STORE_NT
#define DLN_STORE_NT 1
#endif
#ifndef DLN_LOAD_NT
#define DLN_LOAD_NT 0
#endif

template <typename V> __device__ __forceinline__ V ld_stream(const V *p) {
#if DLN_LOAD_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

// Loads of data that a kernel reads exactly once (X, R, dY and dH in the wave and block
// schemes, which hold their rows in registers): nontemporal. Measured on MI355X, cache-cold,
// against ordinary loads: LayerNorm bf16 16384 x 4096 backward 76.6 -> 73.0 us, RMSNorm bf16
// 32768 x 4096 backward 135.7 -> 129.5 us, residual RMSNorm 65536 x 7168 forward 646 -> 618 us.
template <typename V> __device__ __forceinline__ V ld_once(const V *p) {
  return __builtin_nontemporal_load(p);
}

template <typename V> __device__ __forceinline__ void st_stream(V *p, V v) {
#if DLN_STORE_NT
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

__device__ __forceinline__ float bf16_lo(unsigned u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(unsigned u) {
  return __builtin_bit_cast(float, u & 0xffff0000u);
}
// Two fp32 values to two bf16 (round to nearest even, gfx950 v_cvt_pk_bf16_f32), packed.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}
__device__ __forceinline__ float round_bf16(float v) {
  unsigned p = pack_bf16x2(v, 0.0f);
  return bf16_lo(p);
}

// The same for fp16 (IEEE binary16).
__device__ __forceinline__ float f16_lo(unsigned u) {
  return (float)__builtin_bit_cast(f16_t, (uint16_t)(u & 0xffffu));
}
__device__ __forceinline__ float f16_hi(unsigned u) {
  return (float)__builtin_bit_cast(f16_t, (uint16_t)(u >> 16));
}
__device__ __forceinline__ unsigned pack_f16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, f16x2));
}
__device__ __forceinline__ float round_f16(float v) { return (float)(f16_t)v; }

// Two 16-bit values of type T (bf16_bits or f16_t) in one 32-bit word, to and from fp32.
template <typename T> __device__ __forceinline__ float lo16(unsigned u) {
  if constexpr (__is_same(T, f16_t)) return f16_lo(u);
  else return bf16_lo(u);
}
template <typename T> __device__ __forceinline__ float hi16(unsigned u) {
  if constexpr (__is_same(T, f16_t)) return f16_hi(u);
  else return bf16_hi(u);
}
template <typename T> __device__ __forceinline__ unsigned pack16x2(float lo, float hi) {
  if constexpr (__is_same(T, f16_t)) return pack_f16x2(lo, hi);
  else return pack_bf16x2(lo, hi);
}
template <typename T> __device__ __forceinline__ float round16(float v) {
  if constexpr (__is_same(T, f16_t)) return round_f16(v);
  else return round_bf16(v);
}

// Acc<T, E>: one memory access of E elements of T, converted to / from fp32. E * sizeof(T) is
// 16, 8 or 4 bytes on the vector paths (whole 32-bit words, E = full_epv<T>() and its halves
// down to two elements); E = 1 is the element-wise path.
template <typename T> constexpr int full_epv() { return 16 / (int)sizeof(T); }

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
template <int NW> struct Words;
template <> struct Words<4> { typedef u32x4 type; };
template <> struct Words<2> { typedef u32x2 type; };
template <> struct Words<1> { typedef unsigned type; };
// Word i of a raw access, read into a scalar first: this clang's __builtin_bit_cast applied
// directly to a vector subscript (v[i]) reads element 0 whatever i is.
__device__ __forceinline__ unsigned word(u32x4 v, int i) { const unsigned u = v[i]; return u; }
__device__ __forceinline__ unsigned word(u32x2 v, int i) { const unsigned u = v[i]; return u; }
__device__ __forceinline__ unsigned word(unsigned v, int) { return v; }
__device__ __forceinline__ void set_word(u32x4 &v, int i, unsigned u) { v[i] = u; }
__device__ __forceinline__ void set_word(u32x2 &v, int i, unsigned u) { v[i] = u; }
__device__ __forceinline__ void set_word(unsigned &v, int, unsigned u) { v = u; }

template <typename T, int E> struct Acc {
  static_assert(E >= 2 && E <= full_epv<T>() && (E & (E - 1)) == 0, "whole-word accesses");
  static constexpr int EPV = E;
  static constexpr int NW = E * (int)sizeof(T) / 4;
  static constexpr bool B16 = sizeof(T) == 2; // bf16 or fp16
  typedef typename Words<NW>::type raw;
  __device__ static raw ld(const T *p) { return ld_stream(reinterpret_cast<const raw *>(p)); }
  __device__ static raw ld_once(const T *p) {
    return dln::ld_once(reinterpret_cast<const raw *>(p));
  }
  __device__ static raw ld_cached(const T *p) { return *reinterpret_cast<const raw *>(p); }
  __device__ static void st(T *p, raw v) { st_stream(reinterpret_cast<raw *>(p), v); }
  __device__ static void unpack(raw v, float *f) {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const unsigned u = word(v, i);
      if constexpr (B16) {
        f[2 * i] = lo16<T>(u);
        f[2 * i + 1] = hi16<T>(u);
      } else {
        f[i] = __builtin_bit_cast(float, u);
      }
    }
  }
  __device__ static raw pack(const float *f) {
    raw v;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      if constexpr (B16)
        set_word(v, i, pack16x2<T>(f[2 * i], f[2 * i + 1]));
      else
        set_word(v, i, __builtin_bit_cast(unsigned, f[i]));
    }
    return v;
  }
  __device__ static float round(float v) {
    if constexpr (B16) return round16<T>(v);
    return v;
  }
  __device__ static raw zero() {
    raw v;
#pragma unroll
    for (int i = 0; i < NW; ++i) set_word(v, i, 0u);
    return v;
  }
};

template <> struct Acc<float, 1> {
  static constexpr int EPV = 1;
  typedef float raw;
  __device__ static raw ld(const float *p) { return *p; }
  __device__ static raw ld_once(const float *p) { return dln::ld_once(p); }
  __device__ static raw ld_cached(const float *p) { return *p; }
  __device__ static void st(float *p, raw v) { *p = v; }
  __device__ static void unpack(raw v, float *f) { f[0] = v; }
  __device__ static raw pack(const float *f) { return f[0]; }
  __device__ static float round(float v) { return v; }
  __device__ static raw zero() { return 0.0f; }
};

template <> struct Acc<bf16_bits, 1> {
  static constexpr int EPV = 1;
  typedef bf16_bits raw;
  __device__ static raw ld(const bf16_bits *p) { return *p; }
  __device__ static raw ld_once(const bf16_bits *p) { return dln::ld_once(p); }
  __device__ static raw ld_cached(const bf16_bits *p) { return *p; }
  __device__ static void st(bf16_bits *p, raw v) { *p = v; }
  __device__ static void unpack(raw v, float *f) {
    f[0] = __builtin_bit_cast(float, ((unsigned)v) << 16);
  }
  __device__ static raw pack(const float *f) { return (raw)(pack_bf16x2(f[0], 0.0f) & 0xffffu); }
  __device__ static float round(float v) { return round_bf16(v); }
  __device__ static raw zero() { return 0; }
};

template <> struct Acc<f16_t, 1> {
  static constexpr int EPV = 1;
  typedef uint16_t raw; // the element's bits
  __device__ static raw ld(const f16_t *p) { return *reinterpret_cast<const raw *>(p); }
  __device__ static raw ld_once(const f16_t *p) {
    return dln::ld_once(reinterpret_cast<const raw *>(p));
  }
  __device__ static raw ld_cached(const f16_t *p) { return *reinterpret_cast<const raw *>(p); }
  __device__ static void st(f16_t *p, raw v) { *reinterpret_cast<raw *>(p) = v; }
  __device__ static void unpack(raw v, float *f) { f[0] = (float)__builtin_bit_cast(f16_t, v); }
  __device__ static raw pack(const float *f) { return __builtin_bit_cast(raw, (f16_t)f[0]); }
  __device__ static float round(float v) { return round_f16(v); }
  __device__ static raw zero() { return 0; }
};

// Settle a value loaded from memory at this point: an empty asm that takes it in VGPRs and may
// rewrite it, so the wait for its load is placed here. Kernels settle the weight and bias once,
// after the first row group's loads are issued; left to itself the compiler may place that wait
// inside the row loop, behind the loads issued for the next row group, and then every
// iteration drains the software pipeline.
__device__ __forceinline__ void settle(float &v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void settle(unsigned &v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void settle(u32x2 &v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void settle(u32x4 &v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void settle(bf16_bits &v) {
  unsigned u = v;
  asm volatile("" : "+v"(u));
  v = (bf16_bits)u;
}

// WAcc<T, TW, E>: the weight (or bias) values of one access of E elements of T, stored as TW.
// With the same storage type as the activations they stay packed; fp32 weights next to bf16 or
// fp16 activations are E fp32 values (E * 4 bytes: two 16-byte loads for E = 8, one 8-byte load for
// E = 2). get() gives fp32; store() writes E fp32 sums as TW (the final dW / dB).
template <typename T, typename TW, int E> struct WAcc;

template <typename T, int EV> struct WAcc<T, T, EV> {
  using A = Acc<T, EV>;
  static constexpr int E = A::EPV;
  typename A::raw r;
  __device__ void zero() { r = A::zero(); }
  __device__ void load(const T *p) { r = A::ld_cached(p); }
  // E weights from p at any element alignment (one unaligned access)
  __device__ void load_any(const T *p) { __builtin_memcpy(&r, p, sizeof(r)); }
  __device__ void get(float *f) const { A::unpack(r, f); }
  __device__ void settle() { dln::settle(r); }
  __device__ static void store(T *p, const float *f) { A::st(p, A::pack(f)); }
};

template <int EV> struct WAccF32 {
  static constexpr int E = EV;
  // words per load: 16-byte loads when E is a multiple of 4, else one E-word load
  static constexpr int LW = E % 4 == 0 ? 4 : E;
  typedef typename Words<LW>::type raw;
  float w[E];
  __device__ void zero() {
#pragma unroll
    for (int e = 0; e < E; ++e) w[e] = 0.0f;
  }
  __device__ void load(const float *p) {
#pragma unroll
    for (int i = 0; i < E / LW; ++i) {
      const raw v = *reinterpret_cast<const raw *>(p + LW * i);
#pragma unroll
      for (int j = 0; j < LW; ++j) w[LW * i + j] = __builtin_bit_cast(float, word(v, j));
    }
  }
  __device__ void load_any(const float *p) { __builtin_memcpy(w, p, sizeof(w)); }
  __device__ void get(float *f) const {
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = w[e];
  }
  __device__ void settle() {
#pragma unroll
    for (int e = 0; e < E; ++e) dln::settle(w[e]);
  }
  __device__ static void store(float *p, const float *f) {
#pragma unroll
    for (int i = 0; i < E / LW; ++i) {
      raw v;
#pragma unroll
      for (int j = 0; j < LW; ++j) set_word(v, j, __builtin_bit_cast(unsigned, f[LW * i + j]));
      *reinterpret_cast<raw *>(p + LW * i) = v;
    }
  }
};
template <int EV> struct WAcc<bf16_bits, float, EV> : WAccF32<EV> {};
template <int EV> struct WAcc<f16_t, float, EV> : WAccF32<EV> {};

// ---- reductions -------------------------------------------------------------------------

template <int CTRL> __device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float read_lane(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// DPP move into the rows of ROWMASK only; the other rows get 0.
template <int CTRL, int ROWMASK> __device__ __forceinline__ float dpp_rows(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, ROWMASK, 0xF, false));
}

// Sum over the 64 lanes of a wavefront, returned as a wave-uniform value. Four symmetric
// steps leave every lane of each 16-lane row with that row's sum r0..r3; two row broadcasts
// (lane 15 of a row into the next row, then lane 31 into rows 2 and 3) leave
// (r3 + r2) + (r1 + r0) in lane 63, which is read out. The order is fixed, so the result is
// the same bits on every call with the same inputs. All 64 lanes must be active.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xB1>(v);         // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_mov<0x4E>(v);         // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_mov<0x141>(v);        // row_half_mirror: quad 0 <-> quad 1 within each 8 lanes
  v += dpp_mov<0x140>(v);        // row_mirror: the two 8-lane halves of each 16-lane row
  v += dpp_rows<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_rows<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return read_lane(v, 63);
}

// LDS scratch for team sums: 2 alternating slots x up to 12 values x 16 waves, plus one row of
// padding for the fixed-length reads below.
constexpr int RED_VALS = 12;
constexpr int RED_WAVES = 16;
constexpr int RED_FLOATS = 2 * RED_VALS * RED_WAVES + RED_WAVES;

// Sums NV values over one team of `waves` consecutive wavefronts of the workgroup (the team's
// first wave is `wave0`, a multiple of 4; this thread's wave is `wave`). MAXW (compile time)
// bounds `waves`. Every thread of the workgroup must call it with the same slot and NV (it
// contains one barrier when waves > 1). Alternating the slot between consecutive calls makes
// one barrier per call enough: a slot is rewritten only after the next call's barrier, by
// which time every thread has read it. The read-back is branch-free: MAXW/4 broadcast 16-byte
// LDS reads per value, adding the team's `waves` partials in wave order (words past the team
// are read and discarded).
template <int NV, int MAXW>
__device__ __forceinline__ void team_sum(float (&v)[NV], float *red, int slot, int waves,
                                         int wave0, int wave, int lane) {
  static_assert(NV <= RED_VALS, "too many values for one team sum");
  static_assert(MAXW == 1 || MAXW % 4 == 0, "wave bound must be 1 or a multiple of 4");
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = wave_sum(v[i]);
  if (MAXW == 1 || waves == 1) return;
  float *base = red + slot * (RED_VALS * RED_WAVES);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) base[i * RED_WAVES + wave] = v[i];
  }
  __syncthreads();
  if (waves == MAXW) {
    // the whole workgroup is one team: every word read is a partial (same order, no selects)
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const float4 *q = reinterpret_cast<const float4 *>(base + i * RED_WAVES);
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < (MAXW == 1 ? 1 : MAXW / 4); ++j) {
        const float4 f = q[j];
        s += f.x;
        s += f.y;
        s += f.z;
        s += f.w;
      }
      v[i] = s;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const float4 *q = reinterpret_cast<const float4 *>(base + i * RED_WAVES + wave0);
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < (MAXW == 1 ? 1 : MAXW / 4); ++j) {
      const float4 f = q[j];
      s += (4 * j + 0 < waves) ? f.x : 0.0f;
      s += (4 * j + 1 < waves) ? f.y : 0.0f;
      s += (4 * j + 2 < waves) ? f.z : 0.0f;
      s += (4 * j + 3 < waves) ? f.w : 0.0f;
    }
    v[i] = s;
  }
}

// a * b rounded to fp32 and never fused into a following add (device code is compiled with
// FMA contraction on). A row mean formed this way is the same fp32 value at every use, which
// the mean-correction sums rely on.
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}

// 1 / sqrt(v): the hardware reciprocal square root (about 1 ulp).
__device__ __forceinline__ float rsqrt_f32(float v) { return __builtin_amdgcn_rsqf(v); }

// A variance formed by subtraction, with a negative rounding residue set to 0. A NaN passes
// through (fmaxf would turn it into 0 and give a NaN row the finite rstd eps^-1/2).
__device__ __forceinline__ float clamp_var(float v) { return v < 0.0f ? 0.0f : v; }

// Elements in chunk c of a split row of nacc accesses of E elements, chunk_acc accesses per
// chunk (the last chunk may be short).
__device__ __forceinline__ float split_chunk_elems(int64_t c, int32_t chunk_acc, int32_t nacc,
                                                   int E) {
  const int64_t left = (int64_t)nacc - c * chunk_acc;
  return (float)((left < chunk_acc ? left : chunk_acc) * E);
}

// LayerNorm statistics of a row from its chunks' partials (the split scheme, both forms): chunk
// c has n_c elements, mean m_c, q_c = sum (x - m_c)^2 and s_c = sum (x - m_c). With d_c = m_c -
// shift (shift: chunk 0's mean), A = sum n_c d_c + s_c gives the row mean shift + A / N, and
// B = sum q_c + 2 d_c s_c + n_c d_c^2 the squared deviation B - A^2 / N: an exact regrouping of
// sum_c q_c + 2 (m_c - mean) s_c + n_c (m_c - mean)^2, whose terms stay small and positive.
__device__ __forceinline__ void ln_chunk_terms(float n, float mc, float q, float s, float shift,
                                               float &A, float &B) {
  const float d = mc - shift;
  A += n * d + s;
  B += q + 2.0f * d * s + n * d * d;
}
// From the team-summed A and B: delta = A / N (the mean is shift + delta) and rstd.
__device__ __forceinline__ float ln_combined_rstd(float A, float B, float inv_n, float eps,
                                                  float &delta) {
  delta = A * inv_n;
  return rsqrt_f32(clamp_var((B - delta * A) * inv_n) + eps);
}

} // namespace dln
