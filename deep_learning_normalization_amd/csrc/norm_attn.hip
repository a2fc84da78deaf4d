// norm_attn.hip -- attention whose queries and keys are normalised inside the attention kernel.
//
// Method (web page "Towards Free Normalization: Fusing Normalization into GEMM and Attention
// Kernels", brifing.si), item 5: several norms fused around an attention kernel. Reading taken
// here: the norm (RMSNorm, or LayerNorm with its beta; one gamma of D entries for the queries
// and one for the keys, shared by every head) of every query and key vector along the head
// dimension, applied where the kernel stages those vectors for the scores, so that the
// normalised Q and K never reach HBM. The attention is the softmax of the scaled scores times V,
// evaluated one key tile at a time with a running maximum and sum per query, so neither the
// scores nor the weights reach HBM either.
//
//   grid       one workgroup per (batch, query head, block of 256 queries). Workgroup ids are
//              renumbered so that each XCD walks one contiguous range of them: the query heads
//              that share a key/value head are adjacent, and their K and V tiles stay in that
//              XCD's L2. With the causal mask, the longest blocks of each head go first.
//   workgroup  512 threads, eight wavefronts of 32 queries each, two per SIMD (one computes
//              its softmax while the other's matrix products run). Each wavefront holds its
//              queries' normalised vectors (bf16) in registers as the B operand of S^T = K Q^T:
//              lane l then owns query l % 32 and half (l / 32) of the keys of each 32-key MFMA
//              block, so a query's running maximum and sum stay in its two lanes.
//   key tiles  64 keys at a time through double-buffered LDS. Wavefronts 4-7 load K, normalise
//              each key vector (16 lanes per key, DPP row sums) and store it as bf16; wavefronts
//              0-3 load V and store it transposed, so that O^T = V^T P^T takes its B operand P
//              straight from the score registers (MFMA 32x32x16 bf16, fp32 accumulation, for
//              both products). The next tile's global loads are in flight during the products.
//
// Numerics: the normalised vectors are rounded once to bf16 (as a separate norm pass would
// store them), the scores and the output accumulate in fp32, the weights P are rounded to bf16
// for the second product, and O is rounded once to bf16.
#include <cmath>

#include "norm_attn.hpp"
#include "norm_device.hpp"

namespace dln {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int D = kAttnD, BQ = kAttnBQ, BK = kAttnBK;
constexpr int kThreads = 512;
constexpr int kKRow = D + 8;   // bf16 per staged key row: 272 bytes, so that the 16-byte operand
                               // reads of 16 consecutive keys start on distinct bank groups
constexpr int kVRow = BK + 8;  // bf16 per staged row of V^T (one head dimension): 144 bytes
static_assert(BQ == 8 * 32, "eight wavefronts of 32 queries");
static_assert(D == 128 && BK == 64, "the staging maps below assume D = 128 and 64-key tiles");

// Score register r of lane l for 32-key block j holds key 32j + 8(r/4) + 4(l/32) + r%4 of the
// tile. The second product takes the 16 keys 16s .. 16s+15 as the k range of one MFMA step:
// lane l supplies registers 8(s%2) .. 8(s%2)+7 of block s/2, that is keys 16s + 4h + i
// (i < 4) and 16s + 8 + 4h + (i - 4) (i >= 4), h = l / 32, in that order. Its A operand, V^T,
// must list the same keys in the same order; so V^T stores key kk of the tile in slot
// 16(kk/16) + swap of bits 2 and 3 of (kk % 16), and lane half h reads slots 16s + 8h .. +7.
//
// Element (dim d, slot p) of the staged V^T tile. Slots go in 16-byte units of 8; the unit
// index is XORed with bits 4 and 5 of d, which spreads both the transposing 8-byte writes and
// the 16-byte operand reads over the LDS banks.
__device__ __forceinline__ int vt_off(int d, int p) {
  return d * kVRow + ((((p >> 3) ^ ((d >> 3) & 6))) << 3) + (p & 7);
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the same bits.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);   // lane ^ 1
  v += dpp_mov<0x4E>(v);   // lane ^ 2
  v += dpp_mov<0x141>(v);  // the other quad of the 8-lane half
  v += dpp_mov<0x140>(v);  // the other 8-lane half of the row
  return v;
}

__device__ __forceinline__ void unpack8(uint4 u, float (&f)[8]) {
  const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

template <int NORM, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_kernel(AttnArgs a) {
  __shared__ __align__(16) uint16_t sk[2][BK * kKRow];
  __shared__ __align__(16) uint16_t svt[2][D * kVRow];
  constexpr bool LN = NORM == ATTN_LAYERNORM;
  constexpr bool NORMED = NORM != ATTN_NO_NORM;
  constexpr float kInvD = 1.0f / (float)D;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int half = lane >> 5, col = lane & 31;

  // workgroup -> (batch, query head, query block)
  int bid = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);
  const int qbr = bid % a.qblocks;
  const int bh = bid / a.qblocks;
  const int head = bh % a.Hq, b = bh / a.Hq;
  const int qb = CAUSAL ? a.qblocks - 1 - qbr : qbr;
  const int hk = head / (a.Hq / a.Hk);
  const int S = a.S;
  const int q0 = qb * BQ;
  const int wq0 = q0 + wave * 32;  // this wavefront's first query
  const int myq = wq0 + col;       // the query lane l owns
  const bool wactive = wq0 < S;
  const int wlast = min(wq0 + 31, S - 1);

  // ---- this wavefront's queries, normalised, as MFMA B operands: lane l holds dims
  // 16ks + 8h .. 16ks + 8h + 7 of query l % 32 in qf[ks]
  bf16x8_t qf[8];
  {
    const int qrow = myq < S ? myq : S - 1;
    const uint16_t *qp = a.q + ((int64_t)b * S + qrow) * a.ldq + (int64_t)head * D + half * 8;
    float x[8][8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) unpack8(*reinterpret_cast<const uint4 *>(qp + ks * 16), x[ks]);
    if constexpr (NORMED) {
      float mean = 0.0f;
      if constexpr (LN) {
        float s = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
          for (int i = 0; i < 8; ++i) s += x[ks][i];
        s += __shfl_xor(s, 32);
        mean = s * kInvD;
      }
      float q2 = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float d = x[ks][i] - mean;
          q2 = __builtin_fmaf(d, d, q2);
        }
      q2 += __shfl_xor(q2, 32);
      const float rstd = rsqrt_f32(q2 * kInvD + a.eps);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        float g[8], be[8];
        unpack8(*reinterpret_cast<const uint4 *>(a.wq + ks * 16 + half * 8), g);
        if constexpr (LN)
          unpack8(a.bq ? *reinterpret_cast<const uint4 *>(a.bq + ks * 16 + half * 8)
                       : make_uint4(0u, 0u, 0u, 0u),
                  be);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float y = (x[ks][i] - mean) * rstd * g[i];
          x[ks][i] = LN ? y + be[i] : y;
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = __builtin_bit_cast(bf16x8_t, pack8(x[ks]));
  }

  // ---- staging roles: wavefronts 4-7 stage K, 0-3 stage V. Thread st of a role owns the
  // 16-byte chunk sc (dims 8sc .. 8sc+7) of K rows srow + 16i, or of V keys 4srow + i, i < 4.
  const bool kstage = wave >= 4;
  const int st = t & 255, sc = st & 15, srow = st >> 4;
  uint4 gk = make_uint4(0u, 0u, 0u, 0u), bk = gk;
  if (NORMED && kstage) {
    gk = *reinterpret_cast<const uint4 *>(a.wk + sc * 8);
    if (LN && a.bk) bk = *reinterpret_cast<const uint4 *>(a.bk + sc * 8);
  }
  const uint16_t *sbase = kstage ? a.k : a.v;
  const int64_t sld = kstage ? a.ldk : a.ldv;
  sbase += (int64_t)b * S * sld + (int64_t)hk * D + sc * 8;
  uint4 pre[4];
  auto load_tile = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int key = kb * BK + (kstage ? srow + 16 * i : 4 * srow + i);
      key = key < S ? key : S - 1;  // rows past the end: a real row, masked out of the scores
      pre[i] = *reinterpret_cast<const uint4 *>(sbase + (int64_t)key * sld);
    }
  };
  auto stage_tile = [&](int buf) {
    if (kstage) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x[8];
        unpack8(pre[i], x);
        if constexpr (NORMED) {
          float mean = 0.0f;
          if constexpr (LN) {
            float s = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) s += x[e];
            mean = row16_sum(s) * kInvD;
          }
          float q2 = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float d = x[e] - mean;
            q2 = __builtin_fmaf(d, d, q2);
          }
          const float rstd = rsqrt_f32(row16_sum(q2) * kInvD + a.eps);
          float g[8], be[8];
          unpack8(gk, g);
          if constexpr (LN) unpack8(bk, be);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float y = (x[e] - mean) * rstd * g[e];
            x[e] = LN ? y + be[e] : y;
          }
        }
        *reinterpret_cast<uint4 *>(&sk[buf][(srow + 16 * i) * kKRow + sc * 8]) = pack8(x);
      }
    } else {
      // keys 4srow .. 4srow+3 land in four consecutive slots (see vt_off)
      const int p = 16 * (srow >> 2) + 8 * (srow & 1) + 4 * ((srow >> 1) & 1);
      const unsigned w0[4] = {pre[0].x, pre[0].y, pre[0].z, pre[0].w};
      const unsigned w1[4] = {pre[1].x, pre[1].y, pre[1].z, pre[1].w};
      const unsigned w2[4] = {pre[2].x, pre[2].y, pre[2].z, pre[2].w};
      const unsigned w3[4] = {pre[3].x, pre[3].y, pre[3].z, pre[3].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int d = sc * 8 + 2 * w;
        const uint2 lo = make_uint2((w0[w] & 0xffffu) | (w1[w] << 16),
                                    (w2[w] & 0xffffu) | (w3[w] << 16));
        const uint2 hi = make_uint2((w0[w] >> 16) | (w1[w] & 0xffff0000u),
                                    (w2[w] >> 16) | (w3[w] & 0xffff0000u));
        *reinterpret_cast<uint2 *>(&svt[buf][vt_off(d, p)]) = lo;
        *reinterpret_cast<uint2 *>(&svt[buf][vt_off(d + 1, p)]) = hi;
      }
    }
  };

  // ---- key tiles
  const int nkt_all = (S + BK - 1) / BK;
  const int qlast = min(q0 + BQ, S) - 1;
  const int nkt = CAUSAL ? min(nkt_all, qlast / BK + 1) : nkt_all;
  const float c = a.scale_log2;
  f32x16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  float m = -INFINITY, l = 0.0f;  // running maximum (log2 units) and this lane's share of the sum

  load_tile(0);
  stage_tile(0);
  __syncthreads();
  for (int kb = 0; kb < nkt; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkt) load_tile(kb + 1);
    const int k0 = kb * BK;
    if (wactive && (!CAUSAL || k0 <= wlast)) {
      f32x16_t s[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[j][r] = 0.0f;
      const uint16_t *kp = &sk[buf][col * kKRow + half * 8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const bf16x8_t kf = *reinterpret_cast<const bf16x8_t *>(kp + j * 32 * kKRow + ks * 16);
          s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[j], 0, 0, 0);
        }
      // keys past the end, and (causal) keys after the query
      if (k0 + BK > S || (CAUSAL && k0 + BK - 1 > wq0)) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * j + 8 * (r >> 2) + 4 * half + (r & 3);
            if (key >= S || (CAUSAL && key > myq)) s[j][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[j][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // key 0 is in the first tile of every query, so m is finite from the first tile on
      const float mnew = fmaxf(m, mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      float ls = 0.0f;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j][r], c, -mnew));
          s[j][r] = p;
          ls += p;
        }
      l = __builtin_fmaf(l, alpha, ls);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
#pragma unroll
      for (int ss = 0; ss < 4; ++ss) {
        const int j = ss >> 1, r0 = 8 * (ss & 1);
        const uint4 pw = make_uint4(pack_bf16x2(s[j][r0], s[j][r0 + 1]),
                                    pack_bf16x2(s[j][r0 + 2], s[j][r0 + 3]),
                                    pack_bf16x2(s[j][r0 + 4], s[j][r0 + 5]),
                                    pack_bf16x2(s[j][r0 + 6], s[j][r0 + 7]));
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x8_t vf = *reinterpret_cast<const bf16x8_t *>(
              &svt[buf][vt_off(32 * dt + col, 16 * ss + 8 * half)]);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, o[dt], 0, 0, 0);
        }
      }
    }
    if (kb + 1 < nkt) stage_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- O = O^T's column / sum, rounded once; lse = ln(sum) + max
  const float lt = l + __shfl_xor(l, 32);
  if (wactive && myq < S) {
    const float inv = 1.0f / lt;
    uint16_t *op = a.o + ((int64_t)b * S + myq) * a.ldo + (int64_t)head * D + 4 * half;
    // register r of O^T block dt holds dim 32dt + 8(r/4) + 4h + r%4 of this lane's query
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint2 w = make_uint2(pack_bf16x2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                                   pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv));
        *reinterpret_cast<uint2 *>(op + 32 * dt + 8 * g) = w;
      }
    if (a.lse && half == 0)
      a.lse[((int64_t)b * a.Hq + head) * S + myq] = (m + __log2f(lt)) * 0.69314718055994531f;
  }
}

template <int NORM>
hipError_t launch_norm(bool causal, dim3 grid, dim3 block, hipStream_t s, const AttnArgs &a) {
  return causal ? launch(attn_fwd_kernel<NORM, true>, grid, block, s, a)
                : launch(attn_fwd_kernel<NORM, false>, grid, block, s, a);
}

} // namespace

norm_status_t launch_attention(int norm, bool causal, const AttnArgs &a, hipStream_t s) {
  const int64_t wg = (int64_t)a.B * a.Hq * a.qblocks;
  if (wg <= 0 || wg > 0x7fffffffLL) return NORM_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)wg), block(kThreads);
  hipError_t e;
  switch (norm) {
  case ATTN_LAYERNORM: e = launch_norm<ATTN_LAYERNORM>(causal, grid, block, s, a); break;
  case ATTN_RMSNORM: e = launch_norm<ATTN_RMSNORM>(causal, grid, block, s, a); break;
  case ATTN_NO_NORM: e = launch_norm<ATTN_NO_NORM>(causal, grid, block, s, a); break;
  default: return NORM_ERR_INVALID_ARG;
  }
  return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

} // namespace dln
