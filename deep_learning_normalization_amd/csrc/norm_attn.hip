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
//              renumbered so that each XCD takes a contiguous range of heads: the query heads
//              that share a key/value head are adjacent, and their K and V tiles stay in that
//              XCD's L2. With the causal mask, the longest blocks go first.
//   workgroup  512 threads, eight wavefronts of 32 queries each, two per SIMD (one computes
//              its softmax while the other's matrix products run). Each wavefront holds its
//              queries' normalised vectors (bf16) in registers as the B operand of S^T = K Q^T:
//              lane l then owns query l % 32 and half (l / 32) of the keys of each 32-key MFMA
//              block, so a query's running maximum and sum stay in its two lanes.
//   key tiles  64 keys at a time through double-buffered LDS. Wavefronts 4-7 copy K as it is
//              and form each key's statistics (16 lanes per key, DPP row sums); wavefronts 0-3
//              load V and store it transposed, so that O^T = V^T P^T takes its B operand P
//              straight from the score registers (MFMA 32x32x16 bf16, fp32 accumulation, for
//              both products). The next tile's global loads are in flight during the products.
//   key norm   with a workspace, a pass of its own (attn_knorm_kernel) before the attention
//              kernel; else deferred past the product, as a norm into a matrix product can be
//              (the page's items 3-4): the key gamma is folded into each query once, the keys
//              are staged as they are (LayerNorm: centred) and each key's rstd scales its
//              column of scores in fp32. A key is read by every query block of every query
//              head of its group; normalising it there in full would repeat that vector work
//              for each of them.
//
// Numerics: with the key pass, the normalised queries and keys are each rounded once to bf16;
// with the deferred key norm, the normalised queries times the key gamma are, and the keys
// enter the product exactly (LayerNorm: centred, rounded once to bf16). Scores and output
// accumulate in fp32, the weights P are rounded to bf16 for the second product, and O is
// rounded once to bf16.
#include <cmath>
#include <type_traits>

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
constexpr int kVRow = BK + 16; // bf16 per staged row of V^T (one head dimension): 160 bytes
static_assert(BQ == 8 * 32, "eight wavefronts of 32 queries");
static_assert(D == 128 && BK == 64, "the staging maps below assume D = 128 and 64-key tiles");

// Score register r of lane l for 32-key block j holds key 32j + 8(r/4) + 4(l/32) + r%4 of the
// tile. The second product takes the 16 keys 16s .. 16s+15 as the k range of one MFMA step:
// lane l supplies registers 8(s%2) .. 8(s%2)+7 of block s/2, that is keys 16s + 4h + i
// (i < 4) and 16s + 8 + 4h + (i - 4) (i >= 4), h = l / 32, in that order. Its A operand, V^T,
// must list the same keys in the same order; so V^T stores key kk of the tile in slot
// 16(kk/16) + swap of bits 2 and 3 of (kk % 16), and lane half h reads slots 16s + 8h .. +7.
//
// Element (dim d, slot p) of the staged V^T tile. Slots go in 16-byte units of 8; rows are 160
// bytes apart and the unit index is XORed with bits 4-6 of d. Chosen by measurement (the LDS
// bank-conflict counter over candidate strides and XOR patterns, for these exact read and write
// patterns): the 16-byte operand reads are conflict-free and the transposing 8-byte writes
// lose 4 cycles each; the earlier 144-byte rows with bits 4-5 of d cost 4 cycles per read and
// 12 per write.
__device__ __forceinline__ int vt_off(int d, int p) {
  return d * kVRow + ((((p >> 3) ^ ((d >> 4) & 7))) << 3) + (p & 7);
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

template <int NORM, bool KPRE, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_kernel(AttnArgs a) {
  __shared__ __align__(16) uint16_t sk[2][BK * kKRow];
  __shared__ __align__(16) uint16_t svt[2][D * kVRow];
  __shared__ __align__(16) float srs[2][BK];  // per key of the tile: rstd
  constexpr bool LN = NORM == ATTN_LAYERNORM;
  constexpr bool NORMED = NORM != ATTN_NO_NORM;
  // KPRE: the keys arrive normalised (by attn_knorm_kernel); else their norm is deferred
  constexpr bool DEFER = NORMED && !KPRE;
  constexpr float kInvD = 1.0f / (float)D;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int half = lane >> 5, col = lane & 31;

  // workgroup -> (batch, query head, query block). Workgroup ids reach the eight XCDs in turn
  // (id % 8); XCD x gets a contiguous eighth of the (batch, head) pairs, so the heads that
  // share a key/value head share its L2. Without the mask, each head's query blocks follow one
  // another. With it, a block's cost grows with its index, and the XCD takes its heads' longest
  // blocks first, all heads at once, then the next longest (dispatch in decreasing cost leaves
  // no long block for the end).
  const int bid = blockIdx.x, nwg = gridDim.x, nbh = a.B * a.Hq;
  int qbr, bh;
  if (CAUSAL && (nbh & 7) == 0) {
    const int hx = nbh >> 3, i = bid >> 3;
    qbr = i / hx;
    bh = (bid & 7) * hx + (i - qbr * hx);
  } else {
    const int idx = (nwg & 7) == 0 ? (bid & 7) * (nwg >> 3) + (bid >> 3) : bid;
    qbr = idx % a.qblocks;
    bh = idx / a.qblocks;
  }
  const int head = bh % a.Hq, b = bh / a.Hq;
  const int qb = CAUSAL ? a.qblocks - 1 - qbr : qbr;
  const int hk = head / (a.Hq / a.Hk);
  const int S = a.S;
  const int q0 = qb * BQ;
  const int wq0 = q0 + wave * 32;  // this wavefront's first query
  const int myq = wq0 + col;       // the query lane l owns
  const bool wactive = wq0 < S;
  const int wlast = min(wq0 + 31, S - 1);

  bf16x8_t qf[8];
  float c2 = 0.0f;

  // ---- staging roles: wavefronts 4-7 stage K, 0-3 stage V. Thread st of a role owns the
  // 16-byte chunk sc (dims 8sc .. 8sc+7) of K rows srow + 16i, or of V keys 4srow + i, i < 4.
  // the role is uniform in the wavefront: the tile's base address is then a scalar, and each
  // load adds this lane's 32-bit byte offset (token strides are below 2^24, checked on the host)
  const bool kstage = __builtin_amdgcn_readfirstlane(wave) >= 4;
  const int st = t & 255, sc = st & 15, srow = st >> 4;
  const int64_t sld = kstage ? a.ldk : a.ldv;
  const char *sbase = reinterpret_cast<const char *>((kstage ? a.k : a.v) +
                                                     (int64_t)b * S * sld + (int64_t)hk * D);
  int srows[4];
  uint32_t soff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    srows[i] = kstage ? srow + 16 * i : 4 * srow + i;
    soff[i] = (uint32_t)(((int64_t)srows[i] * sld + sc * 8) * 2);
  }
  uint4 pre[4];
  auto load_tile = [&](int kb) {
    const char *tb = sbase + (int64_t)kb * BK * sld * 2;
    if (kb * BK + BK <= S) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pre[i] = *reinterpret_cast<const uint4 *>(tb + soff[i]);
    } else {  // the last tile: rows past the end read the last row, masked out of the scores
      const int last = S - 1 - kb * BK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = srows[i] < last ? srows[i] : last;
        pre[i] = *reinterpret_cast<const uint4 *>(tb + (uint32_t)(((int64_t)r * sld + sc * 8) * 2));
      }
    }
  };
  auto stage_tile = [&](int buf) {
    if (kstage) {
      if constexpr (!(DEFER && LN)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<uint4 *>(&sk[buf][(srow + 16 * i) * kKRow + sc * 8]) = pre[i];
      }
      if constexpr (DEFER) {
        // the statistics of the four keys, two passes over each key's 128 values (16 lanes,
        // DPP row sums; the four rows interleaved), each pass unpacking the loaded values
        float mean[4] = {0.0f, 0.0f, 0.0f, 0.0f}, q2[4];
        if constexpr (LN) {
          float sm[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x[8];
            unpack8(pre[i], x);
            sm[i] = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) sm[i] += x[e];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) mean[i] = row16_sum(sm[i]) * kInvD;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x[8];
          unpack8(pre[i], x);
          q2[i] = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float d = x[e] - mean[i];
            q2[i] = __builtin_fmaf(d, d, q2[i]);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) q2[i] = rsqrt_f32(row16_sum(q2[i]) * kInvD + a.eps);
        if constexpr (LN) {  // the centred keys
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x[8];
            unpack8(pre[i], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] -= mean[i];
            *reinterpret_cast<uint4 *>(&sk[buf][(srow + 16 * i) * kKRow + sc * 8]) = pack8(x);
          }
        }
        if (sc == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) srs[buf][srow + 16 * i] = q2[i];
        }
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
  // m: the exponent offset (log2 units) of this query's weights, kept within kSlack of the
  // running maximum: O and l are rescaled only when the maximum outgrows it, so the weights
  // stay below 2^kSlack. l: this lane's share of the sum of the weights (fp32).
  constexpr float kSlack = 8.0f;
  float m = -INFINITY, l = 0.0f;

  // One key tile: the two products and the softmax update between them. MASK: the tile holds
  // keys past the end or (causal) after some query of the workgroup; only those tiles pay for
  // the per-score test, and only there do wavefronts whose queries all precede the tile skip
  // it. Every wavefront of the workgroup takes part in the staging and the barrier.
  auto tile = [&](int kb, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int buf = kb & 1;
    if (kb + 1 < nkt) load_tile(kb + 1);
    const int k0 = kb * BK;
    if (!MASK || (wactive && (!CAUSAL || k0 <= wlast))) {
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
      // the key statistics: register r of block j is key 32j + 8(r/4) + 4h + r%4
      if constexpr (DEFER) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int k4 = 32 * j + 8 * g + 4 * half;
            const float4 rs = *reinterpret_cast<const float4 *>(&srs[buf][k4]);
            const float rv[4] = {rs.x, rs.y, rs.z, rs.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) s[j][4 * g + i] *= rv[i];
          }
      }
      if constexpr (MASK) {
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
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * c;
      // key 0 is in the first tile of every query, so m is finite from the first tile on
      if (__any(mx > m + kSlack)) {
        // a real branch: the compiler would otherwise turn it into 64 multiplies by 1
        asm volatile("" ::: "memory");
        const float mnew = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j][r], c, -m));
          s[j][r] = p;
          l += p;
        }
      // V^T operand rows: vt_off(32dt + col, 16ss + 8h). With d = 32dt + col, bits 4-6 of d
      // are 2dt + col/16, so the unit index (2ss + h) ^ (2dt + col/16) is
      // 2(ss ^ dt) + (h ^ col/16): one per-lane base plus a constant per (dt, ss).
      const uint16_t *vrow = &svt[buf][col * kVRow + 8 * (half ^ (col >> 4))];
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
              vrow + dt * 32 * kVRow + 16 * (ss ^ dt));
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, o[dt], 0, 0, 0);
        }
      }
    }
    if (kb + 1 < nkt) stage_tile(buf ^ 1);
    __syncthreads();
  };

  // Tiles before kb_mask need no test for any query of the workgroup: they end at or before
  // the last whole tile of the sequence and (causal) before the workgroup's first query.
  int kb_mask = S / BK;
  if (CAUSAL && q0 / BK < kb_mask) kb_mask = q0 / BK;
  if (kb_mask > nkt) kb_mask = nkt;
  load_tile(0);  // in flight while the queries are normalised
  // ---- this wavefront's queries as MFMA B operands: lane l holds dims 16ks + 8h .. +7 of
  // query l % 32 in qf[ks]. With a norm, the query is normalised (q'). When the key norm is
  // deferred (DEFER), the key gamma is folded in, qf = bf16(q' * gamma_k), the keys enter the
  // product as they are (LayerNorm: centred as they are staged, rounded once to bf16) and
  // their own rstd scales the scores:
  //   q' . k'_j = rstd_j * (qf . (k_j [- mean_j])) [+ q' . beta_k]
  // (brackets: LayerNorm). The last term is the same for every key of the query, so the
  // softmax drops it; it returns in lse (c2).
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
      const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int d0 = ks * 16 + half * 8;
        float g[8], be[8], gk[8], bk[8];
        unpack8(*reinterpret_cast<const uint4 *>(a.wq + d0), g);
        if constexpr (LN) unpack8(a.bq ? *reinterpret_cast<const uint4 *>(a.bq + d0) : zero, be);
        if constexpr (DEFER) {
          unpack8(*reinterpret_cast<const uint4 *>(a.wk + d0), gk);
          if constexpr (LN) unpack8(a.bk ? *reinterpret_cast<const uint4 *>(a.bk + d0) : zero, bk);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float y = (x[ks][i] - mean) * rstd * g[i];  // q'
          if constexpr (LN) y += be[i];
          if constexpr (DEFER) {
            if constexpr (LN) c2 = __builtin_fmaf(y, bk[i], c2);
            y *= gk[i];
          }
          x[ks][i] = y;
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = __builtin_bit_cast(bf16x8_t, pack8(x[ks]));
    if constexpr (LN && DEFER) c2 += __shfl_xor(c2, 32);
  }

  stage_tile(0);
  __syncthreads();
  int kb = 0;
  for (; kb < kb_mask; ++kb) tile(kb, std::false_type{});
  for (; kb < nkt; ++kb) tile(kb, std::true_type{});

  // ---- O = O^T's column / sum, rounded once; lse = ln(sum) + offset (+ the dropped term)
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
    if (a.lse && half == 0) {
      float v = (m + __log2f(lt)) * 0.69314718055994531f;
      if constexpr (LN && DEFER) v = __builtin_fmaf(a.scale, c2, v);
      a.lse[((int64_t)b * a.Hq + head) * S + myq] = v;
    }
  }
}

// The key norm as a pass of its own, for calls whose keys are each read by many query blocks
// and heads: 16 lanes per key vector (8 values each; two passes over the values in registers,
// DPP row sums), y = (x - mean) * rstd * gamma (+ beta), rounded once to bf16, stored densely
// as [B * S][Hk][D].
template <bool LN>
__global__ __launch_bounds__(256) void attn_knorm_kernel(KnormArgs a) {
  constexpr float kInvD = 1.0f / (float)D;
  const int t = threadIdx.x, sc = t & 15;
  const int64_t kv = (int64_t)blockIdx.x * 16 + (t >> 4);
  const int64_t kvc = kv < a.nkeys ? kv : a.nkeys - 1;
  const int64_t tok = kvc / a.Hk, h = kvc - tok * a.Hk;
  float x[8], g[8], be[8];
  unpack8(*reinterpret_cast<const uint4 *>(a.k + tok * a.ldk + h * D + sc * 8), x);
  unpack8(*reinterpret_cast<const uint4 *>(a.wk + sc * 8), g);
  if constexpr (LN)
    unpack8(a.bk ? *reinterpret_cast<const uint4 *>(a.bk + sc * 8) : make_uint4(0u, 0u, 0u, 0u),
            be);
  float mean = 0.0f;
  if constexpr (LN) {
    float sm = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sm += x[e];
    mean = row16_sum(sm) * kInvD;
  }
  float q2 = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float d = x[e] - mean;
    q2 = __builtin_fmaf(d, d, q2);
  }
  const float rstd = rsqrt_f32(row16_sum(q2) * kInvD + a.eps);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float y = (x[e] - mean) * rstd * g[e];
    x[e] = LN ? y + be[e] : y;
  }
  if (kv < a.nkeys) *reinterpret_cast<uint4 *>(a.out + kv * D + sc * 8) = pack8(x);
}

template <int NORM, bool KPRE>
hipError_t launch_norm(bool causal, dim3 grid, dim3 block, hipStream_t s, const AttnArgs &a) {
  return causal ? launch(attn_fwd_kernel<NORM, KPRE, true>, grid, block, s, a)
                : launch(attn_fwd_kernel<NORM, KPRE, false>, grid, block, s, a);
}

} // namespace

norm_status_t launch_key_norm(bool layernorm, const KnormArgs &a, hipStream_t s) {
  const int64_t wg = (a.nkeys + 15) / 16;
  if (wg <= 0 || wg > 0x7fffffffLL) return NORM_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)wg), block(256);
  const hipError_t e = layernorm ? launch(attn_knorm_kernel<true>, grid, block, s, a)
                                 : launch(attn_knorm_kernel<false>, grid, block, s, a);
  return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

norm_status_t launch_attention(int norm, bool keys_normed, bool causal, const AttnArgs &a,
                               hipStream_t s) {
  const int64_t wg = (int64_t)a.B * a.Hq * a.qblocks;
  if (wg <= 0 || wg > 0x7fffffffLL) return NORM_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)wg), block(kThreads);
  hipError_t e;
  switch (norm) {
  case ATTN_LAYERNORM:
    e = keys_normed ? launch_norm<ATTN_LAYERNORM, true>(causal, grid, block, s, a)
                    : launch_norm<ATTN_LAYERNORM, false>(causal, grid, block, s, a);
    break;
  case ATTN_RMSNORM:
    e = keys_normed ? launch_norm<ATTN_RMSNORM, true>(causal, grid, block, s, a)
                    : launch_norm<ATTN_RMSNORM, false>(causal, grid, block, s, a);
    break;
  case ATTN_NO_NORM: e = launch_norm<ATTN_NO_NORM, false>(causal, grid, block, s, a); break;
  default: return NORM_ERR_INVALID_ARG;
  }
  return e == hipSuccess ? NORM_OK : NORM_ERR_HIP;
}

} // namespace dln
