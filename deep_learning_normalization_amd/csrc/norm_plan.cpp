// norm_plan.cpp -- shape dispatcher and argument checks (host only, no HIP).
//
// Scheme choice follows the method's split between short and long reductions (web page
// "PyTorch atinge desempenho SOTA em normalização com torch.compile", matsubara.tec.br,
// para. 5: rows of about a thousand elements or fewer are reduced whole, without a loop; para. 6:
// very large shapes are their own class; paras. 9 and 11: the number of rows each block sums into
// the workspace trades parallelism against workspace traffic):
//   N <= 1024                       -> wave scheme (one row per wavefront, registers only)
//   row fits a team's registers      -> block scheme (one row per team of wavefronts)
//   otherwise                        -> split scheme (a row spread over several workgroups)
// The persistent grid size sets how many partial rows the backward writes (its SPLIT_SIZE).
#include "norm_plan.hpp"

#include <cmath>

namespace dln {
namespace {

Tuning g_tuning;

constexpr int64_t kMaxN = 2147483647;   // row length fits a 32-bit int
constexpr int64_t kMaxGrid = 2147483647; // workgroups per launch
constexpr int kWaveThreads = 256;        // wave scheme: four one-wave teams per workgroup
constexpr int kSplitThreads = 256;
constexpr int kWaveMaxRow = 1024;        // wave scheme for rows up to this many elements
constexpr int kBlockTeamTarget = 256;    // preferred largest team for the block scheme
constexpr int kBlockTeamTargetBwd = 640; // the backward prefers one access per thread longer
constexpr int kLoopThreads = 512;        // looped backward: workgroup (= team) size bound
constexpr int kLoopSegFull = 4;          // looped backward: full-width accesses per thread
constexpr int64_t kLoopTwoMaxAcc = 1792; // looped backward: longest row (16-byte accesses) run
                                         // two workgroups per CU
constexpr int kLoopSeg3 = 3;             // looped backward: segments of the short 16-bit
                                         // LayerNorm kernel
constexpr int kLoopMaxEq = kLoopThreads * kLoopSegFull; // longest row, full-width accesses

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
bool valid_kind(int k) { return k == NORM_LAYERNORM || k == NORM_RMSNORM; }
bool valid_dtype(int d) {
  return d == NORM_F32 || d == NORM_BF16 || d == NORM_BF16_F32W || d == NORM_F16 ||
         d == NORM_F16_F32W;
}
int vec_epv(norm_dtype_t d) { return d == NORM_F32 ? 4 : 8; }
// bytes per element of the activations (X, R, Y, H, dY, dH, dX, dR) and of W, B, dW, dB
size_t elem_size(int d) { return d == NORM_F32 ? 4 : 2; }
size_t weight_size(int d) { return (d == NORM_BF16 || d == NORM_F16) ? 2 : 4; }
// Pointer alignment an access of e elements needs: e activation elements in one load, and the
// matching e weights (read 16 bytes at a time when they span 16 bytes or more).
size_t access_align(int d, int e) {
  const size_t act = (size_t)e * elem_size(d), w = (size_t)e * weight_size(d);
  const size_t wneed = w < 16 ? w : 16;
  return act > wneed ? act : wneed;
}
int lb_of(int threads) { return threads <= 256 ? 256 : threads <= 512 ? 512 : 1024; }

// Access width classes: element-wise, full (16-byte) vectors, narrow (8- or 4-byte) vectors.
// Narrow shapes are given in full-width units: the kernel runs vpt * scale narrow accesses.
enum Width { kElem = 0, kFull = 1, kNarrow = 2 };

// Compiled kernel shapes (must match the menus in the kernel sources).
bool wave_menu(int wc, int vpt, int rows) {
  if (wc == kElem) return rows == 1 && (vpt == 1 || vpt == 2 || vpt == 4 || vpt == 8 || vpt == 16);
  if (wc == kNarrow) return rows == 1 && (vpt == 1 || vpt == 2 || vpt == 4);
  switch (vpt) {
  case 1:
  case 2: return rows == 1 || rows == 2 || rows == 4;
  case 4: return rows == 1 || rows == 2;
  case 8: return rows == 1;
  default: return false;
  }
}

// 4-byte accesses (scale 4) need an address register pair per access once the accesses of a
// thread span more than the load's immediate offset; shapes that then spill are left out: the
// residual forward beyond 4 full-width accesses per 256 threads, and 1024-thread backwards.
bool narrow_spills(int sc, bool bwd, bool resid, int vpt, int lb) {
  if (sc < 4) return false;
  if (bwd) return lb >= 1024;
  return resid && vpt * (lb / 256) > 4;
}

bool block_menu(int wc, bool bwd, int vpt, int rows, int lb, int sc = 1, bool resid = false) {
  if (wc == kElem) return lb == 1024 && rows == 1 && (vpt == 4 || vpt == 8);
  if (wc == kNarrow) {
    if (rows != 1 || narrow_spills(sc, bwd, resid, vpt, lb)) return false;
    switch (lb) {
    case 256: return vpt == 1 || vpt == 2 || vpt == 4 || (!bwd && vpt == 8);
    case 512: return vpt == 1 || vpt == 2 || (!bwd && vpt == 4);
    case 1024: return vpt == 1 || (!bwd && vpt == 2);
    default: return false;
    }
  }
  switch (lb) {
  case 256:
    return (vpt == 1 && (rows == 1 || rows == 2 || rows == 4)) ||
           (vpt == 2 && (rows == 1 || rows == 2 || rows == 4)) || (vpt == 4 && rows == 1) ||
           (vpt == 8 && rows == 1);
  case 512:
    return (vpt == 1 && (rows == 1 || rows == 2 || rows == 4)) ||
           (vpt == 2 && (rows == 1 || rows == 2)) || (vpt == 4 && rows == 1);
  case 768: return vpt == 1 && (rows == 1 || rows == 2);
  case 1024:
    return (vpt == 1 && (rows == 1 || rows == 2)) || (vpt == 2 && rows == 1);
  default: return false;
  }
}

// Register budget: a 1024-thread workgroup leaves 128 VGPRs per lane, 512 threads 256. The
// backward holds more per access (prefetched X and dY, dW and dB accumulators), so it gets
// fewer accesses per thread; these limits are the compiled shapes that do not spill.
bool block_fits_registers(int wc, bool bwd, int vpt, int rows, int lb) {
  const int slots = vpt * rows;
  if (wc == kElem) return !bwd || vpt <= 4;
  if (!bwd) {
    if (lb >= 1024) return slots <= 2;
    if (lb >= 512) return slots <= 4;
    return slots <= 8;
  }
  if (lb >= 768) return vpt == 1 && slots <= 2;
  if (lb >= 512) return vpt <= 2 && slots <= 4;
  return vpt <= 4 && slots <= 8;
}

bool split_fwd_menu(int wc, int vpt) {
  if (wc == kElem) return vpt == 8;
  if (wc == kNarrow) return vpt == 4;
  return vpt == 1 || vpt == 2 || vpt == 4;
}
bool split_bwd_menu(int wc, int vpt, int rows) {
  if (wc == kElem) return vpt == 8 && rows == 1;
  if (wc == kNarrow) return vpt == 4 && rows == 1;
  switch (vpt) {
  case 1:
  case 2: return rows == 1 || rows == 2 || rows == 4;
  case 4: return rows == 1 || rows == 2;
  default: return false;
  }
}

} // namespace

const Tuning &tuning() { return g_tuning; }

norm_status_t set_tuning(norm_tune_t key, int64_t v) {
  switch (key) {
  case NORM_TUNE_SCHEME:
    if (v != -1 && v != NORM_SCHEME_WAVE && v != NORM_SCHEME_BLOCK && v != NORM_SCHEME_SPLIT &&
        v != NORM_SCHEME_LOOP)
      return NORM_ERR_INVALID_ARG;
    g_tuning.scheme = (int)v;
    return NORM_OK;
  case NORM_TUNE_GRID_PER_CU:
    if (v != -1 && (v < 1 || v > 4096)) return NORM_ERR_INVALID_ARG;
    g_tuning.grid_per_cu = (int)v;
    return NORM_OK;
  case NORM_TUNE_ROWS_PER_ITER:
    if (v != -1 && v != 1 && v != 2 && v != 4) return NORM_ERR_INVALID_ARG;
    g_tuning.rows = (int)v;
    return NORM_OK;
  case NORM_TUNE_TEAM_THREADS:
    if (v != -1 && (v < 64 || v > 1024 || v % 64 != 0)) return NORM_ERR_INVALID_ARG;
    g_tuning.team_threads = (int)v;
    return NORM_OK;
  case NORM_TUNE_SPLIT_CHUNK:
    if (v != -1 && (v < 1 || v > kMaxN)) return NORM_ERR_INVALID_ARG;
    g_tuning.split_chunk = v;
    return NORM_OK;
  case NORM_TUNE_ROW_GROUPS:
    if (v != -1 && v < 1) return NORM_ERR_INVALID_ARG;
    g_tuning.row_groups = v;
    return NORM_OK;
  case NORM_TUNE_TEAMS_PER_WG:
    if (v != -1 && (v < 1 || v > 16)) return NORM_ERR_INVALID_ARG;
    g_tuning.teams = (int)v;
    return NORM_OK;
  case NORM_TUNE_ROW_ORDER:
    if (v != -1 && v != 0 && v != 1) return NORM_ERR_INVALID_ARG;
    g_tuning.row_order = (int)v;
    return NORM_OK;
  case NORM_TUNE_SPLIT_EXCHANGE:
    if (v != -1 && v != 0 && v != 1) return NORM_ERR_INVALID_ARG;
    g_tuning.xchg = (int)v;
    return NORM_OK;
  case NORM_TUNE_EXCHANGE_POLLS:
    if (v != -1 && (v < 1 || v > kXchgPollsMax)) return NORM_ERR_INVALID_ARG;
    g_tuning.xchg_polls = v;
    return NORM_OK;
  case NORM_TUNE_EXCHANGE_WITHHOLD:
    if (v != -1 && v != 0 && v != 1) return NORM_ERR_INVALID_ARG;
    g_tuning.xchg_withhold = (int)v;
    return NORM_OK;
  case NORM_TUNE_UNALIGNED:
    if (v != -1 && v != 0 && v != 1) return NORM_ERR_INVALID_ARG;
    g_tuning.unaligned = (int)v;
    return NORM_OK;
  case NORM_TUNE_ATTN_KEY_PASS:
    if (v != -1 && v != 0 && v != 1) return NORM_ERR_INVALID_ARG;
    g_tuning.attn_key_pass = (int)v;
    return NORM_OK;
  default: return NORM_ERR_INVALID_ARG;
  }
}

norm_status_t make_plan(norm_kind_t kind, norm_dtype_t dtype, norm_pass_t pass, int64_t M,
                        int64_t N, int residual, int align, int phase0, int dphase, int cu,
                        const Tuning &t, Plan *out) {
  if (!out || !valid_kind(kind) || !valid_dtype(dtype) ||
      (pass != NORM_PASS_FWD && pass != NORM_PASS_BWD && pass != NORM_PASS_STATS) || M < 0 ||
      N <= 0 || N > kMaxN ||
      cu <= 0)
    return NORM_ERR_INVALID_ARG;
  Plan p;
  const bool bwd = pass == NORM_PASS_BWD;
  const bool stats = pass == NORM_PASS_STATS; // the forward's kernels without Y
  // The widest whole-word access (16, 8, then 4 bytes; at least two elements) that divides the
  // row length and that every pointer's alignment allows; else one element per access.
  const int ev = vec_epv(dtype);
  p.epv = 1;
  for (int e = ev; e >= 2; e /= 2)
    if (N % e == 0 && align > 0 && (size_t)align >= access_align(dtype, e)) {
      p.epv = e;
      break;
    }
  // Rows off 16-byte boundaries (their length, stride or start) with every [M, N] tensor at
  // one phase: the wave and block schemes still take 16-byte accesses, each workgroup on the
  // rows of one phase class (see the team kernels), in place of element-wise and of 8- and
  // 4-byte accesses unless tuned off (measured on MI355X against 8- / 4-byte accesses:
  // LayerNorm 16384 x 4100 forward 61 / 57 us, backward 96 / 96-100 us; 16384 x 4098 61 / 66,
  // 96 / 145 us; RMSNorm 32768 x 4100 92 / 105, 140 / 187 us; LayerNorm 65536 x 1002 56 / 56,
  // 75 / 80 us).
  int64_t nal = 0;
  int period = 0;
  // (rows of at least one access: a row's edge accesses load its first and last 16 bytes)
  if (p.epv < ev && N >= ev && t.unaligned != 0 && phase0 >= 0 && dphase >= 0) {
    int g = ev; // gcd(dphase, ev): rows repeat their phase every ev / g rows
    if (dphase % ev) {
      int x = dphase % ev, y = ev;
      while (x) {
        const int r = y % x;
        y = x;
        x = r;
      }
      g = y;
    }
    period = ev / g;
    for (int c = 0; c < period; ++c) {
      const int pe = (int)((phase0 + (int64_t)c * dphase) % ev);
      const int64_t n = cdiv(N + pe, ev);
      if (n > nal) nal = n;
    }
    // the scheme a full-width row of this length takes (below)
    int sch = t.scheme == NORM_SCHEME_LOOP && !bwd ? NORM_SCHEME_AUTO : t.scheme;
    if (sch == NORM_SCHEME_AUTO)
      sch = N <= kWaveMaxRow ? NORM_SCHEME_WAVE
            : nal <= (bwd ? 1024 : 2048) ? NORM_SCHEME_BLOCK
                                         : NORM_SCHEME_SPLIT;
    // (the wave backward over phase classes is compiled up to 4 accesses per thread only: its
    // 8-access form gave wrong results on MI355X, cause not found, and is never launched)
    const bool wave_ok = sch == NORM_SCHEME_WAVE && !(bwd && nal > 4 * 64);
    if (wave_ok || sch == NORM_SCHEME_BLOCK) {
      p.epv = ev;
      p.period = period;
    }
  }
  p.vector = p.epv > 1 ? 1 : 0;
  p.scale = p.vector ? ev / p.epv : 1;
  p.access_bytes = (int)((size_t)p.epv * elem_size(dtype));
  const bool vec = p.vector != 0;
  const int wc = !vec ? kElem : p.scale == 1 ? kFull : kNarrow;
  const int sc = p.scale;
  const int64_t nacc = p.period ? nal : N / p.epv;
  p.nacc = nacc;
  // rows of the largest phase class (every row without classes); grids count its workgroups
  // and are multiplied by the classes at the end
  const int64_t PC = p.period ? p.period : 1;
  const int64_t Mc = cdiv(M > 0 ? M : 1, PC);
  // accesses per row in full-width units: the narrow paths size teams and pick schemes as the
  // 16-byte path would for the same row
  const int64_t nacc_eq = cdiv(nacc, sc);
  const int64_t Mm = M > 0 ? M : 1; // M == 0 launches nothing; size as one row

  int scheme = t.scheme;
  // the looped scheme is the backward's; a forced one leaves the forward to the choice below
  if (scheme == NORM_SCHEME_LOOP && !bwd) scheme = NORM_SCHEME_AUTO;
  if (scheme == NORM_SCHEME_AUTO) {
    if (N <= kWaveMaxRow)
      scheme = NORM_SCHEME_WAVE;
    else if (nacc_eq <= (!vec ? (bwd ? 4096 : 8192) : (bwd || (sc == 4 && residual)) ? 1024 : 2048))
      scheme = NORM_SCHEME_BLOCK;
    else if (bwd && vec && sc <= 2 && nacc_eq <= kLoopMaxEq)
      scheme = NORM_SCHEME_LOOP;
    else
      scheme = NORM_SCHEME_SPLIT;
  }
  p.scheme = scheme;

  if (scheme == NORM_SCHEME_WAVE) {
    static const int menu[] = {1, 2, 4, 8, 16};
    int vpt = 0;
    for (int v : menu)
      if (64LL * v * sc >= nacc && wave_menu(wc, v, 1)) {
        vpt = v;
        break;
      }
    if (!vpt) return NORM_ERR_UNSUPPORTED;
    int rows = t.rows > 0 ? t.rows : 1;
    // Backwards of 16-bit rows of at most one 16-byte access per lane (N <= 512) hold several
    // rows per wavefront: four for RMSNorm, two for LayerNorm (measured on MI355X, bf16, one
    // row against four / two: RMSNorm 65536 x 256 43.4 -> 28.9 us, 65536 x 512 50.0 -> 40.2,
    // 262144 x 512 177.8 -> 139.2, fp16 65536 x 512 49.3 -> 40.6; LayerNorm 65536 x 256 37.1 ->
    // 35.7, 65536 x 512 44.2 -> 42.0, 262144 x 512 147.9 -> 140.4). Two accesses per lane
    // (768, 1024) gain nothing from more rows and lose 10-40% with four. fp32 rows of at most
    // 256 elements alike (65536 rows: RMSNorm 48.6 -> 39.6 us, LayerNorm 43.4 -> 39.9), and
    // fp32 weights beside bf16 rows (RMSNorm 65536 x 512 51.1 -> 40.7).
    if (t.rows <= 0 && bwd && vpt == 1 && sc == 1 && !p.period && !residual)
      rows = kind == NORM_RMSNORM ? 4 : 2;
    if (!wave_menu(wc, vpt, rows)) rows = 1;
    p.vpt = vpt * sc;
    p.rows = rows;
    p.threads = kWaveThreads;
    p.lb = kWaveThreads;
    p.team_threads = 64;
    const int64_t groups = cdiv(Mc, (int64_t)(kWaveThreads / 64) * rows);
    // 8- and 4-byte forwards stream better from 16 workgroups per CU (measured on MI355X:
    // LayerNorm 65536 x 1002 57.8 -> 53.4 us)
    const int64_t gpc = t.grid_per_cu > 0 ? t.grid_per_cu : (bwd ? 2 : sc > 1 ? 16 : 8);
    const int64_t cap = cu * gpc / PC > 0 ? cu * gpc / PC : 1; // per phase class
    p.grid = PC * (groups < cap ? groups : cap);
    p.row_order = t.row_order > 0 ? 1 : 0;
  } else if (scheme == NORM_SCHEME_BLOCK) {
    static const int vmenu[] = {1, 2, 4, 8};
    static const int smenu[] = {4, 8};
    const int *menu = vec ? vmenu : smenu;
    const int nmenu = vec ? 4 : 2;
    int vpt = 0, tt = 0, rows = 1, lb_pick = 1024;
    // pass 0: the team size override if one is set, else the preferred team size;
    // pass 1: any team size up to 1024 (an override that cannot hold the row is ignored)
    for (int pass_i = 0; pass_i < 2 && !vpt; ++pass_i) {
      const bool use_override = pass_i == 0 && t.team_threads > 0;
      for (int i = 0; i < nmenu && !vpt; ++i) {
        const int v = menu[i];
        int cand = (int)(cdiv(cdiv(nacc, (int64_t)v * sc), 64) * 64);
        if (use_override) {
          if ((int64_t)t.team_threads * v * sc < nacc) continue;
          cand = t.team_threads;
        }
        // forward: teams up to 256 threads, or 512 with four accesses per thread rather than
        // eight (measured on MI355X: 12288-16384 bf16 rows run 10-20% faster). Rows over phase
        // classes, which often need one access past a power of two (N = 4097: 513), take two
        // accesses per thread up to 384 threads and, in the backward, one up to 512 (measured on
        // MI355X, LayerNorm 16384 x 4097: forward 4 x 192 threads 68 us, 2 x 320 62 us;
        // backward 1 x 576 121 us, 2 x 320 with two rows 96 us)
        const bool part = p.period > 0;
        const int fwd_limit = v >= 4 ? 2 * kBlockTeamTarget
                              : (part && v == 2) ? kBlockTeamTarget + 128 : kBlockTeamTarget;
        const int bwd_limit = part && v == 1 ? 512 : kBlockTeamTargetBwd;
        const int limit = (pass_i == 0 && !use_override)
                              ? (vec ? (bwd ? bwd_limit : fwd_limit) : 1024)
                              : 1024;
        if (cand > limit) continue;
        // Backward teams of 513-768 threads with one full-width access per thread are compiled
        // for 768 threads (3 wavefronts per SIMD, about 170 VGPRs), which holds two rows without
        // spilling; a 1024-thread bound leaves 128 VGPRs, and the two-row kernel spilled there.
        const bool mid = bwd && wc == kFull && v == 1 && cand > 512 && cand <= 768;
        const int lb = mid ? 768 : vec ? lb_of(cand) : 1024;
        // Backward teams of up to 512 threads with one access per thread hold two rows at
        // once by default (measured on MI355X, with the saved statistics prefetched as well:
        // fewer, fuller workgroups; wider teams or more accesses per thread do better with one).
        // Teams of 513-768 threads: two rows for RMSNorm, one for LayerNorm (measured on one
        // GPU at 640 threads: RMSNorm 32768 x 5120 197 against 202 us; LayerNorm 32768 x 5120
        // 228 against 188 us, fp32 32768 x 2560 200 against 174 us)
        const int two_upto = kind == NORM_RMSNORM ? 768 : 512;
        const bool two = bwd && ((v == 1 && cand <= two_upto) || (part && v == 2 && cand <= 384));
        int r = t.rows > 0 ? t.rows : (two ? 2 : 1);
        const bool res = residual != 0;
        auto ok = [&](int rr) {
          return block_menu(wc, bwd, v, rr, lb, sc, res) &&
                 block_fits_registers(wc, bwd, v, rr, lb);
        };
        // RMSNorm backward over bf16 rows on 256-thread teams with one access each (rows of
        // 1544-2048 elements): four rows at a time, so half the workgroups and half the dW
        // partial rows (measured on MI355X, 32768 rows: 1600 68.8 -> 66.0 us, 1792 72.0 ->
        // 66.2, 2048 75.2 -> 71.6; 65536 x 2048 143.2 -> 137.9; but fp16 2048 75.4 against
        // 77.2, and no gain at 1536 or 1280 (192-thread teams) or for LayerNorm, which loses)
        // Rows over phase classes on 320-384-thread teams with one access each hold four rows
        // too (measured on MI355X: LayerNorm bf16 16384 x 2049 83.9 -> 77.0 us, fp16 87.9 ->
        // 79.0, fp32 16384 x 1025 73.7 -> 65.3; RMSNorm 32768 x 2049 122.1 -> 111.9; 2561 a
        // 1-4% gain; teams of 256 threads or fewer lose 1-8% and 448-512 threads tie)
        const bool four = bwd && !res && v == 1 && t.rows <= 0 &&
                          ((kind == NORM_RMSNORM && dtype == NORM_BF16 && wc == kFull && !part &&
                            cand == 256) ||
                           (part && cand >= 320 && cand <= 384 && dtype != NORM_BF16_F32W &&
                            dtype != NORM_F16_F32W));
        if (four && ok(4)) r = 4;
        if (!ok(r)) r = 1;
        if (!ok(r)) continue;
        vpt = v;
        tt = cand;
        rows = r;
        lb_pick = lb;
      }
    }
    if (!vpt) return NORM_ERR_UNSUPPORTED;
    // RMSNorm backward over 16-bit rows (16-bit weights) of 576-768 full-width accesses
    // (4608-6144 elements), aligned, no residual: 256-thread teams with four accesses each,
    // one row at a time, beat the 576-768-thread teams with one access (measured on MI355X,
    // bf16, 32768 rows: 4608 183.8 -> 179.5 us, 5120 190.3 -> 182.5, 6144 216.3 -> 198.6;
    // 16384 x 5120 99.6 -> 95.4), but not at 4352 (175.8 against 179.4), at fp32 2560 (178
    // against 189), for the residual form at 7168 or for LayerNorm (5120: 175 against 221).
    if (bwd && kind == NORM_RMSNORM && !residual && vec && wc == kFull && !p.period &&
        (dtype == NORM_BF16 || dtype == NORM_F16) && nacc >= 576 && nacc <= 768 &&
        t.team_threads <= 0 && t.rows <= 0 && block_menu(wc, bwd, 4, 1, 256, sc, false) &&
        block_fits_registers(wc, bwd, 4, 1, 256)) {
      vpt = 4;
      tt = 256;
      rows = 1;
      lb_pick = 256;
    }
    // LayerNorm backward over 16-bit rows of 257-384 accesses (2056-3072 elements): 256-thread
    // teams with two accesses each and one row, two workgroups per CU, instead of 320-384
    // threads with one access and two rows on one (measured on MI355X, bf16, 65536 rows: 2304
    // 224.0 -> 187.6 us, 2560 228.7 -> 186.5, 2816 225.4 -> 193.6, 3072 230.6 -> 204.6; fp16
    // 2560 234.7 -> 208.1; fp32 weights 2560 226.3 -> 181.6; 16384 rows 4-10%)
    if (bwd && kind == NORM_LAYERNORM && !residual && vec && wc == kFull && !p.period &&
        dtype != NORM_F32 && nacc > 256 && nacc <= 384 &&
        t.team_threads <= 0 && t.rows <= 0 && block_menu(wc, bwd, 2, 1, 256, sc, false) &&
        block_fits_registers(wc, bwd, 2, 1, 256)) {
      vpt = 2;
      tt = 256;
      rows = 1;
      lb_pick = 256;
    }
    // Backward: several row teams share a workgroup (up to 1024 threads) when the larger
    // workgroup still fits its registers; their dW/dB partials merge in LDS, so the partial
    // rows written (and re-read by the column reduction) drop by the team count.
    // (a team's partial sums sit at a 16-byte aligned LDS offset: team sizes of 4k wavefronts)
    // Default one team per workgroup: measured on MI355X, separate workgroups (each with its
    // own barrier) outrun one large workgroup whose barrier waits for every wavefront.
    int teams = t.teams > 0 ? t.teams : 1;
    if (tt % 256 != 0) teams = 1;
    while (teams > 1 && (tt * teams > 1024 ||
                         !block_menu(wc, bwd, vpt, rows, lb_of(tt * teams), sc, residual != 0) ||
                         !block_fits_registers(wc, bwd, vpt, rows, lb_of(tt * teams))))
      --teams;
    if (!vec && teams > 1 && tt * teams > 1024) teams = 1;
    p.vpt = vpt * sc;
    p.rows = rows;
    p.team_threads = tt;
    p.threads = tt * teams;
    p.lb = vec ? (teams > 1 ? lb_of(p.threads) : lb_pick) : 1024;
    const int64_t groups = cdiv(Mc, (int64_t)rows * teams);
    const bool wide_fwd =
        !bwd && !stats && vec && wc == kFull && !p.period && vpt == 4 && tt > 256 &&
        (dtype != NORM_F32 ? (kind == NORM_LAYERNORM && !residual) || tt <= 384
                           : kind == NORM_LAYERNORM && !residual && tt <= 320);
    auto capped = [&](int64_t gpc) { // persistent: gpc workgroups per CU over all classes
      const int64_t cap = cu * gpc / PC > 0 ? cu * gpc / PC : 1;
      return PC * (groups < cap ? groups : cap);
    };
    if (bwd) {
      // Backward: persistent, about 1024 16-byte accesses per tensor in flight per CU; every
      // workgroup writes one partial row, so fewer, longer-lived workgroups.
      const int64_t load = (int64_t)p.threads * vpt * rows; // full-width units
      int64_t gpc = 1024 / load > 0 ? 1024 / load : 1;
      // Two-row teams of 16-bit rows with one access per thread round up instead: teams of 192
      // threads (rows of 1032-1536 elements) run three workgroups per CU, RMSNorm teams of
      // 320-384 threads (2056-3072) two (measured on MI355X, bf16, 65536 rows: 1280 RMSNorm
      // 119.8 -> 98.8 us, LayerNorm 126.6 -> 106.8; 1536 RMSNorm 127.1 -> 108.4, LayerNorm
      // 131.3 -> 117.8, fp16 RMSNorm 126.5 -> 109.1; RMSNorm 2560 219.6 -> 168.1, 3072 230.5 ->
      // 203.5; at 16384 rows 5-20% alike). RMSNorm on 448 threads (3584) loses 0-8% with two,
      // and LayerNorm on 320-384 threads loses 4-5% (it takes 256-thread teams instead). fp32
      // rows: RMSNorm on 320-384 threads gains too (65536 x 1280 202.3 -> 166.6, x 1536 216.6
      // -> 210.1), LayerNorm on 320 threads (1280: 192.9 -> 170.3) but not on 384 (1536: 196.6
      // against 218.7). fp32 weights beside 16-bit rows follow the 16-bit rows (65536 rows,
      // RMSNorm 1536 126.1 -> 109.5, 2560 218.0 -> 168.2; LayerNorm 1536 135.0 -> 115.1).
      const bool d16 = dtype != NORM_F32;
      const bool up =
          bwd && vpt == 1 && rows == 2 && sc == 1 && !p.period && !residual &&
          p.threads == p.team_threads &&
          ((d16 && p.threads == 192) ||
           ((d16 || dtype == NORM_F32) && kind == NORM_RMSNORM && p.threads >= 320 &&
            p.threads <= 384) ||
           (dtype == NORM_F32 && kind == NORM_LAYERNORM && p.threads == 320));
      if (up) gpc = cdiv(1024, load);
      p.grid = capped(t.grid_per_cu > 0 ? t.grid_per_cu : gpc);
    } else if (t.grid_per_cu > 0 || stats || sc > 1 || p.period || wide_fwd) {
      // the statistics pass alone, with no stores to overlap, streams best from a persistent
      // grid of 8 workgroups per CU (measured on MI355X: LayerNorm 16384 x 4096 30.6 -> 28.7 us);
      // 8- and 4-byte forwards from 16 (LayerNorm 16384 x 4100 54.4 -> 49.8 us, 16384 x 4098
      // 68.8 -> 60.4 us); forwards over phase classes, whose workgroups gather their weights
      // first, from enough workgroups for about 12 wavefronts per CU (measured on MI355X,
      // LayerNorm 16384 x 2049 / 3073 / 4097 with 3 / 4 / 5 wavefronts each: best at 4 / 3 / 2
      // workgroups per CU, 35 / 44 / 62 us, against 50 / 54 / 108 us from short-lived ones)
      // (4 accesses per thread take about 180 VGPRs, so 2 wavefronts per SIMD: 8 per CU;
      // RMSNorm 16384 x 8185 99 us from 2 workgroups of 4 wavefronts, 108 us from 3)
      // Forwards of 16-bit rows on teams of 320-512 threads with four accesses each (rows of
      // 8200-16384 elements) run from a persistent grid of 2 workgroups per CU (measured on
      // MI355X, 16384 rows, short-lived against persistent: LayerNorm 10240 173.7 -> 130.9 us,
      // 12288 181.4 -> 140.6, 14336 191.1 -> 170.2, 16384 211 -> 181; RMSNorm 10240 144.3 ->
      // 112.0, 12288 150.0 -> 136.7, but 14336 161.2 against 167.1 and 16384 a tie, so RMSNorm
      // keeps short-lived workgroups on teams of more than 384 threads; 8192, on 256 threads,
      // ties either way). The residual form gains on 320-384 threads (16384 x 10240 289.7 ->
      // 238.9 us, x 12288 333.5 -> 275.8) and ties on 512. fp32 weights beside 16-bit rows
      // gain alike (LayerNorm 8200 169.7 -> 114.1, 16384 208.1 -> 181.0; RMSNorm 10240 140.5
      // -> 112.2). fp32 rows gain only for LayerNorm on 320 threads (4100 104.5 -> 95.1, 4608
      // 109.0 -> 101.6, 5120 a tie); on more threads, and for RMSNorm, they lose 1-7% (6144
      // 132.5 -> 140.4) and keep short-lived workgroups.
      const int64_t waves = (p.threads + 63) / 64, budget = vpt >= 4 ? 8 : 12;
      const int64_t gpc_part = budget / waves > 0 ? budget / waves : 1;
      p.grid = capped(t.grid_per_cu > 0 ? t.grid_per_cu
                      : stats                ? 8
                      : p.period             ? gpc_part
                      : wide_fwd             ? 2
                                             : 16);
    } else {
      // Forward (measured on MI355X): short-lived workgroups of two row groups each (the second
      // group's loads overlap the first's reductions), one for the residual variant, whose
      // four streams per row already keep enough requests in flight.
      p.grid = PC * (residual ? groups : cdiv(groups, 2));
    }
    p.row_order = t.row_order > 0 ? 1 : 0;
  } else if (scheme == NORM_SCHEME_LOOP) {
    // one row per workgroup, kLoopSegFull full-width accesses per thread (twice as many 8-byte
    // ones; 4-byte accesses are not compiled for it); one or two resident workgroups per CU,
    // each writing one partial row
    if (!vec || sc > 2 || nacc_eq > kLoopMaxEq) return NORM_ERR_UNSUPPORTED;
    // Teams of the full 512 threads even where fewer would cover the row (the last segments
    // are then partly empty): with one resident workgroup per CU the team size is the CU's
    // whole parallelism (measured on MI355X: RMSNorm 16384 x 12288 297 -> 253 us, fp32
    // 32768 x 4098 705 -> 519 us). A smaller override is taken where it still covers the row.
    // LayerNorm on 16-bit rows of at most 1536 accesses runs a kernel of three segments (127
    // VGPRs against the four-segment kernel's 158), which leaves room for a second workgroup.
    const bool seg3 = kind == NORM_LAYERNORM && dtype != NORM_F32 && sc == 1 && !p.period &&
                      nacc <= kLoopSeg3 * kLoopThreads;
    const int seg = seg3 ? kLoopSeg3 : kLoopSegFull * sc;
    const int need = (int)(cdiv(cdiv(nacc, seg), 64) * 64);
    int tt = kLoopThreads;
    if (t.team_threads > 0 && t.team_threads <= kLoopThreads && t.team_threads >= need)
      tt = t.team_threads;
    p.vpt = seg;
    p.rows = 1;
    p.team_threads = tt;
    p.threads = tt;
    p.lb = kLoopThreads;
    // Two workgroups per CU where the kernel's registers leave room for two 512-thread teams
    // (at most 128 VGPRs: the 16-byte kernels of RMSNorm on 16-bit rows, 124, and of either
    // kind on fp32 rows, 72-93; LayerNorm on 16-bit rows takes 158) and rows of at most 28 KB,
    // so that two rows of X and dY per CU still stay in the L2 between the sweeps. Measured on
    // MI355X, 16384 rows, one against two per CU: RMSNorm bf16 8200 210.2 -> 174.8 us, 10240
    // 237.8 -> 198.0, 12288 258.9 -> 229.9, 14336 313.4 -> 277.5 (fp16, fp32 weights and the
    // residual form alike); fp32 LayerNorm 4100 211.4 -> 175.0, 7168 313.3 -> 282.9; full 32 KB
    // rows tie (bf16 16384) or lose (fp32 8192 309.8 -> 321.6).
    // LayerNorm on 16-bit rows with four segments keeps its dB sums in LDS (127-128 VGPRs) and
    // runs two per CU at every length (16384 rows, one against two: bf16 12800 344.6 -> 277.6
    // us, 14336 353.3 -> 300.5, 16384 363.0 -> 350.5; fp16 12800 337.9 -> 272.2, 14336 347.7
    // -> 295.5, 16384 370.8 -> 351.0; fp32 weights alike; the LDS sums cost nothing at one per
    // CU).
    const bool dbl = kind == NORM_LAYERNORM && sc == 1 && !seg3 && dtype != NORM_F32;
    const bool two = sc == 1 && !p.period &&
                     (((dtype == NORM_F32 || kind == NORM_RMSNORM || seg3) &&
                       nacc <= kLoopTwoMaxAcc) || dbl);
    const int64_t gpc = t.grid_per_cu > 0 ? t.grid_per_cu : two ? 2 : 1;
    p.grid = Mm < cu * gpc ? Mm : cu * gpc;
    p.row_order = 0;
  } else if (scheme == NORM_SCHEME_SPLIT) {
    int vpt = vec ? 4 : 8; // full-width units on the vector paths
    if (t.split_chunk > 0 && wc == kFull) { // the other widths have one chunk size
      const int64_t per = (int64_t)kSplitThreads * p.epv;
      if (t.split_chunk % per) return NORM_ERR_UNSUPPORTED;
      vpt = (int)(t.split_chunk / per);
    }
    if (!split_fwd_menu(wc, vpt)) return NORM_ERR_UNSUPPORTED;
    const int64_t chunk_acc = (int64_t)kSplitThreads * vpt * sc;
    p.vpt = vpt * sc;
    p.threads = kSplitThreads;
    p.lb = kSplitThreads;
    p.team_threads = kSplitThreads;
    p.chunks = cdiv(nacc, chunk_acc);
    p.chunk_elems = chunk_acc * p.epv;
    if (Mm * p.chunks > kMaxGrid) return NORM_ERR_UNSUPPORTED;
    if (!bwd) {
      p.rows = 1;
      p.grid = Mm * p.chunks;
    } else {
      // one (row group, chunk) workgroup per CU for the second pass
      int64_t G = t.row_groups > 0 ? t.row_groups : cdiv((int64_t)cu, p.chunks);
      if (G < 1) G = 1;
      if (G > Mm) G = Mm;
      const int64_t rpg = cdiv(Mm, G);
      G = cdiv(Mm, rpg);
      int rows = t.rows > 0 ? t.rows : (vpt >= 4 ? 1 : 2);
      if (!split_bwd_menu(wc, vpt, rows)) rows = 1;
      if (!split_bwd_menu(wc, vpt, rows)) return NORM_ERR_UNSUPPORTED;
      p.rows = rows;
      p.row_groups = G;
      p.rows_per_group = rpg;
      p.grid = G * p.chunks;
    }
    // The single-pass exchange form (16-byte accesses, the default chunk, no residual input):
    // its whole grid must fit on the device at once, and a row group must hold every chunk of
    // a row. The forward also wants room for two row groups: with one, every workgroup walks
    // every row and the two-pass form streams faster (LayerNorm 4 x 4194304 bf16: 23.9 against
    // 20.9 us). Unless forced, a row also gathers at most 512 chunk partials forward and 640
    // backward (LayerNorm three per chunk, RMSNorm one): every workgroup of a row polls them
    // all, and beyond that the two-pass form is faster. Measured on MI355X, bf16, forward /
    // backward in us, single pass against two passes:
    //   LayerNorm 32 x 524288 (64 chunks)    17.7 / 40.8  against 18.4 / 48.0
    //   LayerNorm 16 x 1048576 (128 chunks)  18.3 / 41.5  against 18.7 / 48.2
    //   LayerNorm 12 x 1572864 (192 chunks)  22.8 / 50.2  against 20.8 / 59.1
    //   LayerNorm 8 x 2097152 (256 chunks)   20.6 / 43.1  against 19.6 / 32.2
    //   LayerNorm 4 x 4194304 (512 chunks)   27.6 / 34.7  against 21.0 / 31.8
    //   RMSNorm 16 x 1048576 / 8 x 2097152 / 4 x 4194304: 15.4 / 32.0, 16.2 / 32.6,
    //   17.3 / 26.0 against 17.4 / 35.5, 17.6 / 30.3, 18.6 / 30.3
    // (256 x 262144, 32 chunks: the single pass wins for both kinds). The statistics pass
    // keeps the forward's plan and workspace but never runs it (it writes no Y, so its second
    // pass re-reads nothing).
    const int64_t row_partials = p.chunks * (kind == NORM_LAYERNORM ? 3 : 1);
    const int64_t auto_max = bwd ? kXchgAutoMaxPartialsBwd : kXchgAutoMaxPartialsFwd;
    if (t.xchg != 0 && (t.xchg > 0 || row_partials <= auto_max) && wc == kFull && vpt == 4 &&
        !residual) {
      const int64_t cap = (int64_t)cu * (bwd ? kXchgBwdPerCu : xchg_fwd_per_cu(dtype));
      if (p.chunks <= kXchgMaxChunks && p.chunks * (bwd ? 1 : 2) <= cap) {
        int64_t G = cap / p.chunks;
        if (bwd && t.row_groups > 0 && t.row_groups < G) G = t.row_groups;
        p.xchg = 1;
        p.xrow_groups = G < Mm ? G : Mm;
      }
    }
  } else {
    return NORM_ERR_INVALID_ARG;
  }
  if (p.chunk_elems == 0) p.chunk_elems = N;

  // Every workspace starts with the header; forwards of the wave and block schemes need none.
  size_t off = 0;
  p.off_header = 0;
  if (bwd) {
    p.partials = scheme == NORM_SCHEME_SPLIT ? p.row_groups : p.grid;
    if (p.xchg && p.xrow_groups > p.partials) p.partials = p.xrow_groups;
    p.off_colpart = kWsHeaderBytes;
    off = align256(kWsHeaderBytes + (size_t)2 * (size_t)p.partials * (size_t)N * 4);
    if (scheme == NORM_SCHEME_SPLIT) {
      p.off_rowpart = off;
      off = align256(off + (size_t)Mm * (size_t)p.chunks * 4 * 4);
      p.off_stats = off;
      off = align256(off + (size_t)2 * (size_t)Mm * 4);
    }
  } else if (scheme == NORM_SCHEME_SPLIT) {
    p.off_rowpart = kWsHeaderBytes;
    off = align256(kWsHeaderBytes + (size_t)Mm * (size_t)p.chunks * 4 * 4);
  }
  if (p.xchg) {
    p.off_xpart = off;
    off = align256(off + (size_t)Mm * (size_t)p.chunks * kXchgWordsPerChunk * 8);
  }
  p.ws_bytes = off;
  *out = p;
  return NORM_OK;
}

norm_status_t workspace_bytes(norm_kind_t kind, norm_dtype_t dtype, norm_pass_t pass, int64_t M,
                              int64_t N, int residual, int cu, const Tuning &t, size_t *bytes) {
  if (!bytes) return NORM_ERR_INVALID_ARG;
  // Size for every pointer alignment (each may pick another access width). A tuning override
  // may leave a narrower width without a kernel; a call with such pointers then fails with
  // NORM_ERR_UNSUPPORTED anyway, so only the 16-byte-aligned plan has to succeed.
  // (phase classes: 1, 2, 4 or 8 classes, their grids and row lengths differing; every phase
  // pair that gives a class count is tried, with the alignments that still take that mode)
  Plan p;
  norm_status_t s = make_plan(kind, dtype, pass, M, N, residual, 16, 0, 0, cu, t, &p);
  if (s != NORM_OK) return s;
  size_t best = p.ws_bytes;
  // (a row step of d elements gives the classes of gcd(d, epv): steps 0, 1, 2 and 4 cover them)
  const int ev = vec_epv(dtype);
  for (int align : {16, 8, 4, 2, 1})
    for (int ph0 = -1; ph0 < ev; ++ph0)
      for (int dph : {-1, 0, 1, 2, 4})
        if (dph < ev &&
            make_plan(kind, dtype, pass, M, N, residual, align, ph0, dph, cu, t, &p) ==
                NORM_OK &&
            p.ws_bytes > best)
          best = p.ws_bytes;
  *bytes = best;
  return NORM_OK;
}

norm_status_t workspace_bytes_any_device(norm_kind_t kind, norm_dtype_t dtype, norm_pass_t pass,
                                         int64_t M, int64_t N, int residual, const Tuning &t,
                                         size_t *bytes) {
  if (!bytes) return NORM_ERR_INVALID_ARG;
  size_t best = 0;
  for (int cu = 1; cu <= kMaxCuCount; ++cu) {
    size_t b = 0;
    const norm_status_t s = workspace_bytes(kind, dtype, pass, M, N, residual, cu, t, &b);
    if (s != NORM_OK) return s;
    if (b > best) best = b;
  }
  *bytes = best;
  return NORM_OK;
}

// ---- argument checks -----------------------------------------------------------------------

namespace {

struct Span {
  const void *p;
  size_t n;
};

bool overlap(Span a, Span b) {
  if (!a.p || !b.p || !a.n || !b.n) return false;
  const uintptr_t x = (uintptr_t)a.p, y = (uintptr_t)b.p;
  return x < y + b.n && y < x + a.n;
}

// Every output must be disjoint from every input and from every other output.
bool disjoint(const Span *in, int nin, const Span *outs, int nout) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], in[j])) return false;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return false;
  }
  return true;
}

bool sizes_ok(int64_t M, int64_t N) {
  if (M < 0 || N <= 0 || N > kMaxN) return false;
  return M <= (INT64_MAX / 16) / N;
}

// A row stride is at least N and keeps (M - 1) * ld + N elements addressable.
bool stride_ok(int64_t M, int64_t N, int64_t ld) {
  if (ld < N) return false;
  return M <= (INT64_MAX / 16) / ld;
}

// bytes an [M, N] tensor with row stride ld spans
size_t span(int64_t M, int64_t N, int64_t ld, size_t s) {
  return M > 0 ? ((size_t)(M - 1) * (size_t)ld + (size_t)N) * s : 0;
}

} // namespace

norm_status_t check_fwd(const FwdCheck &c) {
  if (!valid_kind(c.kind) || !valid_dtype(c.dtype)) return NORM_ERR_INVALID_ARG;
  if (!sizes_ok(c.M, c.N)) return NORM_ERR_INVALID_ARG;
  if (!(std::isfinite(c.eps) && c.eps >= 0.0f)) return NORM_ERR_INVALID_ARG;
  if (c.kind == NORM_RMSNORM && (c.B || c.mean)) return NORM_ERR_INVALID_ARG;
  if ((c.R != nullptr) != (c.H != nullptr)) return NORM_ERR_INVALID_ARG;
  if (c.stats_only) {
    if (c.W || c.B || c.Y) return NORM_ERR_INVALID_ARG;
    if (!c.mean && !c.rstd && !c.H) return NORM_ERR_INVALID_ARG; // nothing to compute
  } else if (!c.W) {
    return NORM_ERR_INVALID_ARG;
  }
  if (c.M == 0) return NORM_OK;
  if (!c.X || (!c.Y && !c.stats_only)) return NORM_ERR_INVALID_ARG;
  // the strides of the tensors the call has (R and H are optional)
  if (!stride_ok(c.M, c.N, c.ldx) || (c.Y && !stride_ok(c.M, c.N, c.ldy)) ||
      (c.R && !stride_ok(c.M, c.N, c.ldr)) || (c.H && !stride_ok(c.M, c.N, c.ldh)))
    return NORM_ERR_INVALID_ARG;
  const size_t s = elem_size(c.dtype);
  const size_t n = (size_t)c.N * weight_size(c.dtype), m = (size_t)c.M * 4;
  const Span in[] = {{c.X, span(c.M, c.N, c.ldx, s)}, {c.R, span(c.M, c.N, c.ldr, s)},
                     {c.W, n}, {c.B, n}};
  const Span outs[] = {{c.Y, span(c.M, c.N, c.ldy, s)}, {c.H, span(c.M, c.N, c.ldh, s)},
                       {c.mean, m}, {c.rstd, m}, {c.ws, c.ws_bytes}};
  if (!disjoint(in, 4, outs, 5)) return NORM_ERR_INVALID_ARG;
  return NORM_OK;
}

norm_status_t check_bwd(const BwdCheck &c) {
  if (!valid_kind(c.kind) || !valid_dtype(c.dtype)) return NORM_ERR_INVALID_ARG;
  if (!sizes_ok(c.M, c.N)) return NORM_ERR_INVALID_ARG;
  if (c.need_dx) {
    if (!(std::isfinite(c.eps) && c.eps >= 0.0f)) return NORM_ERR_INVALID_ARG;
    if (c.kind == NORM_RMSNORM && c.mean) return NORM_ERR_INVALID_ARG;
    if (c.kind == NORM_LAYERNORM && ((c.mean == nullptr) != (c.rstd == nullptr)))
      return NORM_ERR_INVALID_ARG;
    if (!c.W) return NORM_ERR_INVALID_ARG;
  }
  if (c.need_dw) {
    if (!c.dW) return NORM_ERR_INVALID_ARG;
    if (c.kind == NORM_RMSNORM && c.dB) return NORM_ERR_INVALID_ARG;
  }
  if (c.M == 0) return NORM_OK;
  if (c.need_dx && (!c.X || !c.dY || !c.dX)) return NORM_ERR_INVALID_ARG;
  if (c.need_dx) {
    // the strides of the tensors the call has (dH and dR are optional)
    if (!stride_ok(c.M, c.N, c.ldx) || !stride_ok(c.M, c.N, c.lddy) ||
        !stride_ok(c.M, c.N, c.lddx) || (c.dH && !stride_ok(c.M, c.N, c.lddh)) ||
        (c.dR && !stride_ok(c.M, c.N, c.lddr)))
      return NORM_ERR_INVALID_ARG;
    if (c.dR && c.dR == c.dX && c.lddr != c.lddx) return NORM_ERR_INVALID_ARG;
  }
  const size_t s = elem_size(c.dtype);
  const size_t n = (size_t)c.N * weight_size(c.dtype), m = (size_t)c.M * 4;
  const void *dr = c.dR == c.dX ? nullptr : c.dR; // dR may alias dX
  const bool dx = c.need_dx != 0;
  const Span in[] = {{c.X, dx ? span(c.M, c.N, c.ldx, s) : 0},
                     {c.dY, dx ? span(c.M, c.N, c.lddy, s) : 0},
                     {c.dH, dx ? span(c.M, c.N, c.lddh, s) : 0},
                     {c.W, n}, {c.mean, m}, {c.rstd, m}};
  const Span outs[] = {{c.dX, dx ? span(c.M, c.N, c.lddx, s) : 0},
                       {dr, dx ? span(c.M, c.N, c.lddr, s) : 0},
                       {c.dW, n}, {c.dB, n}, {c.ws, c.ws_bytes}};
  if (!disjoint(in, 6, outs, 5)) return NORM_ERR_INVALID_ARG;
  return NORM_OK;
}

bool all_aligned16(const void *const *ptrs, int n) { return common_align(ptrs, n) >= 16; }

int common_align(const void *const *ptrs, int n) {
  uintptr_t bits = 16;
  for (int i = 0; i < n; ++i)
    if (ptrs[i]) bits |= (uintptr_t)ptrs[i];
  return (int)(bits & (~bits + 1)); // lowest set bit, at most 16
}

int fold_stride_align(int align, const int64_t *ld, int n, size_t elem_bytes) {
  uintptr_t bits = (uintptr_t)(align > 0 ? align : 1);
  for (int i = 0; i < n; ++i) bits |= (uintptr_t)((size_t)ld[i] * elem_bytes);
  return (int)(bits & (~bits + 1));
}

void common_phase(const void *const *ptrs, const int64_t *ld, int n, size_t elem_bytes,
                  int *phase0, int *dphase) {
  int b = -1, d = -1;
  for (int i = 0; i < n; ++i) {
    if (!ptrs[i]) continue;
    const uintptr_t a = (uintptr_t)ptrs[i];
    if (a % elem_bytes) { // not even element-aligned
      b = d = -2;
      break;
    }
    const int bi = (int)((a % 16) / elem_bytes);
    const int di = (int)((((uint64_t)ld[i] * elem_bytes) % 16) / elem_bytes);
    if (b == -1) {
      b = bi;
      d = di;
    } else if (bi != b || di != d) {
      b = d = -2;
      break;
    }
  }
  *phase0 = b < 0 ? -1 : b;
  *dphase = d < 0 ? -1 : d;
}

size_t act_elem_size(norm_dtype_t d) { return elem_size(d); }

size_t weight_align_need(norm_dtype_t d, int epv) {
  const size_t w = (size_t)epv * weight_size(d);
  return w < 16 ? w : 16;
}

} // namespace dln
