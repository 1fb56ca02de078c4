// C ABI of libqgemv_q4 (declared in include/qgemv_q4.h): argument checks,
// kernel-variant choice and launches on the caller's stream.
//
// Every product entry point reduces to a list of "parts": weight tensors of
// one format that share x, each with its rows and its output slice.  The
// kernel that computes a weight tensor (its "path") is chosen from the format,
// M, K, the group size, that tensor's own alignment and size, and the two
// process-wide settings (matrix-core threshold, kernel mask), read once per
// call.  Parts whose paths differ run in separate launches, so a dual,
// multi-part or fused-split call computes every weight tensor exactly as the
// single call on that tensor would, bit for bit.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "qgemv_q4.h"
#include "kernels/gemv.hpp"
#include "kernels/mfma.hpp"
#include "kernels/mma_gemv.hpp"
#include "kernels/xr_gemv.hpp"
#include "kernels/split.hpp"

using namespace qg;

namespace {

thread_local char g_err[512] = "";
std::atomic<int64_t> g_mfma_min_m{64};
constexpr uint32_t kAllKernels = QG_KERNEL_KSLICED | QG_KERNEL_XR | QG_KERNEL_MMA;
std::atomic<uint32_t> g_kernel_mask{kAllKernels};

// The process-wide settings as one call sees them (read once per call).
struct CallCfg {
  int64_t mfma_min_m;
  uint32_t mask;
};
CallCfg call_cfg() { return {g_mfma_min_m.load(), g_kernel_mask.load()}; }

qg_status fail(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return QG_EINVAL;
}

qg_status launch_status(const char* op) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(g_err, sizeof(g_err), "%s: kernel launch failed: %s", op, hipGetErrorString(e));
    return QG_ELAUNCH;
  }
  g_err[0] = '\0';
  return QG_OK;
}

qg_status launch_error(const char* op, const char* what, hipError_t e) {
  snprintf(g_err, sizeof(g_err), "%s: %s: %s", op, what, hipGetErrorString(e));
  return QG_ELAUNCH;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // keeps every in-kernel 32-bit index in range
constexpr int kMaxDevices = 64;                  // GPUs per process the library keeps state for
constexpr int64_t k2G = (int64_t)1 << 31;
constexpr size_t kLdsBudget = 64 * 1024;       // per-workgroup x tile when K is tiled
constexpr size_t kLdsPersistent = 150 * 1024;  // whole-K x tile of a persistent workgroup
constexpr size_t kLdsMax = 160 * 1024;

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return 256;
  if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// One weight tensor of a product (host side).  Stream 1 is used by the dual
// Q4_0 projection only.
struct HostPart {
  const void* w[2];
  const float* scales;
  const float* biases;
  float* y[2];
  int64_t ldy;
  int64_t n;
};

// Bytes per weight row of each format.
template <int FMT> int64_t row_bytes_of(int64_t k);
template <> int64_t row_bytes_of<FMT_Q40>(int64_t k) { return k / 32 * 18; }
template <> int64_t row_bytes_of<FMT_Q4K>(int64_t k) { return k / 256 * 144; }
template <> int64_t row_bytes_of<FMT_AFF>(int64_t k) { return k; }
template <> int64_t row_bytes_of<FMT_AFF4>(int64_t k) { return k / 2; }

// ------------------------------------------------------------------ paths
// The kernel that computes one weight tensor.  Plain: one thread per output
// (shapes and alignments the vector loaders do not take).  FMA: the chunked or
// the K-sliced GEMV (same bits).  XR: the x-resident matrix-core GEMV (3 rows
// of x up to the threshold).  MMA: the streamed matrix-core GEMV for affine
// codes (2 rows of x up to the threshold, or where XR does not apply).  MFMA:
// the matrix-core GEMM from the threshold on.
enum Path { P_PLAIN, P_FMA, P_XR, P_MMA, P_MFMA };

// Matrix-core GEMM: M at the threshold, K a whole number of 64-column stages,
// group size 32..512, the weights aligned for its vector loads and below 2 GiB
// (32-bit offsets), x below 2^31 elements.
template <int FMT>
bool mfma_ok(const CallCfg& cfg, int64_t m, int64_t k, int64_t gs, const void* w, int64_t n) {
  if (m < cfg.mfma_min_m || k % 64 != 0 || gs < 32 || gs > 512) return false;
  if (m * k >= k2G) return false;
  const uintptr_t al = FMT == FMT_AFF || FMT == FMT_Q4K ? 16 : FMT == FMT_AFF4 ? 8 : 4;
  return aligned(w, al) && n * row_bytes_of<FMT>(k) < k2G;
}

// The chunked loaders take 64-weight chunks of Q4_0 (4-byte aligned), 16-byte
// aligned Q4_K rows, and 32-code chunks of 16-byte aligned affine codes inside
// one group.
template <int FMT>
bool plain_needed(int64_t k, int64_t gs, const void* w) {
  if constexpr (FMT == FMT_Q40) return k % 64 != 0;
  else if constexpr (FMT == FMT_Q4K) return !aligned(w, 16);
  else return k % 32 != 0 || gs < 32 || !aligned(w, 16);
}

// x-resident matrix-core GEMV: from 3 rows of x, K a multiple of 512 up to
// 4096 (one wave per 512 columns), 16-byte aligned weights, affine group size
// >= 64.  Measured (graph replay, K = 4096): at 2 rows the K-sliced FMA kernel
// is ahead (N = 4096: 6.2 vs 7.4 us), from 3 rows this one (N = 14336: 19.4 vs
// 13.9 us at 3 rows, 50.1 vs 15.4 us at 8).
template <int FMT>
bool xr_ok(const CallCfg& cfg, int64_t m, int64_t k, int64_t gs, const void* w) {
  if (!(cfg.mask & QG_KERNEL_XR)) return false;
  if (m < 3 || k % 512 != 0 || k > 512 * kXrMaxWaves) return false;
  if ((FMT == FMT_AFF || FMT == FMT_AFF4) && gs < 64) return false;
  return aligned(w, 16);
}

// Streamed matrix-core GEMV for the affine formats from 2 rows of x: group
// size >= 64, K a multiple of 512 with K/512 in {1, 2, 4, 8} (up to 8 pairs of
// 32-column blocks per wave, so x of 8 rows fits in LDS), codes aligned for
// its vector loads.
template <int FMT>
bool mma_ok(const CallCfg& cfg, int64_t m, int64_t k, int64_t gs, const void* w) {
  if constexpr (FMT != FMT_AFF && FMT != FMT_AFF4) {
    return false;
  } else {
    if (!(cfg.mask & QG_KERNEL_MMA)) return false;
    if (m < 2 || gs < 64 || k % 512 != 0) return false;
    const int64_t np = k / 512;
    if (np != 1 && np != 2 && np != 4 && np != 8) return false;
    return aligned(w, FMT == FMT_AFF ? 16 : 8);
  }
}

// The path of one weight tensor of n rows at w (the whole fused weight for the
// fused split, whose parts are row ranges of it).
template <int FMT>
Path path_of(const CallCfg& cfg, int64_t m, int64_t k, int64_t gs, const void* w, int64_t n) {
  if (mfma_ok<FMT>(cfg, m, k, gs, w, n)) return P_MFMA;
  if (plain_needed<FMT>(k, gs, w)) return P_PLAIN;
  if (xr_ok<FMT>(cfg, m, k, gs, w)) return P_XR;
  if (mma_ok<FMT>(cfg, m, k, gs, w)) return P_MMA;
  return P_FMA;
}

// ------------------------------------------------------------------ GEMV
struct GemvPlan {
  int mt, l, r, kt;
  size_t lds;
  bool persistent;
};

// Launch shape of the chunked GEMV kernel that fixes its arithmetic: rows of
// x per tile (MT), lanes per row (L), row sets per wave (R) and the x tile.
// It depends on the format, M and K only, so the arithmetic of an output
// never depends on N or on the part list.  x of one m-tile is staged in LDS
// once per workgroup when it fits (persistent workgroups walk several row
// groups); otherwise each workgroup owns one row group and stages x in K
// tiles.  Measured on MI355X (graph replay of the 4096^2 Q4 and 12288x4096
// affine decode shapes): Q4 formats are fastest with 32 lanes per row and
// one row set at every M; affine codes with 64 lanes and two row sets.
template <int FMT>
GemvPlan plan_gemv(int64_t m, int64_t k, int nw) {
  constexpr int CH = FmtTraits<FMT>::CH;
  constexpr bool SUMS = FmtTraits<FMT>::SUMS;
  constexpr bool Q4 = FMT == FMT_Q40 || FMT == FMT_Q4K;
  GemvPlan pl{};
  const int64_t chunks = k / CH;
  pl.mt = m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : 8;
  // Q4 formats: 32 lanes per row, except one or two x rows with 64 to 256
  // chunks per row (K = 4096 .. 16384), where the K-sliced kernel takes 64
  // lanes and 8 waves (one or more chunks for every lane): Q4_K 4096 x 4096
  // 4.72 -> 4.50 us, dual Q4_0 6.7 -> 6.2 us, multi-part q|k|v 6.7 -> 6.3 us;
  // at two x rows Q4_0 4096 x 4096 6.3 -> 5.6 us, 14336 x 4096 12.8 -> 11.5 us.
  pl.l = Q4 ? (pl.mt <= 2 && chunks >= 64 && chunks <= 256 ? 64 : 32) : (chunks >= 64 ? 64 : 32);
  int r = 1;
  if (!Q4 && chunks >= 64 && (pl.mt * nw <= 2 || (nw == 1 && pl.mt == 8))) r = 2;
  // affine codes at one x row with 64 to 256 chunks per row (K = 2048 .. 8192):
  // one row per lane on the K-sliced kernel (12288 x 4096 gs 64: u8 12.7 ->
  // 12.1 us, packed 8.9 -> 8.6 us against two rows per lane)
  if (!Q4 && pl.mt == 1 && chunks >= 64 && chunks <= 256) r = 1;
  pl.r = r;
  auto lds_for = [&](int64_t kt) {
    const int64_t ct = kt / CH;
    return (size_t)(pl.mt * (CH / 4) * (ct + 1) * 16 + (SUMS ? pl.mt * ct * 8 : 0));
  };
  pl.persistent = lds_for(k) <= kLdsPersistent;
  if (pl.persistent) {
    pl.kt = (int)k;
    pl.lds = lds_for(k);
  } else {
    const int64_t step = (int64_t)pl.l * CH;
    int64_t kt = step;
    while (kt + step <= k && lds_for(kt + step) <= kLdsBudget) kt += step;
    pl.kt = (int)kt;
    pl.lds = lds_for(kt);
  }
  return pl;
}

// Waves per workgroup and the grid, which do not change the arithmetic.  A
// persistent workgroup stages x once and walks row groups; every workgroup
// should walk the same number of them (a partly filled last round leaves CUs
// idle), so the shape with the best balance wins, then the preferred one:
// 8 waves (one workgroup per CU) except for affine codes at M <= 2.
struct GemvGrid {
  int waves;
  int64_t groups_rows;  // rows per group
  int64_t grid;
};

template <int FMT>
GemvGrid grid_gemv(const GemvPlan& pl, const HostPart* parts, int nparts) {
  const int64_t cus = device_cus();
  auto groups_for = [&](int64_t rpg) {
    int64_t g = 0;
    for (int pi = 0; pi < nparts; ++pi) g += cdiv(parts[pi].n, rpg);
    return g;
  };
  const int pref = ((FMT == FMT_AFF || FMT == FMT_AFF4) && pl.mt <= 2) ? 4 : 8;
  GemvGrid best{};
  if (!pl.persistent) {
    best.waves = 4;
    best.groups_rows = (int64_t)best.waves * (64 / pl.l) * pl.r;
    best.grid = groups_for(best.groups_rows);
    return best;
  }
  double best_eff = -1.0;
  const int cand[2] = {pref, pref == 8 ? 4 : 8};
  for (int ci = 0; ci < 2; ++ci) {
    const int w = cand[ci];
    const int64_t rpg = (int64_t)w * (64 / pl.l) * pl.r;
    const int64_t groups = groups_for(rpg);
    int fit = (int)(kLdsMax / (pl.lds ? pl.lds : 1));
    const int cap_b = w == 8 ? 1 : 4;
    fit = fit < 1 ? 1 : fit > cap_b ? cap_b : fit;
    for (int b = fit; b >= 1; --b) {
      const int64_t slots = cus * b;
      const int64_t used = groups < slots ? groups : slots;
      const double eff = (double)groups / (double)(cdiv(groups, slots) * used);
      if (eff > best_eff + 1e-9) {
        best_eff = eff;
        best.waves = w;
        best.groups_rows = rpg;
        best.grid = used;
      }
    }
  }
  return best;
}

// Kernels whose LDS exceeds the default 64 KB need the limit raised once.
template <typename K>
hipError_t allow_lds(K kern, size_t lds, std::atomic<bool>& raised) {
  if (lds <= 64 * 1024 || raised.load()) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
  if (e == hipSuccess) raised.store(true);
  return e;
}

template <int FMT, int MT, int NW, int L, int R>
hipError_t launch_gemv_t(const GemvParams& p, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
  // multi-part variants exist for the formats whose entry points take parts
  constexpr bool kHasMulti = NW == 1 && (FMT == FMT_Q4K || FMT == FMT_AFF);
  if constexpr (kHasMulti) {
    if (p.parts > 1) {
      auto kern = gemv_kernel<FMT, MT, NW, L, R, true>;
      static std::atomic<bool> raised{false};
      const hipError_t e = allow_lds(kern, lds, raised);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, grid, block, lds, s, p);
      return hipSuccess;
    }
  }
  if (p.parts != 1) return hipErrorInvalidValue;
  auto kern = gemv_kernel<FMT, MT, NW, L, R, false>;
  static std::atomic<bool> raised{false};
  const hipError_t e = allow_lds(kern, lds, raised);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, block, lds, s, p);
  return hipSuccess;
}

template <int FMT, int MT, int NW, int L>
hipError_t launch_gemv_r(int r, const GemvParams& p, dim3 g, dim3 b, size_t lds, hipStream_t s) {
  // two row sets per wave where plan_gemv takes them (affine codes)
  if constexpr (FMT == FMT_AFF || FMT == FMT_AFF4) {
    if (r == 2) {
      if constexpr (MT * NW <= 2 || (NW == 1 && MT == 8)) return launch_gemv_t<FMT, MT, NW, L, 2>(p, g, b, lds, s);
      return hipErrorInvalidValue;
    }
  }
  if (r == 1) return launch_gemv_t<FMT, MT, NW, L, 1>(p, g, b, lds, s);
  return hipErrorInvalidValue;
}

template <int FMT, int MT, int NW>
hipError_t launch_gemv_l(int l, int r, const GemvParams& p, dim3 g, dim3 b, size_t lds, hipStream_t s) {
  switch (l) {
    case 64: return launch_gemv_r<FMT, MT, NW, 64>(r, p, g, b, lds, s);
    case 32: return launch_gemv_r<FMT, MT, NW, 32>(r, p, g, b, lds, s);
  }
  return hipErrorInvalidValue;
}

template <int FMT, int NW>
hipError_t launch_gemv_mt(const GemvPlan& pl, const GemvParams& p, dim3 g, dim3 b, hipStream_t s) {
  switch (pl.mt) {
    case 1: return launch_gemv_l<FMT, 1, NW>(pl.l, pl.r, p, g, b, pl.lds, s);
    case 2: return launch_gemv_l<FMT, 2, NW>(pl.l, pl.r, p, g, b, pl.lds, s);
    case 4: return launch_gemv_l<FMT, 4, NW>(pl.l, pl.r, p, g, b, pl.lds, s);
    case 8: return launch_gemv_l<FMT, 8, NW>(pl.l, pl.r, p, g, b, pl.lds, s);
  }
  return hipErrorInvalidValue;
}

// The K-sliced kernels' leading scalar arguments (preloaded into scalar
// registers).  Single part (or a part table read from p): x, part 0's
// weights (both streams), its first output, K, its rows, the row stride and
// the group count.  Parts in the arguments (up to three Q4_K parts): x, the
// parts' weights, K, their rows and the first groups of parts 1 and 2 (a
// two-part launch repeats part 1's weights, gives part 2 no rows and the
// group count as its first group).
#define KS_ARGS(p)                                                                                             \
  (p).x, (p).part0.w[0], (p).part0.w[1], (p).part0.y[0], (p).k, (p).part0.n, (int)(p).row_bytes, (p).n_groups, \
      (p)
#define KS_MP_ARGS(p)                                                                                           \
  (p).x, (p).hot.w[0], (p).hot.w[1], (p).parts > 2 ? (p).hot.w[2] : (p).hot.w[1], (p).k, (p).hot.n[0],       \
      (p).hot.n[1], (p).parts > 2 ? (p).hot.n[2] : 0, (p).hot.group0[1],                                       \
      (p).parts > 2 ? (p).hot.group0[2] : (p).n_groups, (p)

// K-sliced kernel for tiles of MT rows of x (same bits as the chunked kernel
// with the same MT, L and R); J = chunks per lane and row.
template <int FMT, int MT, int NW, int L, int R, int J, int WV>
hipError_t launch_gemv_ks_j(const GemvParams& p, dim3 grid, size_t lds, hipStream_t s) {
  if (p.parts > 1) {
    if constexpr (NW == 1 && (FMT == FMT_Q4K || FMT == FMT_AFF)) {
      // up to three Q4_K parts take their part table from the arguments too
      if constexpr (FMT == FMT_Q4K) {
        if (p.parts <= 3) {
          hipLaunchKernelGGL((gemv_ks_mp_kernel<FMT, MT, NW, L, R, J, WV>), grid, dim3(64 * WV), lds, s,
                             KS_MP_ARGS(p));
          return hipSuccess;
        }
      }
      hipLaunchKernelGGL((gemv_ks_kernel<FMT, MT, NW, L, R, J, WV, true>), grid, dim3(64 * WV), lds, s, KS_ARGS(p));
      return hipSuccess;
    }
    return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL((gemv_ks_kernel<FMT, MT, NW, L, R, J, WV, false>), grid, dim3(64 * WV), lds, s, KS_ARGS(p));
  return hipSuccess;
}

template <int FMT>
size_t ks_lds(int mt, int nw, int l, int r, int j, int wv) {
  const size_t ne4 = FmtTraits<FMT>::CH / 4;
  const size_t u = (size_t)(l / wv) * j;
  const size_t rows = (size_t)(kWave / (l / wv)) * r;
  const size_t sums = FmtTraits<FMT>::SUMS ? wv * 2 * u * 4 : 0;
  return (size_t)mt * (wv * ne4 * (u + 1) * 16 + sums + 2 * (size_t)nw * wv * rows * 4);
}

// Waves per workgroup of the K-sliced kernel (the arithmetic is the same
// either way).  The affine formats use 8.  For the 64-weight chunks of
// Q4_0/Q4_K at 32 lanes per row, 4 waves of 8 virtual lanes (row groups of 8
// rows, twice the workgroups) measured faster where every virtual lane has a
// chunk (K >= 2048): 6.6 vs 7.0 us for the multi-part q|k|v product, 11.5 vs
// 12.3 us for its three separate calls, a tie at 4096 x 4096; at K = 1024 8
// waves are faster (2.35 vs 2.48 us).  64 lanes per row take 8 waves (8
// virtual lanes per wave and row), or 16 waves of 4 (row groups of 16 rows,
// one workgroup per CU) for one weight stream and one x row when those row
// groups fill the CUs in whole rounds (or one round at least three quarters
// full) and each lane holds at most two chunks (K <= 8192; more would spill
// at 128 VGPRs): x is then read into each CU once instead of twice.  Q4_K
// x 4096 at M = 1: 4096 rows 4.45 -> 4.34 us, 8192 rows 6.1 -> 5.9 us, 16384
// rows 10.7 -> 9.6 us (Q4_0 alike); with two weight streams per group (6.5 ->
// 6.9 us; a dual product runs as a pair launch instead, see
// launch_gemv_ks_pair) or a part-filled last round (6144 rows: 6.1 -> 6.9 us)
// 16 waves are slower.
template <int FMT>
int ks_waves(int64_t k, int l, int mt, int nw, int64_t rows) {
  if constexpr (FMT != FMT_Q40 && FMT != FMT_Q4K) return 8;
  if (l == 64) {
    const int64_t groups16 = cdiv(rows, 16);
    const int64_t cus = device_cus();
    const bool rounds = (groups16 <= cus && 4 * groups16 >= 3 * cus) || groups16 % cus == 0;
    return nw == 1 && mt == 1 && k / 64 <= 2 * 64 && rounds ? 16 : 8;
  }
  return k / 64 >= 32 ? 4 : 8;
}

// Chunks per lane the K-sliced kernel takes for this call (0: the chunked
// kernel runs instead): x in LDS for the whole K and the chunked kernel's
// shape (L, R) = (32, 1) for the 64-weight chunks of Q4_0/Q4_K (one or two
// weight streams; one x row, or tiles of 2 or 4 rows where 4 waves are used),
// (64, 1) for them at one or two x rows with 64..256 chunks per row (8 waves),
// or (64, 1) / (64, 2) for the 32-code chunks of the affine formats (one x
// row).
template <int FMT, int NW>
int ks_chunks(const CallCfg& cfg, const GemvPlan& pl, int64_t k) {
  if (!(cfg.mask & QG_KERNEL_KSLICED)) return 0;
  constexpr bool Q4 = FMT == FMT_Q40 || FMT == FMT_Q4K;
  if (!pl.persistent) return 0;
  // tiles of 2 or 4 rows of x: the dual Q4_0 product at M = 4 takes 11.0 us
  // here against 14.1 us on the chunked kernel; at 8 rows (22.1 vs 18.5 us)
  // the chunked kernel stays
  if (pl.mt > 1 && !(Q4 && ((pl.l == 32 && pl.mt <= 4 && ks_waves<FMT>(k, pl.l, pl.mt, NW, 0) == 4) || (pl.l == 64 && pl.mt == 2))))
    return 0;
  if (Q4 ? !((pl.l == 32 || (pl.l == 64 && pl.mt <= 2)) && pl.r == 1) : !(pl.l == 64 && (pl.r == 1 || pl.r == 2)))
    return 0;
  const int64_t j = cdiv(k / FmtTraits<FMT>::CH, pl.l);
  return j >= 1 && j <= 4 ? (int)j : 0;
}

template <int FMT, int MT, int NW, int L, int R, int WV>
hipError_t launch_gemv_ks_lr(int j, const GemvParams& p, dim3 grid, hipStream_t s) {
  const size_t lds = ks_lds<FMT>(MT, NW, L, R, j, WV);
  switch (j) {
    case 1: return launch_gemv_ks_j<FMT, MT, NW, L, R, 1, WV>(p, grid, lds, s);
    case 2: return launch_gemv_ks_j<FMT, MT, NW, L, R, 2, WV>(p, grid, lds, s);
  }
  if constexpr (WV <= 8) {  // 16 waves take at most two chunks per lane
    switch (j) {
      case 3: return launch_gemv_ks_j<FMT, MT, NW, L, R, 3, WV>(p, grid, lds, s);
      case 4: return launch_gemv_ks_j<FMT, MT, NW, L, R, 4, WV>(p, grid, lds, s);
    }
  }
  return hipErrorInvalidValue;
}

template <int FMT, int NW>
hipError_t launch_gemv_ks(const GemvPlan& pl, int j, int wv, const GemvParams& p, dim3 grid, hipStream_t s) {
  if constexpr (FMT == FMT_Q40 || FMT == FMT_Q4K) {
    if (pl.l == 64 && pl.r == 1 && pl.mt == 1) {
      if constexpr (NW == 1) {
        if (wv == 16) return j <= 2 ? launch_gemv_ks_lr<FMT, 1, NW, 64, 1, 16>(j, p, grid, s) : hipErrorInvalidValue;
      }
      return launch_gemv_ks_lr<FMT, 1, NW, 64, 1, 8>(j, p, grid, s);
    }
    if (pl.l == 64 && pl.r == 1 && pl.mt == 2) return launch_gemv_ks_lr<FMT, 2, NW, 64, 1, 8>(j, p, grid, s);
    if (!(pl.l == 32 && pl.r == 1)) return hipErrorInvalidValue;
    const bool four = wv == 4;
    switch (pl.mt) {
      case 1: return four ? launch_gemv_ks_lr<FMT, 1, NW, 32, 1, 4>(j, p, grid, s)
                          : launch_gemv_ks_lr<FMT, 1, NW, 32, 1, 8>(j, p, grid, s);
      case 2: return four ? launch_gemv_ks_lr<FMT, 2, NW, 32, 1, 4>(j, p, grid, s) : hipErrorInvalidValue;
      case 4: return four ? launch_gemv_ks_lr<FMT, 4, NW, 32, 1, 4>(j, p, grid, s) : hipErrorInvalidValue;
    }
    return hipErrorInvalidValue;
  } else if constexpr (NW == 1) {
    if (pl.l != 64 || pl.mt != 1) return hipErrorInvalidValue;
    return pl.r == 1 ? launch_gemv_ks_lr<FMT, 1, NW, 64, 1, 8>(j, p, grid, s)
                     : pl.r == 2 ? launch_gemv_ks_lr<FMT, 1, NW, 64, 2, 8>(j, p, grid, s) : hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
}

template <int FMT, int NP>
hipError_t launch_gemv_mma_np(const GemvParams& p, dim3 grid, hipStream_t s) {
  constexpr size_t lds = (size_t)mma_lds_bytes(NP);
  auto kern = p.parts > 1 ? gemv_mma_kernel<FMT, NP, true> : gemv_mma_kernel<FMT, NP, false>;
  static std::atomic<bool> raised[2] = {false, false};
  const hipError_t e = allow_lds(kern, lds, raised[p.parts > 1 ? 1 : 0]);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(512), lds, s, p);
  return hipSuccess;
}

template <int FMT>
hipError_t launch_gemv_mma(int np, const GemvParams& p, dim3 grid, hipStream_t s) {
  if constexpr (FMT != FMT_AFF && FMT != FMT_AFF4) {
    return hipErrorInvalidValue;
  } else {
    switch (np) {
      case 1: return launch_gemv_mma_np<FMT, 1>(p, grid, s);
      case 2: return launch_gemv_mma_np<FMT, 2>(p, grid, s);
      case 4: return launch_gemv_mma_np<FMT, 4>(p, grid, s);
      case 8: return launch_gemv_mma_np<FMT, 8>(p, grid, s);
    }
    return hipErrorInvalidValue;
  }
}

// Part table of a GEMV launch: every weight stream of the part list, with row
// groups of `rows_per_group` rows numbered part after part.  `split_streams`
// (the x-resident kernel) makes each stream of a dual part a part of its own.
GemvParams gemv_params(const HostPart* parts, int nparts, int nw, bool split_streams, int64_t rows_per_group,
                       int64_t k, int gs, int64_t row_bytes) {
  GemvParams p{};
  for (int i = 0; i < kLaunchParts; ++i) p.hot.group0[i] = INT_MAX;  // unused slots: past every group
  int64_t groups = 0;
  int np = 0;
  for (int pi = 0; pi < nparts; ++pi) {
    const int ns = split_streams ? nw : 1;
    for (int st = 0; st < ns && np < kLaunchParts; ++st) {  // callers check kLaunchParts streams
      GemvPart gp{};
      for (int j = 0; j < 2; ++j) {
        const int src = split_streams ? st : j;
        gp.w[j] = static_cast<const uint8_t*>(parts[pi].w[src] ? parts[pi].w[src] : parts[pi].w[0]);
        gp.y[j] = parts[pi].y[src] ? parts[pi].y[src] : parts[pi].y[0];
      }
      gp.scales = parts[pi].scales;
      gp.biases = parts[pi].biases;
      gp.ldy = parts[pi].ldy;
      gp.n = (int)parts[pi].n;
      gp.group0 = (int)groups;
      groups += cdiv(parts[pi].n, rows_per_group);
      if (np == 0) p.part0 = gp;
      // the multi-part table: one stream per part (a dual part is a
      // multi-part launch only with split_streams)
      p.hot.group0[np] = gp.group0;
      p.hot.n[np] = gp.n;
      p.hot.w[np] = gp.w[0];
      p.out.y[np] = gp.y[0];
      p.out.ldy[np] = gp.ldy;
      p.aff.scales[np] = gp.scales;
      p.aff.biases[np] = gp.biases;
      ++np;
    }
  }
  p.parts = np;
  p.n_groups = (int)groups;
  p.row_bytes = row_bytes;
  p.k = (int)k;
  p.gs = gs;
  return p;
}

// The m-tile of rows m0.. of a launch: x and every output pointer advanced.
GemvParams m_tile(const GemvParams& p, const float* x, int64_t m0, int64_t m, int64_t k, int mt) {
  GemvParams q = p;
  q.x = x + m0 * k;
  for (int st = 0; st < 2; ++st) q.part0.y[st] = p.part0.y[st] + m0 * p.part0.ldy;
  for (int pi = 0; pi < p.parts; ++pi) q.out.y[pi] = p.out.y[pi] + m0 * p.out.ldy[pi];
  q.m_rows = (int)(m - m0 < mt ? m - m0 : mt);
  return q;
}

// x-resident matrix-core GEMV: every weight stream of the part list (both of a
// dual product) becomes one part of the launch.
template <int FMT>
qg_status run_gemv_xr(const char* op, const HostPart* parts, int nparts, int nw, const float* x, int64_t m,
                      int64_t k, int gs, hipStream_t s) {
  if (nparts * nw > kLaunchParts) return fail("%s: too many weight streams for one launch", op);
  (void)hipGetLastError();
  const GemvParams p = gemv_params(parts, nparts, nw, true, 16, k, gs, row_bytes_of<FMT>(k));
  // x of a workgroup lives in its waves' registers: one workgroup per CU for
  // K = 4096, more for shorter rows
  const int waves = (int)(k / 512);
  const int64_t cap = (int64_t)device_cus() * (kXrMaxWaves / waves);
  const int64_t grid = p.n_groups < cap ? p.n_groups : cap;
  auto kern = waves > 4 ? (p.parts > 1 ? gemv_xr_kernel<FMT, true, 8> : gemv_xr_kernel<FMT, false, 8>)
                        : (p.parts > 1 ? gemv_xr_kernel<FMT, true, 4> : gemv_xr_kernel<FMT, false, 4>);
  for (int64_t m0 = 0; m0 < m; m0 += kXrMaxM) {
    const GemvParams q = m_tile(p, x, m0, m, k, kXrMaxM);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * waves), 0, s, q.x,
                       q.part0.w[0], q.k, q.m_rows, q.n_groups, q.part0.n, q.part0.group0, (int)q.row_bytes, q);
  }
  return launch_status(op);
}

// Streamed matrix-core GEMV (affine codes, one stream per part).
template <int FMT>
qg_status run_gemv_mma(const char* op, const HostPart* parts, int nparts, const float* x, int64_t m, int64_t k,
                       int gs, hipStream_t s) {
  if (nparts > kLaunchParts) return fail("%s: too many weight streams for one launch", op);
  (void)hipGetLastError();
  const GemvParams p = gemv_params(parts, nparts, 1, false, 16, k, gs, row_bytes_of<FMT>(k));
  // one workgroup per CU (the x tile fills most of the LDS), walking row groups
  const int64_t grid = p.n_groups < device_cus() ? p.n_groups : device_cus();
  for (int64_t m0 = 0; m0 < m; m0 += kMmaMaxM) {
    const hipError_t e = launch_gemv_mma<FMT>((int)(k / 512), m_tile(p, x, m0, m, k, kMmaMaxM),
                                              dim3((unsigned)grid), s);
    if (e != hipSuccess) return launch_error(op, "launch setup failed", e);
  }
  return launch_status(op);
}

// Plain kernel: one launch per part and m-chunk.
template <int FMT, int NW>
qg_status run_plain(const char* op, const HostPart* parts, int nparts, const float* x, int64_t m, int64_t k,
                    int gs, hipStream_t s) {
  (void)hipGetLastError();
  const int64_t rb = row_bytes_of<FMT>(k);
  const dim3 block(256);
  for (int pi = 0; pi < nparts; ++pi) {
    const HostPart& hp = parts[pi];
    for (int64_t m0 = 0; m0 < m; m0 += 65535) {
      const int64_t mc = m - m0 < 65535 ? m - m0 : 65535;
      PlainParams q{};
      for (int st = 0; st < 2; ++st) {
        q.w[st] = static_cast<const uint8_t*>(hp.w[st] ? hp.w[st] : hp.w[0]);
        q.y[st] = (hp.y[st] ? hp.y[st] : hp.y[0]) + m0 * hp.ldy;
      }
      q.scales = hp.scales;
      q.biases = hp.biases;
      q.x = x + m0 * k;
      q.ldy = hp.ldy;
      q.row_bytes = rb;
      q.n = (int)hp.n;
      q.k = (int)k;
      q.gs = gs;
      const dim3 grid((unsigned)cdiv(hp.n, 256), (unsigned)mc);
      hipLaunchKernelGGL((gemv_plain_kernel<FMT, NW>), grid, block, 0, s, q, (int)mc);
    }
  }
  return launch_status(op);
}

// The two weight streams of a dual Q4_0 product as one stream of twice the
// row groups (16-wave K-sliced kernel, one x row): each group holds one
// stream's rows, as in the single calls, which take the same kernel shape.
template <int FMT>
hipError_t launch_gemv_ks_pair(int j, const GemvParams& p, dim3 grid, hipStream_t s) {
  if constexpr (FMT == FMT_Q40) {
    const size_t lds = ks_lds<FMT>(1, 1, 64, 1, j, 16);
    switch (j) {
      case 1:
        hipLaunchKernelGGL((gemv_ks_kernel<FMT, 1, 1, 64, 1, 1, 16, false, true>), grid, dim3(1024), lds, s,
                           KS_ARGS(p));
        return hipSuccess;
      case 2:
        hipLaunchKernelGGL((gemv_ks_kernel<FMT, 1, 1, 64, 1, 2, 16, false, true>), grid, dim3(1024), lds, s,
                           KS_ARGS(p));
        return hipSuccess;
    }
  }
  return hipErrorInvalidValue;
}

// FMA GEMV: the K-sliced kernel where it applies, else the chunked one (same
// bits), over all m-tiles of x.
template <int FMT, int NW>
qg_status run_gemv_fma(const char* op, const CallCfg& cfg, const HostPart* parts, int nparts, const float* x,
                       int64_t m, int64_t k, int gs, hipStream_t s) {
  if (nparts * NW > kLaunchParts) return fail("%s: too many weight streams for one launch", op);
  (void)hipGetLastError();
  const GemvPlan pl = plan_gemv<FMT>(m, k, NW);
  const int ks = ks_chunks<FMT, NW>(cfg, pl, k);
  if (ks) {
    // Up to 16 waves per CU (one 16-wave, two 8-wave or four 4-wave
    // workgroups; they are resident together where the kernel stays within
    // 128 VGPRs), walking row groups beyond that.  Measured on Q4_K K = 4096
    // at N = 6144 ... 28672 rows: 3-12% faster than 8 waves per CU.
    int64_t rows16 = 0;  // rows of all parts, each rounded up to 16-row groups
    for (int pi = 0; pi < nparts; ++pi) rows16 += cdiv(parts[pi].n, 16) * 16;
    if constexpr (FMT == FMT_Q40 && NW == 2) {
      // A dual product whose two streams together fill the CUs in whole
      // rounds of 16-row groups: one stream of twice the groups on 16 waves.
      // Q4_0 4096 x 4096 at M = 1: 6.43 -> 5.9 us against the two-stream
      // kernel on 8 waves (whose 16-wave form measured 6.9 us).
      if (m == 1 && nparts == 1 && pl.mt == 1 && pl.l == 64 && pl.r == 1 && ks <= 2 &&
          ks_waves<FMT>(k, pl.l, 1, 1, 2 * rows16) == 16) {
        GemvParams p = m_tile(gemv_params(parts, 1, 2, false, 16, k, gs, row_bytes_of<FMT>(k)), x, 0, 1, k, 1);
        p.n_groups *= 2;
        p.kt = pl.kt;
        const int64_t cus = device_cus();
        const int64_t grid = p.n_groups < cus ? p.n_groups : cus;
        const hipError_t e = launch_gemv_ks_pair<FMT>(ks, p, dim3((unsigned)grid), s);
        if (e != hipSuccess) return launch_error(op, "launch setup failed", e);
        return launch_status(op);
      }
    }
    const int ks_wv = ks_waves<FMT>(k, pl.l, pl.mt, NW, rows16);
    const int64_t rows_per_group = kWave / (pl.l / ks_wv) * pl.r;
    GemvParams p = gemv_params(parts, nparts, NW, false, rows_per_group, k, gs, row_bytes_of<FMT>(k));
    p.kt = pl.kt;
    const int64_t cap = (16 / ks_wv) * device_cus();
    const int64_t grid = p.n_groups < cap ? p.n_groups : cap;
    for (int64_t m0 = 0; m0 < m; m0 += pl.mt) {
      const hipError_t e = launch_gemv_ks<FMT, NW>(pl, ks, ks_wv, m_tile(p, x, m0, m, k, pl.mt), dim3((unsigned)grid), s);
      if (e != hipSuccess) return launch_error(op, "launch setup failed", e);
    }
    return launch_status(op);
  }
  const GemvGrid gg = grid_gemv<FMT>(pl, parts, nparts);
  GemvParams p = gemv_params(parts, nparts, NW, false, gg.groups_rows, k, gs, row_bytes_of<FMT>(k));
  p.kt = pl.kt;
  const dim3 block(64 * gg.waves);
  for (int64_t m0 = 0; m0 < m; m0 += pl.mt) {
    const hipError_t e = launch_gemv_mt<FMT, NW>(pl, m_tile(p, x, m0, m, k, pl.mt), dim3((unsigned)gg.grid), block, s);
    if (e != hipSuccess) return launch_error(op, "launch setup failed", e);
  }
  return launch_status(op);
}

// ------------------------------------------------------------------ MFMA
// Bytes of the matrix-core path's scratch for M rows of x: x_hi and x_lo as
// bf16 [M, K], and (formats with a bias term) the group sums of x as bf16 hi
// and lo [M, K/gs], each array 256-byte aligned.
template <int FMT>
size_t mfma_scratch_bytes(int64_t m, int64_t k, int64_t gs) {
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t bx = up((size_t)m * k * sizeof(__bf16));
  const size_t bs = FMT == FMT_Q40 ? 0 : up((size_t)m * (k / gs) * sizeof(__bf16));
  return 2 * bx + 2 * bs;
}

// Row tiles per XCD block of the matrix-core kernel (0: consecutive tiles).
// The 8 XCDs each take an equal block of mb row tiles by nb column tiles that
// together tile the grid; an XCD's L2 then fetches mb tiles' x split (xb
// bytes each) and nb tiles' weight rows (wb bytes each), and the block shape
// with the fewest such bytes wins.  Q4_0 512 x 4096 x 4096 (8 x 32 tiles of
// 64 x 128): 4 x 8 blocks fetch 4 MB of x and 2.4 MB of weights per XCD
// where the consecutive order (8 x 4) fetched the whole 8 MB x split.
int xcd_block_rows(int64_t tiles_m, int64_t tiles_n, int64_t xb, int64_t wb) {
  const int64_t total = tiles_m * tiles_n;
  if (total % 8 != 0) return 0;
  const int64_t per = total / 8;
  int best = 0;
  int64_t best_cost = 0;
  for (int64_t mb = tiles_m; mb >= 1 && mb * 8 >= tiles_m; mb /= 2) {
    if (tiles_m % mb != 0 || per % mb != 0) continue;
    const int64_t nb = per / mb;
    if (tiles_n % nb != 0 || (tiles_m / mb) * (tiles_n / nb) != 8) continue;
    const int64_t cost = mb * xb + nb * wb;
    if (best == 0 || cost < best_cost) best = (int)mb, best_cost = cost;
  }
  return best;
}

// x -> (x_hi, x_lo, group sums) in `scratch` (mfma_scratch_bytes, 256-byte
// aligned), then one launch of the matrix-core kernel over every weight
// stream's column tiles (both streams of a dual part are two parts of it).
template <int FMT>
qg_status launch_mfma(const char* op, const HostPart* parts, int nparts, int nw, const float* x, int64_t m,
                      int64_t k, int gs, void* scratch, hipStream_t s) {
  if (nparts * nw > kMaxParts) return fail("%s: too many weight streams for one launch", op);
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const int64_t groups = k / gs;
  __bf16* xh = static_cast<__bf16*>(scratch);
  __bf16* xl = reinterpret_cast<__bf16*>(reinterpret_cast<char*>(xh) + up((size_t)m * k * sizeof(__bf16)));
  __bf16* sh = nullptr;
  __bf16* sl = nullptr;
  if constexpr (FMT != FMT_Q40) {
    sh = reinterpret_cast<__bf16*>(reinterpret_cast<char*>(xl) + up((size_t)m * k * sizeof(__bf16)));
    sl = reinterpret_cast<__bf16*>(reinterpret_cast<char*>(sh) + up((size_t)m * groups * sizeof(__bf16)));
  }
  const int64_t items = m * (k / 8);
  hipLaunchKernelGGL(affine_prep_kernel, dim3((unsigned)cdiv(items, 256)), dim3(256), 0, s, x, xh, xl, sh, sl,
                     (int)m, (int)k, gs);
  MfmaParams mp{};
  mp.xh = xh;
  mp.xl = xl;
  mp.sh = sh;
  mp.sl = sl;
  int64_t tiles_n = 0;
  int np = 0;
  for (int pi = 0; pi < nparts; ++pi) {
    for (int st = 0; st < nw; ++st) {
      MfmaPart& q = mp.part[np++];
      q.w = static_cast<const uint8_t*>(parts[pi].w[st]);
      q.scales = parts[pi].scales;
      q.biases = parts[pi].biases;
      q.y = parts[pi].y[st];
      q.ldy = parts[pi].ldy;
      q.n = (int)parts[pi].n;
      q.tile0 = (int)tiles_n;
      tiles_n += cdiv(parts[pi].n, 128);
    }
  }
  // Tile shape: 128x128 (16 waves) while that gives every other CU a tile,
  // else 64x128 (8 waves, two workgroups per CU); both run four waves per
  // SIMD.  Measured on MI355X: Q4_0 512x4096x4096 takes 107 us on 128 tiles
  // of 128x128 and 100 us on 256 tiles of 64x128; the affine 512x8192x2048
  // product 64 us on 256 tiles of 128x128 and 72 us on 512 of 64x128.  The
  // arithmetic of an output does not depend on the shape.
  const int sm = 2 * cdiv(m, 128) * tiles_n > device_cus() ? 2 : 1;
  for (int pi = np; pi < kMaxParts; ++pi) mp.part[pi].tile0 = INT_MAX;  // never reached
  mp.parts = np;
  mp.row_bytes = row_bytes_of<FMT>(k);
  mp.m = (int)m;
  mp.k = (int)k;
  mp.gs = gs;
  mp.tiles_m = (int)cdiv(m, 64 * sm);
  mp.tiles_n = (int)tiles_n;
  mp.xcd_mb = xcd_block_rows(mp.tiles_m, mp.tiles_n, 64 * sm * k * 4, 128 * mp.row_bytes);
  const dim3 grid((unsigned)(mp.tiles_m * mp.tiles_n));
  // 128x128 runs as 4 x 2 wave pairs of 32x64 sub-tiles, 64x128 as 2 x 2
  const dim3 block((unsigned)(512 * sm));
  const bool multi = np > 1;
  if (sm == 2) {
    if (multi) hipLaunchKernelGGL((qmm_mfma_kernel<FMT, true, 4, 2, 2>), grid, block, 0, s, mp);
    else hipLaunchKernelGGL((qmm_mfma_kernel<FMT, false, 4, 2, 2>), grid, block, 0, s, mp);
  } else if (k % 128 == 0) {
    // 64x128 tiles take two 64-column K steps per barrier (one workgroup per CU)
    if (multi) hipLaunchKernelGGL((qmm_mfma_kernel<FMT, true, 2, 2, 2, 2>), grid, block, 0, s, mp);
    else hipLaunchKernelGGL((qmm_mfma_kernel<FMT, false, 2, 2, 2, 2>), grid, block, 0, s, mp);
  } else {
    if (multi) hipLaunchKernelGGL((qmm_mfma_kernel<FMT, true, 2, 2, 2>), grid, block, 0, s, mp);
    else hipLaunchKernelGGL((qmm_mfma_kernel<FMT, false, 2, 2, 2>), grid, block, 0, s, mp);
  }
  return launch_status(op);
}

// Scratch of a matrix-core call made while its stream is being captured into
// a graph.  hipMallocAsync / hipFreeAsync there would become memory nodes of
// the graph, which cost about 10 us per replay (512 x 8192 x 2048 prefill:
// 64.4 vs 53.8 us with a fixed buffer).  Instead the call takes a buffer owned
// by the graph under capture: a user object retained by that graph holds it,
// and once the graph and every executable graph made from it are destroyed
// (and their launches are done) the runtime calls graph_buf_release, which
// returns the buffer to a per-device free list that later captures draw on.
// Buffers are never handed back to the device, so no later call pays for a
// synchronising hipFree.  Executable graphs made from one captured graph (or
// from its clones) share its buffers and must not run at the same time; the
// runtime already orders the launches of one executable graph.
struct GraphBuf {
  void* p;
  size_t bytes;
  int dev;
};
struct GraphBufPool {
  std::mutex mu;
  std::vector<GraphBuf> released[kMaxDevices];
};
// Never destroyed: the runtime may release user objects while the process exits.
GraphBufPool& graph_bufs() {
  static GraphBufPool* pool = new GraphBufPool;
  return *pool;
}

// User-object destructor: runs on a runtime thread and makes no HIP call.
void graph_buf_release(void* arg) {
  GraphBuf* b = static_cast<GraphBuf*>(arg);
  {
    GraphBufPool& pool = graph_bufs();
    std::lock_guard<std::mutex> lock(pool.mu);
    pool.released[b->dev].push_back(*b);
  }
  delete b;
}

qg_status capture_scratch(const char* op, hipStream_t s, size_t bytes, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return launch_error(op, "hipGetDevice failed", e);
  if (dev < 0 || dev >= kMaxDevices) return fail("%s: device %d outside 0..%d", op, dev, kMaxDevices - 1);
  GraphBuf* b = nullptr;
  {
    // the smallest released buffer of this device that is large enough
    GraphBufPool& pool = graph_bufs();
    std::lock_guard<std::mutex> lock(pool.mu);
    std::vector<GraphBuf>& list = pool.released[dev];
    size_t best = list.size();
    for (size_t i = 0; i < list.size(); ++i)
      if (list[i].bytes >= bytes && (best == list.size() || list[i].bytes < list[best].bytes)) best = i;
    if (best < list.size()) {
      b = new GraphBuf(list[best]);
      list[best] = list.back();
      list.pop_back();
    }
  }
  if (b == nullptr) {
    // an allocation is a "potentially unsafe" call during a global-mode
    // capture: make it from this thread in relaxed mode, then restore the mode
    hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
    e = hipThreadExchangeStreamCaptureMode(&mode);
    if (e != hipSuccess) return launch_error(op, "capture mode exchange failed", e);
    void* p = nullptr;
    const hipError_t ea = hipMalloc(&p, bytes);
    e = hipThreadExchangeStreamCaptureMode(&mode);
    if (ea != hipSuccess) {
      snprintf(g_err, sizeof(g_err), "%s: scratch allocation of %zu bytes failed: %s", op, bytes,
               hipGetErrorString(ea));
      return QG_ELAUNCH;
    }
    b = new GraphBuf{p, bytes, dev};
    if (e != hipSuccess) {
      graph_buf_release(b);
      return launch_error(op, "capture mode exchange failed", e);
    }
  }
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  hipGraph_t g = nullptr;
  e = hipStreamGetCaptureInfo_v2(s, &st, nullptr, &g, nullptr, nullptr);
  if (e != hipSuccess || st != hipStreamCaptureStatusActive || g == nullptr) {
    graph_buf_release(b);
    return launch_error(op, "stream capture query failed", e != hipSuccess ? e : hipErrorStreamCaptureInvalidated);
  }
  void* p = b->p;  // read before the graph owns b
  hipUserObject_t obj = nullptr;
  e = hipUserObjectCreate(&obj, b, graph_buf_release, 1, hipUserObjectNoDestructorSync);
  if (e != hipSuccess) {
    graph_buf_release(b);
    return launch_error(op, "user object creation failed", e);
  }
  e = hipGraphRetainUserObject(g, obj, 1, hipGraphUserObjectMove);
  if (e != hipSuccess) {
    (void)hipUserObjectRelease(obj, 1);  // runs graph_buf_release
    return launch_error(op, "graph user object retain failed", e);
  }
  *out = p;
  return QG_OK;
}

// The matrix-core path.  Its scratch is stream-ordered, allocated and released
// on the caller's stream for this call, except under stream capture, where it
// belongs to the graph being captured (capture_scratch).
template <int FMT>
qg_status run_mfma(const char* op, const HostPart* parts, int nparts, int nw, const float* x, int64_t m, int64_t k,
                   int gs, hipStream_t s) {
  const size_t bytes = mfma_scratch_bytes<FMT>(m, k, gs);
  (void)hipGetLastError();
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &cs);
  if (e != hipSuccess) return launch_error(op, "stream capture query failed", e);
  void* scratch = nullptr;
  if (cs == hipStreamCaptureStatusActive) {
    const qg_status st = capture_scratch(op, s, bytes, &scratch);
    if (st != QG_OK) return st;
    return launch_mfma<FMT>(op, parts, nparts, nw, x, m, k, gs, scratch, s);
  }
  e = hipMallocAsync(&scratch, bytes, s);
  if (e != hipSuccess) {
    snprintf(g_err, sizeof(g_err), "%s: scratch allocation of %zu bytes failed: %s", op, bytes,
             hipGetErrorString(e));
    return QG_ELAUNCH;
  }
  const qg_status ls = launch_mfma<FMT>(op, parts, nparts, nw, x, m, k, gs, scratch, s);
  e = hipFreeAsync(scratch, s);
  if (ls == QG_OK && e != hipSuccess) return launch_error(op, "scratch release failed", e);
  return ls;
}

// Runs one part list whose weight streams all take `path`.  A GEMV launch
// takes at most kLaunchParts weight streams; longer lists run as several
// launches (each part's arithmetic does not depend on its launch).
template <int FMT, int NW>
qg_status run_path(const char* op, Path path, const CallCfg& cfg, const HostPart* parts, int nparts,
                   const float* x, int64_t m, int64_t k, int gs, hipStream_t s) {
  const int per = kLaunchParts / NW;
  if (path != P_MFMA && path != P_PLAIN && nparts > per) {
    for (int p0 = 0; p0 < nparts; p0 += per) {
      const qg_status st = run_path<FMT, NW>(op, path, cfg, parts + p0, nparts - p0 < per ? nparts - p0 : per, x,
                                             m, k, gs, s);
      if (st != QG_OK) return st;
    }
    return QG_OK;
  }
  switch (path) {
    case P_MFMA: return run_mfma<FMT>(op, parts, nparts, NW, x, m, k, gs, s);
    case P_PLAIN: return run_plain<FMT, NW>(op, parts, nparts, x, m, k, gs, s);
    case P_XR: return run_gemv_xr<FMT>(op, parts, nparts, NW, x, m, k, gs, s);
    case P_MMA:
      if constexpr (NW == 1) return run_gemv_mma<FMT>(op, parts, nparts, x, m, k, gs, s);
      break;
    case P_FMA: return run_gemv_fma<FMT, NW>(op, cfg, parts, nparts, x, m, k, gs, s);
  }
  snprintf(g_err, sizeof(g_err), "%s: no kernel for this path", op);
  return QG_ELAUNCH;
}

// A part list of single-stream parts: each part takes the path its single
// call would take; parts of one path share a launch.
template <int FMT>
qg_status run_parts(const char* op, const CallCfg& cfg, const HostPart* parts, int nparts, const float* x,
                    int64_t m, int64_t k, int gs, hipStream_t s) {
  Path path[kMaxParts];
  for (int pi = 0; pi < nparts; ++pi) path[pi] = path_of<FMT>(cfg, m, k, gs, parts[pi].w[0], parts[pi].n);
  bool done[kMaxParts] = {};
  for (int pi = 0; pi < nparts; ++pi) {
    if (done[pi]) continue;
    HostPart group[kMaxParts];
    int ng = 0;
    for (int pj = pi; pj < nparts; ++pj)
      if (!done[pj] && path[pj] == path[pi]) {
        group[ng++] = parts[pj];
        done[pj] = true;
      }
    const qg_status st = run_path<FMT, 1>(op, path[pi], cfg, group, ng, x, m, k, gs, s);
    if (st != QG_OK) return st;
  }
  return QG_OK;
}

// ------------------------------------------------------------------ checks
qg_status check_mk(const char* op, int64_t m, int64_t k) {
  if (m < 1 || k < 1) return fail("%s: M and K must be > 0; got (%lld, %lld)", op, (long long)m, (long long)k);
  if (m > kMaxDim || k > kMaxDim)
    return fail("%s: M and K must each be <= 2^30; got (%lld, %lld)", op, (long long)m, (long long)k);
  return QG_OK;
}

qg_status check_mnk(const char* op, int64_t m, int64_t n, int64_t k) {
  if (m < 1 || n < 1 || k < 1)
    return fail("%s: M, N, K must all be > 0; got (%lld, %lld, %lld)", op, (long long)m, (long long)n,
                (long long)k);
  if (m > kMaxDim || n > kMaxDim || k > kMaxDim)
    return fail("%s: M, N, K must each be <= 2^30; got (%lld, %lld, %lld)", op, (long long)m,
                (long long)n, (long long)k);
  return QG_OK;
}

qg_status check_xy(const char* op, const float* x, const float* y) {
  if (!x || !y) return fail("%s: null pointer", op);
  if (!aligned(x, 4) || !aligned(y, 4)) return fail("%s: x and y must be 4-byte aligned", op);
  if (x == y) return fail("%s: y must not alias x", op);
  return QG_OK;
}

qg_status check_group(const char* op, int64_t k, int64_t group_size) {
  if (group_size < 2 || group_size > 1024 || (group_size & (group_size - 1)) != 0)
    return fail("%s: group_size must be a power of two in [2, 1024]; got %lld", op, (long long)group_size);
  if (k % group_size != 0)
    return fail("%s: K (%lld) must be divisible by group_size (%lld)", op, (long long)k, (long long)group_size);
  return QG_OK;
}

qg_status q40_common(const char* op, const void* w, const float* x, float* y, int64_t m, int64_t n,
                     int64_t k) {
  qg_status st = check_mnk(op, m, n, k);
  if (st != QG_OK) return st;
  if (k % 32 != 0) return fail("%s: K (%lld) must be divisible by QK4_0 (32)", op, (long long)k);
  if (!w) return fail("%s: null weight pointer", op);
  if (!aligned(w, 4)) return fail("%s: Q4_0 weights must be 4-byte aligned", op);
  return check_xy(op, x, y);
}

qg_status affine_args(const char* op, const float* x, const uint8_t* q, const float* scales, const float* biases,
                      const float* y, int64_t m, int64_t n, int64_t k, int64_t group_size) {
  qg_status st = check_mnk(op, m, n, k);
  if (st != QG_OK) return st;
  st = check_group(op, k, group_size);
  if (st != QG_OK) return st;
  if (!q || !scales || !biases) return fail("%s: null pointer", op);
  if (!aligned(scales, 4) || !aligned(biases, 4)) return fail("%s: scales/biases must be 4-byte aligned", op);
  return check_xy(op, x, y);
}

// ------------------------------------------------------------------ static scratch
// Scratch of the allocation-free entry point (qmm_affine_t_noalloc): one
// array per GPU, in the code object's device memory, resident until the
// process ends.  Host code never passes `g_scratch` itself (on the host it
// names a stand-in, not device memory): the device address is looked up once
// per device with hipGetSymbolAddress, on that device, and kept in
// g_scratch_dev.  Every call on a GPU shares that GPU's array; the matrix-core
// path writes all of the scratch it reads (x_hi, x_lo and the group sums)
// before reading it, so nothing needs clearing, and calls that overlap on one
// GPU race.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t g_scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

qg_status static_scratch(const char* op, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return launch_error(op, "hipGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices) return fail("%s: device %d outside 0..%d", op, dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_scratch));
    if (e != hipSuccess || p == nullptr) return launch_error(op, "device address of the static scratch", e);
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return QG_OK;
}

HostPart single_part(const void* w, const float* scales, const float* biases, float* y, int64_t ldy, int64_t n) {
  HostPart hp{};
  hp.w[0] = w;
  hp.scales = scales;
  hp.biases = biases;
  hp.y[0] = y;
  hp.ldy = ldy;
  hp.n = n;
  return hp;
}

}  // namespace

extern "C" {

const char* qg_last_error(void) { return g_err; }

qg_status qg_set_mfma_min_m(int64_t m) {
  if (m < 1) return fail("qg_set_mfma_min_m: m must be >= 1; got %lld", (long long)m);
  g_mfma_min_m.store(m);
  return QG_OK;
}

int64_t qg_get_mfma_min_m(void) { return g_mfma_min_m.load(); }

qg_status qg_set_kernel_mask(uint32_t mask) {
  if (mask & ~kAllKernels) return fail("qg_set_kernel_mask: unknown bits 0x%x", (unsigned)(mask & ~kAllKernels));
  g_kernel_mask.store(mask);
  return QG_OK;
}

uint32_t qg_get_kernel_mask(void) { return g_kernel_mask.load(); }

qg_status qgemv_q4_0(const void* w, const float* x, float* y, int64_t M, int64_t N, int64_t K,
                     void* stream) {
  const char* op = "qgemv_q4_0";
  qg_status st = q40_common(op, w, x, y, M, N, K);
  if (st != QG_OK) return st;
  const CallCfg cfg = call_cfg();
  const HostPart hp = single_part(w, nullptr, nullptr, y, N, N);
  return run_parts<FMT_Q40>(op, cfg, &hp, 1, x, M, K, 32, static_cast<hipStream_t>(stream));
}

qg_status qgemv_dual_q4_0(const void* w_a, const void* w_b, const float* x, float* y_a, float* y_b,
                          int64_t M, int64_t N, int64_t K, void* stream) {
  const char* op = "qgemv_dual_q4_0";
  qg_status st = q40_common(op, w_a, x, y_a, M, N, K);
  if (st != QG_OK) return st;
  st = q40_common(op, w_b, x, y_b, M, N, K);
  if (st != QG_OK) return st;
  if (y_a == y_b) return fail("%s: dst_a and dst_b must be different buffers", op);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const CallCfg cfg = call_cfg();
  const HostPart one[2] = {single_part(w_a, nullptr, nullptr, y_a, N, N),
                           single_part(w_b, nullptr, nullptr, y_b, N, N)};
  const Path pa = path_of<FMT_Q40>(cfg, M, K, 32, w_a, N);
  const Path pb = path_of<FMT_Q40>(cfg, M, K, 32, w_b, N);
  // the two weights on different paths (e.g. one of them not 16-byte
  // aligned): each runs as its single call would
  if (pa != pb) {
    st = run_path<FMT_Q40, 1>(op, pa, cfg, &one[0], 1, x, M, K, 32, s);
    return st != QG_OK ? st : run_path<FMT_Q40, 1>(op, pb, cfg, &one[1], 1, x, M, K, 32, s);
  }
  // one pass over x for both weights
  HostPart hp = one[0];
  hp.w[1] = w_b;
  hp.y[1] = y_b;
  return run_path<FMT_Q40, 2>(op, pa, cfg, &hp, 1, x, M, K, 32, s);
}

qg_status qgemv_q4_k(const void* w, const float* x, float* y, int64_t M, int64_t N, int64_t K,
                     void* stream) {
  const char* op = "qgemv_q4_k";
  qg_status st = check_mnk(op, M, N, K);
  if (st != QG_OK) return st;
  if (K % 256 != 0) return fail("%s: K (%lld) must be a multiple of 256", op, (long long)K);
  if (!w) return fail("%s: null weight pointer", op);
  st = check_xy(op, x, y);
  if (st != QG_OK) return st;
  const CallCfg cfg = call_cfg();
  const HostPart hp = single_part(w, nullptr, nullptr, y, N, N);
  return run_parts<FMT_Q4K>(op, cfg, &hp, 1, x, M, K, 32, static_cast<hipStream_t>(stream));
}

qg_status qgemv_q4_k_multi(const void* const* w, float* const* y, const int64_t* n, const int64_t* ldy,
                           int64_t parts, const float* x, int64_t M, int64_t K, void* stream) {
  const char* op = "qgemv_q4_k_multi";
  if (parts < 1 || parts > kMaxParts)
    return fail("%s: parts must be in [1, %d]; got %lld", op, kMaxParts, (long long)parts);
  if (!w || !y || !n || !ldy) return fail("%s: null pointer", op);
  qg_status st = check_mk(op, M, K);
  if (st != QG_OK) return st;
  if (K % 256 != 0) return fail("%s: K (%lld) must be a multiple of 256", op, (long long)K);
  if (!x || !aligned(x, 4)) return fail("%s: x must be a non-null 4-byte aligned pointer", op);
  HostPart hp[kMaxParts];
  for (int64_t p = 0; p < parts; ++p) {
    if (n[p] < 1 || n[p] > kMaxDim)
      return fail("%s: part %lld: rows must be in [1, 2^30]; got %lld", op, (long long)p, (long long)n[p]);
    if (ldy[p] < n[p] || ldy[p] > kMaxDim)
      return fail("%s: part %lld: ldy (%lld) must be in [rows (%lld), 2^30]", op, (long long)p,
                  (long long)ldy[p], (long long)n[p]);
    if (!w[p]) return fail("%s: part %lld: null weight pointer", op, (long long)p);
    st = check_xy(op, x, y[p]);
    if (st != QG_OK) return st;
    hp[p] = single_part(w[p], nullptr, nullptr, y[p], ldy[p], n[p]);
  }
  // each part on the path of its own single call; parts of one path share a launch
  return run_parts<FMT_Q4K>(op, call_cfg(), hp, (int)parts, x, M, K, 32, static_cast<hipStream_t>(stream));
}

qg_status qmm_affine_t(const float* x, const uint8_t* q, const float* scales, const float* biases,
                       float* y, int64_t M, int64_t N, int64_t K, int64_t group_size, void* stream) {
  const char* op = "qmm_affine_t";
  const qg_status st = affine_args(op, x, q, scales, biases, y, M, N, K, group_size);
  if (st != QG_OK) return st;
  const HostPart hp = single_part(q, scales, biases, y, N, N);
  return run_parts<FMT_AFF>(op, call_cfg(), &hp, 1, x, M, K, (int)group_size, static_cast<hipStream_t>(stream));
}

qg_status qmm_affine_t_noalloc(const float* x, const uint8_t* q, const float* scales, const float* biases,
                               float* y, int64_t M, int64_t N, int64_t K, int64_t group_size, void* stream) {
  const char* op = "qmm_affine_t_noalloc";
  qg_status st = affine_args(op, x, q, scales, biases, y, M, N, K, group_size);
  if (st != QG_OK) return st;
  const CallCfg cfg = call_cfg();
  const HostPart hp = single_part(q, scales, biases, y, N, N);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Path path = path_of<FMT_AFF>(cfg, M, K, group_size, q, N);
  // the other paths use no scratch
  if (path != P_MFMA) return run_path<FMT_AFF, 1>(op, path, cfg, &hp, 1, x, M, K, (int)group_size, s);
  const size_t need = mfma_scratch_bytes<FMT_AFF>(M, K, group_size);
  if (need > kStaticScratchBytes)
    return fail("%s: M = %lld, K = %lld, group_size = %lld needs %zu bytes of scratch on the matrix-core path; "
                "the static buffer holds %zu (use qmm_affine_t, which allocates)",
                op, (long long)M, (long long)K, (long long)group_size, need, kStaticScratchBytes);
  void* scr = nullptr;
  st = static_scratch(op, &scr);
  if (st != QG_OK) return st;
  (void)hipGetLastError();
  return launch_mfma<FMT_AFF>(op, &hp, 1, 1, x, M, K, (int)group_size, scr, s);
}

qg_status qmm_affine_t_packed(const float* x, const uint32_t* w_packed, const float* scales,
                              const float* biases, float* y, int64_t M, int64_t N, int64_t K,
                              int64_t group_size, void* stream) {
  const char* op = "qmm_affine_t_packed";
  qg_status st = check_mnk(op, M, N, K);
  if (st != QG_OK) return st;
  if (K % 8 != 0) return fail("%s: K (%lld) must be divisible by the pack factor (8)", op, (long long)K);
  st = check_group(op, K, group_size);
  if (st != QG_OK) return st;
  if (!w_packed || !scales || !biases) return fail("%s: null pointer", op);
  if (!aligned(w_packed, 4)) return fail("%s: w_packed must be 4-byte aligned", op);
  if (!aligned(scales, 4) || !aligned(biases, 4)) return fail("%s: scales/biases must be 4-byte aligned", op);
  st = check_xy(op, x, y);
  if (st != QG_OK) return st;
  const HostPart hp = single_part(w_packed, scales, biases, y, N, N);
  return run_parts<FMT_AFF4>(op, call_cfg(), &hp, 1, x, M, K, (int)group_size, static_cast<hipStream_t>(stream));
}

qg_status qmm_affine_t_qkv(const float* x, const uint8_t* q, const float* scales, const float* biases,
                           float* q_out, float* k_out, float* v_out, int64_t M, int64_t K,
                           int64_t group_size, int64_t q_sp, int64_t k_sp, int64_t v_sp, void* stream) {
  const char* op = "qmm_affine_t_qkv";
  if (q_sp < 1 || k_sp < 1 || v_sp < 1) return fail("%s: q_sp, k_sp, v_sp must all be > 0", op);
  if (q_sp > kMaxDim || k_sp > kMaxDim || v_sp > kMaxDim) return fail("%s: spans must be <= 2^30", op);
  const int64_t N = q_sp + k_sp + v_sp;
  qg_status st = check_mnk(op, M, N, K);
  if (st != QG_OK) return st;
  st = check_group(op, K, group_size);
  if (st != QG_OK) return st;
  if (!q || !scales || !biases) return fail("%s: null pointer", op);
  if (!aligned(scales, 4) || !aligned(biases, 4)) return fail("%s: scales/biases must be 4-byte aligned", op);
  float* outs[3] = {q_out, k_out, v_out};
  for (int i = 0; i < 3; ++i) {
    st = check_xy(op, x, outs[i]);
    if (st != QG_OK) return st;
  }
  if (q_out == k_out || q_out == v_out || k_out == v_out) return fail("%s: outputs must not alias each other", op);
  const int64_t groups = K / group_size;
  const int64_t span[3] = {q_sp, k_sp, v_sp};
  HostPart hp[3];
  int64_t row0 = 0;
  for (int i = 0; i < 3; ++i) {
    hp[i] = single_part(q + row0 * K, scales + row0 * groups, biases + row0 * groups, outs[i], span[i], span[i]);
    row0 += span[i];
  }
  // the path of the product of the whole fused weight, which the result must equal
  const CallCfg cfg = call_cfg();
  const Path path = path_of<FMT_AFF>(cfg, M, K, group_size, q, N);
  return run_path<FMT_AFF, 1>(op, path, cfg, hp, 3, x, M, K, (int)group_size, static_cast<hipStream_t>(stream));
}

qg_status qkv_split_f32(const float* qkv, float* q, float* k, float* v, int64_t seq, int64_t q_sp,
                        int64_t k_sp, int64_t v_sp, void* stream) {
  const char* op = "qkv_split_f32";
  if (seq < 1 || q_sp < 1 || k_sp < 1 || v_sp < 1)
    return fail("%s: seq, q_sp, k_sp, v_sp must all be > 0", op);
  const int64_t ch = q_sp + k_sp + v_sp;
  if (q_sp > 0xFFFFFFFFLL || k_sp > 0xFFFFFFFFLL || v_sp > 0xFFFFFFFFLL || ch > 0xFFFFFFFFLL)
    return fail("%s: q_sp + k_sp + v_sp overflows u32", op);
  if (ch > kMaxDim) return fail("%s: q_sp + k_sp + v_sp must be <= 2^30", op);
  if (seq > ((int64_t)1 << 40) / ch) return fail("%s: seq * channels too large", op);
  if (!qkv || !q || !k || !v) return fail("%s: null pointer", op);
  if (!aligned(qkv, 4) || !aligned(q, 4) || !aligned(k, 4) || !aligned(v, 4))
    return fail("%s: pointers must be 4-byte aligned", op);
  if (q == k || q == v || k == v || qkv == q || qkv == k || qkv == v)
    return fail("%s: outputs must not alias each other or the input", op);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const bool vec = q_sp % 4 == 0 && k_sp % 4 == 0 && v_sp % 4 == 0 && aligned(qkv, 16) && aligned(q, 16) &&
                   aligned(k, 16) && aligned(v, 16);
  const int64_t per_row = vec ? ch / 4 : ch;
  const int64_t bx = cdiv(per_row, 256) < 64 ? cdiv(per_row, 256) : 64;
  const int64_t by = seq < 65535 ? seq : 65535;
  const dim3 grid((unsigned)bx, (unsigned)by);
  if (vec) {
    hipLaunchKernelGGL(qkv_split_kernel<f32x4>, grid, dim3(256), 0, s, reinterpret_cast<const f32x4*>(qkv),
                       reinterpret_cast<f32x4*>(q), reinterpret_cast<f32x4*>(k), reinterpret_cast<f32x4*>(v),
                       (long long)seq, (int)(q_sp / 4), (int)(k_sp / 4), (int)(v_sp / 4));
  } else {
    hipLaunchKernelGGL(qkv_split_kernel<float>, grid, dim3(256), 0, s, qkv, q, k, v, (long long)seq,
                       (int)q_sp, (int)k_sp, (int)v_sp);
  }
  return launch_status(op);
}

}  // extern "C"
