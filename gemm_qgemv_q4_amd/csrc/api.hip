// C ABI of libqgemv_q4 (declared in include/qgemv_q4.h): argument checks,
// kernel-variant choice and launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "qgemv_q4.h"
#include "kernels/gemv.hpp"
#include "kernels/mfma.hpp"
#include "kernels/split.hpp"

using namespace qg;

namespace {

thread_local char g_err[512] = "";
std::atomic<int64_t> g_mfma_min_m{64};

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

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // keeps every in-kernel 32-bit index in range
constexpr size_t kLdsBudget = 64 * 1024;       // per-workgroup x tile when K is tiled
constexpr size_t kLdsPersistent = 150 * 1024;  // whole-K x tile of a persistent workgroup
constexpr size_t kLdsMax = 160 * 1024;

// ------------------------------------------------------------------ GEMV
struct GemvPlan {
  int mt, l, r, waves, kt, grid;
  size_t lds;
  bool persistent;
};

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return 256;
  return cus;
}

// Launch shape of the chunked GEMV kernel.  x of one m-tile is staged in LDS
// once per workgroup when it fits (persistent workgroups walk several row
// groups); otherwise each workgroup owns one row group and stages x in K tiles.
template <int FMT>
GemvPlan plan_gemv(int64_t m, int64_t n, int64_t k, int nw) {
  constexpr int CH = FmtTraits<FMT>::CH;
  constexpr bool SUMS = FmtTraits<FMT>::SUMS;
  GemvPlan pl{};
  const int64_t chunks = k / CH;
  pl.mt = m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : 8;
  // Measured on MI355X: at MT >= 4 two rows per wave side by side (L = 32) and
  // one 512-thread workgroup per CU are best; at MT <= 2 a full wave per row.
  // Rows shorter than 32 chunks still get 32 lanes (two rows per wave; the
  // lanes past the row's end idle), which measured faster than narrower groups.
  const int lmax = pl.mt >= 4 ? 32 : 64;
  pl.l = chunks >= lmax ? lmax : 32;
  auto lds_for = [&](int64_t kt) {
    const int64_t ct = kt / CH;
    return (size_t)(pl.mt * (CH / 4) * (ct + 1) * 16 + (SUMS ? pl.mt * ct * 8 : 0));
  };
  // Tuning override "L,R,W,B" (0 keeps the automatic choice; B = workgroups per CU
  // of the persistent grid), e.g. QG_GEMV_PLAN=32,2,4,2
  int el = 0, er = 0, ew = 0, eb = 0;
  if (const char* env = getenv("QG_GEMV_PLAN")) {
    if (sscanf(env, "%d,%d,%d,%d", &el, &er, &ew, &eb) < 1) el = er = ew = eb = 0;
  }
  if (el == 8 || el == 16 || el == 32 || el == 64) pl.l = el;
  const int p_rows = 64 / pl.l;
  const int64_t mtiles = cdiv(m, pl.mt);
  int r = (pl.mt * nw <= 2 && chunks >= 64) ? 2 : 1;
  if (er == 1 || (er == 2 && pl.mt * nw <= 2) || (er == 4 && pl.mt * nw == 1)) r = er;
  pl.r = r;

  pl.persistent = lds_for(k) <= kLdsPersistent;
  if (pl.persistent) {
    pl.kt = (int)k;
    pl.lds = lds_for(k);
    pl.waves = (FMT == FMT_AFF && pl.mt <= 2) ? 4 : 8;
    if (ew == 1 || ew == 2 || ew == 4 || ew == 8) pl.waves = ew;
    int bpc = (int)(kLdsMax / (pl.lds ? pl.lds : 1));
    const int bpc_max = pl.waves == 8 ? 1 : 4;
    bpc = bpc < 1 ? 1 : bpc > bpc_max ? bpc_max : bpc;
    if (eb >= 1 && eb <= 8 && (size_t)eb * pl.lds <= kLdsMax) bpc = eb;
    const int64_t groups = cdiv(n, (int64_t)pl.waves * p_rows * r);
    const int64_t cap = (int64_t)device_cus() * bpc;
    pl.grid = (int)(groups < cap ? groups : cap);
  } else {
    pl.waves = 4;
    if (ew == 1 || ew == 2 || ew == 4) pl.waves = ew;
    const int64_t step = (int64_t)pl.l * CH;
    int64_t kt = step;
    while (kt + step <= k && lds_for(kt + step) <= kLdsBudget) kt += step;
    pl.kt = (int)kt;
    pl.lds = lds_for(kt);
    pl.grid = (int)cdiv(n, (int64_t)pl.waves * p_rows * r);
  }
  (void)mtiles;
  return pl;
}

template <int FMT, int MT, int NW, int L, int R>
hipError_t launch_gemv_t(const GemvParams& p, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
  auto kern = gemv_kernel<FMT, MT, NW, L, R>;
  if (lds > 64 * 1024) {
    static std::atomic<bool> raised{false};
    if (!raised.load()) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
      if (e != hipSuccess) return e;
      raised.store(true);
    }
  }
  hipLaunchKernelGGL(kern, grid, block, lds, s, p);
  return hipSuccess;
}

template <int FMT, int MT, int NW, int L>
hipError_t launch_gemv_r(int r, const GemvParams& p, dim3 g, dim3 b, size_t lds, hipStream_t s) {
  // row sets per wave that fit the 256-VGPR budget of a 512-thread workgroup
  switch (r) {
    case 4:
      if constexpr (MT * NW == 1) return launch_gemv_t<FMT, MT, NW, L, 4>(p, g, b, lds, s);
      break;
    case 2:
      if constexpr (MT * NW <= 2) return launch_gemv_t<FMT, MT, NW, L, 2>(p, g, b, lds, s);
      break;
    case 1: return launch_gemv_t<FMT, MT, NW, L, 1>(p, g, b, lds, s);
  }
  return hipErrorInvalidValue;
}

template <int FMT, int MT, int NW>
hipError_t launch_gemv_l(int l, int r, const GemvParams& p, dim3 g, dim3 b, size_t lds, hipStream_t s) {
  switch (l) {
    case 64: return launch_gemv_r<FMT, MT, NW, 64>(r, p, g, b, lds, s);
    case 32: return launch_gemv_r<FMT, MT, NW, 32>(r, p, g, b, lds, s);
    case 16: return launch_gemv_r<FMT, MT, NW, 16>(r, p, g, b, lds, s);
    case 8: return launch_gemv_r<FMT, MT, NW, 8>(r, p, g, b, lds, s);
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

// Runs the chunked kernel (or the plain one when `plain`) over all m-tiles.
template <int FMT, int NW>
qg_status run_gemv(const char* op, GemvParams p, int64_t m, bool plain, hipStream_t s) {
  (void)hipGetLastError();
  if (plain) {
    const dim3 block(256);
    for (int64_t m0 = 0; m0 < m; m0 += 65535) {
      const int64_t mc = m - m0 < 65535 ? m - m0 : 65535;
      GemvParams q = p;
      q.x = p.x + m0 * p.k;
      q.y0 = p.y0 + m0 * p.n;
      if (NW == 2) q.y1 = p.y1 + m0 * p.n;
      const dim3 grid((unsigned)cdiv(p.n, 256), (unsigned)mc);
      hipLaunchKernelGGL((gemv_plain_kernel<FMT, NW>), grid, block, 0, s, q, (int)mc);
    }
    return launch_status(op);
  }
  const GemvPlan pl = plan_gemv<FMT>(m, p.n, p.k, NW);
  const int p_rows = 64 / pl.l;
  p.kt = pl.kt;
  p.rows_per_block = pl.waves * p_rows * pl.r;
  const dim3 block(64 * pl.waves);
  const int64_t blocks_x = pl.grid;
  for (int64_t m0 = 0; m0 < m; m0 += pl.mt) {
    GemvParams q = p;
    q.x = p.x + m0 * p.k;
    q.y0 = p.y0 + m0 * p.n;
    if (NW == 2) q.y1 = p.y1 + m0 * p.n;
    q.m_rows = (int)(m - m0 < pl.mt ? m - m0 : pl.mt);
    const hipError_t e = launch_gemv_mt<FMT, NW>(pl, q, dim3((unsigned)blocks_x), block, s);
    if (e != hipSuccess) {
      snprintf(g_err, sizeof(g_err), "%s: launch setup failed: %s", op, hipGetErrorString(e));
      return QG_ELAUNCH;
    }
  }
  return launch_status(op);
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

qg_status q40_common(const char* op, const void* w, const float* x, float* y, int64_t m, int64_t n,
                     int64_t k) {
  qg_status st = check_mnk(op, m, n, k);
  if (st != QG_OK) return st;
  if (k % 32 != 0) return fail("%s: K (%lld) must be divisible by QK4_0 (32)", op, (long long)k);
  if (!w) return fail("%s: null weight pointer", op);
  if (!aligned(w, 4)) return fail("%s: Q4_0 weights must be 4-byte aligned", op);
  return check_xy(op, x, y);
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

qg_status qgemv_q4_0(const void* w, const float* x, float* y, int64_t M, int64_t N, int64_t K,
                     void* stream) {
  const char* op = "qgemv_q4_0";
  qg_status st = q40_common(op, w, x, y, M, N, K);
  if (st != QG_OK) return st;
  GemvParams p{};
  p.w0 = static_cast<const uint8_t*>(w);
  p.x = x;
  p.y0 = y;
  p.row_bytes = K / 32 * 18;
  p.n = (int)N;
  p.k = (int)K;
  return run_gemv<FMT_Q40, 1>(op, p, M, K % 64 != 0, static_cast<hipStream_t>(stream));
}

qg_status qgemv_dual_q4_0(const void* w_a, const void* w_b, const float* x, float* y_a, float* y_b,
                          int64_t M, int64_t N, int64_t K, void* stream) {
  const char* op = "qgemv_dual_q4_0";
  qg_status st = q40_common(op, w_a, x, y_a, M, N, K);
  if (st != QG_OK) return st;
  st = q40_common(op, w_b, x, y_b, M, N, K);
  if (st != QG_OK) return st;
  if (y_a == y_b) return fail("%s: dst_a and dst_b must be different buffers", op);
  GemvParams p{};
  p.w0 = static_cast<const uint8_t*>(w_a);
  p.w1 = static_cast<const uint8_t*>(w_b);
  p.x = x;
  p.y0 = y_a;
  p.y1 = y_b;
  p.row_bytes = K / 32 * 18;
  p.n = (int)N;
  p.k = (int)K;
  return run_gemv<FMT_Q40, 2>(op, p, M, K % 64 != 0, static_cast<hipStream_t>(stream));
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
  GemvParams p{};
  p.w0 = static_cast<const uint8_t*>(w);
  p.x = x;
  p.y0 = y;
  p.row_bytes = K / 256 * 144;
  p.n = (int)N;
  p.k = (int)K;
  return run_gemv<FMT_Q4K, 1>(op, p, M, !aligned(w, 16), static_cast<hipStream_t>(stream));
}

qg_status qmm_affine_t(const float* x, const uint8_t* q, const float* scales, const float* biases,
                       float* y, int64_t M, int64_t N, int64_t K, int64_t group_size, void* stream) {
  const char* op = "qmm_affine_t";
  qg_status st = check_mnk(op, M, N, K);
  if (st != QG_OK) return st;
  if (group_size < 2 || group_size > 1024 || (group_size & (group_size - 1)) != 0)
    return fail("%s: group_size must be a power of two in [2, 1024]; got %lld", op, (long long)group_size);
  if (K % group_size != 0)
    return fail("%s: K (%lld) must be divisible by group_size (%lld)", op, (long long)K,
                (long long)group_size);
  if (!q || !scales || !biases) return fail("%s: null pointer", op);
  if (!aligned(scales, 4) || !aligned(biases, 4)) return fail("%s: scales/biases must be 4-byte aligned", op);
  st = check_xy(op, x, y);
  if (st != QG_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int gs = (int)group_size;

  if (M >= g_mfma_min_m.load() && gs >= 32 && gs <= 512 && K % 64 == 0 && aligned(q, 16) &&
      M * K < ((int64_t)1 << 31) && N * K < ((int64_t)1 << 31)) {
    // ---- matrix-core path: prepare x (bf16 hi/lo + group sums), then GEMM
    const int64_t groups = K / gs;
    const size_t bytes_x = (size_t)M * K * sizeof(__bf16);
    const size_t bytes_s = (size_t)M * groups * sizeof(__bf16);
    const size_t bytes = 2 * bytes_x + 2 * bytes_s + 512;
    (void)hipGetLastError();
    void* scratch = nullptr;
    hipError_t e = hipMallocAsync(&scratch, bytes, s);
    if (e != hipSuccess) {
      snprintf(g_err, sizeof(g_err), "%s: scratch allocation of %zu bytes failed: %s", op, bytes,
               hipGetErrorString(e));
      return QG_ELAUNCH;
    }
    auto align256 = [](void* p) {
      return reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(p) + 255) & ~(uintptr_t)255);
    };
    __bf16* xh = static_cast<__bf16*>(scratch);
    __bf16* xl = xh + (size_t)M * K;
    __bf16* sh = static_cast<__bf16*>(align256(xl + (size_t)M * K));
    __bf16* sl = static_cast<__bf16*>(align256(sh + (size_t)M * groups));
    const int64_t items = M * (K / 8);
    hipLaunchKernelGGL(affine_prep_kernel, dim3((unsigned)cdiv(items, 256)), dim3(256), 0, s, x, xh, xl, sh, sl,
                       (int)M, (int)K, gs);
    MfmaParams mp{};
    mp.xh = xh;
    mp.xl = xl;
    mp.sh = sh;
    mp.sl = sl;
    mp.q = q;
    mp.scales = scales;
    mp.biases = biases;
    mp.y = y;
    mp.m = (int)M;
    mp.n = (int)N;
    mp.k = (int)K;
    mp.gs = gs;
    mp.tiles_m = (int)cdiv(M, kBM);
    mp.tiles_n = (int)cdiv(N, kBN);
    hipLaunchKernelGGL(affine_mfma_kernel, dim3((unsigned)(mp.tiles_m * mp.tiles_n)), dim3(512), 0, s, mp);
    const qg_status ls = launch_status(op);
    e = hipFreeAsync(scratch, s);
    if (ls == QG_OK && e != hipSuccess) {
      snprintf(g_err, sizeof(g_err), "%s: scratch release failed: %s", op, hipGetErrorString(e));
      return QG_ELAUNCH;
    }
    return ls;
  }

  GemvParams p{};
  p.w0 = q;
  p.scales = scales;
  p.biases = biases;
  p.x = x;
  p.y0 = y;
  p.row_bytes = K;
  p.n = (int)N;
  p.k = (int)K;
  p.gs = gs;
  const bool plain = (K % 16 != 0) || gs < 16 || !aligned(q, 16);
  return run_gemv<FMT_AFF, 1>(op, p, M, plain, s);
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
