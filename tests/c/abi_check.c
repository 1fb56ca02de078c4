/*
 * abi_check -- drives libqgemv_q4 through its C ABI alone (no Python, no
 * torch): device memory comes from the HIP runtime's C API.  It checks the
 * equalities the header states, bit for bit, on small seeded inputs:
 *   dual Q4_0 = two single Q4_0 calls        (GEMV rows and matrix-core rows)
 *   multi-part Q4_K = one call per part
 *   packed affine codes = u8 affine codes
 *   fused q|k|v product = product, then qkv_split_f32
 *   qkv_split_f32 = an exact copy of each span
 *   the same call twice = the same bits
 * and that a bad argument returns QG_EINVAL with a message before any launch.
 * Without a GPU only the argument checks run.  Exit status 0 means every check
 * passed; the last line printed says which checks ran.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "qgemv_q4.h"

static int g_fail = 0;
#define CHECK(cond, ...)                            \
  do {                                              \
    if (!(cond)) {                                  \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                 \
      fprintf(stderr, "\n");                        \
      g_fail = 1;                                   \
    }                                               \
  } while (0)
#define HIPOK(call)                                                    \
  do {                                                                 \
    hipError_t e_ = (call);                                            \
    if (e_ != hipSuccess) {                                            \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      exit(2);                                                         \
    }                                                                  \
  } while (0)
#define QGOK(call)                                                              \
  do {                                                                          \
    qg_status s_ = (call);                                                      \
    if (s_ != QG_OK) {                                                          \
      fprintf(stderr, "qg error %d (%s) at %s:%d\n", (int)s_, qg_last_error(), __FILE__, __LINE__); \
      exit(3);                                                                  \
    }                                                                           \
  } while (0)

/* 32-bit linear congruential generator (Numerical Recipes constants) */
static uint32_t g_seed = 12345u;
static uint32_t rnd(void) { g_seed = g_seed * 1664525u + 1013904223u; return g_seed; }
static float rndf(void) { return (float)((rnd() >> 8) & 0xFFFF) / 32768.0f - 1.0f; } /* [-1, 1) */

static void* dev_copy(const void* h, size_t bytes) {
  void* d = NULL;
  HIPOK(hipMalloc(&d, bytes));
  HIPOK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  return d;
}
static void* dev_zero(size_t bytes) {
  void* d = NULL;
  HIPOK(hipMalloc(&d, bytes));
  HIPOK(hipMemset(d, 0, bytes));
  return d;
}
static int same_bits(const void* da, const void* db, size_t bytes) {
  unsigned char* a = (unsigned char*)malloc(bytes);
  unsigned char* b = (unsigned char*)malloc(bytes);
  HIPOK(hipMemcpy(a, da, bytes, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(b, db, bytes, hipMemcpyDeviceToHost));
  const int eq = memcmp(a, b, bytes) == 0;
  free(a);
  free(b);
  return eq;
}
static float* host_floats(size_t n) {
  float* v = (float*)malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) v[i] = rndf();
  return v;
}

/* Q4_0 rows: 18-byte blocks, fp16 d in [2^-8, 2^-7) (exponent 7, random mantissa), random nibbles */
static uint8_t* q4_0_rows(int64_t n, int64_t k) {
  const size_t bytes = (size_t)n * (size_t)(k / 32) * 18;
  uint8_t* w = (uint8_t*)malloc(bytes);
  for (size_t b = 0; b < bytes / 18; ++b) {
    const uint16_t d = (uint16_t)((7u << 10) | (rnd() & 0x3FFu));
    w[b * 18] = (uint8_t)(d & 0xFF);
    w[b * 18 + 1] = (uint8_t)(d >> 8);
    for (int i = 2; i < 18; ++i) w[b * 18 + i] = (uint8_t)rnd();
  }
  return w;
}
/* Q4_K rows: 144-byte super-blocks, fp16 d and dmin as above, random scale bytes and nibbles */
static uint8_t* q4_k_rows(int64_t n, int64_t k) {
  const size_t bytes = (size_t)n * (size_t)(k / 256) * 144;
  uint8_t* w = (uint8_t*)malloc(bytes);
  for (size_t b = 0; b < bytes / 144; ++b) {
    for (int h = 0; h < 2; ++h) {
      const uint16_t d = (uint16_t)((7u << 10) | (rnd() & 0x3FFu));
      w[b * 144 + 2 * h] = (uint8_t)(d & 0xFF);
      w[b * 144 + 2 * h + 1] = (uint8_t)(d >> 8);
    }
    for (int i = 4; i < 144; ++i) w[b * 144 + i] = (uint8_t)rnd();
  }
  return w;
}

static void check_arguments(void) {
  /* K = 48 is not a multiple of 32: rejected before any HIP call */
  const qg_status s = qgemv_q4_0((const void*)16, (const float*)16, (float*)16, 1, 1, 48, NULL);
  CHECK(s == QG_EINVAL, "qgemv_q4_0 with K=48 returned %d", (int)s);
  CHECK(strlen(qg_last_error()) > 0, "no message for a rejected call");
  const qg_status z = qkv_split_f32((const float*)16, (float*)32, (float*)48, (float*)64, 0, 1, 1, 1, NULL);
  CHECK(z == QG_EINVAL, "qkv_split_f32 with seq=0 returned %d", (int)z);
}

static void check_dual(int64_t m, int64_t n, int64_t k) {
  uint8_t* wa = q4_0_rows(n, k);
  uint8_t* wb = q4_0_rows(n, k);
  float* x = host_floats((size_t)(m * k));
  const size_t wbytes = (size_t)n * (size_t)(k / 32) * 18, ybytes = (size_t)(m * n) * sizeof(float);
  void* dwa = dev_copy(wa, wbytes);
  void* dwb = dev_copy(wb, wbytes);
  float* dx = (float*)dev_copy(x, (size_t)(m * k) * sizeof(float));
  float *ya = (float*)dev_zero(ybytes), *yb = (float*)dev_zero(ybytes);
  float *sa = (float*)dev_zero(ybytes), *sb = (float*)dev_zero(ybytes);
  QGOK(qgemv_dual_q4_0(dwa, dwb, dx, ya, yb, m, n, k, NULL));
  QGOK(qgemv_q4_0(dwa, dx, sa, m, n, k, NULL));
  QGOK(qgemv_q4_0(dwb, dx, sb, m, n, k, NULL));
  HIPOK(hipDeviceSynchronize());
  CHECK(same_bits(ya, sa, ybytes) && same_bits(yb, sb, ybytes), "dual != two singles at M=%lld", (long long)m);
  /* the same call again gives the same bits */
  QGOK(qgemv_q4_0(dwa, dx, sb, m, n, k, NULL));
  HIPOK(hipDeviceSynchronize());
  CHECK(same_bits(sa, sb, ybytes), "repeated Q4_0 call changed bits at M=%lld", (long long)m);
  hipFree(dwa); hipFree(dwb); hipFree(dx); hipFree(ya); hipFree(yb); hipFree(sa); hipFree(sb);
  free(wa); free(wb); free(x);
}

static void check_multi(int64_t m, int64_t k) {
  const int64_t ns[2] = {96, 40}, total = 136;
  uint8_t* w0 = q4_k_rows(ns[0], k);
  uint8_t* w1 = q4_k_rows(ns[1], k);
  float* x = host_floats((size_t)(m * k));
  const size_t rb = (size_t)(k / 256) * 144;
  void* dw[2] = {dev_copy(w0, rb * ns[0]), dev_copy(w1, rb * ns[1])};
  float* dx = (float*)dev_copy(x, (size_t)(m * k) * sizeof(float));
  float* shared = (float*)dev_zero((size_t)(m * total) * sizeof(float));   /* both parts in one [M, 136] buffer */
  float* s0 = (float*)dev_zero((size_t)(m * ns[0]) * sizeof(float));
  float* s1 = (float*)dev_zero((size_t)(m * ns[1]) * sizeof(float));
  float* ys[2] = {shared, shared + ns[0]};
  const int64_t ldy[2] = {total, total};
  QGOK(qgemv_q4_k_multi((const void* const*)dw, ys, ns, ldy, 2, dx, m, k, NULL));
  QGOK(qgemv_q4_k(dw[0], dx, s0, m, ns[0], k, NULL));
  QGOK(qgemv_q4_k(dw[1], dx, s1, m, ns[1], k, NULL));
  HIPOK(hipDeviceSynchronize());
  float* h = (float*)malloc((size_t)(m * total) * sizeof(float));
  float* h0 = (float*)malloc((size_t)(m * ns[0]) * sizeof(float));
  float* h1 = (float*)malloc((size_t)(m * ns[1]) * sizeof(float));
  HIPOK(hipMemcpy(h, shared, (size_t)(m * total) * sizeof(float), hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(h0, s0, (size_t)(m * ns[0]) * sizeof(float), hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(h1, s1, (size_t)(m * ns[1]) * sizeof(float), hipMemcpyDeviceToHost));
  int ok = 1;
  for (int64_t r = 0; r < m; ++r) {
    ok &= memcmp(h + r * total, h0 + r * ns[0], (size_t)ns[0] * sizeof(float)) == 0;
    ok &= memcmp(h + r * total + ns[0], h1 + r * ns[1], (size_t)ns[1] * sizeof(float)) == 0;
  }
  CHECK(ok, "multi-part Q4_K != one call per part at M=%lld", (long long)m);
  hipFree(dw[0]); hipFree(dw[1]); hipFree(dx); hipFree(shared); hipFree(s0); hipFree(s1);
  free(w0); free(w1); free(x); free(h); free(h0); free(h1);
}

/* affine: u8 codes 0..15, then the same codes packed eight per u32 (element j in bits 4j..4j+3) */
static void check_packed_and_qkv(int64_t m, int64_t k, int64_t gs) {
  const int64_t qs = 64, ks = 32, vs = 32, n = qs + ks + vs, groups = k / gs;
  uint8_t* q = (uint8_t*)malloc((size_t)(n * k));
  uint32_t* qp = (uint32_t*)calloc((size_t)(n * k / 8), sizeof(uint32_t));
  for (int64_t i = 0; i < n * k; ++i) {
    q[i] = (uint8_t)(rnd() & 15u);
    qp[i / 8] |= (uint32_t)q[i] << (4 * (i % 8));
  }
  float* sc = host_floats((size_t)(n * groups));
  float* bi = host_floats((size_t)(n * groups));
  for (int64_t i = 0; i < n * groups; ++i) sc[i] = 0.01f * (sc[i] + 1.5f);
  float* x = host_floats((size_t)(m * k));
  uint8_t* dq = (uint8_t*)dev_copy(q, (size_t)(n * k));
  uint32_t* dqp = (uint32_t*)dev_copy(qp, (size_t)(n * k / 2));
  float* dsc = (float*)dev_copy(sc, (size_t)(n * groups) * sizeof(float));
  float* dbi = (float*)dev_copy(bi, (size_t)(n * groups) * sizeof(float));
  float* dx = (float*)dev_copy(x, (size_t)(m * k) * sizeof(float));
  const size_t yb = (size_t)(m * n) * sizeof(float);
  float *y8 = (float*)dev_zero(yb), *y4 = (float*)dev_zero(yb);
  QGOK(qmm_affine_t(dx, dq, dsc, dbi, y8, m, n, k, gs, NULL));
  QGOK(qmm_affine_t_packed(dx, dqp, dsc, dbi, y4, m, n, k, gs, NULL));
  HIPOK(hipDeviceSynchronize());
  CHECK(same_bits(y8, y4, yb), "packed codes != u8 codes at M=%lld", (long long)m);
  /* fused q|k|v = product, then split */
  float *qo = (float*)dev_zero((size_t)(m * qs) * 4), *ko = (float*)dev_zero((size_t)(m * ks) * 4),
        *vo = (float*)dev_zero((size_t)(m * vs) * 4);
  float *qr = (float*)dev_zero((size_t)(m * qs) * 4), *kr = (float*)dev_zero((size_t)(m * ks) * 4),
        *vr = (float*)dev_zero((size_t)(m * vs) * 4);
  QGOK(qmm_affine_t_qkv(dx, dq, dsc, dbi, qo, ko, vo, m, k, gs, qs, ks, vs, NULL));
  QGOK(qkv_split_f32(y8, qr, kr, vr, m, qs, ks, vs, NULL));
  HIPOK(hipDeviceSynchronize());
  CHECK(same_bits(qo, qr, (size_t)(m * qs) * 4) && same_bits(ko, kr, (size_t)(m * ks) * 4) &&
            same_bits(vo, vr, (size_t)(m * vs) * 4),
        "fused q|k|v != product then split at M=%lld", (long long)m);
  /* the split itself is an exact copy of each span */
  float* h = (float*)malloc(yb);
  float* hq = (float*)malloc((size_t)(m * qs) * 4);
  float* hk = (float*)malloc((size_t)(m * ks) * 4);
  float* hv = (float*)malloc((size_t)(m * vs) * 4);
  HIPOK(hipMemcpy(h, y8, yb, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(hq, qr, (size_t)(m * qs) * 4, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(hk, kr, (size_t)(m * ks) * 4, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(hv, vr, (size_t)(m * vs) * 4, hipMemcpyDeviceToHost));
  int ok = 1;
  for (int64_t r = 0; r < m; ++r) {
    ok &= memcmp(h + r * n, hq + r * qs, (size_t)qs * 4) == 0;
    ok &= memcmp(h + r * n + qs, hk + r * ks, (size_t)ks * 4) == 0;
    ok &= memcmp(h + r * n + qs + ks, hv + r * vs, (size_t)vs * 4) == 0;
  }
  CHECK(ok, "qkv_split_f32 is not an exact copy at M=%lld", (long long)m);
  hipFree(dq); hipFree(dqp); hipFree(dsc); hipFree(dbi); hipFree(dx); hipFree(y8); hipFree(y4);
  hipFree(qo); hipFree(ko); hipFree(vo); hipFree(qr); hipFree(kr); hipFree(vr);
  free(q); free(qp); free(sc); free(bi); free(x); free(h); free(hq); free(hk); free(hv);
}

int main(void) {
  check_arguments();
  int devices = 0;
  if (hipGetDeviceCount(&devices) != hipSuccess || devices == 0) {
    printf("abi_check: %s (no GPU: argument checks only)\n", g_fail ? "FAILED" : "ok");
    return g_fail;
  }
  const int64_t mfma_m = qg_get_mfma_min_m();
  check_dual(3, 200, 512);
  check_dual(mfma_m + 6, 200, 512);
  check_multi(2, 512);
  check_multi(mfma_m + 1, 512);
  check_packed_and_qkv(5, 256, 64);
  check_packed_and_qkv(mfma_m + 3, 256, 64);
  printf("abi_check: %s (argument checks; dual, multi-part, packed, fused q|k|v and split at M below and above %lld)\n",
         g_fail ? "FAILED" : "ok", (long long)mfma_m);
  return g_fail;
}
