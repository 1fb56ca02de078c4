/*
 * libqgemv_q4 -- dequantize-fused GEMV / skinny GEMM with 4-bit block-quantized
 * weights on AMD Instinct MI355X (gfx950).  C ABI.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    keeps no pointer after a call returns.  qmm_affine_t allocates and frees
 *    stream-ordered scratch for its prefill path (see below); nothing else
 *    allocates.
 *  - Row-major, contiguous.  x is [M, K] f32, y is [M, N] f32:
 *        y[m, n] = sum_k x[m, k] * w[n, k]
 *    where w is the dequantized weight.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls are
 *    asynchronous and ordered on that stream, like an encode-then-commit
 *    (mlx-native op modules: dispatch records work, the command buffer commit
 *    runs it).
 *  - Outputs must not overlap inputs or each other.
 *  - Errors: every argument check runs before any HIP call; on error nothing is
 *    launched or written, QG_EINVAL is returned and qg_last_error() names the
 *    problem (the pages' ops return MlxError::InvalidArgument on zero dims,
 *    misaligned K and bad group sizes).  A failed kernel launch returns
 *    QG_ELAUNCH.
 *  - Sizes are int64_t; buffers carry no size, so byte-length checks are the
 *    caller's (the Python binding checks them against its tensors).
 *  - Results are deterministic: the same call on the same data gives the same
 *    bits.  Floating-point results match the exact product within
 *    max |y - y_exact| <= 1e-5 * sum_k |x[m,k] * w[n,k]|.
 */
#ifndef QGEMV_Q4_H
#define QGEMV_Q4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { QG_OK = 0, QG_EINVAL = 1, QG_ELAUNCH = 2 } qg_status;

/* Message for the last failing call on the calling thread ("" if none). */
const char* qg_last_error(void);

/*
 * qgemv_q4_0 -- y = x * W^T with GGML Q4_0 weights.
 * Defined by: mlx-native `fused_dual_proj_q4_0.rs` (preconditions of
 * dispatch_fused_dual_proj_q4_0, which fuses two `kernel_mul_mv_q4_0_f32`
 * products of this kind).
 *   w : [N][K/32] blocks of 18 bytes: little-endian fp16 d, then 16 bytes
 *       qs; the low nibble of qs[j] is element j and the high nibble element
 *       j+16 of the block; value = (nibble - 8) * d.  4-byte aligned.
 *   x : [M, K] f32;  y : [M, N] f32.
 * Errors: M, N, K < 1; K % 32 != 0; null pointers; w not 4-byte aligned;
 *         x or y not 4-byte aligned.
 */
qg_status qgemv_q4_0(const void* w, const float* x, float* y,
                     int64_t M, int64_t N, int64_t K, void* stream);

/*
 * qgemv_q4_k -- y = x * W^T with GGML Q4_K weights.
 * Defined by: ferrum-kernels `q4_k_gemv_v2.rs` (module doc and the `nb01`
 * row stride of dispatch_gemv_q4k_v2_offset: row-major [N][K/256] blocks of
 * 144 bytes, K % 256 == 0).  The page has M = 1; M >= 1 is accepted here.
 *   w : [N][K/256] super-blocks of 144 bytes: fp16 d @0, fp16 dmin @2,
 *       12 bytes of packed 6-bit sub-block scales/mins @4, 128 nibble bytes
 *       @16 (low nibble of qs[32c+l] = element 64c+l, high nibble = element
 *       64c+32+l); value in sub-block j = d*sc[j]*q - dmin*m[j].
 *       Pointer offsets into a larger buffer are plain pointer arithmetic.
 *   x : [M, K] f32;  y : [M, N] f32.
 * Errors: M, N, K < 1; K % 256 != 0; null pointers; x or y not 4-byte aligned.
 */
qg_status qgemv_q4_k(const void* w, const float* x, float* y,
                     int64_t M, int64_t N, int64_t K, void* stream);

/*
 * qgemv_dual_q4_0 -- y_a = x * W_a^T and y_b = x * W_b^T in one pass over x.
 * Defined by: mlx-native `fused_dual_proj_q4_0.rs` (module doc: two weight
 * matrices of the same shape share one input; the result is byte-identical
 * to two single Q4_0 products).  Here: bitwise equal to two qgemv_q4_0
 * calls with the same M, N, K.
 *   w_a, w_b : as `w` of qgemv_q4_0, same shape;  x : [M, K] f32;
 *   y_a, y_b : [M, N] f32.
 * Errors: as qgemv_q4_0 for both weights; y_a == y_b.
 */
qg_status qgemv_dual_q4_0(const void* w_a, const void* w_b, const float* x,
                          float* y_a, float* y_b,
                          int64_t M, int64_t N, int64_t K, void* stream);

/*
 * qmm_affine_t -- y = x * (scales * q + biases)^T, MLX-style affine groups.
 * Defined by: mlx-native `qmm_affine.rs` (dispatch_qmm_affine_t_f32 and the
 * f64 reference qmm_affine_t_cpu in its tests).
 *   x : [M, K] f32;  q : [N, K] u8 codes (any value 0..255);
 *   scales, biases : [N, K/group_size] f32;  y : [M, N] f32.
 *   group_size : power of two in [2, 1024], K % group_size == 0.
 * For M >= qg_get_mfma_min_m() (and 32 <= group_size <= 512, K % 64 == 0,
 * q 16-byte aligned) the product runs on the matrix cores; x is split into
 * two bf16 terms so the f32 tolerance above still holds.  That path takes
 * stream-ordered scratch (hipMallocAsync / hipFreeAsync on `stream`) of
 * M*K*4 + M*(K/group_size)*4 bytes (plus alignment).
 * Errors: M, N, K < 1; bad group_size; K % group_size != 0; null pointers;
 *         misaligned f32 pointers.
 */
qg_status qmm_affine_t(const float* x, const uint8_t* q, const float* scales,
                       const float* biases, float* y,
                       int64_t M, int64_t N, int64_t K, int64_t group_size,
                       void* stream);

/*
 * qkv_split_f32 -- split a fused QKV activation into contiguous q, k, v.
 * Defined by: mlx-native `qkv_split.rs` (module doc and
 * dispatch_qkv_split_f32): qkv[t, :] = [Q (q_sp) | K (k_sp) | V (v_sp)].
 *   qkv : [seq, q_sp + k_sp + v_sp] f32;
 *   q : [seq, q_sp], k : [seq, k_sp], v : [seq, v_sp] f32.
 * Every element is copied bit for bit (NaN payloads and -0 included).
 * Errors: seq, q_sp, k_sp, v_sp < 1; q_sp + k_sp + v_sp above 2^32 - 1 (the
 *         page's u32 channel count); null pointers; misaligned pointers.
 */
qg_status qkv_split_f32(const float* qkv, float* q, float* k, float* v,
                        int64_t seq, int64_t q_sp, int64_t k_sp, int64_t v_sp,
                        void* stream);

/*
 * Tuning knob: smallest M at which qmm_affine_t uses the matrix-core path
 * (default 64).  Process-wide.  qg_set_mfma_min_m returns QG_EINVAL for m < 1.
 */
qg_status qg_set_mfma_min_m(int64_t m);
int64_t qg_get_mfma_min_m(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_Q4_H */
