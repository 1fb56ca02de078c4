/*
 * libqgemv_q4 -- dequantize-fused GEMV / skinny GEMM with 4-bit block-quantized
 * weights on AMD Instinct MI355X (gfx950).  C ABI.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    keeps no pointer after a call returns.  The product calls allocate and
 *    free stream-ordered scratch for their matrix-core path, or under stream
 *    capture take graph-owned scratch (see "Prefill rows" below); nothing
 *    else allocates.
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
 *  - Prefill rows: from M >= qg_get_mfma_min_m() rows of x on (and K % 64 ==
 *    0, the weights aligned for 16-byte loads -- 8 for packed codes, 4 for
 *    Q4_0 -- and for the affine formats 32 <= group_size <= 512) a product
 *    runs on the matrix cores.  x is split into two bf16 terms so the f32
 *    tolerance above still holds.  That path takes stream-ordered scratch
 *    (hipMallocAsync / hipFreeAsync on `stream`) of 4*M*K bytes, plus
 *    4*M*(K/gs) bytes for the formats with an offset or bias term (Q4_K: gs =
 *    32; affine), each array rounded up to 256 bytes.  While `stream` is
 *    being captured into a graph, the call instead takes a device buffer
 *    owned by that graph (hipMalloc in relaxed capture mode on first need,
 *    attached to the graph as a user object); once the graph and every
 *    executable graph made from it are destroyed, the buffer returns to a
 *    per-device pool that later captures reuse (it is never freed back).
 *    Executable graphs made from one captured graph or its clones share
 *    these buffers and must not run at the same time.
 *  - Few rows on the matrix cores: for 2 <= M below that threshold, the
 *    affine formats with group_size >= 64, K a multiple of 512 with K/512 in
 *    {1, 2, 4, 8} and codes aligned (16 bytes for u8, 8 for packed) run on
 *    the matrix cores in launches of up to 8 rows of x, with x split the
 *    same way and no scratch; from 3 <= M below that threshold Q4_0, Q4_K
 *    and the affine formats (group_size >= 64) with K a multiple of 512 up
 *    to 4096 and the weights 16-byte aligned run on the matrix cores with x
 *    held in registers, also without scratch.  The same tolerance holds.
 *  - Which kernel computes a weight tensor depends on the format, M, K, the
 *    group size, that tensor's own alignment and size, and the two settings
 *    at the end of this header as the call reads them; never on the other
 *    tensors of the call.  So the equalities stated below (dual = two
 *    singles, multi-part = one call per part, fused split = product then
 *    split) hold bit for bit for every accepted alignment; packed = unpacked
 *    holds when both code tensors are 16-byte aligned (they are two tensors,
 *    and each takes the kernel its own alignment allows).
 *  - Q4_0 blocks whose codes are all 8 (weights 0) contribute exactly 0 on
 *    every path: a row of such blocks gives +0 or -0 for any finite x.
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
 * calls with the same M, N, K, for any alignment of each weight (when the
 * two weights take different kernels, each runs as its single call would).
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
 * Errors: M, N, K < 1; bad group_size; K % group_size != 0; null pointers;
 *         misaligned f32 pointers.
 */
qg_status qmm_affine_t(const float* x, const uint8_t* q, const float* scales,
                       const float* biases, float* y,
                       int64_t M, int64_t N, int64_t K, int64_t group_size,
                       void* stream);

/*
 * qmm_affine_t_noalloc -- qmm_affine_t that allocates nothing.
 * For callers that cannot allocate device memory during the call: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels and results as qmm_affine_t (bit for bit under the
 * same settings).  Where qmm_affine_t would take stream-ordered scratch (the
 * matrix-core path, from M >= qg_get_mfma_min_m()), this call uses a static
 * device array of 16 MiB per GPU instead, which the library holds on every
 * GPU it runs on until the process ends; the device address is looked up on
 * a device's first call (no allocation).  The scratch needed is 4*M*K bytes
 * plus 4*M*(K/group_size), each rounded up to 256 bytes; a call on that path
 * needing more than 16 MiB returns QG_EINVAL before any launch.  Calls that
 * overlap on one GPU (several streams or threads) share the array and race:
 * order them on one stream.  The caller passes every input and output.
 * Errors: as qmm_affine_t; scratch beyond the 16 MiB limit.
 */
qg_status qmm_affine_t_noalloc(const float* x, const uint8_t* q, const float* scales,
                               const float* biases, float* y,
                               int64_t M, int64_t N, int64_t K, int64_t group_size,
                               void* stream);

/*
 * qgemv_q4_k_multi -- the parts of a fused projection in one launch (up to
 * four parts per launch of the GEMV kernels; more parts take more launches).
 * Defined by: ferrum-kernels `q4_k_gemv_v2.rs` (doc of
 * dispatch_gemv_q4k_v2_offset: each part of a fused projection has its own
 * weights and writes a disjoint slice of a shared output buffer).
 *   parts      : number of parts, 1..8.
 *   w[p]       : Q4_K weights of part p, [n[p]][K/256] super-blocks as for
 *                qgemv_q4_k.
 *   y[p], ldy[p] : output of part p: y[p][m*ldy[p] + j] = sum_k x[m,k] *
 *                W_p[j,k] for j < n[p].  For one shared output Y[M, N_total]
 *                pass y[p] = Y + (first column of part p), ldy[p] = N_total.
 *   x : [M, K] f32 shared by all parts.
 * Each part's result is bitwise equal to qgemv_q4_k on that part alone, for
 * any alignment of each part's weights (parts on different kernels run in
 * separate launches).  Output slices must not overlap each other or x.
 * Errors: parts outside 1..8; M, K, n[p] < 1; K % 256 != 0; ldy[p] < n[p];
 *         null pointers; x or y[p] not 4-byte aligned.
 */
qg_status qgemv_q4_k_multi(const void* const* w, float* const* y, const int64_t* n,
                           const int64_t* ldy, int64_t parts, const float* x,
                           int64_t M, int64_t K, void* stream);

/*
 * qmm_affine_t_packed -- qmm_affine_t with 4-bit codes packed eight per word.
 * Defined by: mlx-native `qmm_affine.rs` (dispatch_qmm_affine_t_packed_simd4_b4
 * and the pack_b4_to_u32 helper of its tests: the code of element 8*kp + j
 * sits in bits 4j..4j+3 of u32 word kp; the packed product is byte-identical
 * to the unpacked one).
 *   w_packed : [N, K/8] u32, 4-byte aligned;  scales, biases : [N, K/gs] f32;
 *   x : [M, K] f32;  y : [M, N] f32.
 *   group_size : power of two in [2, 1024], K % group_size == 0, K % 8 == 0.
 *   (The page's kernel takes group_size 32 only; any group size is taken here.)
 * Bitwise equal to qmm_affine_t on the unpacked u8 codes when w_packed and
 * the u8 codes are both 16-byte aligned.  Half the weight bytes.
 * Errors: as qmm_affine_t; K % 8 != 0.
 */
qg_status qmm_affine_t_packed(const float* x, const uint32_t* w_packed, const float* scales,
                              const float* biases, float* y,
                              int64_t M, int64_t N, int64_t K, int64_t group_size,
                              void* stream);

/*
 * qmm_affine_t_qkv -- fused QKV projection with the split in its epilogue.
 * Defined by: mlx-native `qkv_split.rs` (module doc: the fused projection's
 * output [seq, q|k|v] is split into contiguous q, k, v) over the product of
 * mlx-native `qmm_affine.rs`.
 *   q : [N, K] u8 codes with N = q_sp + k_sp + v_sp (rows 0..q_sp-1 give q,
 *       the next k_sp rows k, the last v_sp rows v); scales, biases:
 *       [N, K/gs] f32;  x : [M, K] f32.
 *   q_out : [M, q_sp], k_out : [M, k_sp], v_out : [M, v_sp] f32.
 * Bitwise equal to qmm_affine_t into a [M, N] buffer followed by
 * qkv_split_f32; the [M, N] intermediate is never written.
 * Errors: as qmm_affine_t; a span < 1; outputs aliasing each other.
 */
qg_status qmm_affine_t_qkv(const float* x, const uint8_t* q, const float* scales,
                           const float* biases, float* q_out, float* k_out, float* v_out,
                           int64_t M, int64_t K, int64_t group_size,
                           int64_t q_sp, int64_t k_sp, int64_t v_sp, void* stream);

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
 * Settings (process-wide; each product call reads both once, at its start).
 * Changing one changes which kernels later calls run, and so their rounding
 * within the stated tolerance; the bitwise equalities above hold between
 * calls made under the same settings.  Calls that run while another thread
 * changes a setting may see either value.
 *
 * qg_set_mfma_min_m: smallest M at which the product calls use the
 *   matrix-core GEMM (default 64).  QG_EINVAL for m < 1.
 * qg_set_kernel_mask: which of the optional kernels may run (default: all).
 *   QG_KERNEL_KSLICED  the K-sliced GEMV at few rows of x; without it the
 *                      chunked GEMV runs, which gives the same bits.
 *   QG_KERNEL_XR       the x-resident matrix-core GEMV (3 rows of x up to
 *                      the threshold); without it the FMA or streamed
 *                      matrix-core GEMV runs.
 *   QG_KERNEL_MMA      the streamed matrix-core GEMV for affine codes (2 rows
 *                      of x up to the threshold); without it the FMA GEMV.
 *   QG_EINVAL for other bits.
 */
enum { QG_KERNEL_KSLICED = 1, QG_KERNEL_XR = 2, QG_KERNEL_MMA = 4 };
qg_status qg_set_mfma_min_m(int64_t m);
int64_t qg_get_mfma_min_m(void);
qg_status qg_set_kernel_mask(uint32_t mask);
uint32_t qg_get_kernel_mask(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_Q4_H */
