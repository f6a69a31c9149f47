/*
 * mxfp8.h - C ABI of the MI355X (gfx950) MXFP8 library.
 *
 * Six operations, each one or two HIP kernels, all asynchronous on the
 * caller's stream:
 *   mxfp8_quantize        BF16 [rows,k] -> E4M3 [rows,k] + UE8M0 scales (one per 32 along k)
 *   rmsnorm_quant_mxfp8   Gemma RMSNorm fused with the same quantisation
 *   add_rmsnorm_quant_mxfp8  the same after a residual add (residual stream updated in place)
 *   mxfp8_swizzle_scales  linear scales -> 128x4 swizzled scales (after a gather)
 *   mxfp8_gemm_bf16out    C[m,n] = sum_k A[m,k] B[n,k] with per-32-K block scales, BF16 out,
 *                         written in M-row chunks (one chunk = one rank's reduce-scatter shard)
 *   mxfp8_gemm_silu_mul_quant  the dense MLP's gate_up GEMM with SiLU(gate) * up and the MXFP8
 *                         quantisation fused: MXFP8 in, MXFP8 (E4M3 + UE8M0) out
 *
 * Formats (vLLM PR #64659 "Details: GEMM-RS with a quantized input"; PR #65496 "Details"):
 *   E4M3  OCP OFP8 "FN": bias 7, max 448, no infinities, S.1111.111 NaN.
 *   UE8M0 OCP MX E8M0 biased exponent: value 2^(code-127).
 *   Block scale of 32 elements: the smallest 2^e with amax <= 448 * 2^e
 *   (e in [-127,127]; an all-zero block gets code 0); codes are E4M3(x * 2^-e),
 *   round to nearest even.
 *
 * Scale layouts:
 *   MXFP8_SCALES_LINEAR          row-major [rows, k/32] bytes.
 *   MXFP8_SCALES_SWIZZLED_128X4  the "F8_128x4" layout of PR #64659 ("Details"): 128 rows x
 *                                4 K-blocks form a 512-byte tile, tiles row-tile major,
 *                                inside a tile (r%32)*16 + ((r%128)/32)*4 + (c%4); rows padded
 *                                to a multiple of 128 and blocks to a multiple of 4, pad bytes 0.
 *                                PR #65496 ("Tradeoff") notes these scales cannot be concatenated
 *                                by rows, so the quantisers can emit both layouts in one pass.
 *
 * Ownership and threading: the caller owns every buffer (device memory unless
 * stated). The library allocates nothing, keeps no state between calls beyond a
 * per-device cache of the compute-unit count, and is safe to call from several
 * host threads. Every call validates its arguments on
 * the host first and returns a negative status without touching the GPU if they
 * are invalid; on success the work is enqueued on `stream` (0 = null stream) and
 * MXFP8_OK is returned. A failed launch returns MXFP8_EHIP. The library never
 * aborts the process.
 */
#ifndef MXFP8_H
#define MXFP8_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXFP8_OK = 0,
  MXFP8_EINVAL = -1,       /* a size, pointer, layout or chunk argument is invalid */
  MXFP8_EALIGN = -2,       /* a pointer or row stride breaks the alignment rule of the call */
  MXFP8_EUNSUPPORTED = -3, /* valid for the format but outside what the kernels handle */
  MXFP8_EHIP = -4          /* the HIP runtime rejected a launch */
} mxfp8_status;

typedef enum {
  MXFP8_SCALES_LINEAR = 0,
  MXFP8_SCALES_SWIZZLED_128X4 = 1
} mxfp8_scale_layout;

/* Bytes of a scale buffer for a [rows, k] operand in `layout`; -1 if the arguments are
 * invalid (rows < 0, k <= 0, k % 32 != 0, unknown layout). Host-only, no HIP call. */
int64_t mxfp8_scale_bytes(int64_t rows, int64_t k, int layout);

/* Static text for a status code. Host-only. */
const char* mxfp8_status_string(int status);

/*
 * mxfp8_quantize - BF16 -> MXFP8, the activation quantisation that GemmRsAr.apply()
 * performs on a BF16 input and skips for a QuantizedActivation (PR #64659, "Details:
 * GEMM-RS with a quantized input"); also the qkv_proj quantisation after the
 * all-gather (PR #65496, "Overview").
 *
 *   x_bf16          [rows, k] BF16, row stride ldx elements. 16-byte aligned, ldx % 8 == 0.
 *   rows >= 0, k > 0 with k % 32 == 0, ldx >= k.
 *   q_e4m3          [rows, k] E4M3 bytes, dense (row stride k). 8-byte aligned.
 *   scales_linear   [rows, k/32] UE8M0, or NULL.
 *   scales_swizzled mxfp8_scale_bytes(rows, k, MXFP8_SCALES_SWIZZLED_128X4) bytes, or NULL.
 *                   Pad bytes are written as 0.
 *   At least one scale pointer must be non-NULL. rows == 0 is a no-op (pointers may be NULL).
 * Non-finite inputs are outside the contract (their codes and scales are unspecified).
 */
int mxfp8_quantize(const void* x_bf16, int64_t rows, int64_t k, int64_t ldx, void* q_e4m3,
                   void* scales_linear, void* scales_swizzled, hipStream_t stream);

/* Host-side argument check of mxfp8_quantize (same rules, no HIP call). */
int mxfp8_quantize_check(const void* x_bf16, int64_t rows, int64_t k, int64_t ldx, const void* q_e4m3,
                         const void* scales_linear, const void* scales_swizzled);

/*
 * rmsnorm_quant_mxfp8 - Gemma-style RMSNorm y = x / sqrt(mean(x^2) + eps) * (1 + w),
 * quantised to MXFP8 in the same pass: the norm that returns a QuantizedActivation
 * for qkv_proj (PR #65496, "Details") and the "Gemma norm + MXFP8 quant" fusion of
 * PR #64111 ("Claims", decode kernels), without the all-reduce.
 * y is formed in fp64 from the BF16 inputs and rounded once to fp32; the scale and
 * code decisions are taken on that fp32 value.
 *
 *   x_bf16          [rows, hidden] BF16, row stride ldx. 16-byte aligned, ldx % 8 == 0.
 *   w_bf16          [hidden] BF16. 16-byte aligned.
 *   rows >= 0, hidden > 0 with hidden % 32 == 0 and hidden <= 16384, ldx >= hidden.
 *   eps             added to mean(x^2) (taken as fp32, used in fp64).
 *   q_e4m3          [rows, hidden] dense E4M3. 8-byte aligned.
 *   scales_linear / scales_swizzled as for mxfp8_quantize (at least one non-NULL).
 *   rows == 0 is a no-op (pointers may be NULL).
 */
int rmsnorm_quant_mxfp8(const void* x_bf16, const void* w_bf16, int64_t rows, int64_t hidden,
                        int64_t ldx, float eps, void* q_e4m3, void* scales_linear,
                        void* scales_swizzled, hipStream_t stream);

/* Host-side argument check of rmsnorm_quant_mxfp8 (same rules, no HIP call). */
int rmsnorm_quant_mxfp8_check(const void* x_bf16, const void* w_bf16, int64_t rows, int64_t hidden,
                              int64_t ldx, const void* q_e4m3, const void* scales_linear,
                              const void* scales_swizzled);

/*
 * add_rmsnorm_quant_mxfp8 - the residual add in front of the Gemma RMSNorm quantiser: the
 * decode fusion of PR #64111 ("Claims": all-reduce + Gemma norm + MXFP8 quant) without the
 * all-reduce, whose output is x here.
 *   h = BF16(x + residual)   (exact sum rounded once to nearest even), written back to residual;
 *   then exactly rmsnorm_quant_mxfp8 applied to h.
 *
 *   x_bf16          [rows, hidden] BF16, row stride ldx (as for rmsnorm_quant_mxfp8).
 *   residual_bf16   [rows, hidden] BF16, row stride ldr (ldr >= hidden, ldr % 8 == 0), 16-byte
 *                   aligned; read and overwritten with h. Must not overlap x.
 *   w_bf16, eps, q_e4m3, scales_linear, scales_swizzled, hidden limits: as for rmsnorm_quant_mxfp8.
 *   rows == 0 is a no-op (pointers may be NULL).
 */
int add_rmsnorm_quant_mxfp8(const void* x_bf16, void* residual_bf16, const void* w_bf16, int64_t rows,
                            int64_t hidden, int64_t ldx, int64_t ldr, float eps, void* q_e4m3,
                            void* scales_linear, void* scales_swizzled, hipStream_t stream);

/* Host-side argument check of add_rmsnorm_quant_mxfp8 (same rules, no HIP call). */
int add_rmsnorm_quant_mxfp8_check(const void* x_bf16, const void* residual_bf16, const void* w_bf16,
                                  int64_t rows, int64_t hidden, int64_t ldx, int64_t ldr,
                                  const void* q_e4m3, const void* scales_linear,
                                  const void* scales_swizzled);

/*
 * mxfp8_swizzle_scales - linear UE8M0 scales -> the 128x4 swizzled layout, the step after an
 * all-gather of MXFP8 activations: swizzled scales cannot be concatenated by rows (PR #65496,
 * "Tradeoff"), so the norm emits linear scales, ranks gather codes and linear scales (half the
 * bytes of a BF16 gather), and the gathered scales are swizzled once before the GEMM.
 *
 *   scales_linear   [rows, k/32] UE8M0 bytes, row-major, any alignment.
 *   rows >= 0, k > 0 with k % 32 == 0 (k is the element count per row; k/32 blocks).
 *   scales_swizzled mxfp8_scale_bytes(rows, k, MXFP8_SCALES_SWIZZLED_128X4) bytes, 16-byte aligned;
 *                   every byte is written (pad bytes 0). Must not overlap scales_linear.
 *   rows == 0 is a no-op (pointers may be NULL).
 */
int mxfp8_swizzle_scales(const void* scales_linear, int64_t rows, int64_t k, void* scales_swizzled,
                         hipStream_t stream);

/* Host-side argument check of mxfp8_swizzle_scales (same rules, no HIP call). */
int mxfp8_swizzle_scales_check(const void* scales_linear, int64_t rows, int64_t k,
                               const void* scales_swizzled);

/*
 * mxfp8_gemm_bf16out - the per-rank MXFP8 GEMM of the o_proj / down_proj GEMM-RS
 * path (PR #64659, "GEMM-RS microbenchmark": N = 6144, K = 2048 or 3072 per rank):
 *   C[m,n] = BF16( sum_kb 2^(sa[m,kb]-127) * 2^(sb[n,kb]-127) * sum_{i<32} A[m,32kb+i] * B[n,32kb+i] )
 * accumulated in fp32 on the scaled MFMA units, rounded to BF16 (nearest even).
 *
 *   a_e4m3   [m, k] E4M3, dense (row stride k). 16-byte aligned.
 *   a_scales scales of A in a_scale_layout (mxfp8_scale_bytes(m, k, layout) bytes). 4-byte aligned.
 *   b_e4m3   [n, k] E4M3, dense: the nn.Linear weight layout (K contiguous). 16-byte aligned.
 *   b_scales scales of B in b_scale_layout. 4-byte aligned.
 *   m, n >= 1; k > 0 with k % 32 == 0 (else MXFP8_EINVAL) and k % 128 == 0
 *   (else MXFP8_EUNSUPPORTED).
 *   Accuracy: the scaled MFMA aligns each group of 8 consecutive K products to the largest
 *   and truncates 13 bits below its leading one, then sums the groups in fp32, so the error
 *   of an output is bounded by its dot product's absolute mass, not by its value. For
 *   k >= 256 the outputs of N(0,1)-like data stay within 2e-2 relative of the exactly
 *   rounded BF16 result; with k == 128 (one 128-K step) the short sums let the truncation
 *   reach about 3e-2 on outputs that cancel, so that bar is not promised there.
 *   c_bf16   [m, ldc] BF16, ldc >= n, ldc % 4 == 0, 8-byte aligned. Only columns < n are written.
 *   num_chunks >= 1 with m % num_chunks == 0: C is produced as num_chunks contiguous
 *   row chunks of m/num_chunks rows (PR #64659 "Overview"/"Details": the reduce-scatter
 *   shard of one TP rank). Output tiles never straddle a chunk, and the tiles are
 *   dispatched chunk by chunk starting at first_chunk (0 <= first_chunk < num_chunks)
 *   and wrapping around, so chunk first_chunk completes first.
 *   chunk_done NULL, or a device int array [num_chunks] that the caller zeroes before the
 *   call: after every output tile of chunk c has been stored and made visible device-wide,
 *   chunk_done[c] is incremented once per tile; the chunk is complete when it reaches
 *   mxfp8_gemm_tiles_per_chunk(m, n, num_chunks, a_scale_layout, b_scale_layout). This is
 *   the hook a reduce-scatter
 *   would wait on.
 * The result does not depend on num_chunks, first_chunk or chunk_done.
 * Performance: large problems run fastest with both scale buffers in the swizzled layout,
 * 16-byte aligned, and m/num_chunks a multiple of 64 (the output is the same bits either way).
 */
int mxfp8_gemm_bf16out(const void* a_e4m3, const void* a_scales, int a_scale_layout,
                       const void* b_e4m3, const void* b_scales, int b_scale_layout, int64_t m,
                       int64_t n, int64_t k, void* c_bf16, int64_t ldc, int num_chunks,
                       int first_chunk, int* chunk_done, hipStream_t stream);

/* Host-side argument check of mxfp8_gemm_bf16out (same rules, no HIP call). */
int mxfp8_gemm_bf16out_check(const void* a_e4m3, const void* a_scales, int a_scale_layout,
                             const void* b_e4m3, const void* b_scales, int b_scale_layout,
                             int64_t m, int64_t n, int64_t k, const void* c_bf16, int64_t ldc,
                             int num_chunks, int first_chunk);

/*
 * mxfp8_gemm_silu_mul_quant - the fused dense GEMM1: the gate_up projection, SiLU(gate) * up and
 * the MXFP8 quantisation of the result in one kernel, so down_proj receives an MXFP8 activation
 * with swizzled scales instead of a BF16 tensor it would quantise itself (PR #64659, "Details":
 * the dense MLP keeps its fused GEMM1, and "GEMM-RS with a quantized input"; PR #64111, "Claims":
 * SM100 fused dense GEMM1).
 *   g[m,j] = C[m,j], u[m,j] = C[m,inter+j] with C as for mxfp8_gemm_bf16out (fp32 accumulation),
 *   y[m,j] = g / (1 + e^-g) * u in fp32 from the accumulators (no BF16 rounding in between),
 *   y quantised per 32 along j exactly as mxfp8_quantize does with an fp32 input.
 *
 *   a_e4m3 / a_scales  [m, k] E4M3 (dense, 16-byte aligned), scales in a_scale_layout (4-byte aligned).
 *   w_e4m3 / w_scales  [2*inter, k] E4M3: rows [0, inter) the gate projection, rows [inter, 2*inter)
 *                      the up projection (the merged gate_up weight); scales in w_scale_layout.
 *   m >= 1; inter >= 32 with inter % 32 == 0; k > 0 with k % 32 == 0 (else MXFP8_EINVAL) and
 *   k % 128 == 0 (else MXFP8_EUNSUPPORTED).
 *   q_e4m3          [m, inter] E4M3, dense, 16-byte aligned.
 *   scales_linear   [m, inter/32] or NULL; scales_swizzled mxfp8_scale_bytes(m, inter, SWIZZLED)
 *                   bytes or NULL (pad bytes written 0); at least one non-NULL.
 * Results do not depend on the tile configuration the library picks.
 */
int mxfp8_gemm_silu_mul_quant(const void* a_e4m3, const void* a_scales, int a_scale_layout,
                              const void* w_e4m3, const void* w_scales, int w_scale_layout, int64_t m,
                              int64_t inter, int64_t k, void* q_e4m3, void* scales_linear,
                              void* scales_swizzled, hipStream_t stream);

/* Host-side argument check of mxfp8_gemm_silu_mul_quant (same rules, no HIP call). */
int mxfp8_gemm_silu_mul_quant_check(const void* a_e4m3, const void* a_scales, int a_scale_layout,
                                    const void* w_e4m3, const void* w_scales, int w_scale_layout,
                                    int64_t m, int64_t inter, int64_t k, const void* q_e4m3,
                                    const void* scales_linear, const void* scales_swizzled);

/* Output tiles per chunk that mxfp8_gemm_bf16out uses for this shape and these scale layouts
 * (the final value of each chunk_done counter): the tile shape follows m, n, num_chunks and
 * whether both scale buffers are swizzled (MXFP8_SCALES_SWIZZLED_128X4), not the buffers'
 * addresses.
 * -1 for invalid arguments. Host-only. */
int64_t mxfp8_gemm_tiles_per_chunk(int64_t m, int64_t n, int num_chunks, int a_scale_layout,
                                   int b_scale_layout);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8_H */
