/*
 * mxfp4.h -- C ABI of the library's MXFP4 comparator format.
 *
 * MXFP4 stores E2M1 codes like NVFP4 but shares one E8M0 scale (a power of
 * two, byte b = 2^(b-127), 0xFF = NaN) across 32 elements and has no
 * tensor-level scale (page "NVFP4 Is a Scaling System, Not Just a 4-Bit
 * Number", section "Generic FP4, MXFP4, and NVFP4"; page "MXFP4 和 NVFP4
 * 的区别", section "MXFP4:开放标准,但精度较粗"). It is the format the gfx950
 * matrix cores scale natively, and serves here to measure NVFP4 against.
 *
 * The scale of a block is the OCP microscaling shared exponent,
 * X = 2^(floor(log2 amax) - 2) (2 = E2M1's largest exponent), clamped to
 * E8M0's range (an all-zero block gets byte 0); a block holding a NaN or an
 * infinity gets byte 0xFF and codes of magnitude 0. Elements are x / X
 * rounded to E2M1, nearest even, saturating at 6; the sign bit is kept.
 *
 * Conventions are those of nvfp4.h (device pointers owned by the caller,
 * asynchronous on `stream`, validation before any launch, NVFP4_* status
 * codes, packed codes with element 2k in the low nibble of byte k) with
 * 32-element blocks: scales are compact row-major [rows][cols/32] for the
 * rowwise layout and [cols][rows/32] for the columnwise one.
 */
#ifndef MXFP4_H
#define MXFP4_H

#include "nvfp4.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * mxfp4_quantize -- MXFP4 codes and E8M0 scales of a bf16 tensor in one
 * pass over it (no amax pass: the format has no tensor scale).
 *   x          bf16 [rows][cols]; NVFP4_ROWWISE needs cols a multiple of 32,
 *              NVFP4_COLWISE rows a multiple of 32 and cols of 8.
 *   flags      NVFP4_ROWWISE and/or NVFP4_COLWISE (at least one); or
 *              NVFP4_COLWISE | NVFP4_RHT: columnwise blocks of the
 *              tensor transformed along its rows by the random-sign
 *              16-point Hadamard transform of nvfp4_rht16 (axis 0, mask
 *              `rht_mask`); each 32-row block is two transformed segments.
 *   codes_row  [rows][cols/2], scales_row [rows][cols/32] (ROWWISE)
 *   codes_col  [cols][rows/2], scales_col [cols][rows/32] (COLWISE)
 *   Unused layouts' pointers may be NULL.
 */
int mxfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint32_t flags,
                   uint16_t rht_mask, uint8_t* codes_row, uint8_t* scales_row,
                   uint8_t* codes_col, uint8_t* scales_col, hipStream_t stream);

/*
 * mxfp4_dequantize -- x = e2m1(code) * 2^(scale - 127) for a [rows][cols]
 * layout (codes [rows][cols/2], scales [rows][cols/32]); exact in binary32
 * and in bf16 for every scale byte below 253 (what mxfp4_quantize writes
 * for bf16 input), NaN for byte 0xFF.
 *   out  [rows][cols] of out_dtype (NVFP4_F32 or NVFP4_BF16)
 * rows >= 1, cols a multiple of 32.
 */
int mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                     void* out, int out_dtype, hipStream_t stream);

/*
 * mxfp4_gemm -- C = A * B^T from MXFP4 operands (TN: both K-contiguous) on
 * the gfx950 block-scaled matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4
 * with E2M1 operands and the E8M0 block scales applied by the
 * instruction), summed in fp32:
 *   C[m][n] = sum_k A^[m][k] B^[n][k],  A^ = e2m1 * 2^(scale - 127).
 * The summation order differs from a sequential sum, so results match the
 * exact product to fp32 rounding, not bit for bit.
 *   a_codes [M][K/2], a_scales [M][K/32]; b_codes [N][K/2], b_scales [N][K/32]
 *   c       [M][N] of c_dtype (fp32, or bf16 by round-to-nearest-even)
 * M, N >= 1 (below 2^23); K a multiple of 32, at most 2^24. Code and output
 * arrays 16-byte aligned.
 */
int mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
               const uint8_t* b_scales, void* c, int c_dtype, int64_t M, int64_t N, int64_t K,
               hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H */
