/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 quantization library.
 *
 * NVFP4 stores a tensor as 4-bit E2M1 codes (two per byte), one FP8 E4M3
 * scale per block of 16 elements (1D) or per 16x16 tile (2D), and one FP32
 * scale for the whole tensor; an element reconstructs as
 *     x = e2m1(code) * e4m3(block scale) * global scale
 * (page "NVFP4 Is a Scaling System, Not Just a 4-Bit Number", section "The
 * smallest example"; page "Melatih model dalam 4 bit: pengaman numerik di
 * balik NVFP4", section "Anatomi NVFP4").
 *
 * Conventions shared by every call:
 *  - Tensors are row-major [rows][cols] with cols contiguous. bf16 inputs
 *    are passed as their 16-bit patterns.
 *  - All pointers are DEVICE pointers (hipMalloc / torch CUDA tensors)
 *    owned by the caller. The library allocates nothing and is safe to
 *    call from several host threads. Between calls it keeps only facts
 *    about the device (how many workgroups of a kernel fit at once, looked
 *    up on first use per device); results never depend on earlier calls.
 *  - Every call is asynchronous on `stream` (0 = the null stream) and never
 *    synchronises the host. Outputs are valid once the stream reaches them.
 *  - Arguments are validated before any HIP call; a failed check returns a
 *    negative status and launches nothing. Device pointers must be 16-byte
 *    aligned.
 *  - Packed codes: element 2k of a row of the output layout is the low
 *    nibble of byte k, element 2k+1 the high nibble; a nibble is
 *    (sign << 3) | magnitude code, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 *  - Scale layouts are compact row-major, no padding: 1D rowwise
 *    [rows][cols/16], 1D columnwise [cols][rows/16], 2D [rows/16][cols/16].
 *  - Non-finite inputs are not an error: the amax becomes Inf or NaN and
 *    the outputs are well defined but meaningless.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define NVFP4_OK 0
#define NVFP4_ERR_NULL (-1)  /* a required pointer is NULL                  */
#define NVFP4_ERR_SHAPE (-2) /* a dimension is not positive / not a multiple */
                             /* of 16 (or of the call's stated granule)      */
#define NVFP4_ERR_ALIGN (-3) /* a pointer is not 16-byte aligned             */
#define NVFP4_ERR_FLAGS (-4) /* unknown flag, mode or unsupported combination */
#define NVFP4_ERR_HIP (-5)   /* the HIP runtime refused a launch             */
#define NVFP4_ERR_SIZE (-6)  /* a size exceeds the supported index range     */

/* ---- flags ----------------------------------------------------------- */
#define NVFP4_ROWWISE 0x1u /* blocks of 16 consecutive elements along cols  */
#define NVFP4_COLWISE 0x2u /* blocks of 16 consecutive rows of one column   */
#define NVFP4_SR 0x4u      /* stochastic rounding (gradients) instead of RNE */
#define NVFP4_RHT 0x8u     /* random-sign 16-point Hadamard along rows first */
#define NVFP4_AMAX_BOTH 0x20u  /* nvfp4_amax with NVFP4_RHT: plain amax too    */

/* Size of the workspace nvfp4_quantize_1d_fused takes. */
#define NVFP4_WORKSPACE_BYTES 32832

/* scale_mode values */
#define NVFP4_SCALE_1D 1 /* one scale per 16 consecutive elements of a row */
#define NVFP4_SCALE_2D 2 /* one scale per 16x16 tile                       */
#define NVFP4_SCALE_2D_T 3 /* 16x16 tile scales of the transposed operand:  */
                           /* row n, K block j at [j][n/16] (GEMM only)     */

/* dtype values */
#define NVFP4_F32 0
#define NVFP4_BF16 1

/* Human-readable text for a status code (static storage; never NULL). */
const char* nvfp4_status_string(int status);

/*
 * nvfp4_amax -- tensor-wide maximum absolute value (page "Melatih model
 * dalam 4 bit", section "Anatomi NVFP4": the global scale is derived from
 * the tensor amax; page "NVFP4 Is a Scaling System", section "The smallest
 * example").
 *   x        bf16 [rows][cols]
 *   flags    0, or NVFP4_RHT: the amax of the Hadamard-transformed tensor
 *            (16-row segments of every column, sign mask `rht_mask`), i.e.
 *            of what nvfp4_rht16(axis 0) would produce; or
 *            NVFP4_RHT | NVFP4_AMAX_BOTH: both amaxes from one read of x
 *            (a gradient needs the plain one for its rowwise dgrad operand
 *            and the transformed one for its columnwise wgrad operand).
 *   amax     one float (two with NVFP4_AMAX_BOTH: [0] plain, [1] of the
 *            transform), written with the result (the call first resets
 *            it, stream-ordered, then reduces into it).
 * Shapes: rows, cols >= 1; with NVFP4_RHT rows must be a multiple of 16.
 * The maximum is an integer maximum of |x| bit patterns, so it is exact and
 * independent of launch geometry; a NaN input yields a NaN amax.
 */
int nvfp4_amax(const uint16_t* x, int64_t rows, int64_t cols, uint32_t flags, uint16_t rht_mask,
               float* amax, hipStream_t stream);

/*
 * nvfp4_quantize_1d -- NVFP4 quantization with 16-element blocks
 * (activations and gradients; page "NVFP4 Is a Scaling System", section "A
 * format is not a training recipe").
 *   x          bf16 [rows][cols]; rows and cols multiples of 16.
 *   amax       device float from nvfp4_amax of the same tensor (with the
 *              same NVFP4_RHT flag and mask when NVFP4_RHT is set).
 *   flags      NVFP4_ROWWISE and/or NVFP4_COLWISE (at least one), plus
 *              NVFP4_SR (stochastic rounding, page "MXFP4 和 NVFP4 的区别",
 *              section "随机舍入") and/or NVFP4_RHT (page "Melatih model
 *              dalam 4 bit", section "Empat pengaman": the transform is
 *              applied to the column-quantized wgrad operands, so
 *              NVFP4_RHT requires NVFP4_COLWISE and excludes NVFP4_ROWWISE).
 *   rht_mask   bit j set = negate element j of every 16-row segment before
 *              the transform (ignored without NVFP4_RHT).
 *   seed       stochastic-rounding key; the draw of element (r, c) is a
 *              pure function of (seed, r*cols + c) (Philox4x32-10, one call
 *              per 8 consecutive flat indices, 16 bits per element), so
 *              both layouts and any launch geometry see the same draws.
 *   codes_row  [rows][cols/2]  (NULL unless ROWWISE)
 *   scales_row [rows][cols/16] (NULL unless ROWWISE)
 *   codes_col  [cols][rows/2]  (NULL unless COLWISE)
 *   scales_col [cols][rows/16] (NULL unless COLWISE)
 *   global_scale  optional (may be NULL): receives S_g = amax / 2688.
 * Per block: s = e4m3_rne(b / (6*S_g)) with b the block's max |x| (after
 * the transform with NVFP4_RHT); each element is |x| * (1 / (s*S_g))
 * rounded to E2M1 (ties to even, saturating at 6) or stochastically.
 */
int nvfp4_quantize_1d(const uint16_t* x, int64_t rows, int64_t cols, const float* amax,
                      uint32_t flags, uint16_t rht_mask, uint64_t seed, uint8_t* codes_row,
                      uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                      float* global_scale, hipStream_t stream);

/*
 * nvfp4_quantize_1d_fused -- nvfp4_quantize_1d that finds the tensor amax
 * itself (page "Melatih model dalam 4 bit", section "Anatomi NVFP4": the
 * global scale comes from the tensor amax), in the same pass over x when
 * the tensor fits on chip: the data stays in registers between the amax and
 * the encoding, so x is read from memory once. Larger tensors take two
 * passes (amax, then quantize) inside the same call.
 *   flags      NVFP4_ROWWISE and/or NVFP4_COLWISE, optionally NVFP4_SR (no
 *              NVFP4_RHT: the transformed operand's amax is nvfp4_amax's).
 *   workspace  caller-owned device memory of NVFP4_WORKSPACE_BYTES bytes,
 *              16-byte aligned, zero-filled before its first use and then
 *              reused as is (each call leaves it ready for the next). Its
 *              first float receives the amax (what nvfp4_amax would give).
 *   Other arguments and the outputs as nvfp4_quantize_1d.
 * The single pass needs all of its workgroups on the device at once; if
 * they are not (another kernel holds the device), a bounded wait expires,
 * the amax is computed from x directly (same result, slower) and 32-bit
 * word 2 of the workspace is incremented. Word 3 sets that wait in ticks of
 * the 100 MHz real-time counter (0, as after zero-filling: 2 ms; a tiny
 * value forces the direct computation, for tests). Calls that overlap in
 * time must use different workspaces.
 */
int nvfp4_quantize_1d_fused(const uint16_t* x, int64_t rows, int64_t cols, uint32_t flags,
                            uint64_t seed, void* workspace, uint8_t* codes_row,
                            uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                            float* global_scale, hipStream_t stream);

/*
 * nvfp4_quantize_1d_fused_noalloc -- for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): nvfp4_quantize_1d_fused without the
 * workspace argument. Its exchange runs in the library's own workspace, a
 * static device array of NVFP4_WORKSPACE_BYTES (32,832 bytes) per GPU,
 * held until the process ends. The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); its first call on a device looks
 * up that device's copy of the array.
 *   amax   optional device float (4-byte aligned, may be NULL) that
 *          receives the amax; the global scale goes to global_scale as in
 *          nvfp4_quantize_1d.
 *   Other arguments, validation and outputs as nvfp4_quantize_1d_fused;
 *   results are bit-identical to it.
 * Size limit: none beyond nvfp4_quantize_1d_fused's. The workspace holds
 * the exchange slots of the largest single pass (1024 workgroups); larger
 * tensors take the two-pass path, which needs no slots.
 * Every such call on one GPU shares the array: calls that overlap in time
 * on one device (different streams, or host threads without ordering)
 * race and give wrong results; order them on one stream. Each call leaves
 * the array ready for the next, so nothing needs clearing.
 */
int nvfp4_quantize_1d_fused_noalloc(const uint16_t* x, int64_t rows, int64_t cols, uint32_t flags,
                                    uint64_t seed, uint8_t* codes_row, uint8_t* scales_row,
                                    uint8_t* codes_col, uint8_t* scales_col, float* global_scale,
                                    float* amax, hipStream_t stream);

/*
 * nvfp4_quantize_2d -- weight quantization with one E4M3 scale per 16x16
 * tile, emitted in both layouts with identical codes (page "Melatih model
 * dalam 4 bit", section "Empat pengaman", second safeguard: rowwise and
 * columnwise quantized weights are numerically the same). Round to
 * nearest even only.
 *   x          bf16 [rows][cols]; rows and cols multiples of 16.
 *   amax       device float from nvfp4_amax(x, flags 0).
 *   codes_row  [rows][cols/2] or NULL;  codes_col [cols][rows/2] or NULL
 *              (at least one non-NULL).
 *   scales     [rows/16][cols/16] (required).
 *   global_scale  optional (may be NULL).
 */
int nvfp4_quantize_2d(const uint16_t* x, int64_t rows, int64_t cols, const float* amax,
                      uint8_t* codes_row, uint8_t* codes_col, uint8_t* scales,
                      float* global_scale, hipStream_t stream);

/*
 * nvfp4_quantize_2d_tscales -- nvfp4_quantize_2d that also writes the tile
 * scales transposed: scales_t [cols/16][rows/16], scales_t[j][i] =
 * scales[i][j], in the same pass. With it, the columnwise copy codes_col
 * ([cols][rows/2]) is a plain 2D-scaled GEMM operand (NVFP4_SCALE_2D with
 * scales_t) whose scale reads are contiguous per row, where
 * NVFP4_SCALE_2D_T on the untransposed grid reads bytes a scale row apart
 * (page "Melatih model dalam 4 bit", section "Empat pengaman": the dgrad
 * GEMM reads the weight's columnwise copy). scales_t: device, any
 * alignment, required. Everything else as nvfp4_quantize_2d.
 */
int nvfp4_quantize_2d_tscales(const uint16_t* x, int64_t rows, int64_t cols, const float* amax,
                              uint8_t* codes_row, uint8_t* codes_col, uint8_t* scales,
                              uint8_t* scales_t, float* global_scale, hipStream_t stream);

/*
 * nvfp4_rht16 -- standalone random-sign 16-point Hadamard transform
 * y = (1/4) * H16 * D * x on every 16-element segment along `axis`
 * (0: 16 consecutive rows of a column; 1: 16 consecutive elements of a
 * row). H16 is the natural-order Sylvester matrix (page "MXFP4 和 NVFP4
 * 的区别", sections "随机 Hadamard 变换" and "构造 Hadamard 矩阵的方法"),
 * evaluated as the add/subtract butterfly in binary32; D negates element j
 * when bit j of rht_mask is set.
 *   x  bf16 [rows][cols];  y  float [rows][cols].
 * The extent along `axis` must be a multiple of 16; the other >= 1 (cols a
 * multiple of 8 for axis 0).
 */
int nvfp4_rht16(const uint16_t* x, int64_t rows, int64_t cols, int axis, uint16_t rht_mask,
                float* y, hipStream_t stream);

/*
 * nvfp4_dequantize -- x = e2m1(code) * e4m3(scale) * S_g (page "NVFP4 Is a
 * Scaling System", section "The smallest example"), in binary32:
 * fl(fl(e2m1*scale) * S_g) (the inner product is exact), converted to bf16
 * by round-to-nearest-even when out_dtype is NVFP4_BF16. Any scale byte is
 * accepted: a set sign bit negates the scale, and the E4M3 NaN bytes (0x7F,
 * 0xFF) give NaN carrying the code's sign.
 *   codes         [rows][cols/2] packed codes of one layout
 *   scales        [rows][cols/16] (NVFP4_SCALE_1D) or [rows/16][cols/16]
 *                 (NVFP4_SCALE_2D)
 *   global_scale  device float S_g
 *   out           [rows][cols] of out_dtype
 * rows and cols multiples of 16.
 */
int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int scale_mode,
                     const float* global_scale, int64_t rows, int64_t cols, void* out,
                     int out_dtype, hipStream_t stream);

/*
 * nvfp4_gemm -- C = A * B^T from packed NVFP4 operands (TN layout: both
 * operands are K-contiguous, as the NVFP4 GEMM takes them; page "NVFP4 Is a
 * Scaling System", section "“4-bit” is a payload count"): every operand
 * element is decoded exactly (e2m1 * e4m3 has at most 6 significant bits
 * and lies in [2^-10, 2688], so it is an fp16 value), products are summed
 * in fp32 on the matrix cores, and the sum is multiplied by
 * fl(S_gA * S_gB). The summation order differs from a sequential sum, so
 * results match an exact product to fp32 rounding, not bit for bit. Each
 * element is accumulated in one fixed order (K ascending, 16 products at a
 * time) whatever M, N and the work split, so a given element of C is
 * reproducible bit for bit across calls and shapes.
 *   a_codes [M][K/2], a_scales per a_scale_mode over [M][K]
 *   b_codes [N][K/2], b_scales per b_scale_mode over [N][K]
 *   Scale modes: NVFP4_SCALE_1D [rows][K/16]; NVFP4_SCALE_2D [rows/16][K/16];
 *   NVFP4_SCALE_2D_T [K/16][rows/16], the tile scales that
 *   nvfp4_quantize_2d writes for the tensor whose column layout is the
 *   operand (a weight's dgrad copy: its codes_col with its scales).
 *   a_global_scale, b_global_scale: device floats
 *   c       [M][N] of c_dtype (fp32 or bf16, round-to-nearest-even)
 * M, N, K multiples of 16.
 */
int nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int a_scale_mode,
               const float* a_global_scale, const uint8_t* b_codes, const uint8_t* b_scales,
               int b_scale_mode, const float* b_global_scale, void* c, int c_dtype, int64_t M,
               int64_t N, int64_t K, hipStream_t stream);

/*
 * nvfp4_gemm_amax -- nvfp4_gemm whose epilogue also reduces the tensor amax
 * of the output it stores: *c_amax = max |C| over the stored values (for a
 * bf16 C, of the bf16 values; the integer maximum of their magnitude bit
 * patterns, so it equals what nvfp4_amax of C returns, NaN included). A
 * following NVFP4 quantization of C (the next layer's input) can take it as
 * its amax and read C once instead of twice: the amax pass is fused into
 * the producer's epilogue. The call resets *c_amax (stream-ordered) before
 * the GEMM. c_amax: one device float, 4-byte aligned. Other arguments,
 * validation and results as nvfp4_gemm.
 */
int nvfp4_gemm_amax(const uint8_t* a_codes, const uint8_t* a_scales, int a_scale_mode,
                    const float* a_global_scale, const uint8_t* b_codes, const uint8_t* b_scales,
                    int b_scale_mode, const float* b_global_scale, void* c, int c_dtype, int64_t M,
                    int64_t N, int64_t K, float* c_amax, hipStream_t stream);

/*
 * nvfp4_gemm_quantize -- nvfp4_gemm whose epilogue quantizes the product
 * instead of storing it: the output that a following NVFP4 quantization of
 * the layer's output would write, produced by the GEMM that makes that
 * output (the quantization fused into the producer's epilogue; in the
 * pages' recipe the inputs of the MLP's three GEMMs are NVFP4, page
 * "Melatih model dalam 4 bit", section "Empat pengaman yang membuat 4 bit
 * bisa konvergen"). C is never written to memory.
 * The result equals, byte for byte,
 *   nvfp4_gemm(..., Y, NVFP4_BF16, ...) followed by
 *   nvfp4_quantize_1d(Y, M, N, y_amax, flags, 0, 0, codes_row, scales_row,
 *                     codes_col, scales_col, global_scale):
 * the bf16 product (each element rounded to nearest even after the
 * fl(S_gA * S_gB) multiply) quantized with round-to-nearest-even E2M1 codes
 * and the global scale S_g derived from *y_amax.
 * The tensor amax must be known before the first tile is quantized, so the
 * caller supplies it: for instance the amax this call reported for the same
 * layer's previous product (c_amax below), or any bound on max |Y|. Blocks
 * whose maximum exceeds it saturate exactly as nvfp4_quantize_1d's do.
 *   y_amax   device float: the amax the quantization takes
 *   flags    NVFP4_ROWWISE and/or NVFP4_COLWISE (no stochastic rounding,
 *            no transform)
 *   codes_row [M][N/2], scales_row [M][N/16], codes_col [N][M/2],
 *   scales_col [N][M/16] for the layouts flags selects (16-byte aligned)
 *   global_scale  optional device float: receives S_g
 *   c_amax   optional device float (4-byte aligned): receives max |Y| of
 *            this product (as nvfp4_gemm_amax with a bf16 C reports it),
 *            reset stream-ordered before the GEMM
 * A, B, their scales and global scales, M, N, K: as nvfp4_gemm (M, N, K
 * multiples of 16).
 */
int nvfp4_gemm_quantize(const uint8_t* a_codes, const uint8_t* a_scales, int a_scale_mode,
                        const float* a_global_scale, const uint8_t* b_codes, const uint8_t* b_scales,
                        int b_scale_mode, const float* b_global_scale, int64_t M, int64_t N,
                        int64_t K, const float* y_amax, uint32_t flags, uint8_t* codes_row,
                        uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                        float* global_scale, float* c_amax, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
