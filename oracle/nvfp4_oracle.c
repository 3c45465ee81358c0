/*
 * NVFP4 reference oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU implementation of the NVFP4 quantization path.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it; the product path (the HIP library) never does, and the two
 * share no code, header, table or constant generator.
 *
 * Build: gcc -O2 -fPIC -shared -ffp-contract=off (no fast-math), so every
 * float operation below is one IEEE-754 binary32 operation rounded to
 * nearest-even, with denormals preserved and no fused multiply-add.
 *
 * Sources (web pages; cited by title and section):
 *  [TE-ID]  "Melatih model dalam 4 bit: pengaman numerik di balik NVFP4"
 *           (iohtechco), sections "Anatomi NVFP4" and "Empat pengaman".
 *  [SCALE]  "NVFP4 Is a Scaling System, Not Just a 4-Bit Number"
 *           (nakranivaibhav), sections "Four bits do not provide many
 *           choices", "The smallest example", "A format is not a training
 *           recipe".
 *  [ZH]     "MXFP4 和 NVFP4 的区别" (blog.daoxuan.cc), sections
 *           "NVFP4 的计算过程", "随机舍入", "随机 Hadamard 变换",
 *           "构造 Hadamard 矩阵的方法", "为什么不用 Conference 矩阵".
 *  [FP4]    "how numbers are stored in computers" (number.rest, FP4 page).
 *  [PHILOX] Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
 *           1, 2, 3", SC'11 -- the Philox4x32-10 counter-based generator.
 *  [MX]     "NVFP4 Is a Scaling System, Not Just a 4-Bit Number", section
 *           "Generic FP4, MXFP4, and NVFP4" (MXFP4: E2M1 payload, one E8M0
 *           power-of-two scale per 32 values, no tensor scale); [ZH] section
 *           "MXFP4:开放标准,但精度较粗"; the shared-exponent rule of the OCP
 *           Microscaling Formats (MX) v1.0 specification, which the pages
 *           name as MXFP4's definition but do not spell out.
 *
 * Readings where the pages are silent:
 *  - global scale S_g = amax / (448*6) is the decode multiplier; encoding
 *    uses reciprocals of it;
 *  - block scale = E4M3 round-to-nearest-even (satfinite) of b / (6*S_g);
 *  - element ratio v = |x| * (1 / (s*S_g)), one reciprocal per block;
 *  - E2M1 ties go to the even code; values above 6 saturate to 6; a NaN
 *    ratio encodes magnitude 0; the sign bit is always copied;
 *  - stochastic rounding rounds up with probability (v-lo)/(hi-lo), drawing
 *    16 bits per element from Philox4x32-10 (one call per 8 elements);
 *  - the Hadamard transform is the natural-order Sylvester H16 applied by
 *    the butterfly in binary32, scaled by 1/4, after a 16-bit sign mask;
 *  - MXFP4 (the comparator format): the block scale is X = 2^(floor(log2
 *    amax) - 2), 2 being E2M1's largest exponent, clamped to E8M0's range
 *    2^-127..2^127 (an all-zero block gets 2^-127); a block holding a NaN
 *    or an infinity gets the E8M0 NaN byte 0xFF; elements are x / X
 *    rounded to E2M1 by the same rule as NVFP4's (so a NaN ratio has
 *    magnitude 0 and the sign bit is kept).
 *
 * Parity status: every function here is pinned by a CPU test
 * (tests/test_oracle_pins.py) except where a function's comment says
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* bf16 -> binary32 is exact: the bf16 bits are the top half of a float. */
static float bf16_bits_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* E2M1 magnitudes, in code order 0..7 ([SCALE] "Four bits do not provide
 * many choices": 0, 0.5, 1, 1.5, 2, 3, 4, 6; the sign bit mirrors them). */
static const double E2M1_MAGNITUDE[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double nvfp4_oracle_e2m1_decode(uint8_t code)
{
    double m = E2M1_MAGNITUDE[code & 7];
    return (code & 8) ? -m : m;
}

/* E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
 * subnormal; 0x7F / 0xFF are NaN; the largest finite value is 448 as
 * [TE-ID] "Anatomi NVFP4" states). Written out from the field layout. */
double nvfp4_oracle_e4m3_decode(uint8_t b)
{
    int sign = b >> 7;
    int e = (b >> 3) & 15;
    int m = b & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = m * ldexp(1.0, -9);
    else
        mag = (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return sign ? -mag : mag;
}

/* Round a non-negative binary32 value to the nearest finite E4M3 value;
 * ties go to the code with an even last bit; values at or above 448
 * saturate to 448 (0x7E); NaN gives 0x7F. Plain nearest search over the
 * 127 non-negative finite codes; distances are exact in double. */
uint8_t nvfp4_oracle_e4m3_encode(float v)
{
    if (isnan(v))
        return 0x7F;
    if (v >= 448.0f)
        return 0x7E;
    if (v <= 0.0f)
        return 0x00; /* +0, -0 (block maxima are never negative) */
    int best = 0;
    double best_d = fabs((double)v - 0.0);
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs((double)v - nvfp4_oracle_e4m3_decode((uint8_t)c));
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)best;
}

/* E2M1 round-to-nearest-even ([ZH] "随机舍入": weights and activations use
 * round-to-nearest-even). v is the element's scaled magnitude. Returns the
 * magnitude code 0..7: the nearest codebook value, ties to the even code,
 * values above 6 (and +inf) saturate to 6, NaN gives 0. */
int nvfp4_oracle_e2m1_rne(float v)
{
    if (isnan(v))
        return 0;
    if (v >= 6.0f)
        return 7;
    int best = 0;
    double best_d = fabs((double)v - E2M1_MAGNITUDE[0]);
    for (int k = 1; k < 8; ++k) {
        double d = fabs((double)v - E2M1_MAGNITUDE[k]);
        if (d < best_d || (d == best_d && (k & 1) == 0)) {
            best = k;
            best_d = d;
        }
    }
    return best;
}

/* E2M1 stochastic rounding ([ZH] "随机舍入"; [TE-ID] "Empat pengaman",
 * third safeguard; [SCALE] "A format is not a training recipe"): between
 * the two neighbouring codebook values lo <= v < hi, round up with
 * probability p = (v - lo) / (hi - lo), so the expectation equals v.
 * The uniform draw is u = h / 2^16 from a 16-bit integer h; round up iff
 * u < p. v >= 6 saturates to 6; NaN gives 0. binary32 arithmetic. */
int nvfp4_oracle_e2m1_sr(float v, uint16_t h)
{
    if (isnan(v))
        return 0;
    if (v >= 6.0f)
        return 7;
    int lo = 0;
    for (int k = 0; k < 8; ++k)
        if ((float)E2M1_MAGNITUDE[k] <= v)
            lo = k;
    float g_lo = (float)E2M1_MAGNITUDE[lo];
    float gap = (float)(E2M1_MAGNITUDE[lo + 1] - E2M1_MAGNITUDE[lo]);
    float p = (v - g_lo) / gap;
    float u = (float)h / 65536.0f;
    return lo + (u < p ? 1 : 0);
}

/* ------------------------------------------------------------------ */
/* Random draws: Philox4x32-10 [PHILOX]                                */
/* ------------------------------------------------------------------ */

/* Ten rounds of the Philox S-box on a 4x32-bit counter under a 2x32-bit
 * key; the key is bumped by the Weyl constants between rounds. Pinned by
 * tests against rocRAND's independent implementation. */
void nvfp4_oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* The 16-bit draw of the element whose row-major flat index in the input
 * tensor is i: counter (i/8 low, i/8 high, 0, 0), key (seed low, seed high);
 * word (i mod 8)/2 of the output, low half for even i, high half for odd. */
uint16_t nvfp4_oracle_sr_draw(uint64_t seed, uint64_t i)
{
    uint64_t call = i >> 3;
    uint32_t ctr[4] = {(uint32_t)call, (uint32_t)(call >> 32), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    nvfp4_oracle_philox4x32_10(ctr, key, w);
    uint32_t word = w[(i & 7) >> 1];
    return (uint16_t)((i & 1) ? (word >> 16) : (word & 0xFFFFu));
}

/* ------------------------------------------------------------------ */
/* Random Hadamard transform ([ZH] "随机 Hadamard 变换" and the         */
/* Sylvester construction under "构造 Hadamard 矩阵的方法"; the          */
/* butterfly under "为什么不用 Conference 矩阵", point 1; [TE-ID]        */
/* "Empat pengaman", first safeguard)                                  */
/* ------------------------------------------------------------------ */

/* y = (1/4) * H16 * D * x for one 16-point segment: D flips the sign of
 * x_j when bit j of mask is set; H16 is the natural-order Sylvester matrix
 * H[j][k] = (-1)^popcount(j & k), applied as four add/subtract butterfly
 * stages (h = 1, 2, 4, 8); every operation is binary32. */
void nvfp4_oracle_rht16(const float x[16], uint16_t mask, float y[16])
{
    float z[16];
    for (int j = 0; j < 16; ++j)
        z[j] = ((mask >> j) & 1) ? -x[j] : x[j];
    for (int h = 1; h < 16; h <<= 1) {
        for (int j = 0; j < 16; ++j) {
            if (j & h)
                continue;
            float a = z[j], b = z[j + h];
            z[j] = a + b;
            z[j + h] = a - b;
        }
    }
    for (int j = 0; j < 16; ++j)
        y[j] = 0.25f * z[j];
}

/* Standalone transform of a bf16 [R][C] tensor along axis 0 (16-row
 * segments of each column) or axis 1 (16-column segments of each row),
 * binary32 output of the same shape. */
void nvfp4_oracle_rht16_tensor(const uint16_t* x, int64_t R, int64_t C, int axis, uint16_t mask,
                               float* y)
{
    float seg[16], out[16];
    if (axis == 0) {
        for (int64_t r0 = 0; r0 < R; r0 += 16)
            for (int64_t c = 0; c < C; ++c) {
                for (int j = 0; j < 16; ++j)
                    seg[j] = bf16_bits_to_float(x[(r0 + j) * C + c]);
                nvfp4_oracle_rht16(seg, mask, out);
                for (int j = 0; j < 16; ++j)
                    y[(r0 + j) * C + c] = out[j];
            }
    } else {
        for (int64_t r = 0; r < R; ++r)
            for (int64_t c0 = 0; c0 < C; c0 += 16) {
                for (int j = 0; j < 16; ++j)
                    seg[j] = bf16_bits_to_float(x[r * C + c0 + j]);
                nvfp4_oracle_rht16(seg, mask, out);
                for (int j = 0; j < 16; ++j)
                    y[r * C + c0 + j] = out[j];
            }
    }
}

/* ------------------------------------------------------------------ */
/* Tensor amax and global scale                                        */
/* ------------------------------------------------------------------ */

/* Largest |x| over the tensor ([TE-ID] "Anatomi NVFP4"; [SCALE] "The
 * smallest example": the global scale comes from the tensor's maximum
 * absolute value). A NaN anywhere makes the result NaN. */
float nvfp4_oracle_amax_bf16(const uint16_t* x, int64_t n)
{
    float a = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float v = fabsf(bf16_bits_to_float(x[i]));
        if (isnan(v))
            return NAN;
        if (v > a)
            a = v;
    }
    return a;
}

/* amax of the Hadamard-transformed tensor (transform along axis 0). */
float nvfp4_oracle_amax_rht_axis0(const uint16_t* x, int64_t R, int64_t C, uint16_t mask)
{
    float seg[16], out[16], a = 0.0f;
    for (int64_t r0 = 0; r0 < R; r0 += 16)
        for (int64_t c = 0; c < C; ++c) {
            for (int j = 0; j < 16; ++j)
                seg[j] = bf16_bits_to_float(x[(r0 + j) * C + c]);
            nvfp4_oracle_rht16(seg, mask, out);
            for (int j = 0; j < 16; ++j) {
                float v = fabsf(out[j]);
                if (isnan(v))
                    return NAN;
                if (v > a)
                    a = v;
            }
        }
    return a;
}

/* S_g = amax / (448 * 6) ([TE-ID] "Anatomi NVFP4": amax divided by the
 * product of the E4M3 maximum 448 and the E2M1 maximum 6). One binary32
 * division; 2688 is exact. */
float nvfp4_oracle_global_scale(float amax)
{
    return amax / 2688.0f;
}

/* ------------------------------------------------------------------ */
/* One block: block scale, element ratio, rounding, sign               */
/* ------------------------------------------------------------------ */

/* Quantize one block of n values (16 for 1D, 256 for a 2D tile).
 * Block scale from the block maximum after the global scale ([SCALE] "The
 * smallest example": local scales come from block maxima once the global
 * scale is known), stored as E4M3 ([ZH] "NVFP4 的计算过程"); each element
 * is divided by its reconstruction unit s*S_g ([SCALE]: x = x_e2m1 *
 * s_block * s_global), rounded to E2M1, and keeps its sign bit.
 *   sr == 0: round-to-nearest-even; sr != 0: stochastic, draw h[k].
 * Writes one unpacked code (sign<<3 | magnitude) per element. */
static void quantize_block(const float* x, int n, float sg, int sr, const uint16_t* h,
                           uint8_t* codes, uint8_t* scale_byte)
{
    float b = 0.0f;
    int has_nan = 0;
    for (int k = 0; k < n; ++k) {
        float a = fabsf(x[k]);
        if (isnan(a))
            has_nan = 1;
        else if (a > b)
            b = a;
    }
    if (has_nan)
        b = NAN;
    float t = 6.0f * sg;
    float s_f = (t == 0.0f) ? 0.0f : b / t;
    uint8_t sb = nvfp4_oracle_e4m3_encode(s_f);
    float s = (float)nvfp4_oracle_e4m3_decode(sb);
    float d = s * sg;
    float r = (d == 0.0f) ? 0.0f : 1.0f / d;
    for (int k = 0; k < n; ++k) {
        float v = fabsf(x[k]) * r;
        int m = sr ? nvfp4_oracle_e2m1_sr(v, h[k]) : nvfp4_oracle_e2m1_rne(v);
        int sign = signbit(x[k]) ? 1 : 0;
        codes[k] = (uint8_t)((sign << 3) | m);
    }
    *scale_byte = sb;
}

/* Two codes per byte ([FP4]); element 2k in the low nibble. */
static void pack_codes(const uint8_t* codes, int n, uint8_t* out)
{
    for (int k = 0; k < n; k += 2)
        out[k / 2] = (uint8_t)(codes[k] | (codes[k + 1] << 4));
}

/* ------------------------------------------------------------------ */
/* 1D quantization ([TE-ID] "Anatomi NVFP4": one E4M3 scale per 16       */
/* consecutive elements; [SCALE] "A format is not a training recipe":   */
/* activations and gradients use 1D 16-value blocks)                    */
/* ------------------------------------------------------------------ */

/* Rowwise: blocks of 16 consecutive elements along C. Rows [r0, r1) of the
 * bf16 [R][C] tensor; codes [r1-r0][C/2], scales [r1-r0][C/16]. */
void nvfp4_oracle_quantize_1d_rows(const uint16_t* x, int64_t R, int64_t C, float sg, int sr,
                                   uint64_t seed, int64_t r0, int64_t r1, uint8_t* codes,
                                   uint8_t* scales)
{
    (void)R;
    float blk[16];
    uint16_t h[16];
    uint8_t q[16];
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t c0 = 0; c0 < C; c0 += 16) {
            for (int j = 0; j < 16; ++j) {
                int64_t i = r * C + c0 + j;
                blk[j] = bf16_bits_to_float(x[i]);
                h[j] = sr ? nvfp4_oracle_sr_draw(seed, (uint64_t)i) : 0;
            }
            quantize_block(blk, 16, sg, sr, h, q, &scales[(r - r0) * (C / 16) + c0 / 16]);
            pack_codes(q, 16, &codes[(r - r0) * (C / 2) + c0 / 2]);
        }
}

/* Columnwise: the same procedure on the transpose, blocks of 16 consecutive
 * rows of one column, optionally after the Hadamard transform along the
 * rows (the wgrad operand path of [TE-ID] "Empat pengaman"). Columns
 * [c0, c1); codes [c1-c0][R/2], scales [c1-c0][R/16]. Stochastic draws
 * use the element's row-major flat index in the input tensor. */
void nvfp4_oracle_quantize_1d_cols(const uint16_t* x, int64_t R, int64_t C, float sg, int sr,
                                   uint64_t seed, int rht, uint16_t mask, int64_t c0, int64_t c1,
                                   uint8_t* codes, uint8_t* scales)
{
    float seg[16], blk[16];
    uint16_t h[16];
    uint8_t q[16];
    for (int64_t c = c0; c < c1; ++c)
        for (int64_t rb = 0; rb < R; rb += 16) {
            for (int j = 0; j < 16; ++j) {
                int64_t i = (rb + j) * C + c;
                seg[j] = bf16_bits_to_float(x[i]);
                h[j] = sr ? nvfp4_oracle_sr_draw(seed, (uint64_t)i) : 0;
            }
            if (rht)
                nvfp4_oracle_rht16(seg, mask, blk);
            else
                memcpy(blk, seg, sizeof blk);
            quantize_block(blk, 16, sg, sr, h, q, &scales[(c - c0) * (R / 16) + rb / 16]);
            pack_codes(q, 16, &codes[(c - c0) * (R / 2) + rb / 2]);
        }
}

/* ------------------------------------------------------------------ */
/* 2D quantization ([TE-ID] "Empat pengaman", second safeguard: one     */
/* scale per 16x16 weight tile, so the row-read and column-read weights */
/* are the same numbers)                                                */
/* ------------------------------------------------------------------ */

/* Tile rows [tr0, tr1) (tile row = 16 tensor rows). Outputs, for the whole
 * tensor: codes_row [R][C/2] (may be NULL), codes_col [C][R/2] (may be
 * NULL), scales [R/16][C/16]; only the tiles in the range are written. */
void nvfp4_oracle_quantize_2d(const uint16_t* x, int64_t R, int64_t C, float sg, int64_t tr0,
                              int64_t tr1, uint8_t* codes_row, uint8_t* codes_col, uint8_t* scales)
{
    float tile[256];
    uint8_t q[256];
    for (int64_t tr = tr0; tr < tr1; ++tr)
        for (int64_t tc = 0; tc < C / 16; ++tc) {
            for (int i = 0; i < 16; ++i)
                for (int j = 0; j < 16; ++j)
                    tile[i * 16 + j] = bf16_bits_to_float(x[(tr * 16 + i) * C + tc * 16 + j]);
            quantize_block(tile, 256, sg, 0, NULL, q, &scales[tr * (C / 16) + tc]);
            for (int i = 0; i < 16; ++i)
                for (int j = 0; j < 16; j += 2) {
                    int64_t r = tr * 16 + i, c = tc * 16 + j;
                    if (codes_row)
                        codes_row[r * (C / 2) + c / 2] =
                            (uint8_t)(q[i * 16 + j] | (q[i * 16 + j + 1] << 4));
                }
            for (int j = 0; j < 16; ++j)
                for (int i = 0; i < 16; i += 2) {
                    int64_t r = tr * 16 + i, c = tc * 16 + j;
                    if (codes_col)
                        codes_col[c * (R / 2) + r / 2] =
                            (uint8_t)(q[i * 16 + j] | (q[(i + 1) * 16 + j] << 4));
                }
        }
}

/* ------------------------------------------------------------------ */
/* Dequantization and the contraction                                  */
/* ------------------------------------------------------------------ */

static uint8_t nibble(const uint8_t* codes, int64_t i)
{
    uint8_t b = codes[i >> 1];
    return (i & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15);
}

/* x = x_e2m1 * s_block * s_global ([SCALE] "The smallest example"; [ZH]
 * "NVFP4 的计算过程"), binary32: fl(fl(G*s) * S_g) with G*s exact, sign
 * applied. Rows [r0, r1) of the [R][C] output (row-major, C contiguous).
 * scale_mode 1: scales [R][C/16]; 2: tile scales [R/16][C/16]. */
void nvfp4_oracle_dequantize(const uint8_t* codes, const uint8_t* scales, int scale_mode, float sg,
                             int64_t R, int64_t C, int64_t r0, int64_t r1, float* out)
{
    (void)R;
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = 0; c < C; ++c) {
            uint8_t q = nibble(codes, r * C + c);
            uint8_t sb = (scale_mode == 2) ? scales[(r / 16) * (C / 16) + c / 16]
                                           : scales[r * (C / 16) + c / 16];
            float g = (float)E2M1_MAGNITUDE[q & 7];
            float s = (float)nvfp4_oracle_e4m3_decode(sb);
            float mag = (g * s) * sg;
            out[(r - r0) * C + c] = (q & 8) ? -mag : mag;
        }
}

/* bf16 output of the reconstruction: the binary32 value of
 * nvfp4_oracle_dequantize rounded to bf16, nearest even. */
static uint16_t float_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

void nvfp4_oracle_dequantize_bf16(const uint8_t* codes, const uint8_t* scales, int scale_mode,
                                  float sg, int64_t R, int64_t C, int64_t r0, int64_t r1,
                                  uint16_t* out)
{
    float tmp[16];
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t c0 = 0; c0 < C; c0 += 16) {
            for (int j = 0; j < 16; ++j) {
                int64_t c = c0 + j;
                uint8_t q = nibble(codes, r * C + c);
                uint8_t sb = (scale_mode == 2) ? scales[(r / 16) * (C / 16) + c / 16]
                                               : scales[r * (C / 16) + c / 16];
                float g = (float)E2M1_MAGNITUDE[q & 7];
                float s = (float)nvfp4_oracle_e4m3_decode(sb);
                float mag = (g * s) * sg;
                tmp[j] = (q & 8) ? -mag : mag;
            }
            for (int j = 0; j < 16; ++j)
                out[(r - r0) * C + c0 + j] = float_to_bf16_rne(tmp[j]);
        }
    (void)R;
}

/* Reconstructed elements in double for the listed rows of a [R][C] operand
 * (exact: at most 6 significant bits times a binary32 global scale):
 * out[t][c] = e2m1(code) * e4m3(scale) * S_g. The contraction itself is
 * a plain double-precision matrix product of these rows (the oracle's
 * Python side calls a library matmul for it). */
void nvfp4_oracle_dequantize_f64_rows(const uint8_t* codes, const uint8_t* scales, int scale_mode,
                                      float sg, int64_t R, int64_t C, const int64_t* rows,
                                      int64_t nrows, double* out)
{
    (void)R;
    for (int64_t t = 0; t < nrows; ++t) {
        int64_t r = rows[t];
        for (int64_t c = 0; c < C; ++c) {
            uint8_t q = nibble(codes, r * C + c);
            uint8_t sb = (scale_mode == 2) ? scales[(r / 16) * (C / 16) + c / 16]
                                           : scales[r * (C / 16) + c / 16];
            out[t * C + c] =
                nvfp4_oracle_e2m1_decode(q) * nvfp4_oracle_e4m3_decode(sb) * (double)sg;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Array forms of the scalar rules (for the tests' exhaustive sweeps)  */
/* ------------------------------------------------------------------ */

void nvfp4_oracle_e2m1_rne_array(const float* v, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint8_t)nvfp4_oracle_e2m1_rne(v[i]);
}

void nvfp4_oracle_e2m1_sr_array(const float* v, const uint16_t* h, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint8_t)nvfp4_oracle_e2m1_sr(v[i], h[i]);
}

void nvfp4_oracle_e4m3_encode_array(const float* v, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = nvfp4_oracle_e4m3_encode(v[i]);
}

void nvfp4_oracle_sr_draw_array(uint64_t seed, const uint64_t* idx, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = nvfp4_oracle_sr_draw(seed, idx[i]);
}

/* ------------------------------------------------------------------ */
/* MXFP4, the comparator format ([MX])                                 */
/* ------------------------------------------------------------------ */

/* E8M0: eight exponent bits, no sign, no mantissa, bias 127; 0xFF is NaN. */
double mxfp4_oracle_e8m0_decode(uint8_t b)
{
    if (b == 0xFF)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* The block's E8M0 byte from its maximum magnitude: the shared exponent
 * floor(log2 amax) minus E2M1's largest exponent (2), clamped to the
 * format's range. log2 of a binary32 value in double is exact enough for
 * the floor: a binary32 value below a power of two is at least 2^-24 below
 * it in relative terms, far above double's rounding. amax = 0 gives
 * -infinity and so the lowest byte; a non-finite amax gives NaN. */
uint8_t mxfp4_oracle_scale_byte(float amax)
{
    if (!isfinite(amax))
        return 0xFF;
    double e = floor(log2((double)amax)) - 2.0;
    if (e < -127.0)
        e = -127.0;
    if (e > 127.0)
        e = 127.0;
    return (uint8_t)(e + 127.0);
}

/* One block of 32 values: scale from the block maximum, each element x / X
 * rounded to E2M1 (round-to-nearest-even, saturating at 6), sign kept.
 * X is a power of two, so the division is exact wherever the quotient is a
 * binary32 normal; below that it only decides quotients far under 0.25,
 * which round to 0 either way. */
static void mx_quantize_block(const float* x, uint8_t* codes, uint8_t* scale_byte)
{
    float b = 0.0f;
    int bad = 0;
    for (int k = 0; k < 32; ++k) {
        float a = fabsf(x[k]);
        if (!isfinite(a))
            bad = 1;
        else if (a > b)
            b = a;
    }
    uint8_t sb = mxfp4_oracle_scale_byte(bad ? NAN : b);
    float X = (float)mxfp4_oracle_e8m0_decode(sb);
    for (int k = 0; k < 32; ++k) {
        float v = fabsf(x[k]) / X;
        int sign = signbit(x[k]) ? 1 : 0;
        codes[k] = (uint8_t)((sign << 3) | nvfp4_oracle_e2m1_rne(v));
    }
    *scale_byte = sb;
}

/* Rowwise: blocks of 32 consecutive elements along C. Rows [r0, r1) of the
 * bf16 [R][C] tensor; codes [r1-r0][C/2], scales [r1-r0][C/32]. */
void mxfp4_oracle_quantize_rows(const uint16_t* x, int64_t R, int64_t C, int64_t r0, int64_t r1,
                                uint8_t* codes, uint8_t* scales)
{
    (void)R;
    float blk[32];
    uint8_t q[32];
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t c0 = 0; c0 < C; c0 += 32) {
            for (int j = 0; j < 32; ++j)
                blk[j] = bf16_bits_to_float(x[r * C + c0 + j]);
            mx_quantize_block(blk, q, &scales[(r - r0) * (C / 32) + c0 / 32]);
            pack_codes(q, 32, &codes[(r - r0) * (C / 2) + c0 / 2]);
        }
}

/* Columnwise: blocks of 32 consecutive rows of one column, optionally after
 * the 16-point Hadamard transform along the rows (each block is two
 * transformed 16-row segments). Columns [c0, c1); codes [c1-c0][R/2],
 * scales [c1-c0][R/32]. */
void mxfp4_oracle_quantize_cols(const uint16_t* x, int64_t R, int64_t C, int rht, uint16_t mask,
                                int64_t c0, int64_t c1, uint8_t* codes, uint8_t* scales)
{
    float seg[16], blk[32];
    uint8_t q[32];
    for (int64_t c = c0; c < c1; ++c)
        for (int64_t rb = 0; rb < R; rb += 32) {
            for (int half = 0; half < 2; ++half) {
                for (int j = 0; j < 16; ++j)
                    seg[j] = bf16_bits_to_float(x[(rb + half * 16 + j) * C + c]);
                if (rht)
                    nvfp4_oracle_rht16(seg, mask, &blk[half * 16]);
                else
                    memcpy(&blk[half * 16], seg, sizeof seg);
            }
            mx_quantize_block(blk, q, &scales[(c - c0) * (R / 32) + rb / 32]);
            pack_codes(q, 32, &codes[(c - c0) * (R / 2) + rb / 2]);
        }
}

/* x = e2m1(code) * X, rows [r0, r1) of [R][C] (scales [R][C/32]), in
 * binary32. Exact for every byte a bf16 input can produce (at most 252):
 * two significant bits times a power of two from 2^-128 up. */
void mxfp4_oracle_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t R, int64_t C,
                             int64_t r0, int64_t r1, float* out)
{
    (void)R;
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = 0; c < C; ++c) {
            uint8_t q = nibble(codes, r * C + c);
            double X = mxfp4_oracle_e8m0_decode(scales[r * (C / 32) + c / 32]);
            out[(r - r0) * C + c] = (float)(nvfp4_oracle_e2m1_decode(q) * X);
        }
}

/* The same reconstruction in double for the listed rows (the GEMM
 * reference's operands). */
void mxfp4_oracle_dequantize_f64_rows(const uint8_t* codes, const uint8_t* scales, int64_t R,
                                      int64_t C, const int64_t* rows, int64_t nrows, double* out)
{
    (void)R;
    for (int64_t t = 0; t < nrows; ++t) {
        int64_t r = rows[t];
        for (int64_t c = 0; c < C; ++c)
            out[t * C + c] = nvfp4_oracle_e2m1_decode(nibble(codes, r * C + c)) *
                             mxfp4_oracle_e8m0_decode(scales[r * (C / 32) + c / 32]);
    }
}
