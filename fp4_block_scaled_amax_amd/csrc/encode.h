// E2M1 encoders shared by the quantize kernels: a pair of scaled values ->
// one byte of two codes, by the gfx950 converters (round to nearest even,
// or stochastic rounding through an exact input mapping) or in software.
// The same functions are exercised exhaustively against the reference rules
// by a test probe.
#pragma once

#include "device.h"

namespace nvfp4 {

// ---- encoders
//
// A pair of values (a, b) -> one byte of codes (a in the low nibble), placed
// at byte BYTE of a 32-bit word. MODE 0: hardware RNE; 1: hardware RNE with
// NaN ratios replaced by a signed zero first (the reference rule gives a NaN
// ratio magnitude 0 and keeps the element's sign; used only when a block
// multiplier is not finite, the one way a ratio can be NaN); 2: software
// stochastic rounding; 3: hardware stochastic rounding; 4: the same with a
// multiplier that already carries the converter's 2^23 operand scaling
// (see sr_operand).

enum { kEncHw = 0, kEncHwSafe = 1, kEncSr = 2, kEncSrHw = 3, kEncSrHwScaled = 4 };

constexpr bool is_sr(int mode) { return mode == kEncSr || mode == kEncSrHw || mode == kEncSrHwScaled; }
constexpr bool is_sr_hw(int mode) { return mode == kEncSrHw || mode == kEncSrHwScaled; }

// ---- stochastic rounding on the hardware converter
//
// v_cvt_scalef32_sr_pk_fp4_f32 rounds its first element up when the
// fraction bits it keeps below the E2M1 grid step (22 of them, aligned to
// the step), plus the top 22 bits of the random word, carry out. With the
// random word's top 16 bits = ~h and the rest ones, that is "up iff
// F > 64 h" for the kept fraction F = floor(p * 2^22) -- the rule's
// "h < p * 2^16" whenever p * 2^22 is an integer. It is for |v| >= 1; below
// 1 the value can have fraction bits under the kept ones, so |v| is first
// rounded up to a multiple of 2^-23 (which makes F = ceil(p * 2^22), and
// "F > 64 h" again equals the rule). The scaling by 2^23 is exact and is
// undone by the converter's power-of-two scale. Checked on the GPU against
// e2m1_sr_nibble for every 16-bit draw and 52,832 values (all binades from
// 2^-40 to 8 with random mantissas, every float within 300 ulp of each grid
// point and midpoint, both signs, zeros, subnormals, infinities,
// saturation); NaN ratios take the software encoder.

// Random word for the draw in the low (HALF = 0) or high half of `w`.
template <int HALF>
__device__ __forceinline__ uint32_t sr_random_word(uint32_t w)
{
    return HALF ? (~w | 0xFFFFu) : ~(w << 16);
}

// v -> the converter operand: 2^23 |v| rounded up to an integer (every
// binary32 value from 2^23 up already is one, so only |v| < 1 changes),
// with the sign of v. SCALED: the argument is already 2^23 v, formed by a
// multiplier that carries the 2^23 (callers use it only where that product
// equals 2^23 fl(v) or, for tiny ratios, rounds up to the same integer).
template <bool SCALED>
__device__ __forceinline__ float sr_operand(float v)
{
    const float tc = __builtin_ceilf(SCALED ? fabsf(v) : fabsf(v) * 0x1p23f);
    return __uint_as_float((__float_as_uint(tc) & 0x7FFFFFFFu) | (__float_as_uint(v) & 0x80000000u));
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Byte BYTE of `word` <- the stochastic codes of (a, b) with random words
// (ra, rb). Each value is converted alone as the first element of a pair
// whose second element is 0 (code 0), into byte 0: only byte 0 of the
// convert's result is used (the instruction leaves the other bytes of its
// destination register as they were, and the compiler does not tie them to
// an input), then the two codes are merged and byte-permuted into place.
template <int BYTE, bool SCALED>
__device__ __forceinline__ uint32_t sr_hw_pair(uint32_t word, float a, float b, uint32_t ra, uint32_t rb)
{
    const f32x2_t pa = {sr_operand<SCALED>(a), 0.0f};
    const f32x2_t pb = {sr_operand<SCALED>(b), 0.0f};
    const uint32_t ca = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, pa, ra, 0x1p23f, 0);
    const uint32_t cb = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, pb, rb, 0x1p23f, 0);
    const uint32_t pair = (cb << 4) | (ca & 0xFu);  // byte 0: code a | code b << 4
    // v_perm: selector bytes 0..3 pick `pair`, 4..7 pick `word`
    constexpr uint32_t sel = ((BYTE == 0 ? 0u : 4u) << 0) | ((BYTE == 1 ? 0u : 5u) << 8) |
                             ((BYTE == 2 ? 0u : 6u) << 16) | ((BYTE == 3 ? 0u : 7u) << 24);
    return __builtin_amdgcn_perm(word, pair, sel);
}

// One value through the stochastic converter into byte BYTE of w, the other
// bytes of w kept: the instruction writes only the selected byte, but the
// compiler's builtin does not tie its destination to an input (it drops the
// earlier contents), so the instruction is written out here with w as a
// read-write operand. The second element of the converted pair is +0 (code
// 0), so the byte's high nibble is 0.
template <int BYTE>
__device__ __forceinline__ void sr_cvt_byte(uint32_t& w, float operand, uint32_t rnd)
{
    const f32x2_t pv = {operand, 0.0f};
    const float scale = 0x1p23f;
    if (BYTE == 0)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3" : "+v"(w) : "v"(pv), "v"(rnd), "s"(scale));
    else if (BYTE == 1)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,0]" : "+v"(w) : "v"(pv), "v"(rnd), "s"(scale));
    else if (BYTE == 2)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,0,1]" : "+v"(w) : "v"(pv), "v"(rnd), "s"(scale));
    else
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,1]" : "+v"(w) : "v"(pv), "v"(rnd), "s"(scale));
}

// Per-element random input of mode MODE for column/element k of a Philox
// output: the 16-bit draw (software encoder) or the converter's random word.
template <int MODE>
__device__ __forceinline__ uint32_t sr_input(const uint4& w, int k)
{
    if (is_sr_hw(MODE)) {
        const uint32_t word = word_at(w, k >> 1);
        return (k & 1) ? sr_random_word<1>(word) : sr_random_word<0>(word);
    }
    return draw16(w, k);
}

__device__ __forceinline__ float nan_to_signed_zero(float v, float x)
{
    return (v != v) ? __uint_as_float(__float_as_uint(x) & 0x80000000u) : v;
}

template <int BYTE>
__device__ __forceinline__ uint32_t cvt_pair(uint32_t old, float a, float b)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, BYTE);
}

// A fresh word whose bytes will all be written: its initial contents do not
// matter, so let the compiler pick any register (no zero-fill).
// A word whose every byte the caller writes before using it. The converter
// writes one byte and keeps the register's others, so its destination is an
// input: an empty asm statement defines the register without an instruction
// (an undefined value folds to a zero that costs a move per word).
__device__ __forceinline__ uint32_t fresh_word()
{
    uint32_t w;
    asm volatile("" : "=v"(w));
    return w;
}

template <int MODE, int BYTE>
__device__ __forceinline__ uint32_t put_pair(uint32_t word, float a, float b, float r, uint32_t ha,
                                             uint32_t hb)
{
    if (MODE == kEncHw)
        return cvt_pair<BYTE>(word, a * r, b * r);
    if (MODE == kEncHwSafe) {
        // fma(x, r, -0) equals x * r for every input; spelling it differently
        // keeps the compiler from sharing (and hoisting) it with the fast path.
        return cvt_pair<BYTE>(word, nan_to_signed_zero(__builtin_fmaf(a, r, -0.0f), a),
                              nan_to_signed_zero(__builtin_fmaf(b, r, -0.0f), b));
    }
    if (is_sr_hw(MODE))
        return sr_hw_pair<BYTE, MODE == kEncSrHwScaled>(word, a * r, b * r, ha, hb);
    const uint32_t lo = e2m1_sr_nibble(fabsf(a) * r, ha, (__float_as_uint(a) >> 28) & 8u);
    const uint32_t hi = e2m1_sr_nibble(fabsf(b) * r, hb, (__float_as_uint(b) >> 28) & 8u);
    return word | ((lo | (hi << 4)) << (8 * BYTE));
}

// 16 values of one column (rows in order) -> 8 bytes of codes.
template <int MODE>
__device__ __forceinline__ uint2 encode_column16(const float (&y)[16], float r,
                                                 const uint4 (&draws)[16], int j)
{
    if (is_sr_hw(MODE)) {
        // Rows 2B (low nibble) and 2B+1 (high nibble) of each half go to byte
        // B: the even rows' codes are converted straight into the bytes of
        // one word, the odd rows' into another, and one shift-or joins them.
        uint32_t w[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            uint32_t we = fresh_word(), wo = fresh_word();
#define NVFP4_SR_BYTE(B)                                                                          \
    {                                                                                             \
        const int i = 8 * half + 2 * (B);                                                         \
        sr_cvt_byte<B>(we, sr_operand<MODE == kEncSrHwScaled>(y[i] * r), sr_input<MODE>(draws[i], j));         \
        sr_cvt_byte<B>(wo, sr_operand<MODE == kEncSrHwScaled>(y[i + 1] * r), sr_input<MODE>(draws[i + 1], j)); \
    }
            NVFP4_SR_BYTE(0) NVFP4_SR_BYTE(1) NVFP4_SR_BYTE(2) NVFP4_SR_BYTE(3)
#undef NVFP4_SR_BYTE
            w[half] = we | (wo << 4);
        }
        return make_uint2(w[0], w[1]);
    }
    uint32_t w[2] = {MODE == kEncSr ? 0u : fresh_word(), MODE == kEncSr ? 0u : fresh_word()};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#define NVFP4_PAIR(B)                                                                      \
    {                                                                                      \
        const int i = 8 * half + 2 * (B);                                                  \
        const uint32_t ha = is_sr(MODE) ? sr_input<MODE>(draws[i], j) : 0u;               \
        const uint32_t hb = is_sr(MODE) ? sr_input<MODE>(draws[i + 1], j) : 0u;           \
        w[half] = put_pair<MODE, B>(w[half], y[i], y[i + 1], r, ha, hb);                   \
    }
        NVFP4_PAIR(0) NVFP4_PAIR(1) NVFP4_PAIR(2) NVFP4_PAIR(3)
#undef NVFP4_PAIR
    }
    return make_uint2(w[0], w[1]);
}

}  // namespace nvfp4
