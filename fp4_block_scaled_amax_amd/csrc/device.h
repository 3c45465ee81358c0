// Device-side building blocks of the NVFP4 kernels (gfx950, wave64).
//
// Every floating-point step here is a single binary32 operation rounded to
// nearest even (the library is compiled with -ffp-contract=off, IEEE
// division and denormals on), so results are bit-identical to a scalar
// evaluation of the same steps in the same order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// --------------------------------------------------------- vector memory

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load that streams past the caches (last use of the data).
__device__ __forceinline__ uint4 load16_stream(const void* p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 load16(const void* p)
{
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load8_stream(const void* p)
{
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void store16_stream(void* p, uint4 v)
{
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void store16_stream(void* p, float4 v)
{
    __builtin_nontemporal_store(f32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4_t*>(p));
}

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Element j (0..7) of a 16-byte vector of bf16 as binary32.
__device__ __forceinline__ float bf16_at(const uint4& v, int j)
{
    uint32_t w = (j >> 1) == 0 ? v.x : (j >> 1) == 1 ? v.y : (j >> 1) == 2 ? v.z : v.w;
    return (j & 1) ? bf16_hi(w) : bf16_lo(w);
}

__device__ __forceinline__ uint32_t word_at(const uint4& v, int k)
{
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

// Packed max of two u16 lanes (|bf16| bit patterns; integer order of
// non-negative floats is their numeric order).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b)
{
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    u16x2 x = __builtin_bit_cast(u16x2, a);
    u16x2 y = __builtin_bit_cast(u16x2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

// ------------------------------------------------------------ E4M3 scale

// Round a non-negative binary32 (or NaN) to E4M3, nearest even, with
// subnormals; values >= 448 (and +inf) saturate to 448 (0x7E); NaN -> 0x7F.
// Branch-free: both the subnormal and the normal rounding are formed and
// the right one is selected.
__device__ __forceinline__ uint32_t e4m3_encode(float v)
{
    const uint32_t sub = (uint32_t)__builtin_rintf(v * 512.0f);      // multiples of 2^-9, RNE
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFFu + ((u >> 20) & 1u);                                 // RNE at mantissa bit 20
    const uint32_t nrm = (u >> 20) - (120u << 3);                     // rebias exponent 127 -> 7
    uint32_t b = (v < 0.015625f) ? sub : nrm;                        // below 2^-6: subnormal
    b = (v >= 448.0f) ? 0x7Eu : b;
    return (v != v) ? 0x7Fu : b;
}

__device__ __forceinline__ float e4m3_decode(uint32_t b)
{
    uint32_t e = (b >> 3) & 15u, m = b & 7u;
    if (b == 0x7Fu)
        return __uint_as_float(0x7FC00000u);
    if (e == 0)
        return (float)m * 0.001953125f;                  // m * 2^-9, exact
    return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Element multiplier of a block whose scale byte is `byte`:
// r = 1 / (e4m3(byte) * sg), or 0 when that unit is 0.
__device__ __forceinline__ float unit_reciprocal(uint32_t byte, float sg)
{
    const float d = e4m3_decode(byte) * sg;
    return (d == 0.0f) ? 0.0f : 1.0f / d;
}

// Scale byte of a block. b_bits: binary32 bits of the block's max |x|;
// t = 6 * sg with sg = amax / 2688. The IEEE division, exactly as the rule
// states it.
__device__ __forceinline__ uint32_t block_scale_byte(uint32_t b_bits, float t)
{
    const float b = __uint_as_float(b_bits);
    const float s_f = (t == 0.0f) ? 0.0f : b / t;
    return e4m3_encode(s_f);
}

// Same byte, cheaper: one multiply by inv_t = fl(1/t) instead of the IEEE
// division. y = fl(b * inv_t) is within 3 ulp of fl(b / t), so both round to
// the same E4M3 value unless an E4M3 rounding midpoint lies within 3 ulp of y
// (low 20 mantissa bits within 3 of 0x80000) or y is in the E4M3 subnormal
// range (below 2^-6, different rounding granularity); those lanes take the
// exact division. Requires t > 0 with t and inv_t finite (then b <= amax is
// finite and y <= 448 * (1 + 2^-22)).
__device__ __forceinline__ uint32_t block_scale_byte_fast(uint32_t b_bits, float t, float inv_t)
{
    const float b = __uint_as_float(b_bits);
    float y = b * inv_t;
    const uint32_t u = __float_as_uint(y);
    if (!(y >= 0.015625f) || (((u & 0xFFFFFu) - 0x7FFFDu) < 7u))
        return block_scale_byte(b_bits, t);
    const uint32_t r = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
    return r < 0x7Eu ? r : 0x7Eu;  // 432 and above round to (or saturate at) 448
}

// What decides whether a batch of block_scale_byte_approx results are all
// exact: every y must be a normal E4M3 value (2^-6 <= y, byte <= 0x7E, so
// not NaN, infinite or past the rounding to 480) and no y may lie within 3
// ulp of an E4M3 rounding midpoint.
struct ScaleVote {
    uint32_t min_y = 0xFFFFFFFFu;
    uint32_t min_guard = 0xFFFFFFFFu;
    uint32_t max_byte = 0u;
    __device__ __forceinline__ bool ok() const
    {
        return min_y >= 0x3C800000u && min_guard >= (7u << 12) && max_byte <= 0x7Eu;
    }
};

// Branch-free form of block_scale_byte_fast for batches: the byte of
// y = fl(b * inv_t) by integer rounding (exponent rebiased in the same add),
// with the checks deferred to `vote`. When vote.ok() holds for the batch,
// every byte equals block_scale_byte(b, t).
__device__ __forceinline__ uint32_t block_scale_byte_approx(uint32_t b_bits, float inv_t,
                                                            ScaleVote& vote)
{
    const uint32_t u = __float_as_uint(__uint_as_float(b_bits) * inv_t);
    vote.min_y = min(vote.min_y, u);
    // (low 20 bits of u) - 0x7FFFD, taken modulo 2^20 in the top 20 bits (one
    // shift-add): below 7 << 12 exactly when that difference is 0..6.
    vote.min_guard = min(vote.min_guard, (u << 12) - (0x7FFFDu << 12));
    const uint32_t byte = (u + (0x7FFFFu - (960u << 20)) + ((u >> 20) & 1u)) >> 20;
    vote.max_byte = max(vote.max_byte, byte);
    return byte;
}

// The 128 possible multipliers of a tensor (one per scale byte 0..127),
// built once per workgroup in LDS by the first 128 threads, each times a
// power of two `factor` (exact where the caller uses it; see
// fold_sr_scale_ok and fold_quarter_ok).
__device__ __forceinline__ void build_reciprocal_table(float* table, float sg, float factor = 1.0f)
{
    if (threadIdx.x < 128)
        table[threadIdx.x] = unit_reciprocal(threadIdx.x, sg) * factor;
}

// Sufficient for every multiplier of a byte 0..126 to be finite: then
// d = fl(s * sg) is 0 (byte 0) or lies in [2^-109, 2^109] for the scales
// s in [2^-9, 448], so 1/d is finite. False for NaN.
__device__ __forceinline__ bool reciprocals_finite(float sg)
{
    return sg >= 0x1p-100f && sg <= 0x1p100f;
}

// Folding powers of two into the multipliers. Every bf16 value is an
// integer multiple of 2^-133, and so is every binary32 sum and difference
// of such values (a rounded result of magnitude >= 2^-110 lands on a grid
// of at least 2^-133; a smaller exact one has at most 23 significant bits
// and needs no rounding): the Hadamard outputs z included. Hence:
//  - fold_quarter_ok: y = z / 4 is exact for every z, so fl(y * r) equals
//    fl(z * (r / 4)) whenever r / 4 is exact, which holds for every
//    multiplier when S_g is in [2^-100, 2^100] (r in [2^-109, 2^109]).
//  - fold_sr_scale_ok(sg, shift): the stochastic operand ceil(2^23 fl(v))
//    with v = fl(w * r) (w = x, or y = z/4 with shift 2) equals
//    ceil(fl(w' * r')) with r' = 2^(23 - shift) r: both are exact scalings
//    of one product while fl(v) is normal, and while it is not, both round
//    up to 1 as long as no nonzero product underflows to 0, i.e.
//    |w| r > 2^-150. |w| >= 2^-133 (2^-135 for y) and r = 1/(s S_g) >=
//    fl(1/(448 S_g)), so S_g <= 256 keeps it for x (r > 2^-16.9) and
//    S_g <= 32 for y (r > 2^-13.9); S_g >= 2^-95 keeps r' <= 2^127.
__device__ __forceinline__ bool fold_quarter_ok(float sg) { return reciprocals_finite(sg); }

template <int SHIFT>
__device__ __forceinline__ bool fold_sr_scale_ok(float sg)
{
    return sg >= 0x1p-95f && sg <= (SHIFT == 2 ? 32.0f : 256.0f);
}

// ----------------------------------------------------------- E2M1 codes
//
// Software stochastic rounding (used where a block multiplier is not finite;
// the hardware converters cover every other case). For a scaled magnitude
// v, the E2M1 grid has spacing 1/2 on [0, 2), 1 on [2, 4) and 2 on [4, 6].
// With j = clamp(exponent(v), 1, 3), vs = v * 2^(2-j) is exact: its integer
// part counts grid steps below v and its fraction is p = (v - lo)/(hi - lo).
// The element rounds up when h < p * 2^16 for its 16-bit draw h. Adding
// 2^23 + 2(j-1) + 8*sign in binary32 leaves the 4-bit code (the even offset
// keeps the parity) in the low bits of the result.
__device__ __forceinline__ uint32_t e2m1_sr_nibble(float v, uint32_t h16, uint32_t sign8)
{
    v = fminf(fmaxf(v, 0.0f), 6.0f);
    int e = __builtin_amdgcn_frexp_expf(v);
    int j = min(max(e, 1), 3);
    float vs = __builtin_amdgcn_ldexpf(v, 2 - j);
    float f = __builtin_floorf(vs);
    float p = vs - f;                                    // exact, in [0, 1)
    uint32_t up = ((float)h16 < p * 65536.0f) ? 1u : 0u;
    float q = f + __uint_as_float(0x4B000000u + 2u * (uint32_t)(j - 1) + sign8);
    return (__float_as_uint(q) + up) & 0xFu;
}

// ---------------------------------------------------- Philox4x32-10 draws
//
// Salmon et al., "Parallel random numbers: as easy as 1, 2, 3" (SC'11):
// ten rounds of two 32x32->64 multiplies and xors, key bumped by the Weyl
// constants between rounds. counter = (lo, hi, 0, 0).
__device__ __forceinline__ uint4 philox4x32_10(uint32_t ctr_lo, uint32_t ctr_hi, uint32_t k0,
                                               uint32_t k1)
{
    uint32_t c0 = ctr_lo, c1 = ctr_hi, c2 = 0u, c3 = 0u;
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        // three-input XORs (truth table 0x96) in one instruction each
        uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        uint32_t n3 = (uint32_t)p0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    return make_uint4(c0, c1, c2, c3);
}

// The 8 draws of flat indices 8q .. 8q+7: draw k is half (k & 1) of word k/2.
__device__ __forceinline__ uint32_t draw16(const uint4& w, int k)
{
    uint32_t word = word_at(w, k >> 1);
    return (k & 1) ? (word >> 16) : (word & 0xFFFFu);
}

// ----------------------------------------------- 16-point Hadamard (FWHT)
//
// y = (1/4) H16 D x: D negates element j of a 16-element segment when bit j
// of the mask is set, H16 is the natural-order (Sylvester) Hadamard matrix,
// evaluated as butterflies h = 1, 2, 4, 8 in binary32. D is applied to the
// packed bf16 words before unpacking (a sign flip is exact), so the
// butterfly takes already signed values.

// XOR pattern of D for a 16-row segment: row i's packed bf16 words.
__device__ __forceinline__ uint32_t rht_row_sign(uint32_t mask, int i)
{
    return ((mask >> i) & 1u) ? 0x80008000u : 0u;
}

// XOR pattern of D for a segment along a row: word k (elements 2k, 2k+1).
__device__ __forceinline__ uint32_t rht_pair_sign(uint32_t mask, int k)
{
    return (((mask >> (2 * k)) & 1u) << 15) | (((mask >> (2 * k + 1)) & 1u) << 31);
}

// The butterflies alone (H16 z, not yet scaled by 1/4).
__device__ __forceinline__ void hadamard16(float (&z)[16])
{
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j & h)
                continue;
            float a = z[j], b = z[j + h];
            z[j] = a + b;
            z[j + h] = a - b;
        }
    }
}

// y = (1/4) H16 z for signed inputs z = D x.
__device__ __forceinline__ void rht16_signed(float (&z)[16])
{
    hadamard16(z);
#pragma unroll
    for (int j = 0; j < 16; ++j)
        z[j] = 0.25f * z[j];
}

// ------------------------------------------------------------ wave utils

// Exchange with the neighbouring lane (lane ^ 1) through DPP quad_perm.
__device__ __forceinline__ uint32_t swap_lane1(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ float swap_lane1(float v)
{
    return __uint_as_float(swap_lane1(__float_as_uint(v)));
}

// The value of the even (from_even_lane) or odd lane of each lane pair, on
// both lanes of the pair.
__device__ __forceinline__ float from_even_lane(float v)
{
    return __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp((int)__float_as_uint(v), 0xA0, 0xF, 0xF, false));
}
__device__ __forceinline__ float from_odd_lane(float v)
{
    return __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp((int)__float_as_uint(v), 0xF5, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    return v;
}

// Global amax -> (S_g, 6*S_g).
__device__ __forceinline__ float global_scale_from_amax(float amax) { return amax / 2688.0f; }

}  // namespace nvfp4
