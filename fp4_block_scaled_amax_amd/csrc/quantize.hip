// NVFP4 quantization kernels: 1D (rowwise / columnwise / both, RNE or
// stochastic, optional Hadamard) and 2D (16x16 tiles, both layouts).
//
// One workgroup (256 threads, 4 waves) owns a 128 x 256 tile of the bf16
// input. A work item is 16 rows x 8 columns (sixteen 16-byte loads); the 32
// lanes of a half-wave cover 256 consecutive columns of a row (512
// contiguous bytes per load), the two half-waves of a wave cover two row
// blocks. Inside an item:
//   - a columnwise block is one column's 16 rows (all in one lane);
//   - a rowwise block is one row's 16 columns, split over the lane pair
//     (2k, 2k+1), which trade maxima and multipliers through DPP;
//   - a 2D tile is the lane pair's 16 x 16 elements.
// Rowwise codes are stored straight from registers (128 contiguous bytes per
// row per half-wave). Columnwise codes are staged in LDS; quantize_kernel
// writes them as 64-byte column segments (tiles walked down the rows per
// XCD, so the two halves of a line meet in one L2), while
// quantize_fused_kernel holds two vertically adjacent tiles per workgroup
// and writes whole 128-byte column lines. The fused kernel serves the
// in-kernel amax (single pass) and, with the amax given, both layouts.
//
// Encoding: the element ratio v = x * r (r = 1 / (s * S_g) of its block) is
// rounded to E2M1 by the gfx950 converter v_cvt_scalef32_pk_fp4_f32 with a
// unit scale, which rounds to nearest even and saturates at +-6 exactly like
// the reference rule for every non-NaN input (checked over all 2^32 binary32
// patterns); a NaN ratio needs a non-finite r, and such blocks first map NaN
// ratios to a signed zero. Stochastic rounding runs on the SR converter
// v_cvt_scalef32_sr_pk_fp4_f32 through an input mapping that reproduces the
// rule exactly (see sr_operand); blocks with a non-finite multiplier use the
// software encoder e2m1_sr_nibble.
#include <atomic>

#include "device.h"
#include "kernels.h"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kTileR = 128;
constexpr int kTileC = 256;
constexpr int kRowBlocks = kTileR / 16;  // 8
constexpr int kColGroups = kTileC / 8;   // 32
static_assert(kRowBlocks * kColGroups == kThreads, "one item per thread");

struct Params {
    const uint16_t* x;
    int64_t rows, cols;
    const float* amax;
    uint32_t mask, seed_lo, seed_hi;
    uint8_t* codes_row;
    uint8_t* scales_row;
    uint8_t* codes_col;
    uint8_t* scales_col;
    float* sg_out;
    int tiles_r, tiles_c;
    int amax_given;  // quantize_fused_kernel: *amax holds the amax, no exchange
};

// Map the workgroup index to a tile so that each XCD (workgroups are dealt
// round-robin over 8) walks a contiguous run of tiles; `vertical` makes the
// run go down the rows first.
__device__ __forceinline__ void tile_of_block(int tiles_r, int tiles_c, bool vertical, int& tr,
                                              int& tc)
{
    const int nt = tiles_r * tiles_c;
    int t = blockIdx.x;
    if ((nt & 7) == 0) {
        const int per = nt >> 3;
        t = (t & 7) * per + (t >> 3);
    }
    if (vertical) {
        tr = t % tiles_r;
        tc = t / tiles_r;
    } else {
        tc = t % tiles_c;
        tr = t / tiles_c;
    }
}

__device__ __forceinline__ bool finite_bits(float r)
{
    return (__float_as_uint(r) & 0x7F800000u) != 0x7F800000u;
}

// ---- encoders
//
// A pair of values (a, b) -> one byte of codes (a in the low nibble), placed
// at byte BYTE of a 32-bit word. MODE 0: hardware RNE; 1: hardware RNE with
// NaN ratios replaced by a signed zero first (the reference rule gives a NaN
// ratio magnitude 0 and keeps the element's sign; used only when a block
// multiplier is not finite, the one way a ratio can be NaN); 2: software
// stochastic rounding.

enum { kEncHw = 0, kEncHwSafe = 1, kEncSr = 2, kEncSrHw = 3 };

constexpr bool is_sr(int mode) { return mode == kEncSr || mode == kEncSrHw; }

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
// with the sign of v.
__device__ __forceinline__ float sr_operand(float v)
{
    const float tc = __builtin_ceilf(fabsf(v) * 0x1p23f);
    return __uint_as_float((__float_as_uint(tc) & 0x7FFFFFFFu) | (__float_as_uint(v) & 0x80000000u));
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Byte BYTE of `word` <- the stochastic codes of (a, b) with random words
// (ra, rb). Each value is converted alone as the first element of a pair
// whose second element is 0 (code 0), into byte 0: only byte 0 of the
// convert's result is used (the instruction leaves the other bytes of its
// destination register as they were, and the compiler does not tie them to
// an input), then the two codes are merged and byte-permuted into place.
template <int BYTE>
__device__ __forceinline__ uint32_t sr_hw_pair(uint32_t word, float a, float b, uint32_t ra, uint32_t rb)
{
    const f32x2_t pa = {sr_operand(a), 0.0f};
    const f32x2_t pb = {sr_operand(b), 0.0f};
    const uint32_t ca = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, pa, ra, 0x1p23f, 0);
    const uint32_t cb = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, pb, rb, 0x1p23f, 0);
    const uint32_t pair = (cb << 4) | (ca & 0xFu);  // byte 0: code a | code b << 4
    // v_perm: selector bytes 0..3 pick `pair`, 4..7 pick `word`
    constexpr uint32_t sel = ((BYTE == 0 ? 0u : 4u) << 0) | ((BYTE == 1 ? 0u : 5u) << 8) |
                             ((BYTE == 2 ? 0u : 6u) << 16) | ((BYTE == 3 ? 0u : 7u) << 24);
    return __builtin_amdgcn_perm(word, pair, sel);
}

// Per-element random input of mode MODE for column/element k of a Philox
// output: the 16-bit draw (software encoder) or the converter's random word.
template <int MODE>
__device__ __forceinline__ uint32_t sr_input(const uint4& w, int k)
{
    if (MODE == kEncSrHw) {
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
__device__ __forceinline__ uint32_t fresh_word() { return __builtin_nondeterministic_value(0u); }

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
    if (MODE == kEncSrHw)
        return sr_hw_pair<BYTE>(word, a * r, b * r, ha, hb);
    const uint32_t lo = e2m1_sr_nibble(fabsf(a) * r, ha, (__float_as_uint(a) >> 28) & 8u);
    const uint32_t hi = e2m1_sr_nibble(fabsf(b) * r, hb, (__float_as_uint(b) >> 28) & 8u);
    return word | ((lo | (hi << 4)) << (8 * BYTE));
}

// 16 values of one column (rows in order) -> 8 bytes of codes.
template <int MODE>
__device__ __forceinline__ uint2 encode_column16(const float (&y)[16], float r,
                                                 const uint4 (&draws)[16], int j)
{
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

// Row-and/or-column encoding of a whole item in 2x2 groups: elements
// (i, 2k), (i, 2k+1), (i+1, 2k), (i+1, 2k+1) are unpacked once and feed byte
// k of the two row words and byte (i/2 mod 4) of the two column words.
template <int MODE, int IP, bool ROW, bool COL>
__device__ __forceinline__ void encode_row_pair(const uint4 (&v)[16], const float (&rr)[16],
                                                const float (&rc)[8], const uint4 (&draws)[16],
                                                uint32_t (&roww)[2], uint32_t (&colw)[8][2])
{
    constexpr int i = 2 * IP;
    constexpr int cb = IP & 3;     // byte within the column word
    constexpr int ch = IP >> 2;    // which column word (rows 0..7 or 8..15)
    roww[0] = roww[1] = MODE == kEncSr ? 0u : fresh_word();
    if (MODE != kEncSr && COL && cb == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            colw[j][ch] = fresh_word();
    }
#define NVFP4_GROUP(K)                                                                      \
    {                                                                                       \
        const uint32_t w0 = word_at(v[i], K), w1 = word_at(v[i + 1], K);                    \
        const float a = bf16_lo(w0), b = bf16_hi(w0), c = bf16_lo(w1), d = bf16_hi(w1);     \
        uint32_t ha = 0u, hb = 0u, hc = 0u, hd = 0u;                                        \
        if (is_sr(MODE)) {                                                                  \
            ha = sr_input<MODE>(draws[i], 2 * K);                                           \
            hb = sr_input<MODE>(draws[i], 2 * K + 1);                                       \
            hc = sr_input<MODE>(draws[i + 1], 2 * K);                                       \
            hd = sr_input<MODE>(draws[i + 1], 2 * K + 1);                                   \
        }                                                                                   \
        if (ROW) {                                                                          \
            roww[0] = put_pair<MODE, K>(roww[0], a, b, rr[i], ha, hb);                      \
            roww[1] = put_pair<MODE, K>(roww[1], c, d, rr[i + 1], hc, hd);                  \
        }                                                                                   \
        if (COL) {                                                                          \
            colw[2 * K][ch] = put_pair<MODE, cb>(colw[2 * K][ch], a, c, rc[2 * K], ha, hc);         \
            colw[2 * K + 1][ch] = put_pair<MODE, cb>(colw[2 * K + 1][ch], b, d, rc[2 * K + 1], hb, hd); \
        }                                                                                   \
    }
    NVFP4_GROUP(0) NVFP4_GROUP(1) NVFP4_GROUP(2) NVFP4_GROUP(3)
#undef NVFP4_GROUP
}

template <int MODE, bool ROW, bool COL>
__device__ __forceinline__ void encode_item(const uint4 (&v)[16], const float (&rr)[16],
                                            const float (&rc)[8], const uint4 (&draws)[16],
                                            uint8_t* row_dst, int64_t row_pitch,
                                            uint32_t (&colw)[8][2])
{
    // A half-wave's rowwise codes of one row are a whole 128-byte line:
    // stream them past the caches.
    uint32_t roww[2];
#define NVFP4_ROWS(IP)                                                                   \
    encode_row_pair<MODE, IP, ROW, COL>(v, rr, rc, draws, roww, colw);                    \
    if (ROW) {                                                                           \
        uint8_t* d = row_dst + (2 * IP) * row_pitch;                                     \
        __builtin_nontemporal_store(roww[0], reinterpret_cast<uint32_t*>(d));            \
        __builtin_nontemporal_store(roww[1], reinterpret_cast<uint32_t*>(d + row_pitch)); \
    }
    NVFP4_ROWS(0) NVFP4_ROWS(1) NVFP4_ROWS(2) NVFP4_ROWS(3)
    NVFP4_ROWS(4) NVFP4_ROWS(5) NVFP4_ROWS(6) NVFP4_ROWS(7)
#undef NVFP4_ROWS
}

// Position of this thread's work item inside a tile.
struct ItemPos {
    int64_t tile_r0, tile_c0, r0, c0;
    int rb, cg;
    bool odd, valid;
};

__device__ __forceinline__ ItemPos item_pos(int tr, int tc, int64_t rows, int64_t cols)
{
    ItemPos q;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    q.tile_r0 = (int64_t)tr * kTileR;
    q.tile_c0 = (int64_t)tc * kTileC;
    q.cg = lane & 31;
    q.rb = wave * 2 + (lane >> 5);
    q.odd = (lane & 1) != 0;
    q.r0 = q.tile_r0 + q.rb * 16;
    q.c0 = q.tile_c0 + q.cg * 8;
    // Both lanes of a pair agree: cols is a multiple of 16.
    q.valid = q.r0 < rows && q.c0 < cols;
    return q;
}

__device__ __forceinline__ void load_item(const Params& p, const ItemPos& q, uint4 (&v)[16])
{
    if (q.valid) {
        const uint16_t* src = p.x + q.r0 * p.cols + q.c0;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            v[i] = load16_stream(src + i * p.cols);
    }
}

// Block maxima of an item as packed pairs of |bf16| patterns (16 bits each,
// the upper 16 bits of the binary32 maximum).
//   col[k]: columns 2k (low half) and 2k+1 (high half), over the 16 rows;
//   row[k]: the rowwise blocks (16 columns, split over the lane pair) of
//           rows 2k (low half) and 2k+1 (high half) of this lane's half of
//           the item's rows: rows 0..7 on even lanes, 8..15 on odd lanes.
// Both depend on the data alone, so the fused kernel takes them before the
// grid-wide amax is known.
struct BlockMax {
    uint32_t col[4];
    uint32_t row[4];
};

__device__ __forceinline__ void column_maxima(const uint4 (&v)[16], BlockMax& bm)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t pm = 0u;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            pm = pk_max_u16(pm, word_at(v[i], k) & 0x7FFF7FFFu);
        bm.col[k] = pm;
    }
}

// Row maxima trade halves through DPP with the pair lane: every lane of the
// pair must be active (both are, as the item validity is pairwise).
__device__ __forceinline__ void row_maxima(const uint4 (&v)[16], bool odd, BlockMax& bm)
{
    uint32_t pm[16];  // per row: packed maxima of the lane's 4 column pairs
#pragma unroll
    for (int i = 0; i < 16; ++i)
        pm[i] = pk_max_u16(pk_max_u16(v[i].x & 0x7FFF7FFFu, v[i].y & 0x7FFF7FFFu),
                           pk_max_u16(v[i].z & 0x7FFF7FFFu, v[i].w & 0x7FFF7FFFu));
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
        // This lane's maxima of rows k, k+1 (low, high half) and of rows
        // k+8, k+9: the low halves of a row pair in one word, the high
        // halves in the other, then one packed max.
        const uint32_t lo = pk_max_u16(__builtin_amdgcn_perm(pm[k + 1], pm[k], 0x05040100u),
                                       __builtin_amdgcn_perm(pm[k + 1], pm[k], 0x07060302u));
        const uint32_t hi = pk_max_u16(__builtin_amdgcn_perm(pm[k + 9], pm[k + 8], 0x05040100u),
                                       __builtin_amdgcn_perm(pm[k + 9], pm[k + 8], 0x07060302u));
        const uint32_t own = odd ? hi : lo;
        const uint32_t send = odd ? lo : hi;
        bm.row[k >> 1] = pk_max_u16(own, swap_lane1(send));
    }
}

// Binary32 bits of a packed half: the low (H = 0) or high (H = 1) 16 bits.
template <int H>
__device__ __forceinline__ uint32_t half_bits(uint32_t packed)
{
    return H ? (packed & 0xFFFF0000u) : (packed << 16);
}

__device__ __forceinline__ uint32_t col_max_bits(const BlockMax& bm, int j)
{
    return (j & 1) ? half_bits<1>(bm.col[j >> 1]) : half_bits<0>(bm.col[j >> 1]);
}

__device__ __forceinline__ uint32_t row_max_bits(const BlockMax& bm, int k)
{
    return (k & 1) ? half_bits<1>(bm.row[k >> 1]) : half_bits<0>(bm.row[k >> 1]);
}

__device__ __forceinline__ uint32_t item_max(const BlockMax& bm)
{
    uint32_t pm = pk_max_u16(pk_max_u16(bm.col[0], bm.col[1]), pk_max_u16(bm.col[2], bm.col[3]));
    return max(pm & 0xFFFFu, pm >> 16) << 16;
}

// Per-tensor constants of the scale chain.
struct ScaleCtx {
    float sg, t6, inv_t6;
    bool fast;      // t6 > 0 with t6 and 1/t6 finite: block_scale_byte_fast applies
    bool table_ok;  // every multiplier of a byte 0..126 is known to be finite
};

__device__ __forceinline__ ScaleCtx scale_ctx(float amax)
{
    ScaleCtx c;
    c.sg = global_scale_from_amax(amax);
    c.t6 = 6.0f * c.sg;
    c.inv_t6 = 1.0f / c.t6;
    c.fast = c.t6 > 0.0f && finite_bits(c.t6) && finite_bits(c.inv_t6);
    c.table_ok = reciprocals_finite(c.sg);
    return c;
}

__device__ __forceinline__ uint32_t scale_byte(uint32_t b_bits, const ScaleCtx& c)
{
    return c.fast ? block_scale_byte_fast(b_bits, c.t6, c.inv_t6) : block_scale_byte(b_bits, c.t6);
}

// Quantize one work item held in registers: block scales, codes; rowwise
// outputs go straight to memory, columnwise outputs to the LDS staging.
// bm: the item's block maxima (column maxima are ignored with RHT, which
// recomputes them from the transformed values; row maxima are needed for
// rowwise 1D only).
template <bool ROW, bool COL, bool TWO_D, bool SR, bool RHT>
__device__ __forceinline__ void compute_item(const Params& p, const ItemPos& q,
                                             const uint4 (&v)[16], const BlockMax& bm,
                                             const ScaleCtx& sc, const float* lds_rcp,
                                             uint2* lds_codes, uint8_t* lds_scales)
{
    const int64_t cols = p.cols;
    const int64_t r0 = q.r0, c0 = q.c0;
    const int rb = q.rb, cg = q.cg;
    const bool odd = q.odd;
    // Stochastic-rounding draws: one Philox call per row covers the
    // item's 8 consecutive flat indices.
    uint4 draws[16];
    if (SR) {
        const uint64_t flat0 = (uint64_t)(r0 * cols + c0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint64_t qq = (flat0 + (uint64_t)i * (uint64_t)cols) >> 3;
            draws[i] = philox4x32_10((uint32_t)qq, (uint32_t)(qq >> 32), p.seed_lo, p.seed_hi);
        }
    }

    if (COL && !ROW && !TWO_D) {
        // -------------------------------------------- columnwise only
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float y[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                y[i] = RHT ? bf16_at(make_uint4(v[i].x ^ rht_row_sign(p.mask, i), v[i].y ^ rht_row_sign(p.mask, i),
                                                v[i].z ^ rht_row_sign(p.mask, i), v[i].w ^ rht_row_sign(p.mask, i)), j)
                           : bf16_at(v[i], j);
            uint32_t m;
            if (RHT) {
                rht16_signed(y);
                m = 0u;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    m = max(m, __float_as_uint(y[i]) & 0x7FFFFFFFu);
            } else {
                m = (j & 1) ? half_bits<1>(bm.col[j >> 1]) : half_bits<0>(bm.col[j >> 1]);
            }
            const uint32_t byte = scale_byte(m, sc);
            const float r = lds_rcp[byte];
            uint2 words;
            if (SR)
                words = __all(finite_bits(r)) ? encode_column16<kEncSrHw>(y, r, draws, j)
                                              : encode_column16<kEncSr>(y, r, draws, j);
            else if (__all(finite_bits(r)))
                words = encode_column16<kEncHw>(y, r, draws, j);
            else
                words = encode_column16<kEncHwSafe>(y, r, draws, j);
            const int col = cg * 8 + j;
            lds_codes[col * kRowBlocks + (rb ^ (cg & 7))] = words;
            lds_scales[col * kRowBlocks + rb] = (uint8_t)byte;
        }
        return;
    }

    // ----------------------------- rowwise, rowwise + columnwise, 2D
    float rc[8];   // columnwise multipliers (1D), or the tile's (2D)
    float rr[16];  // rowwise multipliers (1D), or the tile's (2D)
    uint32_t col_byte[8];
    bool fin = true;
    if (TWO_D) {
        uint32_t m = item_max(bm);
        m = max(m, swap_lane1(m));
        const uint32_t byte = scale_byte(m, sc);
        const float r = lds_rcp[byte];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            rc[j] = r;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            rr[i] = r;
        fin = finite_bits(r);
        if (!odd) {
            p.scales_row[(r0 >> 4) * (cols >> 4) + (c0 >> 4)] = (uint8_t)byte;
            if (p.scales_col != nullptr)  // the transposed tile grid, if asked for
                p.scales_col[(c0 >> 4) * (p.rows >> 4) + (r0 >> 4)] = (uint8_t)byte;
        }
    } else {
        // All of the item's scale bytes by the branch-free approximate
        // chain, checked once for the wave; a wave holding any block it
        // cannot settle redoes them all with the exact chain.
        uint32_t row_byte[8];
        ScaleVote vote;
        if (COL) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                col_byte[j] = block_scale_byte_approx(col_max_bits(bm, j), sc.inv_t6, vote);
        }
        if (ROW) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                row_byte[k] = block_scale_byte_approx(row_max_bits(bm, k), sc.inv_t6, vote);
        }
        fin = sc.table_ok;
        if (!__all(sc.fast && vote.ok())) {
            uint32_t mb = 0u;
            if (COL) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    col_byte[j] = scale_byte(col_max_bits(bm, j), sc);
                    mb = max(mb, col_byte[j]);
                }
            }
            if (ROW) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    row_byte[k] = scale_byte(row_max_bits(bm, k), sc);
                    mb = max(mb, row_byte[k]);
                }
            }
            fin = fin && mb <= 0x7Eu;  // 0x7F (a NaN block) has no finite multiplier
        }
        if (COL) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                rc[j] = lds_rcp[col_byte[j]];
        }
        if (ROW) {
            // Even lanes own rows 0..7 of the pair's blocks, odd lanes 8..15.
            const int64_t srow0 = r0 + (odd ? 8 : 0);
            uint8_t* sdst = p.scales_row + srow0 * (cols >> 4) + (c0 >> 4);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                sdst[k * (cols >> 4)] = (uint8_t)row_byte[k];
                const float mine = lds_rcp[row_byte[k]];
                rr[k] = from_even_lane(mine);     // rows 0..7: settled by the even lane
                rr[k + 8] = from_odd_lane(mine);  // rows 8..15: by the odd lane
            }
        }
        if (!sc.table_ok) {
            // Some multiplier is not finite (tiny or non-finite amax): test
            // the ones in use.
            fin = true;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                fin = fin && (!COL || finite_bits(rc[j]));
#pragma unroll
            for (int k = 0; k < 16; ++k)
                fin = fin && (!ROW || finite_bits(rr[k]));
        }
    }
    uint32_t colw[8][2];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        colw[j][0] = colw[j][1] = 0u;
    uint8_t* row_dst = ROW ? p.codes_row + r0 * (cols >> 1) + (c0 >> 1) : nullptr;
    const int64_t row_pitch = cols >> 1;
    if (SR && __all(fin))
        encode_item<kEncSrHw, ROW, COL>(v, rr, rc, draws, row_dst, row_pitch, colw);
    else if (SR)
        encode_item<kEncSr, ROW, COL>(v, rr, rc, draws, row_dst, row_pitch, colw);
    else if (__all(fin))
        encode_item<kEncHw, ROW, COL>(v, rr, rc, draws, row_dst, row_pitch, colw);
    else
        encode_item<kEncHwSafe, ROW, COL>(v, rr, rc, draws, row_dst, row_pitch, colw);
    if (COL) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int col = cg * 8 + j;
            lds_codes[col * kRowBlocks + (rb ^ (cg & 7))] = make_uint2(colw[j][0], colw[j][1]);
            if (!TWO_D)
                lds_scales[col * kRowBlocks + rb] = (uint8_t)col_byte[j];
        }
    }
}

// Write a tile's staged columnwise codes (and 1D column scales) to memory.
template <bool TWO_D>
__device__ __forceinline__ void write_col_tile(const Params& p, int64_t tile_r0, int64_t tile_c0,
                                               const uint2* lds_codes, const uint8_t* lds_scales)
{
    const int64_t rows = p.rows, cols = p.cols;
    // Codes: 8-byte chunks; 8 lanes cover one tile column's 64 bytes.
    const int64_t pitch = rows >> 1;
#pragma unroll
    for (int k = 0; k < kTileC * kRowBlocks / kThreads; ++k) {
        const int q = k * kThreads + threadIdx.x;
        const int col = q >> 3, part = q & 7;
        const int64_t c = tile_c0 + col, r = tile_r0 + part * 16;
        if (c < cols && r < rows) {
            const int slot = part ^ ((col >> 3) & 7);
            *reinterpret_cast<uint2*>(p.codes_col + c * pitch + (r >> 1)) =
                lds_codes[col * kRowBlocks + slot];
        }
    }
    if (!TWO_D) {
        // Scales: one tile column's 8 bytes per thread.
        const int col = threadIdx.x;
        const int64_t c = tile_c0 + col;
        if (c < cols) {
            const int64_t spitch = rows >> 4;
            uint8_t* dst = p.scales_col + c * spitch + (tile_r0 >> 4);
            const int64_t nb64 = (rows - tile_r0) >> 4;
            const int nb = nb64 < kRowBlocks ? (int)nb64 : kRowBlocks;
            const uint8_t* srcs = &lds_scales[col * kRowBlocks];
            if (nb == kRowBlocks && ((reinterpret_cast<uintptr_t>(dst) & 7) == 0)) {
                *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(srcs);
            } else {
                for (int b = 0; b < nb; ++b)
                    dst[b] = srcs[b];
            }
        }
    }
}

template <bool ROW, bool COL, bool TWO_D, bool SR, bool RHT>
__global__ __launch_bounds__(kThreads) void quantize_kernel(Params p)
{
    // Columnwise staging: per tile column, 8 row blocks x 8 bytes; the slot
    // of a row block is swizzled by the column group to spread LDS banks.
    __shared__ uint2 lds_codes[COL ? kTileC * kRowBlocks : 1];
    __shared__ uint8_t lds_scales[(COL && !TWO_D) ? kTileC * kRowBlocks : 16];
    __shared__ float lds_rcp[128];

    int tr, tc;
    tile_of_block(p.tiles_r, p.tiles_c, COL, tr, tc);
    const ItemPos q = item_pos(tr, tc, p.rows, p.cols);
    uint4 v[16];
    load_item(p, q, v);

    const ScaleCtx sc = scale_ctx(*p.amax);
    if (p.sg_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
        *p.sg_out = sc.sg;
    build_reciprocal_table(lds_rcp, sc.sg);
    __syncthreads();

    if (q.valid) {
        BlockMax bm;
        if (!RHT)
            column_maxima(v, bm);
        if (ROW && !TWO_D)
            row_maxima(v, q.odd, bm);
        compute_item<ROW, COL, TWO_D, SR, RHT>(p, q, v, bm, sc, lds_rcp, lds_codes, lds_scales);
    }
    if (COL) {
        __syncthreads();
        write_col_tile<TWO_D>(p, q.tile_r0, q.tile_c0, lds_codes, lds_scales);
    }
}

// ---------------------------------------------------------------------------
// Fused amax + quantize: one persistent launch in which every thread keeps
// two work items (2 x 256 bytes of bf16) in registers, so the tensor is read
// from HBM once. The workgroups exchange their block-local maxima through a
// small workspace without read-modify-write atomics: each workgroup posts
// (generation, max) in its own arrival slot, workgroup 0 collects them all
// and posts (generation, amax) in every workgroup's own release slot, so no
// address is polled by more than a few workgroups. The grid is sized so all
// workgroups fit on the device at once; the waits are bounded by wall-clock
// time and, should they expire (workgroups not co-resident), a workgroup
// computes the exact amax directly from the tensor, so the result is always
// the same and the device can never hang. With Params::amax_given the
// kernel takes the amax from memory instead and skips the exchange (then any
// grid size works): the two-layout quantize with a given amax uses it for
// its paired tiles.
//
// Workspace (32-bit words): [0] amax bits, [1] generation of the last
// completed call, [2] slow-path counter, [3] wait limit in ticks of the
// 100 MHz counter (0: the default; a tiny value makes every wait expire, so
// tests can drive the fallback), then 2 words per workgroup of arrival
// slots and 2 words per workgroup of release slots.

constexpr int kWsAmax = 0, kWsGen = 1, kWsSlow = 2, kWsWait = 3, kWsArrive = 16;
constexpr int kMaxFusedBlocks = 2048;                       // slots in the workspace
constexpr int kWsRelease = kWsArrive + 2 * kMaxFusedBlocks;
constexpr int kMaxFusedGrid = 1024;                         // largest grid launched
constexpr uint64_t kWaitTicks = 200000;  // 2 ms of the 100 MHz real-time counter

// All exchange traffic is relaxed device-scope atomics: the value travels
// inside the atomic word itself, so no other memory needs ordering (and
// acquire/release at device scope would write back or invalidate the
// non-coherent per-XCD L2s).
__device__ __forceinline__ uint32_t ws_load(const uint32_t* a)
{
    return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ws_store(uint32_t* a, uint32_t v)
{
    __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A (generation, value) pair in one 64-bit word, so a reader sees both or neither.
__device__ __forceinline__ uint64_t slot_load(const uint32_t* a)
{
    return __hip_atomic_load(reinterpret_cast<const uint64_t*>(a), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void slot_store(uint32_t* a, uint32_t gen, uint32_t value)
{
    __hip_atomic_store(reinterpret_cast<uint64_t*>(a), ((uint64_t)value << 32) | gen,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Maximum over the workgroup; every thread gets the result.
__device__ __forceinline__ uint32_t workgroup_max(uint32_t m, uint32_t* red)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    m = wave_max_u32(m);
    __syncthreads();
    if (lane == 0)
        red[wave] = m;
    __syncthreads();
    uint32_t r = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w)
        r = max(r, red[w]);
    return r;
}

// Exact amax of the whole tensor by this workgroup alone (slow path).
__device__ uint32_t direct_amax(const Params& p, uint32_t* red)
{
    const int64_t n = p.rows * p.cols;
    uint32_t pm = 0u;
    for (int64_t i = (int64_t)threadIdx.x * 8; i < n; i += (int64_t)kThreads * 8) {
        const uint4 v = load16(p.x + i);
        pm = pk_max_u16(pm, v.x & 0x7FFF7FFFu);
        pm = pk_max_u16(pm, v.y & 0x7FFF7FFFu);
        pm = pk_max_u16(pm, v.z & 0x7FFF7FFFu);
        pm = pk_max_u16(pm, v.w & 0x7FFF7FFFu);
    }
    return workgroup_max(max(pm & 0xFFFFu, pm >> 16) << 16, red);
}

// This call's generation: one more than the last completed call's. Read at
// the start of the kernel, off the exchange's critical path (the word only
// changes once every workgroup of this call has posted its arrival).
__device__ __forceinline__ uint32_t call_generation(const uint32_t* ws)
{
    return ws_load(&ws[kWsGen]) + 1u;
}

// Grid-wide maximum of one value per workgroup (binary32 bits); every
// workgroup returns the same result. gen0 and wait0 (workspace word 3: the
// bound on each wait in 100 MHz ticks, 0 for the default) are read by
// thread 0 at the start of the kernel.
__device__ uint32_t grid_max(uint32_t m, uint32_t gen0, uint32_t wait0, uint32_t* ws, const Params& p)
{
    __shared__ uint32_t red[kThreads / 64];
    __shared__ uint32_t gen_s, wait_s, result_s, ok_s;
    m = workgroup_max(m, red);
    if (threadIdx.x == 0) {
        gen_s = gen0;
        wait_s = wait0;
        slot_store(&ws[kWsArrive + 2 * blockIdx.x], gen0, m);
    }
    __syncthreads();
    const uint32_t gen = gen_s;
    const uint64_t wait = wait_s != 0u ? (uint64_t)wait_s : kWaitTicks;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    if (blockIdx.x == 0) {
        // Collect every workgroup's maximum. Each thread watches the slots
        // t, t + 256, ...; every round re-reads all of its pending slots at
        // once, so their round trips overlap.
        constexpr int kPer = kMaxFusedGrid / kThreads;
        uint32_t mm = 0u;
        bool ok = true;
        uint32_t pending = 0u;
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            if ((int)threadIdx.x + k * kThreads < (int)gridDim.x)
                pending |= 1u << k;
        while (pending != 0u) {
            uint64_t w[kPer];
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                w[k] = (pending >> k) & 1u ? slot_load(&ws[kWsArrive + 2 * (threadIdx.x + k * kThreads)]) : 0u;
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                if (((pending >> k) & 1u) && (uint32_t)w[k] == gen) {
                    mm = max(mm, (uint32_t)(w[k] >> 32));
                    pending &= ~(1u << k);
                }
            }
            if (pending == 0u)
                break;
            if (__builtin_amdgcn_s_memrealtime() - t0 > wait) {
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(4);
        }
        if (threadIdx.x == 0)
            ok_s = 1u;
        __syncthreads();
        if (!ok)
            ok_s = 0u;
        const uint32_t r = workgroup_max(mm, red);
        if (ok_s == 0u) {
            result_s = direct_amax(p, red);
        } else if (threadIdx.x == 0) {
            result_s = r;
        }
        __syncthreads();
        const uint32_t amax = result_s;
        if (threadIdx.x == 0) {
            ws_store(&ws[kWsAmax], amax);
            if (ok_s == 0u)
                __hip_atomic_fetch_add(&ws[kWsSlow], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        for (int i = threadIdx.x; i < (int)gridDim.x; i += kThreads)
            slot_store(&ws[kWsRelease + 2 * i], gen, amax);
        __syncthreads();
        if (threadIdx.x == 0)
            ws_store(&ws[kWsGen], gen);
        return amax;
    }
    if (threadIdx.x == 0) {
        uint64_t w = slot_load(&ws[kWsRelease + 2 * blockIdx.x]);
        ok_s = 1u;
        while ((uint32_t)w != gen) {
            if (__builtin_amdgcn_s_memrealtime() - t0 > wait) {
                ok_s = 0u;
                break;
            }
            __builtin_amdgcn_s_sleep(4);
            w = slot_load(&ws[kWsRelease + 2 * blockIdx.x]);
        }
        result_s = (uint32_t)(w >> 32);
    }
    __syncthreads();
    if (ok_s == 0u) {
        const uint32_t amax = direct_amax(p, red);
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(&ws[kWsSlow], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return amax;
    }
    return result_s;
}

// Write the staged columnwise output of two vertically adjacent tiles (A at
// rows tile_r0.., B below it; B may be absent or ragged). Per column the
// pair covers 256 rows: 128 bytes of codes, one whole line, written by 8
// lanes as 16-byte streaming stores, and 16 scale bytes.
__device__ __forceinline__ void write_col_pair(const Params& p, int64_t tile_r0, int64_t tile_c0,
                                               const uint2* codes_a, const uint2* codes_b,
                                               const uint8_t* scales_a, const uint8_t* scales_b)
{
    typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
    const int64_t rows = p.rows, cols = p.cols;
    const int64_t pitch = rows >> 1;
    const bool wide = (pitch & 15) == 0;  // 16-byte chunks are aligned
#pragma unroll
    for (int k = 0; k < kTileC * 8 / kThreads; ++k) {
        const int q = k * kThreads + threadIdx.x;
        const int col = q >> 3, part = q & 7;  // part: 32 rows = two row blocks
        const int64_t c = tile_c0 + col, r = tile_r0 + part * 32;
        if (c >= cols || r >= rows)
            continue;
        const uint2* src = part < 4 ? codes_a : codes_b;
        const int swz = (col >> 3) & 7;
        const int rb0 = (2 * part) & 7;
        const uint2 lo = src[col * kRowBlocks + (rb0 ^ swz)];
        uint8_t* dst = p.codes_col + c * pitch + (r >> 1);
        if (r + 32 <= rows) {
            const uint2 hi = src[col * kRowBlocks + ((rb0 + 1) ^ swz)];
            if (wide) {
                __builtin_nontemporal_store(u32x4_nt{lo.x, lo.y, hi.x, hi.y},
                                            reinterpret_cast<u32x4_nt*>(dst));
            } else {
                *reinterpret_cast<uint2*>(dst) = lo;
                *reinterpret_cast<uint2*>(dst + 8) = hi;
            }
        } else {
            *reinterpret_cast<uint2*>(dst) = lo;  // ragged bottom: one row block
        }
    }
    // Scales: one column's 16 bytes (8 per tile) per thread.
    const int col = threadIdx.x;
    const int64_t c = tile_c0 + col;
    if (c < cols) {
        const int64_t spitch = rows >> 4;
        uint8_t* dst = p.scales_col + c * spitch + (tile_r0 >> 4);
        const int64_t nb64 = (rows - tile_r0) >> 4;
        const int nb = nb64 < 2 * kRowBlocks ? (int)nb64 : 2 * kRowBlocks;
        const uint2 sa = *reinterpret_cast<const uint2*>(&scales_a[col * kRowBlocks]);
        if (nb == 2 * kRowBlocks && ((reinterpret_cast<uintptr_t>(dst) & 15) == 0)) {
            const uint2 sb = *reinterpret_cast<const uint2*>(&scales_b[col * kRowBlocks]);
            *reinterpret_cast<uint4*>(dst) = make_uint4(sa.x, sa.y, sb.x, sb.y);
        } else {
            for (int b = 0; b < nb; ++b)
                dst[b] = b < kRowBlocks ? scales_a[col * kRowBlocks + b] : scales_b[col * kRowBlocks + b - kRowBlocks];
        }
    }
}

template <bool ROW, bool COL, bool SR>
__global__ __launch_bounds__(kThreads) void quantize_fused_kernel(Params p, uint32_t* ws)
{
    // Columnwise staging for the two tiles.
    __shared__ uint2 lds_codes[2][COL ? kTileC * kRowBlocks : 1];
    __shared__ uint8_t lds_scales[2][COL ? kTileC * kRowBlocks : 16];
    __shared__ float lds_rcp[128];

    // Two vertically adjacent tiles per workgroup (B below A), so a
    // column's codes of the pair form whole 128-byte lines.
    const int tra = 2 * (blockIdx.x / p.tiles_c), tc = blockIdx.x % p.tiles_c;
    const bool has_b = tra + 1 < p.tiles_r;  // uniform over the workgroup
    const ItemPos qa = item_pos(tra, tc, p.rows, p.cols);
    const ItemPos qb = item_pos(tra + 1, tc, p.rows, p.cols);
    uint32_t gen = 0u, wait = 0u;
    if (!p.amax_given && threadIdx.x == 0) {
        gen = call_generation(ws);
        wait = ws_load(&ws[kWsWait]);
    }
    uint4 va[16], vb[16];
    load_item(p, qa, va);
    if (has_b)
        load_item(p, qb, vb);

    // Block maxima while the data arrives; the workgroup's maximum follows.
    // (With stochastic rounding the row maxima wait until after the
    // exchange: holding them across it would cost occupancy.)
    constexpr bool kEarlyRows = ROW && !SR;
    BlockMax ba, bb;
    uint32_t m = 0u;
    if (qa.valid) {
        column_maxima(va, ba);
        if (kEarlyRows)
            row_maxima(va, qa.odd, ba);
        m = item_max(ba);
    }
    if (has_b && qb.valid) {
        column_maxima(vb, bb);
        if (kEarlyRows)
            row_maxima(vb, qb.odd, bb);
        m = max(m, item_max(bb));
    }
    const uint32_t amax_bits = p.amax_given ? __float_as_uint(*p.amax) : grid_max(m, gen, wait, ws, p);

    const ScaleCtx sc = scale_ctx(__uint_as_float(amax_bits));
    if (p.sg_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
        *p.sg_out = sc.sg;
    build_reciprocal_table(lds_rcp, sc.sg);
    __syncthreads();

    if (qa.valid) {
        if (ROW && !kEarlyRows)
            row_maxima(va, qa.odd, ba);
        compute_item<ROW, COL, false, SR, false>(p, qa, va, ba, sc, lds_rcp, lds_codes[0], lds_scales[0]);
    }
    if (has_b && qb.valid) {
        if (ROW && !kEarlyRows)
            row_maxima(vb, qb.odd, bb);
        compute_item<ROW, COL, false, SR, false>(p, qb, vb, bb, sc, lds_rcp, lds_codes[1], lds_scales[1]);
    }
    if (COL) {
        __syncthreads();
        write_col_pair(p, qa.tile_r0, qa.tile_c0, lds_codes[0], lds_codes[1], lds_scales[0], lds_scales[1]);
    }
}

// Workgroups of one fused kernel that fit on the device at once (cached).
template <bool ROW, bool COL, bool SR>
int fused_capacity()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 0;
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0)
        return c;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(quantize_fused_kernel<ROW, COL, SR>), kThreads, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    c = per_cu * cus;
    if (c > 0)
        cache[dev].store(c, std::memory_order_relaxed);
    return c;
}

template <bool ROW, bool COL, bool SR>
hipError_t launch_fused_variant(Params p, uint32_t* ws, hipStream_t stream, bool& launched)
{
    launched = false;
    const int grid = ((p.tiles_r + 1) / 2) * p.tiles_c;
    if (grid > kMaxFusedGrid || grid > fused_capacity<ROW, COL, SR>())
        return hipSuccess;
    hipLaunchKernelGGL((quantize_fused_kernel<ROW, COL, SR>), dim3(grid), dim3(kThreads), 0, stream, p,
                       ws);
    launched = true;
    return hipGetLastError();
}

// The paired-tile kernel with the amax given: no exchange, so any grid size.
template <bool ROW, bool COL, bool SR>
hipError_t launch_paired(Params p, hipStream_t stream)
{
    p.amax_given = 1;
    const int64_t grid = (int64_t)((p.tiles_r + 1) / 2) * p.tiles_c;
    hipLaunchKernelGGL((quantize_fused_kernel<ROW, COL, SR>), dim3((unsigned)grid), dim3(kThreads), 0,
                       stream, p, nullptr);
    return hipGetLastError();
}

template <bool ROW, bool COL, bool TWO_D, bool SR, bool RHT>
hipError_t launch_variant(const Params& p, hipStream_t stream)
{
    const int grid = p.tiles_r * p.tiles_c;
    hipLaunchKernelGGL((quantize_kernel<ROW, COL, TWO_D, SR, RHT>), dim3(grid), dim3(kThreads), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t stream)
{
    if (a.fused_amax) {
        Params p;
        p.x = a.x;
        p.rows = a.rows;
        p.cols = a.cols;
        p.amax = reinterpret_cast<const float*>(a.workspace);
        p.mask = 0u;
        p.seed_lo = (uint32_t)a.seed;
        p.seed_hi = (uint32_t)(a.seed >> 32);
        p.codes_row = a.codes_row;
        p.scales_row = a.scales_row;
        p.codes_col = a.codes_col;
        p.scales_col = a.scales_col;
        p.sg_out = a.global_scale;
        p.tiles_r = (int)((a.rows + kTileR - 1) / kTileR);
        p.tiles_c = (int)((a.cols + kTileC - 1) / kTileC);
        p.amax_given = 0;
        bool launched = false;
        hipError_t e;
        if (a.rowwise && a.colwise)
            e = a.sr ? launch_fused_variant<true, true, true>(p, a.workspace, stream, launched)
                     : launch_fused_variant<true, true, false>(p, a.workspace, stream, launched);
        else if (a.rowwise)
            e = a.sr ? launch_fused_variant<true, false, true>(p, a.workspace, stream, launched)
                     : launch_fused_variant<true, false, false>(p, a.workspace, stream, launched);
        else
            e = a.sr ? launch_fused_variant<false, true, true>(p, a.workspace, stream, launched)
                     : launch_fused_variant<false, true, false>(p, a.workspace, stream, launched);
        if (e != hipSuccess || launched)
            return e;
        // Too large to keep on chip: the two-pass path, amax into the workspace.
        float* amax = reinterpret_cast<float*>(a.workspace);
        e = launch_amax(a.x, a.rows * a.cols, amax, stream);
        if (e != hipSuccess)
            return e;
        QuantizeArgs b = a;
        b.fused_amax = false;
        b.amax = amax;
        return launch_quantize(b, stream);
    }
    Params p;
    p.x = a.x;
    p.rows = a.rows;
    p.cols = a.cols;
    p.amax = a.amax;
    p.mask = a.mask;
    p.seed_lo = (uint32_t)a.seed;
    p.seed_hi = (uint32_t)(a.seed >> 32);
    p.codes_row = a.codes_row;
    p.scales_row = a.scales_row;
    p.codes_col = a.codes_col;
    p.scales_col = a.scales_col;
    p.sg_out = a.global_scale;
    p.tiles_r = (int)((a.rows + kTileR - 1) / kTileR);
    p.tiles_c = (int)((a.cols + kTileC - 1) / kTileC);
    p.amax_given = 0;

    if (a.two_d) {
        if (a.rowwise && a.colwise)
            return launch_variant<true, true, true, false, false>(p, stream);
        if (a.rowwise)
            return launch_variant<true, false, true, false, false>(p, stream);
        return launch_variant<false, true, true, false, false>(p, stream);
    }
    if (a.rht) {
        // Hadamard path: columnwise only (validated by the caller).
        return a.sr ? launch_variant<false, true, false, true, true>(p, stream)
                    : launch_variant<false, true, false, false, true>(p, stream);
    }
    // Both layouts: the paired-tile kernel (whole-line columnwise stores,
    // here without its exchange) for round-to-nearest on tensors up to 2^25
    // elements (8192x4096: 25 against 26.6 us); the one-tile kernel on
    // larger ones (8192x14336: 78 against 88 us) and with stochastic
    // rounding at every size (8192x4096: 43 against 57 us; 8192x14336: 144
    // against 204 us).
    if (a.rowwise && a.colwise) {
        if (!a.sr && a.rows * a.cols <= ((int64_t)1 << 25))
            return launch_paired<true, true, false>(p, stream);
        return a.sr ? launch_variant<true, true, false, true, false>(p, stream)
                    : launch_variant<true, true, false, false, false>(p, stream);
    }
    // One layout: one tile per workgroup measured faster than the pairs.
    if (a.rowwise)
        return a.sr ? launch_variant<true, false, false, true, false>(p, stream)
                    : launch_variant<true, false, false, false, false>(p, stream);
    return a.sr ? launch_variant<false, true, false, true, false>(p, stream)
                : launch_variant<false, true, false, false, false>(p, stream);
}

}  // namespace nvfp4
