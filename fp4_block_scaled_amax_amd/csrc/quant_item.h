// Item-level NVFP4 quantization shared by the quantize kernels and the
// quantizing epilogue of the GEMM: the 128 x 256 tile geometry, a work
// item's position, block maxima, scale chain and encoding, and the writers
// of the staged columnwise output.
//
// A work item is 16 rows x 8 columns of bf16 held by one lane (sixteen
// 16-byte rows). Its columnwise blocks are the lane's own columns; its
// rowwise blocks span the lane pair (2k, 2k+1), which trade maxima and
// multipliers through DPP; a 2D tile is the lane pair's 16 x 16 elements.
// Rowwise codes go straight from registers to memory (128 contiguous bytes
// per row per half-wave); columnwise codes are staged in LDS.
#pragma once

#include "device.h"
#include "encode.h"

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
    float* amax_out;  // quantize_fused_kernel: optional copy of the amax it finds
};

// Map the workgroup index to a tile so that each XCD (workgroups are dealt
// round-robin over 8) walks a contiguous run of tiles; `vertical` makes the
// run go down the rows first.
__device__ __forceinline__ void tile_of_index(int t, int tiles_r, int tiles_c, bool vertical, int& tr,
                                              int& tc)
{
    const int nt = tiles_r * tiles_c;
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

__device__ __forceinline__ void tile_of_block(int tiles_r, int tiles_c, bool vertical, int& tr, int& tc)
{
    tile_of_index(blockIdx.x, tiles_r, tiles_c, vertical, tr, tc);
}

__device__ __forceinline__ bool finite_bits(float r)
{
    return (__float_as_uint(r) & 0x7F800000u) != 0x7F800000u;
}

// Row-and/or-column encoding of a whole item in 2x2 groups: elements
// (i, 2k), (i, 2k+1), (i+1, 2k), (i+1, 2k+1) are unpacked once and feed byte
// k of the two row words and byte (i/2 mod 4) of the two column words.
template <bool PAIR, int I>
__device__ __forceinline__ float row_multiplier(const float (&rm)[8])
{
    if (!PAIR)
        return rm[I & 7];
    return I < 8 ? from_even_lane(rm[I & 7]) : from_odd_lane(rm[I & 7]);
}

template <int MODE, int IP, bool ROW, bool COL, bool PAIR>
__device__ __forceinline__ void encode_row_pair(const uint4 (&v)[16], const float (&rm)[8],
                                                const float (&rc)[8], const uint4 (&draws)[16],
                                                uint32_t (&roww)[2], uint32_t (&colw)[8][2])
{
    constexpr int i = 2 * IP;
    constexpr int cb = IP & 3;     // byte within the column word
    constexpr int ch = IP >> 2;    // which column word (rows 0..7 or 8..15)
    roww[0] = MODE == kEncSr ? 0u : fresh_word();
    roww[1] = MODE == kEncSr ? 0u : fresh_word();
    if (MODE != kEncSr && COL && cb == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            colw[j][ch] = fresh_word();
    }
    // The rare encoders (non-finite multipliers, software rounding) take
    // their words through an empty asm statement: the compiler then cannot
    // share their unpacking with the common encoder's and hoist it above the
    // branch between them, which would keep every unpacked value of the item
    // live at once.
#define NVFP4_GROUP(K)                                                                      \
    {                                                                                       \
        uint32_t w0 = word_at(v[i], K), w1 = word_at(v[i + 1], K);                          \
        if (MODE == kEncHwSafe || MODE == kEncSr)                                           \
            asm volatile("" : "+v"(w0), "+v"(w1)); /* see below */                          \
        const float a = bf16_lo(w0), b = bf16_hi(w0), c = bf16_lo(w1), d = bf16_hi(w1);     \
        uint32_t ha = 0u, hb = 0u, hc = 0u, hd = 0u;                                        \
        if (is_sr(MODE)) {                                                                  \
            ha = sr_input<MODE>(draws[i], 2 * K);                                           \
            hb = sr_input<MODE>(draws[i], 2 * K + 1);                                       \
            hc = sr_input<MODE>(draws[i + 1], 2 * K);                                       \
            hd = sr_input<MODE>(draws[i + 1], 2 * K + 1);                                   \
        }                                                                                   \
        if (ROW) {                                                                          \
            roww[0] = put_pair<MODE, K>(roww[0], a, b, rr0, ha, hb);                        \
            roww[1] = put_pair<MODE, K>(roww[1], c, d, rr1, hc, hd);                        \
        }                                                                                   \
        if (COL) {                                                                          \
            colw[2 * K][ch] = put_pair<MODE, cb>(colw[2 * K][ch], a, c, rc[2 * K], ha, hc);         \
            colw[2 * K + 1][ch] = put_pair<MODE, cb>(colw[2 * K + 1][ch], b, d, rc[2 * K + 1], hb, hd); \
        }                                                                                   \
    }
    const float rr0 = ROW ? row_multiplier<PAIR, i>(rm) : 0.0f;
    const float rr1 = ROW ? row_multiplier<PAIR, i + 1>(rm) : 0.0f;
    NVFP4_GROUP(0) NVFP4_GROUP(1) NVFP4_GROUP(2) NVFP4_GROUP(3)
#undef NVFP4_GROUP
}

template <int MODE, bool ROW, bool COL, bool PAIR, int IP0, int IP1>
__device__ __forceinline__ void encode_item(const uint4 (&v)[16], const float (&rm)[8],
                                            const float (&rc)[8], const uint4 (&draws)[16],
                                            uint8_t* row_dst, int64_t row_pitch,
                                            uint32_t (&colw)[8][2])
{
    // A half-wave's rowwise codes of one row are a whole 128-byte line:
    // stream them past the caches.
    uint32_t roww[2];
#define NVFP4_ROWS(IP)                                                                       \
    if constexpr (IP >= IP0 && IP < IP1) {                                                   \
        encode_row_pair<MODE, IP, ROW, COL, PAIR>(v, rm, rc, draws, roww, colw);             \
        if (ROW) {                                                                           \
            uint8_t* d = row_dst + (2 * IP) * row_pitch;                                     \
            __builtin_nontemporal_store(roww[0], reinterpret_cast<uint32_t*>(d));            \
            __builtin_nontemporal_store(roww[1], reinterpret_cast<uint32_t*>(d + row_pitch)); \
        }                                                                                    \
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

__device__ __forceinline__ ItemPos item_pos(int tr, int tc, int64_t rows, int64_t cols, int tid)
{
    ItemPos q;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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

__device__ __forceinline__ ItemPos item_pos(int tr, int tc, int64_t rows, int64_t cols)
{
    return item_pos(tr, tc, rows, cols, threadIdx.x);
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

// The same loads, unconditional: an item outside the tensor reads the first
// item instead (always present, as rows and cols are positive multiples of
// 16), so the data is defined on every path and no join of loaded and
// undefined values splits its registers; the caller skips such items.
__device__ __forceinline__ void load_item_any(const Params& p, const ItemPos& q, uint4 (&v)[16])
{
    const uint16_t* src = p.x + (q.valid ? q.r0 * p.cols + q.c0 : 0);
#pragma unroll
    for (int i = 0; i < 16; ++i)
        v[i] = load16_stream(src + i * p.cols);
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

// Row maxima from each row's packed maxima of the lane's 4 column pairs.
// They trade halves through DPP with the pair lane: every lane of the pair
// must be active (both are, as the item validity is pairwise).
__device__ __forceinline__ void row_maxima_of(const uint32_t (&pm)[16], bool odd, BlockMax& bm)
{
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

__device__ __forceinline__ void row_maxima(const uint4 (&v)[16], bool odd, BlockMax& bm)
{
    uint32_t pm[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        pm[i] = pk_max_u16(pk_max_u16(v[i].x & 0x7FFF7FFFu, v[i].y & 0x7FFF7FFFu),
                           pk_max_u16(v[i].z & 0x7FFF7FFFu, v[i].w & 0x7FFF7FFFu));
    row_maxima_of(pm, odd, bm);
}

// Column and row maxima in one pass: each magnitude word feeds both at
// once, so the masked words are never all live together.
__device__ __forceinline__ void block_maxima(const uint4 (&v)[16], bool odd, BlockMax& bm)
{
    uint32_t pm[16];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        bm.col[k] = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t w0 = v[i].x & 0x7FFF7FFFu, w1 = v[i].y & 0x7FFF7FFFu;
        const uint32_t w2 = v[i].z & 0x7FFF7FFFu, w3 = v[i].w & 0x7FFF7FFFu;
        bm.col[0] = pk_max_u16(bm.col[0], w0);
        bm.col[1] = pk_max_u16(bm.col[1], w1);
        bm.col[2] = pk_max_u16(bm.col[2], w2);
        bm.col[3] = pk_max_u16(bm.col[3], w3);
        pm[i] = pk_max_u16(pk_max_u16(w0, w1), pk_max_u16(w2, w3));
    }
    row_maxima_of(pm, odd, bm);
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
// fold (uniform): the multipliers in lds_rcp carry a power of two
// (kFoldFactor): 1/4 of the transform (its outputs then stay unscaled) and,
// with stochastic rounding, the converter's 2^23 operand scaling; the
// caller has checked that this is exact (fold_quarter_ok, fold_sr_scale_ok).
template <bool SR, bool RHT>
constexpr float kFoldFactor = SR ? (RHT ? 0x1p21f : 0x1p23f) : (RHT ? 0.25f : 1.0f);

// Stochastic-rounding draws of an item: one Philox call per row covers the
// item's 8 consecutive flat indices. They do not depend on the data, so the
// kernels compute them right after issuing the item's loads; `pin` makes
// them complete at that point (an empty statement that uses them, then a
// scheduling barrier that keeps the data's first uses below), so they run
// while the loads are in flight.
__device__ __forceinline__ void item_draws(const Params& p, const ItemPos& q, uint4 (&draws)[16], bool pin)
{
    const uint64_t flat0 = (uint64_t)(q.r0 * p.cols + q.c0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint64_t qq = (flat0 + (uint64_t)i * (uint64_t)p.cols) >> 3;
        draws[i] = philox4x32_10((uint32_t)qq, (uint32_t)(qq >> 32), p.seed_lo, p.seed_hi);
    }
    if (pin) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            asm volatile("" ::"v"(draws[i].x), "v"(draws[i].y), "v"(draws[i].z), "v"(draws[i].w));
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <bool ROW, bool COL, bool TWO_D, bool SR, bool RHT>
__device__ __forceinline__ void compute_item(const Params& p, const ItemPos& q,
                                             const uint4 (&v)[16], const BlockMax& bm,
                                             const uint4 (&draws)[16], const ScaleCtx& sc,
                                             const float* lds_rcp, uint2* lds_codes,
                                             uint8_t* lds_scales, bool fold)
{
    const int64_t cols = p.cols;
    const int64_t r0 = q.r0, c0 = q.c0;
    const int rb = q.rb, cg = q.cg;
    const bool odd = q.odd;

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
                // z = H D x. Every z is a multiple of 2^-133 (see
                // fold_quarter_ok), so y = z / 4 is exact and max |y| =
                // max |z| / 4. Largest magnitude from the raw bits: the
                // signed maximum finds the largest positive value, the
                // unsigned one the negative value of largest magnitude.
                hadamard16(y);
                int32_t mi = 0;
                uint32_t mu = 0u;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    mi = max(mi, (int32_t)__float_as_uint(y[i]));
                    mu = max(mu, __float_as_uint(y[i]));
                }
                m = __float_as_uint(0.25f * __uint_as_float(max((uint32_t)mi, mu & 0x7FFFFFFFu)));
                if (!fold) {  // the 1/4 is not in the multipliers
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        y[i] = 0.25f * y[i];
                }
            } else {
                m = (j & 1) ? half_bits<1>(bm.col[j >> 1]) : half_bits<0>(bm.col[j >> 1]);
            }
            const uint32_t byte = scale_byte(m, sc);
            const float r = lds_rcp[byte];
            uint2 words;
            // Stochastic rounding takes the hardware converter when the
            // multipliers carry its 2^23 (the common case); otherwise, or for
            // a block whose multiplier is not finite, the software encoder.
            if (SR)
                words = (fold && __all(finite_bits(r)))
                            ? encode_column16<kEncSrHwScaled>(y, r, draws, j)
                            : encode_column16<kEncSr>(y, fold ? r * 0x1p-23f : r, draws, j);
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
    float rc[8];  // columnwise multipliers (1D), or the tile's (2D)
    float rm[8];  // this lane's rowwise multipliers (1D: rows 0..7 on even
                  // lanes, 8..15 on odd ones), or the tile's (2D)
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
        for (int i = 0; i < 8; ++i)
            rm[i] = r;
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
            if constexpr (COL) {
                // Rows and columns: one block at a time, through this
                // thread's own 16 words of the columnwise staging (untouched
                // until its encode), so that this rare path needs few
                // registers of its own.
                uint32_t* const stage = reinterpret_cast<uint32_t*>(lds_codes);
                const int base = 2 * ((cg * 8) * kRowBlocks + (rb ^ (cg & 7)));
                auto word = [&](int n) -> uint32_t& {
                    return stage[base + 2 * kRowBlocks * (n >> 1) + (n & 1)];
                };
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    word(n) = bm.col[n];
                    word(4 + n) = bm.row[n];
                }
#pragma unroll 1
                for (int b = 0; b < 16; ++b) {
                    // b < 8: column block b; b >= 8: row block b - 8.
                    const uint32_t pk = word(b >> 1);
                    const uint32_t byte = scale_byte((b & 1) ? (pk & 0xFFFF0000u) : (pk << 16), sc);
                    reinterpret_cast<uint8_t*>(&word(8 + (b >> 2)))[b & 3] = (uint8_t)byte;
                    mb = max(mb, byte);
                }
                const uint32_t cw0 = word(8), cw1 = word(9), rw0 = word(10), rw1 = word(11);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    col_byte[j] = ((j < 4 ? cw0 : cw1) >> (8 * (j & 3))) & 0xFFu;
                    row_byte[j] = ((j < 4 ? rw0 : rw1) >> (8 * (j & 3))) & 0xFFu;
                }
            } else {
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
            for (int j = 0; j < 8; ++j) {
                rc[j] = lds_rcp[col_byte[j]];
                lds_scales[(cg * 8 + j) * kRowBlocks + rb] = (uint8_t)col_byte[j];
            }
        }
        if (ROW) {
            // Even lanes own rows 0..7 of the pair's blocks, odd lanes 8..15.
            const int64_t srow0 = r0 + (odd ? 8 : 0);
            uint8_t* sdst = p.scales_row + srow0 * (cols >> 4) + (c0 >> 4);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                sdst[k * (cols >> 4)] = (uint8_t)row_byte[k];
                rm[k] = lds_rcp[row_byte[k]];
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
            for (int k = 0; k < 8; ++k)
                fin = fin && (!ROW || finite_bits(rm[k]));  // the wave's vote covers the pair
        }
    }
    uint32_t colw[8][2];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        colw[j][0] = colw[j][1] = 0u;
    uint8_t* row_dst = ROW ? p.codes_row + r0 * (cols >> 1) + (c0 >> 1) : nullptr;
    const int64_t row_pitch = cols >> 1;
    constexpr bool kPair = !TWO_D;
    const bool all_fin = __all(fin);
    uint32_t* const lds_words = reinterpret_cast<uint32_t*>(lds_codes);
    // Rows 0..7, then 8..15: each half's column words go to the staging as
    // soon as they are complete.
#define NVFP4_ENC(MODE, H) \
    encode_item<MODE, ROW, COL, kPair, 4 * H, 4 * H + 4>(v, rm, rc, draws, row_dst, row_pitch, colw)
#define NVFP4_HALF(H)                                                                              \
    {                                                                                              \
        if (SR && all_fin)                                                                         \
            NVFP4_ENC(kEncSrHw, H);                                                                \
        else if (SR)                                                                               \
            NVFP4_ENC(kEncSr, H);                                                                  \
        else if (all_fin)                                                                          \
            NVFP4_ENC(kEncHw, H);                                                                  \
        else                                                                                       \
            NVFP4_ENC(kEncHwSafe, H);                                                              \
        if (COL) {                                                                                 \
            _Pragma("unroll") for (int j = 0; j < 8; ++j)                                          \
                lds_words[2 * ((cg * 8 + j) * kRowBlocks + (rb ^ (cg & 7))) + H] = colw[j][H];   \
        }                                                                                          \
    }
    NVFP4_HALF(0)
    NVFP4_HALF(1)
#undef NVFP4_HALF
#undef NVFP4_ENC
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


// Write the staged columnwise output of two vertically adjacent tiles (A at
// rows tile_r0.., B below it; B may be absent or ragged). Per column the
// pair covers 256 rows: 128 bytes of codes, one whole line, written by 8
// lanes as 16-byte streaming stores, and 16 scale bytes. tid: the thread's
// index among the NT writers (a caller inside a loop can pass an opaque copy,
// so that the addresses are not computed ahead of the loop).
template <int NT = kThreads>
__device__ __forceinline__ void write_col_pair(const Params& p, int64_t tile_r0, int64_t tile_c0,
                                               const uint2* codes_a, const uint2* codes_b,
                                               const uint8_t* scales_a, const uint8_t* scales_b,
                                               int tid = (int)threadIdx.x)
{
    typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
    const int64_t rows = p.rows, cols = p.cols;
    const int64_t pitch = rows >> 1;
    const bool wide = (pitch & 15) == 0;  // 16-byte chunks are aligned
#pragma unroll
    for (int k = 0; k < kTileC * 8 / NT; ++k) {
        const int q = k * NT + tid;
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
    const int col = tid;
    const int64_t c = tile_c0 + col;
    if (col < kTileC && c < cols) {
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

}  // namespace

}  // namespace nvfp4
