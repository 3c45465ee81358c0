// MXFP4 quantization and dequantization: E2M1 codes with one E8M0
// (power-of-two) scale per 32 elements and no tensor scale -- the
// comparator format, which gfx950's block-scaled matrix cores take natively.
//
// Scale rule (the OCP microscaling shared exponent): X = 2^(floor(log2 amax)
// - 2) for the block maximum amax, 2 being E2M1's largest exponent, clamped
// to E8M0's range; a block holding a NaN or an infinity gets the NaN byte
// 0xFF. For a binary32 maximum with exponent field E the byte is
// max(E - 2, 0) (E = 0, a zero or subnormal maximum, clamps to 2^-127), so
// the rule is two integer operations on the maximum's bit pattern. Elements
// are x * 2^-(byte - 127) -- exact where it matters, the multiplier being a
// normal power of two -- rounded to E2M1 by the gfx950 converter with a unit
// scale (nearest even, saturating at 6). In a NaN-scale block only the
// elements' sign bits are kept, so every code has magnitude 0.
//
// Two kernels:
//   - rowwise alone, without LDS (mx_quantize_rows_kernel);
//   - any columnwise output (mx_quantize_pair_kernel): 512 threads take a
//     256 x 256 block, one 16 x 8 work item per thread in registers; a
//     columnwise block is one column of lanes l and l ^ 32, a rowwise block
//     one row of a lane quad; with the Hadamard transform (columnwise only)
//     each column of an item, one 16-row group, is sign-flipped on the packed
//     words, butterflied and scaled by 1/4 in registers exactly as the NVFP4
//     columnwise path does; the columnwise codes are staged in LDS and leave
//     as whole 128-byte lines.
#include "device.h"
#include "kernels.h"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;

// E8M0 byte of a block from the bit pattern of its maximum |x| (binary32).
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t m)
{
    if (m >= 0x7F800000u)
        return 0xFFu;
    const int e = (int)(m >> 23) - 2;
    return e > 0 ? (uint32_t)e : 0u;
}

// Multiplier 2^(127 - byte) for a finite byte (<= 252 here), 1 for 0xFF.
__device__ __forceinline__ float mx_inverse_scale(uint32_t byte)
{
    return byte == 0xFFu ? 1.0f : __uint_as_float((254u - byte) << 23);
}

// Two binary32 values -> one byte of codes (a in the low nibble) at byte SEL.
template <int SEL>
__device__ __forceinline__ uint32_t mx_pair(uint32_t old, float a, float b)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// 8 values -> one 32-bit word of codes.
__device__ __forceinline__ uint32_t mx_word(const float (&v)[8])
{
    uint32_t w = 0u;
    w = mx_pair<0>(w, v[0], v[1]);
    w = mx_pair<1>(w, v[2], v[3]);
    w = mx_pair<2>(w, v[4], v[5]);
    w = mx_pair<3>(w, v[6], v[7]);
    return w;
}

// ------------------------------------------------------------ paired tiles
// Columnwise output without the transform (with or without the rowwise
// layout): one workgroup of 512 threads takes a 256 x 256 block, one work
// item of 16 rows x 8 columns per thread, loaded straight into registers.
// Lane l of wave w holds rows 16 (2w + (l >> 5)) .. +15 and columns
// 8 (l & 31) .. +7 of the block, so a columnwise block (32 rows) is one
// column of lanes l and l ^ 32 (a permlane32 swap joins their maxima) and a
// rowwise block (32 columns) is one row of the lane quad 4q .. 4q + 3 (two
// DPP steps). Rowwise codes leave straight from registers (a half-wave
// writes one 128-byte row segment); columnwise codes are staged in LDS and
// leave as whole 128-byte lines per column.
constexpr int kPairThreads = 512;
constexpr int kPairRows = 256;
constexpr int kPairCols = 256;

// A word whose every byte is written before use (an empty asm statement
// defines the register without an instruction).
__device__ __forceinline__ uint32_t mx_fresh()
{
    uint32_t w;
    asm volatile("" : "=v"(w));
    return w;
}

// Scale byte n of four packed in a word.
__device__ __forceinline__ uint32_t packed_byte(const uint32_t (&w)[4], int n)
{
    return (w[n >> 2] >> (8 * (n & 3))) & 0xFFu;
}

// The value of lane K of each lane quad, on all four lanes.
template <int K>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, K | (K << 2) | (K << 4) | (K << 6), 0xF, 0xF, false);
}

// Row I's multiplier (and, SAFE, its mask): lane I & 3 of the quad holds
// rows 4m + (I & 3) in slot m = I >> 2.
template <int I>
__device__ __forceinline__ float row_mult(const float (&rm)[4])
{
    return __uint_as_float(quad_bcast<I & 3>(__float_as_uint(rm[I >> 2])));
}
template <int I>
__device__ __forceinline__ uint32_t row_keep(uint32_t rown)
{
    const uint32_t own = ((rown >> (8 * (I >> 2))) & 0xFFu) == 0xFFu ? 0x80008000u : 0xFFFFFFFFu;
    return quad_bcast<I & 3>(own);
}

// Encode rows 2 IP, 2 IP + 1 of an item: byte K of the two row words
// (columns 2K, 2K+1) and byte IP & 3 of column words 2K, 2K+1. SAFE: some
// blocks may have a non-finite maximum (byte 0xFF, multiplier 1), whose
// values become signed zeros; the masks come from the packed row bytes rb
// (rows 4m .. 4m + 3 in word m) and column bytes cb (columns likewise).
template <int IP, bool ROW, bool SAFE>
__device__ __forceinline__ void mx_pair_rows(const uint4 (&v)[16], const float (&rm)[4], const float (&rc)[8],
                                             uint32_t rown, const uint32_t (&cbt)[4],
                                             uint32_t (&roww)[2], uint32_t (&colw)[8][2])
{
    constexpr int i = 2 * IP, cb = IP & 3, ch = IP >> 2;
    uint32_t kr0 = 0xFFFFFFFFu, kr1 = 0xFFFFFFFFu;
    float rr0 = 1.0f, rr1 = 1.0f;
    if (ROW) {
        rr0 = row_mult<i>(rm);
        rr1 = row_mult<i + 1>(rm);
        if (SAFE) {
            kr0 = row_keep<i>(rown);
            kr1 = row_keep<i + 1>(rown);
        }
    }
    if (ROW) {
        roww[0] = mx_fresh();
        roww[1] = mx_fresh();
    }
    if (cb == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            colw[j][ch] = mx_fresh();
    }
#define MX_GROUP(K)                                                                                     \
    {                                                                                                   \
        uint32_t w0 = word_at(v[i], K), w1 = word_at(v[i + 1], K);                                      \
        uint32_t kcw = 0xFFFFFFFFu;                                                                     \
        if (SAFE) {                                                                                     \
            asm volatile("" : "+v"(w0), "+v"(w1));                                                      \
            kcw = (packed_byte(cbt, 2 * K) == 0xFFu ? 0x8000u : 0xFFFFu) |                              \
                  (packed_byte(cbt, 2 * K + 1) == 0xFFu ? 0x80000000u : 0xFFFF0000u);                   \
        }                                                                                               \
        if (ROW) {                                                                                      \
            const uint32_t x0 = SAFE ? (w0 & kr0) : w0, x1 = SAFE ? (w1 & kr1) : w1;                    \
            roww[0] = mx_pair<K>(roww[0], bf16_lo(x0) * rr0, bf16_hi(x0) * rr0);                        \
            roww[1] = mx_pair<K>(roww[1], bf16_lo(x1) * rr1, bf16_hi(x1) * rr1);                        \
        }                                                                                               \
        const uint32_t y0 = SAFE ? (w0 & kcw) : w0, y1 = SAFE ? (w1 & kcw) : w1;                        \
        colw[2 * K][ch] = mx_pair<cb>(colw[2 * K][ch], bf16_lo(y0) * rc[2 * K], bf16_lo(y1) * rc[2 * K]); \
        colw[2 * K + 1][ch] =                                                                           \
            mx_pair<cb>(colw[2 * K + 1][ch], bf16_hi(y0) * rc[2 * K + 1], bf16_hi(y1) * rc[2 * K + 1]);   \
    }
    MX_GROUP(0) MX_GROUP(1) MX_GROUP(2) MX_GROUP(3)
#undef MX_GROUP
}

template <bool ROW, bool SAFE>
__device__ __forceinline__ void mx_encode_item(const uint4 (&v)[16], const float (&rm)[4], const float (&rc)[8],
                                               uint32_t rown, const uint32_t (&cbt)[4],
                                               uint8_t* row_dst, int64_t row_pitch, uint32_t* lds_words,
                                               int col_slot)
{
    uint32_t roww[2];
    uint32_t colw[8][2];
#define MX_ROWS(IP)                                                                                  \
    mx_pair_rows<IP, ROW, SAFE>(v, rm, rc, rown, cbt, roww, colw);                                 \
    if (ROW) {                                                                                       \
        __builtin_nontemporal_store(roww[0], reinterpret_cast<uint32_t*>(row_dst + (2 * IP) * row_pitch)); \
        __builtin_nontemporal_store(roww[1], reinterpret_cast<uint32_t*>(row_dst + (2 * IP + 1) * row_pitch)); \
    }
#define MX_HALF(H)                                                                                   \
    _Pragma("unroll") for (int j = 0; j < 8; ++j)                                                    \
        lds_words[2 * (col_slot + 16 * j) + H] = colw[j][H];  /* column 8 cg + j */
    MX_ROWS(0) MX_ROWS(1) MX_ROWS(2) MX_ROWS(3)
    MX_HALF(0)
    MX_ROWS(4) MX_ROWS(5) MX_ROWS(6) MX_ROWS(7)
    MX_HALF(1)
#undef MX_HALF
#undef MX_ROWS
}

// Columnwise with the transform, in the paired kernel: column j of an item
// (its 16 rows are one 16-row group of the transform) is sign-flipped on the
// packed words, butterflied and scaled by 1/4 in registers, its half-block
// maximum joined with lane l ^ 32's, then scaled and encoded into two code
// words (rows 0..7, 8..15), one column at a time.
__device__ __forceinline__ void mx_rht_column(const uint4 (&v)[16], int j, uint32_t mask, uint32_t& byte,
                                              uint32_t (&words)[2])
{
    float y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t w = word_at(v[i], j >> 1) ^ rht_row_sign(mask, i);
        y[i] = (j & 1) ? bf16_hi(w) : bf16_lo(w);
    }
    rht16_signed(y);
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        m = max(m, __float_as_uint(y[i]) & 0x7FFFFFFFu);
    const auto sw = __builtin_amdgcn_permlane32_swap(m, m, false, false);
    m = max(sw[0], sw[1]);  // the whole 32-row block
    byte = mx_scale_byte(m);
    const float inv = mx_inverse_scale(byte);
    const uint32_t keep = byte == 0xFFu ? 0x80000000u : 0xFFFFFFFFu;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float f[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            f[k] = __uint_as_float(__float_as_uint(y[8 * h + k]) & keep) * inv;
        words[h] = mx_word(f);
    }
}

template <bool ROW, bool RHT>
__global__ __launch_bounds__(kPairThreads) __attribute__((amdgpu_waves_per_eu(4)))
void mx_quantize_pair_kernel(MxQuantizeArgs p, int blocks_c)
{
    static_assert(!(ROW && RHT), "the transform is columnwise only");
    __shared__ uint2 lds_codes[kPairCols * 16];    // [column][16-row group, swizzled]
    __shared__ uint8_t lds_scales[kPairCols * 8];  // [column][32-row block]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cg = lane & 31;
    const int rg = 2 * wave + (lane >> 5);  // 16-row group of the block, 0..15
    const int64_t br0 = (int64_t)(blockIdx.x / blocks_c) * kPairRows;
    const int64_t bc0 = (int64_t)(blockIdx.x % blocks_c) * kPairCols;
    const int64_t r0 = br0 + 16 * rg, c0 = bc0 + 8 * cg;
    // rows % 32 == 0 and cols % 8 == 0 (32 with the rowwise layout): an item
    // is whole or absent, and lanes l, l ^ 32 and each quad agree. Every lane
    // takes part in the cross-lane steps; an absent item loads the first one
    // (always present) and stores nothing.
    const bool valid = r0 < p.rows && c0 < p.cols;
    uint4 v[16];
    {
        const uint16_t* src = p.x + (valid ? r0 * p.cols + c0 : 0);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            v[i] = load16_stream(src + i * p.cols);
    }

    const int col_slot = (8 * cg) * 16 + (rg ^ (cg & 15));
    uint32_t* const lds_words = reinterpret_cast<uint32_t*>(lds_codes);
    if constexpr (RHT) {
        // Every lane takes part (the swap joins lanes l and l ^ 32); absent
        // items stage nothing.
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t byte, words[2];
            mx_rht_column(v, j, p.mask, byte, words);
            if (valid) {
                lds_words[2 * (col_slot + 16 * j)] = words[0];
                lds_words[2 * (col_slot + 16 * j) + 1] = words[1];
            }
            if (lane < 32)
                lds_scales[(8 * cg + j) * 8 + (rg >> 1)] = (uint8_t)byte;
        }
    } else {
    // Block maxima as |bf16| patterns: colm[k] packs columns 2k, 2k+1 over
    // the item's 16 rows; rowm[k] packs rows 2k, 2k+1 over its 8 columns.
    uint32_t colm[4] = {0u, 0u, 0u, 0u};
    uint32_t rowm[8];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t w0 = v[i].x & 0x7FFF7FFFu, w1 = v[i].y & 0x7FFF7FFFu;
        const uint32_t w2 = v[i].z & 0x7FFF7FFFu, w3 = v[i].w & 0x7FFF7FFFu;
        colm[0] = pk_max_u16(colm[0], w0);
        colm[1] = pk_max_u16(colm[1], w1);
        colm[2] = pk_max_u16(colm[2], w2);
        colm[3] = pk_max_u16(colm[3], w3);
        if (ROW) {
            const uint32_t pm = pk_max_u16(pk_max_u16(w0, w1), pk_max_u16(w2, w3));
            const uint32_t m = max(pm & 0xFFFFu, pm >> 16);
            rowm[i >> 1] = (i & 1) ? (rowm[i >> 1] | (m << 16)) : m;
        }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const auto r = __builtin_amdgcn_permlane32_swap(colm[k], colm[k], false, false);
        colm[k] = pk_max_u16(r[0], r[1]);  // this lane's and lane l ^ 32's
    }
    if (ROW) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint32_t t = rowm[k];
            t = pk_max_u16(t, (uint32_t)__builtin_amdgcn_mov_dpp((int)t, 0xB1, 0xF, 0xF, false));  // lane ^ 1
            t = pk_max_u16(t, (uint32_t)__builtin_amdgcn_mov_dpp((int)t, 0x4E, 0xF, 0xF, false));  // lane ^ 2
            rowm[k] = t;
        }
    }

    // Scale bytes and multipliers: all eight column blocks; of the 16
    // rowwise blocks, which the four lanes of a quad share, lane t computes
    // and stores rows 4m + t (slot m) and lends them to the others by DPP.
    float rc[8], rm[4];
    uint32_t cbytes[4] = {0u, 0u, 0u, 0u};  // columns 4m .. 4m + 3 in word m (m < 2)
    uint32_t rown = 0u;                      // rows 4m + t in byte m
    bool any_ff = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t bits = (j & 1) ? (colm[j >> 1] & 0xFFFF0000u) : (colm[j >> 1] << 16);
        const uint32_t byte = mx_scale_byte(bits);
        rc[j] = mx_inverse_scale(byte);
        any_ff = any_ff || byte == 0xFFu;
        cbytes[j >> 2] |= byte << (8 * (j & 3));
    }
    if (ROW) {
        const int t = lane & 3;
        // row 4m + t: half t & 1 of rowm[2m + (t >> 1)], picked by masks (a
        // select here becomes an indexed load from a stack copy of rowm)
        const uint32_t hi_word = 0u - (uint32_t)(t >> 1);
        const int half_shift = (t & 1) ? 0 : 16;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t w = (rowm[2 * m] & ~hi_word) | (rowm[2 * m + 1] & hi_word);
            const uint32_t bits = (w << half_shift) & 0xFFFF0000u;
            const uint32_t byte = mx_scale_byte(bits);
            rm[m] = mx_inverse_scale(byte);
            any_ff = any_ff || byte == 0xFFu;
            rown |= byte << (8 * m);
        }
        if (valid) {
            uint8_t* sdst = p.scales_row + (r0 + t) * (p.cols >> 5) + (c0 >> 5);
#pragma unroll
            for (int m = 0; m < 4; ++m)
                sdst[4 * m * (p.cols >> 5)] = (uint8_t)(rown >> (8 * m));
        }
    } else {
#pragma unroll
        for (int m = 0; m < 4; ++m)
            rm[m] = 1.0f;
    }
    if (lane < 32) {  // the lower lane of each l, l ^ 32 pair stages the column scales
#pragma unroll
        for (int j = 0; j < 8; ++j)
            lds_scales[(8 * cg + j) * 8 + (rg >> 1)] = (uint8_t)packed_byte(cbytes, j);
    }

    uint8_t* const row_dst = ROW ? p.codes_row + r0 * (p.cols >> 1) + (c0 >> 1) : nullptr;
    if (valid) {
        if (__any(any_ff))
            mx_encode_item<ROW, true>(v, rm, rc, rown, cbytes, row_dst, p.cols >> 1, lds_words, col_slot);
        else
            mx_encode_item<ROW, false>(v, rm, rc, rown, cbytes, row_dst, p.cols >> 1, lds_words, col_slot);
    }
    }  // not RHT
    __syncthreads();

    // Columnwise codes: per column 256 rows = 128 bytes, written by 8 lanes
    // as 16-byte streaming stores (rows % 32 == 0 keeps every chunk whole and
    // aligned).
    typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
    const int64_t pitch = p.rows >> 1;
#pragma unroll
    for (int k = 0; k < kPairCols * 8 / kPairThreads; ++k) {
        const int q = k * kPairThreads + threadIdx.x;
        const int col = q >> 3, part = q & 7;  // part: rows 32 part .. + 31
        const int64_t c = bc0 + col, r = br0 + 32 * part;
        if (c < p.cols && r < p.rows) {
            const int swz = (col >> 3) & 15;
            const uint2 lo = lds_codes[col * 16 + ((2 * part) ^ swz)];
            const uint2 hi = lds_codes[col * 16 + ((2 * part + 1) ^ swz)];
            __builtin_nontemporal_store(u32x4_nt{lo.x, lo.y, hi.x, hi.y},
                                        reinterpret_cast<u32x4_nt*>(p.codes_col + c * pitch + (r >> 1)));
        }
    }
    // Columnwise scales: one column's 8 bytes per thread.
    if (threadIdx.x < kPairCols) {
        const int col = threadIdx.x;
        const int64_t c = bc0 + col;
        if (c < p.cols) {
            const int64_t spitch = p.rows >> 5;
            uint8_t* dst = p.scales_col + c * spitch + (br0 >> 5);
            const int64_t nb64 = (p.rows - br0) >> 5;
            const int nb = nb64 < 8 ? (int)nb64 : 8;
            const uint8_t* src = &lds_scales[col * 8];
            if (nb == 8 && (reinterpret_cast<uintptr_t>(dst) & 7) == 0) {
                *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
            } else {
                for (int b = 0; b < nb; ++b)
                    dst[b] = src[b];
            }
        }
    }
}

// Rowwise only, without LDS: a rowwise block is 32 consecutive elements of
// the row-major tensor (cols is a multiple of 32), so a lane takes 16 bytes
// (8 elements) and a quad of consecutive lanes holds one block; the block
// maximum is two DPP steps within the quad. Codes leave as one 32-bit store
// per lane (256 contiguous bytes per wave), the scale byte from the quad's
// first lane. U vectors in flight per thread.
template <int U>
__global__ __launch_bounds__(kThreads) void mx_quantize_rows_kernel(const uint16_t* __restrict__ x, int64_t nvec,
                                                                   uint8_t* __restrict__ codes,
                                                                   uint8_t* __restrict__ scales)
{
    // Each pass of a workgroup takes U * 256 consecutive vectors, one
    // contiguous span (its U loads per thread are 4 KB runs side by side),
    // read past the caches.
    constexpr int64_t stride = kThreads;
    const bool first = (threadIdx.x & 3) == 0;
    for (int64_t v0 = (int64_t)blockIdx.x * kThreads * U + threadIdx.x; v0 < nvec;
         v0 += (int64_t)gridDim.x * kThreads * U) {
        uint4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = v0 + u * stride;
            w[u] = load16_stream(x + 8 * (v < nvec ? v : 0));  // a quad is all in or all out
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = v0 + u * stride;
            uint32_t pm = pk_max_u16(pk_max_u16(w[u].x & 0x7FFF7FFFu, w[u].y & 0x7FFF7FFFu),
                                     pk_max_u16(w[u].z & 0x7FFF7FFFu, w[u].w & 0x7FFF7FFFu));
            uint32_t m = max(pm & 0xFFFFu, pm >> 16);
            m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));  // lane ^ 1
            m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));  // lane ^ 2
            const uint32_t byte = mx_scale_byte(m << 16);
            const float inv = mx_inverse_scale(byte);
            const uint32_t keep = byte == 0xFFu ? 0x80008000u : 0xFFFFFFFFu;
            const uint32_t q[4] = {w[u].x & keep, w[u].y & keep, w[u].z & keep, w[u].w & keep};
            float f[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                f[2 * k] = bf16_lo(q[k]) * inv;
                f[2 * k + 1] = bf16_hi(q[k]) * inv;
            }
            if (v < nvec) {
                reinterpret_cast<uint32_t*>(codes)[v] = mx_word(f);
                if (first)
                    scales[v >> 2] = (uint8_t)byte;
            }
        }
    }
}

// Dequantize: each lane reconstructs E consecutive elements (8 for bf16
// output, 4 for binary32: one 16-byte store), so a wave's stores are one
// contiguous run; the lanes of a 32-element block share its scale byte.
// Every reconstruction e2m1 * 2^(byte - 127) is exact in binary32 and in
// bf16 (two significant bits; 2^-128 and up), so the bf16 output is the
// binary32 result's top half. U chunks per thread have their loads in
// flight together.
template <bool BF16_OUT>
__global__ __launch_bounds__(kThreads) void mx_dequantize_kernel(const uint8_t* __restrict__ codes,
                                                                const uint8_t* __restrict__ scales,
                                                                int64_t nchunks, void* __restrict__ out)
{
    constexpr int E = BF16_OUT ? 8 : 4;
    constexpr int U = 4;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t c0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; c0 < nchunks; c0 += U * stride) {
        uint32_t w[U], sb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + u * stride;
            w[u] = 0u;
            sb[u] = 0u;
            if (c < nchunks) {
                w[u] = BF16_OUT ? *reinterpret_cast<const uint32_t*>(codes + c * 4)
                                : (uint32_t)*reinterpret_cast<const uint16_t*>(codes + c * 2);
                sb[u] = scales[(c * E) >> 5];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + u * stride;
            if (c >= nchunks)
                break;
            const float X = sb[u] == 0xFFu ? __uint_as_float(0x7FC00000u)
                            : sb[u] == 0u  ? __uint_as_float(0x00400000u)
                                           : __uint_as_float(sb[u] << 23);
            float v[E];
#pragma unroll
            for (int j = 0; j < E / 2; ++j) {
                const auto g = j == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 0)
                             : j == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 1)
                             : j == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 2)
                                      : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 3);
                v[2 * j] = g[0] * X;
                v[2 * j + 1] = g[1] * X;
            }
            if (BF16_OUT) {
                uint32_t h[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    h[k] = (__float_as_uint(v[2 * k]) >> 16) | (__float_as_uint(v[2 * k + 1]) & 0xFFFF0000u);
                reinterpret_cast<uint4*>(out)[c] = make_uint4(h[0], h[1], h[2], h[3]);
            } else {
                reinterpret_cast<float4*>(out)[c] = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
}

}  // namespace

hipError_t launch_mx_quantize(const MxQuantizeArgs& a, hipStream_t stream)
{
    if (a.rowwise && !a.colwise && !a.rht) {
        constexpr int kU = 4;
        const int64_t nvec = a.rows * (a.cols >> 3);
        int64_t g = (nvec + kThreads * kU - 1) / (kThreads * kU);
        if (g > 8192)
            g = 8192;
        hipLaunchKernelGGL(mx_quantize_rows_kernel<kU>, dim3((unsigned)g), dim3(kThreads), 0, stream, a.x, nvec,
                           a.codes_row, a.scales_row);
        return hipGetLastError();
    }
    if (a.colwise) {
        if (a.rht && a.rowwise)
            return hipErrorInvalidValue;  // the transform is columnwise only
        const int blocks_r = (int)((a.rows + kPairRows - 1) / kPairRows);
        const int blocks_c = (int)((a.cols + kPairCols - 1) / kPairCols);
        const dim3 grid((unsigned)((int64_t)blocks_r * blocks_c));
        if (a.rht)
            hipLaunchKernelGGL((mx_quantize_pair_kernel<false, true>), grid, dim3(kPairThreads), 0, stream, a,
                               blocks_c);
        else if (a.rowwise)
            hipLaunchKernelGGL((mx_quantize_pair_kernel<true, false>), grid, dim3(kPairThreads), 0, stream, a,
                               blocks_c);
        else
            hipLaunchKernelGGL((mx_quantize_pair_kernel<false, false>), grid, dim3(kPairThreads), 0, stream, a,
                               blocks_c);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;  // the transform is columnwise only
}

hipError_t launch_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                                void* out, bool bf16_out, hipStream_t stream)
{
    // chunks of 8 (bf16) or 4 (binary32) elements; cols is a multiple of 32
    const int64_t nchunks = rows * cols / (bf16_out ? 8 : 4);
    int64_t g = (nchunks + 4 * kThreads - 1) / (4 * kThreads);
    if (g > 8192)
        g = 8192;
    if (bf16_out)
        hipLaunchKernelGGL(mx_dequantize_kernel<true>, dim3((unsigned)g), dim3(kThreads), 0, stream, codes,
                           scales, nchunks, out);
    else
        hipLaunchKernelGGL(mx_dequantize_kernel<false>, dim3((unsigned)g), dim3(kThreads), 0, stream, codes,
                           scales, nchunks, out);
    return hipGetLastError();
}

}  // namespace nvfp4
