// Dequantize-and-contract NVFP4 GEMM: C = (S_gA * S_gB) * sum_k Ahat Bhat,
// TN layout (both operands K-contiguous).
//
// Every operand element e2m1(code) * e4m3(scale) has at most 6 significant
// bits and lies in [2^-10, 2688], so it is exact in fp16; products are summed
// in fp32 by v_mfma_f32_16x16x32_f16. One MFMA consumes K = 32, two NVFP4
// scale blocks.
//
// Structure (one workgroup = 8 waves, a 256 x 256 tile of C at a time):
//   - K advances 64 at a time (32 when K is not a multiple of 64). Each of
//     the 512 threads owns one row (256 of A, then 256 of B) for the stage:
//     it loads 32 bytes of packed codes and the four scale bytes and decodes
//     the 64 codes into LDS. Deeper stages halve the barriers per MFMA. Decoding is
//     three exact hardware steps: both scale bytes to fp16 in one E4M3
//     convert, two codes to fp16 per E2M1 convert, one packed fp16 multiply
//     per two codes. Each element is decoded once per workgroup.
//   - A stage in LDS is K-chunk major: for each chunk of 8 K-elements, the
//     16 bytes of all 512 rows side by side (A rows, then B rows). The 16
//     lanes of a fragment read that share a chunk read 16 consecutive rows,
//     256 contiguous bytes, and the decode's 16-byte writes of consecutive
//     threads are contiguous too: both without bank conflicts or padding.
//   - Waves form a 4 x 2 grid; each computes a 64 x 128 sub-tile (4 x 8 MFMA
//     tiles of 16 x 16, 128 fp32 accumulators per lane), so two waves share a
//     SIMD and one's decode overlaps the other's MFMAs. Stages are double-buffered in
//     LDS, and the packed codes are fetched two stages ahead into two
//     alternating register sets.
//   - A 2D-scaled operand's tile scales (16 row groups x K/16 bytes) are
//     staged in LDS once per tile with coalesced loads (transposed storage,
//     NVFP4_SCALE_2D_T, transposed on the way in), so its rows fetch only
//     codes per stage. The region holds kLdsScaleK bytes per operand, or
//     twice that for a lone 2D operand; larger K falls back to per-row
//     scale loads.
//   - The grid is persistent (one workgroup per CU); a tile's output stores
//     drain while the next tile starts. A last round that would occupy at
//     most half the grid runs as a second launch of 256 x 128 half tiles
//     (waves of 64 x 64) on twice as many workgroups.
//   - Optionally the epilogue also reduces max |C| of the stored values (the
//     tensor amax a following NVFP4 quantization of C needs), so that
//     quantization reads C once instead of twice.
#include <atomic>

#include "device.h"
#include "kernels.h"
#include "quant_item.h"

namespace nvfp4 {

namespace {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) float floatx4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kGemmThreads = 512;
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kGroupM = 4;  // tile rows per group of the tile order

// Stage geometry for a stage of KS = 32 or 64 K-elements: KS / 8 chunk
// arrays of 512 rows x 16 bytes (fp16 K-elements 8c .. 8c + 7 of every row,
// A rows then B rows), two stages, and the largest K whose 2D tile scales a
// tile stages in LDS next to them.
template <int KS>
struct Geo {
    static constexpr int kChunkStride = (kBM + kBN) * 16;
    static constexpr int kStageBytes = (KS / 8) * kChunkStride;
    static constexpr int kLdsScaleK = KS == 32 ? 16384 : 8192;
    static_assert(2 * kStageBytes + 2 * kLdsScaleK <= 160 * 1024, "LDS");
};

// Byte SEL of `w` (two codes) -> two fp16, times the packed pair `s2`
// (both halves the block's scale). Both converts are exact: E2M1 and E4M3
// values are fp16 values, and so is their product (at most 6 significant
// bits, magnitude in [2^-10, 2688]).
template <int SEL>
__device__ __forceinline__ uint32_t decode_pair(uint32_t w, f16x2 s2)
{
    const auto g = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, g) * s2);
}

// One row's packed codes for a K stage: KS / 2 bytes and the KS / 16 scale
// bytes (low byte: first 16 codes).
template <int KS>
struct RowStage {
    uint4 codes[KS / 32];
    uint32_t scales;
};

// Scale bytes read by rows past the end of an operand: scale 0 makes every
// code of such a row decode to zero without touching the loaded values.
__device__ __attribute__((aligned(16))) const uint8_t kZeroScales[16] = {};

// Fetch stage `stage` of this thread's row: KS / 2 bytes of codes and the
// KS / 16 scale bytes, the first at scale_row + stage * sstride and the
// next ones bstride apart (bstride 1: adjacent; transposed 2D scales: one
// scale row apart; sstride = bstride = 0 for rows past the end, which read
// kZeroScales).
template <int KS, bool WIDE>
__device__ __forceinline__ RowStage<KS> fetch_stage(const uint8_t* code_row, const uint8_t* scale_row,
                                                    int stage, int64_t sstride, int64_t bstride, int64_t K,
                                                    const uint8_t* lds_scales)
{
    RowStage<KS> st;
    const int64_t k0 = (int64_t)stage * KS;
    if constexpr (KS == 64) {
        // K is a multiple of 64 and the scale arrays are 4-byte aligned.
        st.codes[0] = load16(code_row + (k0 >> 1));
        st.codes[1] = load16(code_row + (k0 >> 1) + 16);
        if (lds_scales != nullptr) {
            st.scales = *reinterpret_cast<const uint32_t*>(lds_scales + 4 * stage);
        } else {
            const uint8_t* sp = scale_row + (int64_t)stage * sstride;
            const __attribute__((address_space(1))) uint8_t* gp =
                (const __attribute__((address_space(1))) uint8_t*)sp;
            if (bstride == 1)  // uniform over the wave (its rows are all A or all B)
                st.scales = *(const __attribute__((address_space(1))) uint32_t*)sp;
            else
                st.scales = (uint32_t)gp[0] | ((uint32_t)gp[bstride] << 8) | ((uint32_t)gp[2 * bstride] << 16) |
                            ((uint32_t)gp[3 * bstride] << 24);
        }
        return st;
    }
    if (lds_scales != nullptr) {
        // 2D tile scales staged in LDS: this row group's K/16 bytes
        const uint8_t* q = lds_scales + 2 * stage;
        if (WIDE) {
            st.codes[0] = load16(code_row + (k0 >> 1));
            st.scales = *reinterpret_cast<const uint16_t*>(q);
        } else {
            const bool has2 = k0 + 16 < K;
            const uint2 lo = *reinterpret_cast<const uint2*>(code_row + (k0 >> 1));
            const uint2 hi = has2 ? *reinterpret_cast<const uint2*>(code_row + (k0 >> 1) + 8) : make_uint2(0u, 0u);
            st.codes[0] = make_uint4(lo.x, lo.y, hi.x, hi.y);
            st.scales = (uint16_t)(q[0] | (has2 ? (uint32_t)q[1] << 8 : 0u));
        }
        return st;
    }
    const uint8_t* sp = scale_row + (int64_t)stage * sstride;
    const __attribute__((address_space(1))) uint8_t* gp = (const __attribute__((address_space(1))) uint8_t*)sp;
    if (WIDE) {
        st.codes[0] = load16(code_row + (k0 >> 1));
        if (bstride == 1)  // uniform over the wave (its rows are all A or all B)
            st.scales = *(const __attribute__((address_space(1))) uint16_t*)sp;
        else
            st.scales = (uint16_t)(gp[0] | ((uint32_t)gp[bstride] << 8));
    } else {
        // K is an odd multiple of 16: the last stage has one block.
        const bool has2 = k0 + 16 < K;
        const uint2 lo = *reinterpret_cast<const uint2*>(code_row + (k0 >> 1));
        const uint2 hi = has2 ? *reinterpret_cast<const uint2*>(code_row + (k0 >> 1) + 8) : make_uint2(0u, 0u);
        st.codes[0] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        st.scales = (uint16_t)(gp[0] | (has2 ? (uint32_t)gp[bstride] << 8 : 0u));
    }
    return st;
}

// Decode one row's stage and write its KS fp16 to LDS: chunk c (16 bytes)
// at lds_row + c * kChunkStride.
template <int KS>
__device__ __forceinline__ void decode_stage_to_lds(const RowStage<KS>& st, uint8_t* lds_row)
{
    // Two scale bytes to fp16 per convert.
    const f16x2 lo = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(st.scales, 1.0f, false));
    f16x2 sc[4] = {{lo[0], lo[0]}, {lo[1], lo[1]}, {}, {}};
    if constexpr (KS == 64) {
        const f16x2 hi = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(st.scales, 1.0f, true));
        sc[2] = f16x2{hi[0], hi[0]};
        sc[3] = f16x2{hi[1], hi[1]};
    }
#pragma unroll
    for (int h = 0; h < KS / 32; ++h) {
        const uint32_t w[4] = {st.codes[h].x, st.codes[h].y, st.codes[h].z, st.codes[h].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f16x2 sq = sc[2 * h + (q >> 1)];
            const u32x4 o = {decode_pair<0>(w[q], sq), decode_pair<1>(w[q], sq), decode_pair<2>(w[q], sq),
                             decode_pair<3>(w[q], sq)};
            *reinterpret_cast<u32x4*>(lds_row + (4 * h + q) * Geo<KS>::kChunkStride) = o;
        }
    }
}

// Row `row`'s 8 fp16 at byte kbyte (a multiple of 16) of its KS-element stage.
template <int KS>
__device__ __forceinline__ f16x8 lds_fragment(const uint8_t* lds, int row, int kbyte)
{
    return __builtin_bit_cast(f16x8,
                              *reinterpret_cast<const u32x4*>(lds + (kbyte >> 4) * Geo<KS>::kChunkStride + row * 16));
}

// The MFMAs of one stage for this wave's 64 x (32 FN) sub-tile: 4 x 2 FN
// tiles of 16 x 16, lane l holding row (A) or column (B) l % 16 of a tile
// and K elements 8 (l / 16) .. + 7 of each 32-element step. The four A
// fragments of a step stay in registers; the B fragments are read one ahead,
// and a scheduling barrier after each B column's MFMAs keeps the compiler
// from hoisting the later reads (which was 4% slower). The wave runs its
// MFMAs at raised priority, so that of the two waves on a SIMD the one with
// matrix work issues first and the other's decode fills the gaps (measured:
// 0-3% on 8192x14336x4096).
template <int KS, int FN>
__device__ __forceinline__ void stage_mfma(const uint8_t* buf, int wm, int wn, int frow, int fk,
                                           floatx4 (&acc)[4][8])
{
    const uint8_t* const bbuf = buf + kBM * 16;  // B rows follow the A rows in every chunk
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < KS / 32; ++ks) {
        f16x8 fa[4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
            fa[a] = lds_fragment<KS>(buf, wm + a * 16 + frow, ks * 64 + fk);
        f16x8 fb = lds_fragment<KS>(bbuf, wn + frow, ks * 64 + fk);
#pragma unroll
        for (int b = 0; b < 2 * FN; ++b) {
            f16x8 next;
            if (b + 1 < 2 * FN)
                next = lds_fragment<KS>(bbuf, wn + (b + 1) * 16 + frow, ks * 64 + fk);
#pragma unroll
            for (int a = 0; a < 4; ++a)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[a], fb, acc[a][b], 0, 0, 0);
            fb = next;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __builtin_amdgcn_s_setprio(0);
}

// Position in the tile order of this workgroup's tile in round `round`.
// Workgroups are dealt round-robin over the 8 XCDs; in each round give each
// XCD a contiguous run of positions.
__device__ __forceinline__ int gemm_tile_index(int round)
{
    const int G = gridDim.x;
    int w = blockIdx.x;
    if ((G & 7) == 0)
        w = (w & 7) * (G >> 3) + (w >> 3);
    return round * G + w;
}

// Stage one operand's 2D tile scales for a tile (its 16 row groups, from
// group g0 on) into LDS as [group][K/16], group-major; groups past the last
// (tile_rows of them) read as 0. t: 0..255, this operand's threads.
// Transposed storage ([K/16][tile_rows]) is transposed on the way in.
__device__ __forceinline__ void stage_tile_scales(uint8_t* dst, const uint8_t* scales, bool transposed,
                                                  int64_t g0, int64_t tile_rows, int64_t K, int t)
{
    const int64_t kb = K >> 4;  // scale blocks per row
    if (!transposed) {
        // The 16 groups' rows are one contiguous span of 16 * kb bytes.
        const uint8_t* src = scales + g0 * kb;
        const int64_t avail = (tile_rows - g0) * kb;  // bytes inside the matrix
        for (int64_t off = (int64_t)t * 16; off < 16 * kb; off += 256 * 16) {
            if (off + 16 <= avail) {
                *reinterpret_cast<uint4*>(dst + off) = load16(src + off);
            } else {
                for (int i = 0; i < 16; ++i)
                    dst[off + i] = off + i < avail ? src[off + i] : (uint8_t)0;
            }
        }
    } else {
        // Row j holds the scales of every group for K block j: 16 bytes of
        // this tile's groups at j * tile_rows + g0.
        const int ng = (int)min((int64_t)16, tile_rows - g0);
        const bool vec = ng == 16 && ((tile_rows & 15) == 0);
        for (int64_t j = t; j < kb; j += 256) {
            const uint8_t* src = scales + j * tile_rows + g0;
            uint8_t b[16];
            if (vec) {
                const uint4 v = load16(src);
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    b[i] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    b[i] = i < ng ? src[i] : (uint8_t)0;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i)
                dst[i * kb + j] = b[i];
        }
    }
}

// Quantizing epilogue (QUANT: 1 rowwise, 2 columnwise, 3 both): the tile's
// bf16 values go to LDS at a padded pitch, then each of the 512 threads
// quantizes one 16 x 8 work item of it with the item code of the quantize
// kernels (the 256 x 256 tile is two 128 x 256 quantize tiles, A above B),
// so the codes equal those nvfp4_quantize_1d writes for the bf16 C.
constexpr int kQuantPitch = 2 * kBN + 16;                    // bytes per tile row
constexpr int kQuantRcp = kQuantPitch * kBM;                 // reciprocal table offset
constexpr int kQuantLds = kQuantRcp + 128 * 4;
constexpr int kQuantStageCodes = kTileC * kRowBlocks * 8;    // one quantize tile's staged codes
static_assert(2 * kQuantStageCodes + 2 * kTileC * kRowBlocks <= kQuantRcp, "staging overlays the tile");
static_assert(kQuantLds <= 160 * 1024, "LDS");
static_assert(kBM == 2 * kTileR && kBN == kTileC, "a GEMM tile is a pair of quantize tiles");

template <int QUANT>
__device__ __forceinline__ void quant_epilogue(const GemmArgs& g, const floatx4 (&acc)[4][8], float scale,
                                               int64_t m0, int64_t n0, int wm, int wn, int lane, int wave,
                                               int round, uint8_t* lds_in, uint32_t& cmax)
{
    constexpr bool QROW = (QUANT & 1) != 0, QCOL = (QUANT & 2) != 0;
    const int t = threadIdx.x;
    // An opaque zero keeps this epilogue's addresses from being hoisted out
    // of the tile loop (where they would stay live across the K loop).
    uint32_t zero = 0u;
    asm volatile("" : "+v"(zero));
    uint8_t* const lds = lds_in + zero;
    const int ln = lane + (int)zero;
    // 1. C x fl(S_gA S_gB), rounded to bf16 (nearest even), into LDS; the
    //    K loop's last barrier has passed, so the stage buffers are free.
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int cl = wn + b * 16 + (ln & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rl = wm + a * 16 + 4 * (ln >> 4) + i;
                const uint32_t u = __float_as_uint(acc[a][b][i] * scale);
                const uint16_t h = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
                *reinterpret_cast<uint16_t*>(lds + rl * kQuantPitch + 2 * cl) = h;
            }
            __builtin_amdgcn_sched_barrier(0);  // one 16 x 16 tile at a time
        }
    const ScaleCtx sc = scale_ctx(*g.q_amax);
    float* const rcp = reinterpret_cast<float*>(lds + kQuantRcp);
    build_reciprocal_table(rcp, sc.sg);
    if (g.q_global_scale != nullptr && blockIdx.x == 0 && t == 0 && round == 0)
        *g.q_global_scale = sc.sg;
    __syncthreads();

    // 2. One work item per thread: tile rows 16 rb .. 16 rb + 15 (rb = 2 wave
    //    + half-wave; rb < 8 in quantize tile A, else B), columns 8 cg ..
    //    8 cg + 7, read into registers before the staging overwrites the tile.
    const int rb = 2 * wave + (ln >> 5), cg = ln & 31;
    uint4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        v[i] = *reinterpret_cast<const uint4*>(lds + (rb * 16 + i) * kQuantPitch + cg * 16);
    ItemPos q;
    q.tile_r0 = m0 + (rb >> 3) * kTileR;
    q.tile_c0 = n0;
    q.rb = rb & 7;
    q.cg = cg;
    q.odd = (ln & 1) != 0;
    q.r0 = m0 + rb * 16;
    q.c0 = n0 + cg * 8;
    q.valid = q.r0 < g.M && q.c0 < g.N;  // both lanes of a pair agree (N % 16 == 0)
    Params p{};
    p.rows = g.M;
    p.cols = g.N;
    p.codes_row = g.q_codes_row;
    p.scales_row = g.q_scales_row;
    p.codes_col = g.q_codes_col;
    p.scales_col = g.q_scales_col;
    uint2* const codes0 = reinterpret_cast<uint2*>(lds);
    uint2* const codes1 = reinterpret_cast<uint2*>(lds + kQuantStageCodes);
    uint8_t* const scales0 = lds + 2 * kQuantStageCodes;
    uint8_t* const scales1 = scales0 + kTileC * kRowBlocks;
    __syncthreads();
    if (q.valid) {
        BlockMax bm;
        column_maxima(v, bm);  // also max |Y| of the item (the reported amax)
        cmax = max(cmax, item_max(bm));
        if (QROW)
            row_maxima(v, q.odd, bm);
        uint4 draws[16];  // unused: round to nearest
        compute_item<QROW, QCOL, false, false, false>(p, q, v, bm, draws, sc, rcp, rb < 8 ? codes0 : codes1,
                                                      rb < 8 ? scales0 : scales1, false);
    }
    if (QCOL) {
        __syncthreads();
        if (t < kThreads)  // the pair writer's 256 threads
            write_col_pair(p, m0, n0, codes0, codes1, scales0, scales1, t + (int)zero);
    }
    __syncthreads();  // the next tile's first stage overwrites this LDS
}

// AMAX: also reduce max |C| over the values as stored (bf16 or fp32 bit
// patterns, an integer maximum like nvfp4_amax's) into *g.c_amax, which the
// launch has reset: a running maximum per lane over its tiles, one atomic
// per wave at the end.
//
// FN = 4: whole 256 x 256 tiles, positions 0 .. count-1 of the tile order.
// FN = 2: half tiles of 256 x 128 (each wave 64 x 64), units 0 .. count-1,
// unit u being half u & 1 of tile first + u / 2: a partial last round of
// whole tiles, split so that it fills twice as many CUs. Every output
// element is summed in the same order either way.
template <bool BF16_OUT, bool WIDE, bool AMAX, int KS, int FN, int QUANT = 0>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmArgs g, int tiles_m, int tiles_n, int first,
                                                        int count)
{
    constexpr int kStageBytes = Geo<KS>::kStageBytes;
    constexpr int kLdsScaleK = Geo<KS>::kLdsScaleK;
    constexpr int kMainLds = 2 * kStageBytes + 2 * kLdsScaleK;
    constexpr int kLdsBytes = (QUANT != 0 && kQuantLds > kMainLds) ? kQuantLds : kMainLds;
    static_assert(QUANT == 0 || (FN == 4 && BF16_OUT && AMAX), "the quantizing epilogue takes whole tiles");
    uint32_t cmax = 0u;
    // Two K stages, then the A and B tile-scale regions; the quantizing
    // epilogue reuses the whole array once a tile's K loop is done.
    __shared__ __attribute__((aligned(16))) uint8_t lds_all[kLdsBytes];
    uint8_t* const lds = lds_all;
    uint8_t* const lds_sc = lds_all + 2 * kStageBytes;  // A, B tile scales

    const int64_t K = g.K;
    const int nstages = (int)((K + KS - 1) / KS);
    const int last = nstages - 1;
    const float scale = (*g.a_sg) * (*g.b_sg);
    // 2D operands read their tile scales from LDS (K small enough, 16-byte
    // aligned scale arrays); the flags are uniform over the workgroup.
    // Each takes half of the region, or all of it when it is the only one.
    const bool a_al = g.a_two_d && ((reinterpret_cast<uintptr_t>(g.a_scales) & 15) == 0);
    const bool b_al = g.b_two_d && ((reinterpret_cast<uintptr_t>(g.b_scales) & 15) == 0);
    const bool a_stage = a_al && (K <= kLdsScaleK || (!b_al && K <= 2 * kLdsScaleK));
    const bool b_stage = b_al && (K <= kLdsScaleK || (!a_al && K <= 2 * kLdsScaleK));

    // Persistent: each workgroup walks tiles; a tile's output stores drain
    // while the next tile's first stages load and decode.
    for (int round = 0;; ++round) {
        const int unit = gemm_tile_index(round);
        if (unit >= count)
            break;
        // The thread's per-tile constants. With the quantizing epilogue they
        // are recomputed every round (an opaque copy of the lane index keeps
        // them from being hoisted out of the tile loop), so that none of
        // them is live while the epilogue runs.
        int lane = threadIdx.x & 63;
        if constexpr (QUANT != 0)
            asm volatile("" : "+v"(lane));
        const int wave = threadIdx.x >> 6;
        const int t = wave * 64 + lane;
        const int wm = (wave >> 1) * 64, wn = (wave & 1) * (32 * FN);
        const int frow = lane & 15;
        const int fk = (lane >> 4) * 16;  // byte offset of the lane's 8 K-elements
        const bool is_b = wave >= kBM / 64;
        const int64_t rows = is_b ? g.N : g.M;
        const bool two_d = is_b ? g.b_two_d : g.a_two_d;
        const bool scales_t = is_b ? g.b_scales_t : g.a_scales_t;
        const uint8_t* codes = is_b ? g.b_codes : g.a_codes;
        const uint8_t* scales = is_b ? g.b_scales : g.a_scales;
        uint8_t* my_row0 = lds + t * 16;
        const bool my_stage = is_b ? b_stage : a_stage;
        uint8_t* const my_sc = lds_sc + (is_b && a_stage ? kLdsScaleK : 0);
        // Half tiles need 128 B rows: the last two waves fetch nothing.
        const bool loads = FN == 4 || !is_b || t - kBM < 64 * FN;
        const int tile = FN == 4 ? unit : first + (unit >> 1);
        const int half = FN == 4 ? 0 : (unit & 1);
        // Tiles are ordered in groups of kGroupM tile rows, column by column
        // inside a group. At one workgroup per CU an XCD's share of a round
        // is 32 consecutive positions, inside a group a 4 x 8 block of tiles:
        // A panels are shared by 8 workgroups and B panels by 4 in its L2.
        const int group = tile / (kGroupM * tiles_n);
        const int gm = min(kGroupM, tiles_m - group * kGroupM);
        const int in_group = tile - group * kGroupM * tiles_n;
        const int tm = group * kGroupM + in_group % gm, tn = in_group / gm;
        const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN + half * (32 * FN * 2);

        // This thread's row: A rows 0..255, then B rows 0..255.
        const int64_t row = is_b ? n0 + (t - kBM) : m0 + t;
        const bool valid = row < rows;
        const int64_t rc = valid ? row : 0;
        const uint8_t* code_row = codes + rc * (K >> 1);
        // Scale of (row, K block j): 1D [row][j], 2D [row/16][j], transposed
        // 2D [j][row/16].
        const int64_t tile_rows = (rows + 15) >> 4;
        const uint8_t* scale_row = !valid    ? kZeroScales
                                   : scales_t ? scales + (rc >> 4)
                                              : scales + (two_d ? (rc >> 4) : rc) * (K >> 4);
        const int64_t bstride = !valid ? 0 : scales_t ? tile_rows : 1;
        const int64_t sstride = (KS / 16) * bstride;
        const int lt = is_b ? t - kBM : t;  // this thread's index among its operand's 256
        const uint8_t* my_lds_scales = my_stage ? my_sc + (lt >> 4) * (K >> 4) : nullptr;
        if (my_stage)
            stage_tile_scales(my_sc, scales, scales_t, (is_b ? n0 : m0) >> 4, tile_rows, K, lt);
        if (a_stage || b_stage)
            __syncthreads();

        floatx4 acc[4][8];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 8; ++b)
                acc[a][b] = floatx4{};

        RowStage<KS> sa, sb;
        if (loads) {
            decode_stage_to_lds<KS>(fetch_stage<KS, WIDE>(code_row, scale_row, 0, sstride, bstride, K, my_lds_scales),
                                    my_row0);
            // Two register sets alternate (stage s+1 in one, s+2 in the
            // other) so a fetch lands in registers the decode has just
            // consumed: no copies of in-flight loads, hence no wait on the
            // newest fetch.
            sa = fetch_stage<KS, WIDE>(code_row, scale_row, min(1, last), sstride, bstride, K, my_lds_scales);
            __builtin_amdgcn_sched_barrier(0);  // issue order sa, sb as in the loop
            sb = fetch_stage<KS, WIDE>(code_row, scale_row, min(2, last), sstride, bstride, K, my_lds_scales);
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();

        int s = 0;
        for (; s + 1 < nstages; s += 2) {
            stage_mfma<KS, FN>(lds, wm, wn, frow, fk, acc);
            if (loads) {
                decode_stage_to_lds<KS>(sa, my_row0 + kStageBytes);
                sa = fetch_stage<KS, WIDE>(code_row, scale_row, min(s + 3, last), sstride, bstride, K, my_lds_scales);
            }
            __syncthreads();
            // keep each half's work in its half: the scheduler would
            // otherwise hoist the next decode and wait on the newest fetch
            __builtin_amdgcn_sched_barrier(0);
            stage_mfma<KS, FN>(lds + kStageBytes, wm, wn, frow, fk, acc);
            if (loads) {
                decode_stage_to_lds<KS>(sb, my_row0);
                sb = fetch_stage<KS, WIDE>(code_row, scale_row, min(s + 4, last), sstride, bstride, K, my_lds_scales);
            }
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        }
        if (s < nstages) {
            stage_mfma<KS, FN>(lds, wm, wn, frow, fk, acc);
            __syncthreads();  // buffer 0 is rewritten by the next tile
        }

        if constexpr (QUANT != 0) {
            quant_epilogue<QUANT>(g, acc, scale, m0, n0, wm, wn, lane, wave, round, lds, cmax);
            continue;
        }
        // An opaque copy of the lane index keeps the store addresses from
        // being computed before the K loop (where they would stay live).
        int el = lane;
        asm volatile("" : "+v"(el));
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 2 * FN; ++b) {
                const int64_t col = n0 + wn + b * 16 + (el & 15);
                if (col >= g.N)
                    continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t r = m0 + wm + a * 16 + 4 * (el >> 4) + i;
                    if (r >= g.M)
                        continue;
                    const float v = acc[a][b][i] * scale;
                    if (BF16_OUT) {
                        const uint32_t u = __float_as_uint(v);
                        const uint16_t h = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
                        reinterpret_cast<uint16_t*>(g.c)[r * g.N + col] = h;
                        if (AMAX)
                            cmax = max(cmax, (uint32_t)(h & 0x7FFFu) << 16);
                    } else {
                        reinterpret_cast<float*>(g.c)[r * g.N + col] = v;
                        if (AMAX)
                            cmax = max(cmax, __float_as_uint(v) & 0x7FFFFFFFu);
                    }
                }
            }
    }
    if (AMAX && g.c_amax != nullptr) {
        cmax = wave_max_u32(cmax);
        if ((threadIdx.x & 63) == 0)
            atomicMax(reinterpret_cast<uint32_t*>(g.c_amax), cmax);
    }
}

__global__ void gemm_amax_reset_kernel(float* a) { *reinterpret_cast<uint32_t*>(a) = 0u; }

// Workgroups resident at once on the current device (one per CU at this
// tile size), cached per device.
template <bool BF16_OUT, bool WIDE, bool AMAX, int KS, int QUANT = 0>
int gemm_capacity()
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
            &per_cu, reinterpret_cast<const void*>(gemm_kernel<BF16_OUT, WIDE, AMAX, KS, 4, QUANT>), kGemmThreads, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    c = (per_cu > 0 ? per_cu : 1) * cus;
    if (c > 0)
        cache[dev].store(c, std::memory_order_relaxed);
    return c;
}

// Whole tiles round by round on a persistent grid; a last round that would
// fill at most half the grid runs instead as half tiles on twice as many
// workgroups (a second launch), so it takes about half a round.
template <bool BF16_OUT, bool WIDE, bool AMAX, int KS>
hipError_t launch_variant(const GemmArgs& a, int tiles_m, int tiles_n, hipStream_t stream)
{
    const int cap = gemm_capacity<BF16_OUT, WIDE, AMAX, KS>();
    if (cap <= 0)
        return hipErrorInvalidDevice;
    const int nt = tiles_m * tiles_n;
    const int rounds = nt / cap, rem = nt % cap;
    const bool split_tail = rem > 0 && 2 * rem <= cap;
    const int whole = split_tail ? rounds * cap : nt;
    if (AMAX)
        hipLaunchKernelGGL(gemm_amax_reset_kernel, dim3(1), dim3(1), 0, stream, a.c_amax);
    if (whole > 0)
        hipLaunchKernelGGL((gemm_kernel<BF16_OUT, WIDE, AMAX, KS, 4>), dim3((unsigned)(whole < cap ? whole : cap)),
                           dim3(kGemmThreads), 0, stream, a, tiles_m, tiles_n, 0, whole);
    if (split_tail)
        hipLaunchKernelGGL((gemm_kernel<BF16_OUT, WIDE, AMAX, KS, 2>), dim3((unsigned)(2 * rem)), dim3(kGemmThreads), 0,
                           stream, a, tiles_m, tiles_n, whole, 2 * rem);
    return hipGetLastError();
}

// The quantizing epilogue: whole tiles only, on a persistent grid.
template <bool WIDE, int KS, int QUANT>
hipError_t launch_quant_variant(const GemmArgs& a, int tiles_m, int tiles_n, hipStream_t stream)
{
    const int cap = gemm_capacity<true, WIDE, true, KS, QUANT>();
    if (cap <= 0)
        return hipErrorInvalidDevice;
    const int nt = tiles_m * tiles_n;
    if (a.c_amax != nullptr)
        hipLaunchKernelGGL(gemm_amax_reset_kernel, dim3(1), dim3(1), 0, stream, a.c_amax);
    hipLaunchKernelGGL((gemm_kernel<true, WIDE, true, KS, 4, QUANT>), dim3((unsigned)(nt < cap ? nt : cap)),
                       dim3(kGemmThreads), 0, stream, a, tiles_m, tiles_n, 0, nt);
    return hipGetLastError();
}

template <bool WIDE, int KS>
hipError_t launch_quant(const GemmArgs& a, int tiles_m, int tiles_n, hipStream_t stream)
{
    switch (a.q_flags) {
    case 1: return launch_quant_variant<WIDE, KS, 1>(a, tiles_m, tiles_n, stream);
    case 2: return launch_quant_variant<WIDE, KS, 2>(a, tiles_m, tiles_n, stream);
    case 3: return launch_quant_variant<WIDE, KS, 3>(a, tiles_m, tiles_n, stream);
    default: return hipErrorInvalidValue;
    }
}

template <bool BF16_OUT, bool WIDE, int KS>
hipError_t launch_amax_or_not(const GemmArgs& a, int tiles_m, int tiles_n, hipStream_t stream)
{
    return a.c_amax != nullptr ? launch_variant<BF16_OUT, WIDE, true, KS>(a, tiles_m, tiles_n, stream)
                               : launch_variant<BF16_OUT, WIDE, false, KS>(a, tiles_m, tiles_n, stream);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream)
{
    const int tiles_m = (int)((a.M + kBM - 1) / kBM);
    const int tiles_n = (int)((a.N + kBN - 1) / kBN);
    // 64-element stages when K allows them and a stage's four scale bytes of
    // a row are one aligned load; else 32-element stages (K a multiple of
    // 32, or an odd multiple of 16).
    const bool k64 = (a.K % 64) == 0 && ((reinterpret_cast<uintptr_t>(a.a_scales) & 3) == 0) &&
                     ((reinterpret_cast<uintptr_t>(a.b_scales) & 3) == 0);
    const bool wide = (a.K % 32) == 0;
    if (a.q_flags != 0) {
        if (k64)
            return launch_quant<true, 64>(a, tiles_m, tiles_n, stream);
        return wide ? launch_quant<true, 32>(a, tiles_m, tiles_n, stream)
                    : launch_quant<false, 32>(a, tiles_m, tiles_n, stream);
    }
    if (k64)
        return a.c_bf16 ? launch_amax_or_not<true, true, 64>(a, tiles_m, tiles_n, stream)
                        : launch_amax_or_not<false, true, 64>(a, tiles_m, tiles_n, stream);
    if (a.c_bf16)
        return wide ? launch_amax_or_not<true, true, 32>(a, tiles_m, tiles_n, stream)
                    : launch_amax_or_not<true, false, 32>(a, tiles_m, tiles_n, stream);
    return wide ? launch_amax_or_not<false, true, 32>(a, tiles_m, tiles_n, stream)
                : launch_amax_or_not<false, false, 32>(a, tiles_m, tiles_n, stream);
}

}  // namespace nvfp4
