// NVFP4 quantization kernels: 1D (rowwise / columnwise / both, RNE or
// stochastic, optional Hadamard) and 2D (16x16 tiles, both layouts).
//
// One workgroup (256 threads, 4 waves) owns a kTileR x kTileC tile of the
// bf16 input. A work item is 16 rows x 8 columns: sixteen 16-byte loads,
// where the 32 lanes of a half-wave cover 256 consecutive columns of a row
// (512 contiguous bytes per load). Inside an item:
//   - a columnwise block is one column's 16 rows (all in one lane);
//   - a rowwise block is one row's 16 columns, split over the lane pair
//     (2k, 2k+1), which trade maxima and multipliers through DPP;
//   - a 2D tile is the lane pair's 16 x 16 elements.
// Rowwise codes are stored straight from registers (128 contiguous bytes
// per row per half-wave). Columnwise codes are staged in LDS and written
// as whole 128-byte column segments.
#include "device.h"
#include "kernels.h"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kTileR = 256;
constexpr int kTileC = 256;
constexpr int kRowBlocks = kTileR / 16;   // 16
constexpr int kColGroups = kTileC / 8;    // 32
constexpr int kItemsPerThread = kRowBlocks * kColGroups / kThreads;  // 2

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
};

// Map the workgroup index to a tile so that each XCD (workgroups are dealt
// round-robin over 8) walks a contiguous run of tiles; `vertical` makes the
// run go down the rows first (columnwise outputs of adjacent tiles then
// share cache lines in the same L2).
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

template <bool ROW, bool COL, bool TWO_D, bool SR, bool RHT>
__global__ __launch_bounds__(kThreads) void quantize_kernel(Params p)
{
    // Columnwise staging: per tile column, 16 row blocks x 8 bytes; the
    // slot of a row block is swizzled by the column group to spread banks.
    __shared__ uint2 lds_codes[COL ? kTileC * kRowBlocks : 1];
    __shared__ uint8_t lds_scales[(COL && !TWO_D) ? kTileC * kRowBlocks : 16];

    int tr, tc;
    tile_of_block(p.tiles_r, p.tiles_c, COL, tr, tc);
    const int64_t tile_r0 = (int64_t)tr * kTileR;
    const int64_t tile_c0 = (int64_t)tc * kTileC;

    const float amax = *p.amax;
    const float sg = global_scale_from_amax(amax);
    const float t6 = 6.0f * sg;
    if (p.sg_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
        *p.sg_out = sg;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int cg = lane & 31;
    const bool odd = (lane & 1) != 0;
    const int64_t rows = p.rows, cols = p.cols;

#pragma unroll 1
    for (int it = 0; it < kItemsPerThread; ++it) {
        const int rb = it * (kRowBlocks / kItemsPerThread) + wave * 2 + (lane >> 5);
        const int64_t r0 = tile_r0 + rb * 16;
        const int64_t c0 = tile_c0 + cg * 8;
        if (r0 >= rows || c0 >= cols)
            continue;  // both lanes of a pair agree: cols is a multiple of 16

        uint4 v[16];
        const uint16_t* src = p.x + r0 * cols + c0;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            v[i] = load16_stream(src + i * cols);

        // ---- element values (binary32) and column maxima
        float y[8][16];
        uint32_t cmax[8];
        if (RHT) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    y[j][i] = bf16_at(v[i], j);
                rht16_inplace(y[j], p.mask);
                uint32_t m = 0u;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    m = max(m, __float_as_uint(y[j][i]) & 0x7FFFFFFFu);
                cmax[j] = m;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    y[j][i] = bf16_at(v[i], j);
            if (COL || TWO_D) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint32_t pm = 0u;
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        pm = pk_max_u16(pm, word_at(v[i], k) & 0x7FFF7FFFu);
                    cmax[2 * k] = pm << 16;
                    cmax[2 * k + 1] = pm & 0xFFFF0000u;
                }
            }
        }

        // ---- block scales
        float rc[8];            // columnwise multipliers (1D)
        float r2 = 0.0f;        // 2D tile multiplier
        uint32_t tile_byte = 0u;
        uint32_t col_byte[8];
        if (TWO_D) {
            uint32_t m = cmax[0];
#pragma unroll
            for (int j = 1; j < 8; ++j)
                m = max(m, cmax[j]);
            m = max(m, swap_lane1(m));
            BlockScale bs = block_scale(m, sg, t6);
            r2 = bs.r;
            tile_byte = bs.byte;
        } else if (COL) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                BlockScale bs = block_scale(cmax[j], sg, t6);
                rc[j] = bs.r;
                col_byte[j] = bs.byte;
            }
        }

        float rr[16];  // rowwise multipliers (1D), one per row of the item
        if (ROW && !TWO_D) {
            uint32_t rm[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                uint32_t pm = pk_max_u16(pk_max_u16(v[i].x & 0x7FFF7FFFu, v[i].y & 0x7FFF7FFFu),
                                         pk_max_u16(v[i].z & 0x7FFF7FFFu, v[i].w & 0x7FFF7FFFu));
                rm[i] = max(pm & 0xFFFFu, pm >> 16) << 16;
            }
            // Even lanes own rows 0..7 of the pair's blocks, odd lanes 8..15.
            const int64_t srow0 = r0 + (odd ? 8 : 0);
            uint8_t* sdst = p.scales_row + srow0 * (cols >> 4) + (c0 >> 4);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t send = odd ? rm[k] : rm[k + 8];
                const uint32_t recv = swap_lane1(send);
                const uint32_t own = odd ? rm[k + 8] : rm[k];
                BlockScale bs = block_scale(max(own, recv), sg, t6);
                sdst[k * (cols >> 4)] = (uint8_t)bs.byte;
                const float other = swap_lane1(bs.r);
                rr[k] = odd ? other : bs.r;
                rr[k + 8] = odd ? bs.r : other;
            }
        }

        // ---- encode, row by row
        uint32_t colw[8][2];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            colw[j][0] = colw[j][1] = 0u;
        const int64_t flat0 = r0 * cols + c0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint4 draws = make_uint4(0u, 0u, 0u, 0u);
            if (SR) {
                const uint64_t q = (uint64_t)(flat0 + i * cols) >> 3;
                draws = philox4x32_10((uint32_t)q, (uint32_t)(q >> 32), p.seed_lo, p.seed_hi);
            }
            uint32_t roww = 0u;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float xv = y[j][i];
                const uint32_t sign8 = (__float_as_uint(xv) >> 28) & 8u;
                const float ax = fabsf(xv);
                const uint32_t h = SR ? draw16(draws, j) : 0u;
                if (TWO_D) {
                    // one code per element, emitted in both layouts
                    const uint32_t nib = e2m1_rne_nibble(ax * r2, sign8);
                    if (ROW)
                        roww |= nib << (4 * j);
                    if (COL)
                        colw[j][i >> 3] |= nib << (4 * (i & 7));
                } else {
                    if (COL) {
                        const float vv = ax * rc[j];
                        const uint32_t nib = SR ? e2m1_sr_nibble(vv, h, sign8) : e2m1_rne_nibble(vv, sign8);
                        colw[j][i >> 3] |= nib << (4 * (i & 7));
                    }
                    if (ROW) {
                        const float vv = ax * rr[i];
                        const uint32_t nib = SR ? e2m1_sr_nibble(vv, h, sign8) : e2m1_rne_nibble(vv, sign8);
                        roww |= nib << (4 * j);
                    }
                }
            }
            if (ROW)
                *reinterpret_cast<uint32_t*>(p.codes_row + (r0 + i) * (cols >> 1) + (c0 >> 1)) = roww;
        }

        if (TWO_D && !odd)
            p.scales_row[(r0 >> 4) * (cols >> 4) + (c0 >> 4)] = (uint8_t)tile_byte;

        if (COL) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int col = cg * 8 + j;
                const int slot = rb ^ (cg & 15);
                lds_codes[col * kRowBlocks + slot] = make_uint2(colw[j][0], colw[j][1]);
                if (!TWO_D)
                    lds_scales[col * kRowBlocks + rb] = (uint8_t)col_byte[j];
            }
        }
    }

    if (COL) {
        __syncthreads();
        // Codes: 8-byte chunks, 16 lanes per tile column (one 128-byte segment).
        const int64_t pitch = rows >> 1;
#pragma unroll
        for (int k = 0; k < kTileC * kRowBlocks / kThreads; ++k) {
            const int q = k * kThreads + threadIdx.x;
            const int col = q >> 4, part = q & 15;
            const int64_t c = tile_c0 + col, r = tile_r0 + part * 16;
            if (c < cols && r < rows) {
                const int slot = part ^ ((col >> 3) & 15);
                *reinterpret_cast<uint2*>(p.codes_col + c * pitch + (r >> 1)) =
                    lds_codes[col * kRowBlocks + slot];
            }
        }
        if (!TWO_D) {
            // Scales: one tile column's 16 bytes per thread.
            const int col = threadIdx.x;
            const int64_t c = tile_c0 + col;
            if (c < cols) {
                const int64_t spitch = rows >> 4;
                uint8_t* dst = p.scales_col + c * spitch + (tile_r0 >> 4);
                const int64_t nb64 = (rows - tile_r0) >> 4;
                const int nb = nb64 < kRowBlocks ? (int)nb64 : kRowBlocks;
                const uint8_t* srcs = &lds_scales[col * kRowBlocks];
                if (nb == kRowBlocks && ((reinterpret_cast<uintptr_t>(dst) & 15) == 0)) {
                    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(srcs);
                } else {
                    for (int b = 0; b < nb; ++b)
                        dst[b] = srcs[b];
                }
            }
        }
    }
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
    if (a.rowwise && a.colwise)
        return a.sr ? launch_variant<true, true, false, true, false>(p, stream)
                    : launch_variant<true, true, false, false, false>(p, stream);
    if (a.rowwise)
        return a.sr ? launch_variant<true, false, false, true, false>(p, stream)
                    : launch_variant<true, false, false, false, false>(p, stream);
    return a.sr ? launch_variant<false, true, false, true, false>(p, stream)
                : launch_variant<false, true, false, false, false>(p, stream);
}

}  // namespace nvfp4
