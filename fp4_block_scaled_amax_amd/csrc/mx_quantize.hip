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
// Rowwise alone runs without LDS (mx_quantize_rows_kernel). Otherwise one
// workgroup (256 threads) stages a 128 x 128 bf16 tile in LDS with
// full-line loads, then:
//   - rowwise: a thread takes one 32-element block of a row per pass (two
//     passes); lanes 0..15 of a wave take 16 consecutive rows, so each
//     group of 8 lanes' 16-byte LDS reads hits distinct banks (rows 272
//     bytes apart);
//   - columnwise: wave w takes row block w (32 rows) of all 128 columns,
//     each lane a column pair read as 32 LDS words (256 contiguous bytes per
//     wave read); with the Hadamard transform each 16-row half of a column
//     is transformed in registers first (sign mask on the packed words,
//     butterflies, 1/4), exactly as the NVFP4 columnwise path does.
// Tiles are dealt to XCDs in runs that go down the rows, so the column
// codes of vertically adjacent tiles (halves of one 128-byte line) meet in
// one L2.
#include "device.h"
#include "kernels.h"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kTR = 128;                 // tile rows
constexpr int kTC = 128;                 // tile columns (bf16)
constexpr int kPitch = kTC * 2 + 16;     // LDS row pitch in bytes

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

// One block of 32 bf16 held as 16 packed words -> 16 code bytes + scale.
__device__ __forceinline__ uint4 mx_encode_bf16_block(const uint32_t (&w)[16], uint32_t& byte)
{
    uint32_t pm = 0u;
#pragma unroll
    for (int k = 0; k < 16; ++k)
        pm = pk_max_u16(pm, w[k] & 0x7FFF7FFFu);
    const uint32_t m = max(pm & 0xFFFFu, pm >> 16) << 16;
    byte = mx_scale_byte(m);
    const float inv = mx_inverse_scale(byte);
    const uint32_t keep = byte == 0xFFu ? 0x80008000u : 0xFFFFFFFFu;
    uint32_t out[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t x = w[4 * q + k] & keep;
            v[2 * k] = bf16_lo(x) * inv;
            v[2 * k + 1] = bf16_hi(x) * inv;
        }
        out[q] = mx_word(v);
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

// One block of 32 binary32 values -> 16 code bytes + scale.
__device__ __forceinline__ uint4 mx_encode_f32_block(const float (&y)[32], uint32_t& byte)
{
    uint32_t m = 0u;
#pragma unroll
    for (int k = 0; k < 32; ++k)
        m = max(m, __float_as_uint(y[k]) & 0x7FFFFFFFu);
    byte = mx_scale_byte(m);
    const float inv = mx_inverse_scale(byte);
    const uint32_t keep = byte == 0xFFu ? 0x80000000u : 0xFFFFFFFFu;
    uint32_t out[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            v[k] = __uint_as_float(__float_as_uint(y[8 * q + k]) & keep) * inv;
        out[q] = mx_word(v);
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

__device__ __forceinline__ void mx_tile_of_block(int tiles_r, int tiles_c, int& tr, int& tc)
{
    const int nt = tiles_r * tiles_c;
    int t = blockIdx.x;
    if ((nt & 7) == 0)
        t = (t & 7) * (nt >> 3) + (t >> 3);
    tr = t % tiles_r;
    tc = t / tiles_r;
}

template <bool ROW, bool COL, bool RHT>
__global__ __launch_bounds__(kThreads) void mx_quantize_kernel(MxQuantizeArgs p, int tiles_r, int tiles_c)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[kTR * kPitch];
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    int tr, tc;
    mx_tile_of_block(tiles_r, tiles_c, tr, tc);
    const int64_t r0 = (int64_t)tr * kTR, c0 = (int64_t)tc * kTC;
    // Rows / columns of this tile inside the tensor: the rowwise layout has
    // whole 32-column blocks, the columnwise one whole 32-row blocks and
    // 8-column chunks (16-byte loads); the other extent may be ragged.
    const int nr = (int)min((int64_t)kTR, p.rows - r0);
    const int nc = (int)min((int64_t)kTC, p.cols - c0);

    // Stage the tile: 128 rows x 16 chunks of 16 bytes; 8 chunks per thread,
    // 16 consecutive threads per row (one 256-byte span).
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int q = t + kThreads * i;
        const int r = q >> 4, part = q & 15;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (r < nr && part * 8 < nc)
            v = load16(p.x + (r0 + r) * p.cols + c0 + part * 8);
        *reinterpret_cast<uint4*>(tile + r * kPitch + part * 16) = v;
    }
    __syncthreads();

    if (ROW) {
        const int blk = lane >> 4;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = 16 * (wave + 4 * j) + (lane & 15);
            if (r < nr && blk * 32 < nc) {
                const uint8_t* src = tile + r * kPitch + blk * 64;
                uint32_t w[16];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint4 v = *reinterpret_cast<const uint4*>(src + 16 * i);
                    w[4 * i] = v.x;
                    w[4 * i + 1] = v.y;
                    w[4 * i + 2] = v.z;
                    w[4 * i + 3] = v.w;
                }
                uint32_t byte;
                const uint4 codes = mx_encode_bf16_block(w, byte);
                const int64_t row = r0 + r;
                *reinterpret_cast<uint4*>(p.codes_row + row * (p.cols >> 1) + ((c0 >> 1) + blk * 16)) = codes;
                p.scales_row[row * (p.cols >> 5) + (c0 >> 5) + blk] = (uint8_t)byte;
            }
        }
    }

    if (COL) {
        const int rb = wave;       // row block of 32
        const int cp = lane;       // column pair
        if (rb * 32 < nr && cp * 2 < nc) {
            uint32_t u[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                u[i] = *reinterpret_cast<const uint32_t*>(tile + (rb * 32 + i) * kPitch + cp * 4);
                if (RHT)
                    u[i] ^= rht_row_sign(p.mask, i & 15);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {   // column 2cp + h: low / high halves
                uint32_t byte;
                uint4 codes;
                if (RHT) {
                    float y[32];
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        float z[16];
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            z[i] = h ? bf16_hi(u[16 * s + i]) : bf16_lo(u[16 * s + i]);
                        rht16_signed(z);
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            y[16 * s + i] = z[i];
                    }
                    codes = mx_encode_f32_block(y, byte);
                } else {
                    // this column's 32 values as 16 packed words
                    uint32_t w[16];
#pragma unroll
                    for (int k = 0; k < 16; ++k) {
                        const uint32_t a = u[2 * k], b = u[2 * k + 1];
                        w[k] = h ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
                    }
                    codes = mx_encode_bf16_block(w, byte);
                }
                const int64_t col = c0 + 2 * cp + h;
                *reinterpret_cast<uint4*>(p.codes_col + col * (p.rows >> 1) + ((r0 >> 1) + rb * 16)) = codes;
                p.scales_col[col * (p.rows >> 5) + (r0 >> 5) + rb] = (uint8_t)byte;
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
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const bool first = (threadIdx.x & 3) == 0;
    for (int64_t v0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; v0 < nvec; v0 += U * stride) {
        uint4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = v0 + u * stride;
            w[u] = load16(x + 8 * (v < nvec ? v : 0));  // a quad is all in or all out
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

template <bool ROW, bool COL, bool RHT>
hipError_t launch_mx_variant(const MxQuantizeArgs& a, hipStream_t stream)
{
    const int tiles_r = (int)((a.rows + kTR - 1) / kTR);
    const int tiles_c = (int)((a.cols + kTC - 1) / kTC);
    hipLaunchKernelGGL((mx_quantize_kernel<ROW, COL, RHT>), dim3((unsigned)(tiles_r * tiles_c)),
                       dim3(kThreads), 0, stream, a, tiles_r, tiles_c);
    return hipGetLastError();
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
    if (a.rowwise && a.colwise)
        return a.rht ? hipErrorInvalidValue : launch_mx_variant<true, true, false>(a, stream);
    if (a.rowwise)
        return a.rht ? hipErrorInvalidValue : launch_mx_variant<true, false, false>(a, stream);
    return a.rht ? launch_mx_variant<false, true, true>(a, stream)
                 : launch_mx_variant<false, true, false>(a, stream);
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
