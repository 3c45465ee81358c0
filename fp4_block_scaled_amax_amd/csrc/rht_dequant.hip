// Standalone 16-point Hadamard transform (binary32 output) and NVFP4
// dequantization.
#include "device.h"
#include "kernels.h"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;

int grid_for(int64_t items)
{
    int64_t g = (items + kThreads - 1) / kThreads;
    if (g < 1)
        g = 1;
    if (g > 8192)
        g = 8192;
    return (int)g;
}

// Axis 0: item = 16 rows x 8 columns; writes the same footprint as fp32.
__global__ __launch_bounds__(kThreads) void rht16_axis0_kernel(const uint16_t* __restrict__ x,
                                                                int64_t rows, int64_t cols,
                                                                uint32_t mask,
                                                                float* __restrict__ y)
{
    const int64_t groups = cols >> 3;
    const int64_t items = (rows >> 4) * groups;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t it = (int64_t)blockIdx.x * kThreads + threadIdx.x; it < items; it += stride) {
        const int64_t rb = it / groups, cg = it - rb * groups;
        const int64_t off = (rb * 16) * cols + cg * 8;
        uint4 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            v[i] = load16_stream(x + off + i * cols);
        float z[8][16];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                z[j][i] = bf16_at(v[i], j);
            rht16_inplace(z[j], mask);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float4* dst = reinterpret_cast<float4*>(y + off + i * cols);
            store16_stream(dst, make_float4(z[0][i], z[1][i], z[2][i], z[3][i]));
            store16_stream(dst + 1, make_float4(z[4][i], z[5][i], z[6][i], z[7][i]));
        }
    }
}

// Axis 1: item = one 16-element segment of a row.
__global__ __launch_bounds__(kThreads) void rht16_axis1_kernel(const uint16_t* __restrict__ x,
                                                                int64_t nseg, uint32_t mask,
                                                                float* __restrict__ y)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t s = (int64_t)blockIdx.x * kThreads + threadIdx.x; s < nseg; s += stride) {
        const uint4 a = load16_stream(x + s * 16);
        const uint4 b = load16_stream(x + s * 16 + 8);
        float z[16];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            z[j] = bf16_at(a, j);
            z[j + 8] = bf16_at(b, j);
        }
        rht16_inplace(z, mask);
        float4* dst = reinterpret_cast<float4*>(y + s * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            store16_stream(dst + q, make_float4(z[4 * q], z[4 * q + 1], z[4 * q + 2], z[4 * q + 3]));
    }
}

// binary32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// One 16-element block per item: 8 bytes of codes and one scale byte.
// Magnitude m decodes through a packed table of 2*value: {0,1,2,3,4,6,8,12}.
template <bool TWO_D, bool BF16>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(const uint8_t* __restrict__ codes,
                                                               const uint8_t* __restrict__ scales,
                                                               const float* __restrict__ sgp,
                                                               int64_t rows, int64_t cols,
                                                               void* __restrict__ out)
{
    const float sg = *sgp;
    const int64_t bpr = cols >> 4;  // blocks per row
    const int64_t nblocks = rows * bpr;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x; blk < nblocks; blk += stride) {
        const uint2 cw = load8_stream(codes + blk * 8);
        const int64_t r = blk / bpr, cb = blk - r * bpr;
        const uint32_t sb = TWO_D ? scales[(r >> 4) * bpr + cb] : scales[blk];
        const float hs = 0.5f * e4m3_decode(sb);  // exact
        float val[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const uint32_t word = (k < 8) ? cw.x : cw.y;
            const uint32_t nib = (word >> (4 * (k & 7))) & 15u;
            const uint32_t twice = __builtin_amdgcn_ubfe(0xC8643210u, 4u * (nib & 7u), 4u);
            const float mag = ((float)twice * hs) * sg;
            val[k] = __uint_as_float(__float_as_uint(mag) | ((nib & 8u) << 28));
        }
        if (BF16) {
            uint4* dst = reinterpret_cast<uint4*>(out) + blk * 2;
            uint32_t w[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                w[q] = f32_to_bf16_rne(val[2 * q]) | (f32_to_bf16_rne(val[2 * q + 1]) << 16);
            store16_stream(dst, make_uint4(w[0], w[1], w[2], w[3]));
            store16_stream(dst + 1, make_uint4(w[4], w[5], w[6], w[7]));
        } else {
            float4* dst = reinterpret_cast<float4*>(out) + blk * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                store16_stream(dst + q, make_float4(val[4 * q], val[4 * q + 1], val[4 * q + 2], val[4 * q + 3]));
        }
    }
}

}  // namespace

hipError_t launch_rht16(const uint16_t* x, int64_t rows, int64_t cols, int axis, uint32_t mask,
                        float* y, hipStream_t stream)
{
    if (axis == 0) {
        const int64_t items = (rows >> 4) * (cols >> 3);
        hipLaunchKernelGGL(rht16_axis0_kernel, dim3(grid_for(items)), dim3(kThreads), 0, stream, x,
                           rows, cols, mask, y);
    } else {
        const int64_t nseg = rows * (cols >> 4);
        hipLaunchKernelGGL(rht16_axis1_kernel, dim3(grid_for(nseg)), dim3(kThreads), 0, stream, x,
                           nseg, mask, y);
    }
    return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, bool two_d,
                             const float* global_scale, int64_t rows, int64_t cols, void* out,
                             bool bf16_out, hipStream_t stream)
{
    const int grid = grid_for(rows * (cols >> 4));
    if (two_d) {
        if (bf16_out)
            hipLaunchKernelGGL((dequantize_kernel<true, true>), dim3(grid), dim3(kThreads), 0, stream,
                               codes, scales, global_scale, rows, cols, out);
        else
            hipLaunchKernelGGL((dequantize_kernel<true, false>), dim3(grid), dim3(kThreads), 0, stream,
                               codes, scales, global_scale, rows, cols, out);
    } else {
        if (bf16_out)
            hipLaunchKernelGGL((dequantize_kernel<false, true>), dim3(grid), dim3(kThreads), 0, stream,
                               codes, scales, global_scale, rows, cols, out);
        else
            hipLaunchKernelGGL((dequantize_kernel<false, false>), dim3(grid), dim3(kThreads), 0, stream,
                               codes, scales, global_scale, rows, cols, out);
    }
    return hipGetLastError();
}

}  // namespace nvfp4
