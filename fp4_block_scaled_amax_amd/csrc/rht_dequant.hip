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

// Axis 0: item = 16 rows x 4 columns (an 8-byte load and a 16-byte binary32
// store per row), so the 64 lanes of a wave cover 256 consecutive columns:
// 512 contiguous bytes per load and 1 KB per store instruction. The output
// uses plain stores (the streaming hint measured 18% slower here).
__global__ __launch_bounds__(kThreads) void rht16_axis0_kernel(const uint16_t* __restrict__ x,
                                                                int64_t rows, int64_t cols,
                                                                uint32_t mask,
                                                                float* __restrict__ y)
{
    const int64_t groups = cols >> 2;
    const int64_t items = (rows >> 4) * groups;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t it = (int64_t)blockIdx.x * kThreads + threadIdx.x; it < items; it += stride) {
        const int64_t rb = it / groups, cg = it - rb * groups;
        const int64_t off = (rb * 16) * cols + cg * 4;
        uint2 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            v[i] = load8_stream(x + off + i * cols);
            v[i].x ^= rht_row_sign(mask, i);
            v[i].y ^= rht_row_sign(mask, i);
        }
        float z[4][16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            z[0][i] = bf16_lo(v[i].x);
            z[1][i] = bf16_hi(v[i].x);
            z[2][i] = bf16_lo(v[i].y);
            z[3][i] = bf16_hi(v[i].y);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            rht16_signed(z[j]);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            *reinterpret_cast<float4*>(y + off + i * cols) = make_float4(z[0][i], z[1][i], z[2][i], z[3][i]);
    }
}

// Axis 1: item = one 16-element segment of a row.
__global__ __launch_bounds__(kThreads) void rht16_axis1_kernel(const uint16_t* __restrict__ x,
                                                                int64_t nseg, uint32_t mask,
                                                                float* __restrict__ y)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t s = (int64_t)blockIdx.x * kThreads + threadIdx.x; s < nseg; s += stride) {
        uint4 a = load16_stream(x + s * 16);
        uint4 b = load16_stream(x + s * 16 + 8);
        a = make_uint4(a.x ^ rht_pair_sign(mask, 0), a.y ^ rht_pair_sign(mask, 1), a.z ^ rht_pair_sign(mask, 2),
                       a.w ^ rht_pair_sign(mask, 3));
        b = make_uint4(b.x ^ rht_pair_sign(mask, 4), b.y ^ rht_pair_sign(mask, 5), b.z ^ rht_pair_sign(mask, 6),
                       b.w ^ rht_pair_sign(mask, 7));
        float z[16];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            z[j] = bf16_at(a, j);
            z[j + 8] = bf16_at(b, j);
        }
        rht16_signed(z);
        float4* dst = reinterpret_cast<float4*>(y + s * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            dst[q] = make_float4(z[4 * q], z[4 * q + 1], z[4 * q + 2], z[4 * q + 3]);
    }
}

// binary32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Each thread owns E consecutive elements of a row (E = 4 for binary32
// output, 8 for bf16: 16 bytes either way) and walks down the rows, four
// adjacent rows at a time whose codes and scales are all loaded before
// decoding, so a wave's stores are 1 KB contiguous and the loads' latency
// overlaps. Plain stores: the streaming hint measured slower here. Decoding is exact hardware work: the
// scale byte through the E4M3 convert, two codes per E2M1 convert (unit
// scale); then (G * s) is exact and one rounding multiplies by S_g. A NaN
// scale gives NaN with the code's sign (the reconstruction negates the
// block's NaN magnitude for negative codes).
template <bool TWO_D, bool BF16>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(const uint8_t* __restrict__ codes,
                                                               const uint8_t* __restrict__ scales,
                                                               const float* __restrict__ sgp,
                                                               int64_t rows, int64_t cols,
                                                               void* __restrict__ out)
{
    constexpr int E = BF16 ? 8 : 4;
    constexpr int U = 4;  // adjacent rows whose loads are in flight together
    const int64_t chunk = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t c0 = chunk * E;
    if (c0 >= cols)
        return;
    const float sg = *sgp;
    const int64_t bpr = cols >> 4;  // scale blocks per row
    const int64_t step = gridDim.y;
    for (int64_t r0 = (int64_t)blockIdx.y * U; r0 < rows; r0 += step * U) {
        // All loads of U rows first: each row's codes and scale are a few
        // bytes, so one row at a time would leave the thread waiting on
        // load latency for every row.
        uint32_t w[U], sb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t r = r0 + u;
            w[u] = 0u;
            sb[u] = 0u;
            if (r < rows) {
                const uint8_t* cp = codes + ((r * cols + c0) >> 1);
                w[u] = BF16 ? *reinterpret_cast<const uint32_t*>(cp)
                            : (uint32_t)*reinterpret_cast<const uint16_t*>(cp);
                sb[u] = TWO_D ? scales[(r >> 4) * bpr + (c0 >> 4)] : scales[r * bpr + (c0 >> 4)];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t r = r0 + u;
            if (r >= rows)
                break;
            const float s = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sb[u], 1.0f, false)[0];
            float v[E];
#pragma unroll
            for (int j = 0; j < E / 2; ++j) {
                auto g = j == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 0)
                       : j == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 1)
                       : j == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 2)
                                : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 3);
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    v[2 * j + h] = (g[h] * s) * sg;
                if (s != s) {
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        v[2 * j + h] = __uint_as_float(0x7FC00000u | (__float_as_uint(g[h]) & 0x80000000u));
                }
            }
            if (BF16) {
                uint32_t q[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    q[k] = f32_to_bf16_rne(v[2 * k]) | (f32_to_bf16_rne(v[2 * k + 1]) << 16);
                *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + r * cols + c0) = make_uint4(q[0], q[1], q[2], q[3]);
            } else {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + r * cols + c0) = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
}

}  // namespace

hipError_t launch_rht16(const uint16_t* x, int64_t rows, int64_t cols, int axis, uint32_t mask,
                        float* y, hipStream_t stream)
{
    if (axis == 0) {
        const int64_t items = (rows >> 4) * (cols >> 2);
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
    // x: 16-byte column chunks of a row; y: groups of 4 rows, walked with a
    // stride so that about 4096 workgroups cover the tensor.
    const int64_t chunks = cols / (bf16_out ? 8 : 4);
    const int64_t gx = (chunks + kThreads - 1) / kThreads;
    int64_t gy = 4096 / gx;
    gy = gy < 1 ? 1 : gy;
    gy = gy > (rows + 3) / 4 ? (rows + 3) / 4 : gy;
    gy = gy > 65535 ? 65535 : gy;
    if (gx > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)gx, (unsigned)gy);
    if (two_d) {
        if (bf16_out)
            hipLaunchKernelGGL((dequantize_kernel<true, true>), grid, dim3(kThreads), 0, stream, codes,
                               scales, global_scale, rows, cols, out);
        else
            hipLaunchKernelGGL((dequantize_kernel<true, false>), grid, dim3(kThreads), 0, stream, codes,
                               scales, global_scale, rows, cols, out);
    } else {
        if (bf16_out)
            hipLaunchKernelGGL((dequantize_kernel<false, true>), grid, dim3(kThreads), 0, stream, codes,
                               scales, global_scale, rows, cols, out);
        else
            hipLaunchKernelGGL((dequantize_kernel<false, false>), grid, dim3(kThreads), 0, stream, codes,
                               scales, global_scale, rows, cols, out);
    }
    return hipGetLastError();
}

}  // namespace nvfp4
