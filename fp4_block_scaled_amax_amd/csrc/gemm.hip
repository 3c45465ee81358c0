// Dequantize-and-contract NVFP4 GEMM: C = (S_gA * S_gB) * sum_k Ahat Bhat,
// TN layout (both operands K-contiguous).
//
// Every operand element e2m1(code) * e4m3(scale) has at most 6 significant
// bits and lies in [2^-10, 2688], so it is exact in bf16; the products are
// summed in fp32 by v_mfma_f32_32x32x16_bf16. One MFMA consumes K = 16, i.e.
// exactly one NVFP4 scale block per row, so a lane's 8 operand elements
// share one scale byte.
#include "device.h"
#include "kernels.h"

namespace nvfp4 {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float floatx16;

constexpr int kThreads = 256;
constexpr int kTileM = 128;
constexpr int kTileN = 128;

// 8 packed codes (one u32) times a scale -> 8 bf16 (exact).
__device__ __forceinline__ bf16x8 decode8(uint32_t codes, float hs)
{
    uint32_t out[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t h[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const uint32_t nib = (codes >> (8 * q + 4 * e)) & 15u;
            const uint32_t twice = __builtin_amdgcn_ubfe(0xC8643210u, 4u * (nib & 7u), 4u);
            const float mag = (float)twice * hs;  // exact
            h[e] = (__float_as_uint(mag) >> 16) | ((nib & 8u) << 12);
        }
        out[q] = h[0] | (h[1] << 16);
    }
    return __builtin_bit_cast(bf16x8, out);
}

struct Operand {
    const uint8_t* codes;
    const uint8_t* scales;
    bool two_d;
    int64_t rows;
};

// Lane's fragment: row `r`, elements [k0, k0+8) of a K-contiguous operand.
__device__ __forceinline__ bf16x8 load_fragment(const Operand& op, int64_t r, int64_t k0, int64_t K)
{
    if (r >= op.rows)
        return bf16x8{};
    const uint32_t codes = *reinterpret_cast<const uint32_t*>(op.codes + r * (K >> 1) + (k0 >> 1));
    const int64_t kb = k0 >> 4;
    const uint32_t sb = op.two_d ? op.scales[(r >> 4) * (K >> 4) + kb] : op.scales[r * (K >> 4) + kb];
    const float hs = 0.5f * e4m3_decode(sb);
    return decode8(codes, hs);
}

template <bool BF16_OUT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * kTileM + (wave >> 1) * 64;
    const int64_t n0 = (int64_t)blockIdx.x * kTileN + (wave & 1) * 64;
    const Operand A{g.a_codes, g.a_scales, g.a_two_d, g.M};
    const Operand B{g.b_codes, g.b_scales, g.b_two_d, g.N};
    const int64_t K = g.K;

    floatx16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
            acc[a][b] = floatx16{};

    const int row_in = lane & 31;
    const int khalf = (lane >> 5) * 8;
    for (int64_t k = 0; k < K; k += 16) {
        bf16x8 fa[2], fb[2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
            fa[a] = load_fragment(A, m0 + a * 32 + row_in, k + khalf, K);
#pragma unroll
        for (int b = 0; b < 2; ++b)
            fb[b] = load_fragment(B, n0 + b * 32 + row_in, k + khalf, K);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
    }

    const float scale = (*g.a_sg) * (*g.b_sg);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int64_t col = n0 + b * 32 + (lane & 31);
            if (col >= g.N)
                continue;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int64_t row = m0 + a * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                if (row >= g.M)
                    continue;
                const float v = acc[a][b][i] * scale;
                if (BF16_OUT) {
                    const uint32_t u = __float_as_uint(v);
                    reinterpret_cast<uint16_t*>(g.c)[row * g.N + col] =
                        (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
                } else {
                    reinterpret_cast<float*>(g.c)[row * g.N + col] = v;
                }
            }
        }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream)
{
    dim3 grid((unsigned)((a.N + kTileN - 1) / kTileN), (unsigned)((a.M + kTileM - 1) / kTileM));
    if (a.c_bf16)
        hipLaunchKernelGGL(gemm_kernel<true>, grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(gemm_kernel<false>, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace nvfp4
