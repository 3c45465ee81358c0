// Dequantize-and-contract NVFP4 GEMM: C = (S_gA * S_gB) * sum_k Ahat Bhat,
// TN layout (both operands K-contiguous).
//
// Every operand element e2m1(code) * e4m3(scale) has at most 6 significant
// bits and lies in [2^-10, 2688], so it is exact in bf16; products are summed
// in fp32 by v_mfma_f32_32x32x16_bf16. One MFMA consumes K = 16, exactly one
// NVFP4 scale block.
//
// Structure (one workgroup = 8 waves, a 256 x 256 tile of C):
//   - K advances 32 at a time. Each of the 512 threads owns one row (256 of
//     A, then 256 of B) for the stage: it loads 16 bytes of packed codes and
//     the two scale bytes, decodes the 32 codes (hardware FP4 -> fp32
//     convert, times the scale, exact; packed to bf16, exact) and writes them
//     to LDS. Each element is decoded once per workgroup.
//   - LDS rows are 80 bytes apart (32 bf16 + 16 bytes of padding) so the
//     16-byte operand reads of 8 consecutive rows hit distinct banks.
//   - Waves form a 4 x 2 grid; each computes a 64 x 128 sub-tile (2 x 4 MFMA
//     tiles, 128 fp32 accumulators per lane), so two waves share a SIMD and
//     one's decode overlaps the other's MFMAs. Stages are double-buffered in
//     LDS, and the packed codes are fetched two stages ahead.
#include "device.h"
#include "kernels.h"

namespace nvfp4 {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float floatx16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kThreads = 512;
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 32;
constexpr int kRowBytes = kBK * 2 + 16;          // 80: padded LDS row of bf16
constexpr int kStageBytes = (kBM + kBN) * kRowBytes;  // A rows then B rows

// E4M3 scale byte -> binary32, branch-free (0x7F decodes to NaN).
__device__ __forceinline__ float scale_value(uint32_t b)
{
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    const float sub = (float)m * 0.001953125f;  // exponent field 0: m * 2^-9
    const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
    const float v = e == 0u ? sub : nrm;
    return b == 0x7Fu ? __uint_as_float(0x7FC00000u) : v;
}

// Two codes (byte SEL of `w`) times scale s -> two bf16 packed in a dword.
template <int SEL>
__device__ __forceinline__ uint32_t decode_pair(uint32_t w, float s)
{
    const auto g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
    const float a = g[0] * s, b = g[1] * s;  // exact: <= 6 significant bits
    const bf16x2 p = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32 (exact here)
    return __builtin_bit_cast(uint32_t, p);
}

// One row's packed codes for a K stage: 16 bytes (32 codes) and the two
// scale bytes (low byte: first 16 codes).
struct RowStage {
    uint4 codes;
    uint32_t scales;
};

// Fetch stage `stage` of this thread's row; rows past the end read row 0
// of the operand and are zeroed (codes and scales 0 decode to 0).
template <bool WIDE>
__device__ __forceinline__ RowStage fetch_stage(const uint8_t* code_row, const uint8_t* scale_row,
                                                int stage, int64_t K, bool valid)
{
    RowStage st;
    const int64_t k0 = (int64_t)stage * kBK;
    if (WIDE) {
        st.codes = load16(code_row + (k0 >> 1));
        st.scales = *reinterpret_cast<const uint16_t*>(scale_row + (k0 >> 4));
    } else {
        // K is an odd multiple of 16: the last stage has one block.
        const bool has2 = k0 + 16 < K;
        const uint2 lo = *reinterpret_cast<const uint2*>(code_row + (k0 >> 1));
        const uint2 hi = has2 ? *reinterpret_cast<const uint2*>(code_row + (k0 >> 1) + 8) : make_uint2(0u, 0u);
        st.codes = make_uint4(lo.x, lo.y, hi.x, hi.y);
        st.scales = scale_row[k0 >> 4] | (has2 ? (uint32_t)scale_row[(k0 >> 4) + 1] << 8 : 0u);
    }
    if (!valid) {
        st.codes = make_uint4(0u, 0u, 0u, 0u);
        st.scales = 0u;
    }
    return st;
}

// Decode one row's stage and write its 32 bf16 (64 bytes) to LDS.
__device__ __forceinline__ void decode_stage_to_lds(const RowStage& st, uint8_t* lds_row)
{
    const float s0 = scale_value(st.scales & 0xFFu), s1 = scale_value((st.scales >> 8) & 0xFFu);
    const uint32_t w[4] = {st.codes.x, st.codes.y, st.codes.z, st.codes.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float sc = q < 2 ? s0 : s1;
        const u32x4 o = {decode_pair<0>(w[q], sc), decode_pair<1>(w[q], sc), decode_pair<2>(w[q], sc),
                         decode_pair<3>(w[q], sc)};
        *reinterpret_cast<u32x4*>(lds_row + 16 * q) = o;
    }
}

__device__ __forceinline__ bf16x8 lds_fragment(const uint8_t* lds, int row, int kbyte)
{
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(lds + row * kRowBytes + kbyte));
}

// The MFMAs of one stage for this wave's 64 x 128 sub-tile.
__device__ __forceinline__ void stage_mfma(const uint8_t* buf, int wm, int wn, int frow, int fk,
                                           floatx16 (&acc)[2][4])
{
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        bf16x8 fa[2], fb[4];
#pragma unroll
        for (int a = 0; a < 2; ++a)
            fa[a] = lds_fragment(buf, wm + a * 32 + frow, ks * 32 + fk);
#pragma unroll
        for (int b = 0; b < 4; ++b)
            fb[b] = lds_fragment(buf + kBM * kRowBytes, wn + b * 32 + frow, ks * 32 + fk);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
    }
}

// Workgroup -> output tile. Workgroups are dealt round-robin over the 8
// XCDs; give each XCD a contiguous range of tiles, walked along N, so the
// workgroups resident on one XCD share A rows in its L2.
__device__ __forceinline__ void gemm_tile_of_block(int tiles_m, int tiles_n, int& tm, int& tn)
{
    const int nt = tiles_m * tiles_n;
    int t = blockIdx.x;
    if ((nt & 7) == 0) {
        const int per = nt >> 3;
        t = (t & 7) * per + (t >> 3);
    }
    tm = t / tiles_n;
    tn = t % tiles_n;
}

template <bool BF16_OUT, bool WIDE>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g, int tiles_m, int tiles_n)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStageBytes];

    int tm, tn;
    gemm_tile_of_block(tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
    const int64_t K = g.K;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 128;
    const int nstages = (int)((K + kBK - 1) / kBK);

    // This thread's row: A rows 0..255, then B rows 0..255.
    const bool is_b = t >= kBM;
    const int64_t row = is_b ? n0 + (t - kBM) : m0 + t;
    const int64_t rows = is_b ? g.N : g.M;
    const bool valid = row < rows;
    const int64_t rc = valid ? row : 0;
    const uint8_t* code_row = (is_b ? g.b_codes : g.a_codes) + rc * (K >> 1);
    const bool two_d = is_b ? g.b_two_d : g.a_two_d;
    const uint8_t* scale_row = (is_b ? g.b_scales : g.a_scales) + (two_d ? (rc >> 4) : rc) * (K >> 4);
    uint8_t* my_row0 = lds + t * kRowBytes;

    floatx16 acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
            acc[a][b] = floatx16{};

    const int last = nstages - 1;
    decode_stage_to_lds(fetch_stage<WIDE>(code_row, scale_row, 0, K, valid), my_row0);
    RowStage st1 = fetch_stage<WIDE>(code_row, scale_row, min(1, last), K, valid);  // stage s+1
    RowStage st2 = fetch_stage<WIDE>(code_row, scale_row, min(2, last), K, valid);  // stage s+2
    __syncthreads();

    const int frow = lane & 31;
    const int fk = (lane >> 5) * 16;  // byte offset of the lane's 8 K-elements
    for (int s = 0; s < nstages; ++s) {
        const int cur = (s & 1) * kStageBytes;
        // MFMAs of stage s; decode stage s+1 into the other buffer (after the
        // last stage this decodes a repeat of it into the idle buffer).
        stage_mfma(lds + cur, wm, wn, frow, fk, acc);
        decode_stage_to_lds(st1, my_row0 + (kStageBytes - cur));
        // (the compiler interleaves the decode with the MFMAs well enough; an
        // explicit sched_group_barrier pattern measured slower)
        st1 = st2;
        st2 = fetch_stage<WIDE>(code_row, scale_row, min(s + 3, last), K, valid);
        __syncthreads();
    }

    const float scale = (*g.a_sg) * (*g.b_sg);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t col = n0 + wn + b * 32 + (lane & 31);
            if (col >= g.N)
                continue;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int64_t r = m0 + wm + a * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                if (r >= g.M)
                    continue;
                const float v = acc[a][b][i] * scale;
                if (BF16_OUT) {
                    const uint32_t u = __float_as_uint(v);
                    reinterpret_cast<uint16_t*>(g.c)[r * g.N + col] =
                        (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
                } else {
                    reinterpret_cast<float*>(g.c)[r * g.N + col] = v;
                }
            }
        }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream)
{
    const int tiles_m = (int)((a.M + kBM - 1) / kBM);
    const int tiles_n = (int)((a.N + kBN - 1) / kBN);
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    const bool wide = (a.K % kBK) == 0;
    if (a.c_bf16) {
        if (wide)
            hipLaunchKernelGGL((gemm_kernel<true, true>), grid, dim3(kThreads), 0, stream, a, tiles_m, tiles_n);
        else
            hipLaunchKernelGGL((gemm_kernel<true, false>), grid, dim3(kThreads), 0, stream, a, tiles_m, tiles_n);
    } else {
        if (wide)
            hipLaunchKernelGGL((gemm_kernel<false, true>), grid, dim3(kThreads), 0, stream, a, tiles_m, tiles_n);
        else
            hipLaunchKernelGGL((gemm_kernel<false, false>), grid, dim3(kThreads), 0, stream, a, tiles_m, tiles_n);
    }
    return hipGetLastError();
}

}  // namespace nvfp4
