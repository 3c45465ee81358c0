// MXFP4 GEMM on the gfx950 block-scaled matrix cores: C = A * B^T (TN, both
// operands K-contiguous),
//   C[m][n] = sum_k e2m1(A[m][k]) 2^(sa[m][k/32] - 127) e2m1(B[n][k]) 2^(sb[n][k/32] - 127),
// summed in fp32 by v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands. The
// instruction applies the E8M0 block scales itself, so the packed codes go
// from memory to the matrix cores untouched.
//
// Operand layout the instruction takes (checked on the GPU against a double
// product): lane l of a 32x32x64 MFMA holds row l % 32 and the 16 code bytes
// of K elements [32 (l / 32), +32) -- one MXFP4 block -- and that block's
// scale byte, picked out of a 32-bit register by op_sel.
//
// Structure: a workgroup of WAVES_M x WAVES_N waves computes a 256 x 256
// tile of C; K advances 128 per stage (64 code bytes and one 4-byte scale
// word per row). Each stage goes global -> registers -> LDS (rows padded to
// 80 bytes, so the 16-byte reads of 8 consecutive rows hit distinct banks),
// double-buffered, with the next stage's loads in flight during the current
// stage's MFMAs. A wave's scale word for a row is shifted by one byte in the
// upper half-wave, so op_sel 0 / 2 picks each lane's block in the two
// K = 64 steps of a stage. The grid is persistent, in the same XCD-aware
// tile order as the NVFP4 GEMM.
#include <atomic>

#include "device.h"
#include "kernels.h"

namespace nvfp4 {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 128;                       // K per stage
constexpr int kRows = kBM + kBN;               // A rows, then B rows
constexpr int kRowBytes = kBK / 2 + 16;        // 80
constexpr int kCodeBytes = kRows * kRowBytes;  // codes of one stage
constexpr int kStageBytes = kCodeBytes + kRows * 4;  // + one scale word per row
constexpr int kGroupM = 4;
constexpr uint32_t kUnitScales = 0x7F7F7F7Fu;  // four E8M0 ones

template <int WAVES_M, int WAVES_N>
struct Cfg {
    static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
    static constexpr int FM = kBM / WAVES_M / 32;  // 32-row fragments per wave
    static constexpr int FN = kBN / WAVES_N / 32;
    static constexpr int kChunks = kRows * (kBK / 32) / kThreads;  // 16-byte code chunks per thread
    static constexpr int kWords = kRows / kThreads;                 // scale words per thread
    static_assert(kRows % kThreads == 0, "scale words split evenly");
};

template <int NC, int NW>
struct Stage {
    uint4 c[NC];
    uint32_t w[NW];
};

struct Operands {
    const uint8_t* codes[2];   // A, B
    const uint8_t* scales[2];
    int64_t rows[2];           // M, N
    int64_t K;
};

// This thread's share of a stage, fixed for a tile: a 32-bit offset per
// 16-byte code chunk (from the tile's first row of that operand, at stage
// 0) and per scale word, with a validity bit each. The tile bases are
// uniform, so loads address as uniform base + 32-bit lane offset.
template <int NC, int NW>
struct Plan {
    const uint8_t* code_base[2];
    const uint8_t* scale_base[2];
    uint32_t c_off[NC];
    uint32_t w_off[NW];
    uint32_t c_ok, w_ok;   // bit i: chunk / word i lies inside the operand
};

// Chunk q = t + THREADS i covers row q / 4 of the stage (A rows first, then
// B rows; A for i < NC / 2) and its 16-byte part q % 4 (one MXFP4 block).
template <int NC, int NW, int THREADS>
__device__ __forceinline__ Plan<NC, NW> make_plan(const Operands& op, int64_t m0, int64_t n0, int t)
{
    Plan<NC, NW> pl;
    const int64_t row_bytes = op.K >> 1, nkb = op.K >> 5;
    pl.code_base[0] = op.codes[0] + m0 * row_bytes;
    pl.code_base[1] = op.codes[1] + n0 * row_bytes;
    pl.scale_base[0] = op.scales[0] + m0 * nkb;
    pl.scale_base[1] = op.scales[1] + n0 * nkb;
    pl.c_ok = 0u;
    pl.w_ok = 0u;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int q = t + THREADS * i;
        const int o = i >= NC / 2;
        const int r = (q >> 2) - o * kBM;
        pl.c_off[i] = (uint32_t)r * (uint32_t)row_bytes + 16u * (uint32_t)(q & 3);
        pl.c_ok |= ((o ? n0 : m0) + r < op.rows[o] ? 1u : 0u) << i;
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int o = i >= NW / 2 && NW > 1 ? 1 : (NW == 1 && t >= kBM ? 1 : 0);
        const int r = t + THREADS * i - o * kBM;
        pl.w_off[i] = (uint32_t)r * (uint32_t)nkb;
        pl.w_ok |= ((o ? n0 : m0) + r < op.rows[o] ? 1u : 0u) << i;
    }
    return pl;
}

// Scale word of blocks 4 s .. 4 s + 3 of one row; blocks past K read as 1
// (their codes are zero). ALIGNED: K a multiple of 128 and the scale array
// 4-byte aligned, so the word is one load.
template <bool ALIGNED>
__device__ __forceinline__ uint32_t scale_word(const uint8_t* row_scales, int s, int64_t nkb)
{
    if (ALIGNED)
        return *reinterpret_cast<const uint32_t*>(row_scales + 4 * s);
    uint32_t w = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t kb = 4 * (int64_t)s + i;
        w |= (kb < nkb ? (uint32_t)row_scales[kb] : 0x7Fu) << (8 * i);
    }
    return w;
}

template <int NC, int NW, int THREADS, bool ALIGNED>
__device__ __forceinline__ Stage<NC, NW> fetch(const Plan<NC, NW>& pl, int64_t K, int s, int t)
{
    Stage<NC, NW> st;
    const int64_t nkb = K >> 5;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int o = i >= NC / 2;
        const bool in_k = ALIGNED || 4 * (int64_t)s + ((t + THREADS * i) & 3) < nkb;
        st.c[i] = make_uint4(0u, 0u, 0u, 0u);
        if (((pl.c_ok >> i) & 1u) && in_k)
            st.c[i] = load16(pl.code_base[o] + (pl.c_off[i] + 64u * (uint32_t)s));
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int o = i >= NW / 2 && NW > 1 ? 1 : (NW == 1 && t >= kBM ? 1 : 0);
        st.w[i] = ((pl.w_ok >> i) & 1u) ? scale_word<ALIGNED>(pl.scale_base[o] + pl.w_off[i], s, nkb) : kUnitScales;
    }
    return st;
}

template <int NC, int NW, int THREADS>
__device__ __forceinline__ void store_stage(const Stage<NC, NW>& st, uint8_t* buf, int t)
{
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int q = t + THREADS * i;
        *reinterpret_cast<uint4*>(buf + (q >> 2) * kRowBytes + 16 * (q & 3)) = st.c[i];
    }
#pragma unroll
    for (int i = 0; i < NW; ++i)
        *reinterpret_cast<uint32_t*>(buf + kCodeBytes + 4 * (t + THREADS * i)) = st.w[i];
}

__device__ __forceinline__ i32x8 fragment(const uint8_t* buf, int row, int kbyte)
{
    const uint4 v = *reinterpret_cast<const uint4*>(buf + row * kRowBytes + kbyte);
    return i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
}

// The MFMAs of one stage for this wave's (32 FM) x (32 FN) sub-tile.
template <int FM, int FN>
__device__ __forceinline__ void stage_mfma(const uint8_t* buf, int wm, int wn, int lane,
                                           f32x16 (&acc)[FM][FN])
{
    const int frow = lane & 31, half = lane >> 5;
    int sa[FM], sb[FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
        sa[a] = (int)(*reinterpret_cast<const uint32_t*>(buf + kCodeBytes + 4 * (wm + 32 * a + frow)) >> (8 * half));
#pragma unroll
    for (int b = 0; b < FN; ++b)
        sb[b] = (int)(*reinterpret_cast<const uint32_t*>(buf + kCodeBytes + 4 * (kBM + wn + 32 * b + frow)) >>
                      (8 * half));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        i32x8 fa[FM], fb[FN];
#pragma unroll
        for (int a = 0; a < FM; ++a)
            fa[a] = fragment(buf, wm + 32 * a + frow, 32 * ks + 16 * half);
#pragma unroll
        for (int b = 0; b < FN; ++b)
            fb[b] = fragment(buf, kBM + wn + 32 * b + frow, 32 * ks + 16 * half);
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                if (ks == 0)
                    acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[a], fb[b], acc[a][b], 4, 4, 0,
                                                                                sa[a], 0, sb[b]);
                else
                    acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[a], fb[b], acc[a][b], 4, 4, 2,
                                                                                sa[a], 2, sb[b]);
            }
    }
}

__device__ __forceinline__ int mx_tile_index(int round)
{
    const int G = gridDim.x;
    int w = blockIdx.x;
    if ((G & 7) == 0)
        w = (w & 7) * (G >> 3) + (w >> 3);
    return round * G + w;
}

template <int WAVES_M, int WAVES_N, bool BF16_OUT, bool ALIGNED>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void mx_gemm_kernel(MxGemmArgs g, int tiles_m,
                                                                                  int tiles_n)
{
    using C = Cfg<WAVES_M, WAVES_N>;
    constexpr int FM = C::FM, FN = C::FN;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStageBytes];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = (wave / WAVES_N) * (kBM / WAVES_M), wn = (wave % WAVES_N) * (kBN / WAVES_N);
    const int nst = (int)((g.K + kBK - 1) / kBK);
    Operands op;
    op.codes[0] = g.a_codes;
    op.codes[1] = g.b_codes;
    op.scales[0] = g.a_scales;
    op.scales[1] = g.b_scales;
    op.rows[0] = g.M;
    op.rows[1] = g.N;
    op.K = g.K;
    using P = Plan<C::kChunks, C::kWords>;

    const int nt = tiles_m * tiles_n;
    for (int round = 0;; ++round) {
        const int tile = mx_tile_index(round);
        if (tile >= nt)
            break;
        const int group = tile / (kGroupM * tiles_n);
        const int gm = min(kGroupM, tiles_m - group * kGroupM);
        const int in_group = tile - group * kGroupM * tiles_n;
        const int tm = group * kGroupM + in_group % gm, tn = in_group / gm;
        const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
        const P pl = make_plan<C::kChunks, C::kWords, C::kThreads>(op, m0, n0, t);

        f32x16 acc[FM][FN];
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
                acc[a][b] = f32x16{};

        auto st = fetch<C::kChunks, C::kWords, C::kThreads, ALIGNED>(pl, g.K, 0, t);
        store_stage<C::kChunks, C::kWords, C::kThreads>(st, lds, t);
        if (nst > 1)
            st = fetch<C::kChunks, C::kWords, C::kThreads, ALIGNED>(pl, g.K, 1, t);
        __syncthreads();
        for (int s = 0; s < nst; ++s) {
            uint8_t* cur = lds + (s & 1) * kStageBytes;
            stage_mfma<FM, FN>(cur, wm, wn, lane, acc);
            if (s + 1 < nst) {
                store_stage<C::kChunks, C::kWords, C::kThreads>(st, lds + ((s + 1) & 1) * kStageBytes, t);
                if (s + 2 < nst)
                    st = fetch<C::kChunks, C::kWords, C::kThreads, ALIGNED>(pl, g.K, s + 2, t);
            }
            __syncthreads();
        }

        // Epilogue: the wave's sub-tile corner is a uniform base, element
        // offsets are 32-bit. The lane indices are made opaque per tile so
        // the compiler recomputes each offset at its store instead of
        // hoisting all of them out of the tile loop (which would not fit).
        int lr = 4 * (lane >> 5), lc = lane & 31;
        asm volatile("" : "+v"(lr), "+v"(lc));
        const int64_t wr0 = m0 + wm, wc0 = n0 + wn;
        const uint32_t ldc = (uint32_t)g.N;
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            const int c = 32 * b + lc;
            if (wc0 + c >= g.N)
                continue;
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = 32 * a + 8 * (i >> 2) + lr + (i & 3);
                    if (wr0 + r >= g.M)
                        continue;
                    const uint32_t off = (uint32_t)r * ldc + (uint32_t)c;
                    if (BF16_OUT) {
                        const uint32_t u = __float_as_uint(acc[a][b][i]);
                        (reinterpret_cast<uint16_t*>(g.c) + (wr0 * g.N + wc0))[off] =
                            (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
                    } else {
                        (reinterpret_cast<float*>(g.c) + (wr0 * g.N + wc0))[off] = acc[a][b][i];
                    }
                }
        }
    }
}

template <int WAVES_M, int WAVES_N, bool BF16_OUT, bool ALIGNED>
int mx_gemm_capacity()
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
            &per_cu, reinterpret_cast<const void*>(mx_gemm_kernel<WAVES_M, WAVES_N, BF16_OUT, ALIGNED>),
            Cfg<WAVES_M, WAVES_N>::kThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    c = (per_cu > 0 ? per_cu : 1) * cus;
    if (c > 0)
        cache[dev].store(c, std::memory_order_relaxed);
    return c;
}

template <bool BF16_OUT, bool ALIGNED>
hipError_t launch_mx_variant(const MxGemmArgs& a, int tiles_m, int tiles_n, hipStream_t stream)
{
    constexpr int WM = 2, WN = 4;  // wave grid of the 256 x 256 tile: 2 x 4 waves of 128 x 64
    const int cap = mx_gemm_capacity<WM, WN, BF16_OUT, ALIGNED>();
    if (cap <= 0)
        return hipErrorInvalidDevice;
    const int nt = tiles_m * tiles_n;
    const dim3 grid((unsigned)(nt < cap ? nt : cap));
    hipLaunchKernelGGL((mx_gemm_kernel<WM, WN, BF16_OUT, ALIGNED>), grid, dim3(Cfg<WM, WN>::kThreads), 0, stream, a,
                       tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_gemm(const MxGemmArgs& a, hipStream_t stream)
{
    const int tiles_m = (int)((a.M + kBM - 1) / kBM);
    const int tiles_n = (int)((a.N + kBN - 1) / kBN);
    const bool aligned = (a.K % kBK) == 0 && ((reinterpret_cast<uintptr_t>(a.a_scales) & 3) == 0) &&
                         ((reinterpret_cast<uintptr_t>(a.b_scales) & 3) == 0);
    if (a.c_bf16)
        return aligned ? launch_mx_variant<true, true>(a, tiles_m, tiles_n, stream)
                       : launch_mx_variant<true, false>(a, tiles_m, tiles_n, stream);
    return aligned ? launch_mx_variant<false, true>(a, tiles_m, tiles_n, stream)
                   : launch_mx_variant<false, false>(a, tiles_m, tiles_n, stream);
}

}  // namespace nvfp4
