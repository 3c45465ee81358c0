// Tensor-wide amax: integer maximum of |x| bit patterns, one atomic per
// workgroup. Exact and independent of launch geometry.
#include "device.h"
#include "kernels.h"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
// The plain amax is one read pass: few, wide workgroups (one atomic each,
// so a few hundred atomics on one address instead of thousands).
constexpr int kAmaxThreads = 1024;
constexpr int kAmaxMaxBlocks = 256;
// The transform's amax: the pipelined loop (two register sets, two
// workgroups per CU) where the butterflies would otherwise wait for the
// loads, the plain loop (more waves per SIMD) for large tensors.
constexpr int64_t kRhtPipeItems = (int64_t)1 << 18;
constexpr int kRhtPipeBlocks = 512;

__global__ void amax_reset_kernel(uint32_t* out, int n)
{
    if ((int)threadIdx.x < n)
        out[threadIdx.x] = 0u;
}

// Reduce a per-thread maximum (binary32 bits) over the workgroup and merge
// it into *out. PEEK: read *out first and skip the atomic when it cannot
// raise the value (*out only grows during the launch, so the result is the
// same). For launches of one or two workgroups per CU, whose maxima all
// arrive at the end, that leaves few of the same-address atomics to queue:
// the plain amax of 8192x4096 15.5 -> 14.7 us. With four workgroups per CU
// (1024 atomics spread over the launch) the extra read cost more than it
// saved (44.3 -> 46.1 us on 8192x14336), so that path merges directly.
template <int THREADS, bool PEEK>
__device__ __forceinline__ void workgroup_max_to(uint32_t m, uint32_t* out)
{
    __shared__ uint32_t partial[THREADS / 64];
    m = wave_max_u32(m);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0)
        partial[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = partial[0];
#pragma unroll
        for (int w = 1; w < THREADS / 64; ++w)
            r = max(r, partial[w]);
        if (!PEEK || r > __hip_atomic_load(out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            atomicMax(out, r);
    }
}

// bf16 [n]: 16-byte vectors, UNROLL loads in flight per thread. Plain
// (cache-allocating) loads: the quantize pass that follows an amax re-reads
// the same tensor and then finds it in the Infinity Cache (amax + quantize
// row+col of 8192x4096: 35.9 us, against 39.7 us with streaming loads).
template <int UNROLL>
__global__ __launch_bounds__(kAmaxThreads) void amax_bf16_kernel(const uint4* __restrict__ x,
                                                              int64_t nvec,
                                                              const uint16_t* __restrict__ tail,
                                                              int tail_n, uint32_t* __restrict__ out)
{
    uint32_t pm = 0u;  // two u16 maxima of |bf16| patterns
    const int64_t stride = (int64_t)gridDim.x * kAmaxThreads;
    int64_t i = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x;
    for (; i + (UNROLL - 1) * stride < nvec; i += UNROLL * stride) {
        uint4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            v[u] = load16(&x[i + u * stride]);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            pm = pk_max_u16(pm, v[u].x & 0x7FFF7FFFu);
            pm = pk_max_u16(pm, v[u].y & 0x7FFF7FFFu);
            pm = pk_max_u16(pm, v[u].z & 0x7FFF7FFFu);
            pm = pk_max_u16(pm, v[u].w & 0x7FFF7FFFu);
        }
    }
    // The last partial round: fewer than UNROLL strides remain, and all of
    // them are loaded at once so they are in flight together (a loop of
    // single loads left one 16-byte load per thread in flight there: half
    // a round of the 8192x14336 gradient, 0.75 of one for 14336x4096).
    // Indices past the end load the last vector again, which leaves the
    // maximum unchanged and keeps the loads unconditional.
    if (i < nvec) {
        uint4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            v[u] = load16(&x[min(i + u * stride, nvec - 1)]);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            pm = pk_max_u16(pm, v[u].x & 0x7FFF7FFFu);
            pm = pk_max_u16(pm, v[u].y & 0x7FFF7FFFu);
            pm = pk_max_u16(pm, v[u].z & 0x7FFF7FFFu);
            pm = pk_max_u16(pm, v[u].w & 0x7FFF7FFFu);
        }
    }
    uint32_t m = max(pm & 0xFFFFu, pm >> 16);
    if (blockIdx.x == 0 && (int)threadIdx.x < tail_n)
        m = max(m, (uint32_t)(tail[threadIdx.x] & 0x7FFFu));
    workgroup_max_to<kAmaxThreads, true>(m << 16, out);
}

// amax of the 16-point Hadamard transform along axis 0. Work item: 16 rows
// x 8 columns (sixteen 16-byte loads), transformed per column in registers;
// the sign diagonal is applied to the packed words, the 1/4 to the maximum.
// BOTH: the same read also gives the plain amax (into out[0]; the
// transform's into out[1]), half an integer max per element more.
//
// Each thread walks items of 16 rows x 8 columns. PIPE: it loads the next
// item into the other of two register sets before transforming the current
// one, so the butterflies overlap the loads in flight (two waves per SIMD
// with buffer loads, see rht_load_item_buf); else one item at a time, with
// more waves per SIMD to overlap them instead.

// Load one item: 16 rows of 8 bf16, sign-flipped by the mask; with BOTH
// also fold the raw magnitudes into pm.
template <bool BOTH>
__device__ __forceinline__ void rht_load_item(const uint16_t* __restrict__ x, int64_t cols, int64_t groups,
                                              int64_t it, uint4 (&v)[16])
{
    const int64_t rb = it / groups, cg = it - rb * groups;
    const uint16_t* base = x + (rb * 16) * cols + cg * 8;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        v[i] = load16(base + i * cols);
}

// The same item through buffer loads (tensors under 2 GiB): one 32-bit
// offset serves all 16 rows, the row stride rides in a scalar register, so
// an item in flight holds no 64-bit addresses. That keeps the pipelined loop
// at 215 VGPRs (247 with BOTH) and two waves per SIMD; with per-row 64-bit
// addresses it took 256 VGPRs and 26 AGPRs, one wave per SIMD.
__device__ __forceinline__ void rht_load_item_buf(__amdgpu_buffer_rsrc_t rsrc, int64_t cols, int64_t groups,
                                                  int64_t it, uint4 (&v)[16])
{
    const int64_t rb = it / groups, cg = it - rb * groups;
    const int off = (int)(((rb * 16) * cols + cg * 8) * 2);
    const int rs = (int)(cols * 2);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const auto r = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, i * rs, 0);
        v[i] = make_uint4(r[0], r[1], r[2], r[3]);
    }
}

template <bool BOTH>
__device__ __forceinline__ void rht_item_max(uint4 (&v)[16], uint32_t mask, uint32_t& pm, uint32_t& m)
{
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (BOTH) {
            pm = pk_max_u16(pm, v[i].x & 0x7FFF7FFFu);
            pm = pk_max_u16(pm, v[i].y & 0x7FFF7FFFu);
            pm = pk_max_u16(pm, v[i].z & 0x7FFF7FFFu);
            pm = pk_max_u16(pm, v[i].w & 0x7FFF7FFFu);
        }
        const uint32_t sg = rht_row_sign(mask, i);
        v[i] = make_uint4(v[i].x ^ sg, v[i].y ^ sg, v[i].z ^ sg, v[i].w ^ sg);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float z[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            z[i] = bf16_at(v[i], j);
        hadamard16(z);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            m = max(m, __float_as_uint(z[i]) & 0x7FFFFFFFu);
    }
}

template <bool BOTH, bool PIPE, bool BUF>
__global__ __launch_bounds__(kThreads) void amax_rht_kernel(const uint16_t* __restrict__ x,
                                                             int64_t rows, int64_t cols,
                                                             uint32_t mask,
                                                             uint32_t* __restrict__ out)
{
    uint32_t pm = 0u;  // BOTH: two u16 maxima of |bf16| patterns
    const int64_t groups = cols >> 3;
    const int64_t items = (rows >> 4) * groups;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    uint32_t m = 0u;
    int64_t it = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (!PIPE) {
        for (; it < items; it += stride) {
            uint4 v[16];
            rht_load_item<BOTH>(x, cols, groups, it, v);
            rht_item_max<BOTH>(v, mask, pm, m);
        }
    }
    uint4 va[16], vb[16];
    // 0x00020000: the gfx9 raw-buffer configuration word (unused without BUF)
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x), 0, BUF ? (int)(rows * cols * 2) : 0, 0x00020000);
    auto load = [&](int64_t i, uint4 (&v)[16]) {
        if (BUF)
            rht_load_item_buf(rsrc, cols, groups, i, v);
        else
            rht_load_item<BOTH>(x, cols, groups, i, v);
    };
    if (PIPE && it < items)
        load(it, va);
    while (PIPE && it < items) {
        if (it + stride < items)
            load(it + stride, vb);
        rht_item_max<BOTH>(va, mask, pm, m);
        it += stride;
        if (it >= items)
            break;
        if (it + stride < items)
            load(it + stride, va);
        rht_item_max<BOTH>(vb, mask, pm, m);
        it += stride;
    }
    // The 1/4 once, on the maximum: scaling by a power of two is monotone
    // (also where it rounds, in the subnormal range), so
    // max |fl(z / 4)| = fl(max |z| / 4), and NaN stays NaN.
    m = __float_as_uint(0.25f * __uint_as_float(m));
    if (BOTH) {
        workgroup_max_to<kThreads, PIPE>(max(pm & 0xFFFFu, pm >> 16) << 16, out);
        __syncthreads();  // the partials array is reused
        workgroup_max_to<kThreads, PIPE>(m, out + 1);
    } else {
        workgroup_max_to<kThreads, PIPE>(m, out);
    }
}

int grid_for(int64_t work_items, int per_block, int max_blocks)
{
    int64_t g = (work_items + per_block - 1) / per_block;
    if (g < 1)
        g = 1;
    if (g > max_blocks)
        g = max_blocks;
    return (int)g;
}

}  // namespace

hipError_t launch_amax(const uint16_t* x, int64_t n, float* amax, hipStream_t stream)
{
    uint32_t* out = reinterpret_cast<uint32_t*>(amax);
    hipLaunchKernelGGL(amax_reset_kernel, dim3(1), dim3(64), 0, stream, out, 1);
    const int64_t nvec = n >> 3;
    constexpr int kUnroll = 16;
    const int grid = grid_for(nvec, kAmaxThreads * kUnroll, kAmaxMaxBlocks);
    hipLaunchKernelGGL((amax_bf16_kernel<kUnroll>), dim3(grid), dim3(kAmaxThreads), 0, stream,
                       reinterpret_cast<const uint4*>(x), nvec, x + nvec * 8, (int)(n & 7), out);
    return hipGetLastError();
}

hipError_t launch_amax_rht(const uint16_t* x, int64_t rows, int64_t cols, uint32_t mask, float* amax,
                           bool both, hipStream_t stream)
{
    uint32_t* out = reinterpret_cast<uint32_t*>(amax);
    hipLaunchKernelGGL(amax_reset_kernel, dim3(1), dim3(64), 0, stream, out, both ? 2 : 1);
    const int64_t items = (rows >> 4) * (cols >> 3);
    const bool pipe = both || items <= kRhtPipeItems;
    const bool buf = rows * cols * 2 < ((int64_t)1 << 31);  // byte offsets fit the buffer loads
    const int grid = pipe ? grid_for(items, kThreads, kRhtPipeBlocks) : grid_for(items, kThreads, 1024);
    if (both && buf)
        hipLaunchKernelGGL((amax_rht_kernel<true, true, true>), dim3(grid), dim3(kThreads), 0, stream, x, rows,
                           cols, mask, out);
    else if (both)
        hipLaunchKernelGGL((amax_rht_kernel<true, true, false>), dim3(grid), dim3(kThreads), 0, stream, x, rows,
                           cols, mask, out);
    else if (pipe)
        hipLaunchKernelGGL((amax_rht_kernel<false, true, true>), dim3(grid), dim3(kThreads), 0, stream, x, rows,
                           cols, mask, out);
    else
        hipLaunchKernelGGL((amax_rht_kernel<false, false, false>), dim3(grid), dim3(kThreads), 0, stream, x, rows,
                           cols, mask, out);
    return hipGetLastError();
}

}  // namespace nvfp4
