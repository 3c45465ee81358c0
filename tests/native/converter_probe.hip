// Test probe (not part of the library): runs the library's own E2M1
// encoders (fp4_block_scaled_amax_amd/csrc/encode.h, the functions the
// quantize kernels call) over every input they can meet, and condenses the
// results so that the CPU oracle can be compared with them everywhere.
//
// probe_rne_runs: every binary32 pattern of [lo, hi] through the
//   round-to-nearest encoder (unit multiplier, as the kernels call it),
//   both nibbles of all four byte positions; records each pattern whose
//   code differs from the previous pattern's (run starts).
// probe_sr_thresholds: for each value, every 16-bit draw h through the
//   stochastic column encoder in every row and column position (hardware
//   converter with its input mapping, the 2^23 operand scaling applied by
//   the encoder or carried by the multiplier), through the software encoder
//   and through the rowwise pair encoder; records the
//   code for h = 0 and h = 65535 and the number of draws giving the h = 0
//   code, and flags any value whose codes are not a prefix of one code
//   followed by the other, or on which the encoders disagree.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../fp4_block_scaled_amax_amd/csrc/encode.h"

using namespace nvfp4;

namespace {

// Low nibble of byte B of the RNE encoder's output for (v, v).
template <int B>
__device__ __forceinline__ uint32_t rne_pair(float v)
{
    const uint32_t w = put_pair<kEncHw, B>(0u, v, v, 1.0f, 0u, 0u);
    return (w >> (8 * B)) & 0xFFu;
}

__global__ void rne_runs_kernel(uint32_t lo, uint32_t hi, uint32_t chunk, uint32_t* runs, uint32_t cap,
                                uint32_t* count, uint32_t* mismatch)
{
    const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t first = (uint64_t)lo + t * chunk;
    if (first > hi)
        return;
    uint64_t last = first + chunk - 1;
    if (last > hi)
        last = hi;
    uint32_t prev = first == lo ? 0xFFFFFFFFu : (rne_pair<0>(__uint_as_float((uint32_t)(first - 1))) & 0xFu);
    uint32_t bad = 0u;
    for (uint64_t p = first; p <= last; ++p) {
        const float v = __uint_as_float((uint32_t)p);
        const uint32_t b0 = rne_pair<0>(v), b1 = rne_pair<1>(v), b2 = rne_pair<2>(v), b3 = rne_pair<3>(v);
        const uint32_t c = b0 & 0xFu;
        // both nibbles of every byte position must hold the same code
        bad |= (uint32_t)(b0 != (c | (c << 4))) | (uint32_t)(b1 != b0) | (uint32_t)(b2 != b0) |
               (uint32_t)(b3 != b0);
        if (c != prev) {
            const uint32_t k = atomicAdd(count, 1u);
            if (k < cap) {
                runs[2 * k] = (uint32_t)p;
                runs[2 * k + 1] = c;
            }
            prev = c;
        }
    }
    if (bad)
        atomicAdd(mismatch, 1u);
}

// Codes of the stochastic encoders for v with the 16 draws h0 .. h0 + 15:
// the column encoder the columnwise kernels use (encode_column16: the
// hardware converter with the 2^23 carried by the multiplier, and with it
// applied by the encoder; the software encoder), placing draw h0 + i in row
// i of column j; `agree` is cleared where the three differ or a row's code
// is not what the pair encoder (put_pair, rowwise kernels) gives.
__device__ __forceinline__ void sr_codes16(float v, uint32_t h0, int j, uint32_t (&c)[16], bool& agree)
{
    float y[16];
    uint4 draws[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        y[i] = v;
        const uint32_t h = h0 + i;
        const uint32_t word = (j & 1) ? (h << 16) : h;
        draws[i] = make_uint4((j >> 1) == 0 ? word : 0u, (j >> 1) == 1 ? word : 0u, (j >> 1) == 2 ? word : 0u,
                              (j >> 1) == 3 ? word : 0u);
    }
    const uint2 hs = encode_column16<kEncSrHwScaled>(y, 0x1p23f, draws, j);
    const uint2 hw = encode_column16<kEncSrHw>(y, 1.0f, draws, j);
    const uint2 sw = encode_column16<kEncSr>(y, 1.0f, draws, j);
    agree = agree && hs.x == hw.x && hs.y == hw.y && hs.x == sw.x && hs.y == sw.y;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        c[i] = (((i < 8) ? hs.x : hs.y) >> (4 * (i & 7))) & 0xFu;
    // the pair encoder of the rowwise kernels, rows 0 and 1 in byte 2
    const uint32_t pr = put_pair<kEncSrHw, 2>(0u, v, v, 1.0f, sr_input<kEncSrHw>(draws[0], j),
                                              sr_input<kEncSrHw>(draws[1], j));
    agree = agree && ((pr >> 16) & 0xFFu) == (c[0] | (c[1] << 4));
}

__global__ void sr_thresholds_kernel(const float* values, uint32_t n, uint32_t* out)
{
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n)
        return;
    const float v = values[i];
    bool agree = true;
    uint32_t c[16];
    sr_codes16(v, 0u, 0, c, agree);
    const uint32_t c0 = c[0];
    sr_codes16(v, 65520u, 7, c, agree);
    const uint32_t c1 = c[15];
    uint32_t count = 0u;
    bool prefix = true, two_valued = true;
    for (uint32_t h0 = 0; h0 < 65536u; h0 += 16u) {
        sr_codes16(v, h0, (h0 >> 4) & 7, c, agree);  // every column position in turn
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const bool is0 = c[k] == c0;
            two_valued = two_valued && (is0 || c[k] == c1);
            prefix = prefix && (is0 ? count == h0 + k : true);  // every h = 0 code comes first
            count += is0 ? 1u : 0u;
        }
    }
    out[4 * i + 0] = c0;
    out[4 * i + 1] = c1;
    out[4 * i + 2] = count;
    out[4 * i + 3] = (agree ? 1u : 0u) | (prefix ? 2u : 0u) | (two_valued ? 4u : 0u);
}

int status(hipError_t e) { return e == hipSuccess ? 0 : -5; }

}  // namespace

extern "C" {

// Run starts of the RNE code over the patterns lo..hi (inclusive): runs
// receives (pattern, code) pairs in no particular order, *count their
// number (may exceed cap: then only cap were stored), *mismatch the number
// of threads that saw a byte whose two nibbles or byte positions disagree.
// Device pointers; count and mismatch must be zeroed by the caller.
int probe_rne_runs(uint32_t lo, uint32_t hi, uint32_t* runs, uint32_t cap, uint32_t* count, uint32_t* mismatch,
                   hipStream_t stream)
{
    const uint32_t chunk = 4096;
    const uint64_t threads = ((uint64_t)hi - lo) / chunk + 1;
    const uint64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(rne_runs_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, lo, hi, chunk, runs, cap,
                       count, mismatch);
    return status(hipGetLastError());
}

// out[4 i ..]: code for h = 0, code for h = 65535, number of h with the
// h = 0 code, flags (1: encoders agree, 2: prefix, 4: two codes at most).
int probe_sr_thresholds(const float* values, uint32_t n, uint32_t* out, hipStream_t stream)
{
    hipLaunchKernelGGL(sr_thresholds_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, values, n, out);
    return status(hipGetLastError());
}

}  // extern "C"
