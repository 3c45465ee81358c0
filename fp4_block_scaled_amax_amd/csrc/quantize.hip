// NVFP4 quantization kernels: 1D (rowwise / columnwise / both, RNE or
// stochastic, optional Hadamard) and 2D (16x16 tiles, both layouts).
//
// One workgroup (256 threads, 4 waves) owns a 128 x 256 tile of the bf16
// input. A work item is 16 rows x 8 columns (sixteen 16-byte loads); the 32
// lanes of a half-wave cover 256 consecutive columns of a row (512
// contiguous bytes per load), the two half-waves of a wave cover two row
// blocks. Inside an item:
//   - a columnwise block is one column's 16 rows (all in one lane);
//   - a rowwise block is one row's 16 columns, split over the lane pair
//     (2k, 2k+1), which trade maxima and multipliers through DPP;
//   - a 2D tile is the lane pair's 16 x 16 elements.
// Rowwise codes are stored straight from registers (128 contiguous bytes per
// row per half-wave). Columnwise codes are staged in LDS; quantize_kernel
// writes them as 64-byte column segments (tiles walked down the rows per
// XCD, so the two halves of a line meet in one L2), while
// quantize_fused_kernel holds two vertically adjacent tiles per workgroup
// and writes whole 128-byte column lines. The fused kernel serves the
// in-kernel amax (single pass) and, with the amax given, both layouts.
//
// Encoding: the element ratio v = x * r (r = 1 / (s * S_g) of its block) is
// rounded to E2M1 by the gfx950 converter v_cvt_scalef32_pk_fp4_f32 with a
// unit scale, which rounds to nearest even and saturates at +-6 exactly like
// the reference rule for every non-NaN input (checked over all 2^32 binary32
// patterns); a NaN ratio needs a non-finite r, and such blocks first map NaN
// ratios to a signed zero. Stochastic rounding runs on the SR converter
// v_cvt_scalef32_sr_pk_fp4_f32 through an input mapping that reproduces the
// rule exactly (see sr_operand); blocks with a non-finite multiplier use the
// software encoder e2m1_sr_nibble.
#include <atomic>
#include <mutex>

#include "device.h"
#include "encode.h"
#include "kernels.h"
#include "quant_item.h"

namespace nvfp4 {

namespace {

template <bool ROW, bool COL, bool TWO_D, bool SR, bool RHT>
__global__ __launch_bounds__(kThreads) void quantize_kernel(Params p)
{
    // Columnwise staging: per tile column, 8 row blocks x 8 bytes; the slot
    // of a row block is swizzled by the column group to spread LDS banks.
    __shared__ uint2 lds_codes[COL ? kTileC * kRowBlocks : 1];
    __shared__ uint8_t lds_scales[(COL && !TWO_D) ? kTileC * kRowBlocks : 16];
    __shared__ float lds_rcp[128];

    int tr, tc;
    tile_of_block(p.tiles_r, p.tiles_c, COL, tr, tc);
    const ItemPos q = item_pos(tr, tc, p.rows, p.cols);
    uint4 v[16];
    load_item(p, q, v);
    uint4 draws[16];
    if (SR && q.valid)
        item_draws(p, q, draws, true);

    const ScaleCtx sc = scale_ctx(*p.amax);
    if (p.sg_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
        *p.sg_out = sc.sg;
    // Powers of two folded into the multipliers where that is exact
    // (uniform); the columnwise-only kernels take it.
    constexpr bool kCanFold = COL && !ROW && !TWO_D && (SR || RHT);
    const bool fold = kCanFold && (SR ? (RHT ? fold_sr_scale_ok<2>(sc.sg) : fold_sr_scale_ok<0>(sc.sg))
                                      : fold_quarter_ok(sc.sg));
    build_reciprocal_table(lds_rcp, sc.sg, fold ? kFoldFactor<SR, RHT> : 1.0f);
    __syncthreads();

    if (q.valid) {
        BlockMax bm;
        if (!RHT)
            column_maxima(v, bm);
        if (ROW && !TWO_D)
            row_maxima(v, q.odd, bm);
        compute_item<ROW, COL, TWO_D, SR, RHT>(p, q, v, bm, draws, sc, lds_rcp, lds_codes, lds_scales, fold);
    }
    if (COL) {
        __syncthreads();
        write_col_tile<TWO_D>(p, q.tile_r0, q.tile_c0, lds_codes, lds_scales);
    }
}

// Rowwise only: the tensor read as a flat array of 16-byte vectors (8
// elements each). A lane takes one vector, so the lane pair (2k, 2k + 1)
// holds one 16-element block (cols is a multiple of 16, so no block
// straddles two rows) and one DPP swap gives its maximum. A workgroup takes
// kFlatU x 256 consecutive vectors (kFlatU 4 KB runs side by side) with
// streaming loads, issued before it builds its multiplier table; the codes
// leave as one 32-bit store per lane (1 KB contiguous per wave), the scale
// byte from the even lane of each pair. With stochastic rounding a vector's
// 8 draws are one Philox call whose counter is the vector's index (the
// flat index / 8, as everywhere), computed while the loads are in flight.
constexpr int kFlatU = 4;

template <int MODE>
__device__ __forceinline__ uint32_t encode_vector8(uint4 w, float r, const uint4& d)
{
    if (MODE == kEncHwSafe || MODE == kEncSr)  // keep the rare encoders' unpacking their own
        asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
    uint32_t word = MODE == kEncSr ? 0u : fresh_word();
#define NVFP4_FLAT_PAIR(K, X)                                                                         \
    word = put_pair<MODE, K>(word, bf16_lo(w.X), bf16_hi(w.X), r,                                     \
                             is_sr(MODE) ? sr_input<MODE>(d, 2 * K) : 0u,                             \
                             is_sr(MODE) ? sr_input<MODE>(d, 2 * K + 1) : 0u);
    NVFP4_FLAT_PAIR(0, x) NVFP4_FLAT_PAIR(1, y) NVFP4_FLAT_PAIR(2, z) NVFP4_FLAT_PAIR(3, w)
#undef NVFP4_FLAT_PAIR
    return word;
}

template <bool SR>
__global__ __launch_bounds__(kThreads) void quantize_rows_flat_kernel(Params p, int64_t nvec)
{
    __shared__ float lds_rcp[128];
    const int64_t v0 = (int64_t)blockIdx.x * kThreads * kFlatU + threadIdx.x;
    uint4 w[kFlatU];
#pragma unroll
    for (int u = 0; u < kFlatU; ++u) {
        const int64_t v = v0 + u * kThreads;
        w[u] = load16_stream(p.x + 8 * (v < nvec ? v : 0));  // a lane pair is all in or all out
    }
    uint4 draws[kFlatU];
    if (SR) {
#pragma unroll
        for (int u = 0; u < kFlatU; ++u) {
            const uint64_t v = (uint64_t)(v0 + u * kThreads);
            draws[u] = philox4x32_10((uint32_t)v, (uint32_t)(v >> 32), p.seed_lo, p.seed_hi);
        }
    }
    const ScaleCtx sc = scale_ctx(*p.amax);
    if (p.sg_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
        *p.sg_out = sc.sg;
    build_reciprocal_table(lds_rcp, sc.sg);
    __syncthreads();

    // Block maxima and scale bytes by the approximate chain, checked once
    // for the wave (as in the item code); the exact chain where it cannot
    // settle them.
    uint32_t bits[kFlatU], byte[kFlatU];
    ScaleVote vote;
#pragma unroll
    for (int u = 0; u < kFlatU; ++u) {
        const uint32_t pm = pk_max_u16(pk_max_u16(w[u].x & 0x7FFF7FFFu, w[u].y & 0x7FFF7FFFu),
                                       pk_max_u16(w[u].z & 0x7FFF7FFFu, w[u].w & 0x7FFF7FFFu));
        uint32_t m = max(pm & 0xFFFFu, pm >> 16);
        m = max(m, swap_lane1(m));
        bits[u] = m << 16;
        byte[u] = block_scale_byte_approx(bits[u], sc.inv_t6, vote);
    }
    bool fin = sc.table_ok;
    if (!__all(sc.fast && vote.ok())) {
        uint32_t mb = 0u;
#pragma unroll
        for (int u = 0; u < kFlatU; ++u) {
            byte[u] = scale_byte(bits[u], sc);
            mb = max(mb, byte[u]);
        }
        fin = fin && mb <= 0x7Eu;  // 0x7F (a NaN block) has no finite multiplier
    }
    float r[kFlatU];
#pragma unroll
    for (int u = 0; u < kFlatU; ++u)
        r[u] = lds_rcp[byte[u]];
    if (!sc.table_ok) {
        fin = true;
#pragma unroll
        for (int u = 0; u < kFlatU; ++u)
            fin = fin && finite_bits(r[u]);
    }
    const bool all_fin = __all(fin);
    const bool even = (threadIdx.x & 1) == 0;
#pragma unroll
    for (int u = 0; u < kFlatU; ++u) {
        const int64_t v = v0 + u * kThreads;
        if (v < nvec) {
            uint32_t code;
            if (SR)
                code = all_fin ? encode_vector8<kEncSrHw>(w[u], r[u], draws[u])
                               : encode_vector8<kEncSr>(w[u], r[u], draws[u]);
            else
                code = all_fin ? encode_vector8<kEncHw>(w[u], r[u], draws[u])
                               : encode_vector8<kEncHwSafe>(w[u], r[u], draws[u]);
            __builtin_nontemporal_store(code, reinterpret_cast<uint32_t*>(p.codes_row) + v);
            if (even)
                p.scales_row[v >> 1] = (uint8_t)byte[u];
        }
    }
}

// ---------------------------------------------------------------------------
// Fused amax + quantize: one persistent launch in which each workgroup keeps
// two vertically adjacent tiles in registers (one 256-byte work item per
// thread with round to nearest, two with stochastic rounding), so the
// tensor is read from HBM once. The workgroups exchange their block-local maxima through a
// small workspace without read-modify-write atomics: each workgroup posts
// (generation, max) in its own arrival slot, workgroup 0 collects them all
// and posts (generation, amax) in every workgroup's own release slot, so no
// address is polled by more than a few workgroups. The grid is sized so all
// workgroups fit on the device at once; the waits are bounded by wall-clock
// time and, should they expire (workgroups not co-resident), a workgroup
// computes the exact amax directly from the tensor, so the result is always
// the same and the device can never hang. With Params::amax_given the
// kernel takes the amax from memory instead and skips the exchange (then any
// grid size works): the two-layout quantize with a given amax uses it for
// its paired tiles.
//
// Workspace (32-bit words): [0] amax bits, [1] generation of the last
// completed call, [2] slow-path counter, [3] wait limit in ticks of the
// 100 MHz counter (0: the default; a tiny value makes every wait expire, so
// tests can drive the fallback), [4..5] (generation tag, count) of the
// workgroups that went through an expired exchange, then 2 words per
// workgroup of arrival slots and 2 words per workgroup of release slots.
//
// The generation may advance only once every workgroup of the call has read
// it; advancing it earlier would let a workgroup of the same call that
// starts later read the next call's generation and post a stale maximum
// under it, which the next call's workgroup 0 could take for a fresh one.
//  - When workgroup 0 collects every arrival, each arrival carries the
//    generation its workgroup read, so all have read it: workgroup 0 stores
//    the generation right after posting the releases (no atomic operation).
//  - When workgroup 0's wait expires, some workgroups may not have started.
//    Workgroup 0 then flags its releases (bit 31 of the posted amax, which an
//    amax never has), and every workgroup of the call counts itself in words
//    4..5 under the call's generation as a tag: workgroup 0, every workgroup
//    that receives a flagged release, and every workgroup whose own wait
//    expires. Each counts after reading the generation, and the one whose
//    count reaches the grid size stores the generation. (A workgroup whose
//    own wait expired in a call where workgroup 0 collected everything
//    counts too, under that call's tag; no later call shares the tag, and
//    workgroup 0 has already stored the generation.)

constexpr int kWsAmax = 0, kWsGen = 1, kWsSlow = 2, kWsWait = 3, kWsExpired = 4, kWsArrive = 16;
constexpr uint32_t kExpiredFlag = 0x80000000u;
constexpr int kMaxFusedBlocks = 2048;                       // slots in the workspace
constexpr int kWsRelease = kWsArrive + 2 * kMaxFusedBlocks;
constexpr int kMaxFusedGrid = 1024;                         // largest grid launched
constexpr uint64_t kWaitTicks = 200000;  // 2 ms of the 100 MHz real-time counter

// All exchange traffic is relaxed device-scope atomics: the value travels
// inside the atomic word itself, so no other memory needs ordering (and
// acquire/release at device scope would write back or invalidate the
// non-coherent per-XCD L2s).
__device__ __forceinline__ uint32_t ws_load(const uint32_t* a)
{
    return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ws_store(uint32_t* a, uint32_t v)
{
    __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A (generation, value) pair in one 64-bit word, so a reader sees both or neither.
__device__ __forceinline__ uint64_t slot_load(const uint32_t* a)
{
    return __hip_atomic_load(reinterpret_cast<const uint64_t*>(a), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void slot_store(uint32_t* a, uint32_t gen, uint32_t value)
{
    __hip_atomic_store(reinterpret_cast<uint64_t*>(a), ((uint64_t)value << 32) | gen,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Maximum over the workgroup; every thread gets the result.
template <int NT>
__device__ __forceinline__ uint32_t workgroup_max(uint32_t m, uint32_t* red)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    m = wave_max_u32(m);
    __syncthreads();
    if (lane == 0)
        red[wave] = m;
    __syncthreads();
    uint32_t r = red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w)
        r = max(r, red[w]);
    return r;
}

// Exact amax of the whole tensor by this workgroup alone (slow path).
template <int NT>
__device__ uint32_t direct_amax(const Params& p, uint32_t* red)
{
    const int64_t n = p.rows * p.cols;
    uint32_t pm = 0u;
    for (int64_t i = (int64_t)threadIdx.x * 8; i < n; i += (int64_t)NT * 8) {
        const uint4 v = load16(p.x + i);
        pm = pk_max_u16(pm, v.x & 0x7FFF7FFFu);
        pm = pk_max_u16(pm, v.y & 0x7FFF7FFFu);
        pm = pk_max_u16(pm, v.z & 0x7FFF7FFFu);
        pm = pk_max_u16(pm, v.w & 0x7FFF7FFFu);
    }
    return workgroup_max<NT>(max(pm & 0xFFFFu, pm >> 16) << 16, red);
}

// This call's generation: one more than the last completed call's. Read at
// the start of the kernel, off the exchange's critical path (the word only
// changes once every workgroup of this call has read it).

// A workgroup of a call whose exchange expired counts itself under the
// call's generation; the count that reaches the grid size publishes it.
// Only reached when a wait has expired, so the compare-and-swap loop is off
// every common path; each retry means another workgroup's count went in.
__device__ void count_expired(uint32_t* ws, uint32_t gen)
{
    uint64_t* word = reinterpret_cast<uint64_t*>(&ws[kWsExpired]);
    uint64_t seen = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
        const uint32_t n = ((uint32_t)seen == gen) ? (uint32_t)(seen >> 32) + 1u : 1u;
        const uint64_t want = ((uint64_t)n << 32) | gen;
        if (__hip_atomic_compare_exchange_weak(word, &seen, want, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)) {
            if (n == gridDim.x)
                ws_store(&ws[kWsGen], gen);
            return;
        }
    }
}
__device__ __forceinline__ uint32_t call_generation(const uint32_t* ws)
{
    return ws_load(&ws[kWsGen]) + 1u;
}

// Grid-wide maximum of one value per workgroup (binary32 bits); every
// workgroup returns the same result. gen0 and wait0 (workspace word 3: the
// bound on each wait in 100 MHz ticks, 0 for the default) are read by
// thread 0 at the start of the kernel.
template <int NT>
__device__ uint32_t grid_max(uint32_t m, uint32_t gen0, uint32_t wait0, uint32_t* ws, const Params& p)
{
    __shared__ uint32_t red[NT / 64];
    __shared__ uint32_t gen_s, wait_s, result_s, ok_s;
    m = workgroup_max<NT>(m, red);
    if (threadIdx.x == 0) {
        gen_s = gen0;
        wait_s = wait0;
        slot_store(&ws[kWsArrive + 2 * blockIdx.x], gen0, m);
    }
    __syncthreads();
    const uint32_t gen = gen_s;
    const uint64_t wait = wait_s != 0u ? (uint64_t)wait_s : kWaitTicks;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    if (blockIdx.x == 0) {
        // Collect every workgroup's maximum. Each thread watches the slots
        // t, t + 256, ...; every round re-reads all of its pending slots at
        // once, so their round trips overlap.
        constexpr int kPer = kMaxFusedGrid / NT;
        uint32_t mm = 0u;
        bool ok = true;
        uint32_t pending = 0u;
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            if ((int)threadIdx.x + k * NT < (int)gridDim.x)
                pending |= 1u << k;
        while (pending != 0u) {
            uint64_t w[kPer];
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                w[k] = (pending >> k) & 1u ? slot_load(&ws[kWsArrive + 2 * (threadIdx.x + k * NT)]) : 0u;
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                if (((pending >> k) & 1u) && (uint32_t)w[k] == gen) {
                    mm = max(mm, (uint32_t)(w[k] >> 32));
                    pending &= ~(1u << k);
                }
            }
            if (pending == 0u)
                break;
            if (__builtin_amdgcn_s_memrealtime() - t0 > wait) {
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(4);
        }
        if (threadIdx.x == 0)
            ok_s = 1u;
        __syncthreads();
        if (!ok)
            ok_s = 0u;
        const uint32_t r = workgroup_max<NT>(mm, red);
        if (ok_s == 0u) {
            result_s = direct_amax<NT>(p, red);
        } else if (threadIdx.x == 0) {
            result_s = r;
        }
        __syncthreads();
        const uint32_t amax = result_s;
        if (threadIdx.x == 0) {
            ws_store(&ws[kWsAmax], amax);
            if (p.amax_out != nullptr)
                *p.amax_out = __uint_as_float(amax);
            if (ok_s == 0u)
                __hip_atomic_fetch_add(&ws[kWsSlow], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const uint32_t flag = ok_s != 0u ? 0u : kExpiredFlag;
        for (int i = threadIdx.x; i < (int)gridDim.x; i += NT)
            slot_store(&ws[kWsRelease + 2 * i], gen, amax | flag);
        if (threadIdx.x == 0) {
            if (ok_s != 0u)
                ws_store(&ws[kWsGen], gen);  // every workgroup has read it
            else
                count_expired(ws, gen);
        }
        return amax;
    }
    if (threadIdx.x == 0) {
        uint64_t w = slot_load(&ws[kWsRelease + 2 * blockIdx.x]);
        ok_s = 1u;
        while ((uint32_t)w != gen) {
            if (__builtin_amdgcn_s_memrealtime() - t0 > wait) {
                ok_s = 0u;
                break;
            }
            __builtin_amdgcn_s_sleep(4);
            w = slot_load(&ws[kWsRelease + 2 * blockIdx.x]);
        }
        result_s = (uint32_t)(w >> 32);
    }
    __syncthreads();
    if (ok_s == 0u) {
        const uint32_t amax = direct_amax<NT>(p, red);
        if (threadIdx.x == 0) {
            __hip_atomic_fetch_add(&ws[kWsSlow], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            count_expired(ws, gen);
        }
        return amax;
    }
    const uint32_t v = result_s;
    if ((v & kExpiredFlag) != 0u && threadIdx.x == 0)
        count_expired(ws, gen);  // workgroup 0's wait expired
    return v & ~kExpiredFlag;
}

// Threads of the fused kernel. With round to nearest, 512: the first 256
// take tile A and the rest tile B, one item each, at four waves per SIMD
// (128 VGPRs), so two workgroups share each CU. With stochastic rounding an
// item's draws need 64 more registers, so 256 threads hold both tiles.
template <bool SR>
constexpr int kFusedThreads = SR ? 256 : 512;
template <bool SR>
constexpr int kFusedWaves = SR ? 1 : 4;  // minimum waves per SIMD

template <bool ROW, bool COL, bool SR>
__global__ __launch_bounds__(kFusedThreads<SR>) __attribute__((amdgpu_waves_per_eu(kFusedWaves<SR>)))
void quantize_fused_kernel(Params p, uint32_t* ws)
{
    constexpr int NT = kFusedThreads<SR>;
    // Columnwise staging for the two tiles.
    __shared__ uint2 lds_codes[2][COL ? kTileC * kRowBlocks : 1];
    __shared__ uint8_t lds_scales[2][COL ? kTileC * kRowBlocks : 16];
    __shared__ float lds_rcp[128];

    // Two vertically adjacent tiles per workgroup (B below A), so a
    // column's codes of the pair form whole 128-byte lines.
    const int tra = 2 * (blockIdx.x / p.tiles_c), tc = blockIdx.x % p.tiles_c;
    uint32_t gen = 0u, wait = 0u;
    if (!p.amax_given && threadIdx.x == 0) {
        gen = call_generation(ws);
        wait = ws_load(&ws[kWsWait]);
    }
    // Block maxima while the data arrives; the workgroup's maximum follows.
    // (With stochastic rounding the row maxima wait until after the
    // exchange: holding them across it would cost occupancy.)
    constexpr bool kEarlyRows = ROW && !SR;
    uint32_t m = 0u;
    if constexpr (NT == 512) {
        const int half = threadIdx.x >> 8;  // 0: tile A, 1: tile B
        const ItemPos q = item_pos(tra + half, tc, p.rows, p.cols, threadIdx.x & 255);
        uint4 v[16];
        load_item_any(p, q, v);
        BlockMax bm;
        if (q.valid) {
            if (kEarlyRows)
                block_maxima(v, q.odd, bm);
            else
                column_maxima(v, bm);
            m = item_max(bm);
        }
        const uint32_t amax_bits = p.amax_given ? __float_as_uint(*p.amax) : grid_max<NT>(m, gen, wait, ws, p);
        const ScaleCtx sc = scale_ctx(__uint_as_float(amax_bits));
        if (p.sg_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
            *p.sg_out = sc.sg;
        build_reciprocal_table(lds_rcp, sc.sg);
        __syncthreads();
        if (q.valid) {
            if (ROW && !kEarlyRows)
                row_maxima(v, q.odd, bm);
            uint4 draws[16];  // unused: round to nearest
            compute_item<ROW, COL, false, false, false>(p, q, v, bm, draws, sc, lds_rcp, lds_codes[half],
                                                        lds_scales[half], false);
        }
    } else {
        const bool has_b = tra + 1 < p.tiles_r;  // uniform over the workgroup
        const ItemPos qa = item_pos(tra, tc, p.rows, p.cols);
        const ItemPos qb = item_pos(tra + 1, tc, p.rows, p.cols);
        uint4 va[16], vb[16];
        load_item(p, qa, va);
        if (has_b)
            load_item(p, qb, vb);
        BlockMax ba, bb;
        if (qa.valid) {
            column_maxima(va, ba);
            if (kEarlyRows)
                row_maxima(va, qa.odd, ba);
            m = item_max(ba);
        }
        if (has_b && qb.valid) {
            column_maxima(vb, bb);
            if (kEarlyRows)
                row_maxima(vb, qb.odd, bb);
            m = max(m, item_max(bb));
        }
        const uint32_t amax_bits = p.amax_given ? __float_as_uint(*p.amax) : grid_max<NT>(m, gen, wait, ws, p);
        const ScaleCtx sc = scale_ctx(__uint_as_float(amax_bits));
        if (p.sg_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
            *p.sg_out = sc.sg;
        // Columnwise-only stochastic rounding: the converter's 2^23 goes into
        // the multipliers where that is exact (uniform).
        constexpr bool kCanFold = COL && !ROW && SR;
        const bool fold = kCanFold && fold_sr_scale_ok<0>(sc.sg);
        build_reciprocal_table(lds_rcp, sc.sg, fold ? kFoldFactor<SR, false> : 1.0f);
        __syncthreads();

        if (qa.valid) {
            if (ROW && !kEarlyRows)
                row_maxima(va, qa.odd, ba);
            uint4 draws[16];
            if (SR)
                item_draws(p, qa, draws, false);
            compute_item<ROW, COL, false, SR, false>(p, qa, va, ba, draws, sc, lds_rcp, lds_codes[0],
                                                     lds_scales[0], fold);
        }
        if (has_b && qb.valid) {
            if (ROW && !kEarlyRows)
                row_maxima(vb, qb.odd, bb);
            uint4 draws[16];
            if (SR)
                item_draws(p, qb, draws, false);
            compute_item<ROW, COL, false, SR, false>(p, qb, vb, bb, draws, sc, lds_rcp, lds_codes[1],
                                                     lds_scales[1], fold);
        }
    }
    if (COL) {
        __syncthreads();
        write_col_pair<NT>(p, (int64_t)tra * kTileR, (int64_t)tc * kTileC, lds_codes[0], lds_codes[1],
                           lds_scales[0], lds_scales[1]);
    }
}

// Workgroups of one fused kernel that fit on the device at once (cached).
template <bool ROW, bool COL, bool SR>
int fused_capacity()
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
            &per_cu, reinterpret_cast<const void*>(quantize_fused_kernel<ROW, COL, SR>), kFusedThreads<SR>, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    c = per_cu * cus;
    if (c > 0)
        cache[dev].store(c, std::memory_order_relaxed);
    return c;
}

template <bool ROW, bool COL, bool SR>
hipError_t launch_fused_variant(Params p, uint32_t* ws, hipStream_t stream, bool& launched)
{
    launched = false;
    const int grid = ((p.tiles_r + 1) / 2) * p.tiles_c;
    if (grid > kMaxFusedGrid || grid > fused_capacity<ROW, COL, SR>())
        return hipSuccess;
    hipLaunchKernelGGL((quantize_fused_kernel<ROW, COL, SR>), dim3(grid), dim3(kFusedThreads<SR>), 0, stream, p,
                       ws);
    launched = true;
    return hipGetLastError();
}

// The paired-tile kernel with the amax given: no exchange, so any grid size.
template <bool ROW, bool COL, bool SR>
hipError_t launch_paired(Params p, hipStream_t stream)
{
    p.amax_given = 1;
    const int64_t grid = (int64_t)((p.tiles_r + 1) / 2) * p.tiles_c;
    hipLaunchKernelGGL((quantize_fused_kernel<ROW, COL, SR>), dim3((unsigned)grid), dim3(kFusedThreads<SR>), 0,
                       stream, p, nullptr);
    return hipGetLastError();
}

template <bool ROW, bool COL, bool TWO_D, bool SR, bool RHT>
hipError_t launch_variant(const Params& p, hipStream_t stream)
{
    const int grid = p.tiles_r * p.tiles_c;
    hipLaunchKernelGGL((quantize_kernel<ROW, COL, TWO_D, SR, RHT>), dim3(grid), dim3(kThreads), 0,
                       stream, p);
    return hipGetLastError();
}

// The exchange workspace of nvfp4_quantize_1d_fused_noalloc: one copy per
// device (zero when the code object loads), shared by every such call on
// that device and held until the process ends. The exchange leaves it ready
// for the next call, so it is never cleared; calls on one device that
// overlap in time race on it.
constexpr int kScratchWords = kWsRelease + 2 * kMaxFusedBlocks;
static_assert(kScratchWords * 4 == 32832, "the workspace size the C header states");
static_assert(kMaxFusedGrid <= kMaxFusedBlocks, "every workgroup of a single pass has its slots");
static __device__ __align__(256) uint32_t scratch[kScratchWords];

}  // namespace

hipError_t noalloc_workspace(uint32_t** ws)
{
    // Device addresses of `scratch`, looked up once per device with that
    // device current. The host-side name `scratch` is not a device address.
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static uint32_t* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (ptr == nullptr)
            return hipErrorInvalidSymbol;
        addr[dev] = static_cast<uint32_t*>(ptr);
    }
    *ws = addr[dev];
    return hipSuccess;
}

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t stream)
{
    if (a.fused_amax) {
        Params p;
        p.x = a.x;
        p.rows = a.rows;
        p.cols = a.cols;
        p.amax = reinterpret_cast<const float*>(a.workspace);
        p.mask = 0u;
        p.seed_lo = (uint32_t)a.seed;
        p.seed_hi = (uint32_t)(a.seed >> 32);
        p.codes_row = a.codes_row;
        p.scales_row = a.scales_row;
        p.codes_col = a.codes_col;
        p.scales_col = a.scales_col;
        p.sg_out = a.global_scale;
        p.tiles_r = (int)((a.rows + kTileR - 1) / kTileR);
        p.tiles_c = (int)((a.cols + kTileC - 1) / kTileC);
        p.amax_given = 0;
        p.amax_out = a.amax_out;
        bool launched = false;
        hipError_t e;
        if (a.rowwise && a.colwise)
            e = a.sr ? launch_fused_variant<true, true, true>(p, a.workspace, stream, launched)
                     : launch_fused_variant<true, true, false>(p, a.workspace, stream, launched);
        else if (a.rowwise)
            e = a.sr ? launch_fused_variant<true, false, true>(p, a.workspace, stream, launched)
                     : launch_fused_variant<true, false, false>(p, a.workspace, stream, launched);
        else
            e = a.sr ? launch_fused_variant<false, true, true>(p, a.workspace, stream, launched)
                     : launch_fused_variant<false, true, false>(p, a.workspace, stream, launched);
        if (e != hipSuccess || launched)
            return e;
        // Too large to keep on chip: the two-pass path, amax into the
        // workspace (or straight into the caller's copy of it).
        float* amax = a.amax_out != nullptr ? a.amax_out : reinterpret_cast<float*>(a.workspace);
        e = launch_amax(a.x, a.rows * a.cols, amax, stream);
        if (e != hipSuccess)
            return e;
        QuantizeArgs b = a;
        b.fused_amax = false;
        b.amax = amax;
        return launch_quantize(b, stream);
    }
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
    p.amax_given = 0;
    p.amax_out = nullptr;

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
    // Both layouts: the paired-tile kernel (whole-line columnwise stores,
    // here without its exchange) for round-to-nearest on tensors up to 2^25
    // elements (8192x4096: 22.2 against 23.9 us); the one-tile kernel on
    // larger ones (8192x14336: 81-82 against 83-86 us) and with stochastic
    // rounding at every size (8192x4096: 43 against 57 us; 8192x14336: 144
    // against 204 us).
    if (a.rowwise && a.colwise) {
        if (!a.sr && a.rows * a.cols <= ((int64_t)1 << 25))
            return launch_paired<true, true, false>(p, stream);
        return a.sr ? launch_variant<true, true, false, true, false>(p, stream)
                    : launch_variant<true, true, false, false, false>(p, stream);
    }
    // One layout. Rowwise: the flat kernel (8192x4096: 15.4 against 16.9 us
    // for one tile per workgroup and 18.8 for the pairs; with stochastic
    // rounding 23-24 against 27-27.5 us). Columnwise: the pairs' whole lines
    // (17.5-17.9 against 18.5-18.6 us for one tile per workgroup).
    if (a.rowwise) {
        const int64_t nvec = a.rows * a.cols / 8;
        const int64_t grid = (nvec + kThreads * kFlatU - 1) / (kThreads * kFlatU);
        if (a.sr)
            hipLaunchKernelGGL(quantize_rows_flat_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p,
                               nvec);
        else
            hipLaunchKernelGGL(quantize_rows_flat_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p,
                               nvec);
        return hipGetLastError();
    }
    if (!a.sr && a.rows * a.cols <= ((int64_t)1 << 25))
        return launch_paired<false, true, false>(p, stream);
    return a.sr ? launch_variant<false, true, false, true, false>(p, stream)
                : launch_variant<false, true, false, false, false>(p, stream);
}

}  // namespace nvfp4
