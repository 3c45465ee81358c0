// C ABI entry points: argument validation (before any HIP call), then the
// launch. See include/nvfp4.h for the contract of each call.
#include "../../include/mxfp4.h"
#include "../../include/nvfp4.h"
#include "kernels.h"

namespace {

// Flat indices and byte offsets are int64; the SR counter takes i/8 in 64
// bits. Keep every dimension product well inside int64.
constexpr int64_t kMaxElements = (int64_t)1 << 46;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dims_ok(int64_t rows, int64_t cols)
{
    return rows > 0 && cols > 0 && rows <= kMaxElements && cols <= kMaxElements &&
           rows <= kMaxElements / cols;
}

int status_of(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

}  // namespace

extern "C" {

const char* nvfp4_status_string(int status)
{
    switch (status) {
    case NVFP4_OK:
        return "ok";
    case NVFP4_ERR_NULL:
        return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE:
        return "a dimension is not positive or not a multiple of the required granule";
    case NVFP4_ERR_ALIGN:
        return "a pointer is not 16-byte aligned";
    case NVFP4_ERR_FLAGS:
        return "unknown flag or mode, or an unsupported combination";
    case NVFP4_ERR_HIP:
        return "the HIP runtime refused a launch";
    case NVFP4_ERR_SIZE:
        return "a size exceeds the supported index range";
    default:
        return "unknown status";
    }
}

int nvfp4_amax(const uint16_t* x, int64_t rows, int64_t cols, uint32_t flags, uint16_t rht_mask,
               float* amax, hipStream_t stream)
{
    if (x == nullptr || amax == nullptr)
        return NVFP4_ERR_NULL;
    if ((flags & ~(NVFP4_RHT | NVFP4_AMAX_BOTH)) != 0 ||
        ((flags & NVFP4_AMAX_BOTH) && !(flags & NVFP4_RHT)))
        return NVFP4_ERR_FLAGS;
    if (rows <= 0 || cols <= 0)
        return NVFP4_ERR_SHAPE;
    if (!dims_ok(rows, cols))
        return NVFP4_ERR_SIZE;
    if (!aligned16(x) || (reinterpret_cast<uintptr_t>(amax) & 3u) != 0)
        return NVFP4_ERR_ALIGN;
    if (flags & NVFP4_RHT) {
        if (rows % 16 != 0 || cols % 8 != 0)
            return NVFP4_ERR_SHAPE;
        return status_of(nvfp4::launch_amax_rht(x, rows, cols, rht_mask, amax,
                                                (flags & NVFP4_AMAX_BOTH) != 0, stream));
    }
    return status_of(nvfp4::launch_amax(x, rows * cols, amax, stream));
}

int nvfp4_quantize_1d(const uint16_t* x, int64_t rows, int64_t cols, const float* amax,
                      uint32_t flags, uint16_t rht_mask, uint64_t seed, uint8_t* codes_row,
                      uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                      float* global_scale, hipStream_t stream)
{
    const uint32_t known = NVFP4_ROWWISE | NVFP4_COLWISE | NVFP4_SR | NVFP4_RHT;
    if ((flags & ~known) != 0 || (flags & (NVFP4_ROWWISE | NVFP4_COLWISE)) == 0)
        return NVFP4_ERR_FLAGS;
    if ((flags & NVFP4_RHT) && ((flags & NVFP4_ROWWISE) || !(flags & NVFP4_COLWISE)))
        return NVFP4_ERR_FLAGS;
    const bool row = (flags & NVFP4_ROWWISE) != 0, col = (flags & NVFP4_COLWISE) != 0;
    if (x == nullptr || amax == nullptr)
        return NVFP4_ERR_NULL;
    if (row && (codes_row == nullptr || scales_row == nullptr))
        return NVFP4_ERR_NULL;
    if (col && (codes_col == nullptr || scales_col == nullptr))
        return NVFP4_ERR_NULL;
    if (rows <= 0 || cols <= 0 || rows % 16 != 0 || cols % 16 != 0)
        return NVFP4_ERR_SHAPE;
    if (!dims_ok(rows, cols) || rows / 256 >= (1 << 20) || cols / 256 >= (1 << 20))
        return NVFP4_ERR_SIZE;
    if (!aligned16(x) || (row && (!aligned16(codes_row) || !aligned16(scales_row))) ||
        (col && (!aligned16(codes_col) || !aligned16(scales_col))))
        return NVFP4_ERR_ALIGN;
    nvfp4::QuantizeArgs a{};
    a.x = x;
    a.rows = rows;
    a.cols = cols;
    a.amax = amax;
    a.mask = rht_mask;
    a.seed = seed;
    a.rowwise = row;
    a.colwise = col;
    a.two_d = false;
    a.sr = (flags & NVFP4_SR) != 0;
    a.rht = (flags & NVFP4_RHT) != 0;
    a.codes_row = codes_row;
    a.scales_row = scales_row;
    a.codes_col = codes_col;
    a.scales_col = scales_col;
    a.global_scale = global_scale;
    return status_of(nvfp4::launch_quantize(a, stream));
}

namespace {

// Validation shared by the fused entry points; `a` receives the arguments.
int fused_args(const uint16_t* x, int64_t rows, int64_t cols, uint32_t flags, uint64_t seed,
               uint8_t* codes_row, uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
               float* global_scale, nvfp4::QuantizeArgs& a)
{
    const uint32_t known = NVFP4_ROWWISE | NVFP4_COLWISE | NVFP4_SR;
    if ((flags & ~known) != 0 || (flags & (NVFP4_ROWWISE | NVFP4_COLWISE)) == 0)
        return NVFP4_ERR_FLAGS;
    const bool row = (flags & NVFP4_ROWWISE) != 0, col = (flags & NVFP4_COLWISE) != 0;
    if (x == nullptr || (row && (codes_row == nullptr || scales_row == nullptr)) ||
        (col && (codes_col == nullptr || scales_col == nullptr)))
        return NVFP4_ERR_NULL;
    if (rows <= 0 || cols <= 0 || rows % 16 != 0 || cols % 16 != 0)
        return NVFP4_ERR_SHAPE;
    if (!dims_ok(rows, cols) || rows / 256 >= (1 << 20) || cols / 256 >= (1 << 20))
        return NVFP4_ERR_SIZE;
    if (!aligned16(x) || (row && (!aligned16(codes_row) || !aligned16(scales_row))) ||
        (col && (!aligned16(codes_col) || !aligned16(scales_col))))
        return NVFP4_ERR_ALIGN;
    a = nvfp4::QuantizeArgs{};
    a.fused_amax = true;
    a.x = x;
    a.rows = rows;
    a.cols = cols;
    a.seed = seed;
    a.rowwise = row;
    a.colwise = col;
    a.sr = (flags & NVFP4_SR) != 0;
    a.codes_row = codes_row;
    a.scales_row = scales_row;
    a.codes_col = codes_col;
    a.scales_col = scales_col;
    a.global_scale = global_scale;
    return NVFP4_OK;
}

int quantize_2d_common(const uint16_t* x, int64_t rows, int64_t cols, const float* amax,
                       uint8_t* codes_row, uint8_t* codes_col, uint8_t* scales, uint8_t* scales_t,
                       float* global_scale, hipStream_t stream)
{
    if (x == nullptr || amax == nullptr || scales == nullptr ||
        (codes_row == nullptr && codes_col == nullptr))
        return NVFP4_ERR_NULL;
    if (rows <= 0 || cols <= 0 || rows % 16 != 0 || cols % 16 != 0)
        return NVFP4_ERR_SHAPE;
    if (!dims_ok(rows, cols) || rows / 256 >= (1 << 20) || cols / 256 >= (1 << 20))
        return NVFP4_ERR_SIZE;
    if (!aligned16(x) || !aligned16(scales) || (codes_row && !aligned16(codes_row)) ||
        (codes_col && !aligned16(codes_col)))
        return NVFP4_ERR_ALIGN;
    nvfp4::QuantizeArgs a{};
    a.x = x;
    a.rows = rows;
    a.cols = cols;
    a.amax = amax;
    a.rowwise = codes_row != nullptr;
    a.colwise = codes_col != nullptr;
    a.two_d = true;
    a.codes_row = codes_row;
    a.scales_row = scales;
    a.codes_col = codes_col;
    a.scales_col = scales_t;
    a.global_scale = global_scale;
    return status_of(nvfp4::launch_quantize(a, stream));
}

}  // namespace

int nvfp4_quantize_1d_fused(const uint16_t* x, int64_t rows, int64_t cols, uint32_t flags,
                            uint64_t seed, void* workspace, uint8_t* codes_row,
                            uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                            float* global_scale, hipStream_t stream)
{
    nvfp4::QuantizeArgs a;
    const int st = fused_args(x, rows, cols, flags, seed, codes_row, scales_row, codes_col, scales_col,
                              global_scale, a);
    if (st != NVFP4_OK)
        return st;
    if (workspace == nullptr)
        return NVFP4_ERR_NULL;
    if (!aligned16(workspace))
        return NVFP4_ERR_ALIGN;
    a.workspace = static_cast<uint32_t*>(workspace);
    return status_of(nvfp4::launch_quantize(a, stream));
}

int nvfp4_quantize_1d_fused_noalloc(const uint16_t* x, int64_t rows, int64_t cols, uint32_t flags,
                                    uint64_t seed, uint8_t* codes_row, uint8_t* scales_row,
                                    uint8_t* codes_col, uint8_t* scales_col, float* global_scale,
                                    float* amax, hipStream_t stream)
{
    nvfp4::QuantizeArgs a;
    const int st = fused_args(x, rows, cols, flags, seed, codes_row, scales_row, codes_col, scales_col,
                              global_scale, a);
    if (st != NVFP4_OK)
        return st;
    if (amax != nullptr && (reinterpret_cast<uintptr_t>(amax) & 3u) != 0)
        return NVFP4_ERR_ALIGN;
    uint32_t* ws = nullptr;
    if (nvfp4::noalloc_workspace(&ws) != hipSuccess)
        return NVFP4_ERR_HIP;
    a.workspace = ws;
    a.amax_out = amax;
    return status_of(nvfp4::launch_quantize(a, stream));
}

int nvfp4_quantize_2d(const uint16_t* x, int64_t rows, int64_t cols, const float* amax,
                      uint8_t* codes_row, uint8_t* codes_col, uint8_t* scales,
                      float* global_scale, hipStream_t stream)
{
    return quantize_2d_common(x, rows, cols, amax, codes_row, codes_col, scales, nullptr, global_scale,
                              stream);
}

int nvfp4_quantize_2d_tscales(const uint16_t* x, int64_t rows, int64_t cols, const float* amax,
                              uint8_t* codes_row, uint8_t* codes_col, uint8_t* scales,
                              uint8_t* scales_t, float* global_scale, hipStream_t stream)
{
    if (scales_t == nullptr)
        return NVFP4_ERR_NULL;
    return quantize_2d_common(x, rows, cols, amax, codes_row, codes_col, scales, scales_t, global_scale,
                              stream);
}

int nvfp4_rht16(const uint16_t* x, int64_t rows, int64_t cols, int axis, uint16_t rht_mask,
                float* y, hipStream_t stream)
{
    if (x == nullptr || y == nullptr)
        return NVFP4_ERR_NULL;
    if (axis != 0 && axis != 1)
        return NVFP4_ERR_FLAGS;
    if (rows <= 0 || cols <= 0)
        return NVFP4_ERR_SHAPE;
    if (axis == 0 && (rows % 16 != 0 || cols % 8 != 0))
        return NVFP4_ERR_SHAPE;
    if (axis == 1 && cols % 16 != 0)
        return NVFP4_ERR_SHAPE;
    if (!dims_ok(rows, cols))
        return NVFP4_ERR_SIZE;
    if (!aligned16(x) || !aligned16(y))
        return NVFP4_ERR_ALIGN;
    return status_of(nvfp4::launch_rht16(x, rows, cols, axis, rht_mask, y, stream));
}

int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int scale_mode,
                     const float* global_scale, int64_t rows, int64_t cols, void* out,
                     int out_dtype, hipStream_t stream)
{
    if (codes == nullptr || scales == nullptr || global_scale == nullptr || out == nullptr)
        return NVFP4_ERR_NULL;
    if ((scale_mode != NVFP4_SCALE_1D && scale_mode != NVFP4_SCALE_2D) ||
        (out_dtype != NVFP4_F32 && out_dtype != NVFP4_BF16))
        return NVFP4_ERR_FLAGS;
    if (rows <= 0 || cols <= 0 || rows % 16 != 0 || cols % 16 != 0)
        return NVFP4_ERR_SHAPE;
    if (!dims_ok(rows, cols))
        return NVFP4_ERR_SIZE;
    if (!aligned16(codes) || !aligned16(out))
        return NVFP4_ERR_ALIGN;
    return status_of(nvfp4::launch_dequantize(codes, scales, scale_mode == NVFP4_SCALE_2D,
                                              global_scale, rows, cols, out,
                                              out_dtype == NVFP4_BF16, stream));
}

namespace {

// Validation and arguments shared by the GEMM entry points; c == nullptr
// only with a quantizing epilogue (q->q_flags != 0), whose fields q supplies.
int gemm_common(const uint8_t* a_codes, const uint8_t* a_scales, int a_scale_mode,
                const float* a_global_scale, const uint8_t* b_codes, const uint8_t* b_scales,
                int b_scale_mode, const float* b_global_scale, void* c, int c_dtype, int64_t M,
                int64_t N, int64_t K, float* c_amax, hipStream_t stream,
                const nvfp4::GemmArgs* q = nullptr)
{
    const bool quant = q != nullptr && q->q_flags != 0;
    if (a_codes == nullptr || a_scales == nullptr || a_global_scale == nullptr ||
        b_codes == nullptr || b_scales == nullptr || b_global_scale == nullptr || (c == nullptr && !quant))
        return NVFP4_ERR_NULL;
    if (a_scale_mode < NVFP4_SCALE_1D || a_scale_mode > NVFP4_SCALE_2D_T ||
        b_scale_mode < NVFP4_SCALE_1D || b_scale_mode > NVFP4_SCALE_2D_T ||
        (c_dtype != NVFP4_F32 && c_dtype != NVFP4_BF16))
        return NVFP4_ERR_FLAGS;
    if (M <= 0 || N <= 0 || K <= 0 || M % 16 != 0 || N % 16 != 0 || K % 16 != 0)
        return NVFP4_ERR_SHAPE;
    if (!dims_ok(M, K) || !dims_ok(N, K) || !dims_ok(M, N) || M / 128 >= 65535 ||
        N / 128 >= (1 << 30))
        return NVFP4_ERR_SIZE;
    if (!aligned16(a_codes) || !aligned16(b_codes) || (!quant && !aligned16(c)))
        return NVFP4_ERR_ALIGN;
    nvfp4::GemmArgs g{};
    if (quant)
        g = *q;
    g.a_codes = a_codes;
    g.a_scales = a_scales;
    g.a_two_d = a_scale_mode != NVFP4_SCALE_1D;
    g.a_scales_t = a_scale_mode == NVFP4_SCALE_2D_T;
    g.a_sg = a_global_scale;
    g.b_codes = b_codes;
    g.b_scales = b_scales;
    g.b_two_d = b_scale_mode != NVFP4_SCALE_1D;
    g.b_scales_t = b_scale_mode == NVFP4_SCALE_2D_T;
    g.b_sg = b_global_scale;
    g.c = c;
    g.c_bf16 = c_dtype == NVFP4_BF16;
    g.M = M;
    g.N = N;
    g.K = K;
    g.c_amax = c_amax;
    return status_of(nvfp4::launch_gemm(g, stream));
}

}  // namespace

int nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int a_scale_mode,
               const float* a_global_scale, const uint8_t* b_codes, const uint8_t* b_scales,
               int b_scale_mode, const float* b_global_scale, void* c, int c_dtype, int64_t M,
               int64_t N, int64_t K, hipStream_t stream)
{
    return gemm_common(a_codes, a_scales, a_scale_mode, a_global_scale, b_codes, b_scales, b_scale_mode,
                       b_global_scale, c, c_dtype, M, N, K, nullptr, stream);
}

int nvfp4_gemm_amax(const uint8_t* a_codes, const uint8_t* a_scales, int a_scale_mode,
                    const float* a_global_scale, const uint8_t* b_codes, const uint8_t* b_scales,
                    int b_scale_mode, const float* b_global_scale, void* c, int c_dtype, int64_t M,
                    int64_t N, int64_t K, float* c_amax, hipStream_t stream)
{
    if (c_amax == nullptr)
        return NVFP4_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(c_amax) & 3u) != 0)
        return NVFP4_ERR_ALIGN;
    return gemm_common(a_codes, a_scales, a_scale_mode, a_global_scale, b_codes, b_scales, b_scale_mode,
                       b_global_scale, c, c_dtype, M, N, K, c_amax, stream);
}

int nvfp4_gemm_quantize(const uint8_t* a_codes, const uint8_t* a_scales, int a_scale_mode,
                        const float* a_global_scale, const uint8_t* b_codes, const uint8_t* b_scales,
                        int b_scale_mode, const float* b_global_scale, int64_t M, int64_t N,
                        int64_t K, const float* y_amax, uint32_t flags, uint8_t* codes_row,
                        uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                        float* global_scale, float* c_amax, hipStream_t stream)
{
    if ((flags & ~(NVFP4_ROWWISE | NVFP4_COLWISE)) != 0 || (flags & (NVFP4_ROWWISE | NVFP4_COLWISE)) == 0)
        return NVFP4_ERR_FLAGS;
    const bool row = (flags & NVFP4_ROWWISE) != 0, col = (flags & NVFP4_COLWISE) != 0;
    if (y_amax == nullptr || (row && (codes_row == nullptr || scales_row == nullptr)) ||
        (col && (codes_col == nullptr || scales_col == nullptr)))
        return NVFP4_ERR_NULL;
    if ((row && (!aligned16(codes_row) || !aligned16(scales_row))) ||
        (col && (!aligned16(codes_col) || !aligned16(scales_col))) ||
        (c_amax != nullptr && (reinterpret_cast<uintptr_t>(c_amax) & 3u) != 0))
        return NVFP4_ERR_ALIGN;
    nvfp4::GemmArgs q{};
    q.q_flags = (row ? 1u : 0u) | (col ? 2u : 0u);
    q.q_amax = y_amax;
    q.q_codes_row = row ? codes_row : nullptr;
    q.q_scales_row = row ? scales_row : nullptr;
    q.q_codes_col = col ? codes_col : nullptr;
    q.q_scales_col = col ? scales_col : nullptr;
    q.q_global_scale = global_scale;
    return gemm_common(a_codes, a_scales, a_scale_mode, a_global_scale, b_codes, b_scales, b_scale_mode,
                       b_global_scale, nullptr, NVFP4_BF16, M, N, K, c_amax, stream, &q);
}

int mxfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint32_t flags,
                   uint16_t rht_mask, uint8_t* codes_row, uint8_t* scales_row,
                   uint8_t* codes_col, uint8_t* scales_col, hipStream_t stream)
{
    if ((flags & ~(NVFP4_ROWWISE | NVFP4_COLWISE | NVFP4_RHT)) != 0 ||
        (flags & (NVFP4_ROWWISE | NVFP4_COLWISE)) == 0)
        return NVFP4_ERR_FLAGS;
    if ((flags & NVFP4_RHT) && ((flags & NVFP4_ROWWISE) || !(flags & NVFP4_COLWISE)))
        return NVFP4_ERR_FLAGS;
    const bool row = (flags & NVFP4_ROWWISE) != 0, col = (flags & NVFP4_COLWISE) != 0;
    if (x == nullptr || (row && (codes_row == nullptr || scales_row == nullptr)) ||
        (col && (codes_col == nullptr || scales_col == nullptr)))
        return NVFP4_ERR_NULL;
    if (rows <= 0 || cols <= 0 || (row && cols % 32 != 0) || (col && (rows % 32 != 0 || cols % 8 != 0)))
        return NVFP4_ERR_SHAPE;
    if (!dims_ok(rows, cols) || rows / 128 >= (1 << 15) || cols / 128 >= (1 << 15) ||
        (rows / 128 + 1) * (cols / 128 + 1) >= (int64_t)1 << 31)
        return NVFP4_ERR_SIZE;
    if (!aligned16(x) || (row && !aligned16(codes_row)) || (col && !aligned16(codes_col)))
        return NVFP4_ERR_ALIGN;
    nvfp4::MxQuantizeArgs a{};
    a.x = x;
    a.rows = rows;
    a.cols = cols;
    a.mask = rht_mask;
    a.rowwise = row;
    a.colwise = col;
    a.rht = (flags & NVFP4_RHT) != 0;
    a.codes_row = codes_row;
    a.scales_row = scales_row;
    a.codes_col = codes_col;
    a.scales_col = scales_col;
    return status_of(nvfp4::launch_mx_quantize(a, stream));
}

int mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                     void* out, int out_dtype, hipStream_t stream)
{
    if (codes == nullptr || scales == nullptr || out == nullptr)
        return NVFP4_ERR_NULL;
    if (out_dtype != NVFP4_F32 && out_dtype != NVFP4_BF16)
        return NVFP4_ERR_FLAGS;
    if (rows <= 0 || cols <= 0 || cols % 32 != 0)
        return NVFP4_ERR_SHAPE;
    if (!dims_ok(rows, cols))
        return NVFP4_ERR_SIZE;
    if (!aligned16(codes) || !aligned16(out))
        return NVFP4_ERR_ALIGN;
    return status_of(nvfp4::launch_mx_dequantize(codes, scales, rows, cols, out,
                                                 out_dtype == NVFP4_BF16, stream));
}

int mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
               const uint8_t* b_scales, void* c, int c_dtype, int64_t M, int64_t N, int64_t K,
               hipStream_t stream)
{
    if (a_codes == nullptr || a_scales == nullptr || b_codes == nullptr || b_scales == nullptr ||
        c == nullptr)
        return NVFP4_ERR_NULL;
    if (c_dtype != NVFP4_F32 && c_dtype != NVFP4_BF16)
        return NVFP4_ERR_FLAGS;
    if (M <= 0 || N <= 0 || K <= 0 || K % 32 != 0)
        return NVFP4_ERR_SHAPE;
    // 32-bit offsets inside a 256-row panel (256 * K / 2 bytes) and an
    // output sub-tile (128 * N elements).
    if (!dims_ok(M, K) || !dims_ok(N, K) || !dims_ok(M, N) || M / 256 >= (1 << 15) ||
        N / 256 >= (1 << 15) || K > (1 << 24))
        return NVFP4_ERR_SIZE;
    if (!aligned16(a_codes) || !aligned16(b_codes) || !aligned16(c))
        return NVFP4_ERR_ALIGN;
    nvfp4::MxGemmArgs g{};
    g.a_codes = a_codes;
    g.a_scales = a_scales;
    g.b_codes = b_codes;
    g.b_scales = b_scales;
    g.c = c;
    g.c_bf16 = c_dtype == NVFP4_BF16;
    g.M = M;
    g.N = N;
    g.K = K;
    return status_of(nvfp4::launch_mx_gemm(g, stream));
}

}  // extern "C"
