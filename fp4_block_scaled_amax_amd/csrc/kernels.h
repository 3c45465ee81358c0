// Internal launch interface between the C ABI (api.hip) and the kernels.
// Arguments reaching these functions have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

hipError_t launch_amax(const uint16_t* x, int64_t n, float* amax, hipStream_t stream);
// both: amax[0] = plain amax, amax[1] = amax of the transform (one read).
hipError_t launch_amax_rht(const uint16_t* x, int64_t rows, int64_t cols, uint32_t mask, float* amax,
                           bool both, hipStream_t stream);

struct QuantizeArgs {
    const uint16_t* x;
    int64_t rows, cols;
    const float* amax;
    uint32_t mask;
    uint64_t seed;
    bool rowwise, colwise, two_d, sr, rht;
    uint8_t* codes_row;
    uint8_t* scales_row;  // 1D rowwise scales, or the 2D tile scales
    uint8_t* codes_col;
    uint8_t* scales_col;  // 1D columnwise scales; 2D: the transposed tile grid (optional)
    float* global_scale;  // optional
    bool fused_amax;      // compute the amax in the same call (workspace)
    uint32_t* workspace;  // fused_amax: amax bits in word 0, scratch after
    float* amax_out;      // fused_amax: optional copy of the amax
};
hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t stream);

// Device address of the library's own exchange workspace on the current
// device (NVFP4_WORKSPACE_BYTES, never allocated: a static device array).
hipError_t noalloc_workspace(uint32_t** ws);

hipError_t launch_rht16(const uint16_t* x, int64_t rows, int64_t cols, int axis, uint32_t mask,
                        float* y, hipStream_t stream);

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, bool two_d,
                             const float* global_scale, int64_t rows, int64_t cols, void* out,
                             bool bf16_out, hipStream_t stream);

struct GemmArgs {
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    bool a_two_d;
    bool a_scales_t;  // 2D tile scales stored transposed ([K/16][M/16])
    const float* a_sg;
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    bool b_two_d;
    bool b_scales_t;  // 2D tile scales stored transposed ([K/16][N/16])
    const float* b_sg;
    void* c;
    bool c_bf16;
    int64_t M, N, K;
    float* c_amax;  // optional: max |C| of the stored values
    // Quantizing epilogue (q_flags: 1 rowwise, 2 columnwise, 3 both; 0 to
    // store C): C is not stored; its bf16 values are quantized to NVFP4 with
    // the tensor amax *q_amax into the four outputs (nvfp4_quantize_1d's
    // layouts), and *q_global_scale (optional) receives S_g.
    uint32_t q_flags;
    const float* q_amax;
    uint8_t* q_codes_row;
    uint8_t* q_scales_row;
    uint8_t* q_codes_col;
    uint8_t* q_scales_col;
    float* q_global_scale;
};
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);

// MXFP4 (E8M0 scale per 32 elements): quantize, dequantize, GEMM.
struct MxQuantizeArgs {
    const uint16_t* x;
    int64_t rows, cols;  // rowwise: cols % 32 == 0; colwise: rows % 32 == 0, cols % 8 == 0
    uint32_t mask;
    bool rowwise, colwise, rht;
    uint8_t* codes_row;   // [rows][cols/2]
    uint8_t* scales_row;  // [rows][cols/32]
    uint8_t* codes_col;   // [cols][rows/2]
    uint8_t* scales_col;  // [cols][rows/32]
};
hipError_t launch_mx_quantize(const MxQuantizeArgs& a, hipStream_t stream);

hipError_t launch_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                                void* out, bool bf16_out, hipStream_t stream);

struct MxGemmArgs {
    const uint8_t* a_codes;   // [M][K/2]
    const uint8_t* a_scales;  // [M][K/32]
    const uint8_t* b_codes;   // [N][K/2]
    const uint8_t* b_scales;  // [N][K/32]
    void* c;
    bool c_bf16;
    int64_t M, N, K;
};
hipError_t launch_mx_gemm(const MxGemmArgs& a, hipStream_t stream);

}  // namespace nvfp4
