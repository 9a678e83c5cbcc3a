// kernels.hpp -- host-side launchers of the gfx950 kernels (internal to the library).
// Arguments are validated by the C ABI layer (api.hip) before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bitnet_w2a8.h"

namespace bitnet {

hipError_t launch_pack_weights(const float* w, int64_t N, int64_t K, uint8_t* packed,
                               float* scale, hipStream_t stream);
hipError_t launch_unpack_weights(const uint8_t* packed, int64_t N, int64_t K, int8_t* codes,
                                 hipStream_t stream);
hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* a_scale,
                            hipStream_t stream);
// One activation scale for the whole (M, K) tensor, written to every a_scale[m].
hipError_t launch_quant_act_per_tensor(const uint16_t* x, int64_t M, int64_t K, int8_t* xq,
                                       float* a_scale, hipStream_t stream);
// Rewrite packed weights from one 2-bit code table to another (0: code = w + 1; 1: the
// 00/01/11 table); fields holding an unused code become 0 and are counted in *invalid.
hipError_t launch_repack_codes(const uint8_t* in, int64_t N, int64_t K, int from, int to,
                               uint8_t* out, int* invalid, hipStream_t stream);

// Weight-streaming product for 1 <= M <= 16.  When x_bf16 is non-null the activations
// are quantized inside the kernel (xq / a_scale ignored; xq_out / a_out optional copies).
hipError_t launch_skinny(const int8_t* xq, const float* a_scale, const uint16_t* x_bf16,
                         const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                         int64_t K, void* out, int out_dtype, int8_t* xq_out, float* a_out,
                         hipStream_t stream);
// The same product for 1 <= groups <= BITNET_MAX_GROUPS weight matrices (N[g] rows each,
// all K columns) against the same activations, in one launch.
hipError_t launch_skinny_grouped(const int8_t* xq, const float* a_scale, const uint16_t* x_bf16,
                                 int groups, const uint8_t* const* packed,
                                 const float* const* w_scale, const int64_t* N,
                                 void* const* out, int64_t M, int64_t K, int out_dtype,
                                 int8_t* xq_out, float* a_out, hipStream_t stream);

// SwiGLU pair for 1 <= M <= 16 (bf16 activations, fused quantization): the same rows of
// the gate and up matrices in one launch, out = silu(gate product) * (up product), fp32
// (out_dtype 0) or bf16 (1).
hipError_t launch_skinny_swiglu(const uint16_t* x_bf16, const uint8_t* packed_gate,
                                const float* w_scale_gate, const uint8_t* packed_up,
                                const float* w_scale_up, int64_t M, int64_t N, int64_t K,
                                void* out, int out_dtype, int8_t* xq_out, float* a_out,
                                hipStream_t stream);

// bf16 activations times ternary weights (no activation quantization), fp32 accumulation,
// 1 <= M <= 16, K % 64 == 0; out fp32 (0) or bf16 (1).
hipError_t launch_a16(const uint16_t* x, const uint8_t* packed, const float* w_scale, int64_t M,
                      int64_t N, int64_t K, void* out, int out_dtype, hipStream_t stream);

// Product for 1 <= M <= 32 (16 with x_bf16) with the activations read straight into
// matrix-core operands; K % 64 == 0.  With x_bf16 non-null the activations are quantized
// in the kernel (xq / a_scale ignored; xq_out / a_out optional copies), else int8 codes
// xq + a_scale.
hipError_t launch_gemv_direct(const int8_t* xq, const float* a_scale, const uint16_t* x_bf16,
                              const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                              int64_t K, void* out, int out_dtype, int8_t* xq_out, float* a_out,
                              hipStream_t stream);

// Five ternary weights per byte (1.6 bits): bytes per row of the format, the conversion
// from the 2-bit interface format, and the decode product with fused quantization for
// one token (K % 8 == 0, K <= BITNET_B3_MAX_K).
int64_t b3_row_bytes(int64_t K);
hipError_t launch_pack_b3(const uint8_t* packed, int64_t N, int64_t K, uint8_t* b3,
                          hipStream_t stream);
hipError_t launch_quant_gemv_b3(const uint16_t* x, const uint8_t* b3, const float* w_scale,
                                int64_t N, int64_t K, void* out, int out_dtype,
                                hipStream_t stream);

// Tiled int8 matrix-core product for any M.  Device scratch with which a single-matrix
// launch may split K across blocks (int32 partial tiles of every K slice), in bytes; 0
// when the best plan does not split.
size_t tiled_workspace_size(int64_t M, int64_t N, int64_t K);
// The tiled product for 1 <= groups <= BITNET_MAX_GROUPS weight matrices (N[g] rows
// each, all K columns) against the same activations, in one launch; the tile plan is
// chosen for the launch's total tile count.
// The tile plan of a tiled launch over `groups` matrices of N[g] rows: plan[0..4] = block
// rows, block columns, k-groups per block, k per LDS stage, K slices (groups == 1: the
// plan with a workspace; more groups never split); cus <= 0: the current device's.
void tiled_plan(int64_t M, int64_t K, int groups, const int64_t* N, int64_t cus, int* plan);
hipError_t launch_tiled_grouped(const int8_t* xq, const float* a_scale, int groups,
                                const uint8_t* const* packed, const float* const* w_scale,
                                const int64_t* N, void* const* out, int64_t M, int64_t K,
                                int out_dtype, hipStream_t stream);
// workspace: NULL, or ws_bytes of device scratch; K is split across blocks only when
// ws_bytes >= tiled_workspace_size(M, N, K) > 0 (the result is the same either way).
hipError_t launch_tiled(const int8_t* xq, const float* a_scale, const uint8_t* packed,
                        const float* w_scale, int64_t M, int64_t N, int64_t K, void* out,
                        int out_dtype, void* workspace, size_t ws_bytes, hipStream_t stream);

}  // namespace bitnet
