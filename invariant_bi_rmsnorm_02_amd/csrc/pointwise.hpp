// The arithmetic of the decoder layer's elementwise steps, shared by the
// standalone kernels (pointwise.hip) and the GEMM epilogues that fuse them
// (gemm_fused.hip), so a fused and an unfused layer give the same bits.
// Inputs are bf16 values widened to fp32 (exactly); the caller rounds the
// result to bf16 once (pack_bf16x2).
#pragma once

#include "bi_common.hpp"

namespace bi {

// Residual add: the fp32 sum of two bf16 values.
__device__ __forceinline__ float pw_add(float x, float y) { return x + y; }

// Gated activation: silu(g) * u = g / (1 + 2^(-g log2 e)) * u in fp32.
__device__ __forceinline__ float pw_silu_mul(float g, float u) { return g / (1.0f + exp2_hw(-g * kLog2e)) * u; }

}  // namespace bi
