// Common device helpers for the gfx950 kernels: bf16 packing, vector types,
// the one MFMA instruction used by every matrix kernel, and wave reductions.
//
// Numerics rules that keep results batch-invariant (the reduction order of an
// output element must not depend on the batch; "Thinking Machines Lab -
// Defeating Nondeterminism in LLM Inference", section "Achieving Batch-Invariant
// Kernels"): the library is compiled with -ffp-contract=off and without fast
// math, so every floating-point expression is evaluated exactly as written;
// fused multiply-adds appear only where written explicitly (fmaf).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// bf16 word -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest, ties to even, with gfx950's
// v_cvt_pk_bf16_f32 (two values per instruction).  Every rounding to bf16 in
// the library goes through these two functions.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

// The single matrix instruction of the library: v_mfma_f32_16x16x32_bf16.
// D[16x16] = A[16x32] * B[32x16] + C with, for lane l (g = l / 16):
//   A: row l % 16, k = 8g .. 8g+7       B: column l % 16, k = 8g .. 8g+7
//   C/D: column l % 16, rows 4g .. 4g+3
// Every output element is the same function of its own A row, B column and C
// value wherever it sits in the tile, so results do not depend on the other
// rows/columns of the tile.
__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Cross-lane exchange within a wavefront.
__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}
__device__ __forceinline__ int shfl_xor(int v, int mask) { return __shfl_xor(v, mask, kWave); }

// Butterfly sum over the lanes of a wavefront.  Partners add the same two
// values (addition is commutative), so after each step both hold identical
// bits and every lane ends with the same total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = v + shfl_xor(v, o);
  return v;
}

// Exchange across 16-lane rows (lanes l and l ^ 16) and across wavefront
// halves (l and l ^ 32) with v_permlane16_swap / v_permlane32_swap: every lane
// gets the pair {x[l], x[l ^ 16]} (resp. l ^ 32) in one VALU instruction
// instead of a round trip through LDS.  The pair's order depends on the row,
// which neither max nor + (commutative, bit for bit) can see, so these give
// the same bits as v op shfl_xor(v, 16 or 32).
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, shfl_xor(v, o));
  return v;
}

// Hardware base-2 exponential and logarithm (v_exp_f32 / v_log_f32).  Both
// attention kernels and the merge use these same two instructions.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace bi
