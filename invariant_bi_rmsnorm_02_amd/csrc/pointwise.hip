// Elementwise steps of the decoder layer around the reductions: the residual
// add and the gated activation of the MLP.  Each output element is a function
// of its own input elements only, so it is the same in every batch ("Thinking
// Machines Lab - Defeating Nondeterminism in LLM Inference": only reductions
// need a batch-independent order; pointwise work has none to choose).
//
//   add:      out = bf16(x + y)                      (exact fp32 sum of two bf16, one rounding)
//   silu_mul: out = bf16(g / (1 + 2^(-g log2 e)) * u) (fp32, one rounding), g and u the two
//             halves of a fused gate/up projection row
//
// One thread per 8 contiguous elements (one 16-byte load per operand); rows
// are strided, so the views of a fused projection need no copy.  The
// arithmetic itself is in pointwise.hpp (shared with the fused GEMM epilogues).
#include "launch.hpp"
#include "pointwise.hpp"

namespace bi {
namespace {

constexpr int kPwThreads = 256;

__global__ __launch_bounds__(kPwThreads) void add_kernel(const uint16_t* x, int64_t ldx, const uint16_t* y,
                                                         int64_t ldy, uint16_t* out, int64_t ldo, int cols8,
                                                         int64_t total8) {
  const int64_t i = (int64_t)blockIdx.x * kPwThreads + threadIdx.x;
  if (i >= total8) return;
  const int64_t r = i / cols8, c = (i - r * cols8) * 8;
  const u32x4_t a = *reinterpret_cast<const u32x4_t*>(x + r * ldx + c);
  const u32x4_t b = *reinterpret_cast<const u32x4_t*>(y + r * ldy + c);
  u32x4_t o;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = pack_bf16x2(pw_add(bf16_lo(a[e]), bf16_lo(b[e])), pw_add(bf16_hi(a[e]), bf16_hi(b[e])));
  *reinterpret_cast<u32x4_t*>(out + r * ldo + c) = o;
}

__global__ __launch_bounds__(kPwThreads) void silu_mul_kernel(const uint16_t* gu, int64_t ldgu, uint16_t* out,
                                                              int64_t ldo, int f, int f8, int64_t total8) {
  const int64_t i = (int64_t)blockIdx.x * kPwThreads + threadIdx.x;
  if (i >= total8) return;
  const int64_t r = i / f8, c = (i - r * f8) * 8;
  const u32x4_t g = *reinterpret_cast<const u32x4_t*>(gu + r * ldgu + c);
  const u32x4_t u = *reinterpret_cast<const u32x4_t*>(gu + r * ldgu + f + c);
  u32x4_t o;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = pack_bf16x2(pw_silu_mul(bf16_lo(g[e]), bf16_lo(u[e])), pw_silu_mul(bf16_hi(g[e]), bf16_hi(u[e])));
  *reinterpret_cast<u32x4_t*>(out + r * ldo + c) = o;
}

unsigned blocks_for(int64_t total8) { return static_cast<unsigned>((total8 + kPwThreads - 1) / kPwThreads); }

}  // namespace

hipError_t launch_add(const void* x, int64_t ldx, const void* y, int64_t ldy, void* out, int64_t ldo, int64_t rows,
                      int64_t cols, hipStream_t stream) {
  const int64_t total8 = rows * (cols / 8);
  if (total8 == 0) return hipSuccess;
  hipLaunchKernelGGL(add_kernel, dim3(blocks_for(total8)), dim3(kPwThreads), 0, stream,
                     static_cast<const uint16_t*>(x), ldx, static_cast<const uint16_t*>(y), ldy,
                     static_cast<uint16_t*>(out), ldo, static_cast<int>(cols / 8), total8);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const void* gu, int64_t ldgu, void* out, int64_t ldo, int64_t rows, int64_t f,
                           hipStream_t stream) {
  const int64_t total8 = rows * (f / 8);
  if (total8 == 0) return hipSuccess;
  hipLaunchKernelGGL(silu_mul_kernel, dim3(blocks_for(total8)), dim3(kPwThreads), 0, stream,
                     static_cast<const uint16_t*>(gu), ldgu, static_cast<uint16_t*>(out), ldo, static_cast<int>(f),
                     static_cast<int>(f / 8), total8);
  return hipGetLastError();
}

}  // namespace bi
