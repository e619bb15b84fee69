// Row-per-workgroup RMSNorm ("Thinking Machines Lab - Defeating Nondeterminism
// in LLM Inference", section "1. Batch-Invariant RMSNorm", fig. "Data-Parallel
// RMSNorm"): a row's whole reduction stays inside one workgroup, in an order
// fixed by `hidden` alone, for any number of rows.
//
// Reduction order for a row (fp32):
//   thread t owns 16-byte vectors t, t+256, t+512, ...; it accumulates x^2 of
//   its vectors in ascending order with fmaf; then a butterfly over the 64 lanes
//   of its wave; then the four wave totals are added as ((w0 + w1) + w2) + w3.
// y = bf16((x * r) * gamma) with r = rsqrt(sum / hidden + eps).
#include "bi_common.hpp"
#include "launch.hpp"

namespace bi {

constexpr int kNormThreads = 256;

template <int VPT>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(
    const uint16_t* x, int64_t ldx, const uint16_t* __restrict__ gamma, float eps,
    uint16_t* y, int64_t ldy, int hidden) {
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int nvec = hidden >> 3;
  const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(x + row * ldx);
  const u32x4_t* gr = reinterpret_cast<const u32x4_t*>(gamma);

  u32x4_t v[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = tid + i * kNormThreads;
    v[i] = idx < nvec ? __builtin_nontemporal_load(xr + idx) : u32x4_t{0u, 0u, 0u, 0u};
  }
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = bf16_lo(v[i][e]);
      const float hi = bf16_hi(v[i][e]);
      ss = fmaf(lo, lo, ss);
      ss = fmaf(hi, hi, ss);
    }
  }
  ss = wave_sum(ss);
  __shared__ float part[kNormThreads / kWave];
  if ((tid & (kWave - 1)) == 0) part[tid / kWave] = ss;
  __syncthreads();
  float tot = part[0];
#pragma unroll
  for (int w = 1; w < kNormThreads / kWave; ++w) tot = tot + part[w];

  const float r = rsqrtf(tot / static_cast<float>(hidden) + eps);
  u32x4_t* yr = reinterpret_cast<u32x4_t*>(y + row * ldy);
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = tid + i * kNormThreads;
    if (idx < nvec) {
      const u32x4_t gv = gr[idx];
      u32x4_t o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = (bf16_lo(v[i][e]) * r) * bf16_lo(gv[e]);
        const float hi = (bf16_hi(v[i][e]) * r) * bf16_hi(gv[e]);
        o[e] = pack_bf16x2(lo, hi);
      }
      yr[idx] = o;
    }
  }
}

hipError_t launch_rmsnorm(const void* x, int64_t ldx, const void* gamma, float eps, void* y,
                          int64_t ldy, int64_t rows, int hidden, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int nvec = hidden / 8;
  const int vpt = (nvec + kNormThreads - 1) / kNormThreads;  // a function of hidden only
  const dim3 grid(static_cast<unsigned>(rows)), block(kNormThreads);
  auto* xs = static_cast<const uint16_t*>(x);
  auto* gs = static_cast<const uint16_t*>(gamma);
  auto* ys = static_cast<uint16_t*>(y);
  if (vpt <= 1)
    hipLaunchKernelGGL(rmsnorm_kernel<1>, grid, block, 0, stream, xs, ldx, gs, eps, ys, ldy, hidden);
  else if (vpt <= 2)
    hipLaunchKernelGGL(rmsnorm_kernel<2>, grid, block, 0, stream, xs, ldx, gs, eps, ys, ldy, hidden);
  else if (vpt <= 4)
    hipLaunchKernelGGL(rmsnorm_kernel<4>, grid, block, 0, stream, xs, ldx, gs, eps, ys, ldy, hidden);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<8>, grid, block, 0, stream, xs, ldx, gs, eps, ys, ldy, hidden);
  return hipGetLastError();
}

}  // namespace bi
