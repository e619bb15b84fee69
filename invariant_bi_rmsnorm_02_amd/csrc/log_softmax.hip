// Row-wise log_softmax of fp32 logits ("Batch Invariance and Numerical
// Reproducibility", answer on sampler and trainer agreeing on logprobs: the
// logprob of a token must not depend on what else was in the batch).
//
// One workgroup per row, one fixed order whatever the number of rows:
//   thread t takes its float4 vectors t, t+1024, t+2048, ... four at a time
//   (16 values, in order); per group it takes the group max, rescales its
//   running sum once to the new max and adds the 16 terms exp(x - max) in
//   order; threads are combined by a butterfly over each wavefront and the 16
//   wave results are folded in ascending wave order.  out = z - (max + ln sum).
// The next group's loads are issued before the current group is reduced, so
// eight 16-byte loads per thread are in flight; there are no data-dependent
// branches.
#include "launch.hpp"
#include "lse.hpp"

namespace bi {
namespace {

constexpr int kLsmThreads = 1024;

__global__ __launch_bounds__(kLsmThreads) void log_softmax_kernel(const float* z, int64_t ld_in,
                                                                  float* out, int64_t ld_out, int vocab) {
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const f32x4_t* zr = reinterpret_cast<const f32x4_t*>(z + row * ld_in);
  const int nvec = vocab >> 2;

  constexpr int kGroup = 4;   // float4 vectors per thread per step
  // Loads are unconditional (a vector past the row reads the row's last
  // vector); padding is replaced by -inf where the group is reduced, so no
  // load waits on a branch.
  auto load_group = [&](int j0, f32x4_t (&v)[kGroup]) {
#pragma unroll
    for (int q = 0; q < kGroup; ++q) v[q] = zr[min(tid + (j0 + q) * kLsmThreads, nvec - 1)];
  };
  MaxSum acc{-INFINITY, 0.0f};
  const int steps = (nvec + kLsmThreads - 1) / kLsmThreads;   // vectors per thread, rounded up
  f32x4_t cur[kGroup], nxt[kGroup];
  load_group(0, cur);
  for (int j0 = 0; j0 < steps; j0 += kGroup) {
    load_group(j0 + kGroup, nxt);
#pragma unroll
    for (int q = 0; q < kGroup; ++q)
      if (tid + (j0 + q) * kLsmThreads >= nvec) cur[q] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    float gm = cur[0][0];
#pragma unroll
    for (int q = 0; q < kGroup; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) gm = fmaxf(gm, cur[q][e]);
    const float m = fmaxf(acc.m, gm);
    // ms keeps exp finite while every value so far is -inf (padding).
    const float ms = m == -INFINITY ? 0.0f : m;
    float s = acc.m == -INFINITY ? 0.0f : acc.s * exp2_hw((acc.m - ms) * kLog2e);
#pragma unroll
    for (int q = 0; q < kGroup; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) s = s + exp2_hw((cur[q][e] - ms) * kLog2e);
    acc = MaxSum{m, s};
#pragma unroll
    for (int q = 0; q < kGroup; ++q) cur[q] = nxt[q];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    MaxSum other{shfl_xor(acc.m, o), shfl_xor(acc.s, o)};
    acc = combine(acc, other);
  }
  __shared__ MaxSum part[kLsmThreads / kWave];
  if ((tid & (kWave - 1)) == 0) part[tid / kWave] = acc;
  __syncthreads();
  MaxSum tot = part[0];
#pragma unroll
  for (int w = 1; w < kLsmThreads / kWave; ++w) tot = combine(tot, part[w]);
  const float lse = lse_of(tot);

  f32x4_t* orow = reinterpret_cast<f32x4_t*>(out + row * ld_out);
#pragma unroll 4
  for (int i = tid; i < nvec; i += kLsmThreads) {
    const f32x4_t v = zr[i];
    orow[i] = f32x4_t{v[0] - lse, v[1] - lse, v[2] - lse, v[3] - lse};
  }
}

}  // namespace

hipError_t launch_log_softmax(const float* logits, int64_t ld_in, float* out, int64_t ld_out,
                              int64_t rows, int64_t vocab, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(log_softmax_kernel, dim3(static_cast<unsigned>(rows)), dim3(kLsmThreads), 0,
                     stream, logits, ld_in, out, ld_out, static_cast<int>(vocab));
  return hipGetLastError();
}

}  // namespace bi
