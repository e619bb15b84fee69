// lm_head followed by log_softmax, fused into the GEMM's epilogue
// ("Batch Invariance and Numerical Reproducibility", answer on sampler and
// trainer agreeing on logprobs; "Thinking Machines Lab - Defeating
// Nondeterminism in LLM Inference", section "2. Batch-Invariant Matrix
// Multiplication" for the product itself).
//
//   z[m, n]  = sum_k a[m, k] w[n, k]          (the library GEMM: bi_gemm's tile
//                                              for this n, same fp32 MFMA
//                                              chain per element)
//   out[m, n] = z[m, n] - lse[m],   lse[m] = log sum_n e^z[m, n]
//
// Two kernels, one fixed reduction tree for lse that depends on n alone:
//  1. the GEMM writes z into `out` and, for every (row, n-tile), the pair
//     (max, sum e^(z - max)) of the row's values in the tile (64 columns, or
//     128 for a weight of at least kGemmWideMinN rows: the tile is a function
//     of n): each lane folds its values in column order, lanes l ^ 16 and
//     l ^ 32 are combined, then the tile's n-wavefronts in ascending order;
//  2. every workgroup of a row folds the row's tile pairs (thread t: tiles t,
//     t + 1024, ... in order; a butterfly over the wavefront; the 16 wavefront
//     results in ascending order) and subtracts lse from its segment of the
//     row in place.  A row is split into several segments when there are few
//     rows (scheduling only: every workgroup of a row computes the same lse).
// Every row's result is a function of its own z values only, so it does not
// depend on the batch.  z is read and written once more (8 bytes per logit)
// instead of the 12 of a separate log_softmax pass.
//
// Greedy sampling (bi_lm_head_greedy) runs the same two kernels with the
// column index of each maximum carried along (ties to the lower index) and no
// z written at all: the second kernel folds the same pairs in the same tree,
// so its lse - and the chosen token's logprob, max - lse - is bitwise what the
// logprobs path gives for that token.
#include <algorithm>
#include <climits>
#include <type_traits>

#include "gemm_kernel.hpp"
#include "launch.hpp"
#include "lse.hpp"

namespace bi {
namespace {

constexpr int kFinThreads = 1024;
constexpr int64_t kFinBlocks = 512;    // finalize workgroups aimed at when rows are few
constexpr int64_t kFinSegsMax = 256;

template <class Cfg, class Pair>
__global__ __launch_bounds__(Cfg::kThreads, Cfg::OCC) void lm_head_lse_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ W, int64_t ldw,
    float* __restrict__ Z, int64_t ldz, Pair* __restrict__ part, int M, int N, int K, int tiles_m, int tiles_n,
    int vec_store) {
  constexpr bool kArg = std::is_same<Pair, MaxSumArg>::value;

  int tile_m, tile_n;
  gemm_map_tile(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
  const int m0 = tile_m * Cfg::TM, n0 = tile_n * Cfg::TN;
  const int rows_w = min(Cfg::TN, N - n0), rows_a = min(Cfg::TM, M - m0);

  GemmOperands<Cfg> op;
  op.rsw = gemm_rsrc(W + (int64_t)n0 * ldw, (uint32_t)(((int64_t)(rows_w - 1) * ldw + K) * 2));
  op.rsa = gemm_rsrc(A + (int64_t)m0 * lda, (uint32_t)(((int64_t)(rows_a - 1) * lda + K) * 2));
#pragma unroll
  for (int i = 0; i < Cfg::LW; ++i) {
    const int r = gemm_slot_row<Cfg>(i);
    op.wofs[i] = r < rows_w ? (uint32_t)((int64_t)r * ldw * 2) + gemm_slot_chunk_bytes<Cfg>(i) : kBufOOB;
  }
#pragma unroll
  for (int i = 0; i < Cfg::LA; ++i) {
    const int r = gemm_slot_row<Cfg>(i);
    op.aofs[i] = r < rows_a ? (uint32_t)((int64_t)r * lda * 2) + gemm_slot_chunk_bytes<Cfg>(i) : kBufOOB;
  }

  f32x4_t acc[Cfg::NB][Cfg::MB];
  gemm_zero<Cfg>(acc);
  gemm_mainloop<Cfg>(op, K, rows_a, acc);

  if constexpr (!kArg) {
    gemm_epilogue<Cfg>(acc, rows_a, n0, N, [&](int m, int n, f32x4_t v, int cnt) {
      gemm_store4_f32(Z + (int64_t)(m0 + m) * ldz + n, v, cnt, vec_store);
    });
  }

  // Tile pairs.  Lane (l16, g) of wavefront (wn, wm) holds, for m-block j,
  // row wm * WTM + 16 j + l16 at columns wn * WTN + 16 i + 4 g + e.  The
  // wavefronts exchange them through the ring's first W stage, which the main
  // loop has finished with (it ends with every load landed and a barrier).
  using Xw = Pair[Cfg::WGN][Cfg::WGM][Cfg::MB][16];
  static_assert(sizeof(Xw) <= Cfg::TN * Cfg::BK * sizeof(uint16_t), "exchange fits the ring stage");
  Xw& xw = *reinterpret_cast<Xw*>(GemmRing<Cfg>::template w<0>());
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave % Cfg::WGN, wm = wave / Cfg::WGN;
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < Cfg::MB; ++j) {
    float v[Cfg::NB * 4];
#pragma unroll
    for (int i = 0; i < Cfg::NB; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = n0 + wn * Cfg::WTN + 16 * i + 4 * g + e;
        v[4 * i + e] = n < N ? acc[i][j][e] : -INFINITY;
      }
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < Cfg::NB * 4; ++q) mx = fmaxf(mx, v[q]);
    // Column order; every term is >= 0 and never -0, so starting from the
    // first term is 0 + term to the bit.  All-masked lanes (mx = -inf) hold 0.
    float s = mx == -INFINITY ? 0.0f : exp2_hw((v[0] - mx) * kLog2e);
#pragma unroll
    for (int q = 1; q < Cfg::NB * 4; ++q) s = s + (mx == -INFINITY ? 0.0f : exp2_hw((v[q] - mx) * kLog2e));
    Pair t;
    if constexpr (kArg) {
      // The lane's lowest column holding its maximum (columns rise with q).
      int ix = INT_MAX;
#pragma unroll
      for (int q = Cfg::NB * 4 - 1; q >= 0; --q)
        if (v[q] == mx && mx != -INFINITY) ix = n0 + wn * Cfg::WTN + 16 * (q >> 2) + 4 * g + (q & 3);
      t = combine_xor32(combine_xor16(MaxSumArg{mx, s, ix}));
    } else {
      t = combine_xor32(combine_xor16(MaxSum{mx, s}));
    }
    if (g == 0) xw[wn][wm][j][l16] = t;
  }
  __syncthreads();
  if (wn == 0 && g == 0) {
#pragma unroll
    for (int j = 0; j < Cfg::MB; ++j) {
      const int row = wm * Cfg::WTM + 16 * j + l16;
      if (row >= rows_a) continue;
      Pair t = xw[0][wm][j][l16];
#pragma unroll
      for (int w = 1; w < Cfg::WGN; ++w) t = combine(t, xw[w][wm][j][l16]);
      part[(int64_t)(m0 + row) * tiles_n + tile_n] = t;
    }
  }
}

// The row's pairs folded in one fixed tree that depends on tiles_n alone:
// thread t takes tiles t, t + 1024, ... in order; a butterfly over the
// wavefront; the 16 wavefront results in ascending order.  Every thread of the
// workgroup returns the total.
template <class Pair>
__device__ __forceinline__ Pair fold_row_pairs(const Pair* __restrict__ pr, int tiles_n, Pair empty) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  Pair acc = empty;
  for (int t = tid; t < tiles_n; t += kFinThreads) acc = combine(acc, pr[t]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc = combine(acc, shfl_xor_pair(acc, o));
  __shared__ Pair wpart[kFinThreads / kWave];
  if (lane == 0) wpart[wave] = acc;
  __syncthreads();
  Pair tot = wpart[0];
#pragma unroll
  for (int w = 1; w < kFinThreads / kWave; ++w) tot = combine(tot, wpart[w]);
  return tot;
}

__global__ __launch_bounds__(kFinThreads) void lse_finalize_kernel(float* __restrict__ Z, int64_t ldz,
                                                                   const MaxSum* __restrict__ part, int tiles_n,
                                                                   int N, int segs, float* __restrict__ lse_out) {
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x / segs;
  const int seg = blockIdx.x - (int)(row * segs);
  const MaxSum tot = fold_row_pairs(part + row * tiles_n, tiles_n, MaxSum{-INFINITY, 0.0f});
  const float lse = lse_of(tot);
  if (lse_out != nullptr && seg == 0 && tid == 0) lse_out[row] = lse;
  f32x4_t* zr = reinterpret_cast<f32x4_t*>(Z + row * ldz);
  const int nv = N >> 2, per = (nv + segs - 1) / segs;
  const int hi = min(nv, (seg + 1) * per);
#pragma unroll 4
  for (int i = seg * per + tid; i < hi; i += kFinThreads) {
    const f32x4_t v = zr[i];
    zr[i] = f32x4_t{v[0] - lse, v[1] - lse, v[2] - lse, v[3] - lse};
  }
}

// Greedy: the row's token (lowest index of its maximum logit) and that
// token's logprob, max - lse.
__global__ __launch_bounds__(kFinThreads) void greedy_finalize_kernel(const MaxSumArg* __restrict__ part,
                                                                      int tiles_n, int32_t* __restrict__ token,
                                                                      float* __restrict__ logprob) {
  const int64_t row = blockIdx.x;
  const MaxSumArg tot = fold_row_pairs(part + row * tiles_n, tiles_n, MaxSumArg{-INFINITY, 0.0f, INT_MAX});
  if (threadIdx.x == 0) {
    token[row] = tot.i;
    if (logprob != nullptr) logprob[row] = tot.m - lse_of(MaxSum{tot.m, tot.s});
  }
}

// n-tiles of the GEMM configuration bi_gemm uses for this n: the row's pairs.
int lse_tiles(int64_t n) {
  return gemm_with_cfg(n, [&](auto cfg) { return static_cast<int>((n + decltype(cfg)::TN - 1) / decltype(cfg)::TN); });
}

}  // namespace

size_t lm_head_workspace_bytes(int64_t m, int64_t n) {
  const size_t bytes = static_cast<size_t>(m) * static_cast<size_t>(lse_tiles(n)) * sizeof(MaxSum);
  return (bytes + 255) / 256 * 256;
}

hipError_t launch_lm_head_logprobs(const void* a, int64_t lda, const void* w, int64_t ldw, float* out, int64_t ldo,
                                   float* lse, int64_t m, int64_t n, int64_t k, void* workspace,
                                   hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  const int tiles_n = lse_tiles(n);
  auto* part = static_cast<MaxSum*>(workspace);
  hipError_t e = gemm_with_cfg(n, [&](auto cfg) {
    using Cfg = decltype(cfg);
    if (!gemm_offsets_fit<Cfg>(lda, ldw, k)) return hipErrorInvalidValue;
    const int tiles_m = static_cast<int>((m + Cfg::TM - 1) / Cfg::TM);
    hipLaunchKernelGGL((lm_head_lse_kernel<Cfg, MaxSum>), dim3(static_cast<unsigned>(tiles_m * tiles_n)),
                       dim3(Cfg::kThreads), 0, stream, static_cast<const uint16_t*>(a), lda,
                       static_cast<const uint16_t*>(w), ldw, out, ldo, part, (int)m, (int)n, (int)k, tiles_m,
                       tiles_n, 1);
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;
  // Segments per row: enough workgroups to spread few rows over the GPU.
  const int segs = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>({kFinSegsMax, (kFinBlocks + m - 1) / m,
                                                                            (n / 4 + kFinThreads - 1) / kFinThreads})));
  hipLaunchKernelGGL(lse_finalize_kernel, dim3(static_cast<unsigned>(m * segs)), dim3(kFinThreads), 0, stream, out,
                     ldo, part, tiles_n, (int)n, segs, lse);
  return hipGetLastError();
}

size_t lm_head_greedy_workspace_bytes(int64_t m, int64_t n) {
  const size_t bytes = static_cast<size_t>(m) * static_cast<size_t>(lse_tiles(n)) * sizeof(MaxSumArg);
  return (bytes + 255) / 256 * 256;
}

hipError_t launch_lm_head_greedy(const void* a, int64_t lda, const void* w, int64_t ldw, int32_t* token,
                                 float* logprob, int64_t m, int64_t n, int64_t k, void* workspace,
                                 hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  const int tiles_n = lse_tiles(n);
  auto* part = static_cast<MaxSumArg*>(workspace);
  hipError_t e = gemm_with_cfg(n, [&](auto cfg) {
    using Cfg = decltype(cfg);
    if (!gemm_offsets_fit<Cfg>(lda, ldw, k)) return hipErrorInvalidValue;
    const int tiles_m = static_cast<int>((m + Cfg::TM - 1) / Cfg::TM);
    hipLaunchKernelGGL((lm_head_lse_kernel<Cfg, MaxSumArg>), dim3(static_cast<unsigned>(tiles_m * tiles_n)),
                       dim3(Cfg::kThreads), 0, stream, static_cast<const uint16_t*>(a), lda,
                       static_cast<const uint16_t*>(w), ldw, nullptr, 0, part, (int)m, (int)n, (int)k, tiles_m,
                       tiles_n, 1);
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(greedy_finalize_kernel, dim3(static_cast<unsigned>(m)), dim3(kFinThreads), 0, stream, part,
                     tiles_n, token, logprob);
  return hipGetLastError();
}

}  // namespace bi
