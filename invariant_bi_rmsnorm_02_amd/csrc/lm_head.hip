// lm_head followed by log_softmax, fused into the GEMM's epilogue
// ("Batch Invariance and Numerical Reproducibility", answer on sampler and
// trainer agreeing on logprobs; "Thinking Machines Lab - Defeating
// Nondeterminism in LLM Inference", section "2. Batch-Invariant Matrix
// Multiplication" for the product itself).
//
//   z[m, n]  = sum_k a[m, k] w[n, k]          (the library GEMM: the same fp32
//                                              MFMA chain per element as
//                                              bi_gemm, in any of its tiles)
//   out[m, n] = z[m, n] - lse[m],   lse[m] = log sum_n e^z[m, n]
//
// Two kernels, one fixed reduction tree for lse that depends on n alone:
//  1. the GEMM writes z into `out` and, for every (row, record), the pair
//     (max, sum e^(z - max)) of the row's values in the record's columns.  A
//     record is 64 columns, or 128 for a weight of at least kGemmWideMinN rows,
//     made of two units of half that width: each lane folds its values of a
//     unit in column order, lanes l ^ 16 and l ^ 32 are combined, then the
//     record's two units in ascending order.  Records and units are a function
//     of n alone, whichever GEMM tile computes them (the tile may follow M:
//     gemm_with_cfg_wide), so every tile writes the same pairs;
//  2. every workgroup of a row folds the row's record pairs (thread t:
//     records t, t + 1024, ... in order; a butterfly over the wavefront; the 16
//     wavefront results in ascending order) and subtracts lse from its segment
//     of the row in place.  A row is split into several segments when there are
//     few rows (scheduling only: every workgroup of a row computes the same lse).
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

// Record geometry of a weight with n rows: a record is the n-tile of the tile
// bi_gemm used for such weights at small M (128 columns from kGemmWideMinN
// rows on, else 64), a unit is one wavefront's columns of that tile.
template <int REC_, int UNIT_>
struct LseGeom {
  static constexpr int REC = REC_, UNIT = UNIT_;
};
using LseGeomWide = LseGeom<GemmWideCfg::TN, GemmWideCfg::WTN>;
using LseGeomNarrow = LseGeom<GemmLibraryCfg::TN, GemmLibraryCfg::WTN>;

template <class Cfg, class Geom, class Pair>
__global__ __launch_bounds__(Cfg::kThreads, Cfg::OCC) void lm_head_lse_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ W, int64_t ldw,
    float* __restrict__ Z, int64_t ldz, Pair* __restrict__ part, int M, int N, int K, int tiles_m, int tiles_n,
    int recs_n, int vec_store) {
  constexpr bool kArg = std::is_same<Pair, MaxSumArg>::value;
  constexpr int UNIT = Geom::UNIT, REC = Geom::REC;
  constexpr int UPW = Cfg::WTN / UNIT;    // units per wavefront
  constexpr int NBU = UNIT / 16;          // MFMA column blocks per unit
  constexpr int UPT = Cfg::TN / UNIT;     // units per tile
  constexpr int UPR = REC / UNIT;         // units per record
  constexpr int RPT = Cfg::TN / REC;      // records per tile
  static_assert(Cfg::WTN % UNIT == 0 && UNIT % 16 == 0 && REC % UNIT == 0 && Cfg::TN % REC == 0, "record geometry");

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

  // Unit pairs.  Lane (l16, g) of wavefront (wn, wm) holds, for m-block j,
  // row wm * WTM + 16 j + l16 at columns wn * WTN + 16 i + 4 g + e.  The
  // pairs are exchanged through the ring's first W stage, which the main loop
  // has finished with (it ends with every load landed and a barrier).
  using Xw = Pair[UPT][Cfg::TM];
  static_assert(sizeof(Xw) <= Cfg::TN * Cfg::BK * sizeof(uint16_t), "exchange fits the ring stage");
  Xw& xw = *reinterpret_cast<Xw*>(GemmRing<Cfg>::template w<0>());
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave % Cfg::WGN, wm = wave / Cfg::WGN;
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < Cfg::MB; ++j) {
    // An m-block that starts past the tile's last row of A has no pair that is
    // written (a wave-uniform test, so the lane exchanges below always see
    // whole wavefronts).  Measured on MI355X, vocabulary 151936: T = 1 / 8
    // logprobs 203 / 212 -> 197 / 207 us, greedy 206 / 210 -> 196 / 198 us;
    // T >= 64 unchanged within noise.
    if (wm * Cfg::WTM + 16 * j >= rows_a) continue;
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
      const int c0 = n0 + wn * Cfg::WTN + u * UNIT;   // first column of the unit
      float v[NBU * 4];
#pragma unroll
      for (int i = 0; i < NBU; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = c0 + 16 * i + 4 * g + e;
          v[4 * i + e] = n < N ? acc[u * NBU + i][j][e] : -INFINITY;
        }
      float mx = -INFINITY;
#pragma unroll
      for (int q = 0; q < NBU * 4; ++q) mx = fmaxf(mx, v[q]);
      // Column order; every term is >= 0 and never -0, so starting from the
      // first term is 0 + term to the bit.  All-masked lanes (mx = -inf) hold 0.
      float s = mx == -INFINITY ? 0.0f : exp2_hw((v[0] - mx) * kLog2e);
#pragma unroll
      for (int q = 1; q < NBU * 4; ++q) s = s + (mx == -INFINITY ? 0.0f : exp2_hw((v[q] - mx) * kLog2e));
      Pair t;
      if constexpr (kArg) {
        // The lane's lowest column holding its maximum (columns rise with q).
        int ix = INT_MAX;
#pragma unroll
        for (int q = NBU * 4 - 1; q >= 0; --q)
          if (v[q] == mx && mx != -INFINITY) ix = c0 + 16 * (q >> 2) + 4 * g + (q & 3);
        t = combine_xor32(combine_xor16(MaxSumArg{mx, s, ix}));
      } else {
        t = combine_xor32(combine_xor16(MaxSum{mx, s}));
      }
      if (g == 0) xw[wn * UPW + u][wm * Cfg::WTM + 16 * j + l16] = t;
    }
  }
  __syncthreads();
  // A record's units in ascending order, one (record, row) per thread.
  for (int idx = threadIdx.x; idx < RPT * Cfg::TM; idx += Cfg::kThreads) {
    const int r = idx / Cfg::TM, row = idx - r * Cfg::TM;
    const int rec = n0 / REC + r;
    if (row >= rows_a || rec >= recs_n) continue;
    Pair t = xw[r * UPR][row];
#pragma unroll
    for (int u = 1; u < UPR; ++u) t = combine(t, xw[r * UPR + u][row]);
    part[(int64_t)(m0 + row) * recs_n + rec] = t;
  }
}

// The row's pairs folded in one fixed tree that depends on tiles_n (the
// record count) alone: thread t takes records t, t + 1024, ... in order; a butterfly over the
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

// Records of a row: the row's pairs.
int lse_tiles(int64_t n) {
  const int64_t rec = n >= kGemmWideMinN ? LseGeomWide::REC : LseGeomNarrow::REC;
  return static_cast<int>((n + rec - 1) / rec);
}

// Launches lm_head_lse_kernel with the GEMM tile of gemm_with_cfg_wide (wide
// weights) or the 64 x 64 tile, and the record geometry of n.
template <class Pair>
hipError_t launch_lse_gemm(const void* a, int64_t lda, const void* w, int64_t ldw, float* out, int64_t ldo,
                           Pair* part, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  const int recs_n = lse_tiles(n);
  auto go = [&](auto cfg, auto geom) {
    using Cfg = decltype(cfg);
    using Geom = decltype(geom);
    if (!gemm_offsets_fit<Cfg>(lda, ldw, k)) return hipErrorInvalidValue;
    const int tiles_m = static_cast<int>((m + Cfg::TM - 1) / Cfg::TM);
    const int tiles_n = static_cast<int>((n + Cfg::TN - 1) / Cfg::TN);
    hipLaunchKernelGGL((lm_head_lse_kernel<Cfg, Geom, Pair>), dim3(static_cast<unsigned>(tiles_m * tiles_n)),
                       dim3(Cfg::kThreads), 0, stream, static_cast<const uint16_t*>(a), lda,
                       static_cast<const uint16_t*>(w), ldw, out, ldo, part, (int)m, (int)n, (int)k, tiles_m,
                       tiles_n, recs_n, 1);
    return hipGetLastError();
  };
  if (n >= kGemmWideMinN)
    return gemm_with_cfg_wide(lda, ldw, m, k, [&](auto cfg) { return go(cfg, LseGeomWide{}); });
  return go(GemmLibraryCfg{}, LseGeomNarrow{});
}

}  // namespace

bool lm_head_supported(int64_t lda, int64_t ldw, int64_t m, int64_t n, int64_t k) {
  auto ok = [&](auto cfg) {
    using C = decltype(cfg);
    const int64_t tiles = ((m + C::TM - 1) / C::TM) * ((n + C::TN - 1) / C::TN);
    return tiles <= 0x7fffffff && gemm_offsets_fit<C>(lda, ldw, k);
  };
  if (n >= kGemmWideMinN) return gemm_with_cfg_wide(lda, ldw, m, k, ok);
  return ok(GemmLibraryCfg{});
}

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
  hipError_t e = launch_lse_gemm(a, lda, w, ldw, out, ldo, part, m, n, k, stream);
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
  hipError_t e = launch_lse_gemm(a, lda, w, ldw, static_cast<float*>(nullptr), 0, part, m, n, k, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(greedy_finalize_kernel, dim3(static_cast<unsigned>(m)), dim3(kFinThreads), 0, stream, part,
                     tiles_n, token, logprob);
  return hipGetLastError();
}

}  // namespace bi
