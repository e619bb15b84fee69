// Batch-invariant bf16 GEMM, C = A W^T ("Thinking Machines Lab - Defeating
// Nondeterminism in LLM Inference", section "2. Batch-Invariant Matrix
// Multiplication", figs. "Data-Parallel Matrix Multiplication" and "Split-K
// Matmul").
//
// One kernel configuration for every shape: a 128 (n) x 128 (m) output tile per
// workgroup, K consumed in 64-wide LDS stages, one MFMA instruction
// (v_mfma_f32_16x16x32_bf16), and for every output element a single fp32
// accumulator chain over k = 0, 32, 64, ... in ascending order.  No split-K, no
// choice that depends on M.  Rows of A past M are never loaded and their MFMA
// blocks are skipped; that removes only work on padding, never changes the
// instruction sequence of a real row.
//
// The tile is computed transposed (C^T = W A^T): W rows feed the MFMA A operand
// and A rows the B operand, so each lane ends with 4 consecutive n of one m and
// stores them as one 8-byte (bf16) or 16-byte (fp32) vector.
#include "bi_common.hpp"
#include "launch.hpp"

namespace bi {
namespace {

constexpr int TN = 128;         // output columns (rows of W) per workgroup
constexpr int TM = 128;         // output rows (rows of A) per workgroup
constexpr int BK = 64;          // K per LDS stage
constexpr int kThreads = 256;   // 4 waves: 2 along n x 2 along m
constexpr int WN = 64, WM = 64; // per-wave sub-tile
constexpr int NB = WN / 16, MB = WM / 16;
constexpr int kChunks = BK / 8;                       // 16-byte chunks per tile row
constexpr int kLoadsW = TN * kChunks / kThreads;      // 16-byte loads per thread per stage
constexpr int kLoadsA = TM * kChunks / kThreads;

// LDS element offset of 16-byte chunk c of tile row r (XOR swizzle so the 16
// lanes that read one column chunk of 16 consecutive rows hit distinct banks).
__device__ __forceinline__ int lds_off(int r, int c) { return r * BK + ((c ^ (r & 7)) << 3); }

__device__ __forceinline__ void map_tile(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  // Workgroup i runs on XCD i % 8.  Give each XCD a contiguous range of tiles
  // (so tiles sharing A or W rows share an L2), then walk that range in groups
  // of 8 m-tiles.  Only the placement changes; the arithmetic does not.
  const int total = tiles_m * tiles_n;
  const int q = total >> 3, r = total & 7;
  const int x = pid & 7, j = pid >> 3;
  const int lin = (x < r) ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
  constexpr int G = 8;
  const int group = lin / (G * tiles_n);
  const int first_m = group * G;
  const int gsize = min(tiles_m - first_m, G);
  const int in_group = lin - group * G * tiles_n;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

template <bool kF32Out>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ W, int64_t ldw,
    void* __restrict__ C, int64_t ldc, int M, int N, int K, int tiles_m, int tiles_n, int vec_store) {
  __shared__ __attribute__((aligned(16))) uint16_t sW[2][TN * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][TM * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int l16 = lane & 15, g = lane >> 4;

  int tile_m, tile_n;
  map_tile(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
  const int m0 = tile_m * TM, n0 = tile_n * TN;

  // Global -> register staging for one K stage.
  u32x4_t rw[kLoadsW], ra[kLoadsA];
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kLoadsW; ++i) {
      const int id = tid + i * kThreads, r = id / kChunks, c = id % kChunks;
      const int n = n0 + r, k = k0 + c * 8;
      rw[i] = (n < N && k < K) ? *reinterpret_cast<const u32x4_t*>(W + (int64_t)n * ldw + k)
                               : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i) {
      const int id = tid + i * kThreads, r = id / kChunks, c = id % kChunks;
      const int m = m0 + r, k = k0 + c * 8;
      ra[i] = (m < M && k < K) ? *reinterpret_cast<const u32x4_t*>(A + (int64_t)m * lda + k)
                               : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kLoadsW; ++i) {
      const int id = tid + i * kThreads, r = id / kChunks, c = id % kChunks;
      *reinterpret_cast<u32x4_t*>(&sW[buf][lds_off(r, c)]) = rw[i];
    }
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i) {
      const int id = tid + i * kThreads, r = id / kChunks, c = id % kChunks;
      *reinterpret_cast<u32x4_t*>(&sA[buf][lds_off(r, c)]) = ra[i];
    }
  };

  f32x4_t acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Which 16-row blocks of this wave hold at least one real row of A.
  const int wave_m0 = m0 + wm * WM;
  const int live_mb = min(MB, max(0, (M - wave_m0 + 15) >> 4));

  const int KT = (K + BK - 1) / BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_stage((kt + 1) * BK);
    if (live_mb > 0) {
#pragma unroll
      for (int ks = 0; ks < BK / 32; ++ks) {
        const int c = ks * 4 + g;
        u32x4_t af[NB], bf[MB];
#pragma unroll
        for (int i = 0; i < NB; ++i)
          af[i] = *reinterpret_cast<const u32x4_t*>(&sW[cur][lds_off(wn * WN + i * 16 + l16, c)]);
#pragma unroll
        for (int j = 0; j < MB; ++j)
          bf[j] = *reinterpret_cast<const u32x4_t*>(&sA[cur][lds_off(wm * WM + j * 16 + l16, c)]);
#pragma unroll
        for (int j = 0; j < MB; ++j) {
          if (j < live_mb) {
#pragma unroll
            for (int i = 0; i < NB; ++i) acc[i][j] = mfma_16x16x32(af[i], bf[j], acc[i][j]);
          }
        }
      }
    }
    if (kt + 1 < KT) store_stage(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds C[m][n .. n+3].
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int m = wave_m0 + j * 16 + l16;
    if (j >= live_mb || m >= M) continue;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int n = n0 + wn * WN + i * 16 + 4 * g;
      if (n >= N) continue;
      const f32x4_t v = acc[i][j];
      if constexpr (kF32Out) {
        float* cp = static_cast<float*>(C) + (int64_t)m * ldc + n;
        if (vec_store && n + 3 < N) {
          *reinterpret_cast<f32x4_t*>(cp) = v;
        } else {
          for (int e = 0; e < 4 && n + e < N; ++e) cp[e] = v[e];
        }
      } else {
        uint16_t* cp = static_cast<uint16_t*>(C) + (int64_t)m * ldc + n;
        if (vec_store && n + 3 < N) {
          *reinterpret_cast<u32x2_t*>(cp) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        } else {
          for (int e = 0; e < 4 && n + e < N; ++e) cp[e] = static_cast<uint16_t>(f32_to_bf16(v[e]));
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const void* a, int64_t lda, const void* w, int64_t ldw, void* c, int64_t ldc,
                       bool c_f32, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  const int tiles_m = static_cast<int>((m + TM - 1) / TM);
  const int tiles_n = static_cast<int>((n + TN - 1) / TN);
  const dim3 grid(static_cast<unsigned>(tiles_m * tiles_n)), block(kThreads);
  auto* as = static_cast<const uint16_t*>(a);
  auto* ws = static_cast<const uint16_t*>(w);
  // Vector stores need every row start 16-byte (fp32) / 8-byte (bf16) aligned.
  const int vec = (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(c) & 15u) == 0);
  if (c_f32)
    hipLaunchKernelGGL(gemm_kernel<true>, grid, block, 0, stream, as, lda, ws, ldw, c, ldc, (int)m,
                       (int)n, (int)k, tiles_m, tiles_n, vec);
  else
    hipLaunchKernelGGL(gemm_kernel<false>, grid, block, 0, stream, as, lda, ws, ldw, c, ldc, (int)m,
                       (int)n, (int)k, tiles_m, tiles_n, vec);
  return hipGetLastError();
}

}  // namespace bi
