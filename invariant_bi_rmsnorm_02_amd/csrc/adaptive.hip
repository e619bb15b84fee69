// Shape-adaptive comparators: how the same three operations would usually be
// parallelised if batch invariance did not matter.  They exist to measure the
// cost of invariance and to show the hazard; they are NOT batch-invariant and
// nothing in libbi.so uses them.  The hazards they reproduce are the ones named
// in "Thinking Machines Lab - Defeating Nondeterminism in LLM Inference":
//   - split-K matmul when M and N are too small to fill the GPU (section "2.
//     Batch-Invariant Matrix Multiplication", fig. "Split-K Matmul"): the split
//     count follows the tile count, so row m's K order depends on M;
//   - split-KV with a fixed NUMBER of splits (section "3. Batch-Invariant
//     Attention", fig. "Fixed Number Split KV Strategy"): the split size
//     follows a split count S chosen from the batch, so the chunk boundaries
//     move with the batch;
//   - split-reduction RMSNorm at small batch (section "1. Batch-Invariant
//     RMSNorm", fig. "Split-Reduction RMSNorm"): a row's sum of squares is cut
//     into a number of slices that depends on the number of rows.
// Each variant reuses the invariant library's building blocks (GEMM main loop,
// attention chunk step and merge) so that the timing difference is the
// parallelisation, not the code quality.
#include <algorithm>

#include "attn_decode_impl.hpp"
#include "bi_adaptive.h"
#include "gemm_kernel.hpp"
#include "launch.hpp"

namespace bi {
namespace {

constexpr int kTargetWorkgroups = 512;   // 2 x 256 CUs: what the heuristics aim to fill

// ------------------------------------------------------------------ split-K GEMM

using Cfg = GemmLibraryCfg;

struct SplitK {
  int splits;   // number of K slices
  int kc;       // K per slice (multiple of the stage depth)
};

SplitK choose_splitk(int64_t m, int64_t n, int64_t k) {
  const int64_t tiles = ((m + Cfg::TM - 1) / Cfg::TM) * ((n + Cfg::TN - 1) / Cfg::TN);
  int64_t s = 1;
  if (tiles < kTargetWorkgroups) s = std::min<int64_t>((kTargetWorkgroups + tiles - 1) / tiles, k / 256);
  s = std::max<int64_t>(s, 1);
  int64_t kc = (k + s - 1) / s;
  kc = (kc + Cfg::BK - 1) / Cfg::BK * Cfg::BK;
  return SplitK{static_cast<int>((k + kc - 1) / kc), static_cast<int>(kc)};
}

__global__ __launch_bounds__(Cfg::kThreads, 2) void splitk_partial_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ W, int64_t ldw,
    float* __restrict__ ws, int M, int N, int K, int kc, int tiles_m, int tiles_n) {
  const int split = blockIdx.y;
  int tile_m, tile_n;
  gemm_map_tile(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
  const int m0 = tile_m * Cfg::TM, n0 = tile_n * Cfg::TN;
  const int rows_w = min(Cfg::TN, N - n0), rows_a = min(Cfg::TM, M - m0);
  const int k0 = split * kc, klen = min(kc, K - k0);

  GemmOperands<Cfg> op;
  op.rsw = gemm_rsrc(W + (int64_t)n0 * ldw, (uint32_t)(((int64_t)(rows_w - 1) * ldw + K) * 2));
  op.rsa = gemm_rsrc(A + (int64_t)m0 * lda, (uint32_t)(((int64_t)(rows_a - 1) * lda + K) * 2));
#pragma unroll
  for (int i = 0; i < Cfg::LW; ++i) {
    const int r = gemm_slot_row<Cfg>(i);
    op.wofs[i] = r < rows_w ? (uint32_t)(((int64_t)r * ldw + k0) * 2) + gemm_slot_chunk_bytes<Cfg>(i) : kBufOOB;
  }
#pragma unroll
  for (int i = 0; i < Cfg::LA; ++i) {
    const int r = gemm_slot_row<Cfg>(i);
    op.aofs[i] = r < rows_a ? (uint32_t)(((int64_t)r * lda + k0) * 2) + gemm_slot_chunk_bytes<Cfg>(i) : kBufOOB;
  }
  f32x4_t acc[Cfg::NB][Cfg::MB];
  gemm_zero<Cfg>(acc);
  gemm_mainloop<Cfg>(op, klen, rows_a, acc);
  float* part = ws + (int64_t)split * M * N;
  gemm_epilogue<Cfg>(acc, rows_a, n0, N, [&](int m, int n, f32x4_t v, int cnt) {
    gemm_store4_f32(part + (int64_t)(m0 + m) * N + n, v, cnt, (N & 3) == 0);
  });
}

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, int splits, int64_t MN,
                                                            int N, uint16_t* __restrict__ C, int64_t ldc) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < MN; i += (int64_t)gridDim.x * 256) {
    float s = 0.0f;
    for (int p = 0; p < splits; ++p) s = s + ws[(int64_t)p * MN + i];
    C[(i / N) * ldc + i % N] = static_cast<uint16_t>(f32_to_bf16(s));
  }
}

// ------------------------------------------------------------------ decode with a batch-chosen split size

// libbi's decode (attn_decode_impl.hpp: the chunk step, the work queue and its
// placement, the in-wave fold, the merge) with one thing changed: the split
// size is picked from the batch, as a fixed split COUNT would pick it.  S =
// ceil(kTargetWorkgroups / (num_seqs * Hkv)) splits of a max_seq_len-key
// sequence, i.e. ceil(max_seq_len / S) keys, taken as the next power of two
// from max(32, page size) up to kDecodeMaxSplit.  At 256 keys the call is
// libbi's own decode, bit for bit; any other size moves the chunk boundaries,
// and with them the bits, as the batch changes.
constexpr int kDecodeMinSplit = 32;
constexpr int kDecodeMaxSplit = 512;    // longer splits spill the decode loop's fragment registers

int decode_split_keys(int num_seqs, int num_kv_heads, int max_seq_len, int page_size) {
  const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
  const int64_t splits = std::max<int64_t>(1, (kTargetWorkgroups + pairs - 1) / pairs);
  const int64_t want = (std::max(max_seq_len, 1) + splits - 1) / splits;
  int cs = std::max(kDecodeMinSplit, page_size);
  while (cs < want && cs < kDecodeMaxSplit) cs *= 2;
  return cs;
}

template <int D>
hipError_t launch_split_decode(int cs, const void* q, int64_t ld_q, const AttnGeom& g, const int32_t* seq_lens,
                               int num_seqs, int max_seq_len, void* out, float* lse, void* ws, hipStream_t st) {
  switch (cs) {
    case 32: return launch<D, 32>(q, ld_q, g, seq_lens, num_seqs, max_seq_len, out, lse, ws, st);
    case 64: return launch<D, 64>(q, ld_q, g, seq_lens, num_seqs, max_seq_len, out, lse, ws, st);
    case 128: return launch<D, 128>(q, ld_q, g, seq_lens, num_seqs, max_seq_len, out, lse, ws, st);
    case 256: return launch<D, 256>(q, ld_q, g, seq_lens, num_seqs, max_seq_len, out, lse, ws, st);
    case 512: return launch<D, 512>(q, ld_q, g, seq_lens, num_seqs, max_seq_len, out, lse, ws, st);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------------ split-reduction RMSNorm

constexpr int kNormT = 256;

int norm_slices(int64_t rows, int hidden) {
  if (rows >= kTargetWorkgroups / 2) return 1;
  const int by_rows = static_cast<int>((kTargetWorkgroups / 2 + rows - 1) / rows);
  return std::max(1, std::min(by_rows, hidden / (8 * kNormT)));   // a slice is at least one vector per thread
}

// Slice p of row r: 16-byte vectors [p * per, min((p + 1) * per, nvec)).
__global__ __launch_bounds__(kNormT) void norm_partial_kernel(const uint16_t* __restrict__ x, int64_t ldx, int hidden,
                                                              int slices, float* __restrict__ ws) {
  const int p = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const int nvec = hidden >> 3, per = (nvec + slices - 1) / slices;
  const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(x + (int64_t)r * ldx);
  float ss = 0.0f;
  for (int i = p * per + tid; i < min(nvec, (p + 1) * per); i += kNormT) {
    const u32x4_t v = xr[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ss = fmaf(bf16_lo(v[e]), bf16_lo(v[e]), ss);
      ss = fmaf(bf16_hi(v[e]), bf16_hi(v[e]), ss);
    }
  }
  ss = wave_sum(ss);
  __shared__ float part[kNormT / kWave];
  if ((tid & 63) == 0) part[tid / kWave] = ss;
  __syncthreads();
  if (tid == 0) {
    float t = part[0];
    for (int w = 1; w < kNormT / kWave; ++w) t = t + part[w];
    ws[(int64_t)r * slices + p] = t;
  }
}

__global__ __launch_bounds__(kNormT) void norm_apply_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                            const uint16_t* __restrict__ gamma, float eps,
                                                            uint16_t* __restrict__ y, int64_t ldy, int hidden,
                                                            int slices, const float* __restrict__ ws) {
  const int p = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  float tot = 0.0f;
  for (int q = 0; q < slices; ++q) tot = tot + ws[(int64_t)r * slices + q];
  const float rs = rsqrtf(tot / static_cast<float>(hidden) + eps);
  const int nvec = hidden >> 3, per = (nvec + slices - 1) / slices;
  const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(x + (int64_t)r * ldx);
  const u32x4_t* gr = reinterpret_cast<const u32x4_t*>(gamma);
  u32x4_t* yr = reinterpret_cast<u32x4_t*>(y + (int64_t)r * ldy);
  for (int i = p * per + tid; i < min(nvec, (p + 1) * per); i += kNormT) {
    const u32x4_t v = xr[i], gv = gr[i];
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = pack_bf16x2((bf16_lo(v[e]) * rs) * bf16_lo(gv[e]), (bf16_hi(v[e]) * rs) * bf16_hi(gv[e]));
    yr[i] = o;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bi_status from_hip(hipError_t e) { return e == hipSuccess ? BI_OK : BI_ERR_HIP; }

}  // namespace
}  // namespace bi

using namespace bi;

extern "C" {

int32_t bia_gemm_splits(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0) return 1;
  return choose_splitk(m, n, k).splits;
}

size_t bia_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0) return 0;
  const SplitK s = choose_splitk(m, n, k);
  return s.splits > 1 ? (size_t)s.splits * (size_t)m * (size_t)n * sizeof(float) : 0;
}

bi_status bia_gemm(const void* a, int64_t lda, const void* w, int64_t ldw, void* c, int64_t ldc, int64_t m,
                   int64_t n, int64_t k, void* workspace, size_t workspace_bytes, bi_stream_t stream) {
  if (m < 0 || n < 0 || k <= 0) return BI_ERR_INVALID_ARG;
  if (m == 0 || n == 0) return BI_OK;
  if (!a || !w || !c || !aligned16(a) || !aligned16(w)) return BI_ERR_INVALID_ARG;
  if (k % 32 || lda < k || ldw < k || ldc < n || lda % 8 || ldw % 8) return BI_ERR_INVALID_ARG;
  if (!gemm_supported(lda, ldw, m, n, k)) return BI_ERR_UNSUPPORTED;
  const SplitK s = choose_splitk(m, n, k);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s.splits == 1) return from_hip(launch_gemm(a, lda, w, ldw, c, ldc, false, m, n, k, st));
  if (!workspace || !aligned16(workspace) || workspace_bytes < bia_gemm_workspace_bytes(m, n, k))
    return BI_ERR_WORKSPACE;
  const int tiles_m = static_cast<int>((m + Cfg::TM - 1) / Cfg::TM), tiles_n = static_cast<int>((n + Cfg::TN - 1) / Cfg::TN);
  hipLaunchKernelGGL(splitk_partial_kernel, dim3(tiles_m * tiles_n, s.splits), dim3(Cfg::kThreads), 0, st,
                     static_cast<const uint16_t*>(a), lda, static_cast<const uint16_t*>(w), ldw,
                     static_cast<float*>(workspace), (int)m, (int)n, (int)k, s.kc, tiles_m, tiles_n);
  const int64_t mn = m * n;
  const int blocks = static_cast<int>(std::min<int64_t>((mn + 255) / 256, 4096));
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, st, static_cast<const float*>(workspace),
                     s.splits, mn, (int)n, static_cast<uint16_t*>(c), ldc);
  return from_hip(hipGetLastError());
}

int32_t bia_attn_decode_split_keys(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len, int32_t page_size) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || page_size < 16 || page_size > 256 || (page_size & (page_size - 1)))
    return kChunk;
  return decode_split_keys(num_seqs, num_kv_heads, max_seq_len, page_size);
}

size_t bia_attn_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_seq_len, int32_t page_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
  const int cs = bia_attn_decode_split_keys(num_seqs, num_kv_heads, max_seq_len, page_size);
  return decode_workspace_bytes_cs(num_seqs, num_q_heads, head_dim, std::max(max_seq_len, 1), cs);
}

bi_status bia_attn_decode(const void* q, int64_t ld_q, const void* k_cache, const void* v_cache, int32_t num_pages,
                          const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
                          int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t page_size, float softmax_scale, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, bi_stream_t stream) {
  if (num_seqs < 0 || max_seq_len < 0) return BI_ERR_INVALID_ARG;
  if (num_seqs == 0) return BI_OK;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return BI_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || !aligned16(k_cache) || !aligned16(v_cache)) return BI_ERR_INVALID_ARG;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads || num_pages <= 0) return BI_ERR_INVALID_ARG;
  if (max_pages_per_seq <= 0) return BI_ERR_INVALID_ARG;
  const int G = num_q_heads / num_kv_heads;
  if (G > 16 || (head_dim != 64 && head_dim != 128)) return BI_ERR_UNSUPPORTED;
  int l2 = 0;
  while ((1 << l2) < page_size) ++l2;
  if ((1 << l2) != page_size || l2 < 4 || l2 > 8) return BI_ERR_UNSUPPORTED;
  if (ld_q < (int64_t)num_q_heads * head_dim || ld_q % 8) return BI_ERR_INVALID_ARG;
  if (num_seqs > 65535 || max_seq_len > (1 << 24)) return BI_ERR_UNSUPPORTED;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) ||
      workspace_bytes < bia_attn_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                                        page_size))
    return BI_ERR_WORKSPACE;
  const int cs = decode_split_keys(num_seqs, num_kv_heads, max_seq_len, page_size);
  AttnGeom g;
  g.k_cache = k_cache;
  g.v_cache = v_cache;
  g.num_pages = num_pages;
  g.block_table = block_table;
  g.max_pages_per_seq = max_pages_per_seq;
  g.num_q_heads = num_q_heads;
  g.num_kv_heads = num_kv_heads;
  g.head_dim = head_dim;
  g.log2_page = l2;
  g.scale_log2 = static_cast<float>(static_cast<double>(softmax_scale) * 1.4426950408889634);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int msl = std::max(max_seq_len, 1);
  return from_hip(head_dim == 64 ? launch_split_decode<64>(cs, q, ld_q, g, seq_lens, num_seqs, msl, out, lse, workspace, st)
                                 : launch_split_decode<128>(cs, q, ld_q, g, seq_lens, num_seqs, msl, out, lse, workspace,
                                                            st));
}

int32_t bia_rmsnorm_slices(int64_t rows, int64_t hidden) {
  return rows > 0 && hidden > 0 ? norm_slices(rows, static_cast<int>(hidden)) : 1;
}

size_t bia_rmsnorm_workspace_bytes(int64_t rows, int64_t hidden) {
  if (rows <= 0 || hidden <= 0) return 0;
  const int s = norm_slices(rows, static_cast<int>(hidden));
  return s > 1 ? (size_t)rows * s * sizeof(float) : 0;
}

bi_status bia_rmsnorm(const void* x, int64_t ldx, const void* gamma, float eps, void* y, int64_t ldy, int64_t rows,
                      int64_t hidden, void* workspace, size_t workspace_bytes, bi_stream_t stream) {
  if (rows < 0 || hidden <= 0) return BI_ERR_INVALID_ARG;
  if (rows == 0) return BI_OK;
  if (!x || !gamma || !y || !aligned16(x) || !aligned16(gamma) || !aligned16(y)) return BI_ERR_INVALID_ARG;
  if (hidden % 8 || hidden > 16384 || rows > 65535) return BI_ERR_UNSUPPORTED;
  if (ldx < hidden || ldy < hidden || ldx % 8 || ldy % 8) return BI_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int s = norm_slices(rows, static_cast<int>(hidden));
  if (s == 1) return from_hip(launch_rmsnorm(x, ldx, gamma, eps, y, ldy, rows, static_cast<int>(hidden), st));
  if (!workspace || workspace_bytes < bia_rmsnorm_workspace_bytes(rows, hidden)) return BI_ERR_WORKSPACE;
  float* ws = static_cast<float*>(workspace);
  hipLaunchKernelGGL(norm_partial_kernel, dim3(s, rows), dim3(kNormT), 0, st, static_cast<const uint16_t*>(x), ldx,
                     (int)hidden, s, ws);
  hipLaunchKernelGGL(norm_apply_kernel, dim3(s, rows), dim3(kNormT), 0, st, static_cast<const uint16_t*>(x), ldx,
                     static_cast<const uint16_t*>(gamma), eps, static_cast<uint16_t*>(y), ldy, (int)hidden, s, ws);
  return from_hip(hipGetLastError());
}

}  // extern "C"
