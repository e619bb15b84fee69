// Mixture-of-experts FFN for a batch of tokens, batch-invariant: a token's
// output depends only on its own hidden state, its routing and the weights,
// never on which other tokens share its experts ("Batch Invariance and
// Numerical Reproducibility", answer on a fixed per-element reduction order:
// the order may not change with the batch's size or a row's place in it).  The
// expert FFN itself
// is not on the pages; it is the workload's: y_t = sum over the top-k slots s,
// in ascending s, of w[t, s] * W_down[e] SiLU(W_up[e] x_t), e = experts[t, s].
//
// Four steps, all on the caller's stream, no atomics anywhere:
//  1. moe_count_kernel (one workgroup per expert): how many (token, slot)
//     pairs route to the expert.
//  2. moe_place_kernel (one workgroup per expert): expert-major order of the
//     pairs, stable in pair order (p = t * top_k + s), via ballot prefix sums;
//     row r of the order holds pair src; pos[p] = r.  Also each expert's first
//     row and first 64-row tile.
//  3. Grouped GEMMs with a library GEMM configuration and its K loop
//     (gemm_kernel.hpp): h[r] = bf16(SiLU(W_up[e] x[token(r)])) with the A rows
//     gathered from x, then o[r] = W_down[e] h[r] in fp32.  A row's result
//     depends only on that row: where it sits among its expert's rows (which
//     the batch decides) changes which workgroup computes it, not how.
//  4. moe_combine_kernel (one workgroup per token): fp32 sum over s ascending
//     of w[t, s] * o[pos[t, s]], rounded once to bf16.
//
// The router (bi_moe_route) feeds it: logits = x W_gate^T with the library
// GEMM (fp32 out), then moe_topk_kernel (one wavefront per token) picks the
// top_k experts in a total order - the larger logit first, the lower expert
// index among equal logits, a NaN logit below every number - so the choice
// depends on the token's logits alone and not on any reduction order; the
// weights are the softmax of the chosen logits, summed in slot order.
#include <algorithm>
#include <climits>

#include "gemm_kernel.hpp"
#include "launch.hpp"

namespace bi {
namespace {

constexpr int kRouteThreads = 256;

// The grouped GEMMs' configurations.  Both are library GEMM tiles (the same
// fp32 MFMA chain per element over k ascending), so the choice between them,
// made from the average rows per expert, changes no bit.  With few rows per
// expert the 64 x 64 tile gives every expert's weights many streaming
// workgroups; above 32 rows per expert, the 128 x 256 tile holds an
// expert's rows in one m-tile (each weight slab is read once) and re-reads
// the gathered rows for 12 n-tiles of the up projection instead of 24.
// Measured on MI355X, 128 experts 4096 -> 1536 -> 4096, top 8, us (64 x 64 /
// 128 x 256): T = 64: 546 / 575; 512: 676 / 661; 1024: 910 / 734; 2048:
// 1366 / 888.  128 x 128, 256 x 128, 256 x 256, 64 x 256, 96 x 128, 192 x 128,
// 192 x 256, 128 x 192 and 96 x 192 tiles, and different tiles for the up and
// down GEMMs, were within 5 % of the better one or slower.  Both read the
// weights with non-temporal loads: an expert's rows mostly fit one m-tile, so
// each weight strip is read by one workgroup (T = 8 / 64 / 512 on 64 x 64: 243
// / 550 / 666 -> 215 / 493 / 623 us; T = 1024 / 2048 on 128 x 256: 717 / 861
// -> 716 / 843 us).
using MoeSmallCfg = GemmNt<GemmLibraryCfg>::type;
using MoeLargeCfg = GemmNt<GemmWideCfg>::type;
constexpr int64_t kMoeLargeRowsPerExpert = 32;

// Workspace carve-up, shared by the host-side size query and the launcher.
struct MoeWs {
  size_t counts, offsets, tiles, pos, src, h, o, total;
};
inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
MoeWs moe_ws_layout(int64_t T, int64_t top_k, int64_t E, int64_t H, int64_t F) {
  MoeWs w;
  const int64_t P = T * top_k;
  size_t at = 0;
  w.counts = at;  at = align256(at + sizeof(int32_t) * E);
  w.offsets = at; at = align256(at + sizeof(int32_t) * (E + 1));
  w.tiles = at;   at = align256(at + sizeof(int32_t) * (E + 1));
  w.pos = at;     at = align256(at + sizeof(int32_t) * P);
  w.src = at;     at = align256(at + sizeof(int32_t) * P);
  w.h = at;       at = align256(at + sizeof(uint16_t) * P * F);
  w.o = at;       at = align256(at + sizeof(float) * P * H);
  w.total = at;
  return w;
}

// Sum of an int over the workgroup (kRouteThreads threads), same value to all.
__device__ __forceinline__ int block_sum_int(int v, int* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kRouteThreads / 64; ++w) t += red[w];
  return t;
}

// Pairs per thread per pass of the count and place kernels: each thread has
// this many coalesced id loads in flight at once instead of one.
constexpr int kPairsPerThread = 16;

__global__ __launch_bounds__(kRouteThreads) void moe_count_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                                   int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ pos) {
  __shared__ int red[kRouteThreads / 64];
  const int e = blockIdx.x;
  int c = 0;
  for (int base = 0; base < P; base += kRouteThreads * kPairsPerThread) {
    int id[kPairsPerThread];
#pragma unroll
    for (int j = 0; j < kPairsPerThread; ++j) {
      const int p = base + j * kRouteThreads + (int)threadIdx.x;
      id[j] = p < P ? ids[p] : 0;
    }
#pragma unroll
    for (int j = 0; j < kPairsPerThread; ++j) {
      const int p = base + j * kRouteThreads + (int)threadIdx.x;
      c += (p < P && id[j] == e) ? 1 : 0;
      // Pairs whose expert id is out of range belong to no expert; workgroup
      // 0 marks them so the combine skips them.
      if (e == 0 && p < P && (id[j] < 0 || id[j] >= E)) pos[p] = -1;
    }
  }
  c = block_sum_int(c, red);
  if (threadIdx.x == 0) counts[e] = c;
}

__global__ __launch_bounds__(kRouteThreads) void moe_place_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                                   int top_k, int tile_rows,
                                                                   const int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ tiles,
                                                                   int32_t* __restrict__ pos,
                                                                   int32_t* __restrict__ src) {
  __shared__ int red[kRouteThreads / 64];
  __shared__ int wave_tot[2][kPairsPerThread][kRouteThreads / 64];
  const int e = blockIdx.x;
  // First row and first tile of expert e: sums over the experts before it.
  int off = 0, til = 0;
  for (int j = threadIdx.x; j < e; j += kRouteThreads) {
    const int c = counts[j];
    off += c;
    til += (c + tile_rows - 1) / tile_rows;
  }
  off = block_sum_int(off, red);
  til = block_sum_int(til, red);
  if (threadIdx.x == 0) {
    offsets[e] = off;
    tiles[e] = til;
    if (e == E - 1) {
      offsets[E] = off + counts[e];
      tiles[E] = til + (counts[e] + tile_rows - 1) / tile_rows;
    }
  }
  // Stable placement of expert e's pairs in pair order.  A pass covers
  // kPairsPerThread slices of kRouteThreads consecutive pairs; within a slice
  // a pair's rank is the hits of the waves before it plus the hits of the
  // lanes before it (ballot), and slices follow each other in pair order.
  // The per-wave hit counts are double-buffered, so one barrier per pass
  // suffices: a pass writes the buffer the previous pass did not read.
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t lanes_before = (1ull << lane) - 1ull;
  int run = off;
  int buf = 0;
  for (int base = 0; base < P; base += kRouteThreads * kPairsPerThread, buf ^= 1) {
    int id[kPairsPerThread];
#pragma unroll
    for (int j = 0; j < kPairsPerThread; ++j) {
      const int p = base + j * kRouteThreads + (int)threadIdx.x;
      id[j] = p < P ? ids[p] : -1;
    }
    uint64_t bal[kPairsPerThread];
#pragma unroll
    for (int j = 0; j < kPairsPerThread; ++j) {
      bal[j] = __ballot(id[j] == e);
      if (lane == 0) wave_tot[buf][j][wave] = __popcll(bal[j]);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPairsPerThread; ++j) {
      int wbase = 0, total = 0;
#pragma unroll
      for (int w = 0; w < kRouteThreads / 64; ++w) {
        const int t = wave_tot[buf][j][w];
        wbase += w < wave ? t : 0;
        total += t;
      }
      if (id[j] == e) {
        const int p = base + j * kRouteThreads + (int)threadIdx.x;
        const int r = run + wbase + __popcll(bal[j] & lanes_before);
        pos[p] = r;
        src[r] = p / top_k;
      }
      run += total;
    }
  }
}

// Placement of the grouped GEMMs' tiles: workgroup i runs on XCD i % 8, and
// each XCD takes a contiguous range of (m-tile, n-tile) pairs in m-tile-major
// order, so the n-tiles of one m-tile - which share its gathered A rows - run
// together on one XCD and find those rows in its L2.  Only placement changes.
__device__ __forceinline__ void moe_map_tile(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int q = total >> 3, r = total & 7;
  const int x = pid & 7, j = pid >> 3;
  const int lin = (x < r) ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
  tm = lin / tiles_n;
  tn = lin - tm * tiles_n;
}

// Grouped expert GEMM over the expert-major rows.  kUp: A rows are gathered
// from x (row src[r]), W = W_up[e] ([F, H]), output bf16(SiLU(.)) into h.
// Otherwise A = h rows (contiguous), W = W_down[e] ([H, F]), fp32 output into o.
template <class Cfg, bool kUp, bool kMajor = true>
__global__ __launch_bounds__(Cfg::kThreads, Cfg::OCC) void moe_gemm_kernel(
    const uint16_t* __restrict__ A, int64_t lda, int a_rows, const uint16_t* __restrict__ Wb,
    int64_t w_expert_stride, const int32_t* __restrict__ offsets, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ src, int E, int N, int K, int tiles_n, void* __restrict__ out) {

  // The grid is sized for the worst case; only the first tiles[E] * tiles_n
  // workgroups have a tile.  Placing the real tiles (not the padded grid)
  // XCD-aware spreads them over all XCDs however few they are.
  const int tiles_m = tiles[E];
  if ((int)blockIdx.x >= tiles_m * tiles_n) return;
  int mt, tn;
  if constexpr (kMajor)
    moe_map_tile(blockIdx.x, tiles_m, tiles_n, mt, tn);
  else
    gemm_map_tile(blockIdx.x, tiles_m, tiles_n, mt, tn);
  // Expert owning global m-tile mt: the last e with tiles[e] <= mt.
  int lo = 0, hi = E;  // tiles[lo] <= mt < tiles[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tiles[mid] <= mt) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int row0 = offsets[e] + (mt - tiles[e]) * Cfg::TM;   // first expert-major row of the tile
  const int rows_a = min(Cfg::TM, offsets[e + 1] - row0);
  const int n0 = tn * Cfg::TN;
  const int rows_w = min(Cfg::TN, N - n0);
  const uint16_t* W = Wb + (int64_t)e * w_expert_stride;

  GemmOperands<Cfg> op;
  op.rsw = gemm_rsrc(W + (int64_t)n0 * K, (uint32_t)(((int64_t)(rows_w - 1) * K + K) * 2));
#pragma unroll
  for (int i = 0; i < Cfg::LW; ++i) {
    const int r = gemm_slot_row<Cfg>(i);
    op.wofs[i] = r < rows_w ? (uint32_t)((int64_t)r * K * 2) + gemm_slot_chunk_bytes<Cfg>(i) : kBufOOB;
  }
  if constexpr (kUp) {
    // One resource over all of x; each slot's row comes from the gather list.
    op.rsa = gemm_rsrc(A, (uint32_t)(((int64_t)(a_rows - 1) * lda + K) * 2));
#pragma unroll
    for (int i = 0; i < Cfg::LA; ++i) {
      const int r = gemm_slot_row<Cfg>(i);
      op.aofs[i] = r < rows_a ? (uint32_t)((int64_t)src[row0 + r] * lda * 2) + gemm_slot_chunk_bytes<Cfg>(i)
                              : kBufOOB;
    }
  } else {
    op.rsa = gemm_rsrc(A + (int64_t)row0 * lda, (uint32_t)(((int64_t)(rows_a - 1) * lda + K) * 2));
#pragma unroll
    for (int i = 0; i < Cfg::LA; ++i) {
      const int r = gemm_slot_row<Cfg>(i);
      op.aofs[i] = r < rows_a ? (uint32_t)((int64_t)r * lda * 2) + gemm_slot_chunk_bytes<Cfg>(i) : kBufOOB;
    }
  }

  f32x4_t acc[Cfg::NB][Cfg::MB];
  gemm_zero<Cfg>(acc);
  gemm_mainloop<Cfg>(op, K, rows_a, acc);

  gemm_epilogue<Cfg>(acc, rows_a, n0, N, [&](int m, int n, f32x4_t v, int cnt) {
    if constexpr (kUp) {
      // SiLU(v) = v / (1 + 2^(-v log2 e)), in fp32, then one rounding to bf16.
      f32x4_t a;
#pragma unroll
      for (int q = 0; q < 4; ++q) a[q] = v[q] / (1.0f + exp2_hw(-v[q] * kLog2e));
      gemm_store4_bf16(static_cast<uint16_t*>(out) + (int64_t)(row0 + m) * N + n, a, cnt, (N & 3) == 0);
    } else {
      gemm_store4_f32(static_cast<float*>(out) + (int64_t)(row0 + m) * N + n, v, cnt, (N & 3) == 0);
    }
  });
}

__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ o, const int32_t* __restrict__ pos,
                                                          const float* __restrict__ wts, int top_k, int H,
                                                          uint16_t* __restrict__ y, int64_t ldy) {
  const int t = blockIdx.x;
  for (int j = threadIdx.x * 4; j < H; j += 256 * 4) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < top_k; ++s) {
      const int r = pos[(int64_t)t * top_k + s];
      if (r < 0) continue;
      const float w = wts[(int64_t)t * top_k + s];
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(o + (int64_t)r * H + j);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = acc[q] + w * v[q];
    }
    gemm_store4_bf16(y + (int64_t)t * ldy + j, acc, 4, true);
  }
}

// Top-k of one token's router logits.  Lane l holds experts l, l + 64, ...
// (PER of them).  Round s: every lane offers its best remaining expert, a
// butterfly over the wavefront keeps the better of each pair - the larger key,
// or the lower index on equal keys: a total order, so the winner is the same
// whatever the pairing - and the winner's lane marks it taken.  Then lane 0
// forms the weights: e_s = 2^((l_s - l_0) log2 e), their fp32 sum in slot
// order, w_s = e_s / sum.
template <int PER>
__global__ __launch_bounds__(64) void moe_topk_kernel(const float* __restrict__ logits, int E, int top_k,
                                                      int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int t = blockIdx.x, lane = threadIdx.x;
  const float* lr = logits + (int64_t)t * E;
  float key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    const float v = e < E ? lr[e] : -INFINITY;
    key[i] = (e < E && !__builtin_isnan(v)) ? v : -INFINITY;
  }
  uint32_t taken = 0;
  __shared__ int chosen[64];
  for (int s = 0; s < top_k; ++s) {
    float bv = -INFINITY;
    int bi_ = INT_MAX;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      const bool ok = e < E && !((taken >> i) & 1u);
      if (ok && (key[i] > bv || (key[i] == bv && e < bi_))) {
        bv = key[i];
        bi_ = e;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi_, o, kWave);
      if (ov > bv || (ov == bv && oi < bi_)) {
        bv = ov;
        bi_ = oi;
      }
    }
    if (bi_ != INT_MAX && (bi_ & 63) == lane) taken |= 1u << (bi_ >> 6);
    if (lane == 0) chosen[s] = bi_;
  }
  if (lane == 0) {
    const float l0 = lr[chosen[0]];
    float sum = 0.0f;
    for (int s = 0; s < top_k; ++s) sum = sum + exp2_hw((lr[chosen[s]] - l0) * kLog2e);
    for (int s = 0; s < top_k; ++s) {
      ids[(int64_t)t * top_k + s] = chosen[s];
      wts[(int64_t)t * top_k + s] = exp2_hw((lr[chosen[s]] - l0) * kLog2e) / sum;
    }
  }
}

}  // namespace

size_t moe_workspace_bytes(int64_t T, int64_t top_k, int64_t E, int64_t H, int64_t F) {
  return moe_ws_layout(T, top_k, E, H, F).total;
}

bool moe_supported(int64_t T, int64_t ldx, int64_t top_k, int64_t E, int64_t H, int64_t F) {
  const int64_t P = T * top_k;
  if (P > (1 << 24)) return false;
  // Buffer resources: all of x (gathered rows), a tile's slice of a weight, of
  // h and of o must each span fewer than 2^31 bytes (checked for the larger
  // of the two configurations' tiles).
  const int64_t lim = (int64_t)1 << 31;
  if (((T - 1) * ldx + H) * 2 >= lim) return false;
  constexpr int64_t tn = std::max(MoeSmallCfg::TN, MoeLargeCfg::TN), tm = std::max(MoeSmallCfg::TM, MoeLargeCfg::TM);
  if (((tn - 1) * H + H) * 2 >= lim || ((tn - 1) * F + F) * 2 >= lim) return false;
  if (((tm - 1) * F + F) * 2 >= lim) return false;
  const int64_t tiles_m = (P + (MoeSmallCfg::TM - 1) * E) / MoeSmallCfg::TM + 1;
  const int64_t tiles_n = (std::max(H, F) + MoeSmallCfg::TN - 1) / MoeSmallCfg::TN;
  return tiles_m * tiles_n <= 0x7fffffff;
}

// The MoE layer with the grouped GEMMs on configuration Cfg (kMajor: tiles
// placed by moe_map_tile, else by the dense GEMM's gemm_map_tile).
template <class Cfg, bool kMajor = true>
hipError_t launch_moe_ffn_cfg(const void* x, int64_t ldx, const int32_t* expert_ids, const float* expert_weights,
                              int T, int top_k, int E, const void* w_up, const void* w_down, int H, int F, void* y,
                              int64_t ldy, void* workspace, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const MoeWs L = moe_ws_layout(T, top_k, E, H, F);
  char* ws = static_cast<char*>(workspace);
  auto* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  auto* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  auto* tiles = reinterpret_cast<int32_t*>(ws + L.tiles);
  auto* pos = reinterpret_cast<int32_t*>(ws + L.pos);
  auto* src = reinterpret_cast<int32_t*>(ws + L.src);
  auto* h = reinterpret_cast<uint16_t*>(ws + L.h);
  auto* o = reinterpret_cast<float*>(ws + L.o);
  const int P = T * top_k;

  hipLaunchKernelGGL(moe_count_kernel, dim3(E), dim3(kRouteThreads), 0, stream, expert_ids, P, E, counts, pos);
  hipLaunchKernelGGL(moe_place_kernel, dim3(E), dim3(kRouteThreads), 0, stream, expert_ids, P, E, top_k, Cfg::TM,
                     counts, offsets, tiles, pos, src);
  // Grid: an upper bound on the m-tiles of all experts together (each expert
  // adds at most one partial tile); workgroups past the real count exit.
  const int tiles_m_bound = (P + (Cfg::TM - 1) * E) / Cfg::TM + 1;
  const int tn_up = (F + Cfg::TN - 1) / Cfg::TN, tn_down = (H + Cfg::TN - 1) / Cfg::TN;
  hipLaunchKernelGGL((moe_gemm_kernel<Cfg, true, kMajor>), dim3(tiles_m_bound * tn_up), dim3(Cfg::kThreads), 0, stream,
                     static_cast<const uint16_t*>(x), ldx, T, static_cast<const uint16_t*>(w_up), (int64_t)F * H,
                     offsets, tiles, src, E, F, H, tn_up, static_cast<void*>(h));
  hipLaunchKernelGGL((moe_gemm_kernel<Cfg, false, kMajor>), dim3(tiles_m_bound * tn_down), dim3(Cfg::kThreads), 0, stream,
                     static_cast<const uint16_t*>(h), (int64_t)F, P, static_cast<const uint16_t*>(w_down),
                     (int64_t)H * F, offsets, tiles, src, E, H, F, tn_down, static_cast<void*>(o));
  hipLaunchKernelGGL(moe_combine_kernel, dim3(T), dim3(256), 0, stream, o, pos, expert_weights, top_k, H,
                     static_cast<uint16_t*>(y), ldy);
  return hipGetLastError();
}

hipError_t launch_moe_ffn(const void* x, int64_t ldx, const int32_t* expert_ids, const float* expert_weights,
                          int T, int top_k, int E, const void* w_up, const void* w_down, int H, int F, void* y,
                          int64_t ldy, void* workspace, hipStream_t stream) {
  const int64_t P = (int64_t)T * top_k;
  if (P > kMoeLargeRowsPerExpert * (int64_t)E)
    return launch_moe_ffn_cfg<MoeLargeCfg>(x, ldx, expert_ids, expert_weights, T, top_k, E, w_up, w_down, H, F, y,
                                           ldy, workspace, stream);
  return launch_moe_ffn_cfg<MoeSmallCfg>(x, ldx, expert_ids, expert_weights, T, top_k, E, w_up, w_down, H, F, y,
                                         ldy, workspace, stream);
}

}  // namespace bi

namespace bi {

hipError_t launch_moe_route(const void* x, int64_t ldx, const void* w_gate, int T, int H, int E, int top_k,
                            float* logits, int32_t* expert_ids, float* expert_weights, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipError_t e = launch_gemm(x, ldx, w_gate, H, logits, E, true, T, E, H, stream);
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<unsigned>(T)), block(64);
  if (E <= 64)
    hipLaunchKernelGGL(moe_topk_kernel<1>, grid, block, 0, stream, logits, E, top_k, expert_ids, expert_weights);
  else if (E <= 256)
    hipLaunchKernelGGL(moe_topk_kernel<4>, grid, block, 0, stream, logits, E, top_k, expert_ids, expert_weights);
  else
    hipLaunchKernelGGL(moe_topk_kernel<16>, grid, block, 0, stream, logits, E, top_k, expert_ids, expert_weights);
  return hipGetLastError();
}

}  // namespace bi
