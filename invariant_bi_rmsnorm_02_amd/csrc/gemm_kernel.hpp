// Batch-invariant bf16 GEMM kernel template, C = A W^T ("Thinking Machines Lab -
// Defeating Nondeterminism in LLM Inference", section "2. Batch-Invariant
// Matrix Multiplication", figs. "Data-Parallel Matrix Multiplication" and
// "Split-K Matmul").
//
// The library instantiates twenty-one configurations, nine of them also with
// non-temporal weight loads (gemm_with_cfg_mn picks one from the shape; every
// one gives every element the same bits).  Whatever
// the configuration, the arithmetic of an output element is the same: one fp32
// accumulator, v_mfma_f32_16x16x32_bf16 steps over k = 0, 32, 64, ... in
// ascending order, no split of K.  Nothing here depends on
// M except which rows are loaded and which 16-row MFMA blocks are skipped
// because all their rows are past M.
//
// Data movement.  K advances in BK-wide stages held in an S-stage LDS ring.
// Stages travel from memory straight into LDS (buffer loads that write LDS,
// 16 bytes per lane), S - 1 stages ahead of the one being multiplied; no
// register holds them in flight and no instruction copies them.  Every load
// is a raw buffer load whose resource covers only this workgroup's rows: a row
// past N or M, or a k past K, gets an out-of-range offset and the hardware
// writes zeros without touching memory.  Each wavefront's loads for a stage
// fill 1 KB runs of the XOR-swizzled tile: lane l writes 16 bytes at l * 16 of
// its run, so the lane fetches whichever 16-byte chunk of its row the swizzle
// puts there.  The wavefronts read their MFMA operands from the tile.  The tile
// is computed as C^T = W A^T so each lane stores 4 consecutive n.
#pragma once

#include <utility>

#include "bi_common.hpp"

namespace bi {

template <int TN_, int TM_, int WGN_, int WGM_, int S_, int BK_ = 64, int OCC_ = 2, int CPW_ = 0>
struct GemmCfg {
  static constexpr int TN = TN_, TM = TM_;          // workgroup tile: W rows x A rows
  static constexpr int CPW = CPW_;                  // cache-policy bits of the W loads (0 or kCpolNt)
  static constexpr int WGN = WGN_, WGM = WGM_;      // wavefront grid
  static constexpr int S = S_;                      // LDS ring depth (stages)
  static constexpr int BK = BK_;                    // K per stage (32, 64 or 128)
  static constexpr int OCC = OCC_;                  // workgroups per CU the registers and LDS aim at
  static constexpr int kThreads = 64 * WGN * WGM;
  static constexpr int WTN = TN / WGN, WTM = TM / WGM;
  static constexpr int NB = WTN / 16, MB = WTM / 16;
  static constexpr int kChunks = BK / 8;                    // 16-byte chunks per tile row
  static constexpr int LW = TN * kChunks / kThreads;        // W loads per thread per stage
  static constexpr int LA = TM * kChunks / kThreads;        // A loads per thread per stage
  static_assert(LW >= 1 && LA >= 1 && TN * kChunks % kThreads == 0 && TM * kChunks % kThreads == 0, "split");
  static_assert(NB >= 1 && MB >= 1, "wave tile");
  static_assert(S >= 2 && S <= 8, "ring depth");
  static_assert((S - 2) * (LW + LA) < 64, "loads in flight per wave fit the wait counter");
  static_assert(S * (TN + TM) * BK * 2 * OCC <= 160 * 1024, "LDS per CU");
  static_assert(BK == 32 || BK == 64 || BK == 128, "stage depth");
};

// Host-side limit: every offset of a workgroup's buffer resource must fit in
// 31 bits (rows - 1 full row strides plus one row of K elements, in bytes).
template <class Cfg>
inline bool gemm_offsets_fit(int64_t lda, int64_t ldw, int64_t k) {
  const int64_t lim = (int64_t)1 << 31;
  return ((int64_t)(Cfg::TN - 1) * ldw + k) * 2 < lim && ((int64_t)(Cfg::TM - 1) * lda + k) * 2 < lim;
}

// The XOR swizzle of tile row r's 16-byte chunks (KC chunks per row).  An
// MFMA operand read has 16 consecutive rows read one chunk index each; the
// swizzle spreads every 8 of them over distinct 16-byte bank groups.  Rows of
// 128 or 256 bytes (KC = 8, 16) take r mod KC; rows of 64 bytes (KC = 4) put
// four rows in one 256-byte bank period, so the XOR takes the row's group of
// four instead.
template <int KC>
__device__ __forceinline__ int gemm_swz(int r) {
  if constexpr (KC == 4)
    return (r >> 2) & 3;
  else
    return r & (KC - 1);
}

// LDS element offset of 16-byte chunk c of tile row r (KC chunks per row).
template <int KC>
__device__ __forceinline__ int gemm_lds_off(int r, int c) { return r * KC * 8 + ((c ^ gemm_swz<KC>(r)) << 3); }

__device__ __forceinline__ void gemm_map_tile(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  // Workgroup i runs on XCD i % 8.  Give each XCD a contiguous range of tiles
  // (so tiles sharing A or W rows share an L2), then walk that range in groups
  // of 8 m-tiles.  Only placement changes; the arithmetic does not.
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

constexpr uint32_t kBufOOB = 0x80000000u;  // beyond every resource's range: the load returns zeros
// The non-temporal bit of a buffer load's cache-policy operand: the line is not
// kept for reuse.  Only where it is placed in the caches changes, never a value.
constexpr int kCpolNt = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const void* base, uint32_t bytes) {
  // Raw (stride 0) resource; the last word is the gfx9 data-format default.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// The operands of one workgroup tile: a buffer resource over the W rows and
// one over the A rows it reads, and for every load slot of this thread the
// byte offset (within its resource) of the slot's 16-byte chunk in stage 0, or
// kBufOOB when the slot's row does not exist (slots: gemm_slot_row and
// gemm_slot_chunk).
template <class Cfg>
struct GemmOperands {
  __amdgpu_buffer_rsrc_t rsw, rsa;
  uint32_t wofs[Cfg::LW], aofs[Cfg::LA];
};

// Load slot i of a thread writes tile row (tid + i * threads) / chunks at
// swizzled position (tid + i * threads) % chunks; it fetches the row's chunk
// that gemm_lds_off puts there.
template <class Cfg>
__device__ __forceinline__ int gemm_slot_row(int i) {
  return (threadIdx.x + i * Cfg::kThreads) / Cfg::kChunks;
}
template <class Cfg>
__device__ __forceinline__ int gemm_slot_chunk(int i) {
  constexpr int KC = Cfg::kChunks;
  return ((threadIdx.x + i * Cfg::kThreads) % KC) ^ gemm_swz<KC>(gemm_slot_row<Cfg>(i));
}
// Byte offset of load slot i's chunk within its row.
template <class Cfg>
__device__ __forceinline__ uint32_t gemm_slot_chunk_bytes(int i) {
  return (uint32_t)(gemm_slot_chunk<Cfg>(i) * 16);
}

template <int V>
struct GemmInt {
  static constexpr int value = V;
};

// Calls f(GemmInt<I>{}) for each I of the sequence, in order.
template <int... I, class F>
__device__ __forceinline__ void gemm_for_each(std::integer_sequence<int, I...>, F&& f) {
  (f(GemmInt<I>{}), ...);
}

// Calls f(GemmInt<live>{}) for 1 <= live <= L; nothing for live <= 0.
template <int L, class F>
__device__ __forceinline__ void gemm_dispatch_live(int live, F&& f) {
  if constexpr (L >= 1) {
    if (live >= L)
      f(GemmInt<L>{});
    else
      gemm_dispatch_live<L - 1>(live, f);
  }
}

// 16-row blocks of this wave's m-range (tile rows wm*WTM ..) that hold at least
// one of the tile's `rows` real rows.
template <class Cfg>
__device__ __forceinline__ int gemm_live_blocks(int rows) {
  const int wm = (threadIdx.x >> 6) / Cfg::WGN;
  return min(Cfg::MB, max(0, (rows - wm * Cfg::WTM + 15) >> 4));
}

// One 16-byte-per-lane load of the resource at byte offset voff into LDS at
// lds + 16 * lane (lds is the same for the whole wavefront).
// CP: the load's cache-policy bits (0, or kCpolNt for data read once).
template <int CP = 0>
__device__ __forceinline__ void gemm_lds_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint16_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, CP);
}

// Waits until at most N of this wavefront's vector-memory operations are
// outstanding, then joins the workgroup barrier.  Written out because the
// barrier of __syncthreads also waits for every LDS-writing load in flight,
// which would drain the ring; the memory clobber keeps the compiler from
// moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void gemm_wait_then_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// The ring: one W and one A array per stage, each its own __shared__ object,
// so the compiler can tell the stages' loads apart and waits for exactly the
// stage an LDS read needs.  Stages past S are one element (never used).
template <class Cfg>
struct GemmRing {
  template <int I>
  __device__ __forceinline__ static uint16_t* w() {
    __shared__ __attribute__((aligned(16))) uint16_t buf[I < Cfg::S ? Cfg::TN * Cfg::BK : 8];
    return buf;
  }
  template <int I>
  __device__ __forceinline__ static uint16_t* a() {
    __shared__ __attribute__((aligned(16))) uint16_t buf[I < Cfg::S ? Cfg::TM * Cfg::BK : 8];
    return buf;
  }
};

// The main loop for a tile whose first LAL A load slots hold real rows (slot i
// of every thread covers tile rows i * R .. i * R + R - 1, R = threads / chunks
// per row).  The other A slots are not loaded: their rows are past M, so the
// MFMA blocks that would read them are skipped, and their loads would only
// occupy the texture units.  Which slots are live is uniform over the
// workgroup and fixed for the whole loop, so the loop stays branch-free.
//
// Stage kt is loaded into ring slot kt % S by the iteration kt - S + 1 (the
// prologue for the first S - 1 stages).  Iteration kt waits for its own
// loads of stage kt (the S - 2 later stages stay in flight), joins the
// barrier, which also guarantees that every wavefront has finished reading
// the slot read by iteration kt - 1, refills that slot with stage kt + S - 1,
// and multiplies stage kt.  Stages past the end of K load zeros at no memory
// cost, so every wavefront always has the same loads in flight.
template <class Cfg, int LAL>
__device__ __forceinline__ void gemm_mainloop_live(const GemmOperands<Cfg>& op, int K, int live_mb,
                                                   f32x4_t (&acc)[Cfg::NB][Cfg::MB]) {
  constexpr int BK = Cfg::BK, NT = Cfg::kThreads, S = Cfg::S;
  constexpr int NB = Cfg::NB, MB = Cfg::MB, LW = Cfg::LW, TN = Cfg::TN, TM = Cfg::TM;
  constexpr int KC = Cfg::kChunks;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % Cfg::WGN, wm = wave / Cfg::WGN;
  const int l16 = lane & 15, g = lane >> 4;
  const int KT = (K + BK - 1) / BK;
  using Ring = GemmRing<Cfg>;

  // Loads of stage kt: slot i of this wavefront fills the 1 KB run that starts
  // at thread (wave * 64 + i * NT)'s position of the tile.
  auto issue = [&](int kt, uint16_t* dw, uint16_t* da) {
#pragma unroll
    for (int i = 0; i < LW; ++i) {
      const bool ok = op.wofs[i] != kBufOOB && kt * BK + gemm_slot_chunk<Cfg>(i) * 8 < K;
      gemm_lds_load<Cfg::CPW>(op.rsw, ok ? op.wofs[i] + (uint32_t)(kt * BK * 2) : kBufOOB, dw + (wave * 64 + i * NT) * 8);
    }
#pragma unroll
    for (int i = 0; i < LAL; ++i) {
      const bool ok = op.aofs[i] != kBufOOB && kt * BK + gemm_slot_chunk<Cfg>(i) * 8 < K;
      gemm_lds_load(op.rsa, ok ? op.aofs[i] + (uint32_t)(kt * BK * 2) : kBufOOB, da + (wave * 64 + i * NT) * 8);
    }
  };
  // One stage of MFMAs for the first L m-blocks (L known at compile time, so
  // the stage has no branch: every fragment read is issued before the MFMAs
  // that use it).  Each accumulator takes its MFMA steps in ascending k.
  auto compute_live = [&](const uint16_t* sW, const uint16_t* sA, auto live_c) {
    constexpr int L = decltype(live_c)::value;
    u32x4_t af[BK / 32][NB], bf[BK / 32][L];
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int c = ks * 4 + g;
#pragma unroll
      for (int i = 0; i < NB; ++i)
        af[ks][i] = *reinterpret_cast<const u32x4_t*>(&sW[gemm_lds_off<KC>(wn * Cfg::WTN + i * 16 + l16, c)]);
#pragma unroll
      for (int j = 0; j < L; ++j)
        bf[ks][j] = *reinterpret_cast<const u32x4_t*>(&sA[gemm_lds_off<KC>(wm * Cfg::WTM + j * 16 + l16, c)]);
    }
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks)
#pragma unroll
      for (int j = 0; j < L; ++j)
#pragma unroll
        for (int i = 0; i < NB; ++i) acc[i][j] = mfma_16x16x32(af[ks][i], bf[ks][j], acc[i][j]);
  };
  auto compute = [&](const uint16_t* sW, const uint16_t* sA) {
    gemm_dispatch_live<MB>(live_mb, [&](auto live_c) { compute_live(sW, sA, live_c); });
  };
  constexpr int kAfter = (S - 2) * (LW + LAL);   // loads issued after stage kt's when it is awaited
  static_assert(TN * BK > 0 && TM * BK > 0, "tile");

  gemm_for_each(std::make_integer_sequence<int, S - 1>{}, [&](auto pidx) {
    constexpr int p = decltype(pidx)::value;
    issue(p, Ring::template w<p>(), Ring::template a<p>());
  });
  const int KTS = (KT + S - 1) / S * S;
  for (int kb = 0; kb < KTS; kb += S) {
    auto step = [&](auto uidx) {
      constexpr int u = decltype(uidx)::value;
      constexpr int r = (u + S - 1) % S;
      const int kt = kb + u;
      gemm_wait_then_barrier<kAfter>();
      issue(kt + S - 1, Ring::template w<r>(), Ring::template a<r>());
      if (kt < KT) compute(Ring::template w<u>(), Ring::template a<u>());
    };
    gemm_for_each(std::make_integer_sequence<int, S>{}, step);
  }
  // The ring's last loads (zeros past the end) must land before the
  // workgroup's LDS is released or reused by the caller.
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

// Accumulates the workgroup's tile over the whole of K into acc (which the
// caller zeroes): for every output element one fp32 chain of MFMA steps over
// k = 0, 32, 64, ... in ascending order.  rows_a = real A rows of the tile;
// only the MFMA blocks and A load slots that hold one of them are issued (the
// others would only compute or load padding), which changes no real output.
template <class Cfg>
__device__ __forceinline__ void gemm_mainloop(const GemmOperands<Cfg>& op, int K, int rows_a,
                                              f32x4_t (&acc)[Cfg::NB][Cfg::MB]) {
  constexpr int R = Cfg::kThreads / Cfg::kChunks;   // tile rows per load slot
  static_assert(Cfg::kThreads % Cfg::kChunks == 0, "slot rows");
  const int live_mb = gemm_live_blocks<Cfg>(rows_a);
  const int la_live = min(Cfg::LA, (rows_a + R - 1) / R);
  gemm_dispatch_live<Cfg::LA>(la_live, [&](auto lal) {
    gemm_mainloop_live<Cfg, decltype(lal)::value>(op, K, live_mb, acc);
  });
}

// Hands every finished output group to st(m, n, v, cnt): tile-local row m
// (< rows), global column n, v = C[m][n .. n+3], cnt = columns of v below N.
template <class Cfg, class Store>
__device__ __forceinline__ void gemm_epilogue(const f32x4_t (&acc)[Cfg::NB][Cfg::MB], int rows, int n0, int N,
                                              Store&& st) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave % Cfg::WGN, wm = wave / Cfg::WGN;
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < Cfg::MB; ++j) {
    const int m = wm * Cfg::WTM + j * 16 + l16;
    if (m >= rows) continue;
#pragma unroll
    for (int i = 0; i < Cfg::NB; ++i) {
      const int n = n0 + wn * Cfg::WTN + i * 16 + 4 * g;
      if (n >= N) continue;
      st(m, n, acc[i][j], min(4, N - n));
    }
  }
}

template <class Cfg>
__device__ __forceinline__ void gemm_zero(f32x4_t (&acc)[Cfg::NB][Cfg::MB]) {
#pragma unroll
  for (int i = 0; i < Cfg::NB; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::MB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// Stores v (4 consecutive columns, cnt of them real) at cp as bf16 or fp32.
__device__ __forceinline__ void gemm_store4_bf16(uint16_t* cp, f32x4_t v, int cnt, bool vec) {
  if (vec && cnt == 4) {
    *reinterpret_cast<u32x2_t*>(cp) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  } else {
    for (int e = 0; e < cnt; ++e) cp[e] = static_cast<uint16_t>(f32_to_bf16(v[e]));
  }
}
__device__ __forceinline__ void gemm_store4_f32(float* cp, f32x4_t v, int cnt, bool vec) {
  if (vec && cnt == 4) {
    *reinterpret_cast<f32x4_t*>(cp) = v;
  } else {
    for (int e = 0; e < cnt; ++e) cp[e] = v[e];
  }
}

// One workgroup's output tile of C = A W^T: picks the tile from blockIdx.x,
// accumulates it over the whole of K and hands every finished output group to
// st(r, n, v, cnt): global row r of C, global column n, v = C[r][n .. n+3] in
// fp32 (before any rounding), cnt = columns of v below N.  bi_gemm's kernel
// stores the groups; the fused kernels (gemm_fused.hip) transform them first.
template <class Cfg, class Store>
__device__ __forceinline__ void gemm_tile(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t ldw, int M,
                                          int N, int K, int tiles_m, int tiles_n, Store&& st) {
  int tile_m, tile_n;
  gemm_map_tile(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
  const int m0 = tile_m * Cfg::TM, n0 = tile_n * Cfg::TN;
  const int rows_w = min(Cfg::TN, N - n0), rows_a = min(Cfg::TM, M - m0);

  // Resources cover exactly this tile's rows (the host checked the offsets fit).
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

  // Epilogue: lane holds C[m][n .. n+3].
  gemm_epilogue<Cfg>(acc, rows_a, n0, N, [&](int m, int n, f32x4_t v, int cnt) { st(m0 + m, n, v, cnt); });
}

template <class Cfg, bool kF32Out>
__global__ __launch_bounds__(Cfg::kThreads, Cfg::OCC) void gemm_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ W, int64_t ldw,
    void* __restrict__ C, int64_t ldc, int M, int N, int K, int tiles_m, int tiles_n, int vec_store) {
  gemm_tile<Cfg>(A, lda, W, ldw, M, N, K, tiles_m, tiles_n, [&](int r, int n, f32x4_t v, int cnt) {
    if constexpr (kF32Out)
      gemm_store4_f32(static_cast<float*>(C) + (int64_t)r * ldc + n, v, cnt, vec_store);
    else
      gemm_store4_bf16(static_cast<uint16_t*>(C) + (int64_t)r * ldc + n, v, cnt, vec_store);
  });
}

// The configurations (n x m output tile; wavefront grid; LDS ring depth x K
// per stage; workgroups per CU the registers and LDS aim at).  Each stage of
// the ring holds (TN + TM) x BK bf16 values.
//
// 64 x 64, 2 x 2 wavefronts of 32 x 32, 5 x 64, two per CU (80 KB each).  Also
// the expert GEMMs of bi_moe_ffn and the narrow-weight fused lm_head.
using GemmLibraryCfg = GemmCfg<64, 64, 2, 2, 5, 64, 2>;
// 128 x 256, 2 x 4 wavefronts of 64 x 64, 3 x 64, one per CU (144 KB).  With
// at least one 128-row strip per CU a vocabulary-sized weight fills the chip
// even at one m-tile, so it serves such weights (N >= kGemmWideMinN) below
// kGemmBigMinMWide rows.
using GemmWideCfg = GemmCfg<128, 256, 2, 4, 3, 64, 1>;
constexpr int64_t kGemmWideMinN = 256 * GemmWideCfg::TN;
// 256 x 256, 2 x 4 wavefronts of 128 x 64, 2 x 64, one per CU (128 KB).  Each
// wavefront issues 64 MFMAs per stage against 24 fragment reads and one
// barrier; deeper rings of 32-wide stages and the 4 x 2 wavefront layout were
// 2-15 % slower on MI355X.  Vocabulary-sized weights take it from
// kGemmBigMinMWide rows (it is 16 % slower than 128 x 256 at M = 64 there).
using GemmBigCfg = GemmCfg<256, 256, 2, 4, 2, 64, 1>;
constexpr int64_t kGemmBigMinMWide = 512;
// Large- and medium-M tiles: 256 x 192 (2 x 4 of 128 x 48, 2 x 64, 112 KB),
// 192 x 256 (2 x 4 of 96 x 64, 2 x 64, 112 KB), 256 x 160 (2 x 2 of 128 x 80,
// 3 x 64, 160 KB), 256 x 128 (2 x 4 of 128 x 32, 3 x 64, 144 KB), 192 x 128,
// 128 x 192 and 128 x 128 (2 x 2, 4 x 64, 160 / 160 / 128 KB), 96 x 192
// (2 x 2 of 48 x 96, 4 x 64, 144 KB) and 96 x 128 (2 x 2 of 48 x 64, 5 x 64,
// 140 KB), all one per CU.
using Gemm256x192Cfg = GemmCfg<256, 192, 2, 4, 2, 64, 1>;
using Gemm192x256Cfg = GemmCfg<192, 256, 2, 4, 2, 64, 1>;
using Gemm256x160Cfg = GemmCfg<256, 160, 2, 2, 3, 64, 1>;
using Gemm256x128Cfg = GemmCfg<256, 128, 2, 4, 3, 64, 1>;
using Gemm192x128Cfg = GemmCfg<192, 128, 2, 2, 4, 64, 1>;
using Gemm128x192Cfg = GemmCfg<128, 192, 2, 2, 4, 64, 1>;
using GemmSquareCfg = GemmCfg<128, 128, 2, 2, 4, 64, 1>;
using Gemm96x192Cfg = GemmCfg<96, 192, 2, 2, 4, 64, 1>;
using Gemm96x128Cfg = GemmCfg<96, 128, 2, 2, 5, 64, 1>;
// Decode-batch tiles, narrow in n so that many workgroups stream the weight
// (one CU pulls only a few tens of GB/s from HBM): 64 x 128 (2 x 2 of 32 x 64,
// 3 x 64) and 96 x 64 (2 x 2 of 48 x 32, 4 x 64), two per CU; 64 x 64 with
// 4 x 128 (128 KB), one per CU; 32 x 64 (2 x 2 of 16 x 32) with 6 x 64, two per
// CU, or 4 x 128, one per CU; 32 x 32 (2 x 2 of 16 x 16, 8 x 128, 128 KB);
// 16 x 64 (1 x 4 of 16 x 16) with 4 x 128, two per CU, or 8 x 128, one per CU
// (the four 16-row blocks of A share each weight stage); and 32 x 16 (2 x 1 of
// 16 x 16, 6 x 128, two per CU), where each wavefront streams its own 16
// weight rows.
using GemmMidCfg = GemmCfg<64, 128, 2, 2, 3, 64, 2>;
using Gemm96x64Cfg = GemmCfg<96, 64, 2, 2, 4, 64, 2>;
using Gemm64x64K128Cfg = GemmCfg<64, 64, 2, 2, 4, 128, 1>;
using GemmThinCfg = GemmCfg<32, 64, 2, 2, 6, 64, 2>;
using Gemm32x64K128Cfg = GemmCfg<32, 64, 2, 2, 4, 128, 1>;
using Gemm32x32Cfg = GemmCfg<32, 32, 2, 2, 8, 128, 1>;
using GemmStripCfg = GemmCfg<16, 64, 1, 4, 4, 128, 2>;
using Gemm16x64K128Cfg = GemmCfg<16, 64, 1, 4, 8, 128, 1>;
using GemmSkinnyCfg = GemmCfg<32, 16, 2, 1, 6, 128, 2>;
// From kGemmThinMinN weight rows (a fused gate and up projection) at 1 to
// kGemmThinWideMaxM rows the 32 x 64 tile with two workgroups per CU is taken
// without estimate: on 4096 -> 24576 at M = 1 .. 32 it was 5-8 % faster than
// the estimate's pick (96 x 64) on MI355X.
constexpr int64_t kGemmThinMinN = 16384;
constexpr int64_t kGemmThinWideMaxM = 32;

// The same configuration with its weight loads non-temporal.
template <class C>
struct GemmNt;
template <int TN, int TM, int WGN, int WGM, int S, int BK, int OCC, int CPW>
struct GemmNt<GemmCfg<TN, TM, WGN, WGM, S, BK, OCC, CPW>> {
  using type = GemmCfg<TN, TM, WGN, WGM, S, BK, OCC, kCpolNt>;
};

// Tile rule of the vocabulary-sized weights (N >= kGemmWideMinN) and of the
// fused lm_head: the big tile from kGemmBigMinMWide rows on, else the wide
// one, with non-temporal weight loads while its single m-tile holds all of M
// (each weight strip is then read once).  The fused lm_head's per-row reduction records do not depend on the
// tile (lm_head.hip), so this choice changes no bit either.
template <class F>
inline auto gemm_with_cfg_wide(int64_t lda, int64_t ldw, int64_t m, int64_t k, F&& f) {
  if (m >= kGemmBigMinMWide && gemm_offsets_fit<GemmBigCfg>(lda, ldw, k)) return f(GemmBigCfg{});
  if (m <= GemmWideCfg::TM) return f(GemmNt<GemmWideCfg>::type{});
  return f(GemmWideCfg{});
}

// Calls f on configuration C, with its weight loads marked non-temporal when
// the grid has one m-tile of at most 64 rows: then every weight strip is read
// by one workgroup only, and keeping its lines in the caches only displaces
// other data.  Measured on MI355X with the weights streamed from HBM: 2-12 %
// faster at M <= 64 on every such tile (4096 -> 24576 at M = 1 on 32 x 64:
// 38.6 -> 35.5 us; down 12288 -> 4096 on 16 x 64: 21.6 -> 19.7 us), while with
// several m-tiles sharing a strip it was up to 11 % slower.
template <class C, class F>
inline auto gemm_with_stream_w(int64_t m, F&& f) {
  if constexpr (C::TM <= 64) {
    if (m <= C::TM) return f(typename GemmNt<C>::type{});
  }
  return f(C{});
}

// Compute units of the current device (a grid of T tiles puts ceil(T / CUs)
// workgroups on its busiest CU).  Only speed depends on it.
int gemm_device_cus();

// The estimated time of configuration C on an m x n x k product, in us.  The
// busiest CU runs L = ceil(tiles / CUs) workgroups.  One per CU at a time
// (OCC = 1): L rounds.  OCC = 2: L / 2 rounds with two workgroups sharing the
// CU, and when L is odd one more with the CU to itself, which is markedly
// faster per tile.  A round costs w us per MB of the tile's weight rows
// (TN x K bf16) + f us per MFLOP of its MFMA work (the tile's rows of A that
// exist, at most M) + c us; (w1, f1, c1) is the lone-workgroup round.  The
// coefficients were fitted (non-negative least squares, each time weighted by
// its inverse) to every configuration's times on MI355X with the weights
// streamed from HBM: the Qwen3-8B projections QKV 4096 -> 6144, O 4096 ->
// 4096, up 4096 -> 12288, fused gate/up 4096 -> 24576 and down 12288 -> 4096
// at M = 1 .. 4096 (155 shapes).  On those the rule's picks took 0.5 % more
// time in total than the fastest configuration of each shape.
struct GemmCost {
  double w, f, c;
  double w1 = 0.0, f1 = 0.0, c1 = 0.0;
};
template <class C>
inline double gemm_estimate_us(int64_t m, int64_t n, int64_t k, const GemmCost& q, int cus) {
  const int64_t tiles = ((m + C::TM - 1) / C::TM) * ((n + C::TN - 1) / C::TN);
  const int64_t per_cu = (tiles + cus - 1) / cus;
  const double rows = (double)(m < C::TM ? m : C::TM);
  const double wmb = 2.0 * C::TN * (double)k * 1e-6, mflop = 2.0 * rows * C::TN * (double)k * 1e-6;
  const double shared = q.w * wmb + q.f * mflop + q.c;
  if (C::OCC == 1) return (double)per_cu * shared;
  return (double)(per_cu / 2) * shared + (double)(per_cu % 2) * (q.w1 * wmb + q.f1 * mflop + q.c1);
}

// bi_gemm's configuration.  Every configuration computes every output element
// with the same fp32 chain of v_mfma_f32_16x16x32_bf16 steps over k = 0, 32,
// 64, ... and one rounding, so the tile decides speed, never bits: the choice
// may read M without making any row depend on the rest of the batch (the
// tests compare whole products bitwise across the tiles the rule picks).
//   N >= kGemmWideMinN:                                  gemm_with_cfg_wide
//   M <= kGemmThinWideMaxM and N >= kGemmThinMinN:       32 x 64, two per CU
//   otherwise: the candidate with the least gemm_estimate_us (first in the
//     list below on a tie).
// A candidate is passed over when its operand offsets would not fit its
// buffer resources, and one with 128-wide K stages when K is a multiple of 64
// but not of 128.  A tile's last stage runs all of its MFMA steps, those past
// K on zeros; a step on zeros leaves the accumulator as it is, except that it
// turns an exact -0 into +0.  With that exclusion either every candidate ends
// on at least one such step (K not a multiple of 64) or none does, so even the
// sign of an exact zero does not depend on the tile.  The caller checks the
// chosen tile; if none fits, the 32 x 16 tile is returned (it spans fewer rows
// than any other).  The chosen configuration runs through gemm_with_stream_w.
template <class F>
inline auto gemm_with_cfg_mn(int64_t lda, int64_t ldw, int64_t m, int64_t n, int64_t k, F&& f) {
  if (n >= kGemmWideMinN) return gemm_with_cfg_wide(lda, ldw, m, k, f);
  if (m <= kGemmThinWideMaxM && n >= kGemmThinMinN && gemm_offsets_fit<GemmThinCfg>(lda, ldw, k))
    return gemm_with_stream_w<GemmThinCfg>(m, f);
  const int cus = gemm_device_cus();
  const bool k_pads_128 = (k % 128) != 0 && (k % 64) == 0;
  int pick = -1;
  double best = 0.0;
  auto consider = [&](int id, auto cfg, GemmCost q) {
    using C = decltype(cfg);
    if (C::BK == 128 && k_pads_128) return;
    if (!gemm_offsets_fit<C>(lda, ldw, k)) return;
    const double t = gemm_estimate_us<C>(m, n, k, q, cus);
    if (pick < 0 || t < best) {
      best = t;
      pick = id;
    }
  };
  consider(0, GemmBigCfg{}, {28.789, 0.061, 9.436});
  consider(1, Gemm256x192Cfg{}, {30.123, 0.039, 7.480});
  consider(2, Gemm192x256Cfg{}, {32.462, 0.063, 9.529});
  consider(3, Gemm256x160Cfg{}, {17.765, 0.104, 9.087});
  consider(4, Gemm256x128Cfg{}, {17.457, 0.065, 9.572});
  consider(5, GemmWideCfg{}, {22.194, 0.113, 8.461});
  consider(6, Gemm192x128Cfg{}, {18.472, 0.097, 7.899});
  consider(7, Gemm128x192Cfg{}, {20.107, 0.141, 7.245});
  consider(8, Gemm96x192Cfg{}, {21.946, 0.157, 7.526});
  consider(9, GemmSquareCfg{}, {20.521, 0.112, 5.966});
  consider(10, Gemm96x128Cfg{}, {21.514, 0.133, 6.511});
  consider(11, GemmMidCfg{}, {77.378, 0.091, 0.808, 39.154, 0.070, 5.419});
  consider(12, Gemm96x64Cfg{}, {0.000, 0.657, 5.408, 22.353, 0.060, 5.723});
  consider(13, GemmLibraryCfg{}, {57.408, 0.000, 0.928, 23.489, 0.133, 4.674});
  consider(14, Gemm64x64K128Cfg{}, {24.700, 0.078, 3.553});
  consider(15, GemmThinCfg{}, {84.145, 0.000, 0.000, 34.108, 0.226, 3.949});
  consider(16, Gemm32x64K128Cfg{}, {36.872, 0.084, 2.112});
  consider(17, Gemm32x32Cfg{}, {29.535, 0.000, 2.520});
  consider(18, GemmStripCfg{}, {100.503, 0.353, 0.000, 56.774, 0.321, 2.920});
  consider(19, Gemm16x64K128Cfg{}, {47.860, 0.347, 1.434});
  consider(20, GemmSkinnyCfg{}, {35.889, 0.000, 3.331, 22.032, 0.461, 5.352});
  switch (pick) {
    case 0: return gemm_with_stream_w<GemmBigCfg>(m, f);
    case 1: return gemm_with_stream_w<Gemm256x192Cfg>(m, f);
    case 2: return gemm_with_stream_w<Gemm192x256Cfg>(m, f);
    case 3: return gemm_with_stream_w<Gemm256x160Cfg>(m, f);
    case 4: return gemm_with_stream_w<Gemm256x128Cfg>(m, f);
    case 5: return gemm_with_stream_w<GemmWideCfg>(m, f);
    case 6: return gemm_with_stream_w<Gemm192x128Cfg>(m, f);
    case 7: return gemm_with_stream_w<Gemm128x192Cfg>(m, f);
    case 8: return gemm_with_stream_w<Gemm96x192Cfg>(m, f);
    case 9: return gemm_with_stream_w<GemmSquareCfg>(m, f);
    case 10: return gemm_with_stream_w<Gemm96x128Cfg>(m, f);
    case 11: return gemm_with_stream_w<GemmMidCfg>(m, f);
    case 12: return gemm_with_stream_w<Gemm96x64Cfg>(m, f);
    case 13: return gemm_with_stream_w<GemmLibraryCfg>(m, f);
    case 14: return gemm_with_stream_w<Gemm64x64K128Cfg>(m, f);
    case 15: return gemm_with_stream_w<GemmThinCfg>(m, f);
    case 16: return gemm_with_stream_w<Gemm32x64K128Cfg>(m, f);
    case 17: return gemm_with_stream_w<Gemm32x32Cfg>(m, f);
    case 18: return gemm_with_stream_w<GemmStripCfg>(m, f);
    case 19: return gemm_with_stream_w<Gemm16x64K128Cfg>(m, f);
    default: return gemm_with_stream_w<GemmSkinnyCfg>(m, f);
  }
}

template <class Cfg>
hipError_t launch_gemm_cfg(const void* a, int64_t lda, const void* w, int64_t ldw, void* c, int64_t ldc,
                           bool c_f32, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  if (!gemm_offsets_fit<Cfg>(lda, ldw, k)) return hipErrorInvalidValue;
  const int tiles_m = static_cast<int>((m + Cfg::TM - 1) / Cfg::TM);
  const int tiles_n = static_cast<int>((n + Cfg::TN - 1) / Cfg::TN);
  const dim3 grid(static_cast<unsigned>(tiles_m * tiles_n)), block(Cfg::kThreads);
  auto* as = static_cast<const uint16_t*>(a);
  auto* ws = static_cast<const uint16_t*>(w);
  // Vector stores need every row start 16-byte (fp32) / 8-byte (bf16) aligned.
  const int vec = (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(c) & 15u) == 0);
  if (c_f32)
    hipLaunchKernelGGL((gemm_kernel<Cfg, true>), grid, block, 0, stream, as, lda, ws, ldw, c, ldc, (int)m, (int)n,
                       (int)k, tiles_m, tiles_n, vec);
  else
    hipLaunchKernelGGL((gemm_kernel<Cfg, false>), grid, block, 0, stream, as, lda, ws, ldw, c, ldc, (int)m, (int)n,
                       (int)k, tiles_m, tiles_n, vec);
  return hipGetLastError();
}

}  // namespace bi
