// Chunked-prefill attention over the paged KV cache ("Thinking Machines Lab -
// Defeating Nondeterminism in LLM Inference", section "3. Batch-Invariant
// Attention", figs. "FlashAttention2 Strategy" and "FlashAttention with KV
// Cache"; "Como superar a não determinismo na inferência de LLMs", Attention:
// one K/V layout for cached and new tokens).
//
// Parallel over query rows (FlashAttention-2 style): a workgroup owns 128
// (token, q head) rows of one sequence and one kv head - four wavefronts of two
// 16-row column blocks.  The chunk's own keys/values are already in the paged
// cache, so cached and new tokens are read through one path.  The workgroup
// walks the 256-key chunks in ascending order, 32 keys at a time, and every
// wavefront runs the same chunk step as decode on each 32-key sub-block (causal
// mask: a query at position p sees keys 0..p).  After a chunk each column folds
// it with the same merge step as decode, so row p is bitwise what decode
// returns at seq_len p + 1.
//
// K and V sub-blocks travel from HBM straight into LDS (buffer loads that
// write LDS, no register staging): K one sub-block ahead of the scores that
// use it, V one ahead of the values.  Each 1 KB load lies inside one 16-token
// tile, so one scalar buffer resource per load covers it; a tile whose page is
// missing, past the block table or wholly past the last visible key gets an
// empty resource and lands as zeros.  Keys of a valid page past the last
// visible key are masked where they are used (scores of such keys are never
// visible; their V entries are zeroed in LDS on the one sub-block that
// straddles the limit).  Tile indices come from a per-chunk table built one
// chunk ahead.
#include "attn_chunk.hpp"
#include "kv_layout.hpp"
#include "launch.hpp"

namespace bi {
namespace {

constexpr int kWaves = 4;
constexpr int kNB = 2;                              // 16-row column blocks per wavefront
constexpr int kRowsPerWave = 16 * kNB;
constexpr int kRowsPerBlock = kRowsPerWave * kWaves;
constexpr int kThreads = kWaves * 64;

template <int V>
struct StageIdx {
  static constexpr int value = V;
};

// One 16-byte-per-lane load of [base, base + bytes) at byte offset voff into LDS
// at lds + 16 * lane (lds is the same for the whole wavefront).  Offsets at or
// past `bytes` (all of them when bytes = 0) write zeros and read nothing.
__device__ __forceinline__ void lds_dma16(const uint16_t* base, uint32_t bytes, uint32_t voff, uint16_t* lds) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, (int)bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// Waits until at most N of this wavefront's vector-memory operations are
// outstanding, then joins the workgroup barrier.  Written out because the
// barrier of __syncthreads also waits for every LDS-writing load in flight,
// which would drain the ring.  The memory clobber keeps the compiler from
// moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_vmem_then_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// D: head dim.  REGFOLD: column blocks whose fold state stays in registers
// (the rest wait in LDS).  OCC: workgroups per CU the register budget aims at.
template <int D, int REGFOLD, int OCC>
__global__ __launch_bounds__(kThreads, OCC) void attn_prefill_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const int32_t* __restrict__ q_start,
    const int32_t* __restrict__ ctx_lens, int num_seqs, int tiles, int max_q_len, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int num_pages, const int32_t* __restrict__ block_table, int max_pages,
    int Hq, int Hkv, int log2_ps, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    const int32_t* __restrict__ order) {
  constexpr int TE = kTile * D;                          // elements per tile
  constexpr int kPieces = 2 * TE * 2 / 1024;             // 1 KB loads per sub-block of K (two tiles); V the same
  constexpr int IPW = kPieces / kWaves;                  // ... per wavefront
  static_assert(IPW >= 1 && kPieces % kWaves == 0, "staging split");
  // Tiles sit TS elements apart: the 128-byte pad puts tile 1 on the other
  // half of the LDS banks, so a K fragment read (lanes 0-7 in tile 0, lanes
  // 8-15 in tile 1) is free of bank conflicts.
  constexpr int TS = TE + 64;
  // Two K stages and two V stages, each its own array, so the compiler can
  // tell the stages' loads apart and wait only for the stage an LDS read needs.
  __shared__ __attribute__((aligned(16))) uint16_t sk0[2 * TS];
  __shared__ __attribute__((aligned(16))) uint16_t sk1[2 * TS];
  __shared__ __attribute__((aligned(16))) uint16_t sv0[2 * TS];
  __shared__ __attribute__((aligned(16))) uint16_t sv1[2 * TS];
  static_assert(REGFOLD >= 0 && REGFOLD <= kNB, "fold split");

  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  // Work placement (arithmetic does not depend on it).  Items (sequence,
  // tile) are ranked longest first: sequences by descending last key (ties by
  // index), then a sequence's tiles from the last, whose rows see the most
  // keys.  The first half of the workgroups takes the items in that order and
  // the second half in reverse, so the two workgroups that share a CU tend to
  // pair a long item with a short one (measured on MI355X: 3-7% faster than
  // longest-first throughout).  The kv head is the fastest index: workgroups go
  // to the 8 XCDs round-robin, so every workgroup of one kv head shares one L2.
  const int items = tiles * num_seqs, half = (items + 1) / 2;
  const int qi = blockIdx.x / Hkv, h = blockIdx.x % Hkv;
  const int item = qi < half ? qi : items - 1 - (qi - half);
  const int rank = item / tiles, tile = tiles - 1 - item % tiles;
  auto seq_key = [&](int j) { return ctx_lens[j] + min(q_start[j + 1] - q_start[j], max_q_len); };
  int sq = 0;
  // The sequence of this rank: from the order table when prefill_order_kernel
  // wrote one, else ranked here (every sequence against every other).
  if (order != nullptr) sq = order[rank];
  for (int base = 0; order == nullptr && base < num_seqs; base += kWave) {
    const int i = base + lane;
    const int ki = i < num_seqs ? seq_key(i) : 0;
    int r = 0;   // sequences ordered before sequence i
    for (int j = 0; j < num_seqs; ++j) {
      const int kj = seq_key(j);
      r += (kj > ki || (kj == ki && j < i)) ? 1 : 0;
    }
    const uint64_t hit = __ballot(i < num_seqs && r == rank);
    if (hit != 0) {
      sq = base + (int)__builtin_ctzll(hit);
      break;
    }
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = Hq / Hkv;
  const int qs = q_start[sq];
  const int nq = min(q_start[sq + 1] - qs, max_q_len);
  const int ctx = ctx_lens[sq];
  const int rows = nq * G;
  const int row0 = tile * kRowsPerBlock;
  // Uniform over the workgroup, before any barrier.
  if (nq <= 0 || ctx < 0 || row0 >= rows) return;
  const int lim = ctx + (min(row0 + kRowsPerBlock, rows) - 1) / G + 1;   // keys >= lim: no row sees them
  const int wrow0 = row0 + wave * kRowsPerWave;

  int pos[kNB];
  bool row_ok[kNB];
  u32x4_t qf[kNB][D / 32];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int rho = wrow0 + 16 * nb + n;
    row_ok[nb] = rho < rows;
    const int tok = rho / G, hh = rho - tok * G;
    pos[nb] = ctx + tok;
    const uint16_t* qp = q + (int64_t)(qs + tok) * ldq + (h * G + hh) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qf[nb][ks] = row_ok[nb] ? *reinterpret_cast<const u32x4_t*>(qp + 32 * ks) : zero4();
  }

  const int ps = 1 << log2_ps;
  const int32_t* bt = block_table + (int64_t)sq * max_pages;
  // Tile table of a chunk: lane l holds, for tile l % 16 of the chunk (keys
  // 16 (l % 16) .. + 15), the tile's index in the cache counted in tiles of
  // TE elements, or -1 when no row of the workgroup sees it, it lies past the
  // block table, or its page id is outside the pool.  Built one chunk ahead
  // from block-table entries read two chunks ahead (from a clamped index), so
  // neither the read nor the table ever waits.
  const int tiles_per_page = (Hkv << log2_ps) / kTile;
  const int head_tiles = h * (ps / kTile);
  auto raw_entry = [&](int c) {
    return bt[min(c * (kChunk >> log2_ps) + (((lane & 15) * kTile) >> log2_ps), max_pages - 1)];
  };
  auto make_tab = [&](int c, int raw) {
    const int t0 = c * kChunk + (lane & 15) * kTile;
    const bool ok = t0 < lim && (t0 >> log2_ps) < max_pages && raw >= 0 && raw < num_pages;
    return ok ? raw * tiles_per_page + head_tiles + ((t0 & (ps - 1)) >> 4) : -1;
  };

  // The 1 KB pieces of sub-block u (keys 32 u .. 32 u + 31) that this
  // wavefront loads, K or V, into a stage; `tab` is the table of u's chunk.
  // A wavefront's pieces lie in one tile.  Issued for every u, also past the
  // end (as zeros), so every wavefront always has the same number of loads in
  // flight.
  static_assert((TE * 2 / 1024) % IPW == 0, "a wavefront's pieces share a tile");
  auto issue = [&](const uint16_t* cache, int u, int tab, uint16_t* dst) {
    const int pc0 = wave * IPW;                          // first piece of the wavefront
    const int tt = pc0 * 1024 / (TE * 2);                // its tile (0 or 1)
    const int inb0 = pc0 * 1024 - tt * (TE * 2);         // byte offset inside the tile
    const int tile = __builtin_amdgcn_readlane(tab, 2 * (u & (kSubs - 1)) + tt);
    const uint16_t* base = cache + (tile >= 0 ? (int64_t)tile * TE : 0);
#pragma unroll
    for (int j = 0; j < IPW; ++j)
      lds_dma16(base, tile >= 0 ? TE * 2 : 0, inb0 + 1024 * j + lane * 16, dst + tt * TS + (inb0 + 1024 * j) / 2);
  };

  // Running state of the fold over chunks (per column block).  The
  // accumulators are touched once per chunk; those of column blocks >= REGFOLD
  // wait in LDS (each lane owns its slots; no other lane reads them) and leave
  // the registers to the chunk step.
  constexpr int kLdsFold = kNB - REGFOLD;
  __shared__ __attribute__((aligned(16))) f32x4_t s_orun[kWaves][kLdsFold > 0 ? kLdsFold : 1][D / 16][64];
  f32x4_t o_reg[REGFOLD > 0 ? REGFOLD : 1][D / 16];
  auto fold_get = [&](int nb, int dt) -> f32x4_t {
    return nb < REGFOLD ? o_reg[nb < REGFOLD ? nb : 0][dt] : s_orun[wave][nb >= REGFOLD ? nb - REGFOLD : 0][dt][lane];
  };
  auto fold_put = [&](int nb, int dt, f32x4_t v) {
    if (nb < REGFOLD)
      o_reg[nb < REGFOLD ? nb : 0][dt] = v;
    else
      s_orun[wave][nb >= REGFOLD ? nb - REGFOLD : 0][dt][lane] = v;
  };
  float m_run[kNB], l_run[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) fold_put(nb, dt, f32x4_t{0.f, 0.f, 0.f, 0.f});
  }

  // Software pipeline over sub-blocks u = 0 .. nsub - 1 (chunk c = u / 8,
  // sub-block s = u % 8).  Step u waits for K(u + 1) and V(u), refills the
  // stages that step u - 1 finished with (K(u + 2), V(u + 1)), and then, in one
  // branch-free stretch, issues the score MFMAs of u + 1 while it computes the
  // probabilities of u and their value MFMAs.  Sub-block u + 1's mask and
  // reference update close the step.  Per column this is the chunk step's
  // order exactly; only independent work of two sub-blocks is interleaved.
  // Every wavefront runs every sub-block below the workgroup's limit; one its
  // columns cannot see is an exact identity (all p = 0, alpha = 1).
  const int nsub = (lim + kSub - 1) / kSub;
  int c = 0;
  int cur_tab = make_tab(0, raw_entry(0)), next_tab = make_tab(1, raw_entry(1)), raw_ahead = raw_entry(2);
  ChunkAcc<D, kNB> ca;
  chunk_init(ca);
  int nvalid[kNB];
  auto set_nvalid = [&]() {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
      nvalid[nb] = row_ok[nb] ? max(0, min(kChunk, pos[nb] + 1 - c * kChunk)) : 0;
  };
  set_nvalid();
  // Same operand addressing as decode, inside the LDS copy of the two tiles.
  const int kofs = (n >> 3) * TS + g * 128 + (n & 7) * 8;
  const int vofs = (g >> 1) * TS + (g & 1) * 128 + n * 8;
  auto scores = [&](const uint16_t* sK, f32x4_t (&S)[kNB][2]) {
    u32x4_t kf[2][D / 32];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        kf[b][ks] = *reinterpret_cast<const u32x4_t*>(&sK[kofs + 4 * ks * 128 + 8 * b * 8]);
    sub_scores<D, kNB>(kf, qf, S);
  };

  f32x4_t S[kNB][2];
  issue(kc, 0, cur_tab, sk0);
  issue(vc, 0, cur_tab, sv0);
  issue(kc, 1, cur_tab, sk1);
  wait_vmem_then_barrier<0>();
  scores(sk0, S);
  sub_mask<kNB>(S, nvalid, 0);
  sub_reference<D, kNB>(ca, S, scale_log2);

  // P = u % 2: step u reads K stage (u + 1) % 2 and V stage u % 2 and refills
  // K stage u % 2 and V stage (u + 1) % 2.
  auto step = [&](int u, auto par) {
    constexpr int P = decltype(par)::value;
    uint16_t* const sk_rd = P == 0 ? sk1 : sk0;
    uint16_t* const sk_wr = P == 0 ? sk0 : sk1;
    uint16_t* const sv_rd = P == 0 ? sv0 : sv1;
    uint16_t* const sv_wr = P == 0 ? sv1 : sv0;
    wait_vmem_then_barrier<0>();
    issue(kc, u + 2, ((u + 2) >> 3) == c ? cur_tab : next_tab, sk_wr);
    issue(vc, u + 1, ((u + 1) >> 3) == c ? cur_tab : next_tab, sv_wr);
    // The sub-block holding the limit (the workgroup's last): V entries of keys
    // >= lim may hold stale data (even NaN); they are zeroed in LDS, once, so
    // that their p = 0 adds exact zeros.  Keeping this test at the top keeps
    // the rest of the step one branch-free stretch.
    if ((u + 1) * kSub > lim) {
      const int kv0 = lim - u * kSub;   // first stale key of the sub-block, 1 .. 31
      for (int i = tid; i < (kSub - kv0) * D; i += kThreads) {
        const int k = kv0 + i / D, d = i % D;
        sv_rd[(k >> 4) * TS + v_tile_off(k & 15, d)] = 0;
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }

    f32x4_t Sn[kNB][2];
    scores(sk_rd, Sn);
    u32x4_t pb[kNB];
    sub_probs<D, kNB>(ca, S, scale_log2, pb);
    u32x4_t vf[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) vf[dt] = *reinterpret_cast<const u32x4_t*>(&sv_rd[vofs + dt * 256]);
    sub_values<D, kNB>(ca, vf, pb);

    // Chunk end: fold the chunk into the running state, start the next one.
    if (((u + 1) & (kSubs - 1)) == 0 || u + 1 == nsub) {
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const float lc = chunk_l(ca, nb);   // cross-lane: every lane takes part
        if (nvalid[nb] > 0) {
          const MergeCoef k = merge_coef(m_run[nb], ca.m[nb]);
          l_run[nb] = merge_val(l_run[nb], lc, k);
          if (__all(k.alpha == 1.0f)) {
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
              f32x4_t o = fold_get(nb, dt);
#pragma unroll
              for (int i = 0; i < 4; ++i) o[i] = merge_val_unit(o[i], ca.o[nb][dt][i], k);
              fold_put(nb, dt, o);
            }
          } else {
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
              f32x4_t o = fold_get(nb, dt);
#pragma unroll
              for (int i = 0; i < 4; ++i) o[i] = merge_val(o[i], ca.o[nb][dt][i], k);
              fold_put(nb, dt, o);
            }
          }
          m_run[nb] = k.m;
        }
      }
      ++c;
      cur_tab = next_tab;
      next_tab = make_tab(c + 1, raw_ahead);
      raw_ahead = raw_entry(c + 2);
      chunk_init(ca);
      set_nvalid();
    }
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int b = 0; b < 2; ++b) S[nb][b] = Sn[nb][b];
    if (u + 1 < nsub) {
      sub_mask<kNB>(S, nvalid, (u + 1) & (kSubs - 1));
      sub_reference<D, kNB>(ca, S, scale_log2);
    }
  };
  for (int u = 0; u < nsub; u += 2) {
    step(u, StageIdx<0>{});
    if (u + 1 >= nsub) break;
    step(u + 1, StageIdx<1>{});
  }
  // The last loads (zeros past the end) must land before the workgroup's LDS
  // is released.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    if (!row_ok[nb]) continue;
    const int rho = wrow0 + 16 * nb + n;
    const int tok = rho / G, hh = rho - tok * G;
    uint16_t* op = out + ((int64_t)(qs + tok) * Hq + h * G + hh) * D + 4 * g;
    const float inv = finalize_inv(l_run[nb]);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const f32x4_t a = fold_get(nb, dt);
      *reinterpret_cast<u32x2_t*>(op + 16 * dt) =
          u32x2_t{pack_bf16x2(finalize_val(a[0], inv), finalize_val(a[1], inv)),
                  pack_bf16x2(finalize_val(a[2], inv), finalize_val(a[3], inv))};
    }
    if (lse != nullptr && g == 0) lse[(int64_t)(qs + tok) * Hq + h * G + hh] = finalize_lse(m_run[nb], l_run[nb]);
  }
}

// The library's configuration: two workgroups per CU (registers <= 256 and
// LDS <= 80 KB each) and column block 0's fold state in registers.
constexpr int kLibRegFold = 1, kLibOcc = 2;

// The prefill kernel's placement order: order[rank] = the sequence of that
// rank, sequences ranked by descending last key, ties by index (the ranking
// the prefill kernel otherwise computes in every workgroup).  One thread per
// sequence counts the sequences ordered before it, reading the keys 256 at a
// time from LDS; the ranks form a permutation, so every entry is written once.
constexpr int kOrderThreads = 256;
constexpr int kOrderMinSeqs = 16;
__global__ __launch_bounds__(kOrderThreads) void prefill_order_kernel(const int32_t* __restrict__ q_start,
                                                                      const int32_t* __restrict__ ctx_lens,
                                                                      int num_seqs, int max_q_len,
                                                                      int32_t* __restrict__ order) {
  __shared__ int keys[kOrderThreads];
  auto seq_key = [&](int j) { return ctx_lens[j] + min(q_start[j + 1] - q_start[j], max_q_len); };
  const int i = blockIdx.x * kOrderThreads + threadIdx.x;
  const int ki = i < num_seqs ? seq_key(i) : 0;
  int r = 0;
  for (int base = 0; base < num_seqs; base += kOrderThreads) {
    __syncthreads();
    const int j = base + threadIdx.x;
    keys[threadIdx.x] = j < num_seqs ? seq_key(j) : 0;
    __syncthreads();
    const int n = min(kOrderThreads, num_seqs - base);
    for (int u = 0; u < n; ++u) {
      const int kj = keys[u];
      r += (kj > ki || (kj == ki && base + u < i)) ? 1 : 0;
    }
  }
  if (i < num_seqs) order[r] = i;
}

template <int D>
hipError_t launch(const void* q, int64_t ld_q, const int32_t* q_start, const int32_t* ctx_lens, int num_seqs,
                  int max_q_len, const AttnGeom& g, void* out, float* lse, int32_t* order, hipStream_t stream) {
  const int G = g.num_q_heads / g.num_kv_heads;
  const int tiles = (max_q_len * G + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t blocks = (int64_t)tiles * g.num_kv_heads * num_seqs;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  // Tile indices into the cache are 32-bit (a 288 GB pool holds < 2^27 tiles).
  if ((int64_t)g.num_pages * (((int64_t)g.num_kv_heads << g.log2_page) / kTile) > 0x7fffffff)
    return hipErrorInvalidValue;
  if (order != nullptr) {
    hipLaunchKernelGGL(prefill_order_kernel, dim3((num_seqs + kOrderThreads - 1) / kOrderThreads),
                       dim3(kOrderThreads), 0, stream, q_start, ctx_lens, num_seqs, max_q_len, order);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((attn_prefill_kernel<D, kLibRegFold, kLibOcc>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(q), ld_q, q_start, ctx_lens, num_seqs, tiles, max_q_len,
                     static_cast<const uint16_t*>(g.k_cache), static_cast<const uint16_t*>(g.v_cache),
                     g.num_pages, g.block_table, g.max_pages_per_seq, g.num_q_heads, g.num_kv_heads,
                     g.log2_page, g.scale_log2, static_cast<uint16_t*>(out), lse, order);
  return hipGetLastError();
}

}  // namespace

size_t attn_prefill_workspace_bytes(int64_t num_seqs) {
  return ((size_t)num_seqs * sizeof(int32_t) + 255) & ~(size_t)255;
}

hipError_t launch_attn_prefill(const void* q, int64_t ld_q, const int32_t* q_start, const int32_t* ctx_lens,
                               int num_seqs, int max_q_len, const AttnGeom& g, void* out, float* lse,
                               void* workspace, hipStream_t stream) {
  if (num_seqs == 0 || max_q_len == 0) return hipSuccess;
  // With few sequences every workgroup ranks them in a few steps itself, and
  // the order kernel's launch would cost more than it saves.
  auto* order = num_seqs > kOrderMinSeqs ? static_cast<int32_t*>(workspace) : nullptr;
  return g.head_dim == 64 ? launch<64>(q, ld_q, q_start, ctx_lens, num_seqs, max_q_len, g, out, lse, order, stream)
                          : launch<128>(q, ld_q, q_start, ctx_lens, num_seqs, max_q_len, g, out, lse, order, stream);
}

}  // namespace bi
