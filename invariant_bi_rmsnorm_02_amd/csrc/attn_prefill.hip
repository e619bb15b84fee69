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
// K/V sub-blocks travel from HBM straight into a four-stage LDS ring (buffer
// loads that write LDS, no register staging), three sub-blocks ahead of the
// one being computed.  Each 1 KB load lies inside one 16-token tile, so one
// scalar buffer resource per load covers it; a tile whose page is missing,
// past the block table or wholly past the last visible key gets an empty
// resource and lands as zeros.  Keys of a valid page past the last visible key
// are masked where they are used (scores of such keys are never visible; their
// V entries are zeroed on the one sub-block that straddles the limit).  Block-
// table entries are read one chunk ahead.
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

// D: head dim.  STAGES: LDS ring depth in sub-blocks (divides the 8 of a
// chunk, so a sub-block's stage is static).  REGFOLD: column blocks whose fold
// state stays in registers (the rest wait in LDS).  OCC: workgroups per CU the
// register budget aims at.
template <int D, int STAGES, int REGFOLD, int OCC>
__global__ __launch_bounds__(kThreads, OCC) void attn_prefill_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const int32_t* __restrict__ q_start,
    const int32_t* __restrict__ ctx_lens, int num_seqs, int tiles, int max_q_len, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int num_pages, const int32_t* __restrict__ block_table, int max_pages,
    int Hq, int Hkv, int log2_ps, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int TE = kTile * D;                          // elements per tile
  constexpr int kPieces = 2 * TE * 2 / 1024;             // 1 KB loads per sub-block (K or V: two tiles)
  constexpr int IPW = kPieces / kWaves;                  // ... per wavefront
  static_assert(IPW >= 1 && kPieces % kWaves == 0, "staging split");
  // Tiles sit TS elements apart in a stage: the 128-byte pad puts tile 1 on
  // the other half of the LDS banks, so a K fragment read (lanes 0-7 in tile
  // 0, lanes 8-15 in tile 1) is free of bank conflicts.
  constexpr int TS = TE + 64;
  // One array per stage (K tiles at 0 and TS, V tiles at 2 TS and 3 TS), so the compiler can tell the
  // stages' loads apart and wait only for the stage an LDS read needs.
  __shared__ __attribute__((aligned(16))) uint16_t st0[4 * TS];
  __shared__ __attribute__((aligned(16))) uint16_t st1[4 * TS];
  __shared__ __attribute__((aligned(16))) uint16_t st2[4 * TS];
  __shared__ __attribute__((aligned(16))) uint16_t st3[4 * TS];
  static_assert(STAGES == 2 || STAGES == 4, "one array per stage above");
  static_assert(REGFOLD >= 0 && REGFOLD <= kNB, "fold split");
  auto stage = [&](auto idx) -> uint16_t* {
    constexpr int i = decltype(idx)::value;
    if constexpr (i == 0) return st0;
    else if constexpr (i == 1) return st1;
    else if constexpr (i == 2) return st2;
    else return st3;
  };

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
  for (int base = 0; base < num_seqs; base += kWave) {
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
  const int wave_lim = wrow0 < rows ? ctx + (min(wrow0 + kRowsPerWave, rows) - 1) / G + 1 : 0;

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
  const int ppc = kChunk >> log2_ps;   // pages per chunk
  const int32_t* bt = block_table + (int64_t)sq * max_pages;
  const int64_t page_elems = (int64_t)(Hkv << log2_ps) * D;
  const int64_t head_off = (int64_t)h * ps * D;
  // Raw block-table entries of chunk c, one logical page per lane (lane l:
  // page c * ppc + l % ppc), read from a clamped index; validated where used,
  // so loading the next chunk's entries early never waits.
  auto raw_pages = [&](int c) { return bt[min(c * ppc + (lane % ppc), max_pages - 1)]; };

  // Loads of sub-block u (keys 32 u .. 32 u + 31) into a stage: this
  // wavefront's IPW 1 KB pieces of the K tiles and of the V tiles.  `pages`
  // holds the raw entries of the sub-block's chunk.  Issued for every u, also
  // past the end (as zeros), so every wavefront always has the same number of
  // loads in flight.
  auto issue = [&](int u, int pages, uint16_t* dst) {
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int pc = wave * IPW + j;                     // piece of the sub-block
      const int tt = pc * 1024 / (TE * 2);               // its tile (0 or 1)
      const int inb = pc * 1024 - tt * (TE * 2);         // byte offset inside the tile
      const int t0 = u * kSub + kTile * tt;              // the tile's first key
      const int lp = t0 >> log2_ps;
      const int raw = __builtin_amdgcn_readlane(pages, (t0 & (kChunk - 1)) >> log2_ps);
      const bool ok = t0 < lim && lp < max_pages && raw >= 0 && raw < num_pages;
      const int64_t tb = ok ? raw * page_elems + head_off + (int64_t)((t0 & (ps - 1)) >> 4) * TE : 0;
      const uint32_t bytes = ok ? TE * 2 : 0;
      lds_dma16(kc + tb, bytes, inb + lane * 16, dst + tt * TS + inb / 2);
      lds_dma16(vc + tb, bytes, inb + lane * 16, dst + (2 + tt) * TS + inb / 2);
    }
  };
  // Loads issued after sub-block u's when the wavefront waits for u.
  constexpr int kAfter = (STAGES - 2) * 2 * IPW;

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

  const int nch = (lim + kChunk - 1) / kChunk;
  const int last_subs = (lim - (nch - 1) * kChunk + kSub - 1) / kSub;

  ChunkAcc<D, kNB> ca;
  int nvalid[kNB];
  int cur_pages = raw_pages(0), next_pages = raw_pages(1);
  static_assert(STAGES - 1 <= kSubs, "prologue stays in chunk 0");
  issue(0, cur_pages, stage(StageIdx<0>{}));
  if constexpr (STAGES == 4) {
    issue(1, cur_pages, stage(StageIdx<1>{}));
    issue(2, cur_pages, stage(StageIdx<2>{}));
  }
  // Outer loop over chunks, the 8 sub-blocks of a chunk written out so that
  // stages are static: sub-block u = 8 c + s sits in stage s % 4.
  for (int c = 0; c < nch; ++c) {
    const int after_pages = raw_pages(c + 2);
    chunk_init(ca);
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
      nvalid[nb] = row_ok[nb] ? max(0, min(kChunk, pos[nb] + 1 - c * kChunk)) : 0;
    const int subs = c == nch - 1 ? last_subs : kSubs;
    // One 32-key sub-block: wait for its stage, refill the stage that the
    // previous step read with sub-block u + 3, run the chunk step.
    auto step = [&](auto sidx, auto cur_stage, auto refill_stage) {
      constexpr int s = decltype(sidx)::value;
      const int u = c * kSubs + s;
      wait_vmem_then_barrier<kAfter>();
      issue(u + STAGES - 1, s + STAGES - 1 < kSubs ? cur_pages : next_pages, stage(refill_stage));
      const int sub0 = u * kSub;
      if (sub0 < wave_lim) {   // some column of this wave sees a key here
        const uint16_t* sK = stage(cur_stage);
        const uint16_t* sV = sK + 2 * TS;
        const int l16 = n;
        u32x4_t kf[2][D / 32], vf[D / 16];
        // Same operand addressing as decode, inside the LDS copy of the two tiles.
        const int kofs = (l16 >> 3) * TS + g * 128 + (l16 & 7) * 8;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks)
            kf[b][ks] = *reinterpret_cast<const u32x4_t*>(&sK[kofs + 4 * ks * 128 + 8 * b * 8]);
        SubProbs<kNB> sp;
        chunk_scores<D, kNB>(ca, kf, qf, nvalid, s, scale_log2, sp);
        // V is read once the K fragments are dead, which keeps the two apart
        // in the register file.
        const int vofs = (g >> 1) * TS + (g & 1) * 128 + l16 * 8;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) vf[dt] = *reinterpret_cast<const u32x4_t*>(&sV[vofs + dt * 256]);
        // The sub-block holding the limit: V of keys >= lim may be stale.
        if (sub0 + kSub > lim) {
          const KeepMask km = keep_mask(lim - (sub0 + 8 * g));
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) vf[dt] = apply_keep(vf[dt], km);
        }
        chunk_values<D, kNB>(ca, vf, sp);
      }
    };
    // Sub-block s reads stage s % STAGES and refills the stage read by s - 1.
    auto run = [&](auto sidx) {
      constexpr int s = decltype(sidx)::value;
      if (s < subs) step(sidx, StageIdx<s % STAGES>{}, StageIdx<(s + STAGES - 1) % STAGES>{});
    };
    static_assert(kSubs == 8, "sub-blocks below are written out");
    run(StageIdx<0>{});
    run(StageIdx<1>{});
    run(StageIdx<2>{});
    run(StageIdx<3>{});
    run(StageIdx<4>{});
    run(StageIdx<5>{});
    run(StageIdx<6>{});
    run(StageIdx<7>{});
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      if (nvalid[nb] > 0) {
        const MergeCoef k = merge_coef(m_run[nb], ca.m[nb]);
        l_run[nb] = merge_val(l_run[nb], ca.l[nb], k);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          f32x4_t o = fold_get(nb, dt);
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = merge_val(o[i], ca.o[nb][dt][i], k);
          fold_put(nb, dt, o);
        }
        m_run[nb] = k.m;
      }
    }
    cur_pages = next_pages;
    next_pages = after_pages;
  }
  // The ring's last loads (zeros past the end) must land before the
  // workgroup's LDS is released.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    if (!row_ok[nb]) continue;
    const int rho = wrow0 + 16 * nb + n;
    const int tok = rho / G, hh = rho - tok * G;
    uint16_t* op = out + ((int64_t)(qs + tok) * Hq + h * G + hh) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const f32x4_t a = fold_get(nb, dt);
      *reinterpret_cast<u32x2_t*>(op + 16 * dt) =
          u32x2_t{pack_bf16x2(finalize_val(a[0], l_run[nb]), finalize_val(a[1], l_run[nb])),
                  pack_bf16x2(finalize_val(a[2], l_run[nb]), finalize_val(a[3], l_run[nb]))};
    }
    if (lse != nullptr && g == 0) lse[(int64_t)(qs + tok) * Hq + h * G + hh] = finalize_lse(m_run[nb], l_run[nb]);
  }
}

// The library's configuration: two workgroups per CU (registers <= 256 and
// LDS <= 80 KB each), a two-stage ring and column block 0's fold state in
// registers.
constexpr int kLibStages = 2, kLibRegFold = 1, kLibOcc = 2;

template <int D>
hipError_t launch(const void* q, int64_t ld_q, const int32_t* q_start, const int32_t* ctx_lens, int num_seqs,
                  int max_q_len, const AttnGeom& g, void* out, float* lse, hipStream_t stream) {
  const int G = g.num_q_heads / g.num_kv_heads;
  const int tiles = (max_q_len * G + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t blocks = (int64_t)tiles * g.num_kv_heads * num_seqs;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_prefill_kernel<D, kLibStages, kLibRegFold, kLibOcc>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(q), ld_q, q_start, ctx_lens, num_seqs, tiles, max_q_len,
                     static_cast<const uint16_t*>(g.k_cache), static_cast<const uint16_t*>(g.v_cache),
                     g.num_pages, g.block_table, g.max_pages_per_seq, g.num_q_heads, g.num_kv_heads,
                     g.log2_page, g.scale_log2, static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_prefill(const void* q, int64_t ld_q, const int32_t* q_start, const int32_t* ctx_lens,
                               int num_seqs, int max_q_len, const AttnGeom& g, void* out, float* lse,
                               hipStream_t stream) {
  if (num_seqs == 0 || max_q_len == 0) return hipSuccess;
  return g.head_dim == 64 ? launch<64>(q, ld_q, q_start, ctx_lens, num_seqs, max_q_len, g, out, lse, stream)
                          : launch<128>(q, ld_q, q_start, ctx_lens, num_seqs, max_q_len, g, out, lse, stream);
}

}  // namespace bi
