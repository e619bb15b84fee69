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
// walks the 256-key chunks in ascending order, 32 keys at a time: each K/V
// sub-block is fetched from HBM four sub-blocks ahead into a register ring,
// staged once into LDS (double-buffered) and every wavefront runs the same
// chunk step as decode on it (causal mask: a query at position p sees keys
// 0..p).  Block-table entries are read one chunk ahead.
// After a chunk each column folds it with the same merge step as decode, so row
// p is bitwise what decode returns at seq_len p + 1.
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

// LDS holds one staged 32-key sub-block as its two 16-token tiles, in the same
// tiled order as the cache (kv_layout.hpp), so staging is a straight copy of
// contiguous 16-byte pieces and every fragment read is a run of contiguous
// 16-byte LDS words (128 bytes per 8 lanes for K, 256 bytes per 16 lanes for V).

template <int D>
__global__ __launch_bounds__(kThreads) void attn_prefill_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const int32_t* __restrict__ q_start,
    const int32_t* __restrict__ ctx_lens, int max_q_len, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int num_pages, const int32_t* __restrict__ block_table, int max_pages,
    int Hq, int Hkv, int log2_ps, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int TE = kTile * D;                 // elements per tile
  constexpr int NP = 2 * TE / 8 / kThreads;     // 16-byte pieces per thread per sub-block (K and V each)
  static_assert(NP >= 1 && (2 * TE / 8) % kThreads == 0, "staging split");
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][2 * TE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][2 * TE];

  const int tile = blockIdx.x, h = blockIdx.y, sq = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
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

  // Global -> register staging of sub-block u (chunk u / 8, sub-block u % 8),
  // P sub-blocks ahead of the LDS copy: piece pc covers elements 8 pc .. 8 pc
  // + 7 of the sub-block's two tiles.  `pages` holds the raw entries of the
  // sub-block's chunk.  Loads are unconditional (a page that may not be read
  // points at the pool start); the masks are applied when the ring slot is
  // copied into LDS.
  constexpr int P = 4;                 // divides the 8 sub-blocks of a chunk: ring slot of u is u % P
  struct Stage {
    u32x4_t k[NP], v[NP];
    int ok;                            // bit i: piece i's page may be read
  };
  Stage ring[P];
  auto piece_t0 = [&](int u, int i) {  // position of piece i's tile token 0 in sub-block u
    return (u >> 3) * kChunk + (u & 7) * kSub + kTile * (((tid + i * kThreads) * 8) / TE);
  };
  auto load_sub = [&](int u, int pages, Stage& st) {
    st.ok = 0;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int w = ((tid + i * kThreads) * 8) % TE;
      const int t0 = piece_t0(u, i);
      const int lp = t0 >> log2_ps;
      const int raw = __shfl(pages, (t0 & (kChunk - 1)) >> log2_ps, kWave);
      const bool ok = t0 < lim && lp < max_pages && raw >= 0 && raw < num_pages;
      const int64_t tb = ok ? raw * page_elems + head_off + (int64_t)((t0 & (ps - 1)) >> 4) * TE + w : 0;
      st.k[i] = *reinterpret_cast<const u32x4_t*>(kc + tb);
      st.v[i] = *reinterpret_cast<const u32x4_t*>(vc + tb);
      st.ok |= ok ? (1 << i) : 0;
    }
  };
  auto store_sub = [&](int buf, int u, const Stage& st) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int pc = tid + i * kThreads;
      const bool ok = (st.ok >> i) & 1;
      // K rows past lim are masked in the scores; only a missing page is zeroed.
      *reinterpret_cast<u32x4_t*>(&sK[buf][pc * 8]) = ok ? st.k[i] : zero4();
      // V piece: one dim of 8 tokens (half (w / 128) % 2 of the tile); tokens
      // past lim are zeroed.
      const int vt0 = piece_t0(u, i) + 8 * (((pc * 8) % TE >> 7) & 1);
      *reinterpret_cast<u32x4_t*>(&sV[buf][pc * 8]) = ok ? keep_first(st.v[i], lim - vt0) : zero4();
    }
  };

  // Running state of the fold over chunks (per column block).
  float m_run[kNB], l_run[kNB];
  f32x4_t o_run[kNB][D / 16];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o_run[nb][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int nch = (lim + kChunk - 1) / kChunk;
  const int last_subs = (lim - (nch - 1) * kChunk + kSub - 1) / kSub;
  const int U = (nch - 1) * kSubs + last_subs;

  ChunkAcc<D, kNB> ca;
  int nvalid[kNB];
  int cur_pages = raw_pages(0), next_pages = raw_pages(1);
#pragma unroll
  for (int p = 0; p < P; ++p) load_sub(p, cur_pages, ring[p]);
  store_sub(0, 0, ring[0]);
  __syncthreads();
  // Outer loop over chunks, the 8 sub-blocks of a chunk unrolled so that ring
  // slots and LDS buffers are static: sub-block u = 8 c + s sits in ring slot
  // s % P and LDS buffer s & 1.
  for (int c = 0; c < nch; ++c) {
    const int after_pages = raw_pages(c + 2);
    chunk_init(ca);
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
      nvalid[nb] = row_ok[nb] ? max(0, min(kChunk, pos[nb] + 1 - c * kChunk)) : 0;
    const int subs = c == nch - 1 ? last_subs : kSubs;
    // One 32-key sub-block: refill its ring slot with sub-block u + P (chunk c
    // or c + 1; the slot was copied into LDS at the end of step u - 1), run the
    // chunk step on LDS buffer s & 1, copy sub-block u + 1 from its slot into
    // the other buffer.  Ring slots are named statically: slot of u is s % P.
    auto step = [&](int s, Stage& refill, const Stage& next) {
      const int u = c * kSubs + s;
      load_sub(u + P, s + P < kSubs ? cur_pages : next_pages, refill);
      if (c * kChunk + s * kSub < wave_lim) {   // some column of this wave sees a key here
        const int buf = s & 1;
        const int l16 = n;
        u32x4_t kf[2][D / 32], vf[D / 16];
        // Same operand addressing as decode, inside the LDS copy of the two tiles.
        const int kofs = (l16 >> 3) * TE + g * 128 + (l16 & 7) * 8;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks)
            kf[b][ks] = *reinterpret_cast<const u32x4_t*>(&sK[buf][kofs + 4 * ks * 128 + 8 * b * 8]);
        const int vofs = (g >> 1) * TE + (g & 1) * 128 + l16 * 8;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
          vf[dt] = *reinterpret_cast<const u32x4_t*>(&sV[buf][vofs + dt * 256]);
        SubProbs<kNB> sp;
        chunk_scores<D, kNB>(ca, kf, qf, nvalid, s, scale_log2, sp);
        chunk_values<D, kNB>(ca, vf, sp);
      }
      if (u + 1 < U) store_sub((s + 1) & 1, u + 1, next);
      __syncthreads();
    };
    static_assert(P == 4 && kSubs == 8, "ring slots below are written out for P = 4");
    for (int s4 = 0; s4 < kSubs; s4 += 4) {
      if (s4 + 0 < subs) step(s4 + 0, ring[0], ring[1]);
      if (s4 + 1 < subs) step(s4 + 1, ring[1], ring[2]);
      if (s4 + 2 < subs) step(s4 + 2, ring[2], ring[3]);
      if (s4 + 3 < subs) step(s4 + 3, ring[3], ring[0]);
    }
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      if (nvalid[nb] > 0) {
        const MergeCoef k = merge_coef(m_run[nb], ca.m[nb]);
        l_run[nb] = merge_val(l_run[nb], ca.l[nb], k);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) o_run[nb][dt][i] = merge_val(o_run[nb][dt][i], ca.o[nb][dt][i], k);
        m_run[nb] = k.m;
      }
    }
    cur_pages = next_pages;
    next_pages = after_pages;
  }

#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    if (!row_ok[nb]) continue;
    const int rho = wrow0 + 16 * nb + n;
    const int tok = rho / G, hh = rho - tok * G;
    uint16_t* op = out + ((int64_t)(qs + tok) * Hq + h * G + hh) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const f32x4_t a = o_run[nb][dt];
      *reinterpret_cast<u32x2_t*>(op + 16 * dt) =
          u32x2_t{pack_bf16x2(finalize_val(a[0], l_run[nb]), finalize_val(a[1], l_run[nb])),
                  pack_bf16x2(finalize_val(a[2], l_run[nb]), finalize_val(a[3], l_run[nb]))};
    }
    if (lse != nullptr && g == 0) lse[(int64_t)(qs + tok) * Hq + h * G + hh] = finalize_lse(m_run[nb], l_run[nb]);
  }
}

template <int D>
hipError_t launch(const void* q, int64_t ld_q, const int32_t* q_start, const int32_t* ctx_lens, int num_seqs,
                  int max_q_len, const AttnGeom& g, void* out, float* lse, hipStream_t stream) {
  const int G = g.num_q_heads / g.num_kv_heads;
  const int tiles = (max_q_len * G + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(attn_prefill_kernel<D>, dim3(tiles, g.num_kv_heads, num_seqs), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(q), ld_q, q_start, ctx_lens, max_q_len,
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
