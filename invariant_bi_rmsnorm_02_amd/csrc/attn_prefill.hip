// Chunked-prefill attention over the paged KV cache ("Thinking Machines Lab -
// Defeating Nondeterminism in LLM Inference", section "3. Batch-Invariant
// Attention", figs. "FlashAttention2 Strategy" and "FlashAttention with KV
// Cache"; "Como superar a não determinismo na inferência de LLMs", Attention:
// one K/V layout for cached and new tokens).
//
// Parallel over query rows (FlashAttention-2 style): a workgroup owns 64
// (token, q head) rows of one sequence and one kv head, 16 rows per wavefront.
// The chunk's own keys/values are already in the paged cache, so cached and new
// tokens are read through one path.  Each wavefront walks the 256-key chunks in
// ascending order, calls the same chunk routine as decode (causal mask: a query
// at position p sees keys 0..p) and folds every chunk its row can see with the
// same merge step, so row p is bitwise what decode returns at seq_len p + 1.
#include "attn_chunk.hpp"
#include "launch.hpp"

namespace bi {
namespace {

constexpr int kRowsPerWave = 16;
constexpr int kWaves = 4;
constexpr int kRowsPerBlock = kRowsPerWave * kWaves;

template <int D>
__global__ __launch_bounds__(kWaves * 64) void attn_prefill_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const int32_t* __restrict__ q_start,
    const int32_t* __restrict__ ctx_lens, int max_q_len, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int num_pages, const int32_t* __restrict__ block_table,
    int max_pages, int Hq, int Hkv, int log2_ps, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  const int tile = blockIdx.x, h = blockIdx.y, sq = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int G = Hq / Hkv;
  const int qs = q_start[sq];
  const int nq = min(q_start[sq + 1] - qs, max_q_len);
  const int ctx = ctx_lens[sq];
  const int rows = nq * G;
  const int row0 = tile * kRowsPerBlock + wave * kRowsPerWave;
  if (nq <= 0 || ctx < 0 || row0 >= rows) return;  // no barrier in this kernel: early exit is safe
  const int rho = row0 + n;
  const bool row_ok = rho < rows;
  const int tok = rho / G, hh = rho - (rho / G) * G;
  const int pos = ctx + tok;
  const int last = min(row0 + kRowsPerWave, rows) - 1;  // last real row of the wave
  const int lim = ctx + last / G + 1;                     // keys at >= lim no row can see

  u32x4_t qf[D / 32];
  const uint16_t* qp = q + (int64_t)(qs + tok) * ldq + (h * G + hh) * D + 8 * g;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    qf[ks] = row_ok ? *reinterpret_cast<const u32x4_t*>(qp + 32 * ks) : u32x4_t{0u, 0u, 0u, 0u};

  PagedChunk<D> kv;
  kv.kc = kc;
  kv.vc = vc;
  kv.head = h;
  kv.num_kv_heads = Hkv;
  kv.log2_ps = log2_ps;
  kv.lim = lim;
  const int32_t* bt = block_table + (int64_t)sq * max_pages;

  float m = -INFINITY, l = 0.0f;
  f32x4_t acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nch = (lim + kChunk - 1) / kChunk;
  for (int c = 0; c < nch; ++c) {
    kv.chunk_start = c * kChunk;
    kv.page_reg = load_chunk_pages(bt, max_pages, c, log2_ps, lim, num_pages);
    const int nv = row_ok ? max(0, min(kChunk, pos + 1 - c * kChunk)) : 0;
    Partial<D> p;
    chunk_partial<D>(kv, qf, nv, scale_log2, p);
    if (nv > 0) {
      const MergeCoef k = merge_coef(m, p.m);
      l = merge_val(l, p.l, k);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[dt][i] = merge_val(acc[dt][i], p.o[dt][i], k);
      m = k.m;
    }
  }

  if (row_ok) {
    uint16_t* op = out + ((int64_t)(qs + tok) * Hq + h * G + hh) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const f32x4_t a = acc[dt];
      *reinterpret_cast<u32x2_t*>(op + 16 * dt) =
          u32x2_t{pack_bf16x2(finalize_val(a[0], l), finalize_val(a[1], l)),
                  pack_bf16x2(finalize_val(a[2], l), finalize_val(a[3], l))};
    }
    if (lse != nullptr && g == 0) lse[(int64_t)(qs + tok) * Hq + h * G + hh] = finalize_lse(m, l);
  }
}

template <int D>
hipError_t launch(const void* q, int64_t ld_q, const int32_t* q_start, const int32_t* ctx_lens, int num_seqs,
                  int max_q_len, const AttnGeom& g, void* out, float* lse, hipStream_t stream) {
  const int G = g.num_q_heads / g.num_kv_heads;
  const int tiles = (max_q_len * G + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(attn_prefill_kernel<D>, dim3(tiles, g.num_kv_heads, num_seqs), dim3(kWaves * 64),
                     0, stream, static_cast<const uint16_t*>(q), ld_q, q_start, ctx_lens, max_q_len,
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
