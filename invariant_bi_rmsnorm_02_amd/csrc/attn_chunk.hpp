// The one attention reduction shared by decode and chunked prefill.
//
// "Thinking Machines Lab - Defeating Nondeterminism in LLM Inference", section
// "3. Batch-Invariant Attention" (figs. "Fixed Number Split KV Strategy",
// "Fixed Size Split KV Strategy"), and "Batch Invariance and Numerical
// Reproducibility" (answer on fixed-size chunks): the keys of a sequence are
// cut into fixed 256-token chunks anchored at position 0; every chunk yields
// un-normalised softmax statistics and the chunks are folded in ascending
// order.  Both kernels call exactly the routines below, so a query row's result
// depends only on its own query vector, its position and the cache contents -
// not on which kernel, batch, or other query rows it was computed with.
//
// Data layout seen by one wavefront (16 query rows = "columns" n of the MFMA
// output, one kv head, one 256-key chunk):
//   S^T = K Q^T   with MFMA A = K rows (keys), B = Q^T (queries), k = head dim.
//     d of MFMA k index (step ks, lane group g, element j) = 32 ks + 8 g + j.
//     Key of MFMA row m' in block b of 32-key group s:
//       key = 32 s + 8 (m' / 4) + 4 b + (m' % 4),
//     chosen so that lane group g ends up holding the 8 consecutive keys
//     32 s + 8 g + (4 b + i) of its column after the two blocks.
//   O^T = V^T P^T with MFMA A = V^T (head dim rows), B = P^T, k = keys; the k
//     index j of lane group g is key 32 s + 8 g + j, i.e. exactly the keys the
//     lane already holds, so P never leaves its registers.  V is stored
//     dim-major inside a page, so a lane's 8 keys of one dim are 16 contiguous
//     bytes.
// Reduction order inside a chunk, per query column:
//   max: exact (order-free);  sum of p: lane-local over (s, b, i) ascending,
//   then + lane^16, then + lane^32;  O: MFMA chain over s = 0..7 ascending.
// p is rounded once to bf16 for the PV product; the sum uses the fp32 p.
#pragma once

#include "bi_common.hpp"

namespace bi {

constexpr int kChunk = 256;  // fixed split size in tokens

// Paged K/V fragment source for one kv head and one chunk.
//   k_cache: [pages][Hkv][PS][D]   v_cache: [pages][Hkv][D][PS]
// Keys at positions >= lim (no query row of the wave can see them) and pages
// outside [0, num_pages) read as zeros, so unwritten slots never enter.
template <int D>
struct PagedChunk {
  const uint16_t* kc;  // k_cache + head offset handled in address math
  const uint16_t* vc;
  int head;            // kv head
  int num_kv_heads;
  int log2_ps;
  int chunk_start;     // absolute position of key 0 of the chunk
  int lim;             // keys at absolute positions >= lim read as zero
  int page_reg;        // lane l: page id of logical page (chunk page l % pages-per-chunk), or -1

  __device__ __forceinline__ int page_of(int key_in_chunk) const {
    return __shfl(page_reg, key_in_chunk >> log2_ps, kWave);
  }

  // MFMA A operand of S^T for 32-key group s, half b, head-dim step ks.
  __device__ __forceinline__ void k_frags(int s, int b, u32x4_t (&f)[D / 32]) const {
    const int lane = threadIdx.x & 63;
    const int mr = lane & 15, g = lane >> 4;
    const int key = 32 * s + 8 * (mr >> 2) + 4 * b + (mr & 3);
    const int page = page_of(key);
    const int pos = chunk_start + key;
    const int ps = 1 << log2_ps;
    if (pos < lim && page >= 0) {
      const uint16_t* p = kc + (((int64_t)page * num_kv_heads + head) * ps + (pos & (ps - 1))) * D + 8 * g;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) f[ks] = *reinterpret_cast<const u32x4_t*>(p + 32 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) f[ks] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  // MFMA A operand of O^T for head-dim tile dt and 32-key group s.
  __device__ __forceinline__ u32x4_t v_frag(int dt, int s) const {
    const int lane = threadIdx.x & 63;
    const int d = 16 * dt + (lane & 15), g = lane >> 4;
    const int key0 = 32 * s + 8 * g;
    const int page = page_of(key0);
    const int pos0 = chunk_start + key0;
    const int ps = 1 << log2_ps;
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (pos0 < lim && page >= 0) {
      v = *reinterpret_cast<const u32x4_t*>(
          vc + (((int64_t)page * num_kv_heads + head) * D + d) * ps + (pos0 & (ps - 1)));
      const int nv = lim - pos0;  // keys of this fragment that exist
      if (nv < 8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t keep_lo = (2 * e < nv) ? 0x0000ffffu : 0u;
          const uint32_t keep_hi = (2 * e + 1 < nv) ? 0xffff0000u : 0u;
          v[e] &= (keep_lo | keep_hi);
        }
      }
    }
    return v;
  }
};

// Page ids of the chunk, one per lane (lane l holds logical page
// chunk_first_page + l % pages_per_chunk).  Pages past the last one any row of
// the wave can see, or outside the pool, become -1.
__device__ __forceinline__ int load_chunk_pages(const int32_t* bt_row, int max_pages, int chunk,
                                                int log2_ps, int lim, int num_pages) {
  const int lane = threadIdx.x & 63;
  const int ppc = kChunk >> log2_ps;
  const int lp = chunk * ppc + (lane % ppc);
  int pg = -1;
  if (lp < max_pages && (lp << log2_ps) < lim) {
    pg = bt_row[lp];
    if (pg < 0 || pg >= num_pages) pg = -1;
  }
  return pg;
}

template <int D>
struct Partial {
  float m;              // chunk max of scaled scores (log2 units); -inf if no valid key
  float l;              // sum over the chunk of exp2(t - m)
  f32x4_t o[D / 16];    // lane: column n = lane % 16, head dims 16 dt + 4 g + i
};

// Chunk partial for the wave's 16 query columns.  qf: Q^T fragments (lane
// column n = lane % 16, dims 32 ks + 8 g .. +7).  n_valid: number of keys of the
// chunk this lane's query column may see (0..256), keys 0..n_valid-1.
template <int D>
__device__ __forceinline__ void chunk_partial(const PagedChunk<D>& kv, const u32x4_t (&qf)[D / 32],
                                              int n_valid, float scale_log2, Partial<D>& out) {
  const int lane = threadIdx.x & 63, g = lane >> 4;
  f32x4_t S[8][2];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      u32x4_t kf[D / 32];
      kv.k_frags(s, b, kf);
      f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) acc = mfma_16x16x32(kf[ks], qf[ks], acc);
      S[s][b] = acc;
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 32 * s + 8 * g + 4 * b + i;
        const float t = key < n_valid ? S[s][b][i] * scale_log2 : -INFINITY;
        S[s][b][i] = t;
        mx = fmaxf(mx, t);
      }
  mx = fmaxf(mx, shfl_xor(mx, 16));
  mx = fmaxf(mx, shfl_xor(mx, 32));
  const float ms = (mx == -INFINITY) ? 0.0f : mx;

  float ls = 0.0f;
  u32x4_t pb[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    float p[8];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[4 * b + i] = exp2_hw(S[s][b][i] - ms);
        ls = ls + p[4 * b + i];
      }
    pb[s] = u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                    pack_bf16x2(p[6], p[7])};
  }
  ls = ls + shfl_xor(ls, 16);
  ls = ls + shfl_xor(ls, 32);

#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = mfma_16x16x32(kv.v_frag(dt, s), pb[s], acc);
    out.o[dt] = acc;
  }
  out.m = mx;
  out.l = ls;
}

// One step of the ascending log-sum-exp fold: state (m, l, acc) absorbs the
// chunk partial (mc, lc, accc).  The state starts at (-inf, 0, 0); mc is
// finite for every chunk that is folded.  Both kernels call this, element by
// element, with the same operands.
struct MergeCoef {
  float m, alpha, beta;
};
__device__ __forceinline__ MergeCoef merge_coef(float m, float mc) {
  const float mn = fmaxf(m, mc);
  return MergeCoef{mn, exp2_hw(m - mn), exp2_hw(mc - mn)};
}
__device__ __forceinline__ float merge_val(float acc, float accc, const MergeCoef& k) {
  return acc * k.alpha + accc * k.beta;
}

// Final normalisation and output rounding; +0.0f turns a -0 into +0 so that a
// zero result has one bit pattern whichever keys contributed exact zeros.
__device__ __forceinline__ float finalize_val(float acc, float l) { return acc / l + 0.0f; }
__device__ __forceinline__ float finalize_lse(float m, float l) { return (m + log2_hw(l)) * kLn2; }

}  // namespace bi
