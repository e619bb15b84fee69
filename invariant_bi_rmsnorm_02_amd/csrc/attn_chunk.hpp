// The one attention reduction shared by decode and chunked prefill.
//
// "Thinking Machines Lab - Defeating Nondeterminism in LLM Inference", section
// "3. Batch-Invariant Attention" (figs. "Fixed Number Split KV Strategy",
// "Fixed Size Split KV Strategy"), and "Batch Invariance and Numerical
// Reproducibility" (answer on fixed-size chunks): the keys of a sequence are
// cut into fixed 256-token chunks anchored at position 0; every chunk yields
// un-normalised softmax statistics (max, sum, accumulators) and the chunks are
// folded in ascending order.  Both kernels run exactly the arithmetic below,
// so a query row's result depends only on its own query vector, its position
// and the cache contents - never on which kernel, batch or other query rows it
// was computed with.  The kernels differ only in how K/V fragments reach the
// registers (decode: straight from the paged cache; prefill: staged in LDS and
// shared by the workgroup's wavefronts), which moves bits, not arithmetic.
//
// Inside a chunk, keys are consumed in eight 32-key sub-blocks in ascending
// order with a lazily raised reference max m (log2 units): for sub-block s and
// one query column, with c = scale * log2(e) and S_j = q . k_j (masked: -inf),
//   mx    = c * max_j S_j                            (= max_j of c S_j: rounding is monotone)
//   if mx > m + 8:  alpha = (m == -inf ? 1 : 2^(m - mx)),  m = mx   (else alpha = 1)
//   p_j   = 2^(fma(S_j, c, -m'))                     (m' = m, or 0 while m = -inf)
//   l     = l * alpha + sum_j p_j
//   o     = o * alpha + sum_j bf16(p_j) v_j          (one MFMA per 16 head dims)
// starting from (m, l, o) = (-inf, 0, 0).  Any reference gives the same
// softmax in exact arithmetic; raising it only when a score passes it by more
// than 2^8 keeps every p_j <= 256 (far inside fp32 and bf16 range) while the
// rescale of o, the costly part of an online softmax, almost never runs.
// While m = -inf every p so far was 0, so l and o are zeros and alpha = 1
// leaves them as they are.  A sub-block with no key visible to a column leaves
// that column's (m, l, o) bit-identical (alpha = 1, p = 0), so a kernel may
// skip sub-blocks that no column of its wave can see.
// Sums over the 8 keys a lane holds run in key order, then lane^16, lane^32.
//
// Register layout of one wavefront (16 query rows = MFMA columns n):
//   S^T = K Q^T  (MFMA A = keys, B = Q^T, k = head dim; d of k index
//     (step ks, lane group g, element j) = 32 ks + 8 g + j).  Row m' of
//     block b of a sub-block is key 8 (m' / 4) + 4 b + (m' % 4), so lane group
//     g ends up holding keys 8 g .. 8 g + 7 of its column.
//   O^T = V^T P^T (MFMA A = V^T rows = head dims, k = keys 8 g + j of lane
//     group g): P never leaves the registers; V is stored dim-major in a page
//     so a lane's 8 keys of one dim are 16 contiguous bytes.
#pragma once

#include "bi_common.hpp"

namespace bi {

constexpr int kChunk = 256;   // fixed split size in tokens
constexpr int kSub = 32;      // keys per sub-block
constexpr int kSubs = kChunk / kSub;
constexpr float kRefSlack = 8.0f;   // log2 units a score may pass the reference max by

// Key (relative to the sub-block) of MFMA row m' of S^T block b.
__device__ __forceinline__ int sub_key_of_row(int mr, int b) { return 8 * (mr >> 2) + 4 * b + (mr & 3); }

template <int D, int NB>
struct ChunkAcc {
  float m[NB];             // reference max (log2 units), -inf before the first visible key
  float nm[NB];            // -m, or 0 while m = -inf (the exponent offset)
  float l[NB];             // running sum of 2^(c S - m)
  f32x4_t o[NB][D / 16];   // lane: column n = lane % 16, head dims 16 dt + 4 g + i
};

template <int D, int NB>
__device__ __forceinline__ void chunk_init(ChunkAcc<D, NB>& a) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    a.m[nb] = -INFINITY;
    a.nm[nb] = 0.0f;
    a.l[nb] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) a.o[nb][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
}

// One 32-key sub-block s of the chunk, in two halves so that a kernel can
// bring in V between them: chunk_scores (S = K Q^T, online max and sum, the
// bf16 probabilities) and chunk_values (O = O * alpha + V^T P^T).
// kf: S^T A operands [block b][step ks]; vf: O^T A operands [dim tile dt];
// qf: Q^T B operands [n-block][step ks]; n_valid[nb]: keys of the chunk that
// column (lane % 16) of n-block nb may see (keys 0 .. n_valid - 1).
template <int NB>
struct SubProbs {
  u32x4_t pb[NB];   // bf16 p of the lane's 8 keys (MFMA B operand of O^T)
  float alpha[NB];  // rescale of the previous (l, o)
};

template <int D, int NB>
__device__ __forceinline__ void chunk_scores(ChunkAcc<D, NB>& a, const u32x4_t (&kf)[2][D / 32],
                                             const u32x4_t (&qf)[NB][D / 32], const int (&n_valid)[NB], int s,
                                             float scale_log2, SubProbs<NB>& sp) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    f32x4_t S[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      S[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) S[b] = mfma_16x16x32(kf[b][ks], qf[nb][ks], S[b]);
    }
    float t[8];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) t[4 * b + i] = S[b][i];
    // When every column of the wavefront sees the whole sub-block the mask
    // selects nothing; skipping it leaves every value as it is.  Otherwise key
    // 32 s + 8 g + j of the lane is visible iff j < r.
    if (!__all(kSub * (s + 1) <= n_valid[nb])) {
      const int r = n_valid[nb] - kSub * s - 8 * g;
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = j < r ? t[j] : -INFINITY;
    }
    float mx = t[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, t[j]);
    // The column max needs the other lane groups only when some lane's own
    // keys pass the reference by more than the slack; otherwise no column of
    // the wavefront moves and the exchange is skipped.
    float alpha = 1.0f;
    if (__any(mx * scale_log2 > a.m[nb] + kRefSlack)) {
      const float cm = max_xor32(max_xor16(mx)) * scale_log2;
      if (cm > a.m[nb] + kRefSlack) {
        alpha = a.m[nb] == -INFINITY ? 1.0f : exp2_hw(a.m[nb] - cm);
        a.m[nb] = cm;
        a.nm[nb] = -cm;
      }
    }
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = exp2_hw(fmaf(t[j], scale_log2, a.nm[nb]));
    // Key order.  p >= 0 is never -0, so starting from p[0] is 0 + p[0] to the bit.
    float ls = p[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) ls = ls + p[j];
    ls = add_xor32(add_xor16(ls));
    a.l[nb] = a.l[nb] * alpha + ls;
    sp.alpha[nb] = alpha;
    sp.pb[nb] = u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                        pack_bf16x2(p[6], p[7])};
  }
}

template <int D, int NB>
__device__ __forceinline__ void chunk_values(ChunkAcc<D, NB>& a, const u32x4_t (&vf)[D / 16],
                                             const SubProbs<NB>& sp) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float alpha = sp.alpha[nb];
    // alpha == 1 (the running max did not move) in every lane: o * 1 is o, so
    // the rescale is skipped without changing a bit.
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const f32x4_t o = a.o[nb][dt];
        a.o[nb][dt] = f32x4_t{o[0] * alpha, o[1] * alpha, o[2] * alpha, o[3] * alpha};
      }
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) a.o[nb][dt] = mfma_16x16x32(vf[dt], sp.pb[nb], a.o[nb][dt]);
  }
}

// One step of the ascending fold over chunks: state (m, l, acc) absorbs the
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

// Final normalisation; +0.0f turns a -0 into +0 so that a zero result has one
// bit pattern whichever keys contributed exact zeros.
__device__ __forceinline__ float finalize_val(float acc, float l) { return acc / l + 0.0f; }
__device__ __forceinline__ float finalize_lse(float m, float l) { return (m + log2_hw(l)) * kLn2; }

// Page ids of one chunk, one per lane: lane l holds logical page
// chunk * pages_per_chunk + l % pages_per_chunk, or -1 when that page is past
// `lim` (no row can see it), past the table, or outside the pool.
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

__device__ __forceinline__ u32x4_t zero4() { return u32x4_t{0u, 0u, 0u, 0u}; }

// Word masks keeping bf16 elements 0 .. nv-1 of an 8-element fragment.
struct KeepMask {
  uint32_t w[4];
};
__device__ __forceinline__ KeepMask keep_mask(int nv) {
  KeepMask k;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    k.w[e] = ((2 * e < nv) ? 0x0000ffffu : 0u) | ((2 * e + 1 < nv) ? 0xffff0000u : 0u);
  return k;
}
__device__ __forceinline__ u32x4_t apply_keep(u32x4_t v, const KeepMask& k) {
  return u32x4_t{v[0] & k.w[0], v[1] & k.w[1], v[2] & k.w[2], v[3] & k.w[3]};
}
__device__ __forceinline__ u32x4_t keep_first(u32x4_t v, int nv) { return apply_keep(v, keep_mask(nv)); }

}  // namespace bi
