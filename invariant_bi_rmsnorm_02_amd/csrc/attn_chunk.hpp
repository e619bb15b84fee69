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
//   if mx > m + 8:  alpha = (m == m0 ? 1 : 2^(m - mx)),  m = mx   (else alpha = 1)
//   l     = l * alpha,  o = o * alpha
//   p_j   = 2^(fma(S_j, c, -m))
//   l     = l + sum_j p_j                            (per lane, see below)
//   o     = o + sum_j bf16(p_j) v_j                  (one MFMA per 16 head dims)
// starting from (m, l, o) = (m0, 0, 0), m0 = -FLT_MAX: no score is visible
// yet.  The first visible score always moves m (any finite mx > m0 + 8 = m0),
// so a p is only ever taken against a real score's reference; masked scores
// are -inf and give p = 2^-inf = 0 whatever m is.  Any reference gives the same
// softmax in exact arithmetic; raising it only when a score passes it by more
// than 2^8 keeps every p_j <= 256 (far inside fp32 and bf16 range) while the
// rescale of o, the costly part of an online softmax, almost never runs.
// While m = m0 every p so far was 0, so l and o are zeros and alpha = 1
// leaves them as they are.  A sub-block with no key visible to a column leaves
// that column's (m, l, o) bit-identical (alpha = 1, p = 0), so a kernel may
// skip sub-blocks that no column of its wave can see.  Each lane keeps its
// own part of l: the sum over the keys it holds (8 g .. 8 g + 7 of every
// sub-block), added in key order and rescaled with the column; the four parts
// of a column are combined once per chunk, lane^16 then lane^32.
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
constexpr float kRefNone = -3.402823466e38f;   // the reference before any visible score (-FLT_MAX)

template <int D, int NB>
struct ChunkAcc {
  float m[NB];             // reference max (log2 units), kRefNone before the first visible key
  float thr[NB];           // m + kRefSlack
  float l[NB];             // this lane's part of the running sum of 2^(c S - m)
  f32x4_t o[NB][D / 16];   // lane: column n = lane % 16, head dims 16 dt + 4 g + i
};

template <int D, int NB>
__device__ __forceinline__ void chunk_init(ChunkAcc<D, NB>& a) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    a.m[nb] = kRefNone;
    a.thr[nb] = kRefNone + kRefSlack;
    a.l[nb] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) a.o[nb][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
}

// One 32-key sub-block s of the chunk, as five steps that every kernel runs in
// this order for each column (a kernel may interleave the steps of different
// sub-blocks, e.g. start the scores of s + 1 before the values of s):
//   sub_scores    S = K Q^T (raw q . k, one fp32 MFMA chain per element)
//   sub_mask      keys the column cannot see -> -inf
//   sub_reference maybe raise m; a column that moves rescales its l and o
//   sub_probs     p = 2^fma(S, c, -m), l += sum p, P^T in bf16
//   sub_values    O^T += V^T P^T
// kf: S^T A operands [block b][step ks]; vf: O^T A operands [dim tile dt];
// qf: Q^T B operands [n-block][step ks]; n_valid[nb]: keys of the chunk that
// column (lane % 16) of n-block nb may see (keys 0 .. n_valid - 1).
template <int D, int NB>
__device__ __forceinline__ void sub_scores(const u32x4_t (&kf)[2][D / 32], const u32x4_t (&qf)[NB][D / 32],
                                           f32x4_t (&S)[NB][2]) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      S[nb][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) S[nb][b] = mfma_16x16x32(kf[b][ks], qf[nb][ks], S[nb][b]);
    }
}

// Lane group g holds keys 8 g + j of the sub-block, j = 4 b + i for S[nb][b][i].
// When every column of the wavefront sees the whole sub-block the mask selects
// nothing; skipping it leaves every value as it is.  Otherwise key 32 s + 8 g
// + j is visible iff j < r.
template <int NB>
__device__ __forceinline__ void sub_mask(f32x4_t (&S)[NB][2], const int (&n_valid)[NB], int s) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (!__all(kSub * (s + 1) <= n_valid[nb])) {
      const int r = n_valid[nb] - kSub * s - 8 * g;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[nb][b][i] = 4 * b + i < r ? S[nb][b][i] : -INFINITY;
    }
  }
}

// Max of three scores with v_max3_f32.  Scores are MFMA results or -inf and
// never NaN; fmaxf would first quiet each (possibly signalling) MFMA result.
__device__ __forceinline__ float max3_score(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// The column max needs the other lane groups only when some lane's own keys
// pass the reference by more than the slack; otherwise no column of the
// wavefront moves and the exchange is skipped.  A column that moves has its l
// and o multiplied by alpha = 2^(m_old - m_new) (alpha = 1 while m_old =
// kRefNone: l and o are zeros then); the others keep theirs, as alpha = 1 would.
template <int D, int NB>
__device__ __forceinline__ void sub_reference(ChunkAcc<D, NB>& a, const f32x4_t (&S)[NB][2], float scale_log2) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float mx = max3_score(S[nb][0][0], S[nb][0][1], S[nb][0][2]);
    mx = max3_score(mx, S[nb][0][3], S[nb][1][0]);
    mx = max3_score(mx, S[nb][1][1], S[nb][1][2]);
    mx = max3_score(mx, S[nb][1][3], S[nb][1][3]);
    if (__any(mx * scale_log2 > a.thr[nb])) {
      const float cm = max_xor32(max_xor16(mx)) * scale_log2;
      if (cm > a.thr[nb]) {
        const float alpha = a.m[nb] == kRefNone ? 1.0f : exp2_hw(a.m[nb] - cm);
        a.m[nb] = cm;
        a.thr[nb] = cm + kRefSlack;
        a.l[nb] = a.l[nb] * alpha;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const f32x4_t o = a.o[nb][dt];
          a.o[nb][dt] = f32x4_t{o[0] * alpha, o[1] * alpha, o[2] * alpha, o[3] * alpha};
        }
      }
    }
  }
}

template <int D, int NB>
__device__ __forceinline__ void sub_probs(ChunkAcc<D, NB>& a, const f32x4_t (&S)[NB][2], float scale_log2,
                                          u32x4_t (&pb)[NB]) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = exp2_hw(fmaf(S[nb][j >> 2][j & 3], scale_log2, -a.m[nb]));
    float l = a.l[nb];
#pragma unroll
    for (int j = 0; j < 8; ++j) l = l + p[j];
    a.l[nb] = l;
    pb[nb] = u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                     pack_bf16x2(p[6], p[7])};
  }
}

template <int D, int NB>
__device__ __forceinline__ void sub_values(ChunkAcc<D, NB>& a, const u32x4_t (&vf)[D / 16], const u32x4_t (&pb)[NB]) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) a.o[nb][dt] = mfma_16x16x32(vf[dt], pb[nb], a.o[nb][dt]);
}

// The column's l: its four lane parts combined, lane^16 then lane^32 (every
// lane of the column gets the same value).
template <int D, int NB>
__device__ __forceinline__ float chunk_l(const ChunkAcc<D, NB>& a, int nb) {
  return add_xor32(add_xor16(a.l[nb]));
}

// The first four steps of a sub-block in one call (the fifth, sub_values,
// follows once V is in the registers).
template <int D, int NB>
__device__ __forceinline__ void chunk_scores(ChunkAcc<D, NB>& a, const u32x4_t (&kf)[2][D / 32],
                                             const u32x4_t (&qf)[NB][D / 32], const int (&n_valid)[NB], int s,
                                             float scale_log2, u32x4_t (&pb)[NB]) {
  f32x4_t S[NB][2];
  sub_scores<D, NB>(kf, qf, S);
  sub_mask<NB>(S, n_valid, s);
  sub_reference<D, NB>(a, S, scale_log2);
  sub_probs<D, NB>(a, S, scale_log2, pb);
}

// One step of the ascending fold over chunks: state (m, l, acc) absorbs the
// chunk partial (mc, lc, accc).  The state starts at (-inf, 0, 0); mc is
// finite for every chunk that is folded.  Like the chunk step, the state's
// reference moves only when the chunk's passes it by more than the slack, so
// in the common case alpha = 1 and a merge is one fma per element.  Every
// kernel calls these, element by element, with the same operands.
struct MergeCoef {
  float m, alpha, beta;
};
__device__ __forceinline__ MergeCoef merge_coef(float m, float mc) {
  const bool mv = mc > m + kRefSlack;   // always while m = -inf (acc and l are zeros then)
  const float d = exp2_hw(mv ? m - mc : mc - m);
  return MergeCoef{mv ? mc : m, mv && m != -INFINITY ? d : 1.0f, mv ? 1.0f : d};
}
__device__ __forceinline__ float merge_val(float acc, float accc, const MergeCoef& k) {
  return fmaf(accc, k.beta, acc * k.alpha);
}
// merge_val when alpha = 1 (acc * 1 is acc, so the bits are the same).
__device__ __forceinline__ float merge_val_unit(float acc, float accc, const MergeCoef& k) {
  return fmaf(accc, k.beta, acc);
}

// Final normalisation: one correctly rounded reciprocal per row, then a
// product per element; +0.0f turns a -0 into +0 so that a zero result has one
// bit pattern whichever keys contributed exact zeros.
__device__ __forceinline__ float finalize_inv(float l) { return 1.0f / l; }
__device__ __forceinline__ float finalize_val(float acc, float inv_l) { return acc * inv_l + 0.0f; }
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

}  // namespace bi
