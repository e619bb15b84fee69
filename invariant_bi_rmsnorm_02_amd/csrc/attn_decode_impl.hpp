// Decode attention over the paged KV cache with fixed-size split-KV
// ("Thinking Machines Lab - Defeating Nondeterminism in LLM Inference", section
// "3. Batch-Invariant Attention", fig. "Fixed Size Split KV Strategy";
// "Batch Invariance and Numerical Reproducibility", answer on fixed-size chunks):
// the kernels and their launcher, templated on the chunk size CS in keys.
// libbi.so instantiates CS = kChunk (256) only (attn_decode.hip); the
// shape-adaptive comparator (adaptive.hip) instantiates other sizes, picked
// from the batch, to measure what the fixed size costs with every other part
// of the computation - scheduling, chunk step, in-wave fold, merge - the same.
// CS is a power of two from 32 keys up, at least one page and at most 64 pages
// (a chunk's page ids are one per lane); the sub-block loop of a chunk is
// unrolled whole, so registers bound it in practice to 512 keys.
//
// Kernel 1 (grid: chunk x kv head x sequence, one wavefront each): the partial
// statistics of one CS-key chunk for the q heads of one kv head, written to
// the workspace.  A sequence of L tokens has ceil(L / CS) chunks whatever else
// is in the batch; workgroups past a sequence's last chunk exit at once.  K and
// V fragments go from HBM straight into registers in MFMA layout; the next
// 32-key sub-block is in flight while the current one is computed.
// Kernel 2 (grid: q head x sequence): the ascending fold of those partials,
// normalisation and bf16 output.  No floating-point atomics and no ordering
// between workgroups: every output value and every partial is written by
// exactly one wavefront.  (The work-queue path below hands out items with an
// integer atomic counter and sorts them with LDS integer atomics; that decides
// only which wavefront computes an item, never a value.)
#pragma once

#include <algorithm>
#include <climits>

#include "attn_chunk.hpp"
#include "kv_layout.hpp"
#include "launch.hpp"

namespace bi {
namespace {


// Fragments of one chunk of one (sequence, kv head), read from the paged cache
// (tiled layout of kv_layout.hpp: each 16-byte operand load of a wavefront
// covers whole 128-byte lines).  Every K/V byte is read once, so loads carry
// the non-temporal hint.  Loads
// are unconditional: a lane whose key is past `lim` or whose page is outside
// the pool loads from the pool's first bytes instead.  The fetched
// words are masked only where they are used (mask()), so no load waits on a
// branch.  K rows past `lim` need no mask (their scores are masked in the
// chunk step); V keys past `lim` and keys of invalid pages are zeroed.
template <int D, int CS>
struct GlobalChunk {
  const uint16_t* kc;
  const uint16_t* vc;
  int64_t head_k;       // elements from a page start to this kv head's block
  int64_t head_v;       // same for V
  int num_kv_heads;
  int log2_ps;
  int chunk_start;
  int lim;
  int max_pages;
  int num_pages;
  int page_reg;   // raw block-table entry of this lane's logical page (validated where used)
  int lane;       // lane index, re-materialised per chunk so that per-lane address
                  // terms are recomputed rather than held across the chunk loop

  struct Frags {
    u32x4_t k[2][D / 32];
    u32x4_t v[D / 16];
    bool kok;   // this lane's K page is in the pool
    int vnv;    // keys of this lane's V group that exist (<= 0: none)
  };

  // Whether the page holding chunk-relative key `key` may be read: its logical
  // index is inside the block table, the page starts before `lim`, and the
  // table entry names a page of the pool.
  __device__ __forceinline__ bool page_ok(int key, int page) const {
    const int lp = (chunk_start + key) >> log2_ps;
    return lp < max_pages && (lp << log2_ps) < lim && page >= 0 && page < num_pages;
  }

  // Raw block-table entries of `nch` chunks from `chunk`, one per lane as in
  // load_chunk_pages, read from a clamped (always valid) index; nothing here
  // waits for the load, so a later chunk's entries can be fetched early.
  __device__ __forceinline__ static int raw_pages(const int32_t* bt_row, int max_pages, int chunk, int log2_ps) {
    const int ppc = CS >> log2_ps;
    const int lp = chunk * ppc + ((threadIdx.x & 63) % ppc);
    return bt_row[min(lp, max_pages - 1)];
  }

  // active == false, or a page that may not be read, points a lane's loads at
  // the pool's first tile block (the result is never used; the constant
  // per-load offsets stay below the 4 KiB that one page of any supported
  // geometry spans): the loads are still issued so that every path through
  // the caller's loop has the same loads in flight, and the constant offsets
  // fold into the instructions.
  __device__ __forceinline__ void fetch(int s, Frags& f, bool active) const {
    const int l16 = lane & 15, g = lane >> 4;
    const int ps = 1 << log2_ps;
    const int64_t page_elems = (int64_t)(num_kv_heads << log2_ps) * D;   // one page, all kv heads
    // K: lanes l16 < 8 read tile 0 of the sub-block, l16 >= 8 tile 1; in both,
    // the 8 lanes of a group cover 128 contiguous bytes (slots 8 b .. 8 b + 7).
    const int ktile_key = kSub * s + kTile * (l16 >> 3);       // key of the tile's token 0
    const int kpage = __shfl(page_reg, ktile_key >> log2_ps, kWave);
    f.kok = active && page_ok(ktile_key, kpage);
    const uint16_t* kp = kc + (f.kok ? kpage * page_elems + head_k : 0) +
                         (f.kok ? ((ktile_key & (ps - 1)) >> 4) * (kTile * D) + g * 128 + (l16 & 7) * 8 : 0);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        f.k[b][ks] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kp + 4 * ks * 128 + 8 * b * 8));
    // V: lane group g holds keys 8 g .. 8 g + 7 of the sub-block = tile g / 2,
    // half g % 2; the 16 lanes of a group cover 256 contiguous bytes.
    const int vtile_key = kSub * s + kTile * (g >> 1);
    const int vpage = __shfl(page_reg, vtile_key >> log2_ps, kWave);
    const bool vok = active && page_ok(vtile_key, vpage);
    f.vnv = vok ? lim - (chunk_start + kSub * s + 8 * g) : 0;
    const uint16_t* vp = vc + (vok ? vpage * page_elems + head_v : 0) +
                         (vok ? ((vtile_key & (ps - 1)) >> 4) * (kTile * D) + (g & 1) * 128 + l16 * 8 : 0);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      f.v[dt] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vp + dt * 256));
  }

  // Branch-free masking, applied right where each half is consumed so the
  // wait for a fragment never covers the loads of the next sub-block.
  __device__ __forceinline__ static void mask_k(Frags& f) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) f.k[b][ks] = f.kok ? f.k[b][ks] : zero4();
  }
  __device__ __forceinline__ static void mask_v(Frags& f) {
    const KeepMask km = keep_mask(f.vnv);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) f.v[dt] = apply_keep(f.v[dt], km);
  }
};

// One wavefront's work: chunks c_first .. c_first + chunks_per_wave - 1 of
// kv head h of sequence b.  kFold == false: each chunk's partial goes to its
// workspace record and the merge kernel folds them.  kFold == true (c_first
// is 0): the wavefront folds each chunk's partial into a running state right
// after computing it - per element the same merge step, in the same ascending
// order, as the merge kernel - and then either writes out / lse (it had every
// chunk of the sequence) or, with to_record, stores the running state in
// chunk 0's record, from which the merge kernel continues the same fold.
template <int D, bool kFold, int CS>
__device__ __forceinline__ void decode_wave(
    int b, int h, int c_first, bool to_record, const uint16_t* __restrict__ q, int64_t ldq, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int num_pages, const int32_t* __restrict__ block_table,
    int max_pages, const int32_t* __restrict__ seq_lens, int max_seq_len, int Hq, int Hkv, int log2_ps,
    float scale_log2, float* __restrict__ ws, int max_chunks, int chunks_per_wave, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  const int L = min(seq_lens[b], max_seq_len);
  if constexpr (kFold) {
    if (L <= 0) {   // the merge kernel's result for an empty sequence
      const int lane = threadIdx.x, n = lane & 15, g = lane >> 4, G = Hq / Hkv;
      if (n < G) {
        uint16_t* op = out + ((int64_t)b * Hq + h * G + n) * D + 4 * g;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<u32x2_t*>(op + 16 * dt) = u32x2_t{0u, 0u};
        if (lse != nullptr && g == 0) lse[(int64_t)b * Hq + h * G + n] = -INFINITY;
      }
      return;
    }
  }
  if (c_first * CS >= L) return;
  const int c_end = min((L + CS - 1) / CS, c_first + chunks_per_wave);
  constexpr int kCS = CS / kSub;   // sub-blocks per chunk
  const int G = Hq / Hkv;
  const int lane = threadIdx.x, n = lane & 15, g = lane >> 4;
  const bool row_ok = n < G;

  u32x4_t qf[1][D / 32];
  const uint16_t* qp = q + (int64_t)b * ldq + (h * G + n) * D + 8 * g;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    qf[0][ks] = row_ok ? *reinterpret_cast<const u32x4_t*>(qp + 32 * ks) : zero4();

  const int ps = 1 << log2_ps;
  const int32_t* bt_row = block_table + (int64_t)b * max_pages;
  GlobalChunk<D, CS> src;
  src.kc = kc;
  src.vc = vc;
  src.head_k = (int64_t)h * ps * D;
  src.head_v = (int64_t)h * ps * D;
  src.num_kv_heads = Hkv;
  src.log2_ps = log2_ps;
  src.chunk_start = c_first * CS;
  src.lim = L;
  src.max_pages = max_pages;
  src.num_pages = num_pages;
  src.page_reg = GlobalChunk<D, CS>::raw_pages(bt_row, max_pages, c_first, log2_ps);
  src.lane = lane;
  float* rec = ws + (((int64_t)b * Hq + h * G + n) * max_chunks + c_first) * (D + 4);

  // Chunks c_first .. c_end - 1, one after the other.  Each chunk is reduced
  // from a fresh state and written to its own record, exactly as a wavefront
  // of its own would; the sub-block prefetch runs on across the boundary into
  // the next chunk (whose page ids are loaded one chunk ahead).
  using Src = GlobalChunk<D, CS>;
  typename Src::Frags fa, fb;
  u32x4_t sp[1];   // bf16 P^T of the sub-block in flight
  ChunkAcc<D, 1> acc;
  // Fold state (kFold): m and l in registers, the running o in LDS (the
  // wavefront is its own workgroup; lane l owns o_run[.][l]), which keeps it
  // out of the registers the load pipeline needs.
  float m_run = -INFINITY, l_run = 0.0f;
  __shared__ f32x4_t o_run[kFold ? D / 16 : 1][64];
  if constexpr (kFold) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o_run[dt][lane] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  src.fetch(0, fa, true);
  for (int c = c_first; c < c_end; ++c) {
    int ln = threadIdx.x & 63;
    asm volatile("" : "+v"(ln));
    src.lane = ln;
    const bool more = c + 1 < c_end;
    const int next_pages = GlobalChunk<D, CS>::raw_pages(bt_row, max_pages, c + 1, log2_ps);
    const int nvalid[1] = {min(CS, L - c * CS)};
    const int n_sub = (nvalid[0] + kSub - 1) / kSub;
    chunk_init(acc);
    // Ping-pong over sub-blocks: the loads of sub-block s + 1 are always in
    // flight while sub-block s is computed.  After the last fetch of a full
    // chunk, `src` moves on to the next chunk and fetches its sub-block 0
    // (masks are taken at fetch time, so the sub-block still being computed
    // does not need `src`).
#pragma unroll
    for (int s = 0; s < kCS; s += 2) {
      src.fetch(s + 1, fb, s + 1 < n_sub);
      Src::mask_k(fa);
      chunk_scores<D, 1>(acc, fa.k, qf, nvalid, s, scale_log2, sp);
      Src::mask_v(fa);
      sub_values<D, 1>(acc, fa.v, sp);
      if (s + 1 >= n_sub) break;
      if (s + 2 < kCS) {
        src.fetch(s + 2, fa, s + 2 < n_sub);
      } else {
        src.chunk_start += CS;
        src.page_reg = next_pages;
        src.fetch(0, fa, more);
      }
      Src::mask_k(fb);
      chunk_scores<D, 1>(acc, fb.k, qf, nvalid, s + 1, scale_log2, sp);
      Src::mask_v(fb);
      sub_values<D, 1>(acc, fb.v, sp);
      if (s + 2 >= n_sub) break;
    }
    if constexpr (kFold) {
      const MergeCoef k = merge_coef(m_run, acc.m[0]);
      l_run = merge_val(l_run, chunk_l(acc, 0), k);
      if (__all(k.alpha == 1.0f)) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          f32x4_t r = o_run[dt][lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) r[i] = merge_val_unit(r[i], acc.o[0][dt][i], k);
          o_run[dt][lane] = r;
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          f32x4_t r = o_run[dt][lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) r[i] = merge_val(r[i], acc.o[0][dt][i], k);
          o_run[dt][lane] = r;
        }
      }
      m_run = k.m;
    } else {
      const float lc = chunk_l(acc, 0);   // cross-lane: every lane takes part
      if (row_ok) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4_t*>(rec + 16 * dt + 4 * g) = acc.o[0][dt];
        if (g == 0) {
          rec[D] = acc.m[0];
          rec[D + 1] = lc;
        }
      }
      rec += D + 4;
    }
  }
  if constexpr (kFold) {
    if (row_ok && to_record) {
      // rec is chunk c_first = 0's record (the fold path never advances it).
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4_t*>(rec + 16 * dt + 4 * g) = o_run[dt][lane];
      if (g == 0) {
        rec[D] = m_run;
        rec[D + 1] = l_run;
      }
    } else if (row_ok) {
      uint16_t* op = out + ((int64_t)b * Hq + h * G + n) * D + 4 * g;
      const float inv = finalize_inv(l_run);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const f32x4_t a = o_run[dt][lane];
        *reinterpret_cast<u32x2_t*>(op + 16 * dt) =
            u32x2_t{pack_bf16x2(finalize_val(a[0], inv), finalize_val(a[1], inv)),
                    pack_bf16x2(finalize_val(a[2], inv), finalize_val(a[3], inv))};
      }
      if (lse != nullptr && g == 0) lse[(int64_t)b * Hq + h * G + n] = finalize_lse(m_run, l_run);
    }
  }
}

#define BI_DECODE_ARGS                                                                                      \
  const uint16_t *__restrict__ q, int64_t ldq, const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc, \
      int num_pages, const int32_t *__restrict__ block_table, int max_pages, const int32_t *__restrict__ seq_lens, \
      int max_seq_len, int Hq, int Hkv, int log2_ps, float scale_log2, float *__restrict__ ws, int max_chunks,     \
      int chunks_per_wave, uint16_t *__restrict__ out, float *__restrict__ lse
#define BI_DECODE_PASS                                                                                       \
  q, ldq, kc, vc, num_pages, block_table, max_pages, seq_lens, max_seq_len, Hq, Hkv, log2_ps, scale_log2, ws, \
      max_chunks, chunks_per_wave, out, lse

// Grid: chunk group x kv head x sequence, one wavefront each.
template <int D, bool kFold, int CS>
__global__ __launch_bounds__(64, 2) void attn_decode_partial_kernel(BI_DECODE_ARGS) {
  decode_wave<D, kFold, CS>(blockIdx.z, blockIdx.y, blockIdx.x * chunks_per_wave, false, BI_DECODE_PASS);
}

// Wavefronts fed from a work queue.  An item is (sequence, chunk group, kv
// head): chunk group j is chunks j * cg .. j * cg + cg - 1 (cg = chunks_per_wave),
// items in the order decode_order_kernel wrote (most chunks first), kv head
// fastest.  Group 0 is folded in-wave: into out / lse when it holds the whole
// sequence, else into chunk 0's record; a later group writes one partial per
// chunk, and the merge kernel continues the fold from chunk 0's record with
// chunks cg, cg + 1, ... in ascending order - the same left fold, step for
// step, as one wavefront folding the whole sequence (folding the stored state
// into the empty start state is exact for m and l and can only turn a -0 in o
// into +0, which the final + 0.0f makes one bit pattern anyway).  Each
// wavefront takes the next item from the counter whenever it finishes one, so
// a CU whose items happen to be short takes more of them.  Which wavefront
// takes which item, and cg itself, change no bit.  The counter only grows, so
// every wavefront leaves once it passes the item count.  kGroups == false: cg
// covers every chunk, so every item is a whole sequence (no partials, no merge
// kernel), and the kernel holds only the fold path.
template <int D, bool kGroups, int CS>
__global__ __launch_bounds__(64, 2) void attn_decode_queue_kernel(BI_DECODE_ARGS, const int32_t* __restrict__ item_seq,
                                                                  const int32_t* __restrict__ item_group,
                                                                  int* __restrict__ next,
                                                                  const int* __restrict__ total) {
  const int items = *total;
  for (;;) {
    int it = 0;
    if (threadIdx.x == 0) it = atomicAdd(next, 1);
    it = __shfl(it, 0, kWave);
    if (it >= items) break;
    const int i = it / Hkv, h = it % Hkv;
    const int b = item_seq[i], grp = kGroups ? item_group[i] : 0;
    if (!kGroups) {
      decode_wave<D, true, CS>(b, h, 0, false, BI_DECODE_PASS);
    } else if (grp == 0) {
      const int L = min(seq_lens[b], max_seq_len);
      const int C = L > 0 ? (L + CS - 1) / CS : 0;
      decode_wave<D, true, CS>(b, h, 0, C > chunks_per_wave, BI_DECODE_PASS);
    } else {
      decode_wave<D, false, CS>(b, h, grp * chunks_per_wave, false, BI_DECODE_PASS);
    }
  }
}

// The queue's items: every (sequence, chunk group of cg chunks) pair, a
// sequence with no key counting as one item (its wavefront writes out = 0 and
// lse = -inf), ordered by descending chunks in the group (more than
// kOrderBuckets - 1 chunks share the first bucket; the order inside a bucket is
// whatever the atomics give, which is scheduling only); the item count times
// Hkv, and the queue's counter set to zero.  One workgroup; it runs before the
// queue kernel on the same stream.
constexpr int kOrderThreads = 1024;
constexpr int kOrderBuckets = kOrderThreads;
template <int CS>
__global__ __launch_bounds__(kOrderThreads) void decode_order_kernel(const int32_t* __restrict__ seq_lens,
                                                                     int num_seqs, int max_seq_len, int cg, int Hkv,
                                                                     int32_t* __restrict__ item_seq,
                                                                     int32_t* __restrict__ item_group,
                                                                     int* __restrict__ next, int* __restrict__ total) {
  __shared__ int cnt[kOrderBuckets];
  __shared__ int wsum[kOrderThreads / kWave];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  auto chunks = [&](int b) {
    const int L = min(seq_lens[b], max_seq_len);
    return L > 0 ? (L + CS - 1) / CS : 0;
  };
  auto groups = [&](int c) { return c > 0 ? (c + cg - 1) / cg : 1; };
  auto bucket = [&](int c, int j) {
    const int n = c > 0 ? min(cg, c - j * cg) : 0;
    return kOrderBuckets - 1 - min(n, kOrderBuckets - 1);
  };
  cnt[tid] = 0;
  __syncthreads();
  for (int b = tid; b < num_seqs; b += kOrderThreads) {
    const int c = chunks(b), ng = groups(c);
    for (int j = 0; j < ng; ++j) atomicAdd(&cnt[bucket(c, j)], 1);
  }
  __syncthreads();
  // Exclusive prefix sum over the buckets: inclusive within each wavefront,
  // then the totals of the wavefronts before it.
  const int v = cnt[tid];
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) wsum[wave] = x;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wave; ++w) off += wsum[w];
  cnt[tid] = off + x - v;
  if (tid == kOrderThreads - 1) *total = (off + x) * Hkv;
  __syncthreads();
  for (int b = tid; b < num_seqs; b += kOrderThreads) {
    const int c = chunks(b), ng = groups(c);
    for (int j = 0; j < ng; ++j) {
      const int p = atomicAdd(&cnt[bucket(c, j)], 1);
      item_seq[p] = b;
      item_group[p] = j;
    }
  }
  if (tid == 0) *next = 0;
}

constexpr int kMergeThreads = 256;

// Folds a sequence's records in ascending order: chunk 0's record, then
// chunks cg, cg + 1, ..., C - 1 (cg = 1: every chunk's partial; cg > 1: chunk
// 0's record holds the fold of chunks 0 .. cg - 1).  Sequences with C <= done
// were finished by their queue wavefront.  A workgroup folds DS of the D head
// dims of one (sequence, q head) (DS < D: blockIdx.x = head * (D / DS) +
// slice); every element is folded by the same operations whatever DS is (the
// reference and the sum are per head: each slice's workgroup folds them
// identically, and slice 0 writes the lse), so DS is a launch choice: few
// (sequence, head) pairs are spread over more workgroups.
template <int D, int DS, int CS>
__global__ __launch_bounds__(kMergeThreads) void attn_decode_merge_kernel(
    const float* __restrict__ ws, const int32_t* __restrict__ seq_lens, int max_seq_len, int Hq,
    int max_chunks, int cg, int done, uint16_t* __restrict__ out, float* __restrict__ lse) {
  static_assert(D % DS == 0 && DS % 32 == 0, "dim slices");
  constexpr int E = DS >= 64 ? DS / 64 : 1;        // head dims per lane
  constexpr int NL = DS / E;                        // lanes that fold
  constexpr int R = D + 4;                          // floats per record in the workspace
  constexpr int RS = DS + 4;                        // floats per record in LDS: the slice, then m, l
  constexpr int kPieces = RS / 4;                   // 16-byte pieces per record
  constexpr int kBatch = DS == D ? 64 : 128;        // records per LDS batch
  constexpr int kLoads = (kBatch * kPieces + kMergeThreads - 1) / kMergeThreads;   // per thread per batch
  const int head = blockIdx.x / (D / DS), slice = blockIdx.x % (D / DS), b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63;
  const int L = min(seq_lens[b], max_seq_len);
  const int C = L > 0 ? (L + CS - 1) / CS : 0;
  if (C <= done) return;
  const float* rec0 = ws + ((int64_t)b * Hq + head) * max_chunks * R;

  // The records folded, in order: t = 0 is chunk 0's, t >= 1 is chunk cg - 1 + t.
  // The whole workgroup copies them into LDS kBatch at a time (16-byte pieces,
  // every load of a batch issued before the first store waits), so a long
  // sequence waits for one load latency per batch.  Wavefront 0 then folds the
  // batch in two passes that split merge_coef / merge_val by what depends on
  // the running state:
  //  1. the references: 64 records at a time (lane j holds record j's mc), a
  //     ballot finds the first record that passes the current reference by
  //     more than the slack; the reference becomes its mc and the search goes
  //     on after it.  That is the record-by-record rule (records that do not
  //     pass leave the reference as it is), in one ballot per raise.  Lane j
  //     keeps the reference before record j and forms record j's alpha and
  //     beta with merge_coef, all lanes at once;
  //  2. the fold: l and the accumulators take merge_val with each record's
  //     coefficients in record order, eight records' operands read ahead.
  // Every value is computed by the same operations on the same operands as a
  // record-by-record merge_coef / merge_val loop, so the bits are the same.
  __shared__ __attribute__((aligned(16))) float srec[kBatch * RS];
  __shared__ __attribute__((aligned(8))) f32x2_t scoef[kBatch];
  float m = -INFINITY, l = 0.0f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  const int T = C > 0 ? 1 + max(0, C - cg) : 0;
  for (int t0 = 0; t0 < T; t0 += kBatch) {
    const int nb = min(kBatch, T - t0);
    if (t0 > 0) __syncthreads();     // wavefront 0 is done with the previous batch
    f32x4_t piece[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int p = tid + i * kMergeThreads, j = p / kPieces, q = p - j * kPieces, t = t0 + j;
      const int src = q < DS / 4 ? slice * DS + 4 * q : D;   // the slice's dims, then (m, l, pad)
      if (p < nb * kPieces)
        piece[i] = *reinterpret_cast<const f32x4_t*>(rec0 + (int64_t)(t == 0 ? 0 : cg - 1 + t) * R + src);
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int p = tid + i * kMergeThreads, j = p / kPieces, q = p - j * kPieces;
      if (p < nb * kPieces) *reinterpret_cast<f32x4_t*>(&srec[j * RS + 4 * q]) = piece[i];
    }
    __syncthreads();
    if (tid < 64) {
      for (int j0 = 0; j0 < nb; j0 += 64) {
        const bool have = j0 + lane < nb;
        const float mc = have ? srec[(j0 + lane) * RS + DS] : 0.0f;
        float m_before = m;   // lane: the reference before its record
        int from = 0;
        for (;;) {
          const uint64_t raise = __ballot(have && lane >= from && mc > m + kRefSlack);
          if (raise == 0) break;
          const int j = (int)__builtin_ctzll(raise);
          const float mj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mc), j));
          m_before = lane > j ? mj : m_before;
          m = mj;
          from = j + 1;
        }
        if (have) {
          const MergeCoef k = merge_coef(m_before, mc);
          scoef[j0 + lane] = f32x2_t{k.alpha, k.beta};
        }
      }
    }
    __syncthreads();
    if (tid < NL) {
      auto fold = [&](f32x2_t ab, float lc, const float (&c)[E]) {
        const MergeCoef k{0.0f, ab[0], ab[1]};
        l = merge_val(l, lc, k);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = merge_val(acc[e], c[e], k);
      };
      int j = 0;
      for (; j + 8 <= nb; j += 8) {
        f32x2_t ab[8];
        float lc[8], c[8][E];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          ab[u] = scoef[j + u];
          lc[u] = srec[(j + u) * RS + DS + 1];
#pragma unroll
          for (int e = 0; e < E; ++e) c[u][e] = srec[(j + u) * RS + lane * E + e];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) fold(ab[u], lc[u], c[u]);
      }
      for (; j < nb; ++j) {
        float c[E];
#pragma unroll
        for (int e = 0; e < E; ++e) c[e] = srec[j * RS + lane * E + e];
        fold(scoef[j], srec[j * RS + DS + 1], c);
      }
    }
  }
  if (tid >= NL) return;
  uint16_t* op = out + ((int64_t)b * Hq + head) * D + slice * DS + lane * E;
  const bool write_lse = lse != nullptr && lane == 0 && slice == 0;
  if (C > 0) {
    const float inv = finalize_inv(l);
#pragma unroll
    for (int e = 0; e < E; ++e) op[e] = static_cast<uint16_t>(f32_to_bf16(finalize_val(acc[e], inv)));
    if (write_lse) lse[(int64_t)b * Hq + head] = finalize_lse(m, l);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) op[e] = 0;
    if (write_lse) lse[(int64_t)b * Hq + head] = -INFINITY;
  }
}

// The merge launch: (sequence, q head) pairs below kMergeSliceBelow get one
// workgroup per 32 head dims, so a few long sequences are folded by more CUs
// (every slice folds its dims with the same operations; no bit moves).
constexpr int kMergeSliceBelow = 1024;
template <int D, int CS>
hipError_t launch_merge(const float* ws, const int32_t* seq_lens, int max_seq_len, int Hq, int num_seqs,
                        int max_chunks, int cg, int done, uint16_t* out, float* lse, hipStream_t stream) {
  if ((int64_t)Hq * num_seqs < kMergeSliceBelow)
    hipLaunchKernelGGL((attn_decode_merge_kernel<D, 32, CS>), dim3(Hq * (D / 32), num_seqs), dim3(kMergeThreads), 0,
                       stream, ws, seq_lens, max_seq_len, Hq, max_chunks, cg, done, out, lse);
  else
    hipLaunchKernelGGL((attn_decode_merge_kernel<D, D, CS>), dim3(Hq, num_seqs), dim3(kMergeThreads), 0, stream, ws,
                       seq_lens, max_seq_len, Hq, max_chunks, cg, done, out, lse);
  return hipGetLastError();
}

// Scheduling (none of it changes a bit: a chunk is reduced the same way
// whichever wavefront runs it, and every fold is the same ascending left fold).
//  - Few chunks in the batch (at most kDecodeGridItems (sequence, kv head,
//    chunk) items): one wavefront per chunk on a grid, every partial written,
//    then the merge kernel; the grid is (nearly) resident at once, and a work
//    queue's extra launch would only add latency.
//  - Otherwise a work queue of (sequence, chunk group, kv head) items, groups
//    of cg chunks with cg chosen so that there are at most about
//    kDecodeQueueItems of them (cg = every chunk, i.e. whole sequences and no
//    merge launch, once the batch alone gives that many (sequence, kv head)
//    pairs), fed to at most kDecodeQueueWaves wavefronts (two per CU).
// Measured on MI355X: whole-sequence wavefronts from the queue at 1024-4096
// (sequence, kv head) pairs are 10-16% faster than one wavefront per pair in
// grid order (Qwen3-8B at B = 128 / 256 / 512: 187 -> 167, 355 -> 314,
// 705 -> 638 us; Qwen3-235B at B = 256 / 512: 195 -> 164, 382 -> 325 us); four
// or six wavefronts per CU were 3-8% slower than two, and one wavefront per
// pair sorted longest first was slower still (a CU then receives consecutive,
// equally long items).  With fewer pairs a whole-sequence wavefront bounds the
// call by its sequence's length, so sequences are cut into chunk groups:
// Qwen3-8B at B = 64 / 96: 120 -> 105, 176 -> 135 us; Qwen3-235B at B = 64 /
// 128: 69 -> 63, 129 -> 102 us.  Aiming at 2048 or 4096 groups instead of 1024
// was 5-15% slower.  At 4096 chunk items the two are close (Qwen3-8B B = 32:
// grid 4% faster; Qwen3-235B B = 64: queue 9% faster).
constexpr int64_t kDecodeGridItems = 2048;
constexpr int64_t kDecodeQueueItems = 1024;
constexpr int64_t kDecodeQueueWaves = 512;

struct DecodeQueue {
  int* next;          // the counter
  int* total;         // item count x Hkv, written by decode_order_kernel
  int32_t* item_seq;
  int32_t* item_group;
};

// The queue lives after the chunk records: the records' bytes rounded up to
// 256, then the counter and the count (16 bytes), then two arrays of
// num_seqs * max_chunks int32 (a sequence has at most max_chunks groups).
size_t decode_records_bytes(int64_t num_seqs, int64_t hq, int64_t d, int64_t max_chunks) {
  const size_t bytes = (size_t)num_seqs * (size_t)hq * (size_t)max_chunks * (size_t)(d + 4) * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}
DecodeQueue decode_queue(void* workspace, int num_seqs, int hq, int d, int max_chunks) {
  char* base = static_cast<char*>(workspace) + decode_records_bytes(num_seqs, hq, d, max_chunks);
  DecodeQueue qd;
  qd.next = reinterpret_cast<int*>(base);
  qd.total = qd.next + 1;
  qd.item_seq = reinterpret_cast<int32_t*>(base + 16);
  qd.item_group = qd.item_seq + (int64_t)num_seqs * max_chunks;
  return qd;
}

template <int D, int CS>
hipError_t launch(const void* q, int64_t ld_q, const AttnGeom& g, const int32_t* seq_lens, int num_seqs,
                  int max_seq_len, void* out, float* lse, void* workspace, hipStream_t stream) {
  const int max_chunks = (max_seq_len + CS - 1) / CS;
  float* ws = static_cast<float*>(workspace);
  const auto* qs = static_cast<const uint16_t*>(q);
  const auto* kcs = static_cast<const uint16_t*>(g.k_cache);
  const auto* vcs = static_cast<const uint16_t*>(g.v_cache);
  auto* os = static_cast<uint16_t*>(out);
  const int64_t pairs = (int64_t)num_seqs * g.num_kv_heads;
  const int64_t chunk_items = pairs * max_chunks;
  if (chunk_items <= kDecodeGridItems) {
    hipLaunchKernelGGL((attn_decode_partial_kernel<D, false, CS>), dim3(max_chunks, g.num_kv_heads, num_seqs), dim3(64), 0,
                       stream, qs, ld_q, kcs, vcs, g.num_pages, g.block_table, g.max_pages_per_seq, seq_lens,
                       max_seq_len, g.num_q_heads, g.num_kv_heads, g.log2_page, g.scale_log2, ws, max_chunks, 1, os,
                       lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge<D, CS>(ws, seq_lens, max_seq_len, g.num_q_heads, num_seqs, max_chunks, 1, -1, os, lse, stream);
  }
  int64_t cg = std::min<int64_t>(max_chunks, std::max<int64_t>(1, chunk_items / kDecodeQueueItems));
  auto upper = [&](int64_t c) { return pairs * ((max_chunks + c - 1) / c); };   // items, at most
  while (upper(cg) > INT_MAX / 2 && cg < max_chunks) cg = std::min<int64_t>(max_chunks, 2 * cg);
  if (upper(cg) > INT_MAX / 2) return hipErrorInvalidValue;
  const DecodeQueue qd = decode_queue(workspace, num_seqs, g.num_q_heads, D, max_chunks);
  hipLaunchKernelGGL(decode_order_kernel<CS>, dim3(1), dim3(kOrderThreads), 0, stream, seq_lens, num_seqs, max_seq_len,
                     (int)cg, g.num_kv_heads, qd.item_seq, qd.item_group, qd.next, qd.total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int waves = static_cast<int>(std::min<int64_t>(upper(cg), kDecodeQueueWaves));
  auto queue = cg >= max_chunks ? attn_decode_queue_kernel<D, false, CS> : attn_decode_queue_kernel<D, true, CS>;
  hipLaunchKernelGGL(queue, dim3(waves), dim3(64), 0, stream, qs, ld_q, kcs, vcs, g.num_pages, g.block_table,
                     g.max_pages_per_seq, seq_lens, max_seq_len, g.num_q_heads, g.num_kv_heads, g.log2_page,
                     g.scale_log2, ws, max_chunks, (int)cg, os, lse, qd.item_seq, qd.item_group, qd.next, qd.total);
  e = hipGetLastError();
  if (e != hipSuccess || cg >= max_chunks) return e;
  return launch_merge<D, CS>(ws, seq_lens, max_seq_len, g.num_q_heads, num_seqs, max_chunks, (int)cg, (int)cg, os, lse,
                         stream);
}


// Workspace bytes of launch<D, CS>: the chunk records, then the queue.
inline size_t decode_workspace_bytes_cs(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim,
                                        int64_t max_seq_len, int64_t cs) {
  const int64_t chunks = max_seq_len > 0 ? (max_seq_len + cs - 1) / cs : 1;
  const size_t bytes = decode_records_bytes(num_seqs, num_q_heads, head_dim, chunks) + 16 +
                       2 * sizeof(int32_t) * (size_t)num_seqs * (size_t)chunks;
  return (bytes + 255) & ~(size_t)255;
}

}  // namespace
}  // namespace bi
