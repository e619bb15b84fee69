/*
 * bi.h - batch-invariant forward-pass kernels for AMD Instinct MI355X (gfx950).
 *
 * Every entry point computes each output row with a reduction order that is a
 * function of that row's own data and of the problem's feature sizes only: it
 * does not depend on the batch size, on the row's position in the batch, on
 * which other requests share the launch, or on how many query tokens of a
 * sequence are in flight.  Sources (web pages):
 *   [TML]  "Thinking Machines Lab - Defeating Nondeterminism in LLM Inference:
 *          The Core Role of Batch Invariance" (jasonandjarvis.org), sections
 *          "1. Batch-Invariant RMSNorm", "2. Batch-Invariant Matrix
 *          Multiplication", "3. Batch-Invariant Attention".
 *   [BINR] "Batch Invariance and Numerical Reproducibility" (praveentn.live),
 *          answers on fixed-size chunks and on sampler/trainer logprobs.
 *   [HADA] "Como superar a não determinismo na inferência de LLMs"
 *          (pt.news.hada.io), "Projeto de kernels invariantes a batch", Attention.
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises; each call enqueues its kernels on
 *     `stream` (a hipStream_t; NULL means the default stream) and returns.
 *   - bf16 is IEEE bfloat16 stored as 16-bit words; results are rounded to it
 *     once, round-to-nearest-even.  Accumulation is fp32.
 *   - Arguments are validated on the host before anything is launched; on a
 *     negative status nothing was enqueued and no output was touched.
 *     BI_ERR_HIP reports a failed launch (hipGetLastError after the launch).
 *   - No global mutable state: calls are thread-safe.  No environment variable,
 *     flag or tuning table changes the arithmetic.
 *   - Input pointers must be 16-byte aligned and input leading dimensions (in
 *     elements) multiples of 8, so rows can be moved in 16-byte vectors.
 */
#ifndef BI_H
#define BI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t bi_status;
#define BI_OK 0
#define BI_ERR_INVALID_ARG (-1) /* null pointer, bad size, stride or alignment */
#define BI_ERR_UNSUPPORTED (-2) /* a size the kernels are not built for      */
#define BI_ERR_WORKSPACE (-3)   /* workspace missing or too small             */
#define BI_ERR_HIP (-4)         /* the HIP runtime reported a launch failure  */

/* Fixed split size of the split-KV reduction, in tokens ([BINR] fixed-size
 * chunks: a 1,000-token cache is 256 + 256 + 256 + 232). */
#define BI_KV_CHUNK 256

typedef enum { BI_BF16 = 0, BI_F32 = 1 } bi_dtype;

typedef void* bi_stream_t; /* a hipStream_t */

/* Text for a status code (static storage; never NULL). */
const char* bi_status_str(bi_status status);

/* Library version as "major.minor.patch" (static storage). */
const char* bi_version(void);

/*
 * RMSNorm ([TML] "1. Batch-Invariant RMSNorm", fig. "Data-Parallel RMSNorm").
 *   y[r, j] = bf16( x[r, j] * (mean_j x[r, j]^2 + eps)^(-1/2) * gamma[j] )
 * x: [rows, hidden] bf16, row stride ldx; gamma: [hidden] bf16;
 * y: [rows, hidden] bf16, row stride ldy (may alias x when ldy == ldx).
 * One workgroup owns one row and reduces it in one fixed order (per-thread
 * sums, a fixed wavefront butterfly, a fixed sum over waves), whatever `rows`.
 * hidden: 8 <= hidden <= 16384, hidden % 8 == 0.  rows == 0 is a no-op.
 */
bi_status bi_rmsnorm(const void* x, int64_t ldx, const void* gamma, float eps,
                     void* y, int64_t ldy, int64_t rows, int64_t hidden, bi_stream_t stream);

/*
 * GEMM ([TML] "2. Batch-Invariant Matrix Multiplication", figs. "Data-Parallel
 * Matrix Multiplication" and "Split-K Matmul").
 *   C[m, n] = sum_k A[m, k] * W[n, k]       (C = A W^T, W stored [N, K] as in
 *                                            a linear layer's weight)
 * a: [m, k] bf16, row stride lda; w: [n, k] bf16, row stride ldw;
 * c: [m, n] of c_dtype (BI_BF16 or BI_F32), row stride ldc >= n (any value;
 *    c aligned to its element size; ldc % 4 == 0 with a 16-byte-aligned c lets
 *    the epilogue use vector stores, which does not change any value).
 * One MFMA instruction and one ascending K loop with a single fp32
 * accumulator per output element, for every m: no split-K, so row m of C does
 * not depend on the other rows of A.  Every output tile gives every element
 * the same bits, so the tile only sets the speed; it is chosen from the
 * shape (n x m, first rule that applies):
 *   n >= 32768 (a vocabulary-sized weight): 256 x 256 from m >= 512, else
 *     128 x 256 (with non-temporal weight loads up to m = 256);
 *   m <= 32 and n >= 16384: 32 x 64;
 *   otherwise, of twenty-one configurations (tiles from 256 x 256 down to
 *     16 x 64 and 32 x 16), the one whose grid is estimated to finish first,
 *     from the workgroups its busiest compute unit runs and per-round costs
 *     measured on MI355X (bi_gemm_tile reports the choice).  When k is a
 *     multiple of 64 but not of 128, tiles with 128-wide K stages are left
 *     out, so that an exact zero gets the same sign from every candidate.
 * A tile of at most 64 rows that holds all m rows reads the weight with
 * non-temporal loads (each weight row is read once).
 * (A tile is passed over for the next candidate when its operand offsets
 * would not fit, below.)
 * k % 32 == 0; m, n >= 0 (m == 0 or n == 0 is a no-op); k >= 32.
 * BI_ERR_UNSUPPORTED when the chosen tile's slice of A or W spans 2^31 bytes
 * or more ((rows - 1) * ld + k >= 2^30 elements, rows = the tile's m or n
 * extent) or the tile count overflows 32 bits.
 */
bi_status bi_gemm(const void* a, int64_t lda, const void* w, int64_t ldw,
                  void* c, int64_t ldc, int32_t c_dtype,
                  int64_t m, int64_t n, int64_t k, bi_stream_t stream);

/*
 * The kernel configuration bi_gemm (and bi_gemm_add, bi_gemm_silu_mul with
 * n = 2f) runs for these arguments on the current device: an output tile of
 * tile_n weight rows by tile_m rows of A, waves_n x waves_m wavefronts, an LDS
 * ring of `stages` stages of stage_k values of K, aimed at per_cu workgroups
 * per compute unit; stream_w = 1 when the weight loads are marked
 * non-temporal (when one m-tile holds all m rows: tiles of at most 64 rows,
 * and the 128 x 256 tile of vocabulary-sized weights).  It
 * changes no result bit; tests use it to reach every configuration.
 * Host-only, no GPU work.  BI_ERR_INVALID_ARG for a null pointer, m, n or
 * k <= 0, or lda, ldw < k.
 */
typedef struct {
  int32_t tile_n, tile_m, waves_n, waves_m, stages, stage_k, per_cu, stream_w;
} bi_gemm_config;
bi_status bi_gemm_tile(int64_t lda, int64_t ldw, int64_t m, int64_t n, int64_t k, bi_gemm_config* config);

/*
 * GEMM with the residual add in its epilogue (the O and down projections of a
 * decoder layer; [TML] "2. Batch-Invariant Matrix Multiplication" for the
 * product, "Achieving Batch-Invariant Kernels" for the elementwise step):
 *   y[m, n] = bf16( x[m, n] + bf16( sum_k A[m, k] * W[n, k] ) )
 * bit for bit bi_gemm (bf16 output) followed by bi_add, without the
 * intermediate product in memory.  a, w, m, n, k and the tile rule: as bi_gemm.
 * x, y: [m, n] bf16, row strides ldx, ldy (>= n, multiples of 8), 16-byte
 * aligned; y may be x itself (ldy == ldx: the in-place residual), other
 * overlaps are not allowed.
 * Errors: those of bi_gemm, and BI_ERR_INVALID_ARG for x or y.  m == 0 or
 * n == 0 is a no-op.
 */
bi_status bi_gemm_add(const void* a, int64_t lda, const void* w, int64_t ldw, const void* x, int64_t ldx,
                      void* y, int64_t ldy, int64_t m, int64_t n, int64_t k, bi_stream_t stream);

/*
 * GEMM with the gated activation in its epilogue (the gate/up projection of a
 * decoder layer's MLP).  w_gate_up: [2f, k] bf16 holding the gate and up rows
 * interleaved: row 2j is gate row j, row 2j + 1 is up row j.
 *   out[m, j] = bf16( silu(g) * u ),  g = bf16( sum_k A[m, k] * w[2j, k] ),
 *                                     u = bf16( sum_k A[m, k] * w[2j + 1, k] )
 * bit for bit bi_gemm on the [gate; up] weight followed by bi_silu_mul (every
 * GEMM output element is the same function of its own A row and W row, so
 * where a W row sits changes no bit).  a, m, k and the tile rule: as bi_gemm
 * with n = 2f.  out: [m, f] bf16, row stride ldo (>= f, a multiple of 8),
 * 16-byte aligned.  f <= 2^29.
 * Errors: those of bi_gemm, and BI_ERR_INVALID_ARG for out.  m == 0 or f == 0
 * is a no-op.
 */
bi_status bi_gemm_silu_mul(const void* a, int64_t lda, const void* w_gate_up, int64_t ldw, void* out, int64_t ldo,
                           int64_t m, int64_t f, int64_t k, bi_stream_t stream);

/*
 * Paged KV cache layout (one pool per layer; page = `page_size` tokens, a
 * multiple of 16).  Both caches are [num_pages][num_kv_heads][page block] bf16;
 * a page block holds page_size / 16 tiles of 16 tokens, one after the other,
 * and a tile holds 16 * head_dim elements laid out so that the attention
 * kernels read every matrix-core operand as whole, contiguous 128-byte lines:
 *   K tile: element (token j, dim d) at (d / 8) * 128 + slot(j) * 8 + d % 8,
 *           slot(j) = 8 * ((j / 4) % 2) + 4 * (j / 8) + j % 4
 *           (tokens 0-3, 8-11 fill the first 128 bytes of each 8-dim group,
 *           tokens 4-7, 12-15 the second);
 *   V tile: element (token j, dim d) at (d / 16) * 256 + (j / 8) * 128
 *           + (d % 16) * 8 + j % 8.
 * Token t of a sequence lives in page block_table[seq][t / page_size], tile
 * (t % page_size) / 16, token t % 16 of that tile.  Cached and newly appended
 * tokens share this one layout ([HADA] Attention: keep a consistent K/V
 * layout; [TML] fig. "FlashAttention with KV Cache").  Only the library's own
 * kernels write it (bi_kv_append).
 */

/*
 * KV append: write new keys/values into their cache slots before attention.
 * k_new, v_new: [num_tokens][num_kv_heads][head_dim] bf16, heads and dims
 *   contiguous, consecutive tokens ld_new elements apart (ld_new >= Hkv * D,
 *   ld_new % 8 == 0; e.g. the K and V columns of a fused QKV projection);
 * slot_mapping: [num_tokens] int32, slot = page * page_size + offset; a negative
 * slot or one >= num_pages * page_size skips that token (padding).
 * A pure copy: every cache element is written bit-exactly.
 * head_dim in {64, 128}; page_size in {16, 32, 64, 128, 256}.
 */
bi_status bi_kv_append(const void* k_new, const void* v_new, int64_t ld_new, const int32_t* slot_mapping,
                       int32_t num_tokens, void* k_cache, void* v_cache, int32_t num_pages,
                       int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                       bi_stream_t stream);

/*
 * Workspace for bi_attn_decode: per (sequence, q head, chunk) partial results
 * (reference max, sum, D accumulators), fp32: num_seqs * num_q_heads * ceil(max_seq_len/256)
 * * (head_dim + 4) * 4 bytes (accumulators, max, sum, 2 pad words per
 * record), rounded up to 256 bytes; then the work queue: 16 bytes plus
 * 2 * num_seqs * ceil(max_seq_len/256) int32; the total rounded up to 256 bytes.
 */
size_t bi_attn_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                      int32_t max_seq_len);

/*
 * Decode attention over the paged cache, one query token per sequence
 * ([TML] "3. Batch-Invariant Attention", figs. "Fixed Number Split KV Strategy"
 * and "Fixed Size Split KV Strategy"; [BINR] fixed-size chunks).
 *   For q head h, kv head g = h / (num_q_heads / num_kv_heads):
 *   s_j = softmax_scale * <q[b, h], K_b[j, g]>,  j < L_b = seq_lens[b]
 *   out[b, h] = bf16( sum_j softmax(s)_j V_b[j, g] ),  lse[b, h] = log sum_j exp(s_j)
 * The keys are split into fixed 256-token chunks anchored at position 0 (only
 * the last is partial); each chunk yields (m, sum, accumulators) with the sum
 * and accumulators taken relative to a reference m that is raised only when a
 * score passes it by more than 8 in log2 units (so true max - 8 <= m <= true
 * max), and the chunks are merged in ascending order, starting from
 * (-inf, 0, 0), by a log-sum-exp step with the same lazy reference.  In exact
 * arithmetic this is the softmax; the chunking depends on nothing but L_b.
 * q: [num_seqs][num_q_heads][head_dim] bf16, consecutive sequences ld_q
 *   elements apart (ld_q >= Hq * D, ld_q % 8 == 0); out: contiguous
 *   [num_seqs][num_q_heads][head_dim] bf16;
 * lse: [num_seqs][num_q_heads] fp32 or NULL (natural log).
 * block_table: [num_seqs][max_pages_per_seq] int32; seq_lens: [num_seqs] int32.
 * max_seq_len: host-side upper bound of seq_lens (sizes the grid; a seq_len
 * above it is clamped to it).  Page ids outside [0, num_pages) read as zeros.
 * A sequence with seq_len <= 0 gets out = 0 and lse = -inf.
 * workspace: >= bi_attn_decode_workspace_bytes(...) bytes of device memory,
 *   16-byte aligned, owned by the caller; its contents on entry do not
 *   matter.  It holds the chunk partials (or a fold of a sequence's first
 *   chunks in chunk 0's record) and the work queue's items and counter.
 *   Concurrent calls need separate workspaces.  num_seqs * num_kv_heads
 *   <= 2^29 (else BI_ERR_UNSUPPORTED).
 * head_dim in {64, 128}; num_q_heads % num_kv_heads == 0 and the group size
 * num_q_heads / num_kv_heads in {1, 2, 4, 8, 16}; page_size in {16, 32, 64, 128, 256}.
 */
bi_status bi_attn_decode(const void* q, int64_t ld_q, const void* k_cache, const void* v_cache, int32_t num_pages,
                         const int32_t* block_table, int32_t max_pages_per_seq,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t page_size, float softmax_scale, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, bi_stream_t stream);

/*
 * Size of the fixed decode scratch array of bi_attn_decode_noalloc: 128 MiB
 * per GPU the library runs on (e.g. the Qwen3-8B-shaped decode at 256
 * sequences of up to 4096 tokens needs 69 MB of it).
 */
#define BI_DECODE_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * Decode attention that allocates nothing, for callers that cannot allocate
 * or pass device memory of their own for a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Arguments,
 * results and status codes are those of bi_attn_decode without the workspace;
 * the kernels and their arithmetic are the same, so the outputs are bitwise
 * equal to bi_attn_decode's.  The workspace is a fixed device array of
 * BI_DECODE_SCRATCH_BYTES inside the library (one per GPU, held from when the
 * library's code is loaded on that GPU until the process ends); its address
 * is looked up once per device, on the first call with that device current.
 *   BI_ERR_WORKSPACE when bi_attn_decode_workspace_bytes(num_seqs,
 *   num_q_heads, head_dim, max_seq_len) exceeds BI_DECODE_SCRATCH_BYTES
 *   (nothing is enqueued); BI_ERR_HIP when the stream does not belong to the
 *   current device or the lookup fails.
 * Every call on one GPU uses that GPU's one array: calls that can overlap on
 * a GPU (several streams, several host threads) race and must be ordered by
 * the caller.  The array keeps what the last call left; no call needs it
 * cleared (the work-queue counter is written by the call's first kernel).
 */
bi_status bi_attn_decode_noalloc(const void* q, int64_t ld_q, const void* k_cache, const void* v_cache,
                                 int32_t num_pages, const int32_t* block_table, int32_t max_pages_per_seq,
                                 const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                 float softmax_scale, void* out, float* lse, bi_stream_t stream);

/*
 * Chunked-prefill attention over the paged cache ([TML] "3. Batch-Invariant
 * Attention", figs. "FlashAttention2 Strategy" and "FlashAttention with KV
 * Cache"; [HADA] Attention).  Sequence s has ctx_lens[s] cached tokens and a
 * chunk of n_s = q_start[s+1] - q_start[s] new tokens whose K/V were ALREADY
 * written to the cache (bi_kv_append) at positions ctx_lens[s] .. ctx_lens[s]+n_s-1.
 * Query i of sequence s sits at position p = ctx_lens[s] + i and attends keys
 * 0..p (causal, inclusive).  Each query row is reduced with exactly the chunk
 * routine and merge step of bi_attn_decode, so a prefilled row is bitwise equal
 * to decoding the same token with seq_len = p + 1.
 * q: [q_start[num_seqs]][num_q_heads][head_dim] bf16, consecutive tokens ld_q
 * elements apart; out: contiguous, same shape; lse: [..][num_q_heads]
 * fp32 or NULL.  q_start: [num_seqs + 1] int32, non-decreasing from 0;
 * ctx_lens: [num_seqs] int32.  max_q_len: host-side upper bound of n_s (sizes
 * the grid; longer chunks are clamped to it).  Same size limits as decode.
 * workspace: NULL, or at least bi_attn_prefill_workspace_bytes(num_seqs)
 *   bytes of device memory, 16-byte aligned, owned by the caller, contents on
 *   entry irrelevant (else BI_ERR_WORKSPACE).  With it and more than 16
 *   sequences, a small kernel first ranks the sequences (longest last key
 *   first) into a table the attention workgroups read to place their work;
 *   otherwise every workgroup ranks the sequences itself (num_seqs^2 / 64
 *   steps each - fine for a few sequences, costly for hundreds).  Placement
 *   only: the results are the same bits either way.  Concurrent calls need
 *   separate workspaces.
 */
size_t bi_attn_prefill_workspace_bytes(int32_t num_seqs);
bi_status bi_attn_prefill(const void* q, int64_t ld_q, const int32_t* q_start, const int32_t* ctx_lens,
                          int32_t num_seqs, int32_t max_q_len,
                          const void* k_cache, const void* v_cache, int32_t num_pages,
                          const int32_t* block_table, int32_t max_pages_per_seq,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t page_size, float softmax_scale, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, bi_stream_t stream);

/*
 * Mixture-of-experts FFN over a batch of tokens (the routed expert layer of the
 * Qwen3-235B-A22B-shaped workload; the expert FFN is not on the pages).  The
 * invariance rule is [BINR]'s answer on a fixed per-element reduction order,
 * one that neither the batch's size nor a row's place in it may change: a
 * token's output depends
 * only on its own x row, routing and the weights, never on which other tokens
 * share its experts.
 *   y[t] = bf16( sum over s = 0 .. top_k-1 ascending, in fp32, of
 *                w[t, s] * W_down[e] h ),  h = bf16(SiLU(W_up[e] x[t])),
 *          e = expert_ids[t, s],  SiLU(v) = v / (1 + exp(-v)).
 * Both expert products are bi_gemm's configuration and K loop (one fp32
 * accumulator per element, k ascending); the W_down product stays fp32 until
 * the weighted sum.
 * x: [num_tokens, hidden] bf16, row stride ldx (ldx % 8 == 0);
 * expert_ids: [num_tokens, top_k] int32, contiguous; an id outside
 *   [0, num_experts) drops that slot;
 * expert_weights: [num_tokens, top_k] fp32, contiguous;
 * w_up: [num_experts][ffn][hidden] bf16; w_down: [num_experts][hidden][ffn] bf16;
 * y: [num_tokens, hidden] bf16, row stride ldy (ldy % 8 == 0), must not alias x.
 * hidden, ffn: multiples of 32, at most 65536; 1 <= top_k <= 64;
 * 1 <= num_experts <= 65535; num_tokens == 0 is a no-op.  BI_ERR_UNSUPPORTED
 * when num_tokens * top_k > 2^24 or x spans 2^31 bytes or more.
 * workspace: at least bi_moe_workspace_bytes(...) bytes, 256-byte aligned, owned
 * by the caller (routing tables, the bf16 intermediate and the fp32 per-slot
 * outputs; about num_tokens * top_k * (2 * ffn + 4 * hidden) bytes); else
 * BI_ERR_WORKSPACE.
 */
/*
 * Router of the mixture-of-experts layer (workload support, the Qwen3-235B-
 * A22B-shaped layer: 128 experts, top-8; routing is not on the pages, and the
 * invariance rule is [BINR]'s answer on a fixed per-element reduction order,
 * one that neither the batch's size nor a row's place in it may change).
 *   logits[t, e]         = sum_k x[t, k] w_gate[e, k]      (bi_gemm, fp32 out)
 *   expert_ids[t, s]     = the s-th expert in the order: larger logit first,
 *                          lower expert index first among equal logits (a NaN
 *                          logit counts below every number), s < top_k
 *   expert_weights[t, s] = e_s / sum_{j < top_k} e_j,  e_s = exp(l_s - l_0),
 *                          l_s the logit of expert_ids[t, s], the sum in fp32
 *                          in slot order
 * The order is total, so the choice is a function of the token's logits alone
 * (and those are bi_gemm's, batch-invariant); the slot order is the order
 * bi_moe_ffn sums the experts in.
 * x: [num_tokens, hidden] bf16, row stride ldx (ldx % 8 == 0, 16-byte aligned);
 * w_gate: [num_experts, hidden] bf16, contiguous, 16-byte aligned;
 * logits: [num_tokens, num_experts] fp32, contiguous (written);
 * expert_ids: [num_tokens, top_k] int32 and expert_weights: [num_tokens, top_k]
 *   fp32, contiguous.  All outputs are owned by the caller.
 * 1 <= top_k <= num_experts (else BI_ERR_INVALID_ARG); top_k <= 64,
 * num_experts <= 1024 and hidden % 32 == 0 (else BI_ERR_UNSUPPORTED);
 * num_tokens == 0 is a no-op.
 */
bi_status bi_moe_route(const void* x, int64_t ldx, const void* w_gate, int32_t num_tokens, int32_t hidden,
                       int32_t num_experts, int32_t top_k, float* logits, int32_t* expert_ids, float* expert_weights,
                       bi_stream_t stream);

size_t bi_moe_workspace_bytes(int32_t num_tokens, int32_t top_k, int32_t num_experts,
                              int32_t hidden, int32_t ffn);
bi_status bi_moe_ffn(const void* x, int64_t ldx, const int32_t* expert_ids, const float* expert_weights,
                     int32_t num_tokens, int32_t top_k, int32_t num_experts,
                     const void* w_up, const void* w_down, int32_t hidden, int32_t ffn,
                     void* y, int64_t ldy, void* workspace, size_t workspace_bytes, bi_stream_t stream);

/*
 * Row-wise log_softmax of fp32 logits ([BINR] answer on sampler/trainer
 * logprob agreement).  out[r, j] = z[r, j] - (max_j z + log sum_j exp(z - max)).
 * One workgroup per row, one fixed reduction tree whatever `rows`.
 * logits: [rows, vocab] fp32, row stride ld_in; out: [rows, vocab] fp32, row
 * stride ld_out (may alias logits when strides are equal). vocab >= 1,
 * vocab % 4 == 0, strides multiples of 4.
 */
bi_status bi_log_softmax(const float* logits, int64_t ld_in, float* out, int64_t ld_out,
                         int64_t rows, int64_t vocab, bi_stream_t stream);

/*
 * lm_head followed by log_softmax, the reduction fused into the GEMM's
 * epilogue ([BINR] answer on sampler/trainer logprob agreement; the product is
 * bi_gemm's, [TML] section "2. Batch-Invariant Matrix Multiplication").
 *   z[i, j]   = sum_k a[i, k] w[j, k]        (bi_gemm's tile and fp32 K chain)
 *   out[i, j] = z[i, j] - lse[i],  lse[i] = log sum_j exp(z[i, j])
 * lse is reduced in one fixed tree that depends on n only: (max, sum of exp)
 * pairs over the GEMM's n-tiles (64 columns when n < 32768, 128 from 32768 on),
 * folded in ascending tile order.  It is not
 * bi_log_softmax's tree, so the two agree to rounding, not bit for bit; each
 * is batch-invariant on its own.
 * a: [m, k] bf16, row stride lda; w: [n, k] bf16, row stride ldw (k % 32 == 0,
 *   strides multiples of 8, both 16-byte aligned);
 * out: [m, n] fp32 logprobs, row stride ldo >= n, ldo % 4 == 0, 16-byte
 *   aligned; n % 4 == 0; z is staged in out, so out must not overlap a or w;
 * lse: [m] fp32 or NULL;
 * workspace: device memory of at least
 *   bi_lm_head_logprobs_workspace_bytes(m, n) bytes (the tile pairs), 256-byte
 *   aligned, owned by the caller; its contents on entry do not matter.
 * Errors: BI_ERR_INVALID_ARG (sizes, strides, alignment), BI_ERR_UNSUPPORTED
 * (k % 32, n % 4, sizes beyond the GEMM's offset limits), BI_ERR_WORKSPACE
 * (missing, misaligned or short workspace).  Nothing is written on error.
 */
size_t bi_lm_head_logprobs_workspace_bytes(int64_t m, int64_t n);
bi_status bi_lm_head_logprobs(const void* a, int64_t lda, const void* w, int64_t ldw, float* out, int64_t ldo,
                              float* lse, int64_t m, int64_t n, int64_t k, void* workspace, size_t workspace_bytes,
                              bi_stream_t stream);

/*
 * Greedy sampling from the lm_head without materialising the logits ([BINR]
 * answers on sampler/trainer agreement: the sampled token and its logprob
 * must not depend on the batch).
 *   z[i, j]      = sum_k a[i, k] w[j, k]            (as in bi_lm_head_logprobs)
 *   token[i]     = the lowest j with z[i, j] = max_j z[i, j]
 *   logprob[i]   = z[i, token[i]] - lse[i]
 * The (max, sum of exp) pairs of every n-tile are formed and folded exactly
 * as in bi_lm_head_logprobs, with the column of each maximum carried
 * along (ties go to the lower index, which makes the choice independent of
 * the combination order), so logprob[i] is bitwise bi_lm_head_logprobs'
 * out[i, token[i]].  No [m, n] buffer is read or written.
 * a, w: as in bi_lm_head_logprobs (n need not be a multiple of 4);
 * token: [m] int32, 4-byte aligned; logprob: [m] fp32 or NULL;
 * workspace: device memory of at least bi_lm_head_greedy_workspace_bytes(m, n)
 *   bytes, 256-byte aligned, owned by the caller; its contents on entry do not
 *   matter.
 * Errors: as bi_lm_head_logprobs.  Nothing is written on error.
 */
size_t bi_lm_head_greedy_workspace_bytes(int64_t m, int64_t n);
bi_status bi_lm_head_greedy(const void* a, int64_t lda, const void* w, int64_t ldw, int32_t* token, float* logprob,
                            int64_t m, int64_t n, int64_t k, void* workspace, size_t workspace_bytes,
                            bi_stream_t stream);

/*
 * Elementwise steps of a decoder layer ([TML] section "1. Batch-Invariant
 * RMSNorm" context: only reductions need a batch-independent order; these have
 * none).  Every output element depends on its own input elements only.
 *   bi_add:      out[i, j] = bf16(x[i, j] + y[i, j])   (the residual add; the fp32
 *                sum of two bf16 is exact unless their exponents differ by more
 *                than 16, and then it is far from a bf16 rounding midpoint, so
 *                the result is the correctly rounded exact sum)
 *   bi_silu_mul: out[i, j] = bf16(silu(g) * u), g = gate_up[i, j],
 *                u = gate_up[i, f + j], silu(g) = g / (1 + e^-g), in fp32 with one
 *                rounding (the gated MLP on a fused gate/up projection [T, 2f])
 * All tensors bf16, rows strided (ld* elements, multiples of 8, >= the row's
 * width), 16-byte aligned; cols and f multiples of 8.  bi_add's out may be x or
 * y itself (in place); other overlaps are not allowed.
 * Errors: BI_ERR_INVALID_ARG (pointers, strides, alignment), BI_ERR_UNSUPPORTED
 * (widths not a multiple of 8, rows or widths beyond 2^30, more than 2^34
 * output elements).  Nothing is written on error.
 */
bi_status bi_add(const void* x, int64_t ldx, const void* y, int64_t ldy, void* out, int64_t ldo, int64_t rows,
                 int64_t cols, bi_stream_t stream);
bi_status bi_silu_mul(const void* gate_up, int64_t ld_gu, void* out, int64_t ldo, int64_t rows, int64_t f,
                      bi_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BI_H */
