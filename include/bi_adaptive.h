/*
 * bi_adaptive.h - shape-adaptive comparators of libbi_adaptive.so.
 *
 * These are NOT batch-invariant, on purpose.  They parallelise the same three
 * operations the way a throughput-first library would, reproducing the
 * hazards named in "Thinking Machines Lab - Defeating Nondeterminism in LLM
 * Inference": split-K matmul when the tile count is small (section "2.
 * Batch-Invariant Matrix Multiplication", fig. "Split-K Matmul"), split-KV with
 * a fixed number of splits (section "3. Batch-Invariant Attention", fig. "Fixed
 * Number Split KV Strategy") and split-reduction RMSNorm at small batch
 * (section "1. Batch-Invariant RMSNorm", fig. "Split-Reduction RMSNorm").  They
 * exist to measure the cost of invariance against libbi.so (include/bi.h) and
 * to show that a result's bits then depend on the batch.  Nothing in libbi.so
 * calls them.
 *
 * Conventions are those of bi.h: caller-owned device pointers, work enqueued
 * on `stream`, no allocation or synchronisation, validation before any launch,
 * bi_status results.  Where a heuristic picks "one split", the call runs the
 * libbi.so kernel itself and needs no workspace.
 */
#ifndef BI_ADAPTIVE_H
#define BI_ADAPTIVE_H

#include "bi.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Split-K GEMM, C = A W^T (bf16 out), shapes and strides as bi_gemm.
 * splits = min(ceil(512 / tiles), k / 256) when the 64 x 64 tiles number fewer
 * than 512 (two workgroups per CU), else 1; the K slices are rounded to 128 and
 * summed in slice order in fp32 by a second kernel.  workspace: at least
 * bia_gemm_workspace_bytes(m, n, k) bytes (0 when splits == 1), 16-byte aligned.
 */
int32_t bia_gemm_splits(int64_t m, int64_t n, int64_t k);
size_t bia_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);
bi_status bia_gemm(const void* a, int64_t lda, const void* w, int64_t ldw, void* c, int64_t ldc,
                   int64_t m, int64_t n, int64_t k, void* workspace, size_t workspace_bytes,
                   bi_stream_t stream);

/*
 * Decode attention with the split size chosen from the batch, arguments as
 * bi_attn_decode.  It is libbi.so's decode (the same chunk step, work queue,
 * in-wave fold and merge) with one change: chunks of split_keys keys instead
 * of 256, where S = max(1, ceil(512 / (num_seqs * num_kv_heads))) splits of a
 * max_seq_len-key sequence give ceil(max_seq_len / S) keys, rounded up to a
 * power of two between max(32, page_size) and 512
 * (bia_attn_decode_split_keys).  At 256 keys the result is libbi.so's, bit for
 * bit.  workspace: at least bia_attn_decode_workspace_bytes(...) bytes,
 * 256-byte aligned (BI_ERR_WORKSPACE otherwise).
 */
int32_t bia_attn_decode_split_keys(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len, int32_t page_size);
size_t bia_attn_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_seq_len, int32_t page_size);
bi_status bia_attn_decode(const void* q, int64_t ld_q, const void* k_cache, const void* v_cache,
                          int32_t num_pages, const int32_t* block_table, int32_t max_pages_per_seq,
                          const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t page_size, float softmax_scale, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, bi_stream_t stream);

/*
 * Split-reduction RMSNorm, arguments as bi_rmsnorm.  With fewer than 256 rows
 * each row's sum of squares is cut into min(ceil(256 / rows), hidden / 2048)
 * slices reduced by separate workgroups and added in slice order; otherwise
 * libbi.so's kernel runs.  rows <= 65535.  workspace: at least
 * bia_rmsnorm_workspace_bytes(rows, hidden) bytes.
 */
int32_t bia_rmsnorm_slices(int64_t rows, int64_t hidden);
size_t bia_rmsnorm_workspace_bytes(int64_t rows, int64_t hidden);
bi_status bia_rmsnorm(const void* x, int64_t ldx, const void* gamma, float eps, void* y, int64_t ldy,
                      int64_t rows, int64_t hidden, void* workspace, size_t workspace_bytes,
                      bi_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BI_ADAPTIVE_H */
