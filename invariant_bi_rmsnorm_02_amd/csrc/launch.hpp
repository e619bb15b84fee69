// Host-side launchers, one per kernel family.  Arguments have already been
// validated by the C-ABI layer (api.cpp); launchers only shape grids and
// enqueue on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bi {

hipError_t launch_rmsnorm(const void* x, int64_t ldx, const void* gamma, float eps, void* y,
                          int64_t ldy, int64_t rows, int hidden, hipStream_t stream);

// False when the tile count or a workgroup's buffer offsets would overflow.
bool gemm_supported(int64_t lda, int64_t ldw, int64_t m, int64_t n, int64_t k);
// The output tile (n x m) bi_gemm's rule picks for these arguments.
// bi_gemm's configuration for a shape: tile n, tile m, wavefronts n, m, stages, K per stage, per CU,
// non-temporal weight loads (0 / 1).
void gemm_config_of(int64_t lda, int64_t ldw, int64_t m, int64_t n, int64_t k, int out[8]);

hipError_t launch_gemm(const void* a, int64_t lda, const void* w, int64_t ldw, void* c, int64_t ldc,
                       bool c_f32, int64_t m, int64_t n, int64_t k, hipStream_t stream);

// bi_gemm with a residual add / the gated activation in the epilogue
// (gemm_fused.hip); same tile rule and support test as bi_gemm (for
// launch_gemm_silu_mul with n = 2 f).
hipError_t launch_gemm_add(const void* a, int64_t lda, const void* w, int64_t ldw, const void* x, int64_t ldx,
                           void* y, int64_t ldy, int64_t m, int64_t n, int64_t k, hipStream_t stream);
hipError_t launch_gemm_silu_mul(const void* a, int64_t lda, const void* w, int64_t ldw, void* out, int64_t ldo,
                                int64_t m, int64_t f, int64_t k, hipStream_t stream);

hipError_t launch_kv_append(const void* k_new, const void* v_new, int64_t ld_new, const int32_t* slot_mapping,
                            int num_tokens, void* k_cache, void* v_cache, int num_pages,
                            int num_kv_heads, int head_dim, int page_size, hipStream_t stream);

struct AttnGeom {
  const void* k_cache;
  const void* v_cache;
  int num_pages;
  const int32_t* block_table;
  int max_pages_per_seq;
  int num_q_heads;
  int num_kv_heads;
  int head_dim;
  int log2_page;
  float scale_log2;  // softmax_scale * log2(e)
};

// Bytes of workspace bi_attn_decode needs: the per-(sequence, q head, chunk)
// records and the work queue (attn_decode.hip).
size_t attn_decode_workspace_bytes(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim, int64_t max_seq_len);

hipError_t launch_attn_decode(const void* q, int64_t ld_q, const AttnGeom& g, const int32_t* seq_lens, int num_seqs,
                              int max_seq_len, void* out, float* lse, void* workspace,
                              hipStream_t stream);

// The device address and size of this device's fixed decode scratch array
// (scratch.hip).  Looked up once per device (hipGetSymbolAddress, with the
// device current); the stream must belong to the current device.
hipError_t decode_scratch(hipStream_t stream, void** ptr, size_t* bytes);

// Bytes of the optional prefill workspace (the placement order table).
size_t attn_prefill_workspace_bytes(int64_t num_seqs);

hipError_t launch_attn_prefill(const void* q, int64_t ld_q, const int32_t* q_start, const int32_t* ctx_lens,
                               int num_seqs, int max_q_len, const AttnGeom& g, void* out, float* lse,
                               void* workspace, hipStream_t stream);

// Mixture-of-experts FFN (moe.hip).
size_t moe_workspace_bytes(int64_t T, int64_t top_k, int64_t E, int64_t H, int64_t F);
bool moe_supported(int64_t T, int64_t ldx, int64_t top_k, int64_t E, int64_t H, int64_t F);
hipError_t launch_moe_ffn(const void* x, int64_t ldx, const int32_t* expert_ids, const float* expert_weights,
                          int T, int top_k, int E, const void* w_up, const void* w_down, int H, int F, void* y,
                          int64_t ldy, void* workspace, hipStream_t stream);

// Router of the MoE layer: fp32 logits with the library GEMM, then the top-k
// experts and their softmax weights per token (moe.hip).
hipError_t launch_moe_route(const void* x, int64_t ldx, const void* w_gate, int T, int H, int E, int top_k,
                            float* logits, int32_t* expert_ids, float* expert_weights, hipStream_t stream);

// lm_head + log_softmax fused into the GEMM epilogue (lm_head.hip).  False
// when the tile count or a workgroup's buffer offsets would overflow.
bool lm_head_supported(int64_t lda, int64_t ldw, int64_t m, int64_t n, int64_t k);
size_t lm_head_workspace_bytes(int64_t m, int64_t n);
size_t lm_head_greedy_workspace_bytes(int64_t m, int64_t n);
// Elementwise steps of the decoder layer (pointwise.hip).
hipError_t launch_add(const void* x, int64_t ldx, const void* y, int64_t ldy, void* out, int64_t ldo, int64_t rows,
                      int64_t cols, hipStream_t stream);
hipError_t launch_silu_mul(const void* gu, int64_t ldgu, void* out, int64_t ldo, int64_t rows, int64_t f,
                           hipStream_t stream);
hipError_t launch_lm_head_greedy(const void* a, int64_t lda, const void* w, int64_t ldw, int32_t* token,
                                 float* logprob, int64_t m, int64_t n, int64_t k, void* workspace,
                                 hipStream_t stream);
hipError_t launch_lm_head_logprobs(const void* a, int64_t lda, const void* w, int64_t ldw, float* out, int64_t ldo,
                                   float* lse, int64_t m, int64_t n, int64_t k, void* workspace,
                                   hipStream_t stream);

hipError_t launch_log_softmax(const float* logits, int64_t ld_in, float* out, int64_t ld_out,
                              int64_t rows, int64_t vocab, hipStream_t stream);

}  // namespace bi
