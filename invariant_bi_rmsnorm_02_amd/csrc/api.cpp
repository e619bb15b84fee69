// C-ABI entry points declared in include/bi.h: host-side validation, then the
// kernel launchers.  Nothing here allocates, frees or synchronises.  A
// validation failure returns before anything is enqueued.
#include "bi.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "launch.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int log2_exact(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return (1 << l) == v ? l : -1;
}

bi_status from_hip(hipError_t e) { return e == hipSuccess ? BI_OK : BI_ERR_HIP; }

hipStream_t as_stream(bi_stream_t s) { return static_cast<hipStream_t>(s); }

// Common checks of the attention geometry.
bi_status check_attn_geom(const void* k_cache, const void* v_cache, int32_t num_pages,
                          const int32_t* block_table, int32_t max_pages_per_seq,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t page_size, float softmax_scale) {
  if (!k_cache || !v_cache || !block_table) return BI_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return BI_ERR_INVALID_ARG;
  if (num_pages <= 0 || max_pages_per_seq <= 0 || num_q_heads <= 0 || num_kv_heads <= 0)
    return BI_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return BI_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads) return BI_ERR_INVALID_ARG;
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return BI_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return BI_ERR_UNSUPPORTED;
  const int l2 = log2_exact(page_size);
  if (l2 < 4 || l2 > 8) return BI_ERR_UNSUPPORTED;  // 16 .. 256 tokens: whole 16-token tiles, divides the chunk
  return BI_OK;
}

bi::AttnGeom make_geom(const void* k_cache, const void* v_cache, int32_t num_pages,
                       const int32_t* block_table, int32_t max_pages_per_seq, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t page_size, float softmax_scale) {
  bi::AttnGeom g;
  g.k_cache = k_cache;
  g.v_cache = v_cache;
  g.num_pages = num_pages;
  g.block_table = block_table;
  g.max_pages_per_seq = max_pages_per_seq;
  g.num_q_heads = num_q_heads;
  g.num_kv_heads = num_kv_heads;
  g.head_dim = head_dim;
  g.log2_page = log2_exact(page_size);
  // One fp32 rounding of scale * log2(e), done once here for both attention
  // kernels, so decode and prefill scale scores by the same bits.
  g.scale_log2 = static_cast<float>(static_cast<double>(softmax_scale) * 1.4426950408889634);
  return g;
}

// Checks of bi_attn_decode's arguments other than the workspace.
bi_status check_decode(const void* q, int64_t ld_q, const void* k_cache, const void* v_cache, int32_t num_pages,
                       const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
                       int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t page_size, float softmax_scale, const void* out) {
  bi_status st = check_attn_geom(k_cache, v_cache, num_pages, block_table, max_pages_per_seq,
                                 num_q_heads, num_kv_heads, head_dim, page_size, softmax_scale);
  if (st != BI_OK) return st;
  if (!q || !seq_lens || !out) return BI_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out)) return BI_ERR_INVALID_ARG;
  if (ld_q < (int64_t)num_q_heads * head_dim || ld_q % 8) return BI_ERR_INVALID_ARG;
  if (num_seqs > 65535 || num_kv_heads > 65535) return BI_ERR_UNSUPPORTED;  // grid y/z limits
  if ((int64_t)num_seqs * num_kv_heads > (1 << 29)) return BI_ERR_UNSUPPORTED;  // work-queue item count
  return BI_OK;
}

}  // namespace

extern "C" {

const char* bi_status_str(bi_status status) {
  switch (status) {
    case BI_OK: return "ok";
    case BI_ERR_INVALID_ARG: return "invalid argument";
    case BI_ERR_UNSUPPORTED: return "unsupported size";
    case BI_ERR_WORKSPACE: return "workspace missing or too small";
    case BI_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

const char* bi_version(void) { return "0.1.0"; }

bi_status bi_rmsnorm(const void* x, int64_t ldx, const void* gamma, float eps, void* y, int64_t ldy,
                     int64_t rows, int64_t hidden, bi_stream_t stream) {
  if (rows < 0 || hidden <= 0) return BI_ERR_INVALID_ARG;
  if (rows == 0) return BI_OK;
  if (!x || !gamma || !y) return BI_ERR_INVALID_ARG;
  if (hidden % 8 || hidden > 16384) return BI_ERR_UNSUPPORTED;
  if (ldx < hidden || ldy < hidden || ldx % 8 || ldy % 8) return BI_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(y)) return BI_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return BI_ERR_INVALID_ARG;
  if (rows > 0x7fffffff) return BI_ERR_UNSUPPORTED;
  return from_hip(bi::launch_rmsnorm(x, ldx, gamma, eps, y, ldy, rows, static_cast<int>(hidden),
                                     as_stream(stream)));
}

bi_status bi_gemm(const void* a, int64_t lda, const void* w, int64_t ldw, void* c, int64_t ldc,
                  int32_t c_dtype, int64_t m, int64_t n, int64_t k, bi_stream_t stream) {
  if (m < 0 || n < 0 || k <= 0) return BI_ERR_INVALID_ARG;
  if (c_dtype != BI_BF16 && c_dtype != BI_F32) return BI_ERR_INVALID_ARG;
  if (m == 0 || n == 0) return BI_OK;
  if (!a || !w || !c) return BI_ERR_INVALID_ARG;
  if (k % 32) return BI_ERR_UNSUPPORTED;
  if (m > (1 << 30) || n > (1 << 30) || k > (1 << 30)) return BI_ERR_UNSUPPORTED;
  if (lda < k || ldw < k || ldc < n || lda % 8 || ldw % 8) return BI_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(w)) return BI_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(c) % (c_dtype == BI_F32 ? 4u : 2u)) return BI_ERR_INVALID_ARG;
  if (!bi::gemm_supported(lda, ldw, m, n, k)) return BI_ERR_UNSUPPORTED;
  return from_hip(bi::launch_gemm(a, lda, w, ldw, c, ldc, c_dtype == BI_F32, m, n, k, as_stream(stream)));
}

bi_status bi_gemm_tile(int64_t lda, int64_t ldw, int64_t m, int64_t n, int64_t k, bi_gemm_config* config) {
  if (!config || m <= 0 || n <= 0 || k <= 0 || lda < k || ldw < k) return BI_ERR_INVALID_ARG;
  int v[8];
  bi::gemm_config_of(lda, ldw, m, n, k, v);
  *config = bi_gemm_config{v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
  return BI_OK;
}

// The A and W checks of bi_gemm (k, strides, alignment, offset range).
static bi_status check_gemm_operands(const void* a, int64_t lda, const void* w, int64_t ldw, int64_t m, int64_t n,
                                     int64_t k) {
  if (k % 32) return BI_ERR_UNSUPPORTED;
  if (m > (1 << 30) || n > (1 << 30) || k > (1 << 30)) return BI_ERR_UNSUPPORTED;
  if (lda < k || ldw < k || lda % 8 || ldw % 8) return BI_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(w)) return BI_ERR_INVALID_ARG;
  if (!bi::gemm_supported(lda, ldw, m, n, k)) return BI_ERR_UNSUPPORTED;
  return BI_OK;
}

bi_status bi_gemm_add(const void* a, int64_t lda, const void* w, int64_t ldw, const void* x, int64_t ldx, void* y,
                      int64_t ldy, int64_t m, int64_t n, int64_t k, bi_stream_t stream) {
  if (m < 0 || n < 0 || k <= 0) return BI_ERR_INVALID_ARG;
  if (m == 0 || n == 0) return BI_OK;
  if (!a || !w || !x || !y) return BI_ERR_INVALID_ARG;
  if (ldx < n || ldy < n || ldx % 8 || ldy % 8 || !aligned16(x) || !aligned16(y)) return BI_ERR_INVALID_ARG;
  if (x == y && ldx != ldy) return BI_ERR_INVALID_ARG;
  const bi_status st = check_gemm_operands(a, lda, w, ldw, m, n, k);
  if (st != BI_OK) return st;
  return from_hip(bi::launch_gemm_add(a, lda, w, ldw, x, ldx, y, ldy, m, n, k, as_stream(stream)));
}

bi_status bi_gemm_silu_mul(const void* a, int64_t lda, const void* w_gate_up, int64_t ldw, void* out, int64_t ldo,
                           int64_t m, int64_t f, int64_t k, bi_stream_t stream) {
  if (m < 0 || f < 0 || k <= 0) return BI_ERR_INVALID_ARG;
  if (m == 0 || f == 0) return BI_OK;
  if (!a || !w_gate_up || !out) return BI_ERR_INVALID_ARG;
  if (f > (1 << 29)) return BI_ERR_UNSUPPORTED;
  if (ldo < f || ldo % 8 || !aligned16(out)) return BI_ERR_INVALID_ARG;
  const bi_status st = check_gemm_operands(a, lda, w_gate_up, ldw, m, 2 * f, k);
  if (st != BI_OK) return st;
  return from_hip(bi::launch_gemm_silu_mul(a, lda, w_gate_up, ldw, out, ldo, m, f, k, as_stream(stream)));
}

bi_status bi_kv_append(const void* k_new, const void* v_new, int64_t ld_new, const int32_t* slot_mapping,
                       int32_t num_tokens, void* k_cache, void* v_cache, int32_t num_pages,
                       int32_t num_kv_heads, int32_t head_dim, int32_t page_size, bi_stream_t stream) {
  if (num_tokens < 0) return BI_ERR_INVALID_ARG;
  if (num_tokens == 0) return BI_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return BI_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return BI_ERR_INVALID_ARG;
  if (num_pages <= 0 || num_kv_heads <= 0) return BI_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return BI_ERR_UNSUPPORTED;
  const int l2 = log2_exact(page_size);
  if (l2 < 4 || l2 > 8) return BI_ERR_UNSUPPORTED;
  if ((int64_t)num_pages * page_size > 0x7fffffff || num_kv_heads > 65535) return BI_ERR_UNSUPPORTED;
  if (ld_new < (int64_t)num_kv_heads * head_dim || ld_new % 8) return BI_ERR_INVALID_ARG;
  return from_hip(bi::launch_kv_append(k_new, v_new, ld_new, slot_mapping, num_tokens, k_cache, v_cache,
                                       num_pages, num_kv_heads, head_dim, page_size, as_stream(stream)));
}

size_t bi_attn_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                      int32_t max_seq_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  return bi::attn_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_seq_len);
}

bi_status bi_attn_decode(const void* q, int64_t ld_q, const void* k_cache, const void* v_cache, int32_t num_pages,
                         const int32_t* block_table, int32_t max_pages_per_seq,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t page_size, float softmax_scale, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, bi_stream_t stream) {
  if (num_seqs < 0 || max_seq_len < 0) return BI_ERR_INVALID_ARG;
  if (num_seqs == 0) return BI_OK;
  bi_status st = check_decode(q, ld_q, k_cache, v_cache, num_pages, block_table, max_pages_per_seq, seq_lens,
                              num_seqs, num_q_heads, num_kv_heads, head_dim, page_size, softmax_scale, out);
  if (st != BI_OK) return st;
  if (!workspace || !aligned16(workspace)) return BI_ERR_WORKSPACE;
  if (workspace_bytes < bi_attn_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_seq_len))
    return BI_ERR_WORKSPACE;
  const bi::AttnGeom g = make_geom(k_cache, v_cache, num_pages, block_table, max_pages_per_seq,
                                   num_q_heads, num_kv_heads, head_dim, page_size, softmax_scale);
  return from_hip(bi::launch_attn_decode(q, ld_q, g, seq_lens, num_seqs, max_seq_len, out, lse, workspace,
                                         as_stream(stream)));
}

bi_status bi_attn_decode_noalloc(const void* q, int64_t ld_q, const void* k_cache, const void* v_cache,
                                 int32_t num_pages, const int32_t* block_table, int32_t max_pages_per_seq,
                                 const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                 float softmax_scale, void* out, float* lse, bi_stream_t stream) {
  if (num_seqs < 0 || max_seq_len < 0) return BI_ERR_INVALID_ARG;
  if (num_seqs == 0) return BI_OK;
  bi_status st = check_decode(q, ld_q, k_cache, v_cache, num_pages, block_table, max_pages_per_seq, seq_lens,
                              num_seqs, num_q_heads, num_kv_heads, head_dim, page_size, softmax_scale, out);
  if (st != BI_OK) return st;
  if (bi_attn_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_seq_len) > BI_DECODE_SCRATCH_BYTES)
    return BI_ERR_WORKSPACE;
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  if (bi::decode_scratch(as_stream(stream), &scratch, &scratch_bytes) != hipSuccess) return BI_ERR_HIP;
  return bi_attn_decode(q, ld_q, k_cache, v_cache, num_pages, block_table, max_pages_per_seq, seq_lens, num_seqs,
                        max_seq_len, num_q_heads, num_kv_heads, head_dim, page_size, softmax_scale, out, lse,
                        scratch, scratch_bytes, stream);
}

bi_status bi_attn_prefill(const void* q, int64_t ld_q, const int32_t* q_start, const int32_t* ctx_lens,
                          int32_t num_seqs, int32_t max_q_len, const void* k_cache, const void* v_cache,
                          int32_t num_pages, const int32_t* block_table, int32_t max_pages_per_seq,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t page_size, float softmax_scale, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, bi_stream_t stream) {
  if (num_seqs < 0 || max_q_len < 0) return BI_ERR_INVALID_ARG;
  if (num_seqs == 0 || max_q_len == 0) return BI_OK;
  bi_status st = check_attn_geom(k_cache, v_cache, num_pages, block_table, max_pages_per_seq,
                                 num_q_heads, num_kv_heads, head_dim, page_size, softmax_scale);
  if (st != BI_OK) return st;
  if (!q || !q_start || !ctx_lens || !out) return BI_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out)) return BI_ERR_INVALID_ARG;
  if (ld_q < (int64_t)num_q_heads * head_dim || ld_q % 8) return BI_ERR_INVALID_ARG;
  if (num_seqs > 65535 || num_kv_heads > 65535) return BI_ERR_UNSUPPORTED;
  if ((int64_t)max_q_len * (num_q_heads / num_kv_heads) > (1 << 30)) return BI_ERR_UNSUPPORTED;
  if (workspace && (!aligned16(workspace) || workspace_bytes < bi::attn_prefill_workspace_bytes(num_seqs)))
    return BI_ERR_WORKSPACE;
  const bi::AttnGeom g = make_geom(k_cache, v_cache, num_pages, block_table, max_pages_per_seq,
                                   num_q_heads, num_kv_heads, head_dim, page_size, softmax_scale);
  return from_hip(bi::launch_attn_prefill(q, ld_q, q_start, ctx_lens, num_seqs, max_q_len, g, out, lse, workspace,
                                          as_stream(stream)));
}

size_t bi_attn_prefill_workspace_bytes(int32_t num_seqs) {
  if (num_seqs <= 0) return 0;
  return bi::attn_prefill_workspace_bytes(num_seqs);
}

bi_status bi_log_softmax(const float* logits, int64_t ld_in, float* out, int64_t ld_out, int64_t rows,
                         int64_t vocab, bi_stream_t stream) {
  if (rows < 0 || vocab <= 0) return BI_ERR_INVALID_ARG;
  if (rows == 0) return BI_OK;
  if (!logits || !out) return BI_ERR_INVALID_ARG;
  if (vocab % 4 || vocab > (1 << 30)) return BI_ERR_UNSUPPORTED;
  if (ld_in < vocab || ld_out < vocab || ld_in % 4 || ld_out % 4) return BI_ERR_INVALID_ARG;
  if (!aligned16(logits) || !aligned16(out)) return BI_ERR_INVALID_ARG;
  if (rows > 0x7fffffff) return BI_ERR_UNSUPPORTED;
  return from_hip(bi::launch_log_softmax(logits, ld_in, out, ld_out, rows, vocab, as_stream(stream)));
}

size_t bi_moe_workspace_bytes(int32_t num_tokens, int32_t top_k, int32_t num_experts, int32_t hidden,
                              int32_t ffn) {
  if (num_tokens <= 0 || top_k <= 0 || num_experts <= 0 || hidden <= 0 || ffn <= 0) return 0;
  return bi::moe_workspace_bytes(num_tokens, top_k, num_experts, hidden, ffn);
}

bi_status bi_moe_ffn(const void* x, int64_t ldx, const int32_t* expert_ids, const float* expert_weights,
                     int32_t num_tokens, int32_t top_k, int32_t num_experts, const void* w_up, const void* w_down,
                     int32_t hidden, int32_t ffn, void* y, int64_t ldy, void* workspace, size_t workspace_bytes,
                     bi_stream_t stream) {
  if (num_tokens < 0 || top_k <= 0 || num_experts <= 0 || hidden <= 0 || ffn <= 0) return BI_ERR_INVALID_ARG;
  if (num_tokens == 0) return BI_OK;
  if (!x || !expert_ids || !expert_weights || !w_up || !w_down || !y) return BI_ERR_INVALID_ARG;
  if (top_k > 64 || num_experts > 65535) return BI_ERR_UNSUPPORTED;
  if (hidden % 32 || ffn % 32 || hidden > 65536 || ffn > 65536) return BI_ERR_UNSUPPORTED;
  if (ldx < hidden || ldx % 8 || ldy < hidden || ldy % 8) return BI_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(y)) return BI_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(expert_ids) & 3u) || (reinterpret_cast<uintptr_t>(expert_weights) & 3u))
    return BI_ERR_INVALID_ARG;
  if (!bi::moe_supported(num_tokens, ldx, top_k, num_experts, hidden, ffn)) return BI_ERR_UNSUPPORTED;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return BI_ERR_WORKSPACE;
  if (workspace_bytes < bi::moe_workspace_bytes(num_tokens, top_k, num_experts, hidden, ffn)) return BI_ERR_WORKSPACE;
  return from_hip(bi::launch_moe_ffn(x, ldx, expert_ids, expert_weights, num_tokens, top_k, num_experts, w_up,
                                     w_down, hidden, ffn, y, ldy, workspace, as_stream(stream)));
}

bi_status bi_moe_route(const void* x, int64_t ldx, const void* w_gate, int32_t num_tokens, int32_t hidden,
                       int32_t num_experts, int32_t top_k, float* logits, int32_t* expert_ids, float* expert_weights,
                       bi_stream_t stream) {
  if (num_tokens < 0 || hidden <= 0 || num_experts <= 0 || top_k <= 0 || top_k > num_experts)
    return BI_ERR_INVALID_ARG;
  if (top_k > 64 || num_experts > 1024) return BI_ERR_UNSUPPORTED;
  if (num_tokens == 0) return BI_OK;
  if (!x || !w_gate || !logits || !expert_ids || !expert_weights) return BI_ERR_INVALID_ARG;
  if (hidden % 32) return BI_ERR_UNSUPPORTED;
  if (ldx < hidden || ldx % 8) return BI_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_gate)) return BI_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(logits) & 3u) || (reinterpret_cast<uintptr_t>(expert_ids) & 3u) ||
      (reinterpret_cast<uintptr_t>(expert_weights) & 3u))
    return BI_ERR_INVALID_ARG;
  if (!bi::gemm_supported(ldx, hidden, num_tokens, num_experts, hidden)) return BI_ERR_UNSUPPORTED;
  return from_hip(bi::launch_moe_route(x, ldx, w_gate, num_tokens, hidden, num_experts, top_k, logits, expert_ids,
                                       expert_weights, as_stream(stream)));
}

size_t bi_lm_head_logprobs_workspace_bytes(int64_t m, int64_t n) {
  if (m <= 0 || n <= 0) return 0;
  return bi::lm_head_workspace_bytes(m, n);
}

bi_status bi_lm_head_logprobs(const void* a, int64_t lda, const void* w, int64_t ldw, float* out, int64_t ldo,
                              float* lse, int64_t m, int64_t n, int64_t k, void* workspace, size_t workspace_bytes,
                              bi_stream_t stream) {
  if (m < 0 || n <= 0 || k <= 0) return BI_ERR_INVALID_ARG;
  if (m == 0) return BI_OK;
  if (!a || !w || !out) return BI_ERR_INVALID_ARG;
  if (k % 32 || n % 4) return BI_ERR_UNSUPPORTED;
  if (m > (1 << 30) || n > (1 << 30) || k > (1 << 30)) return BI_ERR_UNSUPPORTED;
  if (lda < k || ldw < k || ldo < n || lda % 8 || ldw % 8 || ldo % 4) return BI_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(w) || !aligned16(out)) return BI_ERR_INVALID_ARG;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return BI_ERR_INVALID_ARG;
  if (!bi::lm_head_supported(lda, ldw, m, n, k)) return BI_ERR_UNSUPPORTED;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return BI_ERR_WORKSPACE;
  if (workspace_bytes < bi::lm_head_workspace_bytes(m, n)) return BI_ERR_WORKSPACE;
  return from_hip(bi::launch_lm_head_logprobs(a, lda, w, ldw, out, ldo, lse, m, n, k, workspace, as_stream(stream)));
}

size_t bi_lm_head_greedy_workspace_bytes(int64_t m, int64_t n) {
  if (m <= 0 || n <= 0) return 0;
  return bi::lm_head_greedy_workspace_bytes(m, n);
}

bi_status bi_lm_head_greedy(const void* a, int64_t lda, const void* w, int64_t ldw, int32_t* token, float* logprob,
                            int64_t m, int64_t n, int64_t k, void* workspace, size_t workspace_bytes,
                            bi_stream_t stream) {
  if (m < 0 || n <= 0 || k <= 0) return BI_ERR_INVALID_ARG;
  if (m == 0) return BI_OK;
  if (!a || !w || !token) return BI_ERR_INVALID_ARG;
  if (k % 32) return BI_ERR_UNSUPPORTED;
  if (m > (1 << 30) || n > (1 << 30) || k > (1 << 30)) return BI_ERR_UNSUPPORTED;
  if (lda < k || ldw < k || lda % 8 || ldw % 8) return BI_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(w)) return BI_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(token) & 3u) || (logprob && (reinterpret_cast<uintptr_t>(logprob) & 3u)))
    return BI_ERR_INVALID_ARG;
  if (!bi::lm_head_supported(lda, ldw, m, n, k)) return BI_ERR_UNSUPPORTED;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return BI_ERR_WORKSPACE;
  if (workspace_bytes < bi::lm_head_greedy_workspace_bytes(m, n)) return BI_ERR_WORKSPACE;
  return from_hip(bi::launch_lm_head_greedy(a, lda, w, ldw, token, logprob, m, n, k, workspace, as_stream(stream)));
}

bi_status bi_add(const void* x, int64_t ldx, const void* y, int64_t ldy, void* out, int64_t ldo, int64_t rows,
                 int64_t cols, bi_stream_t stream) {
  if (rows < 0 || cols < 0) return BI_ERR_INVALID_ARG;
  if (rows == 0 || cols == 0) return BI_OK;
  if (!x || !y || !out) return BI_ERR_INVALID_ARG;
  if (cols % 8) return BI_ERR_UNSUPPORTED;
  if (rows > (1 << 30) || cols > (1 << 30) || rows * (cols / 8) > (int64_t(1) << 31)) return BI_ERR_UNSUPPORTED;
  if (ldx < cols || ldy < cols || ldo < cols || ldx % 8 || ldy % 8 || ldo % 8) return BI_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y) || !aligned16(out)) return BI_ERR_INVALID_ARG;
  return from_hip(bi::launch_add(x, ldx, y, ldy, out, ldo, rows, cols, as_stream(stream)));
}

bi_status bi_silu_mul(const void* gate_up, int64_t ld_gu, void* out, int64_t ldo, int64_t rows, int64_t f,
                      bi_stream_t stream) {
  if (rows < 0 || f < 0) return BI_ERR_INVALID_ARG;
  if (rows == 0 || f == 0) return BI_OK;
  if (!gate_up || !out) return BI_ERR_INVALID_ARG;
  if (f % 8) return BI_ERR_UNSUPPORTED;
  if (rows > (1 << 30) || f > (1 << 29) || rows * (f / 8) > (int64_t(1) << 31)) return BI_ERR_UNSUPPORTED;
  if (ld_gu < 2 * f || ldo < f || ld_gu % 8 || ldo % 8) return BI_ERR_INVALID_ARG;
  if (!aligned16(gate_up) || !aligned16(out)) return BI_ERR_INVALID_ARG;
  return from_hip(bi::launch_silu_mul(gate_up, ld_gu, out, ldo, rows, f, as_stream(stream)));
}

}  // extern "C"
