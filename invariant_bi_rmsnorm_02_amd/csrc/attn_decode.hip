// bi_attn_decode's kernels: the fixed-size split-KV decode of
// attn_decode_impl.hpp at the library's chunk size, kChunk = 256 keys ("Thinking
// Machines Lab - Defeating Nondeterminism in LLM Inference", fig. "Fixed Size
// Split KV Strategy"; "Batch Invariance and Numerical Reproducibility", answer
// on fixed-size chunks).
#include "attn_decode_impl.hpp"

namespace bi {

size_t attn_decode_workspace_bytes(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim, int64_t max_seq_len) {
  return decode_workspace_bytes_cs(num_seqs, num_q_heads, head_dim, max_seq_len, kChunk);
}

hipError_t launch_attn_decode(const void* q, int64_t ld_q, const AttnGeom& g, const int32_t* seq_lens,
                              int num_seqs, int max_seq_len, void* out, float* lse, void* workspace,
                              hipStream_t stream) {
  if (num_seqs == 0) return hipSuccess;
  if (max_seq_len <= 0) max_seq_len = 1;  // grid of one empty chunk; merge writes the L <= 0 result
  return g.head_dim == 64
             ? launch<64, kChunk>(q, ld_q, g, seq_lens, num_seqs, max_seq_len, out, lse, workspace, stream)
             : launch<128, kChunk>(q, ld_q, g, seq_lens, num_seqs, max_seq_len, out, lse, workspace, stream);
}

}  // namespace bi
