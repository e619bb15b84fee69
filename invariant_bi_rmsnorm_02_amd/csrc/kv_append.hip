// KV append: copy the new tokens' keys and values into their paged-cache slots
// before attention runs, so cached and new tokens are read through one layout
// ("Como superar a não determinismo na inferência de LLMs", Attention: keep a
// consistent K/V layout; "Thinking Machines Lab - Defeating Nondeterminism in
// LLM Inference", fig. "FlashAttention with KV Cache").  A bit-exact copy into
// the tiled layout of kv_layout.hpp.
#include "kv_layout.hpp"
#include "launch.hpp"

namespace bi {
namespace {

constexpr int kAppendThreads = 128;

__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn, int64_t ld_new,
    const int32_t* __restrict__ slots, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, int num_pages,
    int Hkv, int D, int log2_ps) {
  const int t = blockIdx.x;
  const int slot = slots[t];
  const int ps = 1 << log2_ps;
  if (slot < 0 || (int64_t)slot >= (int64_t)num_pages * ps) return;
  const int64_t page = slot >> log2_ps;
  const int off = slot & (ps - 1);
  const int j = off & (kTile - 1);
  const int nvec = Hkv * D / 8;
  const int64_t src = (int64_t)t * ld_new;
  for (int i = threadIdx.x; i < nvec; i += kAppendThreads) {
    const int h = (i * 8) / D, d0 = (i * 8) % D;
    const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(kn + src + i * 8);
    const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(vn + src + i * 8);
    const int64_t tb = tile_base(page, h, off, Hkv, log2_ps, D);
    *reinterpret_cast<u32x4_t*>(kc + tb + k_tile_off(j, d0)) = kv;   // 8 dims of one token: 16 contiguous bytes
    uint16_t* vp = vc + tb + v_tile_off(j, d0);                     // dims d0 .. d0+7 are 8 elements apart
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vp[(2 * e) * 8] = static_cast<uint16_t>(vv[e] & 0xffffu);
      vp[(2 * e + 1) * 8] = static_cast<uint16_t>(vv[e] >> 16);
    }
  }
}

}  // namespace

hipError_t launch_kv_append(const void* k_new, const void* v_new, int64_t ld_new, const int32_t* slot_mapping,
                            int num_tokens, void* k_cache, void* v_cache, int num_pages, int num_kv_heads,
                            int head_dim, int page_size, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  int log2_ps = 0;
  while ((1 << log2_ps) < page_size) ++log2_ps;
  hipLaunchKernelGGL(kv_append_kernel, dim3(num_tokens), dim3(kAppendThreads), 0, stream,
                     static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), ld_new, slot_mapping,
                     static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), num_pages, num_kv_heads,
                     head_dim, log2_ps);
  return hipGetLastError();
}

}  // namespace bi
