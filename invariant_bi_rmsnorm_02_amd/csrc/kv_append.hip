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

// One workgroup per (group of 16 consecutive new tokens, kv head).  K is
// copied token by token: 8 dimensions of one token are 16 contiguous bytes of
// the tile.  V's 16-byte runs hold 8 tokens of one dimension (slots 8i ..
// 8i + 7 of a tile), so V is written in whole runs wherever 8 consecutive new
// tokens fill such a run in order - a chunk of a prefilled sequence - and 2
// bytes at a time only for the tokens of runs that are not filled that way
// (decode tokens, a chunk's ends, padding).  A run is written by the
// workgroup holding the token of its first slot, which reads up to 7 tokens
// past its own 16; every workgroup decides from the same slot values, so each
// element is written exactly once.  Both ways copy bits.
template <int D>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn, int64_t ld_new,
    const int32_t* __restrict__ slots, int T, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
    int num_pages, int Hkv, int log2_ps) {
  constexpr int kBefore = 8, kRows = kTile + 8;   // slots of tokens t0 - 8 .. t0 + 23; V of t0 .. t0 + 23
  const int t0 = blockIdx.x * kTile, h = blockIdx.y;
  const int ps = 1 << log2_ps;
  const int64_t cap = (int64_t)num_pages * ps;
  __shared__ int ss[kBefore + kRows];
  __shared__ __attribute__((aligned(16))) uint16_t sv[kRows * D];
  if (threadIdx.x < kBefore + kRows) {
    const int t = t0 - kBefore + (int)threadIdx.x;
    const int sl = (t >= 0 && t < T) ? slots[t] : -1;
    ss[threadIdx.x] = (sl >= 0 && (int64_t)sl < cap) ? sl : -1;
  }
  for (int c = threadIdx.x; c < kRows * (D / 8); c += kAppendThreads) {
    const int i = c / (D / 8), d0 = (c % (D / 8)) * 8;
    if (t0 + i < T)
      *reinterpret_cast<u32x4_t*>(&sv[i * D + d0]) =
          *reinterpret_cast<const u32x4_t*>(vn + (int64_t)(t0 + i) * ld_new + h * D + d0);
  }
  __syncthreads();
  // Whether the 8 tokens starting at group index i (-8 <= i < 16) fill the
  // 8-slot V run of their first slot in order.
  auto full_run = [&](int i) {
    const int s = ss[i + kBefore];
    if (s < 0 || (s & 7) || t0 + i < 0 || t0 + i + 7 >= T) return false;
#pragma unroll
    for (int k = 1; k < 8; ++k)
      if (ss[i + kBefore + k] != s + k) return false;
    return true;
  };
  auto tile_of = [&](int s) { return tile_base(s >> log2_ps, h, s & (ps - 1), Hkv, log2_ps, D); };
  for (int c = threadIdx.x; c < kTile * (D / 8); c += kAppendThreads) {
    const int i = c / (D / 8), d0 = (c % (D / 8)) * 8;
    const int s = ss[i + kBefore];
    if (s < 0) continue;
    const int64_t tb = tile_of(s);
    const int j = s & (kTile - 1);
    // K: 8 dimensions of token i, 16 contiguous bytes.
    *reinterpret_cast<u32x4_t*>(kc + tb + k_tile_off(j, d0)) =
        *reinterpret_cast<const u32x4_t*>(kn + (int64_t)(t0 + i) * ld_new + h * D + d0);
    // V, 2 bytes at a time, for a token whose run is not filled in order.
    if (!full_run(i - (s & 7))) {
      uint16_t* vp = vc + tb + v_tile_off(j, d0);                     // dims d0 .. d0+7 are 8 elements apart
#pragma unroll
      for (int e = 0; e < 8; ++e) vp[e * 8] = sv[i * D + d0 + e];
    }
  }
  // V runs that start at one of this group's tokens: one 16-byte store per dimension.
  for (int c = threadIdx.x; c < kTile * D; c += kAppendThreads) {
    const int i = c / D, d = c % D;
    if (!full_run(i)) continue;
    const int s = ss[i + kBefore];
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (uint32_t)sv[(i + 2 * q) * D + d] | ((uint32_t)sv[(i + 2 * q + 1) * D + d] << 16);
    *reinterpret_cast<u32x4_t*>(vc + tile_of(s) + v_tile_off(s & (kTile - 1), d)) = u32x4_t{w[0], w[1], w[2], w[3]};
  }
}

}  // namespace

hipError_t launch_kv_append(const void* k_new, const void* v_new, int64_t ld_new, const int32_t* slot_mapping,
                            int num_tokens, void* k_cache, void* v_cache, int num_pages, int num_kv_heads,
                            int head_dim, int page_size, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  int log2_ps = 0;
  while ((1 << log2_ps) < page_size) ++log2_ps;
  const dim3 grid(static_cast<unsigned>((num_tokens + kTile - 1) / kTile), static_cast<unsigned>(num_kv_heads));
  auto* kn = static_cast<const uint16_t*>(k_new);
  auto* vn = static_cast<const uint16_t*>(v_new);
  auto* kc = static_cast<uint16_t*>(k_cache);
  auto* vc = static_cast<uint16_t*>(v_cache);
  if (head_dim == 64)
    hipLaunchKernelGGL(kv_append_kernel<64>, grid, dim3(kAppendThreads), 0, stream, kn, vn, ld_new, slot_mapping,
                       num_tokens, kc, vc, num_pages, num_kv_heads, log2_ps);
  else
    hipLaunchKernelGGL(kv_append_kernel<128>, grid, dim3(kAppendThreads), 0, stream, kn, vn, ld_new, slot_mapping,
                       num_tokens, kc, vc, num_pages, num_kv_heads, log2_ps);
  return hipGetLastError();
}

}  // namespace bi
