// bi_gemm's launcher: the configuration of gemm_with_cfg_mn (gemm_kernel.hpp,
// which also holds the kernel and why every configuration gives the same bits).
#include <atomic>

#include "gemm_kernel.hpp"
#include "launch.hpp"

namespace bi {

int gemm_device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  const int v = cached[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

void gemm_config_of(int64_t lda, int64_t ldw, int64_t m, int64_t n, int64_t k, int out[8]) {
  gemm_with_cfg_mn(lda, ldw, m, n, k, [&](auto cfg) {
    using C = decltype(cfg);
    const int v[8] = {C::TN, C::TM, C::WGN, C::WGM, C::S, C::BK, C::OCC, C::CPW == kCpolNt ? 1 : 0};
    for (int i = 0; i < 8; ++i) out[i] = v[i];
    return 0;
  });
}

bool gemm_supported(int64_t lda, int64_t ldw, int64_t m, int64_t n, int64_t k) {
  return gemm_with_cfg_mn(lda, ldw, m, n, k, [&](auto cfg) {
    using C = decltype(cfg);
    const int64_t tiles = ((m + C::TM - 1) / C::TM) * ((n + C::TN - 1) / C::TN);
    return tiles <= 0x7fffffff && gemm_offsets_fit<C>(lda, ldw, k);
  });
}

hipError_t launch_gemm(const void* a, int64_t lda, const void* w, int64_t ldw, void* c, int64_t ldc, bool c_f32,
                       int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  return gemm_with_cfg_mn(lda, ldw, m, n, k, [&](auto cfg) {
    return launch_gemm_cfg<decltype(cfg)>(a, lda, w, ldw, c, ldc, c_f32, m, n, k, stream);
  });
}

}  // namespace bi
