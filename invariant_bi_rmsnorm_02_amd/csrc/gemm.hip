// bi_gemm's launcher: the configuration of gemm_with_cfg_mn (gemm_kernel.hpp,
// which also holds the kernel and why every configuration gives the same bits).
#include "gemm_kernel.hpp"
#include "launch.hpp"

namespace bi {

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
