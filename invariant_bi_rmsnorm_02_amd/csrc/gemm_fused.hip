// GEMMs with the decoder layer's elementwise steps in their epilogues
// ("Thinking Machines Lab - Defeating Nondeterminism in LLM Inference",
// sections "2. Batch-Invariant Matrix Multiplication" and "Achieving
// Batch-Invariant Kernels": only the reductions need a batch-independent
// order; the elementwise work after them may be fused freely).
//
//   gemm_add:      y = bf16(x + bf16(A W^T))            (a projection and its residual add)
//   gemm_silu_mul: out[:, j] = bf16(silu(g_j) * u_j),   g_j, u_j = bf16 of columns 2j, 2j+1 of A W^T
//                  (W holds the gate and up rows interleaved)
//
// The main loop, the tile rule and every rounding are bi_gemm's (gemm_tile,
// gemm_with_cfg_mn, pack_bf16x2), and the elementwise arithmetic is that of
// bi_add / bi_silu_mul (pointwise.hpp), so each result is bit for bit the
// unfused pair of calls: the GEMM's output element rounded to bf16, widened
// back, then the same fp32 expression and one rounding.  What the fusion saves
// is the intermediate's round trip through HBM and one launch.
#include "gemm_kernel.hpp"
#include "launch.hpp"
#include "pointwise.hpp"

namespace bi {
namespace {

// X may be Y (an in-place residual): each lane reads its x elements before it
// writes the same y elements, and no two lanes share an element.
template <class Cfg>
__global__ __launch_bounds__(Cfg::kThreads, Cfg::OCC) void gemm_add_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ W, int64_t ldw, const uint16_t* X,
    int64_t ldx, uint16_t* Y, int64_t ldy, int M, int N, int K, int tiles_m, int tiles_n) {
  gemm_tile<Cfg>(A, lda, W, ldw, M, N, K, tiles_m, tiles_n, [&](int r, int n, f32x4_t v, int cnt) {
    const uint16_t* xp = X + (int64_t)r * ldx + n;
    uint16_t* yp = Y + (int64_t)r * ldy + n;
    if (cnt == 4) {   // n % 4 == 0 and 8-aligned rows: 8-byte accesses
      const u32x2_t xv = *reinterpret_cast<const u32x2_t*>(xp);
      const uint32_t c01 = pack_bf16x2(v[0], v[1]), c23 = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<u32x2_t*>(yp) =
          u32x2_t{pack_bf16x2(pw_add(bf16_lo(xv[0]), bf16_lo(c01)), pw_add(bf16_hi(xv[0]), bf16_hi(c01))),
                  pack_bf16x2(pw_add(bf16_lo(xv[1]), bf16_lo(c23)), pw_add(bf16_hi(xv[1]), bf16_hi(c23)))};
    } else {
      for (int e = 0; e < cnt; ++e) {
        const float c = bf16_lo(f32_to_bf16(v[e]));
        yp[e] = static_cast<uint16_t>(f32_to_bf16(pw_add(bf16_lo(xp[e]), c)));
      }
    }
  });
}

// N = 2f is even and n % 4 == 0, so cnt is 2 or 4: one or two (gate, up) pairs.
template <class Cfg>
__global__ __launch_bounds__(Cfg::kThreads, Cfg::OCC) void gemm_silu_mul_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ W, int64_t ldw,
    uint16_t* __restrict__ O, int64_t ldo, int M, int N, int K, int tiles_m, int tiles_n) {
  gemm_tile<Cfg>(A, lda, W, ldw, M, N, K, tiles_m, tiles_n, [&](int r, int n, f32x4_t v, int cnt) {
    uint16_t* op = O + (int64_t)r * ldo + (n >> 1);
    const uint32_t c01 = pack_bf16x2(v[0], v[1]);
    const float h0 = pw_silu_mul(bf16_lo(c01), bf16_hi(c01));
    if (cnt == 4) {
      const uint32_t c23 = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint32_t*>(op) = pack_bf16x2(h0, pw_silu_mul(bf16_lo(c23), bf16_hi(c23)));
    } else {
      *op = static_cast<uint16_t>(f32_to_bf16(h0));
    }
  });
}

template <class Cfg>
dim3 fused_grid(int64_t m, int64_t n, int& tiles_m, int& tiles_n) {
  tiles_m = static_cast<int>((m + Cfg::TM - 1) / Cfg::TM);
  tiles_n = static_cast<int>((n + Cfg::TN - 1) / Cfg::TN);
  return dim3(static_cast<unsigned>(tiles_m * tiles_n));
}

}  // namespace

hipError_t launch_gemm_add(const void* a, int64_t lda, const void* w, int64_t ldw, const void* x, int64_t ldx,
                           void* y, int64_t ldy, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  return gemm_with_cfg_mn(lda, ldw, m, n, k, [&](auto cfg) {
    using Cfg = decltype(cfg);
    if (!gemm_offsets_fit<Cfg>(lda, ldw, k)) return hipErrorInvalidValue;
    int tm, tn;
    const dim3 grid = fused_grid<Cfg>(m, n, tm, tn);
    hipLaunchKernelGGL((gemm_add_kernel<Cfg>), grid, dim3(Cfg::kThreads), 0, stream,
                       static_cast<const uint16_t*>(a), lda, static_cast<const uint16_t*>(w), ldw,
                       static_cast<const uint16_t*>(x), ldx, static_cast<uint16_t*>(y), ldy, (int)m, (int)n, (int)k,
                       tm, tn);
    return hipGetLastError();
  });
}

hipError_t launch_gemm_silu_mul(const void* a, int64_t lda, const void* w, int64_t ldw, void* out, int64_t ldo,
                                int64_t m, int64_t f, int64_t k, hipStream_t stream) {
  if (m == 0 || f == 0) return hipSuccess;
  const int64_t n = 2 * f;
  return gemm_with_cfg_mn(lda, ldw, m, n, k, [&](auto cfg) {
    using Cfg = decltype(cfg);
    if (!gemm_offsets_fit<Cfg>(lda, ldw, k)) return hipErrorInvalidValue;
    int tm, tn;
    const dim3 grid = fused_grid<Cfg>(m, n, tm, tn);
    hipLaunchKernelGGL((gemm_silu_mul_kernel<Cfg>), grid, dim3(Cfg::kThreads), 0, stream,
                       static_cast<const uint16_t*>(a), lda, static_cast<const uint16_t*>(w), ldw,
                       static_cast<uint16_t*>(out), ldo, (int)m, (int)n, (int)k, tm, tn);
    return hipGetLastError();
  });
}

}  // namespace bi
