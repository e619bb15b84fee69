// (max, sum of exponentials) pairs for log-sum-exp reductions over fp32
// logits ("Batch Invariance and Numerical Reproducibility", answer on sampler
// and trainer agreeing on logprobs).  A pair (m, s) stands for s * e^m.
#pragma once

#include "bi_common.hpp"

namespace bi {

struct MaxSum {
  float m, s;
};

// Combine two pairs.  Commutative bit for bit: both orders compute the same
// two products and add them.  A pair with m = -inf (nothing seen yet) adds 0.
__device__ __forceinline__ MaxSum combine(MaxSum a, MaxSum b) {
  const float m = fmaxf(a.m, b.m);
  const float ta = a.m == -INFINITY ? 0.0f : a.s * exp2_hw((a.m - m) * kLog2e);
  const float tb = b.m == -INFINITY ? 0.0f : b.s * exp2_hw((b.m - m) * kLog2e);
  return MaxSum{m, ta + tb};
}

// Combine with the pair of lane l ^ 16 (resp. l ^ 32).  The swap hands every
// lane {own, partner} in a row-dependent order, which combine cannot see.
__device__ __forceinline__ MaxSum combine_xor16(MaxSum v) {
  const auto rm = __builtin_amdgcn_permlane16_swap(__float_as_uint(v.m), __float_as_uint(v.m), false, false);
  const auto rs = __builtin_amdgcn_permlane16_swap(__float_as_uint(v.s), __float_as_uint(v.s), false, false);
  return combine(MaxSum{__uint_as_float(rm[0]), __uint_as_float(rs[0])},
                 MaxSum{__uint_as_float(rm[1]), __uint_as_float(rs[1])});
}
__device__ __forceinline__ MaxSum combine_xor32(MaxSum v) {
  const auto rm = __builtin_amdgcn_permlane32_swap(__float_as_uint(v.m), __float_as_uint(v.m), false, false);
  const auto rs = __builtin_amdgcn_permlane32_swap(__float_as_uint(v.s), __float_as_uint(v.s), false, false);
  return combine(MaxSum{__uint_as_float(rm[0]), __uint_as_float(rs[0])},
                 MaxSum{__uint_as_float(rm[1]), __uint_as_float(rs[1])});
}

// log(s * e^m) in fp32.
__device__ __forceinline__ float lse_of(MaxSum t) { return t.m + log2_hw(t.s) * kLn2; }

}  // namespace bi
