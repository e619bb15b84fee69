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

// A pair with the column index of its maximum (greedy sampling): ties go to
// the lower index.  The (m, s) part is combined exactly as MaxSum's, and the
// index choice depends only on the two values and indices, so it is
// commutative and associative: any combination order picks the lowest index
// holding the maximum.  An empty pair has m = -inf and i = INT_MAX.
struct MaxSumArg {
  float m, s;
  int i;
};
__device__ __forceinline__ MaxSumArg combine(MaxSumArg a, MaxSumArg b) {
  const MaxSum t = combine(MaxSum{a.m, a.s}, MaxSum{b.m, b.s});
  const int i = a.m > b.m ? a.i : (b.m > a.m ? b.i : min(a.i, b.i));
  return MaxSumArg{t.m, t.s, i};
}
__device__ __forceinline__ MaxSumArg combine_xor16(MaxSumArg v) {
  const MaxSum t = combine_xor16(MaxSum{v.m, v.s});
  const auto rm = __builtin_amdgcn_permlane16_swap(__float_as_uint(v.m), __float_as_uint(v.m), false, false);
  const auto ri = __builtin_amdgcn_permlane16_swap((unsigned)v.i, (unsigned)v.i, false, false);
  const float m0 = __uint_as_float(rm[0]), m1 = __uint_as_float(rm[1]);
  const int i0 = (int)ri[0], i1 = (int)ri[1];
  return MaxSumArg{t.m, t.s, m0 > m1 ? i0 : (m1 > m0 ? i1 : min(i0, i1))};
}
__device__ __forceinline__ MaxSumArg combine_xor32(MaxSumArg v) {
  const MaxSum t = combine_xor32(MaxSum{v.m, v.s});
  const auto rm = __builtin_amdgcn_permlane32_swap(__float_as_uint(v.m), __float_as_uint(v.m), false, false);
  const auto ri = __builtin_amdgcn_permlane32_swap((unsigned)v.i, (unsigned)v.i, false, false);
  const float m0 = __uint_as_float(rm[0]), m1 = __uint_as_float(rm[1]);
  const int i0 = (int)ri[0], i1 = (int)ri[1];
  return MaxSumArg{t.m, t.s, m0 > m1 ? i0 : (m1 > m0 ? i1 : min(i0, i1))};
}
__device__ __forceinline__ MaxSumArg shfl_xor_pair(MaxSumArg v, int o) {
  return MaxSumArg{shfl_xor(v.m, o), shfl_xor(v.s, o), shfl_xor(v.i, o)};
}
__device__ __forceinline__ MaxSum shfl_xor_pair(MaxSum v, int o) { return MaxSum{shfl_xor(v.m, o), shfl_xor(v.s, o)}; }

// log(s * e^m) in fp32.
__device__ __forceinline__ float lse_of(MaxSum t) { return t.m + log2_hw(t.s) * kLn2; }

}  // namespace bi
