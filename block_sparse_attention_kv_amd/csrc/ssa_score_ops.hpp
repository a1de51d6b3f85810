// fp64 matrix-instruction dot products of the block scores, shared by the
// score kernels and the fused decode scoring + selection.
#pragma once
#include "ssa_common.hpp"

namespace ssa {

// Scores are small fp64 matrix products, done with the fp64 matrix
// instruction 16x16x4: lane l supplies A[l%16][l/16] and B[l/16][l%16] and
// holds C[l/16 + 4r][l%16], r = 0..3.  Lane l's k-slot covers
// d = 16 (l/16) + s over the 16 steps s, so each lane reads 16 consecutive
// values of a row.  Products and sums are fp64; each score is rounded once to
// fp32.
typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f64x4 mfma_dot64(const double (&a)[16], const double (&b)[16], f64x4 acc) {
#pragma unroll
  for (int st = 0; st < 16; ++st) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a[st], b[st], acc, 0, 0, 0);
  return acc;
}

// B operand: 16 consecutive fp32 values of a summary row, as fp64.
__device__ __forceinline__ void load_row16_f64(const float* __restrict__ p, double (&out)[16]) {
  const float4* r = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float4 v = r[c];
    out[4 * c] = v.x;
    out[4 * c + 1] = v.y;
    out[4 * c + 2] = v.z;
    out[4 * c + 3] = v.w;
  }
}

}  // namespace ssa
