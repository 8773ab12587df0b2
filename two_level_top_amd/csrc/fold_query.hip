// Query fold for the score kernels' epilogue.
//
// The score is sum_h w_h * relu(s_h) with s_h = q_h . k.  Since
// relu(s) = (s + |s|) / 2,
//     score = sum_h (w_h / 2) |s_h|  +  qf . k,     qf = sum_h (w_h / 2) q_h.
// The first sum costs one FMA (with an |x| source modifier) per head instead
// of a max and an FMA; the second is a plain dot product with one folded
// query vector, which the score kernels run on the MFMA as a fifth block of
// 16 "heads".  For that, qf (exact in fp64: w_h is fp32 and q_h has 2-bit
// mantissas) is written as a sum of 16 MXFP4 vectors by greedy residual
// splitting: each term takes, per 32-element group, the ue8m0 scale
// 2^ceil(log2(max|r| / 6)) and the nearest e2m1 code of every element; the
// group's largest residual shrinks at least 3x per term, and the folded
// queries of the index layer need about 14 terms to be represented exactly.
//
// Output per query row (kFoldRowBytes = 1088): 16 x 64 code bytes, then
// 16 x 4 scale bytes -- the byte layout of a 16-head query block, so the
// score kernels load it exactly like a block of query heads.
#include "idx_internal.h"

namespace idxk {

__device__ __forceinline__ double e2m1_value(int code) {
  const int m = code & 7;
  const double mag = m < 4 ? 0.5 * m : (m == 4 ? 2.0 : (m == 5 ? 3.0 : (m == 6 ? 4.0 : 6.0)));
  return (code & 8) ? -mag : mag;
}

// nearest e2m1 magnitude code of a in [0, 6] (ties to the even code)
__device__ __forceinline__ int e2m1_nearest(double a) {
  if (a <= 0.25) return 0;
  if (a < 0.75) return 1;
  if (a <= 1.25) return 2;
  if (a < 1.75) return 3;
  if (a <= 2.5) return 4;
  if (a < 3.5) return 5;
  if (a <= 5.0) return 6;
  return 7;
}

// max over the 32 lanes of a half-wave
__device__ __forceinline__ double halfwave_max(double v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}

// One wave per query row; lane l owns dimensions l and l + 64 (groups l / 32
// and 2 + l / 32).
__global__ __launch_bounds__(256) void fold_query_kernel(QueryArgs q, uint8_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= q.rows) return;
  double r[2] = {0.0, 0.0};
  for (int h = 0; h < q.heads; ++h) {
    const size_t base = (size_t)row * q.heads + h;
    const double wh = 0.5 * (double)q.w[base];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int d = lane + 64 * j;
      const uint8_t byte = q.vals[base * kValBytes + d / 2];
      const int code = (d & 1) ? (byte >> 4) : (byte & 15);
      const int sc = q.scales[base * kScaleBytes + d / 32];
      r[j] = fma(wh, ldexp(e2m1_value(code), sc - 127), r[j]);
    }
  }
  uint8_t* orow = out + (size_t)row * kFoldRowBytes;
  for (int t = 0; t < kFoldTerms; ++t) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int d = lane + 64 * j;
      const double m = halfwave_max(fabs(r[j]));
      int e = -127;
      if (m > 0.0) {
        int x;
        const double f = frexp(m / 6.0, &x);  // m / 6 = f * 2^x, f in [0.5, 1)
        e = f > 0.5 ? x : x - 1;               // ceil(log2(m / 6))
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
      }
      const double a = ldexp(fabs(r[j]), -e);
      int code = e2m1_nearest(a);
      if (r[j] < 0.0 && code != 0) code |= 8;
      r[j] -= ldexp(e2m1_value(code), e);
      const int other = __shfl_xor(code, 1, 64);  // the neighbouring dimension
      if ((d & 1) == 0) orow[t * kValBytes + d / 2] = (uint8_t)(code | (other << 4));
      if ((d & 31) == 0) orow[kFoldTerms * kValBytes + t * kScaleBytes + d / 32] = (uint8_t)(e + 127);
    }
  }
}

hipError_t launch_fold_query(const QueryArgs& q, uint8_t* out, hipStream_t st) {
  if (q.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(fold_query_kernel, dim3((q.rows + 3) / 4), dim3(256), 0, st, q, out);
  return hipGetLastError();
}

}  // namespace idxk
