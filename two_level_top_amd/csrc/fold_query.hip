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

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xf, 0xf, true);
  return __hiloint2double(hi, lo);
}

// 16 lanes per query row (4 rows per wave); lane j of a row owns dimensions
// 8j .. 8j+7, i.e. one 4-byte word of every head's codes, and the 4 lanes of
// an aligned quad together own one 32-element scale group.
constexpr int kFoldRowsPerWG = 16;

__global__ __launch_bounds__(256) void fold_query_kernel(QueryArgs q, uint8_t* __restrict__ out) {
  const int row = blockIdx.x * kFoldRowsPerWG + (threadIdx.x >> 4);
  const bool live = row < q.rows;
  const int rr = live ? row : q.rows - 1;   // dead lanes compute a copy and store nothing
  const int j = threadIdx.x & 15;
  const int g = j >> 2;
  const uint32_t* vrow = reinterpret_cast<const uint32_t*>(q.vals + (size_t)rr * q.heads * kValBytes) + j;
  const uint8_t* srow = q.scales + (size_t)rr * q.heads * kScaleBytes + g;
  const float* wrow = q.w + (size_t)rr * q.heads;
  double r[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) r[k] = 0.0;
  // qf = sum_h (w_h / 2) q_h, exact products, fp64 sums in head order
#pragma unroll 4
  for (int h = 0; h < q.heads; ++h) {
    const uint32_t v = vrow[h * (kValBytes / 4)];
    // (w/2) * 2^(scale - 127), halved again because the codes below are 2|x|
    const double ws = ldexp(0.5 * (double)wrow[h], (int)srow[h * kScaleBytes] - 128);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int code = (v >> (4 * k)) & 15;
      const int m2 = (0xC8643210u >> (4 * (code & 7))) & 15;   // 2 * |e2m1 value|
      r[k] = fma(ws, (double)((code & 8) ? -m2 : m2), r[k]);
    }
  }
  uint8_t* orow = out + (size_t)row * kFoldRowBytes;
  for (int t = 0; t < kFoldTerms; ++t) {
    double m = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmax(m, fabs(r[k]));
    m = fmax(m, dpp_d<0xB1>(m));   // quad_perm [1,0,3,2]
    m = fmax(m, dpp_d<0x4E>(m));   // quad_perm [2,3,0,1]: the group's max
    int e = -127;
    if (m > 0.0) {
      int x;
      const double f = frexp(m / 6.0, &x);  // m / 6 = f * 2^x, f in [0.5, 1)
      e = f > 0.5 ? x : x - 1;               // ceil(log2(m / 6))
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
    }
    uint32_t codes = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      int code = e2m1_nearest(ldexp(fabs(r[k]), -e));
      if (r[k] < 0.0 && code != 0) code |= 8;
      r[k] -= ldexp(e2m1_value(code), e);
      codes |= (uint32_t)code << (4 * k);
    }
    if (live) {
      *reinterpret_cast<uint32_t*>(orow + t * kValBytes + 4 * j) = codes;
      if ((j & 3) == 0) orow[kFoldTerms * kValBytes + t * kScaleBytes + g] = (uint8_t)(e + 127);
    }
  }
}

hipError_t launch_fold_query(const QueryArgs& q, uint8_t* out, hipStream_t st) {
  if (q.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(fold_query_kernel, dim3((q.rows + kFoldRowsPerWG - 1) / kFoldRowsPerWG), dim3(256), 0,
                     st, q, out);
  return hipGetLastError();
}

}  // namespace idxk
