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
// max of lanes l and l ^ 16 (the swap returns, in every lane, the pair's
// even-row value in [0] and its odd-row value in [1])
__device__ __forceinline__ double max16_d(double v) {
  const auto lo = __builtin_amdgcn_permlane16_swap(__double2loint(v), __double2loint(v), false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap(__double2hiint(v), __double2hiint(v), false, false);
  return fmax(__hiloint2double((int)hi[0], (int)lo[0]), __hiloint2double((int)hi[1], (int)lo[1]));
}

// One query row per 128 lanes (two waves), lane d owning dimension d: the
// 32 lanes of an aligned half-wave form one scale group, so a group's
// largest residual is a 32-lane reduction and every step of the split runs
// on all 128 dimensions at once.  The row's codes, scales and weights
// (<= 4.6 KB) are first staged in LDS, so the head loop waits on one memory
// latency rather than one per unrolled batch (few rows, as in decode, are
// latency-bound).
constexpr int kFoldRowsPerWG = 2;
constexpr int kFoldMaxHeads = 64;

__global__ __launch_bounds__(256) void fold_query_kernel(QueryArgs q, uint8_t* __restrict__ out) {
  __shared__ uint4 stage[kFoldRowsPerWG][kFoldMaxHeads * (kValBytes + kScaleBytes + 4) / 16];
  const int half = threadIdx.x >> 7;
  const int row = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kFoldRowsPerWG + half));
  const bool live = row < q.rows;
  const int rr = live ? row : q.rows - 1;   // a dead half computes a copy and stores nothing
  const int d = threadIdx.x & 127;
  const int g = d >> 5;
  const int H = q.heads;
  // stage: codes [H][64] (16-byte loads: vals is 16-byte aligned), then
  // scales [H][4] and weights [H] (4-byte loads)
  uint8_t* sb = reinterpret_cast<uint8_t*>(stage[half]);
  const int vb = H * kValBytes, scb = H * kScaleBytes;
  const uint4* src_v = reinterpret_cast<const uint4*>(q.vals + (size_t)rr * vb);
  const uint32_t* src_s = reinterpret_cast<const uint32_t*>(q.scales + (size_t)rr * scb);
  const uint32_t* src_w = reinterpret_cast<const uint32_t*>(q.w + (size_t)rr * H);
  for (int i = d; i < vb / 16; i += 128) stage[half][i] = src_v[i];
  uint32_t* s32 = reinterpret_cast<uint32_t*>(sb + vb);
  if (d < H) {
    s32[d] = src_s[d];
    s32[H + d] = src_w[d];
  }
  __syncthreads();
  const uint8_t* vrow = sb + (d >> 1);
  const uint8_t* srow = sb + vb + g;
  const float* wrow = reinterpret_cast<const float*>(sb + vb + scb);
  const int nib = 4 * (d & 1);
  // qf[d] = sum_h (w_h / 2) q_h[d], exact products, fp64 sums in head order
  double r = 0.0;
#pragma unroll 8
  for (int h = 0; h < H; ++h) {
    const int code = (vrow[h * kValBytes] >> nib) & 15;
    // (w/2) * 2^(scale - 127), halved again because the codes below are 2|x|
    const double ws = ldexp(0.5 * (double)wrow[h], (int)srow[h * kScaleBytes] - 128);
    const int m2 = (0xC8643210u >> (4 * (code & 7))) & 15;   // 2 * |e2m1 value|
    r = fma(ws, (double)((code & 8) ? -m2 : m2), r);
  }
  uint8_t* orow = out + (size_t)row * kFoldRowBytes;
  for (int t = 0; t < kFoldTerms; ++t) {
    double m = fabs(r);
    m = fmax(m, dpp_d<0xB1>(m));    // quad_perm [1,0,3,2]
    m = fmax(m, dpp_d<0x4E>(m));    // quad_perm [2,3,0,1]
    m = fmax(m, dpp_d<0x141>(m));   // row_half_mirror: 8 lanes
    m = fmax(m, dpp_d<0x140>(m));   // row_mirror: 16 lanes
    m = max16_d(m);                 // the group's 32 lanes
    int e = -127;
    if (m > 0.0) {
      // ceil(log2(m / 6)) with m = f 2^x, f in [0.5, 1): x - 3 if f <= 3/4,
      // else x - 2 (no division)
      int x;
      const double f = frexp(m, &x);
      e = f <= 0.75 ? x - 3 : x - 2;
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
    }
    int code = e2m1_nearest(ldexp(fabs(r), -e));
    if (r < 0.0 && code != 0) code |= 8;
    r -= ldexp(e2m1_value(code), e);
    // byte d / 2 holds dimensions d (low nibble) and d + 1 (high nibble)
    const int partner = __builtin_amdgcn_mov_dpp(code, 0xB1, 0xf, 0xf, true);
    if (live && (d & 1) == 0) orow[t * kValBytes + (d >> 1)] = (uint8_t)(code | (partner << 4));
    if (live && (d & 31) == 0) orow[kFoldTerms * kValBytes + t * kScaleBytes + g] = (uint8_t)(e + 127);
  }
}

hipError_t launch_fold_query(const QueryArgs& q, uint8_t* out, hipStream_t st) {
  if (q.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(fold_query_kernel, dim3((q.rows + kFoldRowsPerWG - 1) / kFoldRowsPerWG), dim3(256), 0,
                     st, q, out);
  return hipGetLastError();
}

}  // namespace idxk
