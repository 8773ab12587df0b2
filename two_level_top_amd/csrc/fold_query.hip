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

// nearest e2m1 magnitude code of a in [0, 6] (ties to the even code), as a
// count of the grid midpoints below a (branch-free)
__device__ __forceinline__ int e2m1_nearest(double a) {
  return (int)(a > 0.25) + (int)(a >= 0.75) + (int)(a > 1.25) + (int)(a >= 1.75) + (int)(a > 2.5) +
         (int)(a >= 3.5) + (int)(a > 5.0);
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xf, 0xf, true);
  return __hiloint2double(hi, lo);
}

// One query row per wave, lane l owning dimensions 2 l and 2 l + 1 (the two
// nibbles of code byte l of every head): the 16 lanes of a DPP row form one
// scale group, so a group's largest residual is a 16-lane reduction and every
// step of the split runs on all 128 dimensions at once.  The row's code bytes
// are staged in LDS, together with the factor (w_h / 4) 2^(scale_hg - 127) of
// every (head, group) and a table giving each code byte's two values as
// 2 |e2m1| with its sign (hence the extra halving), so the head loop is two
// LDS reads and one FMA per dimension.  The fp64 operations and their order
// are those of a plain per-dimension loop over the heads.
constexpr int kFoldRowsPerWG = 4;
constexpr int kFoldMaxHeads = 64;

// 2 * (value of e2m1 code c), as the fp64 the head sums multiply
__device__ __forceinline__ double code_value2(int c) {
  const int m2 = (0xC8643210u >> (4 * (c & 7))) & 15;   // 2 * |e2m1 value|
  return (double)((c & 8) ? -m2 : m2);
}

// Several query batches (index layers) folded in one launch: workgroups
// [wg0[i], wg0[i + 1]) take batch i.  A step's layers are independent of each
// other, so folding them together fills the GPU where one layer's rows would
// not (decode: 64 rows = 16 workgroups per layer).
struct FoldBatch {
  QueryArgs q[kMaxFoldBatches];
  uint8_t* out[kMaxFoldBatches];
  int wg0[kMaxFoldBatches + 1];
  int n;
};

__global__ __launch_bounds__(256) void fold_query_kernel(FoldBatch fb) {
  __shared__ uint4 stage[kFoldRowsPerWG][kFoldMaxHeads * kValBytes / 16];
  __shared__ double hscale[kFoldRowsPerWG][kFoldMaxHeads * 4];
  __shared__ double2 pair[256];
  int bi = 0;   // this workgroup's batch (uniform)
  while (bi + 1 < fb.n && (int)blockIdx.x >= fb.wg0[bi + 1]) ++bi;
  const QueryArgs q = fb.q[bi];
  uint8_t* __restrict__ out = fb.out[bi];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int row = __builtin_amdgcn_readfirstlane((int)((blockIdx.x - fb.wg0[bi]) * kFoldRowsPerWG + wave));
  const bool live = row < q.rows;
  const int rr = live ? row : q.rows - 1;   // a dead wave computes a copy and stores nothing
  const int H = q.heads;
  const int g = lane >> 4;                  // scale group of this lane's two dimensions
  pair[threadIdx.x] = make_double2(code_value2(threadIdx.x & 15), code_value2(threadIdx.x >> 4));
  // codes [H][64] (16-byte loads: vals is 16-byte aligned) and, lane h, head
  // h's weight and 4 scales, all loads issued before any is used (few rows,
  // as in decode, are latency-bound); per (head, group) the factor
  // (w / 2) * 2^(scale - 127), halved again because the codes are 2 |x|
  const uint4* src_v = reinterpret_cast<const uint4*>(q.vals + (size_t)rr * H * kValBytes);
  constexpr int kLoads = kFoldMaxHeads * (kValBytes / 16) / 64;
  uint4 cv[kLoads];
#pragma unroll
  for (int k = 0; k < kLoads; ++k) cv[k] = src_v[min(lane + 64 * k, H * (kValBytes / 16) - 1)];
  uint32_t sc4;
  float w;
  {
    const int h = min(lane, H - 1);
    sc4 = *reinterpret_cast<const uint32_t*>(q.scales + ((size_t)rr * H + h) * kScaleBytes);
    w = q.w[(size_t)rr * H + h];
  }
  // (slots of heads >= H get copies and are never read)
#pragma unroll
  for (int k = 0; k < kLoads; ++k) stage[wave][lane + 64 * k] = cv[k];
#pragma unroll
  for (int gg = 0; gg < kScaleBytes; ++gg)
    hscale[wave][lane * kScaleBytes + gg] = ldexp(0.5 * (double)w, (int)((sc4 >> (8 * gg)) & 255u) - 128);
  __syncthreads();
  const uint8_t* cb = reinterpret_cast<const uint8_t*>(stage[wave]) + lane;
  const double* hs = hscale[wave] + g;
  // qf[d] = sum_h (w_h / 2) q_h[d], exact products, fp64 sums in head order
  double r0 = 0.0, r1 = 0.0;
#pragma unroll 8
  for (int h = 0; h < H; ++h) {
    const double f = hs[h * kScaleBytes];
    const double2 v = pair[cb[h * kValBytes]];
    r0 = fma(f, v.x, r0);
    r1 = fma(f, v.y, r1);
  }
  uint8_t* orow = out + (size_t)row * kFoldRowBytes;
  for (int t = 0; t < kFoldTerms; ++t) {
    double m = fmax(fabs(r0), fabs(r1));
    m = fmax(m, dpp_d<0xB1>(m));    // quad_perm [1,0,3,2]
    m = fmax(m, dpp_d<0x4E>(m));    // quad_perm [2,3,0,1]
    m = fmax(m, dpp_d<0x141>(m));   // row_half_mirror: 8 lanes
    m = fmax(m, dpp_d<0x140>(m));   // row_mirror: the group's 16 lanes
    int e = -127;
    if (m > 0.0) {
      // ceil(log2(m / 6)) with m = f 2^x, f in [0.5, 1): x - 3 if f <= 3/4,
      // else x - 2 (no division)
      int x;
      const double f = frexp(m, &x);
      e = f <= 0.75 ? x - 3 : x - 2;
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
    }
    int c0 = e2m1_nearest(ldexp(fabs(r0), -e));
    int c1 = e2m1_nearest(ldexp(fabs(r1), -e));
    if (r0 < 0.0 && c0 != 0) c0 |= 8;
    if (r1 < 0.0 && c1 != 0) c1 |= 8;
    r0 -= ldexp(code_value2(c0), e - 1);   // the code's value times 2^e, exactly
    r1 -= ldexp(code_value2(c1), e - 1);
    // byte l holds dimensions 2 l (low nibble) and 2 l + 1 (high nibble)
    if (live) orow[t * kValBytes + lane] = (uint8_t)(c0 | (c1 << 4));
    if (live && (lane & 15) == 0) orow[kFoldTerms * kValBytes + t * kScaleBytes + g] = (uint8_t)(e + 127);
  }
}

hipError_t launch_fold_queries(const QueryArgs* q, uint8_t* const* out, int n, hipStream_t st) {
  FoldBatch fb{};
  int wg = 0;
  fb.n = 0;
  for (int i = 0; i < n; ++i) {
    if (q[i].rows <= 0) continue;
    fb.q[fb.n] = q[i];
    fb.out[fb.n] = out[i];
    fb.wg0[fb.n] = wg;
    wg += (q[i].rows + kFoldRowsPerWG - 1) / kFoldRowsPerWG;
    ++fb.n;
  }
  fb.wg0[fb.n] = wg;
  if (wg == 0) return hipSuccess;
  hipLaunchKernelGGL(fold_query_kernel, dim3(wg), dim3(256), 0, st, fb);
  return hipGetLastError();
}

hipError_t launch_fold_query(const QueryArgs& q, uint8_t* out, hipStream_t st) {
  return launch_fold_queries(&q, &out, 1, st);
}

}  // namespace idxk
