// Shared pieces of the two MXFP4 score kernels (dense source, paged sparse
// consumer): query fragments held in registers and the per-tile epilogue.
//
// The score of a query row against a key position is
//     sum_h w[h] * max(0, dot(q[h], k))
// (the head-weighted ReLU "MQA logits" of the DeepSeek-V4.1 index layer).
// On gfx950 one v_mfma_scale_f32_16x16x128_f8f6f4 computes the dot products of
// 16 heads against 16 key positions over all 128 dimensions, applying the
// ue8m0 scales of both operands in hardware.  Heads sit on the M axis, so a
// lane receives 4 heads of one position.
//
// Epilogue: with relu(s) = (s + |s|) / 2 the score is
//     sum_h (w[h]/2) |s_h|  +  qf . k,      qf = sum_h (w[h]/2) q[h]
// (fold_query.hip writes qf as 16 MXFP4 terms).  The qf block is one more
// MFMA whose 4 outputs per lane seed the four accumulation chains; each head
// then costs a single FMA with an |x| source modifier.  The last 4-way sum
// over lane groups is done once per 4 tiles by reduce_scatter4, which also
// leaves 64 consecutive positions in the 64 lanes for a coalesced store.
#pragma once

#include "idx_internal.h"

namespace idxk {

// Register-resident query of one row: HB blocks of 16 heads plus the folded
// block.
template <int HB>
struct RowFrag {
  uint4 a[HB];      // A operand: 32 e2m1 codes of head (l % 16), group (l / 16)
  int sa[HB];       // that group's ue8m0 scale
  float w[HB][4];   // half the weights of the heads 4 * (l / 16) + v of each block
  uint4 at;         // folded query: term (l % 16), group (l / 16)
  int st;
};

template <int HB>
__device__ __forceinline__ void load_row(const QueryArgs& q, const uint8_t* fold, int r, int lane,
                                         RowFrag<HB>& f) {
  const int g = lane >> 4;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int h = hb * 16 + (lane & 15);
    if (h < q.heads) {
      const size_t base = (size_t)r * q.heads + h;
      f.a[hb] = *reinterpret_cast<const uint4*>(q.vals + base * kValBytes + g * 16);
      f.sa[hb] = q.scales[base * kScaleBytes + g];
    } else {
      f.a[hb] = make_uint4(0u, 0u, 0u, 0u);
      f.sa[hb] = 127;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int hw = hb * 16 + 4 * g + v;
      f.w[hb][v] = hw < q.heads ? 0.5f * q.w[(size_t)r * q.heads + hw] : 0.f;
    }
  }
  const uint8_t* fr = fold + (size_t)r * kFoldRowBytes;
  f.at = *reinterpret_cast<const uint4*>(fr + (lane & 15) * kValBytes + g * 16);
  f.st = fr[kFoldTerms * kValBytes + (lane & 15) * kScaleBytes + g];
}

// The HB + 1 MFMAs of one tile (folded block first) ...
template <int HB>
__device__ __forceinline__ void tile_mfma(const RowFrag<HB>& f, uint4 b, int sb, v4f (&acc)[HB + 1]) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  acc[0] = mfma_fp4_16x16x128(f.at, b, f.st, sb, zero);
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) acc[hb + 1] = mfma_fp4_16x16x128(f.a[hb], b, f.sa[hb], sb, zero);
}

// ... and their epilogue: this lane's share of the score for its tile column,
// the folded block's 4 terms plus 4 * HB heads, in four independent chains.
template <int HB>
__device__ __forceinline__ float tile_epilogue(const RowFrag<HB>& f, const v4f (&acc)[HB + 1]) {
  float s0 = acc[0][0], s1 = acc[0][1], s2 = acc[0][2], s3 = acc[0][3];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    s0 = fmaf(f.w[hb][0], fabsf(acc[hb + 1][0]), s0);
    s1 = fmaf(f.w[hb][1], fabsf(acc[hb + 1][1]), s1);
    s2 = fmaf(f.w[hb][2], fabsf(acc[hb + 1][2]), s2);
    s3 = fmaf(f.w[hb][3], fabsf(acc[hb + 1][3]), s3);
  }
  return (s0 + s1) + (s2 + s3);
}

// This lane's share of the score for its tile column (one tile, one row).
template <int HB>
__device__ __forceinline__ float tile_partial(const RowFrag<HB>& f, uint4 b, int sb) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  const v4f lin = mfma_fp4_16x16x128(f.at, b, f.st, sb, zero);
  float s0 = lin[0], s1 = lin[1], s2 = lin[2], s3 = lin[3];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const v4f acc = mfma_fp4_16x16x128(f.a[hb], b, f.sa[hb], sb, zero);
    s0 = fmaf(f.w[hb][0], fabsf(acc[0]), s0);
    s1 = fmaf(f.w[hb][1], fabsf(acc[1]), s1);
    s2 = fmaf(f.w[hb][2], fabsf(acc[2]), s2);
    s3 = fmaf(f.w[hb][3], fabsf(acc[3]), s3);
  }
  return (s0 + s1) + (s2 + s3);
}

}  // namespace idxk
