// Shared pieces of the two MXFP4 score kernels (dense source, paged sparse
// consumer): query fragments held in registers and the per-tile epilogue.
//
// The score of a query row against a key position is
//     sum_h w[h] * max(0, dot(q[h], k))
// (the head-weighted ReLU "MQA logits" of the DeepSeek-V4.1 index layer).
// On gfx950 one v_mfma_scale_f32_16x16x128_f8f6f4 computes the dot products of
// 16 heads against 16 key positions over all 128 dimensions, applying the
// ue8m0 scales of both operands in hardware.  Heads sit on the M axis, so a
// lane receives 4 heads of one position and the ReLU + weighted head sum is
// done in-lane; the last 4-way sum over lane groups is done once per 4 tiles
// by reduce_scatter4, which also leaves 64 consecutive positions in the 64
// lanes for a coalesced store.
#pragma once

#include "idx_internal.h"

namespace idxk {

// Register-resident query of one row: HB blocks of 16 heads.
template <int HB>
struct RowFrag {
  uint4 a[HB];      // A operand: 32 e2m1 codes of head (l % 16), group (l / 16)
  int sa[HB];       // that group's ue8m0 scale
  float w[HB][4];   // weights of the heads 4 * (l / 16) + v this lane accumulates
};

template <int HB>
__device__ __forceinline__ void load_row(const QueryArgs& q, int r, int lane, RowFrag<HB>& f) {
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
      f.w[hb][v] = hw < q.heads ? q.w[(size_t)r * q.heads + hw] : 0.f;
    }
  }
}

// This lane's share of sum_h w[h] * relu(dot) for its tile column: 4 * HB
// heads.  Four independent accumulation chains keep the FMA latency hidden.
template <int HB>
__device__ __forceinline__ float tile_partial(const RowFrag<HB>& f, uint4 b, int sb) {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    acc = mfma_fp4_16x16x128(f.a[hb], b, f.sa[hb], sb, acc);
    s0 = fmaf(f.w[hb][0], fmaxf(acc[0], 0.f), s0);
    s1 = fmaf(f.w[hb][1], fmaxf(acc[1], 0.f), s1);
    s2 = fmaf(f.w[hb][2], fmaxf(acc[2], 0.f), s2);
    s3 = fmaf(f.w[hb][3], fmaxf(acc[3], 0.f), s3);
  }
  return (s0 + s1) + (s2 + s3);
}

}  // namespace idxk
