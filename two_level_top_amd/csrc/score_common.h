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
// block.  The ue8m0 scales of the blocks share one register (byte hb, picked
// by the MFMA's scale byte select), and the row's half weights share one
// register too: lane 16 g + 4 hb + v holds the weight of head 16 hb + 4 g + v,
// which every lane of row g (the 16 lanes that receive heads 4 g .. 4 g + 3 of
// each block) reads with a DPP row broadcast inside its FMA.
template <int HB>
struct RowFrag {
  uint4 a[HB];      // A operand: 32 e2m1 codes of head (l % 16), group (l / 16)
  int sa;           // byte hb: that group's ue8m0 scale in block hb
  float w;          // half weights, laid out as above
  uint4 at;         // folded query: term (l % 16), group (l / 16)
  int st;
};

// FOLD: also load the row's own folded-query block (the dense kernel shares
// one block between two rows instead, see PairFold)
template <int HB, bool FOLD = true>
__device__ __forceinline__ void load_row(const QueryArgs& q, const uint8_t* fold, int r, int lane,
                                         RowFrag<HB>& f) {
  const int g = lane >> 4;
  f.sa = 0;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int h = hb * 16 + (lane & 15);
    int sc = 127;
    if (h < q.heads) {
      const size_t base = (size_t)r * q.heads + h;
      f.a[hb] = *reinterpret_cast<const uint4*>(q.vals + base * kValBytes + g * 16);
      sc = q.scales[base * kScaleBytes + g];
    } else {
      f.a[hb] = make_uint4(0u, 0u, 0u, 0u);
    }
    f.sa |= sc << (8 * hb);
  }
  {
    const int m = lane & 15;   // 4 hb + v
    const int hw = 16 * (m >> 2) + 4 * g + (m & 3);
    f.w = (m >> 2) < HB && hw < q.heads ? 0.5f * q.w[(size_t)r * q.heads + hw] : 0.f;
    asm volatile("s_nop 1" : "+v"(f.w));   // VALU write -> DPP read of f.w
  }
  if (FOLD) {
    const uint8_t* fr = fold + (size_t)r * kFoldRowBytes;
    f.at = *reinterpret_cast<const uint4*>(fr + (lane & 15) * kValBytes + g * 16);
    f.st = fr[kFoldTerms * kValBytes + (lane & 15) * kScaleBytes + g];
  }
}

// The folded queries of a pair of rows as one 16-row MFMA block holding the
// first kPairFoldTerms terms of each row: M row m is term 2 (m / 4) + m % 2 of
// row (m / 2) % 2 of the pair.  The MFMA then gives the lanes of k-group g the
// fold values of terms 2g and 2g + 1 of row 0 in outputs 0 and 1 and of row 1
// in outputs 2 and 3, and the 4-way sum over lane groups adds each row's 8
// terms.  Eight of the 16 greedy terms leave a fold residual whose effect on a
// score is below 1e-5 on these inputs (long chunk K, 8.4M scores: at most
// 4.4e-6); sharing the block saves half an MFMA per tile and row, and two of
// the epilogue's three adds.  r1 < 0: the second half is zero (one row).
constexpr int kPairFoldTerms = 8;

struct PairFold {
  uint4 at;
  int st;
};

__device__ __forceinline__ void load_pair_fold(const uint8_t* fold, int r0, int r1, int lane,
                                               PairFold& p) {
  const int m = lane & 15, g = lane >> 4;
  const int r = ((m >> 1) & 1) ? r1 : r0;
  const int term = 2 * (m >> 2) + (m & 1);
  if (r < 0) {
    p.at = make_uint4(0u, 0u, 0u, 0u);
    p.st = 127;
    return;
  }
  const uint8_t* fr = fold + (size_t)r * kFoldRowBytes;
  p.at = *reinterpret_cast<const uint4*>(fr + term * kValBytes + g * 16);
  p.st = fr[kFoldTerms * kValBytes + term * kScaleBytes + g];
}

// MFMA of query block HBI (scale byte HBI of the packed scales)
template <int HB, int HBI>
__device__ __forceinline__ v4f block_mfma(const RowFrag<HB>& f, uint4 b, int sb) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  v8i av = {(int)f.a[HBI].x, (int)f.a[HBI].y, (int)f.a[HBI].z, (int)f.a[HBI].w, 0, 0, 0, 0};
  v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, zero, 4, 4, HBI, f.sa, 0, sb);
}

// s += (the half weight in lane M of this lane's 16-lane row) * |x|
template <int M>
__device__ __forceinline__ void fma_bcast_abs(float& s, float w, float x) {
  asm("v_fmac_f32_dpp %0, %1, |%2| row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(s) : "v"(w), "v"(x), "i"(M));
}

template <int HB, int HBI = 0>
__device__ __forceinline__ void tile_mfma_blocks(const RowFrag<HB>& f, uint4 b, int sb, v4f (&acc)[HB + 1]) {
  if constexpr (HBI < HB) {
    acc[HBI + 1] = block_mfma<HB, HBI>(f, b, sb);
    tile_mfma_blocks<HB, HBI + 1>(f, b, sb, acc);
  }
}

template <int HB, int HBI = 0>
__device__ __forceinline__ void epilogue_blocks(float& s0, float& s1, float& s2, float& s3, float w,
                                                const v4f (&acc)[HB + 1]) {
  if constexpr (HBI < HB) {
    fma_bcast_abs<4 * HBI + 0>(s0, w, acc[HBI + 1][0]);
    fma_bcast_abs<4 * HBI + 1>(s1, w, acc[HBI + 1][1]);
    fma_bcast_abs<4 * HBI + 2>(s2, w, acc[HBI + 1][2]);
    fma_bcast_abs<4 * HBI + 3>(s3, w, acc[HBI + 1][3]);
    epilogue_blocks<HB, HBI + 1>(s0, s1, s2, s3, w, acc);
  }
}

// two chains: heads 4 hb + {0, 2} into s0, 4 hb + {1, 3} into s1
template <int HB, int HBI = 0>
__device__ __forceinline__ void epilogue_pairs(float& s0, float& s1, float w, const v4f (&acc)[HB + 1]) {
  if constexpr (HBI < HB) {
    fma_bcast_abs<4 * HBI + 0>(s0, w, acc[HBI + 1][0]);
    fma_bcast_abs<4 * HBI + 1>(s1, w, acc[HBI + 1][1]);
    fma_bcast_abs<4 * HBI + 2>(s0, w, acc[HBI + 1][2]);
    fma_bcast_abs<4 * HBI + 3>(s1, w, acc[HBI + 1][3]);
    epilogue_pairs<HB, HBI + 1>(s0, s1, w, acc);
  }
}

// The HB + 1 MFMAs of one tile (folded block first) ...
template <int HB>
__device__ __forceinline__ void tile_mfma(const RowFrag<HB>& f, uint4 b, int sb, v4f (&acc)[HB + 1]) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  acc[0] = mfma_fp4_16x16x128(f.at, b, f.st, sb, zero);
  tile_mfma_blocks<HB>(f, b, sb, acc);
}

// ... and their epilogue: this lane's share of the score for its tile column,
// the folded block's 4 terms plus 4 * HB heads, in four independent chains.
// The FMAs below are inline assembly, which the compiler's hazard tracking
// does not see into: this passes the tile's MFMA results through one asm
// statement that waits out the MFMA-result-to-VALU wait states itself (12;
// the compiler itself keeps 8 between this MFMA and a VALU read of its
// result).
template <int HB>
__device__ __forceinline__ void settle(v4f (&acc)[HB + 1]) {
  if constexpr (HB == 1)
    asm volatile("s_nop 7\n\ts_nop 3" : "+v"(acc[0]), "+v"(acc[1]));
  else if constexpr (HB == 2)
    asm volatile("s_nop 7\n\ts_nop 3" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]));
  else if constexpr (HB == 3)
    asm volatile("s_nop 7\n\ts_nop 3" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
  else
    asm volatile("s_nop 7\n\ts_nop 3"
                 : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]));
}

// the head blocks' wait states only (acc[0] not read)
template <int HB>
__device__ __forceinline__ void settle_heads(v4f (&acc)[HB + 1]) {
  if constexpr (HB == 1)
    asm volatile("s_nop 7\n\ts_nop 3" : "+v"(acc[1]));
  else if constexpr (HB == 2)
    asm volatile("s_nop 7\n\ts_nop 3" : "+v"(acc[1]), "+v"(acc[2]));
  else if constexpr (HB == 3)
    asm volatile("s_nop 7\n\ts_nop 3" : "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
  else
    asm volatile("s_nop 7\n\ts_nop 3" : "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]));
}

// Epilogue of one row of a pair sharing a fold block.  FIRST (the pair's
// first row): acc[0] holds the pair's fold outputs; entries 0 and 1 seed this
// row's two chains, and entries 2 and 3 are handed out in seed0/seed1 for the
// second row.  Otherwise acc[0] is unused and seed0/seed1 seed the chains.
// Each chain takes 2 HB FMAs; one add joins them.
template <int HB, bool FIRST>
__device__ __forceinline__ float tile_epilogue_pair(const RowFrag<HB>& f, const v4f (&acc_in)[HB + 1],
                                                    float& seed0, float& seed1) {
  v4f acc[HB + 1];
#pragma unroll
  for (int i = 0; i <= HB; ++i) acc[i] = acc_in[i];
  float s0, s1;
  if constexpr (FIRST) {
    settle<HB>(acc);
    s0 = acc[0][0];
    s1 = acc[0][1];
    seed0 = acc[0][2];
    seed1 = acc[0][3];
  } else {
    settle_heads<HB>(acc);
    s0 = seed0;
    s1 = seed1;
  }
  epilogue_pairs<HB>(s0, s1, f.w, acc);
  return s0 + s1;
}

template <int HB>
__device__ __forceinline__ float tile_epilogue(const RowFrag<HB>& f, const v4f (&acc_in)[HB + 1]) {
  v4f acc[HB + 1];
#pragma unroll
  for (int i = 0; i <= HB; ++i) acc[i] = acc_in[i];
  settle<HB>(acc);
  float s0 = acc[0][0], s1 = acc[0][1], s2 = acc[0][2], s3 = acc[0][3];
  epilogue_blocks<HB>(s0, s1, s2, s3, f.w, acc);
  return (s0 + s1) + (s2 + s3);
}

}  // namespace idxk
