// idx_score_sparse_paged: a consumer layer's scores at its candidate positions
// only, read straight from the paged MXFP4 index-K pool (the sglang PR
// "[DSv4.1] Score prefill consumer index layers on candidate blocks with
// DeepGEMM", Design, "Level two": scores [tokens, kb * 8] in ascending block
// order; no dense row is formed).
//
// The work list (built by idx_expand_candidates) holds one unit per 64
// candidate blocks of a row.  A wave takes a unit, keeps the row's query in
// registers, loads the unit's 64 pool-block ids once (one per lane) and walks
// 2 candidate blocks (16 positions) per MFMA tile, 4 tiles per group with the
// next group's K prefetched: lane l gathers 16 bytes of position (l % 8) of
// block (l % 16) / 8 -- each block is 512 contiguous value bytes and 32
// contiguous scale bytes of one pool page.
#include "score_common.h"

namespace idxk {

constexpr int kSparseWaves = 4;

// K operands of 4 tiles (8 candidate blocks) of one unit.
struct GroupOps {
  uint4 b[4];
  int sb[4];
};

// Lane l needs position (l % 8) of block 2 t + (l % 16) / 8 of the group;
// the blocks' pool ids come from the unit's id vector `pbv` (lane i holds
// candidate block first + i) by readlane, so no per-tile address load is
// on the critical path.  Blocks past `nblk` (the unit's end) read block 0 of
// the unit and are never stored.
// `bov` holds, in lane i, the byte offset of candidate block first + i's
// values in the pool (its scales sit at bov + 4096 - 7 * 64 * (block in page),
// folded into `sov`).
__device__ __forceinline__ void load_group(const uint8_t* pool, uint32_t bov, uint32_t sov, int g,
                                           int nblk, int lane, GroupOps& o) {
  const int slot = lane & 7;
  const bool half = (lane >> 3) & 1;
  const uint32_t voff = slot * kValBytes + (lane >> 4) * 16;
  const uint32_t soff = slot * kScaleBytes + (lane >> 4);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i0 = min(8 * g + 2 * t, nblk - 1), i1 = min(8 * g + 2 * t + 1, nblk - 1);
    const uint32_t v0 = __builtin_amdgcn_readlane(bov, i0), v1 = __builtin_amdgcn_readlane(bov, i1);
    const uint32_t s0 = __builtin_amdgcn_readlane(sov, i0), s1 = __builtin_amdgcn_readlane(sov, i1);
    o.b[t] = *reinterpret_cast<const uint4*>(pool + (half ? v1 : v0) + voff);
    o.sb[t] = pool[(half ? s1 : s0) + soff];
  }
}

template <int HB>
__global__ __launch_bounds__(256) void score_sparse_kernel(QueryArgs q,
                                                           const uint8_t* __restrict__ fold,
                                                           const uint8_t* __restrict__ pool,
                                                           int num_pages,
                                                           const int32_t* __restrict__ phys,
                                                           const int32_t* __restrict__ n_kept,
                                                           const int32_t* __restrict__ valid_len,
                                                           int kb, const int32_t* __restrict__ sched,
                                                           float* __restrict__ T, int64_t ld) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int max_units = q.rows * ((kb + kUnitBlocks - 1) / kUnitBlocks);
  const int nunits = min(sched[0], max_units);
  for (int u = blockIdx.x * kSparseWaves + wave; u < nunits; u += gridDim.x * kSparseWaves) {
    const int row = __builtin_amdgcn_readfirstlane(sched[4 + 2 * u]);
    const int first = __builtin_amdgcn_readfirstlane(sched[5 + 2 * u]);
    if (row < 0 || row >= q.rows || first < 0) continue;   // not a work list this table built
    const int nk = __builtin_amdgcn_readfirstlane(min(max(n_kept[row], 0), kb));
    const int vl = __builtin_amdgcn_readfirstlane(min(valid_len[row], nk * kBlock));
    const int nblk = min(kUnitBlocks, nk - first);   // candidate blocks of this unit
    if (nblk <= 0) continue;
    RowFrag<HB> f;
    load_row(q, fold, row, lane, f);
    // byte offsets of this lane's candidate block (pools are < 4 GiB here)
    const int pb = phys[(int64_t)row * kb + first + min(lane, nblk - 1)];
    const uint32_t pgo = (uint32_t)clamp_page(pb >> 3, num_pages) * (uint32_t)kPageBytes;
    const uint32_t bov = pgo + (uint32_t)(pb & 7) * (kBlock * kValBytes);
    const uint32_t sov = pgo + kPageValBytes + (uint32_t)(pb & 7) * (kBlock * kScaleBytes);
    float* Tr = T + (int64_t)row * ld + first * kBlock;
    const int ngroups = (nblk + 7) / 8;
    GroupOps cur, nxt;
    load_group(pool, bov, sov, 0, nblk, lane, cur);
    for (int g = 0; g < ngroups; ++g) {
      load_group(pool, bov, sov, min(g + 1, ngroups - 1), nblk, lane, nxt);
      float p[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v4f acc[HB + 1];
        tile_mfma<HB>(f, cur.b[t], cur.sb[t], acc);
        p[t] = tile_epilogue<HB>(f, acc);
      }
      const float tot = reduce_scatter4(p[0], p[1], p[2], p[3]);
      const int c = g * 64 + lane;   // column within the unit
      if (first * kBlock + c < vl && c < nblk * kBlock) Tr[c] = tot;
      cur = nxt;
    }
  }
}

hipError_t launch_score_sparse(const QueryArgs& q, const uint8_t* fold, const uint8_t* pool,
                               int num_pages,
                               const int32_t* phys, const int32_t* n_kept,
                               const int32_t* valid_len, int rows, int kb, const void* schedule,
                               float* T, int64_t ld, hipStream_t st) {
  const int64_t max_units = (int64_t)rows * ((kb + kUnitBlocks - 1) / kUnitBlocks);
  int64_t grid = (max_units + kSparseWaves - 1) / kSparseWaves;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) grid = 0x7fffffffLL;
  const int32_t* sched = static_cast<const int32_t*>(schedule);
  const int hb = (q.heads + 15) / 16;
  switch (hb) {
    case 1: hipLaunchKernelGGL(score_sparse_kernel<1>, dim3((unsigned)grid), dim3(256), 0, st, q, fold, pool, num_pages, phys, n_kept, valid_len, kb, sched, T, ld); break;
    case 2: hipLaunchKernelGGL(score_sparse_kernel<2>, dim3((unsigned)grid), dim3(256), 0, st, q, fold, pool, num_pages, phys, n_kept, valid_len, kb, sched, T, ld); break;
    case 3: hipLaunchKernelGGL(score_sparse_kernel<3>, dim3((unsigned)grid), dim3(256), 0, st, q, fold, pool, num_pages, phys, n_kept, valid_len, kb, sched, T, ld); break;
    default: hipLaunchKernelGGL(score_sparse_kernel<4>, dim3((unsigned)grid), dim3(256), 0, st, q, fold, pool, num_pages, phys, n_kept, valid_len, kb, sched, T, ld); break;
  }
  return hipGetLastError();
}

}  // namespace idxk
