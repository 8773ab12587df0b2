// idx_score_sparse_paged: a consumer layer's scores at its candidate positions
// only, read straight from the paged MXFP4 index-K pool (the sglang PR
// "[DSv4.1] Score prefill consumer index layers on candidate blocks with
// DeepGEMM", Design, "Level two": scores [tokens, kb * 8] in ascending block
// order; no dense row is formed).
//
// The work list (built by idx_expand_candidates) holds one unit per 64
// candidate blocks of a row.  A wave takes a unit, keeps the row's query in
// registers and walks 2 candidate blocks (16 positions) per MFMA tile: lane l
// gathers 16 bytes of position (l % 8) of block (l % 16) / 8 -- each block is
// 512 contiguous value bytes and 32 scale bytes of one pool page.
#include "score_common.h"

namespace idxk {

constexpr int kSparseWaves = 4;

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
  const int wave = threadIdx.x >> 6;
  const int max_units = q.rows * ((kb + kUnitBlocks - 1) / kUnitBlocks);
  const int nunits = min(sched[0], max_units);
  for (int u = blockIdx.x * kSparseWaves + wave; u < nunits; u += gridDim.x * kSparseWaves) {
    const int row = sched[4 + 2 * u];
    const int first = sched[5 + 2 * u];
    if (row < 0 || row >= q.rows || first < 0) continue;   // not a work list this table built
    const int nk = min(max(n_kept[row], 0), kb);
    const int vl = min(valid_len[row], nk * kBlock);
    const int last = min(first + kUnitBlocks, nk);
    RowFrag<HB> f;
    load_row(q, fold, row, lane, f);
    const int32_t* ph = phys + (int64_t)row * kb;
    float* Tr = T + (int64_t)row * ld;
    for (int bb = first; bb < last; bb += 8) {
      float p[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int blk0 = bb + 2 * t;
        if (blk0 < last) {
          const int bi = blk0 + ((lane & 15) >> 3);
          uint4 b = make_uint4(0u, 0u, 0u, 0u);
          int sb = 127;
          if (bi < last) {
            const int pb = ph[bi];
            const int64_t page = clamp_page(pb >> 3, num_pages);
            const int slot = (pb & 7) * kBlock + (lane & 7);
            const uint8_t* pg = pool + page * kPageBytes;
            b = *reinterpret_cast<const uint4*>(pg + slot * kValBytes + (lane >> 4) * 16);
            sb = pg[kPageValBytes + slot * kScaleBytes + (lane >> 4)];
          }
          p[t] = tile_partial<HB>(f, b, sb);
        } else {
          p[t] = 0.f;
        }
      }
      const float tot = reduce_scatter4(p[0], p[1], p[2], p[3]);
      const int c = bb * kBlock + lane;
      if (c < vl) Tr[c] = tot;
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
