// idx_score_dense: the source layer's fp32 score matrix over every reachable
// position of each row (the dense score matrix of the sglang PR "[DSv4.1]
// Score prefill consumer index layers on candidate blocks with DeepGEMM",
// Motivation; the vLLM sparse_attn_indexer page's fp8_fp4_mqa_logits over
// each row's [ks, ke)).
//
// Work decomposition (gfx950: 256 CUs in 8 XCDs, wave64):
//   workgroup = 4 waves, 8 query rows (2 per wave), 1024 positions.
//   workgroup id -> (row group = id / nchunks, chunk = id % nchunks), so
//   consecutive ids -- which the dispatcher spreads over the 8 XCDs -- share
//   a row group and walk different position chunks: each XCD keeps 1/8 of
//   the K pool hot in its L2 and re-reads a row group's query from L2.
//   A wave keeps its two rows' queries (64 heads x 128 dims as MXFP4, plus
//   the folded query block) in registers and streams K one pool page (64
//   positions, 4 MFMA tiles) at a time straight from the paged pool: lane l
//   loads 16 bytes of position (l % 16) of each tile, so a page's 4 KB of
//   codes is read with 4 fully coalesced loads per wave.
// Rows of a wave that belong to different requests are scored one after
// the other (their keys come from different pages).
#include "score_common.h"

namespace idxk {

constexpr int kDenseChunk = 1024;
constexpr int kDenseWaves = 4;
constexpr int kDenseRowsPerWave = 2;

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// K operands of one pool page: 4 MFMA tiles of 16 positions.
struct PageOps {
  uint4 b[4];
  int sb[4];
};

__device__ __forceinline__ void load_page(const uint8_t* pg, int voff, int soff, PageOps& o) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    o.b[t] = *reinterpret_cast<const uint4*>(pg + voff + t * 16 * kValBytes);
    o.sb[t] = pg[soff + t * 16 * kScaleBytes];
  }
}

// Score NR (1 or 2) rows of one request against positions [c0, cend) (c0 on
// a page boundary, at most 16 pages).  Every tile of a page is computed;
// positions past a row's length are never stored.
//
// Software pipeline: the MFMAs of tile i+1 are issued before the epilogue
// FMAs of tile i, so the matrix core and the VALU work at the same time
// within one wave (the epilogue costs about as many cycles as the MFMAs).
template <int HB, int NR>
__device__ __forceinline__ void score_rows(const RowFrag<HB> (&f)[2], float* const (&Srow)[2],
                                           const int (&lens)[2], const uint8_t* pool,
                                           int num_pages, const int32_t* pt, int max_pages,
                                           int c0, int cend, int lane) {
  const int voff = (lane & 15) * kValBytes + (lane >> 4) * 16;
  const int soff = kPageValBytes + (lane & 15) * kScaleBytes + (lane >> 4);
  // the chunk's page ids, one per lane, read back with readlane
  const int npg = (cend - c0 + kPage - 1) / kPage;
  const int pid = (int)clamp_page(pt[min(c0 / kPage + min(lane, npg - 1), max_pages - 1)], num_pages);
  auto page_ptr = [&](int i) {
    return pool + (int64_t)__builtin_amdgcn_readlane(pid, i) * kPageBytes;
  };
  PageOps cur, nxt;
  load_page(page_ptr(0), voff, soff, cur);
  for (int i = 0; i < npg; ++i) {
    load_page(page_ptr(min(i + 1, npg - 1)), voff, soff, nxt);
    float part[NR][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v4f acc[NR][HB + 1];
#pragma unroll
      for (int r = 0; r < NR; ++r) tile_mfma<HB>(f[r], cur.b[t], cur.sb[t], acc[r]);
#pragma unroll
      for (int r = 0; r < NR; ++r) part[r][t] = tile_epilogue<HB>(f[r], acc[r]);
    }
    const int p = c0 + i * kPage + lane;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float tot = reduce_scatter4(part[r][0], part[r][1], part[r][2], part[r][3]);
      if (p < lens[r]) Srow[r][p] = tot;
    }
    cur = nxt;
  }
}

template <int HB>
__global__ __launch_bounds__(256) void score_dense_kernel(QueryArgs q, const uint8_t* __restrict__ fold,
                                                          PoolArgs kp,
                                                          const int32_t* __restrict__ req,
                                                          const int32_t* __restrict__ len,
                                                          float* __restrict__ S, int64_t ld,
                                                          int nchunks) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int chunk = blockIdx.x % nchunks;
  const int rg = blockIdx.x / nchunks;
  const int r0 = (rg * kDenseWaves + wave) * kDenseRowsPerWave;
  if (r0 >= q.rows) return;
  const int r1 = r0 + 1 < q.rows ? r0 + 1 : -1;
  // lengths are clamped to [0, min(ld, max_pages * 64)] so that a bad length
  // can never address outside S or the page table
  const int64_t lcap64 = min(ld, (int64_t)kp.max_pages * kPage);
  const int lcap = (int)min(lcap64, (int64_t)0x7fffffff);
  const int req0 = uniform(clamp_req(req[r0], kp.num_req));
  const int len0 = uniform(min(max(len[r0], 0), lcap));
  const int req1 = r1 >= 0 ? uniform(clamp_req(req[r1], kp.num_req)) : -1;
  const int len1 = r1 >= 0 ? uniform(min(max(len[r1], 0), lcap)) : 0;
  const int c0 = chunk * kDenseChunk;
  RowFrag<HB> f[2];
  float* Srow[2];
  int lens[2];
  if (r1 >= 0 && req1 == req0) {  // both rows read the same keys
    const int cend = min(c0 + kDenseChunk, max(len0, len1));
    if (c0 >= cend) return;
    load_row(q, fold, r0, lane, f[0]);
    load_row(q, fold, r1, lane, f[1]);
    Srow[0] = S + (int64_t)r0 * ld;
    Srow[1] = S + (int64_t)r1 * ld;
    lens[0] = len0;
    lens[1] = len1;
    score_rows<HB, 2>(f, Srow, lens, kp.pool, kp.num_pages, kp.page_table + (int64_t)req0 * kp.max_pages,
                      kp.max_pages, c0, cend, lane);
    return;
  }
  for (int i = 0; i < 2; ++i) {  // rows of different requests, one at a time
    const int r = i == 0 ? r0 : r1;
    if (r < 0) break;
    const int L = i == 0 ? len0 : len1;
    const int rq = i == 0 ? req0 : req1;
    const int cend = min(c0 + kDenseChunk, L);
    if (c0 >= cend) continue;
    load_row(q, fold, r, lane, f[0]);
    Srow[0] = S + (int64_t)r * ld;
    Srow[1] = Srow[0];
    lens[0] = L;
    lens[1] = 0;
    score_rows<HB, 1>(f, Srow, lens, kp.pool, kp.num_pages, kp.page_table + (int64_t)rq * kp.max_pages,
                      kp.max_pages, c0, cend, lane);
  }
}

hipError_t launch_score_dense(const QueryArgs& q, const uint8_t* fold, const PoolArgs& kp,
                              const int32_t* req, const int32_t* len, float* S, int64_t ld,
                              hipStream_t st) {
  const int rows_per_wg = kDenseWaves * kDenseRowsPerWave;
  const int64_t groups = (q.rows + rows_per_wg - 1) / rows_per_wg;
  const int nchunks = (int)((ld + kDenseChunk - 1) / kDenseChunk);
  const int64_t grid = groups * nchunks;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int hb = (q.heads + 15) / 16;
  switch (hb) {
    case 1: hipLaunchKernelGGL(score_dense_kernel<1>, dim3((unsigned)grid), dim3(256), 0, st, q, fold, kp, req, len, S, ld, nchunks); break;
    case 2: hipLaunchKernelGGL(score_dense_kernel<2>, dim3((unsigned)grid), dim3(256), 0, st, q, fold, kp, req, len, S, ld, nchunks); break;
    case 3: hipLaunchKernelGGL(score_dense_kernel<3>, dim3((unsigned)grid), dim3(256), 0, st, q, fold, kp, req, len, S, ld, nchunks); break;
    default: hipLaunchKernelGGL(score_dense_kernel<4>, dim3((unsigned)grid), dim3(256), 0, st, q, fold, kp, req, len, S, ld, nchunks); break;
  }
  return hipGetLastError();
}

}  // namespace idxk
