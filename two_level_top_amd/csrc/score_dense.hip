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
//   A wave keeps its two rows' queries (64 heads x 128 dims as MXFP4) in
//   registers and streams 16-position K tiles straight from the paged pool:
//   lane l loads 16 bytes of position (l % 16) of the tile -- 1 KB
//   contiguous per tile since a tile never crosses a page.
// Rows of a wave that belong to different requests are scored one after
// the other (their keys come from different pages).
#include "score_common.h"

namespace idxk {

constexpr int kDenseChunk = 1024;
constexpr int kDenseWaves = 4;
constexpr int kDenseRowsPerWave = 2;

template <int HB>
__global__ __launch_bounds__(256) void score_dense_kernel(QueryArgs q, PoolArgs kp,
                                                          const int32_t* __restrict__ req,
                                                          const int32_t* __restrict__ len,
                                                          float* __restrict__ S, int64_t ld,
                                                          int nchunks) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int chunk = blockIdx.x % nchunks;
  const int rg = blockIdx.x / nchunks;
  const int r0 = (rg * kDenseWaves + wave) * kDenseRowsPerWave;
  if (r0 >= q.rows) return;
  const int r1 = r0 + 1 < q.rows ? r0 + 1 : -1;
  // lengths are clamped to [0, min(ld, max_pages * 64)] so that a bad length
  // can never address outside S or the page table
  const int64_t lcap64 = min(ld, (int64_t)kp.max_pages * kPage);
  const int lcap = (int)min(lcap64, (int64_t)0x7fffffff);
  const int req0 = clamp_req(req[r0], kp.num_req), len0 = min(max(len[r0], 0), lcap);
  const int req1 = r1 >= 0 ? clamp_req(req[r1], kp.num_req) : -1;
  const int len1 = r1 >= 0 ? min(max(len[r1], 0), lcap) : 0;
  const bool joint = r1 >= 0 && req1 == req0;
  const int c0 = chunk * kDenseChunk;

  for (int pass = 0; pass < 2; ++pass) {
    int ra, rb, rq, la, lb;
    if (pass == 0) {
      ra = r0; rb = joint ? r1 : -1; rq = req0; la = len0; lb = joint ? len1 : 0;
    } else {
      if (joint || r1 < 0) break;
      ra = r1; rb = -1; rq = req1; la = len1; lb = 0;
    }
    const int maxlen = max(la, lb);
    if (c0 >= maxlen) continue;
    const int cend = min(c0 + kDenseChunk, maxlen);
    RowFrag<HB> fa, fb;
    load_row(q, ra, lane, fa);
    if (rb >= 0) load_row(q, rb, lane, fb);
    const int32_t* pt = kp.page_table + (int64_t)rq * kp.max_pages;
    float* Sa = S + (int64_t)ra * ld;
    float* Sb = S + (int64_t)(rb >= 0 ? rb : ra) * ld;

    for (int base = c0; base < cend; base += 64) {
      float pa[4], pb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int p0 = base + 16 * t;
        if (p0 < cend) {
          const int64_t page = clamp_page(pt[min(p0 / kPage, kp.max_pages - 1)], kp.num_pages);
          const int slot = (p0 % kPage) + (lane & 15);
          const uint8_t* pg = kp.pool + page * kPageBytes;
          const uint4 b = *reinterpret_cast<const uint4*>(pg + slot * kValBytes + (lane >> 4) * 16);
          const int sb = pg[kPageValBytes + slot * kScaleBytes + (lane >> 4)];
          pa[t] = tile_partial<HB>(fa, b, sb);
          pb[t] = rb >= 0 ? tile_partial<HB>(fb, b, sb) : 0.f;
        } else {
          pa[t] = 0.f;
          pb[t] = 0.f;
        }
      }
      const int p = base + lane;
      const float ta = reduce_scatter4(pa[0], pa[1], pa[2], pa[3]);
      if (p < la) Sa[p] = ta;
      if (rb >= 0) {
        const float tb = reduce_scatter4(pb[0], pb[1], pb[2], pb[3]);
        if (p < lb) Sb[p] = tb;
      }
    }
  }
}

hipError_t launch_score_dense(const QueryArgs& q, const PoolArgs& kp, const int32_t* req,
                              const int32_t* len, float* S, int64_t ld, hipStream_t st) {
  const int rows_per_wg = kDenseWaves * kDenseRowsPerWave;
  const int64_t groups = (q.rows + rows_per_wg - 1) / rows_per_wg;
  const int nchunks = (int)((ld + kDenseChunk - 1) / kDenseChunk);
  const int64_t grid = groups * nchunks;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int hb = (q.heads + 15) / 16;
  switch (hb) {
    case 1: hipLaunchKernelGGL(score_dense_kernel<1>, dim3((unsigned)grid), dim3(256), 0, st, q, kp, req, len, S, ld, nchunks); break;
    case 2: hipLaunchKernelGGL(score_dense_kernel<2>, dim3((unsigned)grid), dim3(256), 0, st, q, kp, req, len, S, ld, nchunks); break;
    case 3: hipLaunchKernelGGL(score_dense_kernel<3>, dim3((unsigned)grid), dim3(256), 0, st, q, kp, req, len, S, ld, nchunks); break;
    default: hipLaunchKernelGGL(score_dense_kernel<4>, dim3((unsigned)grid), dim3(256), 0, st, q, kp, req, len, S, ld, nchunks); break;
  }
  return hipGetLastError();
}

}  // namespace idxk
