// idx_score_dense: the source layer's fp32 score matrix over every reachable
// position of each row (the dense score matrix of the sglang PR "[DSv4.1]
// Score prefill consumer index layers on candidate blocks with DeepGEMM",
// Motivation; the vLLM sparse_attn_indexer page's fp8_fp4_mqa_logits over
// each row's [ks, ke)).
//
// Work decomposition (gfx950: 256 CUs in 8 XCDs, wave64):
//   workgroup = 4 waves, 8 query rows (2 per wave), 4096 positions (halved,
//   down to 256, while fewer than 2048 workgroups would run, as in decode).
//   workgroup id -> (row group = id / nchunks, chunk = id % nchunks rotated
//   by the row group, see the kernel), so consecutive ids -- which the
//   dispatcher spreads over the 8 XCDs -- share a row group and walk
//   different position chunks: each XCD keeps 1/8 of the K pool hot in its
//   L2 and re-reads a row group's query from L2.
//   A wave keeps its two rows' queries (64 heads x 128 dims as MXFP4, plus
//   the folded query block) in registers and streams K one pool page (64
//   positions, 4 MFMA tiles) at a time straight from the paged pool: lane l
//   loads 16 bytes of position (l % 16) of each tile, so a page's 4 KB of
//   codes is read with 4 fully coalesced loads per wave.  Two pages are in
//   flight (ping-pong registers, no copies); pages are read through a buffer
//   resource and scores/keys stored through resources sized to the row's
//   valid range, so the loop has no branches (out-of-range lanes are dropped
//   by the hardware).
// Rows of a wave that belong to different requests are scored one after
// the other (their keys come from different pages).
//
// Measured on MI355X (long chunk): this 16x16x128 form beat a 32x32x64 form
// of the same epilogue (2 waves per SIMD at 249 VGPRs) by about 12%, and
// issuing the next tile's MFMAs ahead of the epilogue or deferring the
// stores past the next loads gained nothing.  With the weights and block
// scales in one register each (score_common.h) and the two rows' tiles
// scored one after the other, the kernel fits 124 VGPRs and runs 4 waves per
// SIMD: 23.1 ms against 23.6 ms at 3 waves with both rows' MFMAs in flight.
//
// Fused block keys (the prefill PR's follow-up of folding the block amax into
// the score kernel): after the 4-way reduction each lane holds one score of
// 64 consecutive positions, so an aligned 8-lane DPP max gives the key of
// every block of the page without reading S back.  The keys equal what
// idx_amax8_varlen computes from the stored S (the max of the same fp32
// values; the newest block is +inf; rows with nblk <= skip are untouched).
#include "score_common.h"

namespace idxk {

// positions per workgroup: 4096, halved while fewer than kDenseTargetWGs
// workgroups would run (decode).  Longer chunks spread a wave's query loads
// and setup over more tiles: 4096 against 1024 took the long chunk's dense
// pass from 19.37-19.56 to 19.30-19.34 ms.
constexpr int kDenseMaxChunk = 4096;
constexpr int kDenseMinChunk = 256;
constexpr int64_t kDenseTargetWGs = 2048;
constexpr int kDenseWaves = 4;
constexpr int kDenseRowsPerWave = 2;

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
// a pointer the whole wave holds, as a scalar
__device__ __forceinline__ float* uniform_ptr(float* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<float*>(((uint64_t)hi << 32) | lo);
}

// What a launch writes: the scores, the block keys, or both (a keys-only pass
// never materialises the score matrix).
constexpr int kOutScores = 1;
constexpr int kOutKeys = 2;

// Where the fused block keys go (keys == nullptr: not requested).
struct KeyArgs {
  float* keys;
  int64_t ldk;
  int skip;
};

// max over the aligned group of 8 lanes, in every lane of the group: three
// DPP maxes (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror); the s_nop
// covers the VALU-write -> DPP-read hazard.  Written out because the compiler
// would canonicalize both operands of every fmaxf.
__device__ __forceinline__ float max8_lanes(float v) {
  float a, b, c;
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "=v"(a) : "v"(v));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "=v"(b) : "v"(a));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "=v"(c) : "v"(b));
  return c;
}

// K operands of one pool page: the values of its 4 MFMA tiles of 16
// positions, and its 256 scale bytes in one register (lane l: the 4 scale
// bytes of position l), fetched with one 4-byte load per lane instead of one
// 64-lane byte load per tile.
struct PageOps {
  uint4 b[4];
  uint32_t s;
};

__device__ __forceinline__ void load_page(__amdgpu_buffer_rsrc_t pg, uint32_t voff, uint32_t soff, PageOps& o) {
#pragma unroll
  for (int t = 0; t < 4; ++t) o.b[t] = buffer_load_b128(pg, voff + t * 16 * kValBytes);
  o.s = __builtin_amdgcn_raw_buffer_load_b32(pg, soff, 0, 0);
}

// tile t's scale for this lane: byte l / 16 of position 16 t + l % 16's scales
// (the MFMA reads the low byte)
__device__ __forceinline__ int page_tile_scale(const PageOps& o, int t, int sdist, uint32_t sshift) {
  return (int)((uint32_t)__builtin_amdgcn_ds_bpermute(sdist + 64 * t, (int)o.s) >> sshift);
}

// Score NR (1 or 2) rows of one request against positions [c0, cend) (c0 on
// a page boundary, at most 64 pages: their ids sit one per lane).  Every tile of a page is computed;
// positions past a row's length are never stored.  With keys, Krow[r] gets
// the keys of blocks [c0/8, min(cend/8, nblk[r])) (Krow[r] is only used when
// nblk[r] > 0, i.e. the row is keyed).
template <int HB, int NR, int OUTS>
__device__ __forceinline__ void score_rows(const RowFrag<HB> (&f)[2], const PairFold& pf,
                                           float* const (&Srow)[2],
                                           const int (&lens)[2], float* const (&Krow)[2],
                                           const int (&nblk)[2], const uint8_t* pool,
                                           int num_pages, const int32_t* pt, int max_pages,
                                           int c0, int cend, int lane) {
  const uint32_t voff = (uint32_t)((lane & 15) * kValBytes + (lane >> 4) * 16);
  const uint32_t soff = (uint32_t)(kPageValBytes + lane * kScaleBytes);   // position l's scales
  const int sdist = 4 * (lane & 15);
  const uint32_t sshift = 8u * (uint32_t)(lane >> 4);
  const int npg = (cend - c0 + kPage - 1) / kPage;
  const int pid = (int)clamp_page(pt[min(c0 / kPage + min(lane, npg - 1), max_pages - 1)], num_pages);
  auto load = [&](int i, PageOps& o) {
    const int64_t pg = __builtin_amdgcn_readlane(pid, min(i, npg - 1));
    load_page(buffer_rsrc(pool + pg * kPageBytes, kPageBytes), voff, soff, o);
  };
  // the rows' output pointers and bounds, as scalars (the compiler would
  // otherwise keep some in vector registers and build the store resources
  // lane by lane)
  float* const Su[2] = {uniform_ptr(Srow[0]), uniform_ptr(Srow[NR - 1])};
  float* const Ku[2] = {uniform_ptr(Krow[0]), uniform_ptr(Krow[NR - 1])};
  const int lu[2] = {uniform(lens[0]), uniform(lens[NR - 1])};
  const int nbu[2] = {uniform(nblk[0]), uniform(nblk[NR - 1])};
  // per-lane store offsets: score of position l of a page; key of block l / 8
  // from lanes 8j (the others get an offset past every resource: dropped)
  const uint32_t soffs = (uint32_t)lane * 4u;
  const uint32_t koffs = (lane & 7) == 0 ? (uint32_t)(lane >> 3) * 4u : 0x80000000u;
  auto compute = [&](int i, const PageOps& cur) {
    float part[NR][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int sb = page_tile_scale(cur, t, sdist, sshift);
      const v4f zero = {0.f, 0.f, 0.f, 0.f};
      float seed0, seed1;   // the second row's fold values
      {
        v4f acc[HB + 1];
        acc[0] = mfma_fp4_16x16x128(pf.at, cur.b[t], pf.st, sb, zero);   // both rows' folds
        tile_mfma_blocks<HB>(f[0], cur.b[t], sb, acc);
        part[0][t] = tile_epilogue_pair<HB, true>(f[0], acc, seed0, seed1);
      }
      if (NR == 2) {
        v4f acc[HB + 1];
        acc[0] = zero;
        tile_mfma_blocks<HB>(f[1], cur.b[t], sb, acc);
        part[NR - 1][t] = tile_epilogue_pair<HB, false>(f[1], acc, seed0, seed1);
      }
    }
    // the page's store resources start at its first position (block) and end
    // at the row's length (keys), so the per-lane offsets stay fixed; these
    // are scalar operations
    const int pb0 = uniform(c0 + i * kPage);
    const int kb0 = pb0 / kBlock;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float tot = reduce_scatter4(part[r][0], part[r][1], part[r][2], part[r][3]);
      const uint32_t rem = lu[r] > pb0 ? (uint32_t)(lu[r] - pb0) * 4u : 0u;
      if (OUTS & kOutScores)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), buffer_rsrc(Su[r] + pb0, rem), soffs, 0, 0);
      if (OUTS & kOutKeys) {
        // (the newest block's key is overwritten with +inf after the loop)
        const float key = max8_lanes(tot);
        const uint32_t krem = nbu[r] > kb0 ? (uint32_t)(nbu[r] - kb0) * 4u : 0u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(key), buffer_rsrc(Ku[r] + kb0, krem), koffs, 0, 0);
      }
    }
  };
  PageOps A, B;
  load(0, A);
  // Page 0 is peeled so that the loop is entered, from before it and from its
  // own end, with the same memory operations in flight (the next page's
  // loads, the last page's stores, the page after's loads): each wait then
  // covers only the page about to be computed.  With the first page inside
  // the loop, the wait at its top also waited for the stores of the page
  // just computed (long chunk: dense pass 18.66 -> 18.47 ms, mixed chunk
  // 10.87 -> 10.75 ms, bit-identical).  Every load is unconditional (load()
  // clamps past the last page); the scheduling barriers keep each page's
  // scale permutes out of the other page's arithmetic.
  __builtin_amdgcn_sched_barrier(0);
  load(1, B);
  __builtin_amdgcn_sched_barrier(0);
  compute(0, A);
  __builtin_amdgcn_sched_barrier(0);
  load(2, A);
  int i = 1;
  for (; i + 1 < npg; i += 2) {
    __builtin_amdgcn_sched_barrier(0);
    compute(i, B);
    __builtin_amdgcn_sched_barrier(0);
    load(i + 2, B);
    __builtin_amdgcn_sched_barrier(0);
    compute(i + 1, A);
    __builtin_amdgcn_sched_barrier(0);
    load(i + 3, A);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (i < npg) compute(i, B);
  if (OUTS & kOutKeys) {
    // A keyed row's newest block has key +inf: when it lies in these pages,
    // the lane that stored its computed key (lane 8 (b % 8) of its page)
    // stores +inf over it, after it in program order.  (Selecting +inf in
    // every page cost two VALU instructions per row and page: long chunk,
    // dense pass 18.74 -> 18.48 ms, bit-identical.)
    const int kc0 = c0 / kBlock;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int b = nbu[r] - 1;
      if (b >= kc0 && b < kc0 + npg * kBlocksPerPage) {   // (uniform)
        const uint32_t o = lane == 8 * (b & 7) ? 0u : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(__builtin_inff()), buffer_rsrc(Ku[r] + b, 4u), o, 0, 0);
      }
    }
  }
}

template <int HB, int OUTS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void score_dense_kernel(QueryArgs q, const uint8_t* __restrict__ fold,
                                                          PoolArgs kp,
                                                          const int32_t* __restrict__ req,
                                                          const int32_t* __restrict__ len,
                                                          float* __restrict__ S, int64_t ld,
                                                          KeyArgs ka, int nchunks, int chunk_len) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  // Workgroup i runs on XCD i % 8.  Chunk c of row group g is workgroup
  // g * nchunks + (c - (g / 64) % 8) mod nchunks: within 64 row groups each XCD
  // keeps one eighth of the chunks (its share of the K pool stays in its L2),
  // and the eighth rotates every 64 row groups, so that a batch whose short
  // rows only fill the first chunks (the rest exit at once) spreads them over
  // all XCDs instead of the first few.  A mixed prefill + decode batch (9978
  // rows, contexts 8K-262K): dense pass 5.45 -> 4.62 ms, the long chunk's
  // time unchanged.  Rotating every 16 / 32 row groups gave 4.22 / 4.46 ms
  // but, as the in-flight workgroups then span more rotations, 3.4 / 2.3 GB
  // fetched by the long chunk's dense pass against 1.2 GB unrotated and
  // 1.76 GB this way.
  const int rg = blockIdx.x / nchunks;
  const int chunk = (int)((blockIdx.x % nchunks + (rg / 64) % 8) % nchunks);
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
  // keyed rows: nblk > skip, capped like idx_amax8_varlen (ldk and ld / 8);
  // nblk = 0 marks a row without keys
  int nblk[2] = {0, 0};
  float* Krow[2] = {nullptr, nullptr};
  if (OUTS & kOutKeys) {
    const int64_t kcap = min(ka.ldk, ld / kBlock);
    const int nb0 = (int)min((int64_t)((len0 + kBlock - 1) / kBlock), kcap);
    const int nb1 = (int)min((int64_t)((len1 + kBlock - 1) / kBlock), kcap);
    nblk[0] = nb0 > ka.skip ? nb0 : 0;
    nblk[1] = nb1 > ka.skip ? nb1 : 0;
    Krow[0] = ka.keys + (int64_t)r0 * ka.ldk;
    Krow[1] = r1 >= 0 ? ka.keys + (int64_t)r1 * ka.ldk : Krow[0];
  }
  const int c0 = chunk * chunk_len;
  RowFrag<HB> f[2];
  PairFold pf;
  float* Srow[2];
  int lens[2];
  if (r1 >= 0 && req1 == req0) {  // both rows read the same keys
    const int cend = min(c0 + chunk_len, max(len0, len1));
    if (c0 >= cend) return;
    load_row<HB, false>(q, fold, r0, lane, f[0]);
    load_row<HB, false>(q, fold, r1, lane, f[1]);
    load_pair_fold(fold, r0, r1, lane, pf);
    Srow[0] = S + (int64_t)r0 * ld;
    Srow[1] = S + (int64_t)r1 * ld;
    lens[0] = len0;
    lens[1] = len1;
    score_rows<HB, 2, OUTS>(f, pf, Srow, lens, Krow, nblk, kp.pool, kp.num_pages,
                            kp.page_table + (int64_t)req0 * kp.max_pages, kp.max_pages, c0, cend, lane);
    return;
  }
  for (int i = 0; i < 2; ++i) {  // rows of different requests, one at a time
    const int r = i == 0 ? r0 : r1;
    if (r < 0) break;
    const int L = i == 0 ? len0 : len1;
    const int rq = i == 0 ? req0 : req1;
    const int cend = min(c0 + chunk_len, L);
    if (c0 >= cend) continue;
    load_row<HB, false>(q, fold, r, lane, f[0]);
    load_pair_fold(fold, r, -1, lane, pf);   // the row in the first half, as in a pair
    Srow[0] = S + (int64_t)r * ld;
    Srow[1] = Srow[0];
    lens[0] = L;
    lens[1] = 0;
    // selects, not Krow[i]: an array indexed at run time is kept in scratch
    float* const Ki = i == 0 ? Krow[0] : Krow[1];
    float* const Kr[2] = {Ki, Ki};
    const int nb[2] = {i == 0 ? nblk[0] : nblk[1], 0};
    score_rows<HB, 1, OUTS>(f, pf, Srow, lens, Kr, nb, kp.pool, kp.num_pages,
                            kp.page_table + (int64_t)rq * kp.max_pages, kp.max_pages, c0, cend, lane);
  }
}

template <int OUTS>
static void launch_dense_hb(int hb, dim3 grid, hipStream_t st, const QueryArgs& q, const uint8_t* fold,
                            const PoolArgs& kp, const int32_t* req, const int32_t* len, float* S,
                            int64_t ld, const KeyArgs& ka, int nchunks, int chunk_len) {
  switch (hb) {
    case 1: hipLaunchKernelGGL((score_dense_kernel<1, OUTS>), grid, dim3(256), 0, st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len); break;
    case 2: hipLaunchKernelGGL((score_dense_kernel<2, OUTS>), grid, dim3(256), 0, st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len); break;
    case 3: hipLaunchKernelGGL((score_dense_kernel<3, OUTS>), grid, dim3(256), 0, st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len); break;
    default: hipLaunchKernelGGL((score_dense_kernel<4, OUTS>), grid, dim3(256), 0, st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len); break;
  }
}

hipError_t launch_score_dense(const QueryArgs& q, const uint8_t* fold, const PoolArgs& kp,
                              const int32_t* req, const int32_t* len, float* S, int64_t ld,
                              float* keys, int64_t ldk, int skip, hipStream_t st) {
  const int rows_per_wg = kDenseWaves * kDenseRowsPerWave;
  const int64_t groups = (q.rows + rows_per_wg - 1) / rows_per_wg;
  int chunk_len = kDenseMaxChunk;
  while (chunk_len > kDenseMinChunk && groups * ((ld + chunk_len - 1) / chunk_len) < kDenseTargetWGs)
    chunk_len /= 2;
  const int nchunks = (int)((ld + chunk_len - 1) / chunk_len);
  const int64_t grid = groups * nchunks;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int hb = (q.heads + 15) / 16;
  const KeyArgs ka{keys, ldk, skip};
  if (keys && S)
    launch_dense_hb<kOutScores | kOutKeys>(hb, dim3((unsigned)grid), st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len);
  else if (keys)
    launch_dense_hb<kOutKeys>(hb, dim3((unsigned)grid), st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len);
  else
    launch_dense_hb<kOutScores>(hb, dim3((unsigned)grid), st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len);
  return hipGetLastError();
}

}  // namespace idxk
