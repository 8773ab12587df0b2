// idx_score_dense: the source layer's fp32 score matrix over every reachable
// position of each row (the dense score matrix of the sglang PR "[DSv4.1]
// Score prefill consumer index layers on candidate blocks with DeepGEMM",
// Motivation; the vLLM sparse_attn_indexer page's fp8_fp4_mqa_logits over
// each row's [ks, ke)).
//
// Work decomposition (gfx950: 256 CUs in 8 XCDs, wave64):
//   workgroup = 8 waves, one query row each (8 consecutive rows), 1024
//   positions (512 or 256 when there are too few rows to fill the chip
//   otherwise, as in decode).  workgroup id -> (row group = id / nchunks,
//   chunk = id % nchunks), so consecutive ids -- which the dispatcher spreads
//   over the 8 XCDs -- share a row group and walk different position chunks:
//   each XCD keeps 1/8 of the K pool hot in its L2 and re-reads a row
//   group's query from L2.  A wave keeps its row's query (64 heads x 128 dims
//   as MXFP4) in registers.
// K tiles staged in LDS: when the workgroup's rows belong to one request
// (prefill) they read the same pool pages, so each page (64 positions,
// 4352 bytes) is loaded once per workgroup into a ring of 3 LDS slots -- four
// waves load a quarter of its codes each, a fifth its scales -- and every
// wave reads its MFMA operands from there: one 16-byte read per tile and lane
// (16-byte units swizzled so that no two lanes of a read share a bank) and
// one byte for the scale.  Page i + 2 is fetched into registers while page i
// is scored and written to its slot one page later; one barrier per page.
// Compared with each wave streaming its own pages through registers, this
// reads K from L2 once per 8 rows instead of once per 2, and the registers
// it frees (about 30 per wave) let 8 waves run per SIMD instead of 4: the
// MFMA -> epilogue dependency of one wave is hidden by the others.
// Workgroups whose rows span several requests (decode, mixed batches) score
// each row from its own pages, loaded one page at a time into registers.
// Scores and keys are stored through buffer resources sized to the row's
// valid range, so out-of-range lanes are dropped by the hardware.
//
// Fused block keys (the prefill PR's follow-up of folding the block amax into
// the score kernel): after the 4-way reduction each lane holds one score of
// 64 consecutive positions, so an aligned 8-lane DPP max gives the key of
// every block of the page without reading S back.  The keys equal what
// idx_amax8_varlen computes from the stored S (the max of the same fp32
// values; the newest block is +inf; rows with nblk <= skip are untouched).
#include "score_common.h"

#ifndef DENSE_WPE
#define DENSE_WPE 4
#endif

namespace idxk {

// positions per workgroup: 1024, or 512 / 256 when there are few rows (decode)
// so that at least kDenseTargetWGs workgroups run
constexpr int kDenseMaxChunk = 1024;
constexpr int kDenseMinChunk = 256;
constexpr int64_t kDenseTargetWGs = 2048;
constexpr int kDenseWaves = 4;
constexpr int kDenseRowsPerWave = 2;
constexpr int kDenseRows = kDenseWaves * kDenseRowsPerWave;   // rows per workgroup
constexpr int kRingSlots = 3;           // LDS page slots (pages i, i + 1 in use, i + 2 arriving)

struct DenseShared {
  uint8_t ring[kRingSlots][kPageBytes];
  int req[kDenseRows];
  int len[kDenseRows];
};

// 16-byte unit of (position p, k-group g) inside an LDS page slot: g is
// swizzled by (p ^ p / 4) % 4, which puts the 16 (or 8) lanes of one read pass
// on distinct banks for 64- and 32-bank LDS alike
__device__ __forceinline__ int lds_unit(int p, int g) { return p * 4 + (g ^ ((p ^ (p >> 2)) & 3)); }

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

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

// The per-row path reads a page's 256 scale bytes into one register (lane l:
// the 4 scale bytes of position l) with one 4-byte load per lane, instead of
// one 64-lane byte load per tile.  Tile t's scale for this lane is byte l / 16
// of position 16 t + l % 16's scales (the MFMA reads the low byte).
__device__ __forceinline__ int page_tile_scale(uint32_t pscale, int t, int sdist, uint32_t sshift) {
  return (int)((uint32_t)__builtin_amdgcn_ds_bpermute(sdist + 64 * t, (int)pscale) >> sshift);
}

// Where one row's scores and keys go.
struct RowOut {
  __amdgpu_buffer_rsrc_t rs;   // S row, sized to len
  __amdgpu_buffer_rsrc_t rk;   // key row, sized to nblk (KEYS)
  int nblk;
};

// Lane l stores the score of position p0 + l of one row (and, with KEYS, the
// key of its block of 8 from lanes 8j).
template <bool KEYS>
__device__ __forceinline__ void store_page(float tot, const RowOut& o, int p0, int lane) {
  const int p = p0 + lane;
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), o.rs, (uint32_t)p * 4u, 0, 0);
  if (KEYS) {
    const float m = max8_lanes(tot);
    const int blk = p >> 3;
    const float key = blk == o.nblk - 1 ? __builtin_inff() : m;
    const uint32_t koff = (lane & 7) == 0 ? (uint32_t)blk * 4u : 0x80000000u;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(key), o.rk, koff, 0, 0);
  }
}

// Scores of one page (4 tiles) of NR rows sharing the tiles' operands and a
// fold block: the B operand and scale of tile t come from get(t, b, sb).
template <int HB, int NR, bool KEYS, class Get>
__device__ __forceinline__ void score_page(const RowFrag<HB> (&f)[2], const PairFold& pf,
                                           const RowOut (&o)[2], int p0, int lane, Get get) {
  float part[NR][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    uint4 b;
    int sb;
    get(t, b, sb);
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    float seed0, seed1;   // the second row's fold values
    {
      v4f acc[HB + 1];
      acc[0] = mfma_fp4_16x16x128(pf.at, b, pf.st, sb, zero);   // the rows' folds
      tile_mfma_blocks<HB>(f[0], b, sb, acc);
      part[0][t] = tile_epilogue_pair<HB, true>(f[0], acc, seed0, seed1);
    }
    if (NR == 2) {
      v4f acc[HB + 1];
      acc[0] = zero;
      tile_mfma_blocks<HB>(f[1], b, sb, acc);
      part[NR - 1][t] = tile_epilogue_pair<HB, false>(f[1], acc, seed0, seed1);
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r)
    store_page<KEYS>(reduce_scatter4(part[r][0], part[r][1], part[r][2], part[r][3]), o[r], p0, lane);
}

template <int HB, bool KEYS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DENSE_WPE))) void score_dense_kernel(
    QueryArgs q, const uint8_t* __restrict__ fold, PoolArgs kp, const int32_t* __restrict__ req,
    const int32_t* __restrict__ len, float* __restrict__ S, int64_t ld, KeyArgs ka, int nchunks,
    int chunk_len) {
  __shared__ DenseShared sh;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int chunk = blockIdx.x % nchunks;
  const int rg = blockIdx.x / nchunks;
  const int c0 = chunk * chunk_len;
  // lengths are clamped to [0, min(ld, max_pages * 64)] so that a bad length
  // can never address outside S or the page table
  const int64_t lcap64 = min(ld, (int64_t)kp.max_pages * kPage);
  const int lcap = (int)min(lcap64, (int64_t)0x7fffffff);
  int row[2], rq[2], L[2];
  RowOut o[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = rg * kDenseRows + wave * kDenseRowsPerWave + i;
    row[i] = r < q.rows ? r : -1;
    rq[i] = row[i] >= 0 ? uniform(clamp_req(req[r], kp.num_req)) : -1;
    L[i] = row[i] >= 0 ? uniform(min(max(len[r], 0), lcap)) : 0;
    o[i].nblk = 0;
    if (row[i] >= 0) {
      o[i].rs = buffer_rsrc(S + (int64_t)r * ld, (uint32_t)L[i] * 4u);
      if (KEYS) {
        // keyed rows: nblk > skip, capped like idx_amax8_varlen (ldk and
        // ld / 8); nblk = 0 marks a row without keys
        const int64_t kcap = min(ka.ldk, ld / kBlock);
        const int nb = (int)min((int64_t)((L[i] + kBlock - 1) / kBlock), kcap);
        o[i].nblk = nb > ka.skip ? nb : 0;
        o[i].rk = buffer_rsrc(ka.keys + (int64_t)r * ka.ldk, (uint32_t)o[i].nblk * 4u);
      }
    }
    if (lane == 0) {
      sh.req[wave * kDenseRowsPerWave + i] = rq[i];
      sh.len[wave * kDenseRowsPerWave + i] = L[i];
    }
  }
  __syncthreads();
  // one request for every row of the workgroup (rows past the end excepted)?
  const int req0 = sh.req[0];   // the first row always exists
  bool one_req = true;
  int maxlen = 0;
#pragma unroll
  for (int w = 0; w < kDenseRows; ++w) {
    const int qw = sh.req[w];
    one_req = one_req && (qw < 0 || qw == req0);
    maxlen = max(maxlen, sh.len[w]);
  }
  RowFrag<HB> f[2];
  PairFold pf;

  if (one_req) {
    // ---- rows of one request: pages staged once in LDS ----
    const int cend = min(c0 + chunk_len, maxlen);
    if (c0 >= cend) return;   // uniform over the workgroup
    const int npg = (cend - c0 + kPage - 1) / kPage;
    const int wend = min(c0 + chunk_len, max(L[0], L[1]));   // this wave's rows' end
    const bool pair = row[1] >= 0;
    if (c0 < wend) {
      load_row<HB, false>(q, fold, row[0], lane, f[0]);
      if (pair) load_row<HB, false>(q, fold, row[1], lane, f[1]);
      load_pair_fold(fold, row[0], row[1], lane, pf);
    }
    const int32_t* pt = kp.page_table + (int64_t)req0 * kp.max_pages;
    const int pid = (int)clamp_page(pt[min(c0 / kPage + min(lane, npg - 1), kp.max_pages - 1)], kp.num_pages);
    // loaders: wave w fills 16 positions of a page's codes (one 16-byte unit
    // per lane, placed by lds_unit) and, with lanes 0-15, 64 of its 256 scale
    // bytes
    const int u = wave * 64 + lane;          // LDS unit this lane fills
    const int pp = u >> 2, c = u & 3;
    const uint32_t goff = (uint32_t)(pp * kValBytes + ((c ^ ((pp ^ (pp >> 2)) & 3)) * 16));
    const uint32_t loff = (uint32_t)(u * 16);
    const bool sload = lane < 16;
    const uint32_t soff = (uint32_t)(kPageValBytes + (wave * 16 + lane) * kScaleBytes);
    uint4 sv = make_uint4(0u, 0u, 0u, 0u);
    uint32_t ss = 0u;
    auto fetch = [&](int i) {
      const int64_t pg = __builtin_amdgcn_readlane(pid, i);
      const __amdgpu_buffer_rsrc_t prs = buffer_rsrc(kp.pool + pg * kPageBytes, kPageBytes);
      sv = buffer_load_b128(prs, goff);
      if (sload) ss = __builtin_amdgcn_raw_buffer_load_b32(prs, soff, 0, 0);
    };
    auto stash = [&](int i) {
      uint8_t* slot = sh.ring[i % kRingSlots];
      *reinterpret_cast<uint4*>(slot + loff) = sv;
      if (sload) *reinterpret_cast<uint32_t*>(slot + soff) = ss;
    };
    fetch(0);
    stash(0);
    if (npg > 1) fetch(1);
    __syncthreads();
    const int pl = lane & 15, g = lane >> 4;
    for (int i = 0; i < npg; ++i) {
      if (i + 1 < npg) stash(i + 1);   // slot of page i - 2, which every wave is done with
      if (i + 2 < npg) fetch(i + 2);
      const int p0 = c0 + i * kPage;
      if (p0 < wend) {
        const uint8_t* slot = sh.ring[i % kRingSlots];
        auto get = [&](int t, uint4& b, int& sb) {
          const int tp = 16 * t + pl;
          b = *reinterpret_cast<const uint4*>(slot + lds_unit(tp, g) * 16);
          sb = slot[kPageValBytes + tp * kScaleBytes + g];
        };
        if (pair)
          score_page<HB, 2, KEYS>(f, pf, o, p0, lane, get);
        else
          score_page<HB, 1, KEYS>(f, pf, o, p0, lane, get);
      }
      __syncthreads();   // page i + 1 complete; slot of page i free from i + 3 on
    }
    return;
  }

  // ---- rows of several requests: each row from its own pages, in registers ----
  const uint32_t voff = (uint32_t)((lane & 15) * kValBytes + (lane >> 4) * 16);
  const uint32_t soff = (uint32_t)(kPageValBytes + lane * kScaleBytes);   // position l's scales
  const int sdist = 4 * (lane & 15);
  const uint32_t sshift = 8u * (uint32_t)(lane >> 4);
  for (int i = 0; i < 2; ++i) {
    if (row[i] < 0 || c0 >= L[i]) continue;
    load_row<HB, false>(q, fold, row[i], lane, f[0]);
    load_pair_fold(fold, row[i], -1, lane, pf);   // the row in the first half, as in a pair
    const RowOut oi[2] = {o[i], o[i]};
    const int cend = min(c0 + chunk_len, L[i]);
    const int npg = (cend - c0 + kPage - 1) / kPage;
    const int32_t* pt = kp.page_table + (int64_t)rq[i] * kp.max_pages;
    const int pid = (int)clamp_page(pt[min(c0 / kPage + min(lane, npg - 1), kp.max_pages - 1)], kp.num_pages);
    for (int j = 0; j < npg; ++j) {
      const int64_t pg = __builtin_amdgcn_readlane(pid, j);
      const __amdgpu_buffer_rsrc_t prs = buffer_rsrc(kp.pool + pg * kPageBytes, kPageBytes);
      const uint32_t pscale = __builtin_amdgcn_raw_buffer_load_b32(prs, soff, 0, 0);
      score_page<HB, 1, KEYS>(f, pf, oi, c0 + j * kPage, lane, [&](int t, uint4& b, int& sb) {
        b = buffer_load_b128(prs, voff + t * 16 * kValBytes);
        sb = page_tile_scale(pscale, t, sdist, sshift);
      });
    }
  }
}

template <bool KEYS>
static void launch_dense_hb(int hb, dim3 grid, hipStream_t st, const QueryArgs& q, const uint8_t* fold,
                            const PoolArgs& kp, const int32_t* req, const int32_t* len, float* S,
                            int64_t ld, const KeyArgs& ka, int nchunks, int chunk_len) {
  switch (hb) {
    case 1: hipLaunchKernelGGL((score_dense_kernel<1, KEYS>), grid, dim3(64 * kDenseWaves), 0, st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len); break;
    case 2: hipLaunchKernelGGL((score_dense_kernel<2, KEYS>), grid, dim3(64 * kDenseWaves), 0, st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len); break;
    case 3: hipLaunchKernelGGL((score_dense_kernel<3, KEYS>), grid, dim3(64 * kDenseWaves), 0, st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len); break;
    default: hipLaunchKernelGGL((score_dense_kernel<4, KEYS>), grid, dim3(64 * kDenseWaves), 0, st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len); break;
  }
}

hipError_t launch_score_dense(const QueryArgs& q, const uint8_t* fold, const PoolArgs& kp,
                              const int32_t* req, const int32_t* len, float* S, int64_t ld,
                              float* keys, int64_t ldk, int skip, hipStream_t st) {
  const int rows_per_wg = kDenseRows;
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
  if (keys)
    launch_dense_hb<true>(hb, dim3((unsigned)grid), st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len);
  else
    launch_dense_hb<false>(hb, dim3((unsigned)grid), st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len);
  return hipGetLastError();
}

}  // namespace idxk
