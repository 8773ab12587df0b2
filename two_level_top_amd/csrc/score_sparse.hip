// idx_score_sparse_paged: a consumer layer's scores at its candidate positions
// only, read straight from the paged MXFP4 index-K pool (the sglang PR
// "[DSv4.1] Score prefill consumer index layers on candidate blocks with
// DeepGEMM", Design, "Level two": scores [tokens, kb * 8] in ascending block
// order; no dense row is formed).
//
// The work list (built by idx_expand_candidates) holds one unit per 64
// candidate blocks of a row.  A wave takes a run of 4 consecutive units of
// one row (runs ordered so that the waves running at one time hold the same
// run of every row, see the kernel), keeps the row's query in registers across
// them, loads each unit's 64 pool-block ids once (one per lane) and walks
// 2 candidate blocks (16 positions) per MFMA tile, 4 tiles per group, two
// groups in flight (ping-pong registers): lane l gathers 16 bytes of position
// (l % 8) of block (l % 16) / 8 -- each block is 512 contiguous value bytes
// and 32 contiguous scale bytes of one pool page.  Loads go through one
// buffer resource over the pool and scores are stored through a resource
// sized to the unit's valid columns, so the loop has no branches.
#include "score_common.h"

namespace idxk {

constexpr int kSparseWaves = 4;
// Work per wave, chosen at launch from the number of units so that about
// kSparseTargetWaves waves run: up to 4 consecutive units per wave on big
// tables (one unit per wave was 8% slower: the query reload and the wave
// launch per 512 columns; runs of 4, 8 and 16 units measured alike on the
// consumer tables, 4 best on the 513-block source table and on prefill), or a
// unit split over 2, 4 or 8 waves (8 / split groups each) when there are
// fewer units than that.  On 64 decode rows (2048 units) one unit per wave
// ran in 16 us against 26 us split over 4 waves: each wave's query and
// block-id loads are fixed latency.
constexpr int kSparseTargetWaves = 2048;
constexpr int kMaxUnitsPerWave = 4;
// scores are stored non-temporally (cache policy nt): a consumer's 1 GB of
// scores is read once, by its top-k, after the whole table is scored
// (measured 2.13 -> 2.10 ms per call on the long chunk)
constexpr int kStoreNT = 2;

// K operands of 4 tiles (8 candidate blocks) of one unit: each tile's values,
// and the scales of all 8 blocks in one register -- lane l holds the 4 scale
// bytes (one per 32-element group) of position l % 8 of block l / 8.  One
// 4-byte load per lane fetches the group's 256 scale bytes; loading them per
// tile took four 64-lane byte loads, which cost about as much as the value
// loads themselves (long chunk: 2.07 ms per call with them, 1.66 ms without).
struct GroupOps {
  uint4 b[4];
  uint32_t s;
};

// Lane l of tile t of group g needs position (l % 8) of candidate block
// 8 g + 2 t + (l / 8) % 2: 16 bytes at (l / 16) * 16 of its values, and byte
// l / 16 of its scales.  The unit's block byte offsets sit one per lane in
// `bov` (values) and `sov` (scales); ds_bpermute hands each lane its block's
// offset (the tile's block index is the instruction's immediate offset), so
// addressing costs one add per operand.  Blocks past the unit's end repeat
// its last block (the lanes past it hold the last block's offsets) and are
// never stored.
__device__ __forceinline__ void load_group(__amdgpu_buffer_rsrc_t pool, int bov, int sov, int sel,
                                           int ssel, uint32_t voff, uint32_t soff, GroupOps& o) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int a = sel + 8 * t;   // byte address of the source lane (block 8g + 2t + half)
    const uint32_t vb = (uint32_t)__builtin_amdgcn_ds_bpermute(a, bov);
    o.b[t] = buffer_load_b128(pool, vb + voff);
  }
  const uint32_t sb = (uint32_t)__builtin_amdgcn_ds_bpermute(ssel, sov);   // block 8g + l / 8
  o.s = __builtin_amdgcn_raw_buffer_load_b32(pool, sb + soff, 0, 0);
}

// tile t's scale for this lane: the dword of lane 16 t + l % 16 (position l % 8
// of block 2 t + (l / 8) % 2 of the group), byte l / 16 (the MFMA reads the low
// byte)
__device__ __forceinline__ int tile_scale(const GroupOps& o, int t, int sdist, uint32_t sshift) {
  return (int)((uint32_t)__builtin_amdgcn_ds_bpermute(sdist + 64 * t, (int)o.s) >> sshift);
}

// nearest bf16 of a finite fp32 value (ties to even), as its 16 bits
__device__ __forceinline__ uint16_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// BF16: scores are written as bf16 (the prefill PR's consumer output dtype)
template <int HB, bool BF16>
__global__ __launch_bounds__(256) void score_sparse_kernel(QueryArgs q,
                                                           const uint8_t* __restrict__ fold,
                                                           const uint8_t* __restrict__ pool,
                                                           int num_pages,
                                                           const int32_t* __restrict__ phys,
                                                           const int32_t* __restrict__ n_kept,
                                                           const int32_t* __restrict__ valid_len,
                                                           int kb, const int32_t* __restrict__ sched,
                                                           void* __restrict__ T, int64_t ld,
                                                           int upw, int split) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int max_units = q.rows * ((kb + kUnitBlocks - 1) / kUnitBlocks);
  const int nunits = min(sched[0], max_units);
  const __amdgpu_buffer_rsrc_t prs = buffer_rsrc(pool, (uint32_t)num_pages * (uint32_t)kPageBytes);
  const uint32_t voff = (uint32_t)((lane & 7) * kValBytes + (lane >> 4) * 16);
  const uint32_t soff = (uint32_t)((lane & 7) * kScaleBytes);    // this lane's scale dword
  const int sdist = 4 * (lane & 15);                             // source lane of tile 0's scale
  const uint32_t sshift = 8u * (uint32_t)(lane >> 4);            // its byte
  const int half = (lane >> 3) & 1;
  // each wave takes `upw` consecutive units (mostly of one row: the list is
  // row-major) and keeps the row's query in registers across them, or part
  // `part` of one unit when split > 1
  const int wid = blockIdx.x * kSparseWaves + wave;
  int u0 = split > 1 ? wid / split : wid * upw;
  int u1 = min(split > 1 ? u0 + 1 : u0 + upw, nunits);
  if (split == 1 && upw > 1) {
    // When a row's U units split evenly into runs of upw, wave wid takes run
    // b = wid / rows of row wid % rows.  A row's candidates ascend through its
    // context, so run b of every row covers about the same stretch of it;
    // the waves running at one time then gather from the same pool pages
    // (the rows of one request share them), which each XCD's L2 keeps:
    // consumer scores 2.08 -> 2.00 ms on the long chunk, bit-identical.  The
    // last workgroup's spare waves (b past the runs) take no unit.
    const int U = (kb + kUnitBlocks - 1) / kUnitBlocks;
    if (U % upw == 0) {
      const int r = wid % q.rows, b = wid / q.rows;
      u0 = b < U / upw ? r * U + b * upw : nunits;
      u1 = min(u0 + upw, nunits);
    }
  }
  const int part = split > 1 ? wid % split : 0;
  const int gper = 8 / split;                      // groups per part
  int cur_row = -1;
  RowFrag<HB> f;
  PairFold pf;   // the row's fold, first 8 terms (the layout the dense kernel uses)
  for (int u = u0; u < u1; ++u) {
    const int row = __builtin_amdgcn_readfirstlane(sched[4 + 2 * u]);
    const int first = __builtin_amdgcn_readfirstlane(sched[5 + 2 * u]);
    if (row < 0 || row >= q.rows || first < 0) continue;   // not a work list this table built
    const int nk = __builtin_amdgcn_readfirstlane(min(max(n_kept[row], 0), kb));
    const int vl = __builtin_amdgcn_readfirstlane(min(valid_len[row], nk * kBlock));
    const int nblk = min(kUnitBlocks, nk - first);   // candidate blocks of this unit
    if (nblk <= 0) continue;
    if (row != cur_row) {
      load_row<HB, false>(q, fold, row, lane, f);
      load_pair_fold(fold, row, -1, lane, pf);
      cur_row = row;
    }
    // byte offsets of this lane's candidate block (pools are < 4 GiB here)
    const int pb = phys[(int64_t)row * kb + first + min(lane, nblk - 1)];
    const uint32_t pgo = (uint32_t)clamp_page(pb >> 3, num_pages) * (uint32_t)kPageBytes;
    const int bov = (int)(pgo + (uint32_t)(pb & 7) * (kBlock * kValBytes));
    const int sov = (int)(pgo + kPageValBytes + (uint32_t)(pb & 7) * (kBlock * kScaleBytes));
    // valid columns of this unit: stores past them are dropped by the resource
    const int ncols = max(0, min(vl - first * kBlock, nblk * kBlock));
    constexpr uint32_t kEl = BF16 ? 2u : 4u;   // bytes per score
    const __amdgpu_buffer_rsrc_t trs = buffer_rsrc(static_cast<char*>(T) + ((int64_t)row * ld + first * kBlock) * kEl,
                                                   (uint32_t)ncols * kEl);
    const int ngroups = (nblk + 7) / 8;
    auto sel_of = [&](int g) { return 4 * min(8 * g + half, nblk - 1); };
    auto ssel_of = [&](int g) { return 4 * (8 * g + (lane >> 3)); };
    auto compute = [&](int g, const GroupOps& cur) {
      float p[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int sb = tile_scale(cur, t, sdist, sshift);
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
        v4f acc[HB + 1];
        acc[0] = mfma_fp4_16x16x128(pf.at, cur.b[t], pf.st, sb, zero);
        tile_mfma_blocks<HB>(f, cur.b[t], sb, acc);
        float unused0, unused1;
        p[t] = tile_epilogue_pair<HB, true>(f, acc, unused0, unused1);
      }
      const float tot = reduce_scatter4(p[0], p[1], p[2], p[3]);
      if (BF16)
        __builtin_amdgcn_raw_buffer_store_b16(bf16_bits(tot), trs, (uint32_t)(g * 64 + lane) * kEl, 0, kStoreNT);
      else
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), trs, (uint32_t)(g * 64 + lane) * kEl, 0, kStoreNT);
    };
    const int g0 = part * gper;
    const int g1 = min(ngroups, g0 + gper);
    if (g0 >= g1) continue;
    // Two groups in flight: each group's loads are issued before the previous
    // group is computed.  Every load in the loop is unconditional (the last
    // B load repeats group g1 - 1 when the count is odd): a load whose value
    // is used only past a branch is moved there by the compiler, and an
    // optional load makes the wait at the join cover it, both of which left
    // half the groups' gathers exposed (long chunk: 1.98-2.02 -> 1.88-1.90 ms
    // per consumer call, bit-identical).  The scheduling barriers keep the
    // scheduler from pulling the next group's scale permutes into the
    // current group's arithmetic, which would wait on that group's loads.
    GroupOps A, B;
    load_group(prs, bov, sov, sel_of(g0), ssel_of(g0), voff, soff, A);
    __builtin_amdgcn_sched_barrier(0);
    const int gb0 = min(g0 + 1, g1 - 1);
    load_group(prs, bov, sov, sel_of(gb0), ssel_of(gb0), voff, soff, B);
    int g = g0;
    for (; g + 2 < g1; g += 2) {
      __builtin_amdgcn_sched_barrier(0);
      compute(g, A);
      __builtin_amdgcn_sched_barrier(0);
      load_group(prs, bov, sov, sel_of(g + 2), ssel_of(g + 2), voff, soff, A);
      __builtin_amdgcn_sched_barrier(0);
      compute(g + 1, B);
      __builtin_amdgcn_sched_barrier(0);
      const int gb = min(g + 3, g1 - 1);
      load_group(prs, bov, sov, sel_of(gb), ssel_of(gb), voff, soff, B);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(g, A);
    if (g + 1 < g1) compute(g + 1, B);
  }
}

hipError_t launch_score_sparse(const QueryArgs& q, const uint8_t* fold, const uint8_t* pool,
                               int num_pages,
                               const int32_t* phys, const int32_t* n_kept,
                               const int32_t* valid_len, int rows, int kb, const void* schedule,
                               void* T, int64_t ld, bool bf16, hipStream_t st) {
  const int64_t max_units = (int64_t)rows * ((kb + kUnitBlocks - 1) / kUnitBlocks);
  if (max_units <= 0) return hipSuccess;
  int upw = 1, split = 1;
  if (max_units >= (int64_t)kSparseTargetWaves * kMaxUnitsPerWave) {
    upw = kMaxUnitsPerWave;
    // short rows whose units do not split into runs of 4 (the source's
    // 513-block table: 9 units) go whole, one row per wave, when that still
    // gives kSparseTargetWaves waves: the source's rescoring and select on
    // the side stream 1.33 -> 1.08 ms on the long chunk
    const int U = (kb + kUnitBlocks - 1) / kUnitBlocks;
    if (U % upw != 0 && U <= 3 * kMaxUnitsPerWave && max_units >= (int64_t)kSparseTargetWaves * U)
      upw = U;
  }
  else if (max_units >= kSparseTargetWaves)
    upw = (int)(max_units / kSparseTargetWaves);
  else
    while (split < 8 && max_units * split < kSparseTargetWaves) split *= 2;
  const int64_t waves = split > 1 ? max_units * split : (max_units + upw - 1) / upw;
  int64_t grid = (waves + kSparseWaves - 1) / kSparseWaves;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int32_t* sched = static_cast<const int32_t*>(schedule);
  const int hb = (q.heads + 15) / 16;
#define IDX_SPARSE_LAUNCH(H, B)                                                                        \
  hipLaunchKernelGGL((score_sparse_kernel<H, B>), dim3((unsigned)grid), dim3(256), 0, st, q, fold, pool, \
                     num_pages, phys, n_kept, valid_len, kb, sched, T, ld, upw, split)
  if (bf16) {
    switch (hb) {
      case 1: IDX_SPARSE_LAUNCH(1, true); break;
      case 2: IDX_SPARSE_LAUNCH(2, true); break;
      case 3: IDX_SPARSE_LAUNCH(3, true); break;
      default: IDX_SPARSE_LAUNCH(4, true); break;
    }
  } else {
    switch (hb) {
      case 1: IDX_SPARSE_LAUNCH(1, false); break;
      case 2: IDX_SPARSE_LAUNCH(2, false); break;
      case 3: IDX_SPARSE_LAUNCH(3, false); break;
      default: IDX_SPARSE_LAUNCH(4, false); break;
    }
  }
#undef IDX_SPARSE_LAUNCH
  return hipGetLastError();
}

}  // namespace idxk
