// Row-wise exact top-k with a fixed tie rule (lower index wins), written in
// ascending index order.  Serves both
//   idx_topk_blocks  the kb best block keys of each row (sglang PR "[DSv4.1]
//                    Score prefill consumer index layers on candidate blocks
//                    with DeepGEMM", Design, "Level one": ragged top-k over
//                    the keys, trivial path for rows with <= kb blocks,
//                    ascending INT32_MAX-padded block ids), and
//   idx_topk_rows    top-k of a row's first `valid` columns, mapped to
//                    positions, -1 past min(k, valid) (same PR, "Level two",
//                    and the source's own top-512).
//
// One workgroup of 1024 threads per row; thread t owns the 32 consecutive
// elements [32 t, 32 t + 32) of each 32768-element chunk (a whole row of
// keys or of a consumer's scores is one chunk, held in registers).
//   1. radix select on order-preserving u32 keys: three LDS histogram passes
//      (11, 11, 10 bits) find the k-th largest key K and how many elements
//      equal to K are still needed (`need`);
//   2. ordered compaction: element i is kept iff key > K, or key == K and
//      fewer than `need` equal keys precede it.  One block scan of the packed
//      (greater, equal) counts gives every thread its output offset, so the
//      output comes out in ascending index order with no sort.
#include "idx_internal.h"

namespace idxk {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkE = 32;
constexpr int kTopkChunk = kTopkThreads * kTopkE;
constexpr int kHistBins = 2048;

enum { MODE_IDENTITY = 0, MODE_BLOCKMAP = 1, MODE_GATHER = 2, MODE_KEYS = 3 };

struct TopkArgs {
  const float* X;
  int64_t ld;
  const int32_t* nvalid;   // columns per row (modes 0-2)
  const int32_t* len;      // compress_len per row (mode 3: nblk = ceil(len / 8))
  int k;
  const int32_t* blocks;   // [rows][kb] (modes 1, 2)
  int kb;
  const int32_t* pos_offset;
  int32_t* out;            // [rows][k]
  int32_t* n_kept;         // mode 3
};

struct TopkShared {
  uint32_t hist[kHistBins];
  uint32_t wsum[kTopkWaves];
  uint32_t wexcl[kTopkWaves];
  uint32_t total;
  int32_t digit;
  int32_t above;
};

// Exclusive scan over the workgroup; *total receives the sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, TopkShared& sh, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh.wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const uint32_t s = lane < kTopkWaves ? sh.wsum[lane] : 0u;
    uint32_t y = s;
#pragma unroll
    for (int o = 1; o < kTopkWaves; o <<= 1) {
      const uint32_t z = __shfl_up(y, o, 64);
      if (lane >= o) y += z;
    }
    if (lane < kTopkWaves) sh.wexcl[lane] = y - s;
    if (lane == kTopkWaves - 1) sh.total = y;
  }
  __syncthreads();
  const uint32_t r = sh.wexcl[wave] + x - v;
  *total = sh.total;
  __syncthreads();
  return r;
}

template <int MODE>
__device__ __forceinline__ float load_value(const TopkArgs& a, const float* Xr, const int32_t* blk,
                                            int i) {
  if (MODE == MODE_GATHER) {
    int64_t p = (int64_t)blk[i >> 3] * kBlock + (i & 7);
    if (p < 0 || p >= a.ld) p = 0;   // outside the contract: read something in the row
    return Xr[p];
  }
  return Xr[i];
}

template <int MODE>
__device__ __forceinline__ int32_t map_index(const int32_t* blk, int i) {
  if (MODE == MODE_BLOCKMAP || MODE == MODE_GATHER) return blk[i >> 3] * kBlock + (i & 7);
  return i;
}

template <int MODE>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  __shared__ TopkShared sh;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  int n;
  if (MODE == MODE_KEYS) {
    const int L = a.len[row];
    n = L > 0 ? (L + kBlock - 1) / kBlock : 0;
  } else {
    n = a.nvalid[row];
    if (n < 0) n = 0;
    if ((MODE == MODE_BLOCKMAP || MODE == MODE_GATHER) && n > a.kb * kBlock) n = a.kb * kBlock;
  }
  if (MODE != MODE_GATHER && (int64_t)n > a.ld) n = (int)a.ld;   // never read past the row
  const int k = a.k;
  int32_t* out = a.out + (int64_t)row * k;
  const int32_t pad = MODE == MODE_KEYS ? 0x7fffffff : -1;
  const int32_t off = (MODE != MODE_KEYS && a.pos_offset) ? a.pos_offset[row] : 0;
  const int32_t* blk = (MODE == MODE_BLOCKMAP || MODE == MODE_GATHER) ? a.blocks + (int64_t)row * a.kb : nullptr;
  const float* Xr = a.X + (int64_t)row * a.ld;

  if (n <= k) {  // every column is kept
    for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? map_index<MODE>(blk, i) + off : pad;
    if (MODE == MODE_KEYS && tid == 0) a.n_kept[row] = n;
    return;
  }

  uint32_t key[kTopkE];
  const int nchunks = (n + kTopkChunk - 1) / kTopkChunk;
  auto load_chunk = [&](int ch) {
    const int base = ch * kTopkChunk + tid * kTopkE;
#pragma unroll
    for (int e = 0; e < kTopkE; ++e) {
      const int i = base + e;
      key[e] = i < n ? order_key(load_value<MODE>(a, Xr, blk, i)) : 0u;
    }
  };
  if (nchunks == 1) load_chunk(0);

  // ---- 1. radix select of the k-th largest key ----
  uint32_t prefix = 0u, pmask = 0u;
  int remaining = k;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3ffu : 0x7ffu;
    for (int b = tid; b < kHistBins; b += kTopkThreads) sh.hist[b] = 0u;
    __syncthreads();
    for (int ch = 0; ch < nchunks; ++ch) {
      if (nchunks > 1) load_chunk(ch);
      const int base = ch * kTopkChunk + tid * kTopkE;
#pragma unroll
      for (int e = 0; e < kTopkE; ++e) {
        if (base + e < n && (key[e] & pmask) == prefix)
          atomicAdd(&sh.hist[(key[e] >> shift) & dmask], 1u);
      }
    }
    __syncthreads();
    // thread t looks at bins 2047 - 2t (higher) and 2046 - 2t
    const int bh = kHistBins - 1 - 2 * tid, bl = bh - 1;
    const uint32_t ch_ = sh.hist[bh], cl = sh.hist[bl];
    uint32_t tot;
    const uint32_t above = block_exclusive_scan(ch_ + cl, sh, &tot);
    if (above < (uint32_t)remaining && (uint32_t)remaining <= above + ch_ + cl) {
      if (above + ch_ >= (uint32_t)remaining) {
        sh.digit = bh;
        sh.above = (int)above;
      } else {
        sh.digit = bl;
        sh.above = (int)(above + ch_);
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sh.digit << shift;
    pmask |= dmask << shift;
    remaining -= sh.above;
    __syncthreads();
  }
  const uint32_t K = prefix;
  const uint32_t need = (uint32_t)remaining;

  // ---- 2. ordered compaction ----
  uint32_t gt_run = 0u, eq_run = 0u;
  for (int ch = 0; ch < nchunks; ++ch) {
    if (nchunks > 1) load_chunk(ch);
    const int base = ch * kTopkChunk + tid * kTopkE;
    uint32_t gt = 0u, eq = 0u;
#pragma unroll
    for (int e = 0; e < kTopkE; ++e) {
      if (base + e < n) {
        gt += key[e] > K ? 1u : 0u;
        eq += key[e] == K ? 1u : 0u;
      }
    }
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan((gt << 16) | eq, sh, &tot);
    const uint32_t gt_before = gt_run + (ex >> 16);
    uint32_t eq_before = eq_run + (ex & 0xffffu);
    uint32_t o = gt_before + (eq_before < need ? eq_before : need);
#pragma unroll
    for (int e = 0; e < kTopkE; ++e) {
      const int i = base + e;
      if (i < n) {
        bool take = key[e] > K;
        if (key[e] == K) {
          take = eq_before < need;
          ++eq_before;
        }
        if (take) out[o++] = map_index<MODE>(blk, i) + off;
      }
    }
    gt_run += tot >> 16;
    eq_run += tot & 0xffffu;
  }
  if (MODE == MODE_KEYS && tid == 0) a.n_kept[row] = k;
}

hipError_t launch_topk(int mode, const float* X, int64_t ld, const int32_t* nvalid,
                       const int32_t* len_for_blocks, int rows, int k, int64_t /*max_cols*/,
                       const int32_t* blocks, int kb, const int32_t* pos_offset, int32_t* out,
                       int32_t* n_kept, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  TopkArgs a{X, ld, nvalid, len_for_blocks, k, blocks, kb, pos_offset, out, n_kept};
  switch (mode) {
    case MODE_IDENTITY: hipLaunchKernelGGL(topk_kernel<MODE_IDENTITY>, dim3(rows), dim3(kTopkThreads), 0, st, a); break;
    case MODE_BLOCKMAP: hipLaunchKernelGGL(topk_kernel<MODE_BLOCKMAP>, dim3(rows), dim3(kTopkThreads), 0, st, a); break;
    case MODE_GATHER: hipLaunchKernelGGL(topk_kernel<MODE_GATHER>, dim3(rows), dim3(kTopkThreads), 0, st, a); break;
    default: hipLaunchKernelGGL(topk_kernel<MODE_KEYS>, dim3(rows), dim3(kTopkThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace idxk
