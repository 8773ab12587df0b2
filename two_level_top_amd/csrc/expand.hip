// Candidate expansion, the sparse scorer's work list and the tail rows.
//
// idx_expand_candidates (sglang PR "[DSv4.1] Score prefill consumer index
// layers on candidate blocks with DeepGEMM", Design, "Level one": the pool
// slots of the kept blocks and the schedule, built once per chunk and reused
// by every consumer; the vLLM decode page's candidate_blocks_to_sparse_indices
// plays the same part):
//   phys[r][i]   = page_table[req[r]][blocks[r][i] / 8] * 8 + blocks[r][i] % 8
//   valid_len[r] = 8 * n_kept[r] - (8 * nblk - len[r])
// The newest block is always kept and sorts last, so the only partial block
// is the last candidate and the valid columns are exactly [0, valid_len).
//
// Work list layout (int32): [0] entry count = rows * U, [1..3] unused, then
// U = ceil(kb / 64) (row, first block) entries per row, row-major: entry
// (r, u) is (r, 64 u) when the row keeps more than 64 u blocks, else (r, -1),
// an empty unit the scorer skips.  Every entry is written by the thread that
// owns it, so building the list costs one pass and is deterministic.
#include "idx_internal.h"

namespace idxk {

// One workgroup per (row, 256 * VEC candidates): thread t expands candidates
// VEC t .. VEC t + VEC - 1 of its slice (VEC = 4: one 16-byte load of block
// ids and one 16-byte store, when kb % 4 == 0 and both arrays are 16-byte
// aligned).  The row's first workgroup also writes the row's work-list
// entries (and row 0's the entry count), so the list needs no launch of its
// own.
template <int VEC>
__global__ __launch_bounds__(256) void expand_kernel(PoolArgs kp, const int32_t* __restrict__ req,
                                                     const int32_t* __restrict__ len, int rows, int kb,
                                                     const int32_t* __restrict__ blocks,
                                                     const int32_t* __restrict__ n_kept,
                                                     int32_t* __restrict__ phys,
                                                     int32_t* __restrict__ valid_len,
                                                     int32_t* __restrict__ len_out,
                                                     int32_t* __restrict__ req_out,
                                                     int32_t* __restrict__ sched, int chunks) {
  const int row = blockIdx.x / chunks;
  const int chunk = blockIdx.x % chunks;
  const int i0 = (chunk * 256 + (int)threadIdx.x) * VEC;
  const int nk = min(max(n_kept[row], 0), kb);
  const int rq = req[row];
  const int rqc = clamp_req(rq, kp.num_req);
  const int32_t* pt = kp.page_table + (int64_t)rqc * kp.max_pages;
  auto slot = [&](int b) {
    const int pi = min(max(b / kBlocksPerPage, 0), kp.max_pages - 1);
    return pt[pi] * kBlocksPerPage + b % kBlocksPerPage;
  };
  if (i0 < kb) {
    const int64_t base = (int64_t)row * kb + i0;
    if (VEC == 4) {
      const int4 b = *reinterpret_cast<const int4*>(blocks + base);
      int4 v;
      v.x = i0 < nk ? slot(b.x) : -1;
      v.y = i0 + 1 < nk ? slot(b.y) : -1;
      v.z = i0 + 2 < nk ? slot(b.z) : -1;
      v.w = i0 + 3 < nk ? slot(b.w) : -1;
      *reinterpret_cast<int4*>(phys + base) = v;
    } else {
      phys[base] = i0 < nk ? slot(blocks[base]) : -1;
    }
  }
  if (chunk == 0) {
    const int units = (kb + kUnitBlocks - 1) / kUnitBlocks;
    for (int u = (int)threadIdx.x; u < units; u += 256) {
      const int64_t e = (int64_t)row * units + u;
      sched[4 + 2 * e] = row;
      sched[5 + 2 * e] = u * kUnitBlocks < nk ? u * kUnitBlocks : -1;
    }
    if (threadIdx.x == 0) {
      const int L = len[row];
      const int nblk = L > 0 ? (L + kBlock - 1) / kBlock : 0;
      valid_len[row] = L > 0 ? kBlock * nk - (kBlock * nblk - L) : 0;
      len_out[row] = L;
      req_out[row] = rq;
      if (row == 0) sched[0] = rows * units;
    }
  }
}

// Tables whose kb is not a multiple of 4 (the source's own (k + 1)-block
// table: 513 blocks) are expanded as one flat array of rows * kb candidates:
// thread t takes candidates 4 t .. 4 t + 3 with one 16-byte load and store
// (they may straddle two rows), and the owner of candidate (r, u) also
// writes work-list entry (r, u) for u < U, the owner of (r, 0) the row's
// valid_len, len and req.  Per row (256 candidates a workgroup) the 513-block
// table took three workgroups, the last with one candidate: long chunk
// 0.10-0.11 ms for it beside the first consumer's scores, 0.06-0.08 ms this
// way (the chunk time within noise: the kernel runs on the side stream).
__global__ __launch_bounds__(256) void expand_flat_kernel(PoolArgs kp, const int32_t* __restrict__ req,
                                                          const int32_t* __restrict__ len, int rows, int kb,
                                                          const int32_t* __restrict__ blocks,
                                                          const int32_t* __restrict__ n_kept,
                                                          int32_t* __restrict__ phys,
                                                          int32_t* __restrict__ valid_len,
                                                          int32_t* __restrict__ len_out,
                                                          int32_t* __restrict__ req_out,
                                                          int32_t* __restrict__ sched) {
  const int64_t total = (int64_t)rows * kb;
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e0 >= total) return;
  const int units = (kb + kUnitBlocks - 1) / kUnitBlocks;
  const bool whole = e0 + 3 < total;
  int b[4] = {0, 0, 0, 0};
  if (whole) {
    const int4 v = *reinterpret_cast<const int4*>(blocks + e0);
    b[0] = v.x;
    b[1] = v.y;
    b[2] = v.z;
    b[3] = v.w;
  } else {
    for (int q = 0; q < 4 && e0 + q < total; ++q) b[q] = blocks[e0 + q];
  }
  int row = (int)(e0 / kb);
  int i = (int)(e0 - (int64_t)row * kb);
  int o[4] = {-1, -1, -1, -1};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (e0 + q >= total) break;
    if (i == kb) {
      ++row;
      i = 0;
    }
    const int nk = min(max(n_kept[row], 0), kb);
    if (i < nk) {
      const int32_t* pt = kp.page_table + (int64_t)clamp_req(req[row], kp.num_req) * kp.max_pages;
      const int pi = min(max(b[q] / kBlocksPerPage, 0), kp.max_pages - 1);
      o[q] = pt[pi] * kBlocksPerPage + b[q] % kBlocksPerPage;
    }
    if (i < units) {
      const int64_t e = (int64_t)row * units + i;
      sched[4 + 2 * e] = row;
      sched[5 + 2 * e] = i * kUnitBlocks < nk ? i * kUnitBlocks : -1;
    }
    if (i == 0) {
      const int L = len[row];
      const int nblk = L > 0 ? (L + kBlock - 1) / kBlock : 0;
      valid_len[row] = L > 0 ? kBlock * nk - (kBlock * nblk - L) : 0;
      len_out[row] = L;
      req_out[row] = req[row];
      if (row == 0) sched[0] = rows * units;
    }
    ++i;
  }
  if (whole) {
    *reinterpret_cast<int4*>(phys + e0) = make_int4(o[0], o[1], o[2], o[3]);
  } else {
    for (int q = 0; q < 4 && e0 + q < total; ++q) phys[e0 + q] = o[q];
  }
}

// entries of rows [0, rows): one thread per entry
__global__ __launch_bounds__(256) void schedule_kernel(const int32_t* __restrict__ n_kept, int rows,
                                                       int kb, int32_t* __restrict__ sched) {
  const int units = (kb + kUnitBlocks - 1) / kUnitBlocks;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e == 0) sched[0] = rows * units;
  if (e >= (int64_t)rows * units) return;
  const int r = (int)(e / units), u = (int)(e % units);
  const int nk = min(max(n_kept[r], 0), kb);
  sched[4 + 2 * e] = r;
  sched[5 + 2 * e] = u * kUnitBlocks < nk ? u * kUnitBlocks : -1;
}

// Tail row list on the device (so that the tail step never waits on the host
// and can be captured into a graph).  One workgroup walks the requests in
// slices of 1024 with a block-wide scan and writes, per request j,
//   ts[j]  = first tail row of j = sum_{i<j} t_i   (ts[num_req] = all tail rows)
//   src[j] = first source row of j's tail = sum_{i<j} n_i + n_j - t_j
// with n_j = max(rows_per_req[j], 0) and t_j clamped into [0, n_j].
constexpr int kTailScanThreads = 1024;

__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
  for (int w = 0; w < kTailScanThreads / 64; ++w) {
    before += w < wave ? wsum[w] : 0;
    tot += wsum[w];
  }
  __syncthreads();   // wsum is reused by the next scan
  *total = tot;
  return before + x - v;
}

__global__ __launch_bounds__(kTailScanThreads) void tail_index_kernel(
    const int32_t* __restrict__ rows_per_req, const int32_t* __restrict__ tail_len, int num_req,
    int32_t* __restrict__ ts, int32_t* __restrict__ src) {
  __shared__ int wsum[kTailScanThreads / 64];
  int carry_t = 0, carry_n = 0;
  for (int base = 0; base < num_req; base += kTailScanThreads) {
    const int j = base + (int)threadIdx.x;
    int n = 0, t = 0;
    if (j < num_req) {
      n = max(rows_per_req[j], 0);
      t = min(max(tail_len[j], 0), n);
    }
    int tot_t, tot_n;
    const int et = block_excl_scan(t, wsum, &tot_t);
    const int en = block_excl_scan(n, wsum, &tot_n);
    if (j < num_req) {
      ts[j] = carry_t + et;
      src[j] = carry_n + en + n - t;
    }
    carry_t += tot_t;
    carry_n += tot_n;
  }
  if (threadIdx.x == 0) ts[num_req] = carry_t;
}

// Tail row t copies source row src[j] + (t - ts[j]) of the request j whose tail
// holds it (the last j with ts[j] <= t); rows past ts[num_req] (a tail table
// larger than the tail lengths say) are written empty, and source rows are
// clamped into the full table.
__global__ __launch_bounds__(256) void tail_gather_kernel(
    const int32_t* __restrict__ ts, const int32_t* __restrict__ src, int num_req, int full_rows,
    int kb, const int32_t* __restrict__ blocks,
    const int32_t* __restrict__ n_kept, const int32_t* __restrict__ phys,
    const int32_t* __restrict__ valid_len, const int32_t* __restrict__ len,
    const int32_t* __restrict__ req, int32_t* __restrict__ t_blocks, int32_t* __restrict__ t_n_kept,
    int32_t* __restrict__ t_phys, int32_t* __restrict__ t_valid_len, int32_t* __restrict__ t_len,
    int32_t* __restrict__ t_req, int chunks) {
  const int t = blockIdx.x / chunks;
  const int i = (blockIdx.x % chunks) * 256 + threadIdx.x;
  int s = -1;
  if (full_rows > 0 && t < ts[num_req]) {
    int lo = 0, hi = num_req;   // ts[lo] <= t < ts[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (ts[mid] <= t) lo = mid; else hi = mid;
    }
    s = min(max(src[lo] + (t - ts[lo]), 0), full_rows - 1);
  }
  if (i < kb) {
    t_blocks[(int64_t)t * kb + i] = s >= 0 ? blocks[(int64_t)s * kb + i] : 0x7fffffff;
    t_phys[(int64_t)t * kb + i] = s >= 0 ? phys[(int64_t)s * kb + i] : -1;
  }
  if (i == 0) {
    t_n_kept[t] = s >= 0 ? n_kept[s] : 0;
    t_valid_len[t] = s >= 0 ? valid_len[s] : 0;
    t_len[t] = s >= 0 ? len[s] : 0;
    t_req[t] = s >= 0 ? req[s] : 0;
  }
}

size_t schedule_bytes(int rows, int kb) {
  const size_t units = (size_t)(rows > 0 ? rows : 0) * (size_t)((kb + kUnitBlocks - 1) / kUnitBlocks);
  return 16 + units * 8;
}

hipError_t launch_schedule(const int32_t* n_kept, int rows, int kb, void* schedule,
                           hipStream_t st) {
  const int64_t entries = (int64_t)(rows > 0 ? rows : 0) * ((kb + kUnitBlocks - 1) / kUnitBlocks);
  const int64_t grid = entries > 0 ? (entries + 255) / 256 : 1;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(schedule_kernel, dim3((unsigned)grid), dim3(256), 0, st, n_kept, rows, kb,
                     static_cast<int32_t*>(schedule));
  return hipGetLastError();
}

hipError_t launch_expand(const PoolArgs& kp, const int32_t* req, const int32_t* len, int rows,
                         int kb, const int32_t* blocks, const int32_t* n_kept, int32_t* phys,
                         int32_t* valid_len, int32_t* len_out, int32_t* req_out, void* schedule,
                         hipStream_t st) {
  if (rows <= 0) return launch_schedule(n_kept, 0, kb, schedule, st);
  const bool aligned16 = reinterpret_cast<uintptr_t>(blocks) % 16 == 0 &&
                         reinterpret_cast<uintptr_t>(phys) % 16 == 0;
  const bool vec = kb % 4 == 0 && aligned16;
  int32_t* sched = static_cast<int32_t*>(schedule);
  if (!vec && aligned16) {
    const int64_t grid = ((int64_t)rows * kb + 1023) / 1024;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(expand_flat_kernel, dim3((unsigned)grid), dim3(256), 0, st, kp, req, len, rows, kb,
                       blocks, n_kept, phys, valid_len, len_out, req_out, sched);
    return hipGetLastError();
  }
  const int per_wg = vec ? 1024 : 256;
  const int chunks = (kb + per_wg - 1) / per_wg;
  const int64_t grid = (int64_t)rows * chunks;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (vec)
    hipLaunchKernelGGL(expand_kernel<4>, dim3((unsigned)grid), dim3(256), 0, st, kp, req, len, rows, kb,
                       blocks, n_kept, phys, valid_len, len_out, req_out, sched, chunks);
  else
    hipLaunchKernelGGL(expand_kernel<1>, dim3((unsigned)grid), dim3(256), 0, st, kp, req, len, rows, kb,
                       blocks, n_kept, phys, valid_len, len_out, req_out, sched, chunks);
  return hipGetLastError();
}

size_t tail_workspace_bytes(int num_req) {
  const size_t n = (size_t)(num_req > 0 ? num_req : 0);
  return ((2 * n + 1) * sizeof(int32_t) + 15) / 16 * 16;
}

hipError_t launch_tail(const int32_t* rows_per_req, const int32_t* tail_len, int num_req,
                       void* ws, int full_rows, int tail_rows, int kb, const int32_t* blocks,
                       const int32_t* n_kept, const int32_t* phys, const int32_t* valid_len,
                       const int32_t* len, const int32_t* req, int32_t* t_blocks,
                       int32_t* t_n_kept, int32_t* t_phys, int32_t* t_valid_len, int32_t* t_len,
                       int32_t* t_req, hipStream_t st) {
  if (tail_rows <= 0) return hipSuccess;
  int32_t* ts = static_cast<int32_t*>(ws);
  int32_t* src = ts + (num_req > 0 ? num_req : 0) + 1;
  hipLaunchKernelGGL(tail_index_kernel, dim3(1), dim3(kTailScanThreads), 0, st, rows_per_req,
                     tail_len, num_req, ts, src);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int chunks = (kb + 255) / 256;
  const int64_t grid = (int64_t)tail_rows * chunks;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(tail_gather_kernel, dim3((unsigned)grid), dim3(256), 0, st, ts, src, num_req,
                     full_rows, kb, blocks, n_kept, phys, valid_len, len, req, t_blocks, t_n_kept,
                     t_phys, t_valid_len, t_len, t_req, chunks);
  return hipGetLastError();
}

}  // namespace idxk
