// Candidate expansion, the sparse scorer's work list and the tail-row gather.
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
// Work list layout (int32): [0] unit count, [1..3] unused, then one
// (row, first block) pair per unit of 64 candidate blocks, rows in order.  It
// is built by a single workgroup with a block scan, so it is deterministic.
#include "idx_internal.h"

namespace idxk {

__global__ __launch_bounds__(256) void expand_kernel(PoolArgs kp, const int32_t* __restrict__ req,
                                                     const int32_t* __restrict__ len, int kb,
                                                     const int32_t* __restrict__ blocks,
                                                     const int32_t* __restrict__ n_kept,
                                                     int32_t* __restrict__ phys,
                                                     int32_t* __restrict__ valid_len,
                                                     int32_t* __restrict__ len_out,
                                                     int32_t* __restrict__ req_out, int chunks) {
  const int row = blockIdx.x / chunks;
  const int i = (blockIdx.x % chunks) * 256 + threadIdx.x;
  const int nk = min(max(n_kept[row], 0), kb);
  const int rq = req[row];
  const int rqc = clamp_req(rq, kp.num_req);
  if (i < kb) {
    int32_t v = -1;
    if (i < nk) {
      const int b = blocks[(int64_t)row * kb + i];
      const int pi = min(max(b / kBlocksPerPage, 0), kp.max_pages - 1);
      const int32_t page = kp.page_table[(int64_t)rqc * kp.max_pages + pi];
      v = page * kBlocksPerPage + b % kBlocksPerPage;
    }
    phys[(int64_t)row * kb + i] = v;
  }
  if (i == 0) {
    const int L = len[row];
    const int nblk = L > 0 ? (L + kBlock - 1) / kBlock : 0;
    valid_len[row] = L > 0 ? kBlock * nk - (kBlock * nblk - L) : 0;
    len_out[row] = L;
    req_out[row] = rq;
  }
}

constexpr int kSchedThreads = 1024;

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const int32_t* __restrict__ n_kept,
                                                                 int rows, int kb,
                                                                 int32_t* __restrict__ sched) {
  __shared__ int32_t wsum[kSchedThreads / 64];
  __shared__ int32_t wexcl[kSchedThreads / 64 + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int running = 0;
  for (int base = 0; base < rows; base += kSchedThreads) {
    const int r = base + threadIdx.x;
    const int nk = r < rows ? min(max(n_kept[r], 0), kb) : 0;
    const int units = (nk + kUnitBlocks - 1) / kUnitBlocks;
    int x = units;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (wave == 0) {
      const int s = lane < kSchedThreads / 64 ? wsum[lane] : 0;
      int y = s;
#pragma unroll
      for (int o = 1; o < kSchedThreads / 64; o <<= 1) {
        const int z = __shfl_up(y, o, 64);
        if (lane >= o) y += z;
      }
      if (lane < kSchedThreads / 64) wexcl[lane] = y - s;
      if (lane == kSchedThreads / 64 - 1) wexcl[kSchedThreads / 64] = y;
    }
    __syncthreads();
    const int first = running + wexcl[wave] + x - units;
    for (int u = 0; u < units; ++u) {
      sched[4 + 2 * (first + u)] = r;
      sched[5 + 2 * (first + u)] = u * kUnitBlocks;
    }
    running += wexcl[kSchedThreads / 64];
    __syncthreads();
  }
  if (threadIdx.x == 0) sched[0] = running;
}

__global__ __launch_bounds__(256) void tail_gather_kernel(
    const int32_t* __restrict__ src_rows, int kb, const int32_t* __restrict__ blocks,
    const int32_t* __restrict__ n_kept, const int32_t* __restrict__ phys,
    const int32_t* __restrict__ valid_len, const int32_t* __restrict__ len,
    const int32_t* __restrict__ req, int32_t* __restrict__ t_blocks, int32_t* __restrict__ t_n_kept,
    int32_t* __restrict__ t_phys, int32_t* __restrict__ t_valid_len, int32_t* __restrict__ t_len,
    int32_t* __restrict__ t_req, int chunks) {
  const int t = blockIdx.x / chunks;
  const int i = (blockIdx.x % chunks) * 256 + threadIdx.x;
  const int s = src_rows[t];
  if (i < kb) {
    t_blocks[(int64_t)t * kb + i] = blocks[(int64_t)s * kb + i];
    t_phys[(int64_t)t * kb + i] = phys[(int64_t)s * kb + i];
  }
  if (i == 0) {
    t_n_kept[t] = n_kept[s];
    t_valid_len[t] = valid_len[s];
    t_len[t] = len[s];
    t_req[t] = req[s];
  }
}

size_t schedule_bytes(int rows, int kb) {
  const size_t units = (size_t)(rows > 0 ? rows : 0) * (size_t)((kb + kUnitBlocks - 1) / kUnitBlocks);
  return 16 + units * 8;
}

hipError_t launch_schedule(const int32_t* n_kept, int rows, int kb, void* schedule,
                           hipStream_t st) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, st, n_kept, rows, kb,
                     static_cast<int32_t*>(schedule));
  return hipGetLastError();
}

hipError_t launch_expand(const PoolArgs& kp, const int32_t* req, const int32_t* len, int rows,
                         int kb, const int32_t* blocks, const int32_t* n_kept, int32_t* phys,
                         int32_t* valid_len, int32_t* len_out, int32_t* req_out, void* schedule,
                         hipStream_t st) {
  if (rows <= 0) return launch_schedule(n_kept, 0, kb, schedule, st);
  const int chunks = (kb + 255) / 256;
  const int64_t grid = (int64_t)rows * chunks;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(expand_kernel, dim3((unsigned)grid), dim3(256), 0, st, kp, req, len, kb,
                     blocks, n_kept, phys, valid_len, len_out, req_out, chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_schedule(n_kept, rows, kb, schedule, st);
}

hipError_t launch_tail_gather(const int32_t* src_rows, int tail_rows, int kb,
                              const int32_t* blocks, const int32_t* n_kept, const int32_t* phys,
                              const int32_t* valid_len, const int32_t* len, const int32_t* req,
                              int32_t* t_blocks, int32_t* t_n_kept, int32_t* t_phys,
                              int32_t* t_valid_len, int32_t* t_len, int32_t* t_req,
                              hipStream_t st) {
  if (tail_rows <= 0) return hipSuccess;
  const int chunks = (kb + 255) / 256;
  const int64_t grid = (int64_t)tail_rows * chunks;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(tail_gather_kernel, dim3((unsigned)grid), dim3(256), 0, st, src_rows, kb,
                     blocks, n_kept, phys, valid_len, len, req, t_blocks, t_n_kept, t_phys,
                     t_valid_len, t_len, t_req, chunks);
  return hipGetLastError();
}

}  // namespace idxk
