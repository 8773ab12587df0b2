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
// Work list layout (int32): [0] entry count = rows * U, [1..3] unused, then
// U = ceil(kb / 64) (row, first block) entries per row, row-major: entry
// (r, u) is (r, 64 u) when the row keeps more than 64 u blocks, else (r, -1),
// an empty unit the scorer skips.  Every entry is written by the thread that
// owns it, so building the list costs one pass and is deterministic.
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
