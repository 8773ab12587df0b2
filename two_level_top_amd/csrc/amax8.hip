// idx_amax8_varlen: one key per block of 8 scores (the block_amax.cuh contract
// quoted in the review thread of the sglang PR "[DSv4.1] Score prefill consumer
// index layers on candidate blocks with DeepGEMM"; Design, "Level one"):
//   keys[r][i] = max(S[r][8i .. 8i+7]) for i < nblk - 1, keys[r][nblk-1] = +inf,
//   rows with nblk <= skip untouched.
//
// Pure HBM stream.  A wave owns 64 consecutive blocks (2 KB) and reads them
// with 2 fully coalesced 16-byte loads per lane, both in flight at once: in
// load j lane l holds half (l & 1) of block 32 j + l / 2, so every load
// instruction covers one contiguous 1 KB.  A lane takes the max of its 4
// values and one DPP max with its neighbour gives the block's key in the
// even lane, which stores it.  Loads go through a buffer resource over the
// row's readable blocks and stores through one over its keys, so the body
// has no branches: the newest block (whose key is +inf whatever it holds) and
// blocks past the row's end read as 0 and are not stored.  Loads and stores
// are non-temporal (neither is reused).
//
// Measured on MI355X (long chunk, 16.6 GB read + 2.1 GB written): 2.91 ms,
// 6.4 TB/s = 80% of the 8 TB/s peak, with 2 loads per lane in workgroups of
// 2 waves.  Per lane, 1 load ran at 72%, 4 at 74%, 8 at 70% (16 no better);
// at 2 loads, workgroups of 1, 4 and 8 waves ran at 76%, 80% and 77%.  With
// cached loads and stores (8 loads per lane) it took 3.66 ms; one
// LDS-transposed 16-byte key store per lane gained nothing.
#include "idx_internal.h"

namespace idxk {

constexpr int kAmaxThreads = 128;
constexpr int kAmaxLoads = 2;                                   // 16-byte loads per lane
constexpr int kAmaxWaveBlocks = kAmaxLoads * 32;                // 64
constexpr int kAmaxKeys = kAmaxThreads / 64 * kAmaxWaveBlocks;  // 128 blocks per workgroup
constexpr int kNonTemporal = 2;                                 // buffer op cache policy: nt

// max of 4 floats, then of the pair of lanes (l, l ^ 1) in both lanes; written
// out because the compiler would canonicalize every fmaxf operand loaded from
// memory (NaN is outside the contract).  The s_nop covers the VALU-write ->
// DPP-read hazard.
__device__ __forceinline__ float max4_pair(uint4 v) {
  float m, r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(m) : "v"(v.x), "v"(v.y), "v"(v.z));
  asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(m), "v"(v.w));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "=v"(r) : "v"(m));
  return r;
}

__global__ __launch_bounds__(kAmaxThreads) void amax8_kernel(const float* __restrict__ S, int64_t ld,
                                                             const int32_t* __restrict__ len,
                                                             float* __restrict__ keys, int64_t ldk,
                                                             int skip, int chunks) {
  const int row = blockIdx.x / chunks;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int first = (blockIdx.x % chunks) * kAmaxKeys + wave * kAmaxWaveBlocks;
  const int n = len[row];
  const int64_t cap = min(ldk, ld / kBlock);   // a longer row is cut (contract violation)
  const int nblk = (int)min((int64_t)(n > 0 ? (n + kBlock - 1) / kBlock : 0), cap);
  if (nblk <= skip || first >= nblk) return;
  // readable: the blocks below the newest one; keys: all nblk of them
  const __amdgpu_buffer_rsrc_t in =
      buffer_rsrc(S + (int64_t)row * ld + (int64_t)first * kBlock, (uint32_t)(nblk - 1 - first) * 32u);
  const __amdgpu_buffer_rsrc_t out =
      buffer_rsrc(keys + (int64_t)row * ldk + first, (uint32_t)(nblk - first) * 4u);
  uint4 v[kAmaxLoads];
#pragma unroll
  for (int j = 0; j < kAmaxLoads; ++j) {
    const auto t = __builtin_amdgcn_raw_buffer_load_b128(in, (uint32_t)(j * 1024 + lane * 16), 0, kNonTemporal);
    v[j] = make_uint4(t[0], t[1], t[2], t[3]);
  }
  const int newest = nblk - 1 - first;   // wave-relative index of the +inf key
#pragma unroll
  for (int j = 0; j < kAmaxLoads; ++j) {
    const int b = 32 * j + (lane >> 1);
    const float m = max4_pair(v[j]);
    const float key = b == newest ? __builtin_inff() : m;
    // odd lanes (and blocks past the row, which the resource drops) store nothing
    const uint32_t off = (lane & 1) ? 0x80000000u : (uint32_t)b * 4u;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(key), out, off, 0, kNonTemporal);
  }
}

hipError_t launch_amax8(const float* S, int64_t ld, const int32_t* len, int rows, float* keys,
                        int64_t ldk, int skip, hipStream_t st) {
  const int64_t width = ldk < ld / kBlock ? ldk : ld / kBlock;  // keys a row can need
  const int chunks = (int)((width + kAmaxKeys - 1) / kAmaxKeys);
  const int64_t grid = (int64_t)rows * chunks;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(amax8_kernel, dim3((unsigned)grid), dim3(kAmaxThreads), 0, st, S, ld, len,
                     keys, ldk, skip, chunks);
  return hipGetLastError();
}

}  // namespace idxk
