// idx_amax8_varlen: one key per block of 8 scores (the block_amax.cuh contract
// quoted in the review thread of the sglang PR "[DSv4.1] Score prefill consumer
// index layers on candidate blocks with DeepGEMM"; Design, "Level one"):
//   keys[r][i] = max(S[r][8i .. 8i+7]) for i < nblk - 1, keys[r][nblk-1] = +inf,
//   rows with nblk <= skip untouched.
//
// Pure HBM stream: each thread owns 4 keys 256 apart (8 loads of 16 bytes in
// flight), so every load instruction of a wave covers 64 consecutive 32-byte
// blocks (2 KB).  The newest block is never read (its key is +inf whatever it
// holds).  (Measured on MI355X: 4 keys per thread with ordinary cached loads
// streamed fastest; 8 keys, 512 threads or nontemporal loads were slower.)
#include "idx_internal.h"

namespace idxk {

constexpr int kAmaxThreads = 256;
constexpr int kAmaxItems = 4;
constexpr int kAmaxKeys = kAmaxThreads * kAmaxItems;

__global__ __launch_bounds__(kAmaxThreads) void amax8_kernel(const float* __restrict__ S, int64_t ld,
                                                             const int32_t* __restrict__ len,
                                                             float* __restrict__ keys, int64_t ldk,
                                                             int skip, int chunks) {
  const int row = blockIdx.x / chunks;
  const int first = (blockIdx.x % chunks) * kAmaxKeys;
  const int n = len[row];
  const int64_t cap = min(ldk, ld / kBlock);   // a longer row is cut (contract violation)
  const int nblk = (int)min((int64_t)(n > 0 ? (n + kBlock - 1) / kBlock : 0), cap);
  if (nblk <= skip || first >= nblk) return;
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4* in = reinterpret_cast<const f4*>(S + (int64_t)row * ld);
  float* out = keys + (int64_t)row * ldk;
  f4 v[kAmaxItems][2];
#pragma unroll
  for (int j = 0; j < kAmaxItems; ++j) {
    const int i = first + threadIdx.x + j * kAmaxThreads;
    if (i < nblk - 1) {
      v[j][0] = in[2 * i];
      v[j][1] = in[2 * i + 1];
    }
  }
#pragma unroll
  for (int j = 0; j < kAmaxItems; ++j) {
    const int i = first + threadIdx.x + j * kAmaxThreads;
    if (i < nblk - 1) {
      const float a = fmaxf(fmaxf(v[j][0].x, v[j][0].y), fmaxf(v[j][0].z, v[j][0].w));
      const float b = fmaxf(fmaxf(v[j][1].x, v[j][1].y), fmaxf(v[j][1].z, v[j][1].w));
      out[i] = fmaxf(a, b);
    } else if (i == nblk - 1) {
      out[i] = __builtin_inff();
    }
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
