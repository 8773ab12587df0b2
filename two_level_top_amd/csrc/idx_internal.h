// Internal declarations of the gfx950 kernels behind include/idx.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace idxk {

constexpr int kDim = 128;
constexpr int kValBytes = 64;     // packed e2m1 bytes per position
constexpr int kScaleBytes = 4;    // ue8m0 bytes per position
constexpr int kPage = 64;         // positions per pool page
constexpr int kPageValBytes = kPage * kValBytes;               // 4096
constexpr int kPageBytes = kPage * (kValBytes + kScaleBytes);  // 4352
constexpr int kBlock = 8;                                      // positions per block
constexpr int kBlocksPerPage = kPage / kBlock;                 // 8
constexpr int kUnitBlocks = 64;   // candidate blocks per sparse work unit (512 columns)
constexpr int kFoldTerms = 16;    // MXFP4 terms of the folded query (one 16-row MFMA block)
constexpr int kFoldRowBytes = kFoldTerms * (kValBytes + kScaleBytes);  // 1088

// ---------------------------------------------------------------------------
// launch descriptors
// ---------------------------------------------------------------------------
struct QueryArgs {
  const uint8_t* vals;
  const uint8_t* scales;
  const float* w;
  int rows;
  int heads;
};

struct PoolArgs {
  const uint8_t* pool;
  int num_pages;
  const int32_t* page_table;
  int num_req;
  int max_pages;
};

__device__ __forceinline__ int clamp_req(int r, int num_req) {
  return r < 0 ? 0 : (r >= num_req ? num_req - 1 : r);
}

// writes kFoldRowBytes per query row (see fold_query.hip); the batched form
// folds up to kMaxFoldBatches query batches in one launch
constexpr int kMaxFoldBatches = 16;
hipError_t launch_fold_query(const QueryArgs& q, uint8_t* out, hipStream_t st);
hipError_t launch_fold_queries(const QueryArgs* q, uint8_t* const* out, int n, hipStream_t st);

// keys == nullptr: scores only; otherwise also the block keys of
// idx_amax8_varlen(S, ld, len, rows, keys, ldk, skip).
hipError_t launch_score_dense(const QueryArgs& q, const uint8_t* fold, const PoolArgs& kp,
                              const int32_t* req, const int32_t* len, float* S, int64_t ld,
                              float* keys, int64_t ldk, int skip, hipStream_t st);

hipError_t launch_amax8(const float* S, int64_t ld, const int32_t* len, int rows, float* keys,
                        int64_t ldk, int skip, hipStream_t st);

// mode: 0 identity, 1 blockmap, 2 gather, 3 block keys (idx_topk_blocks)
// bf16: X holds bf16 values (modes 0-2)
// mode 3 with k2 > 0: also the k2 best (k2 <= k) into out2 / n_kept2
hipError_t launch_topk(int mode, const void* X, bool bf16, int64_t ld, const int32_t* nvalid,
                       const int32_t* len_for_blocks, int rows, int k, int64_t max_cols,
                       const int32_t* blocks, int kb, const int32_t* pos_offset, int32_t* out,
                       int32_t* n_kept, int k2, int32_t* out2, int32_t* n_kept2, hipStream_t st);

hipError_t launch_expand(const PoolArgs& kp, const int32_t* req, const int32_t* len, int rows,
                         int kb, const int32_t* blocks, const int32_t* n_kept, int32_t* phys,
                         int32_t* valid_len, int32_t* len_out, int32_t* req_out, void* schedule,
                         hipStream_t st);

hipError_t launch_schedule(const int32_t* n_kept, int rows, int kb, void* schedule,
                           hipStream_t st);

hipError_t launch_score_sparse(const QueryArgs& q, const uint8_t* fold, const uint8_t* pool,
                               int num_pages,
                               const int32_t* phys, const int32_t* n_kept,
                               const int32_t* valid_len, int rows, int kb, const void* schedule,
                               void* T, int64_t ld, bool bf16, hipStream_t st);

// the tail table of idx_prefill_tail; ws: tail_workspace_bytes(num_req)
hipError_t launch_tail(const int32_t* rows_per_req, const int32_t* tail_len, int num_req,
                       void* ws, int full_rows, int tail_rows, int kb, const int32_t* blocks,
                       const int32_t* n_kept, const int32_t* phys, const int32_t* valid_len,
                       const int32_t* len, const int32_t* req, int32_t* t_blocks,
                       int32_t* t_n_kept, int32_t* t_phys, int32_t* t_valid_len, int32_t* t_len,
                       int32_t* t_req, hipStream_t st);
size_t tail_workspace_bytes(int num_req);

size_t schedule_bytes(int rows, int kb);
hipError_t launch_q_rope_quant(const uint16_t* q, const int32_t* positions, const float* cos_sin,
                               int max_pos, const float* w, int rows, int heads, bool neox,
                               float softmax_scale, float head_scale, uint8_t* vals,
                               uint8_t* scales, float* w_out, hipStream_t st);

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// One 16x16x128 MXFP4 product: C[16 x 16] += A[16 x 128] * B[128 x 16].
// Lane l supplies row (A) / column (B) l % 16 and the 32 elements
// [32 * (l / 16), 32 * (l / 16) + 32) as 16 bytes, plus that group's ue8m0
// scale.  Output: lane l holds column l % 16, rows 4 * (l / 16) + 0..3.
__device__ __forceinline__ v4f mfma_fp4_16x16x128(uint4 a, uint4 b, int sa, int sb, v4f c) {
  v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  // cbsz = blgp = 4: both operands e2m1
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
}

// v_permlane32_swap: returns {x with its upper half replaced by y's lower half,
//                             x's upper half followed by y's upper half}
__device__ __forceinline__ void swap32(float x, float y, float& lo, float& hi) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// v_permlane16_swap: {x_g0, y_g0, x_g2, y_g2} and {x_g1, y_g1, x_g3, y_g3}
// (g = 16-lane group)
__device__ __forceinline__ void swap16(float x, float y, float& a, float& b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Sum p0..p3 (partials of four 16-column tiles, one per 16-lane group) over
// the four lane groups; lane l receives the total of tile l / 16, column
// l % 16.  Three swaps and three adds.
__device__ __forceinline__ float reduce_scatter4(float p0, float p1, float p2, float p3) {
  float a, b, c, d;
  swap32(p0, p2, a, b);
  const float u = a + b;  // lanes 0-31: tile 0 over groups {g, g+2}; 32-63: tile 2
  swap32(p1, p3, c, d);
  const float v = c + d;  // lanes 0-31: tile 1; 32-63: tile 3
  float e, f;
  swap16(u, v, e, f);
  return e + f;
}

// Raw buffer resource over [p, p + bytes): accesses past the end are dropped
// (stores) or read as zero (loads) by the hardware, so ragged edges need no
// branches.  Dword 3 = 32-bit data format, the raw-buffer setting of gfx9.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buffer_load_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ int64_t clamp_page(int64_t page, int num_pages) {
  return page < 0 ? 0 : (page >= num_pages ? (int64_t)num_pages - 1 : page);
}

}  // namespace idxk
