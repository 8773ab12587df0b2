// C ABI entry points (include/idx.h): host-side validation, then launches on
// the caller's stream.  Nothing is enqueued when validation fails.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "idx.h"
#include "idx_internal.h"

namespace {

thread_local char g_err[512];

idx_status fail(idx_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

idx_status ok() {
  g_err[0] = '\0';
  return IDX_OK;
}

idx_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(IDX_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

idx_status check_query(const idx_query* q, const char* fn) {
  if (!q) return fail(IDX_E_ARG, "%s: query is NULL", fn);
  if (q->rows < 0) return fail(IDX_E_ARG, "%s: query rows < 0", fn);
  if (q->dim != idxk::kDim) return fail(IDX_E_UNSUPPORTED, "%s: dim %d (only 128)", fn, q->dim);
  if (q->heads < 1 || q->heads > 64)
    return fail(IDX_E_UNSUPPORTED, "%s: heads %d (1..64)", fn, q->heads);
  if (q->rows > 0 && (!q->vals || !q->scales || !q->w))
    return fail(IDX_E_ARG, "%s: query vals/scales/w is NULL", fn);
  if (!aligned(q->vals, 16)) return fail(IDX_E_ALIGN, "%s: query vals must be 16-byte aligned", fn);
  if (!aligned(q->scales, 4)) return fail(IDX_E_ALIGN, "%s: query scales must be 4-byte aligned", fn);
  if (!aligned(q->w, 4)) return fail(IDX_E_ALIGN, "%s: query w must be 4-byte aligned", fn);
  if (!aligned(q->folded, 16)) return fail(IDX_E_ALIGN, "%s: folded query must be 16-byte aligned", fn);
  return IDX_OK;
}

idx_status check_pool(const idx_kpool* kp, const char* fn, bool need_table) {
  if (!kp) return fail(IDX_E_ARG, "%s: kpool is NULL", fn);
  if (kp->page_size != idxk::kPage)
    return fail(IDX_E_UNSUPPORTED, "%s: page_size %d (only 64)", fn, kp->page_size);
  if (kp->dim != idxk::kDim) return fail(IDX_E_UNSUPPORTED, "%s: pool dim %d (only 128)", fn, kp->dim);
  if (kp->num_pages < 1 || !kp->pool) return fail(IDX_E_ARG, "%s: empty or NULL pool", fn);
  if (!aligned(kp->pool, 16)) return fail(IDX_E_ALIGN, "%s: pool must be 16-byte aligned", fn);
  if (need_table) {
    if (!kp->page_table) return fail(IDX_E_ARG, "%s: page_table is NULL", fn);
    if (kp->num_req < 1 || kp->max_pages < 1)
      return fail(IDX_E_ARG, "%s: num_req and max_pages must be >= 1", fn);
  }
  return IDX_OK;
}

idx_status check_rows(const idx_rows* r, const char* fn) {
  if (!r) return fail(IDX_E_ARG, "%s: rows is NULL", fn);
  if (r->rows < 0) return fail(IDX_E_ARG, "%s: rows < 0", fn);
  if (r->rows > 0 && (!r->req || !r->len)) return fail(IDX_E_ARG, "%s: req/len is NULL", fn);
  return IDX_OK;
}

idx_status check_score_ws(const void* ws, size_t ws_bytes, int rows, const char* fn) {
  const size_t need = (size_t)(rows > 0 ? rows : 0) * idxk::kFoldRowBytes;
  if (need == 0) return IDX_OK;
  if (!ws || ws_bytes < need)
    return fail(IDX_E_WORKSPACE, "%s: workspace %zu bytes < %zu", fn, ws ? ws_bytes : (size_t)0, need);
  if (!aligned(ws, 16)) return fail(IDX_E_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  return IDX_OK;
}

idx_status check_table(const idx_table* t, const char* fn, bool need_schedule) {
  if (!t) return fail(IDX_E_ARG, "%s: table is NULL", fn);
  if (t->rows < 0) return fail(IDX_E_ARG, "%s: table rows < 0", fn);
  if (t->kb < 1) return fail(IDX_E_ARG, "%s: table kb < 1", fn);
  if (t->rows > 0 && (!t->blocks || !t->n_kept || !t->phys || !t->valid_len || !t->len || !t->req))
    return fail(IDX_E_ARG, "%s: a table buffer is NULL", fn);
  if (need_schedule) {
    if (!t->schedule) return fail(IDX_E_WORKSPACE, "%s: table schedule is NULL", fn);
    const size_t need = idxk::schedule_bytes(t->rows, t->kb);
    if (t->schedule_bytes < need)
      return fail(IDX_E_WORKSPACE, "%s: schedule_bytes %zu < %zu", fn, t->schedule_bytes, need);
    if (!aligned(t->schedule, 4)) return fail(IDX_E_ALIGN, "%s: schedule must be 4-byte aligned", fn);
  }
  return IDX_OK;
}

#define TRY(x)                       \
  do {                               \
    idx_status s_ = (x);             \
    if (s_ != IDX_OK) return s_;     \
  } while (0)

}  // namespace

namespace idxk {

// Scratch of idx_score_sparse_paged_noalloc: the folded queries of up to
// kNoAllocMaxRows query rows, kFoldRowBytes each (4.25 MiB).  Every GPU the
// library runs on holds its own copy until the process ends.  Host code never
// uses this name as an address: the device address comes from
// hipGetSymbolAddress, once per device (scratch_address below).
constexpr int kNoAllocMaxRows = 4096;
__device__ __align__(256) uint8_t scratch[(size_t)kNoAllocMaxRows * kFoldRowBytes];

}  // namespace idxk

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of idxk::scratch, per device

// The current device's address of idxk::scratch (looked up on the first call
// on that device, with that device current).
idx_status scratch_address(void** out, const char* fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(IDX_E_UNSUPPORTED, "%s: device %d beyond the %d the library tracks", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(idxk::scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress of the scratch array");
    if (!p) return fail(IDX_E_HIP, "%s: hipGetSymbolAddress gave a null scratch address", fn);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return IDX_OK;
}

}  // namespace

extern "C" {

const char* idx_last_error(void) { return g_err; }

const char* idx_version(void) { return "idx 0.1 gfx950"; }

size_t idx_workspace_bytes(int op, int32_t rows, int64_t width, int32_t k) {
  (void)width;
  (void)k;
  switch (op) {
    case IDX_OP_TOPK_BLOCKS:
    case IDX_OP_TOPK_ROWS:
      return 0;
    case IDX_OP_SCHEDULE:
      return idxk::schedule_bytes(rows, (int)width);
    case IDX_OP_TAIL:
      return idxk::tail_workspace_bytes(rows);
    case IDX_OP_SCORE:
      return (size_t)(rows > 0 ? rows : 0) * idxk::kFoldRowBytes;
    default:
      return 0;
  }
}

// row offsets of S and of the keys are 32-bit byte offsets inside the kernels
constexpr int64_t kMaxScoreLd = (int64_t)1 << 29;

static idx_status score_dense_impl(const idx_query* q, const idx_kpool* kp, const idx_rows* rows,
                                   float* S, int64_t ld, float* keys, int64_t ldk, int32_t skip,
                                   void* ws, size_t ws_bytes, hipStream_t stream, const char* fn) {
  TRY(check_query(q, fn));
  TRY(check_pool(kp, fn, true));
  TRY(check_rows(rows, fn));
  if (q->rows != rows->rows) return fail(IDX_E_SHAPE, "%s: query rows %d != rows %d", fn, q->rows, rows->rows);
  if (ld < 1) return fail(IDX_E_ARG, "%s: ld < 1", fn);
  if (ld > kMaxScoreLd) return fail(IDX_E_ARG, "%s: ld %lld above 2^29", fn, (long long)ld);
  if (keys) {
    if (skip < 0) return fail(IDX_E_ARG, "%s: skip_le_blocks < 0", fn);
    if (ld % idxk::kBlock != 0)
      return fail(IDX_E_ALIGN, "%s: ld %lld must be a multiple of 8 (whole blocks)", fn, (long long)ld);
    if (ldk < 1) return fail(IDX_E_ARG, "%s: ldk must hold at least one key per row", fn);
  }
  if (rows->rows == 0) return ok();
  if (!S && !keys) return fail(IDX_E_ARG, "%s: S is NULL", fn);   // (keys only: S may be NULL)
  if (!aligned(S, 4)) return fail(IDX_E_ALIGN, "%s: S must be 4-byte aligned", fn);
  if (keys && !aligned(keys, 4)) return fail(IDX_E_ALIGN, "%s: keys must be 4-byte aligned", fn);
  idxk::QueryArgs qa{q->vals, q->scales, q->w, q->rows, q->heads};
  idxk::PoolArgs pa{kp->pool, kp->num_pages, kp->page_table, kp->num_req, kp->max_pages};
  const uint8_t* fold = q->folded;
  if (!fold) {   // fold the query first, into the workspace
    TRY(check_score_ws(ws, ws_bytes, q->rows, fn));
    uint8_t* out = static_cast<uint8_t*>(ws);
    hipError_t e = idxk::launch_fold_query(qa, out, stream);
    if (e != hipSuccess) return hip_status(e, fn);
    fold = out;
  }
  return hip_status(idxk::launch_score_dense(qa, fold, pa, rows->req, rows->len, S, ld, keys, ldk,
                                             skip, stream), fn);
}

idx_status idx_fold_queries(const idx_query* qs_host, int32_t n, void* const* ws_host,
                            const size_t* ws_bytes_host, hipStream_t stream) {
  const char* fn = "idx_fold_queries";
  if (n < 1 || n > idxk::kMaxFoldBatches)
    return fail(IDX_E_ARG, "%s: n = %d (1..%d)", fn, n, idxk::kMaxFoldBatches);
  if (!qs_host || !ws_host || !ws_bytes_host) return fail(IDX_E_ARG, "%s: NULL host array", fn);
  idxk::QueryArgs qa[idxk::kMaxFoldBatches];
  uint8_t* out[idxk::kMaxFoldBatches];
  for (int i = 0; i < n; ++i) {
    TRY(check_query(&qs_host[i], fn));
    TRY(check_score_ws(ws_host[i], ws_bytes_host[i], qs_host[i].rows, fn));
    qa[i] = idxk::QueryArgs{qs_host[i].vals, qs_host[i].scales, qs_host[i].w, qs_host[i].rows,
                            qs_host[i].heads};
    out[i] = static_cast<uint8_t*>(ws_host[i]);
  }
  return hip_status(idxk::launch_fold_queries(qa, out, n, stream), fn);
}

idx_status idx_score_dense(const idx_query* q, const idx_kpool* kp, const idx_rows* rows, float* S,
                           int64_t ld, void* ws, size_t ws_bytes, hipStream_t stream) {
  return score_dense_impl(q, kp, rows, S, ld, nullptr, 0, 0, ws, ws_bytes, stream, "idx_score_dense");
}

idx_status idx_score_dense_keys(const idx_query* q, const idx_kpool* kp, const idx_rows* rows,
                                float* S, int64_t ld, float* keys, int64_t ldk,
                                int32_t skip_le_blocks, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  const char* fn = "idx_score_dense_keys";
  if (!keys && rows && rows->rows > 0) return fail(IDX_E_ARG, "%s: keys is NULL", fn);
  return score_dense_impl(q, kp, rows, S, ld, keys, ldk, skip_le_blocks, ws, ws_bytes, stream, fn);
}

idx_status idx_q_rope_quant(const uint16_t* q, const int32_t* positions, const float* cos_sin,
                            int32_t max_pos, const float* w, int32_t rows, int32_t heads,
                            int32_t is_neox, float softmax_scale, float head_scale, uint8_t* vals,
                            uint8_t* scales, float* w_out, hipStream_t stream) {
  const char* fn = "idx_q_rope_quant";
  if (rows < 0) return fail(IDX_E_ARG, "%s: rows < 0", fn);
  if (heads < 1 || heads > 64) return fail(IDX_E_UNSUPPORTED, "%s: heads %d (1..64)", fn, heads);
  if (max_pos < 1) return fail(IDX_E_ARG, "%s: max_pos < 1", fn);
  if (is_neox != 0 && is_neox != 1) return fail(IDX_E_ARG, "%s: is_neox must be 0 or 1", fn);
  if (rows == 0) return ok();
  if (!q || !positions || !cos_sin || !w || !vals || !scales || !w_out)
    return fail(IDX_E_ARG, "%s: a pointer is NULL", fn);
  if (!aligned(q, 16)) return fail(IDX_E_ALIGN, "%s: q must be 16-byte aligned", fn);
  if (!aligned(cos_sin, 16)) return fail(IDX_E_ALIGN, "%s: cos_sin must be 16-byte aligned", fn);
  if (!aligned(vals, 4) || !aligned(w, 4) || !aligned(w_out, 4))
    return fail(IDX_E_ALIGN, "%s: vals, w and w_out must be 4-byte aligned", fn);
  return hip_status(idxk::launch_q_rope_quant(q, positions, cos_sin, max_pos, w, rows, heads, is_neox == 1,
                                              softmax_scale, head_scale, vals, scales, w_out, stream),
                    fn);
}

idx_status idx_amax8_varlen(const float* S, int64_t ld, const int32_t* len, int32_t rows,
                            float* keys, int64_t ldk, int32_t skip_le_blocks, hipStream_t stream) {
  const char* fn = "idx_amax8_varlen";
  if (rows < 0) return fail(IDX_E_ARG, "%s: rows < 0", fn);
  if (skip_le_blocks < 0) return fail(IDX_E_ARG, "%s: skip_le_blocks < 0", fn);
  if (ld < idxk::kBlock || ld % idxk::kBlock != 0)
    return fail(IDX_E_ALIGN, "%s: ld %lld must be a positive multiple of 8 (32-byte blocks)", fn, (long long)ld);
  if (ld > kMaxScoreLd) return fail(IDX_E_ARG, "%s: ld %lld above 2^29", fn, (long long)ld);
  if (ldk < 1) return fail(IDX_E_ARG, "%s: ldk must hold at least one key per row", fn);
  if (ldk > kMaxScoreLd) return fail(IDX_E_ARG, "%s: ldk %lld above 2^29", fn, (long long)ldk);
  if (rows == 0) return ok();
  if (!S || !len || !keys) return fail(IDX_E_ARG, "%s: S/len/keys is NULL", fn);
  if (!aligned(S, 32)) return fail(IDX_E_ALIGN, "%s: S must be 32-byte aligned", fn);
  if (!aligned(keys, 4)) return fail(IDX_E_ALIGN, "%s: keys must be 4-byte aligned", fn);
  return hip_status(idxk::launch_amax8(S, ld, len, rows, keys, ldk, skip_le_blocks, stream), fn);
}

idx_status idx_topk_blocks(const float* keys, int64_t ldk, const int32_t* len, int32_t rows,
                           int32_t kb, int32_t* blocks, int32_t* n_kept, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  const char* fn = "idx_topk_blocks";
  (void)ws;
  (void)ws_bytes;
  if (rows < 0) return fail(IDX_E_ARG, "%s: rows < 0", fn);
  if (kb < 1) return fail(IDX_E_ARG, "%s: kb < 1", fn);
  if (ldk < 1) return fail(IDX_E_ARG, "%s: ldk < 1", fn);
  if (rows == 0) return ok();
  if (!keys || !len || !blocks || !n_kept) return fail(IDX_E_ARG, "%s: a pointer is NULL", fn);
  return hip_status(idxk::launch_topk(3, keys, false, ldk, nullptr, len, rows, kb, ldk, nullptr, kb,
                                      nullptr, blocks, n_kept, 0, nullptr, nullptr, stream), fn);
}

idx_status idx_topk_blocks_nested(const float* keys, int64_t ldk, const int32_t* len, int32_t rows,
                                  int32_t kb, int32_t* blocks, int32_t* n_kept, int32_t k2,
                                  int32_t* blocks2, int32_t* n_kept2, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  const char* fn = "idx_topk_blocks_nested";
  (void)ws;
  (void)ws_bytes;
  if (rows < 0) return fail(IDX_E_ARG, "%s: rows < 0", fn);
  if (kb < 1) return fail(IDX_E_ARG, "%s: kb < 1", fn);
  if (k2 < 1 || k2 > kb) return fail(IDX_E_ARG, "%s: k2 %d outside [1, kb = %d]", fn, k2, kb);
  if (kb > 4096) return fail(IDX_E_UNSUPPORTED, "%s: kb %d above 4096", fn, kb);
  if (ldk < 1) return fail(IDX_E_ARG, "%s: ldk < 1", fn);
  if (rows == 0) return ok();
  if (!keys || !len || !blocks || !n_kept || !blocks2 || !n_kept2)
    return fail(IDX_E_ARG, "%s: a pointer is NULL", fn);
  return hip_status(idxk::launch_topk(3, keys, false, ldk, nullptr, len, rows, kb, ldk, nullptr, kb,
                                      nullptr, blocks, n_kept, k2, blocks2, n_kept2, stream), fn);
}

idx_status idx_expand_candidates(const idx_kpool* kp, const idx_rows* rows, idx_table* tbl,
                                 hipStream_t stream) {
  const char* fn = "idx_expand_candidates";
  TRY(check_pool(kp, fn, true));
  TRY(check_rows(rows, fn));
  TRY(check_table(tbl, fn, true));
  if (tbl->rows != rows->rows)
    return fail(IDX_E_SHAPE, "%s: table rows %d != rows %d", fn, tbl->rows, rows->rows);
  idxk::PoolArgs pa{kp->pool, kp->num_pages, kp->page_table, kp->num_req, kp->max_pages};
  hipError_t e = idxk::launch_expand(pa, rows->req, rows->len, rows->rows, tbl->kb, tbl->blocks,
                                     tbl->n_kept, tbl->phys, tbl->valid_len, tbl->len, tbl->req,
                                     tbl->schedule, stream);
  if (e != hipSuccess) return hip_status(e, fn);
  if (tbl->ready) return hip_status(hipEventRecord(tbl->ready, stream), "idx_expand_candidates: hipEventRecord");
  return ok();
}

static idx_status score_sparse_impl(const idx_query* q, const idx_kpool* kp, const idx_table* tbl,
                                    void* T, int64_t ld, bool bf16, void* ws, size_t ws_bytes,
                                    hipStream_t stream, const char* fn) {
  TRY(check_query(q, fn));
  TRY(check_pool(kp, fn, false));
  TRY(check_table(tbl, fn, true));
  if (q->rows != tbl->rows) return fail(IDX_E_SHAPE, "%s: query rows %d != table rows %d", fn, q->rows, tbl->rows);
  if (ld < (int64_t)tbl->kb * idxk::kBlock)
    return fail(IDX_E_SHAPE, "%s: ld %lld < kb * 8 = %lld", fn, (long long)ld, (long long)tbl->kb * 8);
  if ((int64_t)kp->num_pages * idxk::kPageBytes > 0xffffffffLL)
    return fail(IDX_E_UNSUPPORTED, "%s: pool of %d pages exceeds 4 GiB", fn, kp->num_pages);
  if (tbl->rows > 0 && !T) return fail(IDX_E_ARG, "%s: T is NULL", fn);
  if (!aligned(T, bf16 ? 2 : 4)) return fail(IDX_E_ALIGN, "%s: T must be %d-byte aligned", fn, bf16 ? 2 : 4);
  // the query fold reads only the query: it is enqueued before the wait on
  // the table, so it can run while the table is still being built
  idxk::QueryArgs qa{q->vals, q->scales, q->w, q->rows, q->heads};
  const uint8_t* fold = q->folded;
  if (!fold) {
    TRY(check_score_ws(ws, ws_bytes, q->rows, fn));
    uint8_t* out = static_cast<uint8_t*>(ws);
    if (tbl->rows > 0) {
      hipError_t e = idxk::launch_fold_query(qa, out, stream);
      if (e != hipSuccess) return hip_status(e, fn);
    }
    fold = out;
  }
  if (tbl->ready) {
    hipError_t e = hipStreamWaitEvent(stream, tbl->ready, 0);
    if (e != hipSuccess) return hip_status(e, "hipStreamWaitEvent on the table's ready event");
  }
  if (tbl->rows == 0) return ok();
  return hip_status(idxk::launch_score_sparse(qa, fold, kp->pool, kp->num_pages, tbl->phys, tbl->n_kept,
                                              tbl->valid_len, tbl->rows, tbl->kb, tbl->schedule, T,
                                              ld, bf16, stream), fn);
}

idx_status idx_score_sparse_paged(const idx_query* q, const idx_kpool* kp, const idx_table* tbl,
                                  float* T, int64_t ld, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  return score_sparse_impl(q, kp, tbl, T, ld, false, ws, ws_bytes, stream, "idx_score_sparse_paged");
}

idx_status idx_score_sparse_paged_noalloc(const idx_query* q, const idx_kpool* kp,
                                          const idx_table* tbl, float* T, int64_t ld,
                                          hipStream_t stream) {
  const char* fn = "idx_score_sparse_paged_noalloc";
  if (!q) return fail(IDX_E_ARG, "%s: query is NULL", fn);
  void* ws = nullptr;
  if (!q->folded) {   // (a folded query needs no scratch)
    if (q->rows > idxk::kNoAllocMaxRows)
      return fail(IDX_E_UNSUPPORTED, "%s: %d query rows above the %d rows of the static scratch", fn,
                  q->rows, idxk::kNoAllocMaxRows);
    if (q->rows > 0) TRY(scratch_address(&ws, fn));
  }
  return score_sparse_impl(q, kp, tbl, T, ld, false, ws, sizeof(idxk::scratch), stream, fn);
}

idx_status idx_score_sparse_paged_bf16(const idx_query* q, const idx_kpool* kp, const idx_table* tbl,
                                       uint16_t* T, int64_t ld, void* ws, size_t ws_bytes,
                                       hipStream_t stream) {
  return score_sparse_impl(q, kp, tbl, T, ld, true, ws, ws_bytes, stream, "idx_score_sparse_paged_bf16");
}

static idx_status topk_rows_impl(const void* X, bool bf16, int64_t ld, const int32_t* valid,
                                 int32_t rows, int32_t k, int mode, const int32_t* blocks, int32_t kb,
                                 const int32_t* pos_offset, int32_t* out, hipStream_t stream,
                                 const char* fn) {
  if (rows < 0) return fail(IDX_E_ARG, "%s: rows < 0", fn);
  if (k < 1) return fail(IDX_E_ARG, "%s: k < 1", fn);
  if (ld < 1) return fail(IDX_E_ARG, "%s: ld < 1", fn);
  if (mode != IDX_COLS_IDENTITY && mode != IDX_COLS_BLOCKMAP && mode != IDX_COLS_GATHER)
    return fail(IDX_E_ARG, "%s: unknown column mode %d", fn, mode);
  if (mode != IDX_COLS_IDENTITY) {
    if (!blocks && rows > 0) return fail(IDX_E_ARG, "%s: blocks is NULL for a block-mapped mode", fn);
    if (kb < 1) return fail(IDX_E_ARG, "%s: kb < 1 for a block-mapped mode", fn);
    if (mode == IDX_COLS_BLOCKMAP && ld < (int64_t)kb * idxk::kBlock)
      return fail(IDX_E_SHAPE, "%s: ld %lld < kb * 8 in block-map mode", fn, (long long)ld);
  }
  if (rows == 0) return ok();
  if (!X || !valid || !out) return fail(IDX_E_ARG, "%s: X/valid/out is NULL", fn);
  if (!aligned(X, bf16 ? 2 : 4)) return fail(IDX_E_ALIGN, "%s: X must be %d-byte aligned", fn, bf16 ? 2 : 4);
  // widest row the call can see: ld columns, or kb * 8 candidate columns
  const int64_t width = mode == IDX_COLS_IDENTITY ? ld : (int64_t)kb * idxk::kBlock;
  return hip_status(idxk::launch_topk(mode, X, bf16, ld, valid, nullptr, rows, k, width, blocks, kb,
                                      pos_offset, out, nullptr, 0, nullptr, nullptr, stream), fn);
}

idx_status idx_topk_rows(const float* X, int64_t ld, const int32_t* valid, int32_t rows, int32_t k,
                         int mode, const int32_t* blocks, int32_t kb, const int32_t* pos_offset,
                         int32_t* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  return topk_rows_impl(X, false, ld, valid, rows, k, mode, blocks, kb, pos_offset, out, stream,
                        "idx_topk_rows");
}

idx_status idx_topk_rows_bf16(const uint16_t* X, int64_t ld, const int32_t* valid, int32_t rows,
                              int32_t k, int mode, const int32_t* blocks, int32_t kb,
                              const int32_t* pos_offset, int32_t* out, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  return topk_rows_impl(X, true, ld, valid, rows, k, mode, blocks, kb, pos_offset, out, stream,
                        "idx_topk_rows_bf16");
}

idx_status idx_prefill_tail(const idx_table* full, const int32_t* rows_per_req,
                            const int32_t* tail_len, int32_t num_req, idx_table* tail, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  const char* fn = "idx_prefill_tail";
  TRY(check_table(full, fn, false));
  TRY(check_table(tail, fn, true));
  if (num_req < 0) return fail(IDX_E_ARG, "%s: num_req < 0", fn);
  if (num_req > 0 && (!rows_per_req || !tail_len))
    return fail(IDX_E_ARG, "%s: rows_per_req/tail_len is NULL", fn);
  if (full->kb != tail->kb) return fail(IDX_E_SHAPE, "%s: kb %d != %d", fn, full->kb, tail->kb);
  if (tail->rows > 0 && (full->rows == 0 || num_req == 0))
    return fail(IDX_E_SHAPE, "%s: %d tail rows from a table of %d rows and %d requests", fn,
                tail->rows, full->rows, num_req);
  const size_t need = idxk::tail_workspace_bytes(num_req);
  if (tail->rows > 0) {
    if (!ws || ws_bytes < need)
      return fail(IDX_E_WORKSPACE, "%s: workspace %zu bytes < %zu", fn, ws ? ws_bytes : (size_t)0, need);
    if (!aligned(ws, 4)) return fail(IDX_E_ALIGN, "%s: workspace must be 4-byte aligned", fn);
  }
  hipError_t e = hipSuccess;
  if (full->ready) {
    e = hipStreamWaitEvent(stream, full->ready, 0);
    if (e != hipSuccess) return hip_status(e, "idx_prefill_tail: hipStreamWaitEvent");
  }
  e = idxk::launch_tail(rows_per_req, tail_len, num_req, ws, full->rows, tail->rows, tail->kb,
                        full->blocks, full->n_kept, full->phys, full->valid_len, full->len,
                        full->req, tail->blocks, tail->n_kept, tail->phys, tail->valid_len,
                        tail->len, tail->req, stream);
  if (e != hipSuccess) return hip_status(e, fn);
  e = idxk::launch_schedule(tail->n_kept, tail->rows, tail->kb, tail->schedule, stream);
  if (e != hipSuccess) return hip_status(e, fn);
  if (tail->ready) return hip_status(hipEventRecord(tail->ready, stream), "idx_prefill_tail: hipEventRecord");
  return ok();
}

}  // extern "C"
