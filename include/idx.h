/*
 * idx.h -- C ABI of the two-level candidate indexer for MI355X (gfx950).
 *
 * The method (DeepSeek-V4.1 hierarchical sparse indexer, as described by the
 * sglang PR "[DSv4.1] Score prefill consumer index layers on candidate blocks
 * with DeepGEMM", Motivation and Design sections, and the sglang PR "dsv4.1:
 * candidate indexer library", Summary):
 *
 *   source layer   score every reachable compressed position of each query
 *                  row (idx_score_dense), reduce the scores to one key per
 *                  block of 8 positions with the newest block forced to +inf
 *                  (idx_amax8_varlen), keep the kb best blocks, ascending
 *                  (idx_topk_blocks), expand them to pool blocks and record
 *                  the ready event (idx_expand_candidates); take its own
 *                  top-k (idx_topk_rows).
 *   consumer layer score only the published blocks, straight from the paged
 *                  index-K pool (idx_score_sparse_paged), and keep its own
 *                  top-k over them (idx_topk_rows).
 *   tail           restrict a published table to the last rows of each
 *                  request (idx_prefill_tail).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer is a device pointer unless its name ends in _host.
 * - The caller owns every buffer, stream and event.  The library never
 *   allocates or frees device memory and never synchronises the host with
 *   the device: every call only enqueues kernels, event records and event
 *   waits, so any sequence of calls can be captured into a HIP graph.
 * - Every call validates its arguments on the host before enqueuing anything;
 *   on error it returns a negative idx_status, enqueues nothing, and
 *   idx_last_error() describes the problem.  Work is asynchronous on the
 *   given stream (0 = the null stream).
 * - Preconditions that live in device memory are NOT checked (the contents
 *   of len/req/page_table/blocks).  They are listed per call.  Out-of-range
 *   page-table entries are clamped into the pool so that a bad table can
 *   give wrong scores but never reads outside the pool.
 * - Index dimension d = 128, pool page = 64 positions, block = 8 positions.
 *
 * MXFP4 (the vLLM sparse_attn_indexer page, MXFP4 layout constants): each
 * 128-element vector is 64 bytes of e2m1 codes, two per byte (element 2i in
 * the low nibble of byte i), plus 4 ue8m0 scale bytes, one per 32 elements;
 * value = e2m1(code) * 2^(scale - 127).  Scale byte 255 is outside the
 * contract.
 *
 * Score (the "MQA logits" of the index layer: one key vector per position,
 * per-(row, head) weights):
 *     score(r, p) = sum_h w[r,h] * max(0, dot(q[r,h], k[p]))     (fp32)
 */
#ifndef IDX_H_
#define IDX_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IDX_OK = 0,
  IDX_E_ARG = -1,         /* null pointer, negative size, bad enum           */
  IDX_E_ALIGN = -2,       /* pointer or stride misaligned                    */
  IDX_E_SHAPE = -3,       /* sizes inconsistent with each other              */
  IDX_E_UNSUPPORTED = -4, /* valid but not implemented (e.g. dim != 128)     */
  IDX_E_HIP = -5,         /* a HIP runtime call failed                       */
  IDX_E_WORKSPACE = -6    /* workspace missing or smaller than required      */
} idx_status;

/* Message of the last failing call on this thread ("" after a success).
 * Valid until the next idx_* call on the same thread. */
const char* idx_last_error(void);

/* Library version string, e.g. "idx 0.1 gfx950". */
const char* idx_version(void);

/* A query batch of one index layer.
 *   vals   u8  [rows][heads][64]   packed e2m1 codes
 *   scales u8  [rows][heads][4]    ue8m0 scales
 *   w      f32 [rows][heads]       head weights (already folded upstream)
 *   folded u8  [rows][1088]        nullable: this batch's weight-folded query
 *                                  as written by idx_fold_queries; when set,
 *                                  the score calls read it instead of folding
 *                                  the query themselves (their ws may then be
 *                                  NULL).  16-byte aligned.
 * 1 <= heads <= 64 (64 in the model; 8 in small tests); dim must be 128.
 * vals 16-byte, scales and w 4-byte aligned (IDX_E_ALIGN otherwise). */
typedef struct {
  const uint8_t* vals;
  const uint8_t* scales;
  const float* w;
  int32_t rows;
  int32_t heads;
  int32_t dim;
  const uint8_t* folded;
} idx_query;

/* The paged MXFP4 index-K pool (the vLLM sparse_attn_indexer page,
 * kv_cache_as_quant_view: pages of page_size positions, 68 bytes each).
 * Byte layout of page g (page_bytes = page_size * 68):
 *     [0, page_size*64)                 values of slots 0..page_size-1
 *     [page_size*64, page_size*68)      scales of slots 0..page_size-1
 * so a block of 8 positions is 512 contiguous value bytes plus 32
 * contiguous scale bytes.  Position p of request j is slot p % page_size of
 * page page_table[j * max_pages + p / page_size].
 *   pool       u8  [num_pages][page_bytes]
 *   page_table i32 [num_req][max_pages]
 * page_size must be 64, dim 128.  The pool must be 16-byte aligned. */
typedef struct {
  const uint8_t* pool;
  int32_t num_pages;
  int32_t page_size;
  int32_t dim;
  const int32_t* page_table;
  int32_t num_req;
  int32_t max_pages;
} idx_kpool;

/* Per-row metadata of a chunk.
 *   req        i32 [rows]  request of each row (0 <= req < num_req)
 *   len        i32 [rows]  compress_len: the row may see positions [0, len)
 *   pos_offset i32 [rows]  nullable; added to output positions (the request's
 *                          first flattened-K column turns request-relative
 *                          positions into flattened-K columns)
 * Device preconditions (not checked): 0 <= len <= max_pages * page_size. */
typedef struct {
  const int32_t* req;
  const int32_t* len;
  const int32_t* pos_offset;
  int32_t rows;
} idx_rows;

/* A published candidate table (the PR's PrefillSparseBlockTable): one row per
 * query row, all buffers caller-owned.
 *   blocks    i32 [rows][kb]  kept block ids, ascending, INT32_MAX padded
 *   n_kept    i32 [rows]      number of kept blocks = min(nblk, kb)
 *   phys      i32 [rows][kb]  pool block of each kept block:
 *                             page * 8 + block-in-page, -1 padded
 *   valid_len i32 [rows]      number of candidate columns below len: column c
 *                             is position blocks[c/8]*8 + c%8, c < valid_len
 *   len, req  i32 [rows]      copies of the rows it was built from
 *   schedule  u8  [schedule_bytes]  work list of the sparse scorer
 *                             (idx_workspace_bytes(IDX_OP_SCHEDULE, rows, kb, 0))
 *   ready     event recorded when the table is complete (nullable). */
typedef struct {
  int32_t* blocks;
  int32_t* n_kept;
  int32_t* phys;
  int32_t* valid_len;
  int32_t* len;
  int32_t* req;
  void* schedule;
  size_t schedule_bytes;
  int32_t rows;
  int32_t kb;
  hipEvent_t ready;
} idx_table;

/* Workspace sizes (bytes) for the calls that take one. */
enum {
  IDX_OP_TOPK_BLOCKS = 1, /* idx_topk_blocks: rows, width = ldk, k = kb     */
  IDX_OP_TOPK_ROWS = 2,   /* idx_topk_rows:   rows, width = columns, k      */
  IDX_OP_SCHEDULE = 3,    /* idx_table.schedule: rows, width = kb           */
  IDX_OP_TAIL = 4,        /* idx_prefill_tail: rows = num_req               */
  IDX_OP_SCORE = 5        /* idx_score_dense / idx_score_sparse_paged: rows */
};
size_t idx_workspace_bytes(int op, int32_t rows, int64_t width, int32_t k);

/*
 * idx_fold_queries -- the weight-folded queries of n query batches (the index
 * layers of one step) in one launch: ws_host[i] gets batch i's
 * sum_h (w_h/2) q_h as 16 MXFP4 terms per row (what the score calls otherwise
 * write into their own workspace first; see idx_score_dense).  Pass
 * ws_host[i] as q->folded of the later score calls: a step's layers are
 * independent, so their folds fill the GPU together where one layer's rows
 * would not (decode), and they leave the critical path between the score
 * calls.  (The score is the prefill PR's Motivation's sum_h w_h relu(q_h.k),
 * computed as relu(s) = (s + |s|)/2: the folded query carries the linear half.)
 *   qs_host       host array of n query descriptors (their `folded` is ignored)
 *   ws_host       host array of n device pointers, 16-byte aligned
 *   ws_bytes_host host array: ws_bytes_host[i] >= idx_workspace_bytes(IDX_OP_SCORE, qs_host[i].rows, 0, 0)
 * 1 <= n <= 16.
 */
idx_status idx_fold_queries(const idx_query* qs_host, int32_t n, void* const* ws_host,
                            const size_t* ws_bytes_host, hipStream_t stream);

/*
 * idx_score_dense -- the source layer's dense scores.
 * Prefill PR, Motivation: the fp32 [tokens, context] score matrix that the
 * source scores in full; vLLM indexer page: fp8_fp4_mqa_logits over
 * [ks, ke) of each row.
 *   S[r * ld + p] = score(r, p) for p < len[r]; S beyond len[r] is not written.
 * q->rows == rows->rows; ld >= max len (not checked: device data) and
 * 1 <= ld <= 2^29; S must be 4-byte aligned.
 * ws: idx_workspace_bytes(IDX_OP_SCORE, q->rows, 0, 0) device bytes, 16-byte
 * aligned; the call first writes there each row's weight-folded query
 * sum_h (w_h/2) q_h as 16 MXFP4 terms (exact), which lets the kernel use
 * relu(s) = (s + |s|)/2 with the linear half on the MFMA.  With q->folded
 * set, the call reads the folded query there instead and ws is unused.
 */
idx_status idx_score_dense(const idx_query* q, const idx_kpool* kp, const idx_rows* rows,
                           float* S, int64_t ld, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * idx_q_rope_quant -- the step before the score calls: RoPE, MXFP4
 * quantisation and head-weight scaling of one layer's projected queries (the
 * vLLM indexer page, rope_quant_q / fused_indexer_q_rope_quant; on the fp4
 * path the query scales stay with the query).  Its outputs are an idx_query.
 *   q         bf16 bits [rows][heads][128]     projected queries
 *   positions i32 [rows]                       position of each row's token
 *   cos_sin   f32 [max_pos][64]                cos in [0, 32), sin in [32, 64)
 *   w         f32 [rows][heads]                head weights before scaling
 *   is_neox   1: rotate pairs (i, i + 32); 0: pairs (2i, 2i + 1), i < 32
 * For each (row, head): dimensions 0..63 rotated, r0 = bf16(x0 cos - x1 sin),
 * r1 = bf16(x1 cos + x0 sin) with separate fp32 products and sums;
 * dimensions 64..127 unchanged.  Per 32-element group: scale
 * 2^ceil(log2(fp32(max(amax, 1e-10) * fp32(1/6)))), codes = e2m1 nearest to
 * x / scale (ties to the even code, saturated at 6, -0 written as 0).
 *   vals   u8 [rows][heads][64], scales u8 [rows][heads][4] (idx_query layout)
 *   w_out  f32 [rows][heads] = (w * softmax_scale) * head_scale
 * Alignment: q and cos_sin 16 bytes; vals, w, w_out 4 bytes.  1 <= heads <=
 * 64.  Device precondition (clamped, not checked): 0 <= positions < max_pos.
 */
idx_status idx_q_rope_quant(const uint16_t* q, const int32_t* positions, const float* cos_sin,
                            int32_t max_pos, const float* w, int32_t rows, int32_t heads,
                            int32_t is_neox, float softmax_scale, float head_scale, uint8_t* vals,
                            uint8_t* scales, float* w_out, hipStream_t stream);

/*
 * idx_amax8_varlen -- block keys (the block_amax.cuh contract quoted in the
 * prefill PR's review thread, and "Level one" of its Design):
 *   keys[r * ldk + i] = max(S[r*ld + 8i .. 8i+7]) for i < nblk - 1,
 *   keys[r * ldk + nblk - 1] = +inf,          nblk = ceil(len[r] / 8);
 *   rows with nblk <= skip_le_blocks are left untouched (0 = never skip).
 * ld % 8 == 0 and S 32-byte aligned (every block is one 32-byte load), else
 * IDX_E_ALIGN; ld and ldk at most 2^29 (a row below 2 GiB), else IDX_E_ARG.
 * Device precondition: nblk <= ldk for every row (a longer row is cut at
 * min(ldk, ld / 8) keys).  NaN scores are outside the contract.
 */
idx_status idx_amax8_varlen(const float* S, int64_t ld, const int32_t* len, int32_t rows,
                            float* keys, int64_t ldk, int32_t skip_le_blocks, hipStream_t stream);

/*
 * idx_score_dense_keys -- the fused source pass: idx_score_dense and
 * idx_amax8_varlen in one kernel, so the block keys come from the scores
 * while they are still on chip instead of re-reading S (the prefill PR's
 * stated follow-up: block amax folded into the score kernel).
 * S is written exactly as by idx_score_dense(q, kp, rows, S, ld, ws, ...);
 * keys exactly as by idx_amax8_varlen(S, ld, rows->len, rows->rows, keys,
 * ldk, skip_le_blocks) on that S (same fp32 values, newest block +inf, rows
 * with nblk <= skip_le_blocks untouched).
 * Arguments and errors: the union of the two calls' (ld % 8 == 0, ldk >= 1,
 * skip_le_blocks >= 0, keys 4-byte aligned and non-NULL); S needs only 4-byte
 * alignment.  Same workspace as idx_score_dense.
 * S == NULL: keys only -- the scores are computed (in full, as above) but
 * never written, so the [rows, ld] score matrix need not exist; ld still
 * bounds the lengths and the key count (ld >= max len, as with S).  The
 * source's own top-k then comes from rescoring its top-(k + 1) blocks (see
 * idx_topk_blocks_nested).
 */
idx_status idx_score_dense_keys(const idx_query* q, const idx_kpool* kp, const idx_rows* rows,
                                float* S, int64_t ld, float* keys, int64_t ldk,
                                int32_t skip_le_blocks, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/*
 * idx_topk_blocks -- the kb best blocks of each row (prefill PR, "Level one":
 * ragged top-k over the keys, trivial path for rows with at most kb blocks,
 * sort_candidate_blocks' ascending INT32_MAX-padded order).
 *   if nblk <= kb: blocks = 0 .. nblk-1
 *   else: the kb largest keys, ties to the lower block id
 *   blocks[r * kb ..] ascending, INT32_MAX padded; n_kept[r] = min(nblk, kb).
 * ws: idx_workspace_bytes(IDX_OP_TOPK_BLOCKS, rows, ldk, kb) bytes (may be 0).
 */
idx_status idx_topk_blocks(const float* keys, int64_t ldk, const int32_t* len, int32_t rows,
                           int32_t kb, int32_t* blocks, int32_t* n_kept, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/*
 * idx_topk_blocks_nested -- idx_topk_blocks plus, nested inside the kb best
 * blocks, the k2 best (1 <= k2 <= kb <= 4096), by the same rule (if nblk <=
 * k2: blocks 0 .. nblk-1, else the k2 largest keys, ties to the lower block
 * id; ascending, INT32_MAX padded; n_kept2 = min(nblk, k2)).
 *   blocks, n_kept     [rows][kb], [rows]: exactly as idx_topk_blocks
 *   blocks2, n_kept2   [rows][k2], [rows]
 * Device precondition: the keys of every row with nblk > k2 are present
 * (written with skip_le_blocks <= k2); rows with nblk <= kb keep all their
 * blocks in `blocks`, but select their k2 best from the keys.
 * Why (the prefill PR, "The interface": the source layer takes its own
 * top-512): with k2 = k + 1 the source's dense top-k lies inside these k2
 * blocks -- every block holding one of the k best positions has at most k - 1
 * blocks other than the newest above it, with ties going to lower ids at both
 * levels -- so scoring just these 8 k2 positions per row gives the top-k
 * exactly, without the dense score matrix.
 */
idx_status idx_topk_blocks_nested(const float* keys, int64_t ldk, const int32_t* len, int32_t rows,
                                  int32_t kb, int32_t* blocks, int32_t* n_kept, int32_t k2,
                                  int32_t* blocks2, int32_t* n_kept2, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/*
 * idx_expand_candidates -- pool blocks, valid lengths and the sparse work list
 * of a table whose blocks/n_kept were written by idx_topk_blocks (prefill PR,
 * "Level one": pool slots and the schedule; vLLM decode page:
 * candidate_blocks_to_sparse_indices + the sparse logits schedule).  Copies
 * rows->len and rows->req into the table, then records tbl->ready on stream.
 *   phys[r*kb + i] = page_table[req[r]][blocks[r*kb+i] / 8] * 8 + blocks % 8
 *   valid_len[r]   = 8 * n_kept[r] - (8 * nblk - len[r])   (0 when len = 0)
 * tbl->rows == rows->rows; tbl->schedule_bytes >= the IDX_OP_SCHEDULE size.
 */
idx_status idx_expand_candidates(const idx_kpool* kp, const idx_rows* rows, idx_table* tbl,
                                 hipStream_t stream);

/*
 * idx_score_sparse_paged -- a consumer's scores at its candidate positions
 * only (prefill PR, "Level two": scores written [tokens, kb*8] in ascending
 * block order, read straight from the paged pool).  Enqueues the query fold
 * into ws, then makes `stream` wait on tbl->ready (if set) before the scores,
 * so the fold may run while another stream still builds the table.
 *   T[r * ld + c] = score'(r, blocks[r][c/8]*8 + c%8) for c < valid_len[r];
 *   T beyond valid_len[r] is not written.
 * q->rows == tbl->rows; ld >= tbl->kb * 8; the pool must be under 4 GiB
 * (986k pages of 64 positions; else IDX_E_UNSUPPORTED).
 * ws: as for idx_score_dense (IDX_OP_SCORE, q->rows).
 */
idx_status idx_score_sparse_paged(const idx_query* q, const idx_kpool* kp, const idx_table* tbl,
                                  float* T, int64_t ld, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/*
 * idx_score_sparse_paged_noalloc -- idx_score_sparse_paged for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same kernels, with the folded
 * queries in a scratch array inside the library instead of a workspace
 * argument.  Same arguments, results (bit for bit) and errors otherwise.
 *   q->rows <= 4096 (else IDX_E_UNSUPPORTED, nothing enqueued): the scratch
 *   holds 4096 rows x 1088 bytes (4.25 MiB), one copy per GPU, held until
 *   the process ends.  With q->folded set the scratch is not used and the
 *   row limit does not apply.
 * The first call on a device looks the scratch address up with that device
 * current (make that first call outside a graph capture).  Every call on a
 * GPU shares that GPU's scratch, which keeps the last call's contents (each
 * call overwrites the rows it reads; nothing needs clearing): calls that
 * overlap on one GPU -- on different streams, or in graphs replayed
 * concurrently -- race, so the caller orders them.
 */
idx_status idx_score_sparse_paged_noalloc(const idx_query* q, const idx_kpool* kp,
                                          const idx_table* tbl, float* T, int64_t ld,
                                          hipStream_t stream);

/*
 * idx_score_sparse_paged_bf16 -- the same scores written as bf16 (the
 * prefill PR's consumer output, "Level two": bf16 [tokens, 2048 x 8]): each
 * element is the fp32 score of idx_score_sparse_paged rounded to the nearest
 * bf16 (ties to even).  T holds bf16 bit patterns, 2-byte aligned; all else as
 * above.  A variant: selections made from it agree with the fp32 ones only
 * up to the bf16 rounding (the PR's test asks for >= 95% agreement and every
 * disagreement within 2^-5 relative of the selection floor).
 */
idx_status idx_score_sparse_paged_bf16(const idx_query* q, const idx_kpool* kp, const idx_table* tbl,
                                       uint16_t* T, int64_t ld, void* ws, size_t ws_bytes,
                                       hipStream_t stream);

/* Column modes of idx_topk_rows. */
enum {
  IDX_COLS_IDENTITY = 0,  /* column c is position c, value X[c]                   */
  IDX_COLS_BLOCKMAP = 1,  /* column c is position blocks[c/8]*8 + c%8, value X[c]
                             (a consumer's compact scores, "Level two")           */
  IDX_COLS_GATHER = 2     /* column c is position blocks[c/8]*8 + c%8 and its
                             value is read at X[position] (dense scores seen
                             through the candidate blocks)                         */
};

/*
 * idx_topk_rows -- top-k of each row over its first valid[r] columns, ties to
 * the lower column (= lower position: the column map is increasing), mapped
 * to positions, plus pos_offset[r] when given, ascending, -1 past
 * min(k, valid[r]) (prefill PR, "Level two": top-k of the first valid_len
 * columns with the page transform, -1 past min(512, valid_len); the source's
 * own top-512 of "The interface").
 *   out i32 [rows][k]
 * blocks: i32 [rows][kb], required for BLOCKMAP and GATHER (then valid[r] <=
 * kb*8 must hold), ignored for IDENTITY.  ld >= valid (IDENTITY, BLOCKMAP) or
 * ld > every gathered position (GATHER); not checked (device data).
 * ws: idx_workspace_bytes(IDX_OP_TOPK_ROWS, rows, width, k) bytes (may be 0).
 * With mode GATHER over a source's own candidate table this equals the dense
 * top-k of its score rows whenever kb >= k + 1 (every block that holds one of
 * the k best positions has at most k - 1 other blocks above it).
 */
idx_status idx_topk_rows(const float* X, int64_t ld, const int32_t* valid, int32_t rows,
                         int32_t k, int mode, const int32_t* blocks, int32_t kb,
                         const int32_t* pos_offset, int32_t* out, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * idx_topk_rows_bf16 -- idx_topk_rows over bf16 values (bit patterns, 2-byte
 * aligned; the prefill PR's topk_transform_bf16_small over a consumer's bf16
 * scores).  Values compare as the fp32 numbers they are exactly; same modes,
 * tie rule, outputs and errors.
 */
idx_status idx_topk_rows_bf16(const uint16_t* X, int64_t ld, const int32_t* valid, int32_t rows,
                              int32_t k, int mode, const int32_t* blocks, int32_t kb,
                              const int32_t* pos_offset, int32_t* out, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/*
 * idx_prefill_tail -- restrict a published table to the last tail_len[j] rows
 * of each request j (prefill PR, "Tail rows" and its prefill_tail: late
 * layers score only each request's last rows; the table keeps its rows'
 * len/req so the work list can be rebuilt for the tail rows).
 * Request j owns rows [start_j, start_j + rows_per_req[j]) of `full`, start_j
 * being the running sum of rows_per_req; its tail rows are the last
 * tail_len[j] of them, and the tail table lists every request's tail rows in
 * row order.  Waits on full->ready (if set), copies the rows, rebuilds
 * tail->schedule and records tail->ready.  The row list is built on the
 * device, so the call never waits for the host and can be captured into a
 * graph.  On the stream that built `full`, pass full->ready = NULL: a stream
 * waiting on an event it recorded itself adds nothing, and such a wait cannot
 * be expressed in a captured graph.
 *   rows_per_req, tail_len: device i32 [num_req]
 * Host checks: tail->kb == full->kb; tail->rows > 0 needs full->rows > 0 and
 * num_req > 0.  Device preconditions (not checked, clamped): 0 <= tail_len[j]
 * <= rows_per_req[j]; sum rows_per_req == full->rows; sum tail_len ==
 * tail->rows.  A tail length is clamped into [0, rows_per_req[j]], a source
 * row into the full table, and tail rows past sum tail_len are written as
 * empty rows (n_kept = valid_len = 0).
 * ws: idx_workspace_bytes(IDX_OP_TAIL, num_req, 0, 0) device bytes, 4-byte
 * aligned (the per-request prefix sums); may be NULL when tail->rows == 0.
 */
idx_status idx_prefill_tail(const idx_table* full, const int32_t* rows_per_req,
                            const int32_t* tail_len, int32_t num_req, idx_table* tail,
                            void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* IDX_H_ */
