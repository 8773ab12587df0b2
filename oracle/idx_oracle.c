/*
 * CPU oracle for the two-level candidate indexer: the score arithmetic.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header or table with the HIP library; the two only read the same input
 * bytes.
 *
 * What it computes (exactly, then one rounding to fp32):
 *
 *   logit(r, p) = sum_h w[r,h] * max(0, q^[r,h] . k^[p])
 *
 * where q^ and k^ are the dequantised MXFP4 vectors of a query head and of
 * the index key at compressed position p.  The formula is the head-weighted
 * ReLU score of the DeepSeek-V4.1 index layer ("MQA logits": one key vector
 * per position shared by all index heads, per-(row, head) weights), as the
 * vLLM sparse_attn_indexer page uses it through fp8_fp4_mqa_logits and the
 * sglang PR "[DSv4.1] Score prefill consumer index layers on candidate blocks
 * with DeepGEMM" (Motivation, Design) calls it the dense score matrix.
 *
 * MXFP4 (vLLM sparse_attn_indexer page, the layout constants and the
 * kv_cache_as_quant_view docstring: two values per byte, one ue8m0 byte
 * per 32 elements, 68 bytes per 128-vector):
 *   - e2m1 nibble: bit 3 is the sign, bits 0..2 index {0,.5,1,1.5,2,3,4,6};
 *   - byte i of a vector holds elements 2i (low nibble) and 2i+1 (high);
 *   - ue8m0 byte e is the power of two 2^(e-127); 255 is not a number.
 *
 * Exactness: twice an e2m1 value is an integer in [-12, 12], so the 32-term
 * group sum of (2a)(2b) is an exact integer; scaling by a power of two and
 * adding four groups in double is exact while the group exponents are
 * within ~38 binades of each other (checked below).  The head sum is done
 * in double (relative rounding error ~1e-16, far below one fp32 ulp) and
 * rounded once to float.
 *
 * Paged K pool: page g holds `page_size` positions: first page_size*64
 * value bytes (position-major), then page_size*4 scale bytes.  Position p
 * of request j lives in page page_table[j*max_pages + p/page_size], slot
 * p % page_size.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define DIM 128
#define VB (DIM / 2)
#define SB (DIM / 32)

/* twice the e2m1 magnitude of codes 0..7 */
static const int E2M1_X2[8] = {0, 1, 2, 3, 4, 6, 8, 12};

double oracle_e2m1_value(int nibble) {
  int m = E2M1_X2[nibble & 7];
  return ((nibble & 8) ? -m : m) * 0.5;
}

double oracle_ue8m0_value(int byte) {
  if (byte == 255) return NAN;
  return ldexp(1.0, byte - 127);
}

/* decode the 128 codes of one vector into twice their e2m1 values */
static void decode_x2(const uint8_t* vals, int8_t* out) {
  for (int i = 0; i < DIM; ++i) {
    unsigned b = vals[i >> 1];
    unsigned n = (i & 1) ? (b >> 4) : (b & 15u);
    int m = E2M1_X2[n & 7u];
    out[i] = (int8_t)((n & 8u) ? -m : m);
  }
}

/* exact q^.k^ from decoded codes and the two vectors' scale bytes;
 * *bad is set when a scale byte is 255 or the exactness bound fails */
static double dot_exact(const int8_t* a2, const uint8_t* as, const int8_t* b2,
                        const uint8_t* bs, int* bad) {
  double s = 0.0;
  int emin = 1 << 30, emax = -(1 << 30);
  for (int g = 0; g < SB; ++g) {
    int acc = 0;
    for (int i = 32 * g; i < 32 * g + 32; ++i) acc += (int)a2[i] * (int)b2[i];
    if (as[g] == 255 || bs[g] == 255) *bad = 1;
    int e = (int)as[g] + (int)bs[g] - 254 - 2; /* (2a)(2b) = 4ab */
    if (acc != 0) {
      if (e < emin) emin = e;
      if (e > emax) emax = e;
    }
    s += ldexp((double)acc, e);
  }
  if (emax - emin > 38) *bad = 1;
  return s;
}

static const uint8_t* key_vals(const uint8_t* pool, const int32_t* page_table, int max_pages,
                               int page_size, int req, int pos) {
  int64_t page = page_table[(int64_t)req * max_pages + pos / page_size];
  return pool + page * (int64_t)page_size * (VB + SB) + (int64_t)(pos % page_size) * VB;
}

static const uint8_t* key_scales(const uint8_t* pool, const int32_t* page_table, int max_pages,
                                 int page_size, int req, int pos) {
  int64_t page = page_table[(int64_t)req * max_pages + pos / page_size];
  return pool + page * (int64_t)page_size * (VB + SB) + (int64_t)page_size * VB +
         (int64_t)(pos % page_size) * SB;
}

/* one logit of query row r (decoded heads q2 [H][128], scales qs [H][4], weights w [H]) */
static float logit_one(const int8_t* q2, const uint8_t* qs, const float* w, int H,
                       const int8_t* k2, const uint8_t* ks, int* bad) {
  double acc = 0.0;
  for (int h = 0; h < H; ++h) {
    double s = dot_exact(q2 + (int64_t)h * DIM, qs + (int64_t)h * SB, k2, ks, bad);
    if (s > 0.0) acc += (double)w[h] * s;
  }
  return (float)acc;
}

/*
 * Dense scores of a list of query rows (the source layer's score matrix).
 *   row_ids [n_out]       : which query rows to score
 *   qv [R][H][64], qs [R][H][4], w [R][H]
 *   req [R], len [R]      : request and compress_len of each row
 *   out [n_out][ld]       : out[i][p] for p < len[row_ids[i]]; untouched beyond
 * Returns the number of (row, position) pairs whose exactness check failed.
 */
int64_t oracle_dense_scores(const int32_t* row_ids, int n_out, const uint8_t* qv,
                            const uint8_t* qs, const float* w, int H, const int32_t* req,
                            const int32_t* len, const uint8_t* pool, const int32_t* page_table,
                            int max_pages, int page_size, float* out, int64_t ld) {
  int64_t nbad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : nbad)
  for (int i = 0; i < n_out; ++i) {
    int r = row_ids[i];
    int8_t* q2 = (int8_t*)malloc((size_t)H * DIM);
    int8_t k2[DIM];
    for (int h = 0; h < H; ++h) decode_x2(qv + ((int64_t)r * H + h) * VB, q2 + (int64_t)h * DIM);
    for (int p = 0; p < len[r]; ++p) {
      int bad = 0;
      decode_x2(key_vals(pool, page_table, max_pages, page_size, req[r], p), k2);
      out[(int64_t)i * ld + p] =
          logit_one(q2, qs + (int64_t)r * H * SB, w + (int64_t)r * H, H, k2,
                    key_scales(pool, page_table, max_pages, page_size, req[r], p), &bad);
      nbad += bad;
    }
    free(q2);
  }
  return nbad;
}

/*
 * Consumer scores at the candidate positions of a list of rows.
 *   positions [n_out][ncol] : request-relative compressed position of each
 *                             candidate column (negative = no column)
 *   out [n_out][ld]          : out[i][c] for every column with positions >= 0
 */
int64_t oracle_scores_at(const int32_t* row_ids, int n_out, const uint8_t* qv, const uint8_t* qs,
                         const float* w, int H, const int32_t* req, const int32_t* positions,
                         int64_t ncol, const uint8_t* pool, const int32_t* page_table,
                         int max_pages, int page_size, float* out, int64_t ld) {
  int64_t nbad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : nbad)
  for (int i = 0; i < n_out; ++i) {
    int r = row_ids[i];
    int8_t* q2 = (int8_t*)malloc((size_t)H * DIM);
    int8_t k2[DIM];
    for (int h = 0; h < H; ++h) decode_x2(qv + ((int64_t)r * H + h) * VB, q2 + (int64_t)h * DIM);
    for (int64_t c = 0; c < ncol; ++c) {
      int p = positions[(int64_t)i * ncol + c];
      if (p < 0) continue;
      int bad = 0;
      decode_x2(key_vals(pool, page_table, max_pages, page_size, req[r], p), k2);
      out[(int64_t)i * ld + c] =
          logit_one(q2, qs + (int64_t)r * H * SB, w + (int64_t)r * H, H, k2,
                    key_scales(pool, page_table, max_pages, page_size, req[r], p), &bad);
      nbad += bad;
    }
    free(q2);
  }
  return nbad;
}
