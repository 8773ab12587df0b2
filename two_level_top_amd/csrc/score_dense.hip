// idx_score_dense: the source layer's fp32 score matrix over every reachable
// position of each row (the dense score matrix of the sglang PR "[DSv4.1]
// Score prefill consumer index layers on candidate blocks with DeepGEMM",
// Motivation; the vLLM sparse_attn_indexer page's fp8_fp4_mqa_logits over
// each row's [ks, ke)).
//
// Work decomposition (gfx950: 256 CUs in 8 XCDs, wave64):
//   workgroup = 4 waves, 8 query rows (2 per wave), 1024 positions (512 or
//   256 when there are too few rows to fill the chip otherwise, as in decode).
//   workgroup id -> (row group = id / nchunks, chunk = id % nchunks), so
//   consecutive ids -- which the dispatcher spreads over the 8 XCDs -- share
//   a row group and walk different position chunks: each XCD keeps 1/8 of
//   the K pool hot in its L2 and re-reads a row group's query from L2.
//
// MFMA form: v_mfma_scale_f32_32x32x64_f8f6f4, heads on M (32 per block),
// 32 key positions on N, half of the 128 dimensions on K; two such products
// chained give a head block's dot products over all 128 dimensions.  Lane l
// supplies head / position l % 32 and the 32-element group 2 kh + l / 32 of
// K half kh; it receives 16 heads of position l % 32.  The folded queries of
// the wave's two rows (8 MXFP4 terms each, score_common.h) form one more
// 32-row block, whose outputs seed the epilogue's chains.  After the head
// FMAs one permlane32 swap adds the two lane halves, leaving position l of a
// 64-position page in lane l for a coalesced store.
//
// Against the 16x16x128 form this issues 11% more MFMA work per score (the
// fold block is half empty) but the longer products hide more of the
// epilogue's VALU work, and the lane-half sum is one swap per page instead
// of three per four tiles.
//
// A wave keeps its two rows' queries in registers and streams K one pool
// page (64 positions, 2 tiles of 32) at a time straight from the paged pool.
// Two pages are in flight (ping-pong registers, no copies); pages are read
// through a buffer resource and scores/keys stored through resources sized
// to the row's valid range, so the loop has no branches (out-of-range lanes
// are dropped by the hardware).  Rows of a wave that belong to different
// requests are scored one after the other (their keys come from different
// pages).
//
// Fused block keys (the prefill PR's follow-up of folding the block amax into
// the score kernel): lane l holds the score of page position l, so an aligned
// 8-lane DPP max gives the key of every block of the page without reading S
// back.  The keys equal what idx_amax8_varlen computes from the stored S (the
// max of the same fp32 values; the newest block is +inf; rows with
// nblk <= skip are untouched).
#include "score_common.h"

namespace idxk {

// positions per workgroup: 1024, or 512 / 256 when there are few rows (decode)
// so that at least kDenseTargetWGs workgroups run
constexpr int kDenseMaxChunk = 1024;
constexpr int kDenseMinChunk = 256;
constexpr int64_t kDenseTargetWGs = 2048;
constexpr int kDenseWaves = 4;
constexpr int kDenseRowsPerWave = 2;

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// What a launch writes: the scores, the block keys, or both (a keys-only pass
// never materialises the score matrix).
constexpr int kOutScores = 1;
constexpr int kOutKeys = 2;

// Where the fused block keys go (keys == nullptr: not requested).
struct KeyArgs {
  float* keys;
  int64_t ldk;
  int skip;
};

typedef float v16f __attribute__((ext_vector_type(16)));

// max over the aligned group of 8 lanes, in every lane of the group: three
// DPP maxes (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror); the s_nop
// covers the VALU-write -> DPP-read hazard.  Written out because the compiler
// would canonicalize both operands of every fmaxf.
__device__ __forceinline__ float max8_lanes(float v) {
  float a, b, c;
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "=v"(a) : "v"(v));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "=v"(b) : "v"(a));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "=v"(c) : "v"(b));
  return c;
}

// One 32x32x64 MXFP4 product C += A[32 x 64] * B[64 x 32]; SA / SB pick the
// scale byte of each operand's scale register.
template <int SA, int SB>
__device__ __forceinline__ v16f mfma32(uint4 a, uint4 b, int sa, int sb, v16f c) {
  v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, SA, sa, SB, sb);
}

// One query row in 32x32x64 operand form: HH blocks of 32 heads, each as two
// K halves.  Lane l holds head 32 hh + l % 32, group 2 kh + l / 32 (16 code
// bytes); byte 2 hh + kh of sa is that group's ue8m0 scale.  w[hh]: the half
// weights, lane 16 R + i holding head 32 hh + 8 (i / 4) + 4 (R / 2) + i % 4,
// the head whose product output i of the lanes of 16-lane row R receives
// (read with a DPP row broadcast inside the FMA).
template <int HH>
struct Row32 {
  uint4 a[HH][2];
  int sa;
  float w[HH];
};

template <int HH>
__device__ __forceinline__ void load_row32(const QueryArgs& q, int r, int lane, Row32<HH>& f) {
  const int g = lane >> 5;
  f.sa = 0;
#pragma unroll
  for (int hh = 0; hh < HH; ++hh) {
    const int h = 32 * hh + (lane & 31);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int grp = 2 * kh + g;
      int sc = 127;
      if (h < q.heads) {
        const size_t base = (size_t)r * q.heads + h;
        f.a[hh][kh] = *reinterpret_cast<const uint4*>(q.vals + base * kValBytes + grp * 16);
        sc = q.scales[base * kScaleBytes + grp];
      } else {
        f.a[hh][kh] = make_uint4(0u, 0u, 0u, 0u);
      }
      f.sa |= sc << (8 * (2 * hh + kh));
    }
    const int i = lane & 15, R = lane >> 4;
    const int hw = 32 * hh + 8 * (i >> 2) + 4 * (R >> 1) + (i & 3);
    f.w[hh] = hw < q.heads ? 0.5f * q.w[(size_t)r * q.heads + hw] : 0.f;
  }
  asm volatile("s_nop 1" : "+v"(f.w[0]), "+v"(f.w[HH - 1]));   // VALU write -> DPP read of the weights
}

// The folded queries of a pair of rows as one 32-row block: M row 16 p + t
// holds term t < 8 of row p of the pair (rows 16 p + 8 .. 16 p + 15 are
// zero), so output i of a lane receives term 4 (l / 32) + i of row 0 for
// i < 4 and of row 1 for 8 <= i < 12.  Eight of the 16 greedy terms leave a
// residual whose effect on a score stays below a tenth of the score
// tolerance on these inputs.  r1 < 0: row 1's terms are zero.
struct Fold32 {
  uint4 at[2];
  int st;   // byte kh
};

__device__ __forceinline__ void load_fold32(const uint8_t* fold, int r0, int r1, int lane, Fold32& p) {
  const int m = lane & 31, g = lane >> 5;
  const int r = m < 16 ? r0 : r1;
  const int t = m & 15;
  p.st = 127 | (127 << 8);
  p.at[0] = p.at[1] = make_uint4(0u, 0u, 0u, 0u);
  if (r < 0 || t >= kPairFoldTerms) return;
  const uint8_t* fr = fold + (size_t)r * kFoldRowBytes;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const int grp = 2 * kh + g;
    p.at[kh] = *reinterpret_cast<const uint4*>(fr + t * kValBytes + grp * 16);
    p.st = (p.st & ~(255 << (8 * kh))) | ((int)fr[kFoldTerms * kValBytes + t * kScaleBytes + grp] << (8 * kh));
  }
}

// s[i % 4] += (the half weight in lane i of this lane's 16-lane row) * |c[i]|
template <int I>
__device__ __forceinline__ void fma_bcast_abs16(float (&s)[4], float w, const v16f& c) {
  if constexpr (I < 16) {
    asm("v_fmac_f32_dpp %0, %1, |%2| row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(s[I & 3]) : "v"(w), "v"(c[I]), "i"(I));
    fma_bcast_abs16<I + 1>(s, w, c);
  }
}

// MFMA-result -> VALU-read wait states for the inline-asm FMAs, which the
// compiler's hazard tracking does not see into: the head products and the
// chain seeds (fold outputs) pass through one asm statement that waits 20
// states after the last of them
template <int HH>
__device__ __forceinline__ void settle32(v16f (&c)[HH], float (&s)[4]) {
  if constexpr (HH == 1)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : "+v"(c[0]), "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3]));
  else
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : "+v"(c[0]), "+v"(c[1]), "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3]));
}

// K operands of one 32-position tile of a pool page (lane l: position
// 32 T + l % 32, group 2 kh + l / 32); the page's 256 scale bytes are one
// register (lane l: the 4 scale bytes of position l), loaded with tile 0.
struct Tile32 {
  uint4 b[2];
};

// the HH head blocks of one row against tile T, then its share of the score
// of position l % 32: the fold seeds plus 32 HH FMAs in four chains
template <int HH>
__device__ __forceinline__ float row_tile32(const Row32<HH>& f, const uint4 (&b)[2], int sb, float s0,
                                            float s1, float s2, float s3) {
  const v16f zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  v16f c[HH];
  c[0] = mfma32<0, 0>(f.a[0][0], b[0], f.sa, sb, zero);
  c[0] = mfma32<1, 2>(f.a[0][1], b[1], f.sa, sb, c[0]);
  if constexpr (HH == 2) {
    c[1] = mfma32<2, 0>(f.a[1][0], b[0], f.sa, sb, zero);
    c[1] = mfma32<3, 2>(f.a[1][1], b[1], f.sa, sb, c[1]);
  }
  float s[4] = {s0, s1, s2, s3};
  settle32<HH>(c, s);
  fma_bcast_abs16<0>(s, f.w[0], c[0]);
  if constexpr (HH == 2) fma_bcast_abs16<0>(s, f.w[1], c[1]);
  return (s[0] + s[1]) + (s[2] + s[3]);
}

// Score NR (1 or 2) rows of one request against positions [c0, cend) (c0 on
// a page boundary, at most 16 pages).  Every tile of a page is computed;
// positions past a row's length are never stored.  With keys, Krow[r] gets
// the keys of blocks [c0/8, min(cend/8, nblk[r])) (Krow[r] is only used when
// nblk[r] > 0, i.e. the row is keyed).
template <int HH, int NR, int OUTS>
__device__ __forceinline__ void score_rows(const Row32<HH> (&f)[2], const Fold32& pf,
                                           float* const (&Srow)[2],
                                           const int (&lens)[2], float* const (&Krow)[2],
                                           const int (&nblk)[2], const uint8_t* pool,
                                           int num_pages, const int32_t* pt, int max_pages,
                                           int c0, int cend, int lane) {
  const uint32_t voff = (uint32_t)((lane & 31) * kValBytes + (lane >> 5) * 16);
  const uint32_t soff = (uint32_t)(kPageValBytes + lane * kScaleBytes);   // position l's scales
  const int sdist = 4 * (lane & 31);
  const uint32_t sshift = 8u * (uint32_t)(lane >> 5);
  const int npg = (cend - c0 + kPage - 1) / kPage;
  const int pid = (int)clamp_page(pt[min(c0 / kPage + min(lane, npg - 1), max_pages - 1)], num_pages);
  // tile j = 2 page + T
  auto load = [&](int j, Tile32& o, uint32_t* sc) {
    const int i = j >> 1, T = j & 1;
    const int64_t pg = __builtin_amdgcn_readlane(pid, min(i, npg - 1));
    const auto rs = buffer_rsrc(pool + pg * kPageBytes, kPageBytes);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) o.b[kh] = buffer_load_b128(rs, voff + T * 32 * kValBytes + kh * 32);
    if (sc) *sc = __builtin_amdgcn_raw_buffer_load_b32(rs, soff, 0, 0);
  };
  // per-lane store offsets: score of position l of a page; key of block l / 8
  // from lanes 8j (the others get an offset past every resource: dropped)
  const uint32_t soffs = (uint32_t)lane * 4u;
  const uint32_t koffs = (lane & 7) == 0 ? (uint32_t)(lane >> 3) * 4u : 0x80000000u;
  const v16f zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float part[NR][2];
  auto tile = [&](int T, const Tile32& cur, uint32_t sc) {
    // position 32 T + l % 32's scale bytes, shifted so that byte 2 kh is
    // group 2 kh + l / 32
    const int sb = (int)((uint32_t)__builtin_amdgcn_ds_bpermute(sdist + 128 * T, (int)sc) >> sshift);
    v16f F = mfma32<0, 0>(pf.at[0], cur.b[0], pf.st, sb, zero);   // both rows' folds
    F = mfma32<1, 2>(pf.at[1], cur.b[1], pf.st, sb, F);
    part[0][T] = row_tile32<HH>(f[0], cur.b, sb, F[0], F[1], F[2], F[3]);
    if (NR == 2) {
      __builtin_amdgcn_sched_barrier(0);
      part[NR - 1][T] = row_tile32<HH>(f[1], cur.b, sb, F[8], F[9], F[10], F[11]);
    }
  };
  auto finish = [&](int i) {
    // the page's store resources start at its first position (block) and end
    // at the row's length (keys), so the per-lane offsets stay fixed; these
    // are scalar operations
    const int pb0 = c0 + i * kPage;
    const int kb0 = pb0 / kBlock;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      float lo, hi;
      swap32(part[r][0], part[r][1], lo, hi);
      const float tot = lo + hi;   // lane l: page position l
      const uint32_t rem = lens[r] > pb0 ? (uint32_t)(lens[r] - pb0) * 4u : 0u;
      if (OUTS & kOutScores)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), buffer_rsrc(Srow[r] + pb0, rem), soffs, 0, 0);
      if (OUTS & kOutKeys) {
        float key = max8_lanes(tot);
        const int newest = nblk[r] - 1 - kb0;   // the newest block's index in the page
        if (newest >= 0 && newest < kBlocksPerPage)   // (uniform) its key is +inf
          key = (lane >> 3) == newest ? __builtin_inff() : key;
        const uint32_t krem = nblk[r] > kb0 ? (uint32_t)(nblk[r] - kb0) * 4u : 0u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(key), buffer_rsrc(Krow[r] + kb0, krem), koffs, 0, 0);
      }
    }
  };
  Tile32 A, B;
  uint32_t sc, sc_next;
  load(0, A, &sc);
  for (int i = 0; i < npg; ++i) {
    load(2 * i + 1, B, nullptr);
    tile(0, A, sc);
    if (i + 1 < npg) load(2 * i + 2, A, &sc_next);
    tile(1, B, sc);
    finish(i);
    sc = sc_next;
  }
}

template <int HH, int OUTS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void score_dense_kernel(QueryArgs q, const uint8_t* __restrict__ fold,
                                                          PoolArgs kp,
                                                          const int32_t* __restrict__ req,
                                                          const int32_t* __restrict__ len,
                                                          float* __restrict__ S, int64_t ld,
                                                          KeyArgs ka, int nchunks, int chunk_len) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int chunk = blockIdx.x % nchunks;
  const int rg = blockIdx.x / nchunks;
  const int r0 = (rg * kDenseWaves + wave) * kDenseRowsPerWave;
  if (r0 >= q.rows) return;
  const int r1 = r0 + 1 < q.rows ? r0 + 1 : -1;
  // lengths are clamped to [0, min(ld, max_pages * 64)] so that a bad length
  // can never address outside S or the page table
  const int64_t lcap64 = min(ld, (int64_t)kp.max_pages * kPage);
  const int lcap = (int)min(lcap64, (int64_t)0x7fffffff);
  const int req0 = uniform(clamp_req(req[r0], kp.num_req));
  const int len0 = uniform(min(max(len[r0], 0), lcap));
  const int req1 = r1 >= 0 ? uniform(clamp_req(req[r1], kp.num_req)) : -1;
  const int len1 = r1 >= 0 ? uniform(min(max(len[r1], 0), lcap)) : 0;
  // keyed rows: nblk > skip, capped like idx_amax8_varlen (ldk and ld / 8);
  // nblk = 0 marks a row without keys
  int nblk[2] = {0, 0};
  float* Krow[2] = {nullptr, nullptr};
  if (OUTS & kOutKeys) {
    const int64_t kcap = min(ka.ldk, ld / kBlock);
    const int nb0 = (int)min((int64_t)((len0 + kBlock - 1) / kBlock), kcap);
    const int nb1 = (int)min((int64_t)((len1 + kBlock - 1) / kBlock), kcap);
    nblk[0] = nb0 > ka.skip ? nb0 : 0;
    nblk[1] = nb1 > ka.skip ? nb1 : 0;
    Krow[0] = ka.keys + (int64_t)r0 * ka.ldk;
    Krow[1] = r1 >= 0 ? ka.keys + (int64_t)r1 * ka.ldk : Krow[0];
  }
  const int c0 = chunk * chunk_len;
  Row32<HH> f[2];
  Fold32 pf;
  float* Srow[2];
  int lens[2];
  if (r1 >= 0 && req1 == req0) {  // both rows read the same keys
    const int cend = min(c0 + chunk_len, max(len0, len1));
    if (c0 >= cend) return;
    load_row32<HH>(q, r0, lane, f[0]);
    load_row32<HH>(q, r1, lane, f[1]);
    load_fold32(fold, r0, r1, lane, pf);
    Srow[0] = S + (int64_t)r0 * ld;
    Srow[1] = S + (int64_t)r1 * ld;
    lens[0] = len0;
    lens[1] = len1;
    score_rows<HH, 2, OUTS>(f, pf, Srow, lens, Krow, nblk, kp.pool, kp.num_pages,
                            kp.page_table + (int64_t)req0 * kp.max_pages, kp.max_pages, c0, cend, lane);
    return;
  }
  for (int i = 0; i < 2; ++i) {  // rows of different requests, one at a time
    const int r = i == 0 ? r0 : r1;
    if (r < 0) break;
    const int L = i == 0 ? len0 : len1;
    const int rq = i == 0 ? req0 : req1;
    const int cend = min(c0 + chunk_len, L);
    if (c0 >= cend) continue;
    load_row32<HH>(q, r, lane, f[0]);
    load_fold32(fold, r, -1, lane, pf);   // the row in the first half, as in a pair
    Srow[0] = S + (int64_t)r * ld;
    Srow[1] = Srow[0];
    lens[0] = L;
    lens[1] = 0;
    float* const Kr[2] = {Krow[i], Krow[i]};
    const int nb[2] = {nblk[i], 0};
    score_rows<HH, 1, OUTS>(f, pf, Srow, lens, Kr, nb, kp.pool, kp.num_pages,
                            kp.page_table + (int64_t)rq * kp.max_pages, kp.max_pages, c0, cend, lane);
  }
}

template <int OUTS>
static void launch_dense_hh(int hh, dim3 grid, hipStream_t st, const QueryArgs& q, const uint8_t* fold,
                            const PoolArgs& kp, const int32_t* req, const int32_t* len, float* S,
                            int64_t ld, const KeyArgs& ka, int nchunks, int chunk_len) {
  if (hh == 1)
    hipLaunchKernelGGL((score_dense_kernel<1, OUTS>), grid, dim3(256), 0, st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len);
  else
    hipLaunchKernelGGL((score_dense_kernel<2, OUTS>), grid, dim3(256), 0, st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len);
}

hipError_t launch_score_dense(const QueryArgs& q, const uint8_t* fold, const PoolArgs& kp,
                              const int32_t* req, const int32_t* len, float* S, int64_t ld,
                              float* keys, int64_t ldk, int skip, hipStream_t st) {
  const int rows_per_wg = kDenseWaves * kDenseRowsPerWave;
  const int64_t groups = (q.rows + rows_per_wg - 1) / rows_per_wg;
  int chunk_len = kDenseMaxChunk;
  while (chunk_len > kDenseMinChunk && groups * ((ld + chunk_len - 1) / chunk_len) < kDenseTargetWGs)
    chunk_len /= 2;
  const int nchunks = (int)((ld + chunk_len - 1) / chunk_len);
  const int64_t grid = groups * nchunks;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int hh = (q.heads + 31) / 32;
  const KeyArgs ka{keys, ldk, skip};
  if (keys && S)
    launch_dense_hh<kOutScores | kOutKeys>(hh, dim3((unsigned)grid), st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len);
  else if (keys)
    launch_dense_hh<kOutKeys>(hh, dim3((unsigned)grid), st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len);
  else
    launch_dense_hh<kOutScores>(hh, dim3((unsigned)grid), st, q, fold, kp, req, len, S, ld, ka, nchunks, chunk_len);
  return hipGetLastError();
}

}  // namespace idxk
