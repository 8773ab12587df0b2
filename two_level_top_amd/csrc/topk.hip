// Row-wise exact top-k with a fixed tie rule (lower index wins), written in
// ascending index order.  Serves both
//   idx_topk_blocks  the kb best block keys of each row (sglang PR "[DSv4.1]
//                    Score prefill consumer index layers on candidate blocks
//                    with DeepGEMM", Design, "Level one": ragged top-k over
//                    the keys, trivial path for rows with <= kb blocks,
//                    ascending INT32_MAX-padded block ids), and
//   idx_topk_rows    top-k of a row's first `valid` columns, mapped to
//                    positions, -1 past min(k, valid) (same PR, "Level two",
//                    and the source's own top-512).
//
// One workgroup per row, of 256, 512 or 1024 threads (the smallest whose
// registers hold the row: 32 elements per thread), so that several rows run
// on a CU at once and their barriers and load latency overlap.  A row is
// processed in chunks of THREADS * 32 elements held in registers (a whole row
// of block keys or of a consumer's scores is one chunk; longer rows are
// streamed in chunks); wave w owns the contiguous 2048-element slice
// [2048 w, 2048 w + 2048) of a chunk and reads it with coalesced 16-byte
// loads: in step j lane l holds elements 256 j + 4 l .. 256 j + 4 l + 3, all
// in one block of 8.
// Values become order-preserving u32 keys (x >= +0: bits + 2^31; x < 0: the
// negated bits, which puts -0 on the key of +0); slots past the row's end get
// key 0, which lies below -inf, so they are never counted as finite, never
// compare greater than or equal to a threshold, and only ever land in the
// -inf bin, below every valid element.  The kernel is bound by its VALU
// instructions per element, which every pass over the registers keeps to a
// few.
//
//   0. (rows held in registers) a sampled bound: the steps below run on a
//      sample of two keys per thread to pick a bound that between k and the
//      list's capacity elements reach, checked by one counting pass; then
//      step 2 runs at once and step 3 finds K on the list from the top bit
//      down.  On this path the registers hold the raw fp32 patterns and are
//      compared as floats with the value of the bound key (no per-element key
//      instructions); the list entries are keyed after the list pass.  A row
//      whose sample does not give such a bound keys its registers in place
//      and takes steps 1-3.
//   1. threshold bin: one histogram pass over the digit
//      1 + ((key - kmin) >> shift), kmin/kmax being the finite extremes of the
//      row and shift the smallest one that fits the span in 2046 bins (-inf
//      gets digit 0, +inf the one above the largest finite digit): one row's
//      data spreads over the bins, so the LDS atomics rarely collide.  The bin
//      holding the k-th largest key K gives a lower bound for every kept key.
//   2. list: one ordered pass writes (position, key) of every element at or
//      above that bound to an LDS list in index order (each wave gets its
//      predecessors' counts from one 16-entry scan, then walks its slice with
//      ballots and mbcnt).  The list holds the k - need elements above the
//      bin plus the bin itself: about k plus a few hundred entries.
//   3. on the list alone: up to two more histogram passes (<= 11 bits each)
//      over the bin's entries fix the low bits of K and `need`, the number of
//      entries equal to K that are selected; then one block-wide scan of the
//      (greater, equal) counts writes entry e iff key > K, or key == K and
//      fewer than `need` equal keys precede it -- in list order, which is
//      ascending index order.
// A row whose list would not fit LDS (many ties at the threshold, a
// degenerate value spread) takes the register path instead: the bin's keys
// go to an LDS candidate list (or are refined straight from the registers if
// that overflows too), and the ordered compaction runs over the registers
// with separate greater / equal ballots.
#include "idx_internal.h"

namespace idxk {

constexpr int kTopkMaxWaves = 16;
constexpr int kTopkSteps = 8;                          // 16-byte loads per lane per chunk
constexpr int kWaveSlice = kTopkSteps * 256;           // 2048
constexpr int kBins = 2048;                            // 0: -inf, 1..2046 finite, 2047: +inf
constexpr uint32_t kPosInf = 0xff800000u;              // value_key(+inf)
constexpr uint32_t kNegInf = 0x00800000u;              // value_key(-inf)
// finite keys lie in [0x00800001, 0xff7fffff]; empty slots are 0

enum { MODE_IDENTITY = 0, MODE_BLOCKMAP = 1, MODE_GATHER = 2, MODE_KEYS = 3 };

struct TopkArgs {
  const void* X;           // float, or bf16 bits for the BF16 kernels
  int64_t ld;
  const int32_t* nvalid;   // columns per row (modes 0-2)
  const int32_t* len;      // compress_len per row (mode 3: nblk = ceil(len / 8))
  int k;
  const int32_t* blocks;   // [rows][kb] (modes 1, 2)
  int kb;
  const int32_t* pos_offset;
  int32_t* out;            // [rows][k]
  int32_t* n_kept;         // mode 3
  int k2;                  // mode 3, > 0: also the k2 best blocks (k2 <= k) ...
  int32_t* out2;           // ... into out2 [rows][k2]
  int32_t* n_kept2;        // ... and n_kept2 [rows]
};

constexpr uint32_t kCand = 4096;   // register path: keys of the threshold bin
// resident rows try a sampled list bound first (section 0 of the kernel)
constexpr bool kSampledBound = true;

template <int THREADS, bool NEST = false>
struct TopkShared {
  static constexpr int kList = 4 * THREADS;   // list path: (position, key) pairs
  uint32_t hist[kBins];
  uint32_t hist2[NEST ? kBins : 1];           // nested select: the second key's histogram
  union {
    uint32_t cand[kCand];
    uint32_t list[2 * kList];
  };
  uint32_t wred[kTopkMaxWaves][2];
  uint32_t wcnt[kTopkMaxWaves][2];
  uint32_t bcast[8];
};

// u32 image of an fp32 bit pattern, monotone in the value, with -0 and +0 on
// one key: x >= +0 -> bits + 2^31, x < 0 -> -bits (mod 2^32).  Never 0.
__device__ __forceinline__ uint32_t value_key(uint32_t u) {
  const uint32_t s = (uint32_t)((int32_t)u >> 31);
  uint32_t c;   // s ? 1 : 2^31, one bitfield insert (the compiler's own form takes three)
  asm("v_bfi_b32 %0, %1, 1, %2" : "=v"(c) : "v"(s), "s"(0x80000000u));
  return (u ^ s) + c;
}

// Raw fp32 bit patterns of a resident row on the sampled path (see the
// kernel): an empty slot holds a quiet NaN, which every float compare puts
// below any bound and the max below ignores.
constexpr uint32_t kRawEmpty = 0x7fc00000u;
// key of a raw pattern; NaN (an empty slot) -> 0, the empty key
__device__ __forceinline__ uint32_t raw_key(uint32_t u) {
  return (u & 0x7fffffffu) > 0x7f800000u ? 0u : value_key(u);
}
// the fp32 value whose key is `key` (keys of finite values and +-inf; +0 for
// the shared key of +0 and -0), for comparing raw patterns against a key bound
__device__ __forceinline__ float key_float(uint32_t key) {
  return __uint_as_float(key >= 0x80000000u ? key - 0x80000000u : 0u - key);
}
// max of three fp32 patterns, NaN operands ignored (IEEE mode); written out
// because the compiler would canonicalize every operand of fmaxf first
__device__ __forceinline__ uint32_t fmax3_bits(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t d;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// Wave-wide reductions and scans on DPP and permlane moves (VALU only; the
// shuffle forms go through LDS with a round trip per step).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, true);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_shr(uint32_t v) {   // row_shr: lanes shifted in read 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, true);
}
// combine each lane with lanes l ^ 32 and then l ^ 16 (rows already reduced)
template <class Op>
__device__ __forceinline__ uint32_t rows_reduce(uint32_t v, Op op) {
  const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = op(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return op(b[0], b[1]);
}
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op) {
  v = op(v, dpp_u<0xB1>(v));    // quad_perm [1,0,3,2]
  v = op(v, dpp_u<0x4E>(v));    // quad_perm [2,3,0,1]
  v = op(v, dpp_u<0x141>(v));   // row_half_mirror: the 8-lane halves
  v = op(v, dpp_u<0x140>(v));   // row_mirror: the 16-lane row
  return rows_reduce(v, op);
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  return wave_reduce(v, [](uint32_t a, uint32_t b) { return min(a, b); });
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  return wave_reduce(v, [](uint32_t a, uint32_t b) { return max(a, b); });
}
// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_shr<0x111>(x);   // row_shr:1
  x += dpp_shr<0x112>(x);   // row_shr:2
  x += dpp_shr<0x114>(x);   // row_shr:4
  x += dpp_shr<0x118>(x);   // row_shr:8
  const uint32_t t0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
  const uint32_t t1 = t0 + (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
  const uint32_t t2 = t1 + (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row == 0 ? 0u : (row == 1 ? t0 : (row == 2 ? t1 : t2)));
}
// Across the workgroup's waves: c[w][s] holds wave w's value (W <= 16 waves,
// written before a barrier).  Lane w of the reading wave loads wave w's
// value, so the first 16-lane row holds them all and a few DPP steps combine
// them; the results are wave-uniform.  (Each lane summing all W values
// itself took 2 W VALU instructions and a held lane mask per wave.)
template <int W>
__device__ __forceinline__ void wave_sums(const uint32_t (&c)[kTopkMaxWaves][2], int s, int wave,
                                          uint32_t* before, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  uint32_t x = lane < W ? c[lane][s] : 0u;
  x += dpp_shr<0x111>(x);   // inclusive scan over the row
  x += dpp_shr<0x112>(x);
  x += dpp_shr<0x114>(x);
  x += dpp_shr<0x118>(x);
  *total = (uint32_t)__builtin_amdgcn_readlane((int)x, W - 1);
  *before = wave > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)x, wave - 1) : 0u;
}
template <int W, class Op>
__device__ __forceinline__ uint32_t wave_combine(const uint32_t (&c)[kTopkMaxWaves][2], int s, uint32_t ident,
                                                 Op op) {
  const int lane = threadIdx.x & 63;
  uint32_t x = lane < W ? c[lane][s] : ident;
  x = op(x, dpp_u<0xB1>(x));
  x = op(x, dpp_u<0x4E>(x));
  x = op(x, dpp_u<0x141>(x));
  x = op(x, dpp_u<0x140>(x));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
}
__device__ __forceinline__ uint32_t min_u(uint32_t a, uint32_t b) { return min(a, b); }
__device__ __forceinline__ uint32_t max_u(uint32_t a, uint32_t b) { return max(a, b); }

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Bit patterns (as fp32) of the 4 consecutive values starting at element i
// (i % 4 == 0) of the row; CHECK: slots at or past n read as 0 and are
// flagged in `ok`.
template <int MODE, bool VEC, bool BF16, bool CHECK>
__device__ __forceinline__ void load4(const TopkArgs& a, const void* Xr, const int32_t* blk, int i,
                                      int n, uint32_t (&u)[4], bool (&ok)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) ok[e] = !CHECK || i + e < n;
  if (VEC && (!CHECK || i + 3 < n)) {
    int64_t p = i;
    if (MODE == MODE_GATHER) {
      p = (int64_t)blk[i >> 3] * kBlock + (i & 7);
      if (p < 0 || p + 3 >= a.ld) p = 0;   // outside the contract: stay inside the row
    }
    if (BF16) {
      const uint2 x = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(Xr) + p);
      u[0] = x.x << 16; u[1] = x.x & 0xffff0000u; u[2] = x.y << 16; u[3] = x.y & 0xffff0000u;
    } else {
      // non-temporal: every score or key is read once (block top-k 1.04 ->
      // 1.01 ms, source top-k 0.73 -> 0.71 ms on the long chunk)
      typedef unsigned int u4v __attribute__((ext_vector_type(4)));
      const u4v t = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(static_cast<const float*>(Xr) + p));
      const uint4 x = make_uint4(t[0], t[1], t[2], t[3]);
      u[0] = x.x; u[1] = x.y; u[2] = x.z; u[3] = x.w;
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int ie = i + e;
    uint32_t x = 0u;
    if (ok[e]) {
      int64_t p = ie;
      if (MODE == MODE_GATHER) {
        p = (int64_t)blk[ie >> 3] * kBlock + (ie & 7);
        if (p < 0 || p >= a.ld) p = 0;
      }
      x = BF16 ? (uint32_t)static_cast<const uint16_t*>(Xr)[p] << 16 : static_cast<const uint32_t*>(Xr)[p];
    }
    u[e] = x;
  }
}

template <int MODE>
__device__ __forceinline__ int32_t map_index(const int32_t* blk, int i) {
  if (MODE == MODE_BLOCKMAP || MODE == MODE_GATHER) return blk[i >> 3] * kBlock + (i & 7);
  return i;
}

// Select the bin holding the rem-th largest of hist[0..kBins) (counted from
// the top).  Returns the bin; *above gets the count of the bins above it and
// *count the bin's own count.
template <int THREADS, class Sh>
__device__ __forceinline__ int find_bin(Sh& sh, uint32_t rem, uint32_t* above_out, uint32_t* count_out) {
  constexpr int W = THREADS / 64;
  constexpr int BPT = kBins / THREADS;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t cb[BPT];
  uint32_t csum = 0u;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    cb[q] = sh.hist[kBins - 1 - BPT * tid - q];
    csum += cb[q];
  }
  const uint32_t x = wave_incl_scan(csum);
  if (lane == 63) sh.wcnt[wave][0] = x;
  __syncthreads();
  uint32_t before, total;
  wave_sums<W>(sh.wcnt, 0, wave, &before, &total);
  const uint32_t above = before + x - csum;
  if (above < rem && rem <= above + csum) {
    uint32_t acc = above;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      if (acc < rem && rem <= acc + cb[q]) {
        sh.bcast[0] = (uint32_t)(kBins - 1 - BPT * tid - q);
        sh.bcast[1] = acc;
        sh.bcast[3] = cb[q];
      }
      acc += cb[q];
    }
  }
  __syncthreads();
  const int b = (int)sh.bcast[0];
  *above_out = sh.bcast[1];
  *count_out = sh.bcast[3];
  __syncthreads();
  return b;
}

// find_bin on hist and hist2 at once (for ranks rem1 and rem2): both
// histograms' counts packed in one word (each half at most the list size,
// < 2^16), one scan.
template <int THREADS, class Sh>
__device__ __forceinline__ void find_bin2(Sh& sh, uint32_t rem1, uint32_t rem2, uint32_t* b1,
                                          uint32_t* above1, uint32_t* count1, uint32_t* b2,
                                          uint32_t* above2, uint32_t* count2) {
  constexpr int W = THREADS / 64;
  constexpr int BPT = kBins / THREADS;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t cb[BPT];
  uint32_t csum = 0u;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    const int b = kBins - 1 - BPT * tid - q;
    cb[q] = sh.hist[b] | (sh.hist2[b] << 16);
    csum += cb[q];
  }
  const uint32_t x = wave_incl_scan(csum);
  if (lane == 63) sh.wcnt[wave][0] = x;
  __syncthreads();
  uint32_t before, total;
  wave_sums<W>(sh.wcnt, 0, wave, &before, &total);
  const uint32_t above = before + x - csum;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int s = 16 * h;
    const uint32_t rem = h ? rem2 : rem1;
    const uint32_t a = (above >> s) & 0xffffu, c = (csum >> s) & 0xffffu;
    if (a < rem && rem <= a + c) {
      uint32_t acc = a;
#pragma unroll
      for (int q = 0; q < BPT; ++q) {
        const uint32_t v = (cb[q] >> s) & 0xffffu;
        if (acc < rem && rem <= acc + v) {
          sh.bcast[4 * h] = (uint32_t)(kBins - 1 - BPT * tid - q);
          sh.bcast[4 * h + 1] = acc;
          sh.bcast[4 * h + 2] = v;
        }
        acc += v;
      }
    }
  }
  __syncthreads();
  *b1 = sh.bcast[0];
  *above1 = sh.bcast[1];
  *count1 = sh.bcast[2];
  *b2 = sh.bcast[4];
  *above2 = sh.bcast[5];
  *count2 = sh.bcast[6];
  __syncthreads();
}

// RESIDENT: every row fits one chunk (n <= THREADS * 32), loaded once.
// NEST (block keys only): also the nested k2 best blocks (a kernel of its own,
// so that the plain block selection carries none of it)
// Waves per SIMD: a resident 1024-thread row needs 8 for two rows per CU; the
// 512-thread score-row selects too (four rows per CU at 64 VGPRs, a few
// spilled: consumer top-512 0.335 -> 0.303 ms on the long chunk), the others
// keep 6 (their extra code would spill more).
template <int MODE, int THREADS, bool RESIDENT>
constexpr int topk_waves_per_eu() {
  if (!RESIDENT) return 4;
  if (THREADS == 1024) return 8;
  if (THREADS == 512) return (MODE == MODE_BLOCKMAP || MODE == MODE_IDENTITY) ? 8 : 6;
  return 4;
}

template <int MODE, bool VEC, int THREADS, bool RESIDENT, bool BF16, bool NEST = false>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(topk_waves_per_eu<MODE, THREADS, RESIDENT>()))) void topk_kernel(TopkArgs a) {
  constexpr int W = THREADS / 64;
  constexpr int kChunk = W * kWaveSlice;
  constexpr bool kMapped = MODE == MODE_BLOCKMAP || MODE == MODE_GATHER;
  using Sh = TopkShared<THREADS, NEST>;
  constexpr int kList = Sh::kList;
  __shared__ Sh sh;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int n;
  if (MODE == MODE_KEYS) {
    const int L = a.len[row];
    n = L > 0 ? (L + kBlock - 1) / kBlock : 0;
  } else {
    n = a.nvalid[row];
    if (n < 0) n = 0;
    if (kMapped && n > a.kb * kBlock) n = a.kb * kBlock;
  }
  if (MODE != MODE_GATHER && (int64_t)n > a.ld) n = (int)a.ld;   // never read past the row
  const int32_t pad = MODE == MODE_KEYS ? 0x7fffffff : -1;
  const int32_t off = (MODE != MODE_KEYS && a.pos_offset) ? a.pos_offset[row] : 0;
  const int32_t* blk = kMapped ? a.blocks + (int64_t)row * a.kb : nullptr;
  const void* Xr = BF16 ? static_cast<const void*>(static_cast<const uint16_t*>(a.X) + (int64_t)row * a.ld)
                        : static_cast<const void*>(static_cast<const float*>(a.X) + (int64_t)row * a.ld);
  // block keys: the kb best into out and, nested in them, the k2 best into
  // out2 (the source's own top-(k+1) blocks).  The list from which the kb
  // best are written (or, on the register path, the list of the kb best
  // themselves) holds the k2 best too, so the second selection runs on it.
  // A row that keeps all its blocks selects only its k2 best ("second").
  const bool want2 = NEST && MODE == MODE_KEYS && a.k2 > 0;
  bool second = false;

  if (n <= a.k) {  // every column is kept
    int32_t* out = a.out + (int64_t)row * a.k;
    for (int i = tid; i < a.k; i += THREADS) out[i] = i < n ? map_index<MODE>(blk, i) + off : pad;
    if (MODE == MODE_KEYS && tid == 0) a.n_kept[row] = n;
    if (!want2) return;
    if (n <= a.k2) {
      int32_t* out2 = a.out2 + (int64_t)row * a.k2;
      for (int i = tid; i < a.k2; i += THREADS) out2[i] = i < n ? i : pad;
      if (tid == 0) a.n_kept2[row] = n;
      return;
    }
    second = true;
  }
  const bool nest = want2 && !second;   // a second selection on the list
  const int k = second ? a.k2 : a.k;
  int32_t* const out = second ? a.out2 + (int64_t)row * a.k2 : a.out + (int64_t)row * a.k;
  int32_t* const n_kept = second ? a.n_kept2 : a.n_kept;

  const int nchunks = RESIDENT ? 1 : (n + kChunk - 1) / kChunk;
  // A resident row that tries the sampled bound is held as raw fp32 patterns
  // (kRawEmpty in empty slots) and compared as floats, which saves the three
  // key instructions per element; only the sample, the list entries and a
  // row that falls back to the full path are turned into keys.
  constexpr bool kRaw = RESIDENT && kSampledBound && MODE != MODE_GATHER;
  uint32_t key[kTopkSteps][4];
  // element index of key[j][e] in chunk c: c * kChunk + ebase + 256 j + e
  const int ebase = wave * kWaveSlice + 4 * lane;
  auto load_chunk = [&](int c) {
    if ((c + 1) * kChunk <= n) {   // the whole chunk is inside the row
#pragma unroll
      for (int j = 0; j < kTopkSteps; ++j) {
        const int i = c * kChunk + ebase + 256 * j;
        uint32_t u[4];
        bool ok[4];
        load4<MODE, VEC, BF16, false>(a, Xr, blk, i, n, u, ok);
#pragma unroll
        for (int e = 0; e < 4; ++e) key[j][e] = kRaw ? u[e] : value_key(u[e]);
      }
    } else {
      // the row ends in this chunk: only the wave's step that straddles the
      // end checks each element; steps wholly inside load as above, steps
      // wholly past it are empty (consumer top-512 0.41 -> 0.39 ms, block
      // top-2048 1.00 -> 0.99 ms on the long chunk).  The gathered mode keeps
      // one checked path: there the split cost registers and ran 13% slower.
#pragma unroll
      for (int j = 0; j < kTopkSteps; ++j) {
        const int i = c * kChunk + ebase + 256 * j;
        const int s0 = __builtin_amdgcn_readfirstlane(c * kChunk + wave * kWaveSlice + 256 * j);
        uint32_t u[4];
        bool ok[4];
        if (MODE != MODE_GATHER && s0 + 256 <= n) {
          load4<MODE, VEC, BF16, false>(a, Xr, blk, i, n, u, ok);
#pragma unroll
          for (int e = 0; e < 4; ++e) key[j][e] = kRaw ? u[e] : value_key(u[e]);
        } else if (MODE != MODE_GATHER && s0 >= n) {
#pragma unroll
          for (int e = 0; e < 4; ++e) key[j][e] = kRaw ? kRawEmpty : 0u;
        } else {
          load4<MODE, VEC, BF16, true>(a, Xr, blk, i, n, u, ok);
#pragma unroll
          for (int e = 0; e < 4; ++e) key[j][e] = ok[e] ? (kRaw ? u[e] : value_key(u[e])) : (kRaw ? kRawEmpty : 0u);
        }
      }
    }
  };
  if (nchunks == 1) load_chunk(0);

  // write (index, key) of chunk c's elements >= F to the LDS list in index
  // order, from slot p of this wave on (p: the elements >= F before this
  // wave's slice).  Both callers have counted the row's elements >= F (or an
  // upper bound of them) to at most the list's capacity first, so every slot
  // is inside the list.
  auto write_list = [&](int c, uint32_t F0, uint32_t p) {
    // an opaque copy of the bound keeps the counting ballots of the caller
    // from being reused (and all held live) here
    uint32_t F = __builtin_amdgcn_readfirstlane(F0);
    asm volatile("" : "+s"(F));
#pragma unroll
    for (int j = 0; j < kTopkSteps; ++j) {
      uint64_t G[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) G[e] = __ballot(key[j][e] >= F);
      if ((G[0] | G[1] | G[2] | G[3]) != 0u) {
        uint32_t q = p;
#pragma unroll
        for (int e = 0; e < 4; ++e) q += lanes_below(G[e]);
        const int ib = c * kChunk + ebase + 256 * j;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (key[j][e] >= F) {
            *reinterpret_cast<uint2*>(&sh.list[2 * q]) = make_uint2((uint32_t)(ib + e), key[j][e]);
            ++q;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) p += (uint32_t)__popcll(G[e]);
      }
    }
  };

  // write_list on raw patterns (the sampled path): elements whose value is at
  // or above the bound key F0's value, written as raw patterns (keyed after)
  auto write_list_raw = [&](uint32_t F0, uint32_t p) {
    float F = key_float(__builtin_amdgcn_readfirstlane(F0));
    asm volatile("" : "+s"(F));
#pragma unroll
    for (int j = 0; j < kTopkSteps; ++j) {
      uint64_t G[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) G[e] = __ballot(__uint_as_float(key[j][e]) >= F);
      if ((G[0] | G[1] | G[2] | G[3]) != 0u) {
        uint32_t q = p;
#pragma unroll
        for (int e = 0; e < 4; ++e) q += lanes_below(G[e]);
        const int ib = ebase + 256 * j;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (__uint_as_float(key[j][e]) >= F) {
            *reinterpret_cast<uint2*>(&sh.list[2 * q]) = make_uint2((uint32_t)(ib + e), key[j][e]);
            ++q;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) p += (uint32_t)__popcll(G[e]);
      }
    }
  };

  // ---- 3b. ordered output from the list ----
  // K = the k-th largest key, need = how many entries equal to K are kept:
  // thread t takes entries [t E, t E + E); one scan of the packed
  // (greater << 16 | equal) counts gives every entry its output slot; kk =
  // the row's selection size (recorded in n_kept for block keys)
  auto ordered_output = [&](uint32_t K, uint32_t need, uint32_t m, int32_t* out, int32_t* n_kept, int kk) {
    const uint32_t E = (m + THREADS - 1) / THREADS;
    const uint32_t s0 = min((uint32_t)tid * E, m), s1 = min(s0 + E, m);
    uint32_t cnt = 0u;
    for (uint32_t i = s0; i < s1; ++i) {
      const uint32_t x = sh.list[2 * i + 1];
      cnt += x > K ? 0x10000u : (x == K ? 1u : 0u);
    }
    const uint32_t x = wave_incl_scan(cnt);
    if (lane == 63) sh.wcnt[wave][1] = x;
    __syncthreads();
    uint32_t before, total;
    wave_sums<W>(sh.wcnt, 1, wave, &before, &total);
    const uint32_t excl = before + x - cnt;
    uint32_t gpre = excl >> 16, qpre = excl & 0xffffu;
    for (uint32_t i = s0; i < s1; ++i) {
      const uint2 ent = *reinterpret_cast<const uint2*>(&sh.list[2 * i]);
      const bool g = ent.y > K, q = ent.y == K;
      if (g || (q && qpre < need)) out[gpre + min(qpre, need)] = map_index<MODE>(blk, (int)ent.x) + off;
      gpre += g ? 1u : 0u;
      qpre += q ? 1u : 0u;
    }
    if (MODE == MODE_KEYS && tid == 0) n_kept[row] = kk;
  };

  // ---- 3a. on the m list entries: fix the bits of K - base below `low`
  // (the bits above are `fixed`; `need` counts the entries still to take
  // from those with the fixed high bits), 11 bits per histogram pass; then
  // the ordered output
  constexpr bool kRankFinish = MODE == MODE_BLOCKMAP || MODE == MODE_IDENTITY;
  auto refine_output = [&](uint32_t base, uint32_t fixed, int low, uint32_t need, uint32_t m,
                           int32_t* out, int32_t* n_kept, int kk) {
    while (low > 0) {
      const int width = low < 11 ? low : 11;
      const int sh_lo = low - width;
      const uint32_t hi_mask = low >= 32 ? 0u : ~((1u << low) - 1u);
      for (int b = tid; b < kBins; b += THREADS) sh.hist[b] = 0u;
      if (tid == 0) sh.bcast[2] = 0u;
      __syncthreads();
      for (uint32_t i = tid; i < m; i += THREADS) {
        const uint32_t r = sh.list[2 * i + 1] - base;
        if ((r & hi_mask) == fixed) atomicAdd(&sh.hist[(r >> sh_lo) & ((1u << width) - 1u)], 1u);
      }
      __syncthreads();
      uint32_t ab, cnt;
      const uint32_t d = (uint32_t)find_bin<THREADS>(sh, need, &ab, &cnt);
      need -= ab;
      fixed |= d << sh_lo;
      low = sh_lo;
      if (cnt == need) {
        // every entry of the bin is kept: the selection is the entries at or
        // above the bin's lower edge (ties inside it are all taken, so the
        // tie rule has nothing to decide), and the low bits need no pass
        ordered_output(base + fixed - 1u, 0u, m, out, n_kept, kk);
        return;
      }
      // (score rows only: in the gathered and nested block selects the extra
      // code cost more registers than the saved pass gained)
      if (kRankFinish && low > 0 && cnt <= 64u) {
        // a few entries left with K's high bits: rank them directly instead
        // of further passes.  Their keys go to hist[0 .. cnt) (free again
        // after find_bin); wave w ranks keys w, w + W, ...: key i is K when
        // fewer than `need` keys are above it and at least `need` at or above
        // it (each wave compares one key with all of them, one per lane).
        const uint32_t lo_mask = ~((1u << low) - 1u);
        for (uint32_t i = tid; i < m; i += THREADS) {
          const uint32_t x = sh.list[2 * i + 1];
          if (((x - base) & lo_mask) == fixed) sh.hist[atomicAdd(&sh.bcast[2], 1u)] = x;
        }
        __syncthreads();
        const bool in = lane < (int)cnt;
        const uint32_t xl = in ? sh.hist[lane] : 0u;
        for (uint32_t i = wave; i < cnt; i += W) {
          const uint32_t xi = sh.hist[i];
          const uint32_t g = (uint32_t)__popcll(__ballot(in && xl > xi));
          const uint32_t eq = (uint32_t)__popcll(__ballot(in && xl == xi));
          if (lane == 0 && g < need && need <= g + eq) {   // (equal keys write equal values)
            sh.bcast[0] = xi;
            sh.bcast[1] = need - g;
          }
        }
        __syncthreads();
        const uint32_t K = sh.bcast[0], neq = sh.bcast[1];
        ordered_output(K, neq, m, out, n_kept, kk);
        return;
      }
    }
    ordered_output(base + fixed, need, m, out, n_kept, kk);
  };

  // Both selections of a nested row from one list (every entry >= base, the
  // k best and, nested in them, the k2 best): their keys are refined in the
  // same passes, one histogram each, then written one after the other.
  auto refine_dual = [&](uint32_t base, int low, uint32_t m) {
    uint32_t need1 = (uint32_t)a.k, need2 = (uint32_t)a.k2, fixed1 = 0u, fixed2 = 0u;
    // a selection whose bin is kept whole is done (as in refine_output): its
    // threshold is the bin's lower edge, and it takes no more passes
    bool done1 = false, done2 = false;
    while (low > 0 && !(done1 && done2)) {
      const int width = low < 11 ? low : 11;
      const int sh_lo = low - width;
      const uint32_t hi_mask = low >= 32 ? 0u : ~((1u << low) - 1u);
      const uint32_t msk = (1u << width) - 1u;
      for (int b = tid; b < kBins; b += THREADS) {
        sh.hist[b] = 0u;
        sh.hist2[b] = 0u;
      }
      __syncthreads();
      for (uint32_t i = tid; i < m; i += THREADS) {
        const uint32_t r = sh.list[2 * i + 1] - base;
        const uint32_t hi = r & hi_mask, d = (r >> sh_lo) & msk;
        if (!done1 && hi == fixed1) atomicAdd(&sh.hist[d], 1u);
        if (!done2 && hi == fixed2) atomicAdd(&sh.hist2[d], 1u);
      }
      __syncthreads();
      uint32_t d1, ab1, c1, d2, ab2, c2;
      find_bin2<THREADS>(sh, need1, need2, &d1, &ab1, &c1, &d2, &ab2, &c2);
      if (!done1) {
        need1 -= ab1;
        fixed1 |= d1 << sh_lo;
        done1 = c1 == need1;
      }
      if (!done2) {
        need2 -= ab2;
        fixed2 |= d2 << sh_lo;
        done2 = c2 == need2;
      }
      low = sh_lo;
    }
    ordered_output(done1 ? base + fixed1 - 1u : base + fixed1, done1 ? 0u : need1, m,
                   a.out + (int64_t)row * a.k, a.n_kept, a.k);
    __syncthreads();   // the first output has read the list counts
    ordered_output(done2 ? base + fixed2 - 1u : base + fixed2, done2 ? 0u : need2, m,
                   a.out2 + (int64_t)row * a.k2, a.n_kept2, a.k2);
  };

  // the k2 best blocks from the list of a first selection: every entry is at
  // or above `bound`, and the list holds at least k2 entries
  auto nested_output = [&](uint32_t bound, uint32_t m) {
    __syncthreads();   // the first output has read the list counts
    const uint32_t span = kPosInf - bound;
    refine_output(bound, 0u, span ? 32 - __clz(span) : 0, (uint32_t)a.k2, m,
                  a.out2 + (int64_t)row * a.k2, a.n_kept2, a.k2);
  };



  // ---- 0. resident rows: a threshold from a sample ----
  // Two keys per thread, spread over each wave's slice, go through the same
  // adaptive histogram as the whole row would (section 1 below), and the
  // lower edge of the bin holding the sample's r-th largest key, r = k / 16
  // plus three standard deviations (the sample is 1/16 of a full chunk),
  // becomes the list's bound: k (1 + 3 / sqrt(k / 16)) elements of the row
  // are expected at or above it.  One counting pass checks that at least k
  // and at most the list's capacity are; then the list pass runs at once,
  // and K is found on the list alone (its bits from the top, 11 per pass).
  // Otherwise -- a sample too small or too skewed, the k-th key at -inf --
  // the row takes the path below.  The extremes and histogram passes over
  // every element (and their LDS atomics) are skipped; the result is the
  // same.  (Long chunk: block top-2048 0.99 -> 0.84 ms, consumer top-512
  // 0.39 -> 0.36 ms.  The gathered mode, bound by its scattered loads, ran
  // 25% slower with it, whatever the sample positions, so it keeps the full
  // path.)
  if (kRaw) {
    const uint32_t sa = raw_key(key[0][0]), sb = raw_key(key[kTopkSteps / 2][2]);
    uint32_t symax = max(sa + 0x00800000u, sb + 0x00800000u);
    uint32_t szmin = min(sa - 0x00800001u, sb - 0x00800001u);
    // the row's largest key (+inf included): the refine width
    uint32_t vmax = kRawEmpty;
#pragma unroll
    for (int j = 0; j < kTopkSteps; ++j) vmax = fmax3_bits(fmax3_bits(vmax, key[j][0], key[j][1]), key[j][2], key[j][3]);
    uint32_t kall = raw_key(vmax);
    symax = wave_max(symax);
    szmin = wave_min(szmin);
    kall = wave_max(kall);
    if (lane == 0) {
      sh.wred[wave][0] = szmin;
      sh.wred[wave][1] = symax;
      sh.wcnt[wave][1] = kall;
    }
    for (int b = tid; b < kBins; b += THREADS) sh.hist[b] = 0u;
    __syncthreads();
    szmin = wave_combine<W>(sh.wred, 0, 0xffffffffu, min_u);
    symax = wave_combine<W>(sh.wred, 1, 0u, max_u);
    kall = wave_combine<W>(sh.wcnt, 1, 0u, max_u);
    uint32_t smin = 0x80000000u, smax = 0x80000000u;
    if (szmin <= 0xfefffffeu) {
      smin = szmin + 0x00800001u;
      smax = symax - 0x00800000u;
    }
    smin = __builtin_amdgcn_readfirstlane(smin);
    smax = __builtin_amdgcn_readfirstlane(smax);
    kall = __builtin_amdgcn_readfirstlane(kall);
    const uint32_t sspan = smax - smin;
    const int sspan_bits = sspan ? 32 - __clz(sspan) : 0;
    int sshift = sspan_bits > 11 ? sspan_bits - 11 : 0;
    if ((sspan >> sshift) > (uint32_t)(kBins - 3)) ++sshift;
    const uint32_t slo = smin - (1u << sshift), stop = smax + (1u << sshift) - slo;
    const uint32_t sinf = stop >> sshift;
    atomicAdd(&sh.hist[min(__builtin_elementwise_sub_sat(sa, slo), stop) >> sshift], 1u);
    atomicAdd(&sh.hist[min(__builtin_elementwise_sub_sat(sb, slo), stop) >> sshift], 1u);
    __syncthreads();
    // r = k/16 plus three standard deviations of the sample's count (a margin:
    // the bare v_sqrt_f32 serves, not the correctly rounded sqrtf sequence)
    const float kq = (float)k * (1.0f / 16.0f);
    const uint32_t r = min((uint32_t)(2 * THREADS), (uint32_t)(kq + 3.0f * __builtin_amdgcn_sqrtf(kq)) + 1u);
    uint32_t sab, scnt;
    const uint32_t sbin = (uint32_t)find_bin<THREADS>(sh, r, &sab, &scnt);
    const uint32_t theta = sbin == 0u ? kPosInf : (sbin >= sinf ? kPosInf : slo + (sbin << sshift));
    // (theta >= the sample's smallest finite key, so it is the key of a value:
    // a float compare with that value counts the elements whose key is >= theta)
    const float thf = key_float(theta);
    uint32_t wn = 0u;
#pragma unroll
    for (int j = 0; j < kTopkSteps; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) wn += (uint32_t)__popcll(__ballot(__uint_as_float(key[j][e]) >= thf));
    if (lane == 0) sh.wcnt[wave][0] = wn;
    __syncthreads();
    uint32_t p, tot;
    wave_sums<W>(sh.wcnt, 0, wave, &p, &tot);
    if (sbin != 0u && tot >= (uint32_t)k && tot <= (uint32_t)kList) {   // uniform
      write_list_raw(theta, p);
      __syncthreads();
      for (uint32_t i = tid; i < tot; i += THREADS) sh.list[2 * i + 1] = value_key(sh.list[2 * i + 1]);
      __syncthreads();
      const uint32_t span = kall - theta;
      if constexpr (NEST) {
        if (nest) {   // (kall >= every list key: the width covers both selections)
          refine_dual(theta, span ? 32 - __clz(span) : 0, tot);
          return;
        }
      }
      refine_output(theta, 0u, span ? 32 - __clz(span) : 0, (uint32_t)k, tot, out, n_kept, k);
      return;
    }
  }


  if (kRaw) {   // the sample gave no bound: the row's keys, in place
#pragma unroll
    for (int j = 0; j < kTopkSteps; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) key[j][e] = raw_key(key[j][e]);
  }

  // ---- 1a. finite extremes of the row ----
  // y = key + 2^23 sends +inf to 0 (below every finite key); z = key - 2^23 - 1
  // sends -inf, the empty slots and +inf above every finite key, so plain
  // max / min ignore the non-finite keys
  uint32_t ymax = 0u, zmin = 0xffffffffu;
  for (int c = 0; c < nchunks; ++c) {
    if (nchunks > 1) load_chunk(c);
#pragma unroll
    for (int j = 0; j < kTopkSteps; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ymax = max(ymax, key[j][e] + 0x00800000u);
        zmin = min(zmin, key[j][e] - 0x00800001u);
      }
  }
  ymax = wave_max(ymax);
  zmin = wave_min(zmin);
  if (lane == 0) {
    sh.wred[wave][0] = zmin;
    sh.wred[wave][1] = ymax;
  }
  if (tid == 0) sh.bcast[2] = 0u;   // register path: candidate list length
  __syncthreads();
  zmin = wave_combine<W>(sh.wred, 0, 0xffffffffu, min_u);
  ymax = wave_combine<W>(sh.wred, 1, 0u, max_u);
  uint32_t kmin = 0x80000000u, kmax = 0x80000000u;   // no finite key: any finite stand-in
  if (zmin <= 0xfefffffeu) {
    kmin = zmin + 0x00800001u;
    kmax = ymax - 0x00800000u;
  }
  kmin = __builtin_amdgcn_readfirstlane(kmin);
  kmax = __builtin_amdgcn_readfirstlane(kmax);
  const uint32_t span = kmax - kmin;
  const int span_bits = span ? 32 - __clz(span) : 0;
  int shift = span_bits > 11 ? span_bits - 11 : 0;
  if ((span >> shift) > (uint32_t)(kBins - 3)) ++shift;   // finite digits fit in 0..2045
  // digit: -inf and the empty slots -> 0, finite x -> 1 + ((x - kmin) >> shift),
  // +inf -> one above the largest finite digit; monotone in x
  const uint32_t lo = kmin - (1u << shift), hi = kmax + (1u << shift);
  const uint32_t top = hi - lo;
  auto digit0 = [&](uint32_t x) -> uint32_t {
    return min(__builtin_elementwise_sub_sat(x, lo), top) >> shift;
  };
  const uint32_t inf_digit = top >> shift;

  // ---- 1b. pass 0: histogram of the digits ----
  for (int b = tid; b < kBins; b += THREADS) sh.hist[b] = 0u;
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    if (nchunks > 1) load_chunk(c);
#pragma unroll
    for (int j = 0; j < kTopkSteps; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) atomicAdd(&sh.hist[digit0(key[j][e])], 1u);
  }
  __syncthreads();
  uint32_t above, bin_count;
  const uint32_t bin = (uint32_t)find_bin<THREADS>(sh, (uint32_t)k, &above, &bin_count);
  uint32_t need = (uint32_t)k - above;
  bool known = true;
  uint32_t K = 0u;
  if (bin == 0u) {
    K = kNegInf;
  } else if (bin >= inf_digit) {
    K = kPosInf;
  } else if (shift == 0) {
    K = kmin + (bin - 1u);
  } else {
    known = false;
  }
  // every kept key is >= floor_key; above + bin_count elements reach it (an
  // upper bound in the -inf bin, which also counts the empty slots)
  const uint32_t floor_key = known ? K : lo + (bin << shift);

  if (above + bin_count <= (uint32_t)kList) {
    // ---- 2. list of the elements >= floor_key, in index order ----
    uint32_t m = 0u;
    for (int c = 0; c < nchunks; ++c) {
      if (nchunks > 1) load_chunk(c);
      uint32_t wn = 0u;
#pragma unroll
      for (int j = 0; j < kTopkSteps; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) wn += (uint32_t)__popcll(__ballot(key[j][e] >= floor_key));
      if (lane == 0) sh.wcnt[wave][0] = wn;
      __syncthreads();
      uint32_t p, tot;
      wave_sums<W>(sh.wcnt, 0, wave, &p, &tot);
      p += m;
      write_list(c, floor_key, p);
      m += tot;
      __syncthreads();
    }
    m = min(m, (uint32_t)kList);
    if (known)
      refine_output(K, 0u, 0, need, m, out, n_kept, k);
    else
      refine_output(kmin, (bin - 1u) << shift, shift, need, m, out, n_kept, k);
    if (nest) nested_output(floor_key, m);
    return;
  }

  // ==== register path: the list would not fit ====
  if (!known) {
    // ---- the chosen bin's keys: refine their low `shift` bits ----
    // (an opaque copy of the digit bounds keeps the compiler from holding
    // every element's digit from pass 0 in registers until here)
    uint32_t lo_c = __builtin_amdgcn_readfirstlane(lo), top_c = __builtin_amdgcn_readfirstlane(top);
    asm volatile("" : "+s"(lo_c), "+s"(top_c));
    auto digit0c = [&](uint32_t x) -> uint32_t {
      return min(__builtin_elementwise_sub_sat(x, lo_c), top_c) >> shift;
    };
    for (int c = 0; c < nchunks; ++c) {
      if (nchunks > 1) load_chunk(c);
      // per-lane hit count, one LDS atomic per wave, then in-order slots
      uint32_t mine = 0u;
#pragma unroll
      for (int j = 0; j < kTopkSteps; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) mine += digit0c(key[j][e]) == bin ? 1u : 0u;
      const uint32_t x = wave_incl_scan(mine);
      const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
      if (wtot != 0u) {
        uint32_t base = 0u;
        if (lane == 0) base = atomicAdd(&sh.bcast[2], wtot);
        base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
        uint32_t pre = base + x - mine;
#pragma unroll
        for (int j = 0; j < kTopkSteps; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (digit0c(key[j][e]) == bin) {
              if (pre < kCand) sh.cand[pre] = key[j][e] - kmin;
              ++pre;
            }
          }
      }
    }
    __syncthreads();
    const uint32_t m = sh.bcast[2];
    const bool in_lds = m <= kCand;
    uint32_t fixed = (bin - 1u) << shift;     // known bits of (key - kmin)
    int low = shift;                          // bits below `low` still unknown
    while (low > 0) {
      const int width = low < 11 ? low : 11;
      const int sh_lo = low - width;
      const uint32_t hi_mask = ~((1u << low) - 1u);
      for (int b = tid; b < kBins; b += THREADS) sh.hist[b] = 0u;
      __syncthreads();
      if (in_lds) {
        for (uint32_t i = tid; i < m; i += THREADS) {
          const uint32_t r = sh.cand[i];
          if ((r & hi_mask) == fixed) atomicAdd(&sh.hist[(r >> sh_lo) & ((1u << width) - 1u)], 1u);
        }
      } else {
        // (an opaque copy of kmin keeps key - kmin from being hoisted out of
        // the refine loop: 32 more live registers)
        uint32_t kmin_c = kmin;
        asm volatile("" : "+s"(kmin_c));
        for (int c = 0; c < nchunks; ++c) {
          if (nchunks > 1) load_chunk(c);
#pragma unroll
          for (int j = 0; j < kTopkSteps; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t x = key[j][e];
              const uint32_t r = x - kmin_c;
              if (digit0c(x) == bin && (r & hi_mask) == fixed)
                atomicAdd(&sh.hist[(r >> sh_lo) & ((1u << width) - 1u)], 1u);
            }
        }
      }
      __syncthreads();
      uint32_t ab, cnt;
      const uint32_t d = (uint32_t)find_bin<THREADS>(sh, need, &ab, &cnt);
      need -= ab;
      fixed |= d << sh_lo;
      low = sh_lo;
    }
    K = kmin + fixed;
  }

  // ---- ordered compaction over the registers ----
  uint32_t gt_run = 0u, eq_run = 0u;   // block-wide, over previous chunks
  for (int c = 0; c < nchunks; ++c) {
    if (nchunks > 1) load_chunk(c);
    uint32_t gt = 0u, eq = 0u;
#pragma unroll
    for (int j = 0; j < kTopkSteps; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gt += (uint32_t)__popcll(__ballot(key[j][e] > K));
        eq += (uint32_t)__popcll(__ballot(key[j][e] == K));
      }
    }
    if (lane == 0) {
      sh.wcnt[wave][0] = gt;
      sh.wcnt[wave][1] = eq;
    }
    __syncthreads();
    uint32_t gbefore, ebefore, gtot, etot;
    wave_sums<W>(sh.wcnt, 0, wave, &gbefore, &gtot);
    wave_sums<W>(sh.wcnt, 1, wave, &ebefore, &etot);
    gbefore += gt_run;
    ebefore += eq_run;
    // an opaque copy of K keeps the counting ballots above from being reused
    // (and all held live) here
    uint32_t Kc = __builtin_amdgcn_readfirstlane(K);
    asm volatile("" : "+s"(Kc));
#pragma unroll
    for (int j = 0; j < kTopkSteps; ++j) {
      uint64_t G[4], Q[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        G[e] = __ballot(key[j][e] > Kc);
        Q[e] = __ballot(key[j][e] == Kc);
      }
      if (((G[0] | G[1] | G[2] | G[3]) | (Q[0] | Q[1] | Q[2] | Q[3])) != 0u) {
        uint32_t gpre = gbefore, qpre = ebefore;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gpre += lanes_below(G[e]);
          qpre += lanes_below(Q[e]);
        }
        const int ib = c * kChunk + ebase + 256 * j;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool g = key[j][e] > Kc, q = key[j][e] == Kc;
          if (g || (q && qpre < need)) {
            const uint32_t slot = gpre + min(qpre, need);
            out[slot] = map_index<MODE>(blk, ib + e) + off;
            // (nested selection: the kept entries, in index order, as a list)
            if (nest) *reinterpret_cast<uint2*>(&sh.list[2 * slot]) = make_uint2((uint32_t)(ib + e), key[j][e]);
          }
          gpre += g ? 1u : 0u;
          qpre += q ? 1u : 0u;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gbefore += (uint32_t)__popcll(G[e]);
          ebefore += (uint32_t)__popcll(Q[e]);
        }
      }
    }
    gt_run += gtot;
    eq_run += etot;
    __syncthreads();
  }
  if (MODE == MODE_KEYS && tid == 0) n_kept[row] = k;
  if (nest) nested_output(K, (uint32_t)k);   // the list holds the k kept entries
}

template <int MODE, int THREADS, bool RESIDENT, bool BF16, bool NEST>
static void launch_sized(const TopkArgs& a, int rows, bool vec, hipStream_t st) {
  if (vec)
    hipLaunchKernelGGL((topk_kernel<MODE, true, THREADS, RESIDENT, BF16, NEST>), dim3(rows), dim3(THREADS), 0, st, a);
  else
    hipLaunchKernelGGL((topk_kernel<MODE, false, THREADS, RESIDENT, BF16, NEST>), dim3(rows), dim3(THREADS), 0, st, a);
}

// the workgroup size is chosen from the widest row the call can see
template <int MODE, bool BF16, bool NEST = false>
static void launch_mode(const TopkArgs& a, int rows, int64_t width, bool vec, hipStream_t st) {
  if (width <= 4 * kWaveSlice)
    launch_sized<MODE, 256, true, BF16, NEST>(a, rows, vec, st);
  else if (width <= 8 * kWaveSlice)
    launch_sized<MODE, 512, true, BF16, NEST>(a, rows, vec, st);
  else if (width <= 16 * kWaveSlice)
    launch_sized<MODE, 1024, true, BF16, NEST>(a, rows, vec, st);
  else
    launch_sized<MODE, 1024, false, BF16, NEST>(a, rows, vec, st);
}

hipError_t launch_topk(int mode, const void* X, bool bf16, int64_t ld, const int32_t* nvalid,
                       const int32_t* len_for_blocks, int rows, int k, int64_t max_cols,
                       const int32_t* blocks, int kb, const int32_t* pos_offset, int32_t* out,
                       int32_t* n_kept, int k2, int32_t* out2, int32_t* n_kept2, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  TopkArgs a{X, ld, nvalid, len_for_blocks, k, blocks, kb, pos_offset, out, n_kept, k2, out2, n_kept2};
  // a nested selection keeps the k first-selection entries as an LDS list of
  // 4 * THREADS entries: at least k / 4 threads
  if (mode == MODE_KEYS && k2 > 0) max_cols = max(max_cols, (int64_t)8 * k);
  // vector loads (4 elements) need rows aligned to them
  const size_t vbytes = bf16 ? 8 : 16;
  const bool vec = (ld % 4 == 0) && (reinterpret_cast<uintptr_t>(X) % vbytes == 0);
  if (bf16) {
    switch (mode) {
      case MODE_IDENTITY: launch_mode<MODE_IDENTITY, true>(a, rows, max_cols, vec, st); break;
      case MODE_BLOCKMAP: launch_mode<MODE_BLOCKMAP, true>(a, rows, max_cols, vec, st); break;
      case MODE_GATHER: launch_mode<MODE_GATHER, true>(a, rows, max_cols, vec, st); break;
      default: return hipErrorInvalidValue;   // block keys are fp32
    }
  } else {
    switch (mode) {
      case MODE_IDENTITY: launch_mode<MODE_IDENTITY, false>(a, rows, max_cols, vec, st); break;
      case MODE_BLOCKMAP: launch_mode<MODE_BLOCKMAP, false>(a, rows, max_cols, vec, st); break;
      case MODE_GATHER: launch_mode<MODE_GATHER, false>(a, rows, max_cols, vec, st); break;
      default:
        if (k2 > 0)
          launch_mode<MODE_KEYS, false, true>(a, rows, max_cols, vec, st);
        else
          launch_mode<MODE_KEYS, false>(a, rows, max_cols, vec, st);
        break;
    }
  }
  return hipGetLastError();
}

}  // namespace idxk
