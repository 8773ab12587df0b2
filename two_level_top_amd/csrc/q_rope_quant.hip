// idx_q_rope_quant: the step before the index layers' score calls -- RoPE on
// the first 64 dimensions of each head's projected query, MXFP4 quantisation
// of the 128-dimension result, and the head-weight scaling (the vLLM indexer
// page, rope_quant_q and fused_indexer_q_rope_quant; the fp4 path keeps the
// query scales with the query instead of folding them into the weights).
//
//   r0 = bf16(x0 cos - x1 sin), r1 = bf16(x1 cos + x0 sin) over the pairs
//   (i, i + 32) (NeoX) or (2i, 2i + 1) (interleaved) of dimensions 0..63;
//   dimensions 64..127 pass through; per 32-element group the ue8m0 scale
//   2^ceil(log2(max(amax, 1e-10) * (1/6))) and the e2m1 code of each
//   element / scale (nearest, ties to the even code, saturated at 6);
//   w_out = w * softmax_scale * head_scale.
// Products and sums are separate fp32 roundings (no fused multiply-add), so
// the bytes are a deterministic function of the inputs.
//
// Layout: one workgroup per (row, 64 heads); 16 lanes per head, lane j owning dimensions 8j .. 8j+7 (one
// 16-byte load of 8 bf16, one 4-byte store of 8 codes); a 32-element scale
// group is an aligned quad of lanes.  In the NeoX layout lane j < 4 holds x0
// and lane j + 4 the matching x1, exchanged with one lane swizzle (xor 4).
// Memory-bound: 256 bytes read and 72 bytes written per (row, head).
#include "idx_internal.h"

// every product and sum in this file is rounded on its own (hipcc contracts
// a * b +- c * d into fused multiply-adds by default)
#pragma clang fp contract(off)

namespace idxk {

constexpr int kRqPerLane = 4;                  // heads per 16-lane group
constexpr int kRqHeadsPerWG = 16 * kRqPerLane;   // heads per 256-thread workgroup

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// nearest bf16 (ties to even) of two fp32 values, as fp32: one
// v_cvt_pk_bf16_f32 (which rounds finite values, subnormals and ties exactly
// as (u + 0x7fff + ((u >> 16) & 1)) >> 16 does) and two unpacks
__device__ __forceinline__ void round2_bf16(float& a, float& b) {
  const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)a);
  const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)b);
  a = __uint_as_float(lo << 16);
  b = __uint_as_float(hi << 16);
}

// gfx950's v_cvt_scalef32_pk_fp4_f32 writes byte SEL of `old` with the e2m1
// codes of a / scale (low nibble) and b / scale: nearest, ties to the even
// code, saturated at 6 (checked against the rule above over a sweep of
// values, ties, subnormals and values past 6 at several scales).  It writes
// a negative value that rounds to zero as code 8 (-0); the caller maps those
// to 0.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t old, float a, float b, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
}

__device__ __forceinline__ float swizzle_xor4(float v) {
  // ds_swizzle bit mode: and_mask 0x1f, or_mask 0, xor_mask 4
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101f));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, true);
}

// quantise 8 values (dims 8j .. 8j+7) of one head; lanes of an aligned quad
// share a 32-element group
__device__ __forceinline__ void quantize8(const float (&x)[8], uint32_t& codes, int& e) {
  // |x| maximum of the 8 values: v_max3_f32 with |.| source modifiers (finite
  // inputs: the bit pattern of the largest magnitude), written out because
  // the compiler would canonicalize every operand of fmaxf first
  uint32_t am;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|\n\t"
      "v_max3_f32 %0, %0, |%4|, |%5|\n\t"
      "v_max3_f32 %0, %0, |%6|, |%7|\n\t"
      "v_max3_f32 %0, %0, |%8|, %0\n\t"
      "s_nop 1"   // VALU write -> the DPP reads of am below
      : "=&v"(am)
      : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]));
  am = max(am, dpp_u<0xB1>(am));   // quad_perm [1,0,3,2]
  am = max(am, dpp_u<0x4E>(am));   // quad_perm [2,3,0,1]
  const float raw_scale = fmaxf(__uint_as_float(am), 1e-10f) * (1.0f / 6.0f);
  const uint32_t rb = __float_as_uint(raw_scale);          // a positive normal value
  e = (int)((rb >> 23) & 0xffu) - 127 + ((rb & 0x7fffffu) != 0u ? 1 : 0);   // ceil(log2)
  // e lies in [-35, 126] (amax is at least 1e-10 and finite), so 2^e is a
  // normal fp32 value and x / 2^e is exact
  const float scale = __uint_as_float((uint32_t)(e + 127) << 23);
  uint32_t w = 0u;
  w = cvt_fp4x2<0>(w, x[0], x[1], scale);
  w = cvt_fp4x2<1>(w, x[2], x[3], scale);
  w = cvt_fp4x2<2>(w, x[4], x[5], scale);
  w = cvt_fp4x2<3>(w, x[6], x[7], scale);
  // -0 (code 8) -> code 0: keep a nibble's sign bit only where its magnitude
  // is nonzero (magnitude + 7 carries into bit 3 exactly then; no nibble
  // carries into the next)
  const uint32_t mag = w & 0x77777777u;
  codes = mag | (w & ((mag + 0x77777777u) & 0x88888888u));
}

// One workgroup per (row, 64 heads): 16 lanes per head, each 16-lane group
// taking heads g, g + 16, g + 32, g + 48 with all four loads issued first; the
// row's rotary angles are loaded once per lane.
template <bool NEOX>
__global__ __launch_bounds__(256) void q_rope_quant_kernel(const uint16_t* __restrict__ q,
                                                           const int32_t* __restrict__ positions,
                                                           const float* __restrict__ cos_sin,
                                                           int max_pos, const float* __restrict__ w,
                                                           int heads, float softmax_scale,
                                                           float head_scale, uint8_t* __restrict__ vals,
                                                           uint8_t* __restrict__ scales,
                                                           float* __restrict__ w_out) {
  const int hgroups = (heads + kRqHeadsPerWG - 1) / kRqHeadsPerWG;
  const int row = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / (unsigned)hgroups));
  const int h0 = (int)(blockIdx.x % (unsigned)hgroups) * kRqHeadsPerWG + (int)(threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  const int pos = min(max(positions[row], 0), max_pos - 1);
  const float* cs = cos_sin + (int64_t)pos * 64;
  const int64_t rbase = (int64_t)row * heads;

  uint4 raw[kRqPerLane];
#pragma unroll
  for (int t = 0; t < kRqPerLane; ++t) {
    const int h = min(h0 + 16 * t, heads - 1);   // past the last head: a copy, never stored
    raw[t] = *reinterpret_cast<const uint4*>(q + (rbase + h) * kDim + 8 * j);
  }
  // this lane's angles: NeoX pairs i = 8 (j % 4) + k, interleaved i = 4j + m.
  // In the NeoX layout lane j < 4 computes r0 = x0 cos - x1 sin as
  // x0 cos + x1 (-sin) (the same rounded products and sum), so that both
  // halves of the pair run one code path.
  float c[8], s[8];
  if (j < 8) {
    const int i0 = NEOX ? 8 * (j & 3) : 4 * j;
    const float4 c0 = *reinterpret_cast<const float4*>(cs + i0);
    const float4 s0 = *reinterpret_cast<const float4*>(cs + 32 + i0);
    c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
    s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
    if (NEOX) {
      const float4 c1 = *reinterpret_cast<const float4*>(cs + i0 + 4);
      const float4 s1 = *reinterpret_cast<const float4*>(cs + 32 + i0 + 4);
      c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
      s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
      if (j < 4) {
#pragma unroll
        for (int k = 0; k < 8; ++k) s[k] = -s[k];
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kRqPerLane; ++t) {
    const int h_raw = h0 + 16 * t;
    float x[8];
    const uint32_t rw[4] = {raw[t].x, raw[t].y, raw[t].z, raw[t].w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      x[2 * m] = bf16_bits_to_f32(rw[m] & 0xffffu);
      x[2 * m + 1] = bf16_bits_to_f32(rw[m] >> 16);
    }
    if (NEOX) {
      // pairs (i, i + 32): lane j < 4 holds x0 of i = 8j + k, lane j + 4 its x1
      float other[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) other[k] = swizzle_xor4(x[k]);
      if (j < 8) {   // r0 (j < 4, sines negated above) or r1
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = x[k] * c[k] + other[k] * s[k];
#pragma unroll
        for (int k = 0; k < 8; k += 2) round2_bf16(x[k], x[k + 1]);
      }
    } else if (j < 8) {
      // pairs (2i, 2i + 1): lane j holds i = 4j .. 4j+3
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float x0 = x[2 * m], x1 = x[2 * m + 1];
        x[2 * m] = x0 * c[m] - x1 * s[m];
        x[2 * m + 1] = x1 * c[m] + x0 * s[m];
        round2_bf16(x[2 * m], x[2 * m + 1]);
      }
    }
    uint32_t codes;
    int e;
    quantize8(x, codes, e);
    if (h_raw < heads) {
      const int64_t item = rbase + h_raw;
      *reinterpret_cast<uint32_t*>(vals + item * kValBytes + 4 * j) = codes;
      if ((j & 3) == 0) scales[item * kScaleBytes + (j >> 2)] = (uint8_t)(e + 127);
      if (j == 0) w_out[item] = (w[item] * softmax_scale) * head_scale;
    }
  }
}

hipError_t launch_q_rope_quant(const uint16_t* q, const int32_t* positions, const float* cos_sin,
                               int max_pos, const float* w, int rows, int heads, bool neox,
                               float softmax_scale, float head_scale, uint8_t* vals,
                               uint8_t* scales, float* w_out, hipStream_t st) {
  if (rows <= 0 || heads <= 0) return hipSuccess;
  const int64_t grid = (int64_t)rows * ((heads + kRqHeadsPerWG - 1) / kRqHeadsPerWG);
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (neox)
    hipLaunchKernelGGL(q_rope_quant_kernel<true>, dim3((unsigned)grid), dim3(256), 0, st, q, positions,
                       cos_sin, max_pos, w, heads, softmax_scale, head_scale, vals, scales, w_out);
  else
    hipLaunchKernelGGL(q_rope_quant_kernel<false>, dim3((unsigned)grid), dim3(256), 0, st, q, positions,
                       cos_sin, max_pos, w, heads, softmax_scale, head_scale, vals, scales, w_out);
  return hipGetLastError();
}

}  // namespace idxk
