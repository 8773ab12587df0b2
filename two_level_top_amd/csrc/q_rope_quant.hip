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

// nearest bf16 (ties to even), as fp32; finite inputs
__device__ __forceinline__ float round_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint32_t e2m1_code(float a) {   // a >= 0
  if (a <= 0.25f) return 0u;
  if (a < 0.75f) return 1u;
  if (a <= 1.25f) return 2u;
  if (a < 1.75f) return 3u;
  if (a <= 2.5f) return 4u;
  if (a < 3.5f) return 5u;
  if (a <= 5.0f) return 6u;
  return 7u;
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
  uint32_t am = 0u;
#pragma unroll
  for (int k = 0; k < 8; ++k) am = max(am, __float_as_uint(x[k]) & 0x7fffffffu);
  am = max(am, dpp_u<0xB1>(am));   // quad_perm [1,0,3,2]
  am = max(am, dpp_u<0x4E>(am));   // quad_perm [2,3,0,1]
  const float raw_scale = fmaxf(__uint_as_float(am), 1e-10f) * (1.0f / 6.0f);
  const uint32_t rb = __float_as_uint(raw_scale);          // a positive normal value
  e = (int)((rb >> 23) & 0xffu) - 127 + ((rb & 0x7fffffu) != 0u ? 1 : 0);   // ceil(log2)
  codes = 0u;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float y = ldexpf(x[k], -e);   // exact: power-of-two scale
    uint32_t c = e2m1_code(fabsf(y));
    if (y < 0.f && c != 0u) c |= 8u;
    codes |= c << (4 * k);
  }
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
  // this lane's angles: NeoX pairs i = 8 (j % 4) + k, interleaved i = 4j + m
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
      if (j < 4) {
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = round_bf16(x[k] * c[k] - other[k] * s[k]);   // r0
      } else if (j < 8) {
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = round_bf16(x[k] * c[k] + other[k] * s[k]);   // r1
      }
    } else if (j < 8) {
      // pairs (2i, 2i + 1): lane j holds i = 4j .. 4j+3
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float x0 = x[2 * m], x1 = x[2 * m + 1];
        x[2 * m] = round_bf16(x0 * c[m] - x1 * s[m]);
        x[2 * m + 1] = round_bf16(x1 * c[m] + x0 * s[m]);
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
