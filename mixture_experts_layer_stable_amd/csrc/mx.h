// MX formats (OCP Microscaling v1.0) on gfx950: MXFP8 (FP8 E4M3 elements) and MXFP4
// (FP4 E2M1 elements), one E8M0 scale per 32 values.
//
// Block quantisation (the block's values are finite and already rounded to bf16):
//   amax = largest magnitude; s = floor(log2 amax) - 8 (8 = exponent of E4M3's
//   largest normal, 448 = 1.75 * 2^8), clamped to [-127, 127]; the scale byte is
//   s + 127 = max(exponent field of amax - 8, 0) (amax below 2^-119, including 0
//   and fp32 subnormals, gives byte 0); element = E4M3 of v * 2^-s, rounded to
//   nearest even and saturated at +-448. v * 2^-s is exact in fp32 (a power-of-two
//   scaling of a bf16 value, below 2^9 in magnitude), so the one rounding is the
//   E4M3 conversion: v_cvt_pk_fp8_f32, which rounds to nearest even with
//   subnormals; it is given values already clamped to +-448 (it does not saturate).
#pragma once
#include "common.h"

namespace mok {

__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  return (uint32_t)max(e - 8, 0);
}

// 2^-s for scale byte b (s = b - 127): exponent field 254 - b; b <= 247 for finite amax.
__device__ __forceinline__ float mx_inv_scale(uint32_t b) { return __uint_as_float((254u - b) << 23); }

__device__ __forceinline__ float mx_clamp(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// Four values -> four E4M3 bytes (little-endian in the word) of v * inv.
__device__ __forceinline__ uint32_t mx_pack4(float a, float b, float c, float d, float inv) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(mx_clamp(a * inv), mx_clamp(b * inv), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(mx_clamp(c * inv), mx_clamp(d * inv), w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ uint4 mx_pack16(const float (&v)[16], float inv) {
  return make_uint4(mx_pack4(v[0], v[1], v[2], v[3], inv), mx_pack4(v[4], v[5], v[6], v[7], inv),
                    mx_pack4(v[8], v[9], v[10], v[11], inv), mx_pack4(v[12], v[13], v[14], v[15], inv));
}

// One 32-value block held as 16 values by each lane of the pair (l, l ^ 1), the
// even lane holding the first half. Both lanes must call. Returns this lane's 16
// E4M3 bytes and the block's scale byte in *sbyte.
__device__ __forceinline__ uint4 mx_quant16_pair(const float (&v)[16], uint32_t* sbyte) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  m = fmaxf(m, __shfl_xor(m, 1));
  const uint32_t b = mx_scale_byte(m);
  *sbyte = b;
  return mx_pack16(v, mx_inv_scale(b));
}

// MXFP4 (OCP MX v1.0 FP4 E2M1 elements, same E8M0 block scale): s = floor(log2 amax) - 2
// (2 = exponent of E2M1's largest normal, 6 = 1.5 * 2^2), so the scale byte is
// max(exponent field of amax - 2, 0); elements are v * 2^-s rounded to nearest even
// onto {0, 0.5, 1, 1.5, 2, 3, 4, 6} and saturated at 6. Codes: sign bit 3, exponent
// bits 2..1, mantissa bit 0 (the magnitude's code is its index in that list), two per
// byte, the even element in the low nibble. The MFMA takes a row's 32-element block as
// 16 consecutive bytes in one lane.
__device__ __forceinline__ uint32_t mx4_scale_byte(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  return (uint32_t)max(e - 2, 0);
}

// Nearest E2M1 code of v (|v| < 8 after scaling; larger saturates): the magnitude code
// counts the midpoints below |v|, a midpoint itself going to the code with mantissa 0.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
                     (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return m | (v < 0.0f ? 8u : 0u);
}

// 16 values -> 8 bytes of E2M1 codes of v * inv.
__device__ __forceinline__ uint2 mx4_pack16(const float (&v)[16], float inv) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i >> 3] |= e2m1_code(v[i] * inv) << (4 * (i & 7));
  return make_uint2(w[0], w[1]);
}

// As mx_quant16_pair, for E2M1: this lane's 8 bytes of the pair's 32-element block.
__device__ __forceinline__ uint2 mx4_quant16_pair(const float (&v)[16], uint32_t* sbyte) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  m = fmaxf(m, __shfl_xor(m, 1));
  const uint32_t b = mx4_scale_byte(m);
  *sbyte = b;
  return mx4_pack16(v, mx_inv_scale(b));
}

// Element format of an MX GEMM path: 0 = E4M3 (MXFP8), 1 = E2M1 (MXFP4).
// KTILE: elements per 128-byte tile row (one K-tile); SD: scale dwords per row and
// K-tile (the scale arrays keep 4 bytes per 128 elements in either format).
template <int F>
struct MxFmt {
  static constexpr int BITS = F == 0 ? 8 : 4;
  static constexpr int KTILE = F == 0 ? 128 : 256;
  static constexpr int SD = KTILE / 128;
  static __device__ __forceinline__ int64_t bytes(int64_t elems) { return F == 0 ? elems : elems / 2; }
  // quantise a lane pair's 32-element block (16 values here) and store this lane's part
  // of it at element offset `elem` of q (elem a multiple of 16)
  static __device__ __forceinline__ uint32_t quant_store16(const float (&v)[16], uint8_t* q, int64_t elem) {
    uint32_t sb;
    if constexpr (F == 0) {
      stg16(q + elem, mx_quant16_pair(v, &sb));
    } else {
      const uint2 o = mx4_quant16_pair(v, &sb);
      *reinterpret_cast<uint2*>(q + elem / 2) = o;
    }
    return sb;
  }
};

// Round 16 floats to bf16 values (as floats): the stored value a quantiser sees.
__device__ __forceinline__ void round16_bf16(float (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = bf16_to_f32(f32_to_bf16(v[i]));
}

}  // namespace mok
