// MX block quantization of eight fp32 values per lane (a 32-block is a lane
// quad), shared by the activation quantizer and the weight solver so that
// both take the same decisions (Section 3 of the DualQuant paper: nearest grid
// point, clipped; OCP microscaling shared exponent for the E8M0 scale).
#pragma once

#include "common.h"

namespace w4a4 {

// floor(log2 a) for finite a > 0 (subnormals included)
__device__ __forceinline__ int floor_log2(float a) {
  const uint32_t u = __float_as_uint(a);
  const int ef = (u >> 23) & 0xff;
  if (ef) return ef - 127;
  return (31 - __clz(u & 0x7fffffu)) - 149;
}

// value of the lane whose index differs in bit 0 / bit 1 (within a quad)
__device__ __forceinline__ float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ int quad_xor1(int v) { return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true); }
__device__ __forceinline__ int quad_xor2(int v) { return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true); }

// Codes and the scale byte of one 32-block from this lane's 8 elements (the
// block is spread over 4 consecutive lanes, which must all be present).
template <int FMT>
__device__ __forceinline__ void quant8_mx(const float (&x)[8], uint32_t& word, uint32_t& sbyte) {
  // block amax as the integer maximum of the magnitude bit patterns: for
  // finite values they order as the values do, and any Inf or NaN gives a
  // pattern above the largest finite one, so one reduction yields both
  uint32_t abits = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) abits = max(abits, __float_as_uint(x[i]) & 0x7fffffffu);
  // the 4 lanes of a block form a quad: two DPP quad permutations
  abits = max(abits, uint32_t(quad_xor1(int(abits))));
  abits = max(abits, uint32_t(quad_xor2(int(abits))));
  const bool bad = abits > 0x7f7fffffu;  // Inf or NaN in the block

  int e = -127;
  if (abits != 0) e = max(-127, min(127, floor_log2(__uint_as_float(abits)) - 2));

  word = 0;
  if (FMT == MXFP4) {
    // the hardware FP4 conversion (round to nearest even, saturating, sign
    // kept for values that round to zero) of the exactly scaled values
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, ldexpf(x[0], -e), ldexpf(x[1], -e), 1.0f, 0);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, ldexpf(x[2], -e), ldexpf(x[3], -e), 1.0f, 1);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, ldexpf(x[4], -e), ldexpf(x[5], -e), 1.0f, 2);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, ldexpf(x[6], -e), ldexpf(x[7], -e), 1.0f, 3);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q = fminf(rintf(ldexpf(x[i], -e)), 7.0f);  // |v| < 8, so only +8 needs clipping
      word |= (uint32_t(int(q)) & 15u) << (4 * i);
    }
  }
  sbyte = uint32_t(e + 127);
  if (bad) {
    word = 0;
    sbyte = 0xff;
  }
}

// The 8-bit MX variants (MXFP8: E4M3 elements, emax_elem = 8; MXINT8: int8
// elements, emax_elem = 6): codes (one byte each) and the scale byte of one
// 32-block from this lane's 8 elements, same lane-quad layout and the same
// shared-exponent rule.
template <int FMT>
__device__ __forceinline__ void quant8_mx8(const float (&x)[8], uint32_t (&word)[2], uint32_t& sbyte) {
  uint32_t abits = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) abits = max(abits, __float_as_uint(x[i]) & 0x7fffffffu);
  abits = max(abits, uint32_t(quad_xor1(int(abits))));
  abits = max(abits, uint32_t(quad_xor2(int(abits))));
  const bool bad = abits > 0x7f7fffffu;  // Inf or NaN in the block
  constexpr int EMAX = FMT == MXFP8 ? 8 : 6;
  int e = -127;
  if (abits != 0) e = max(-127, min(127, floor_log2(__uint_as_float(abits)) - EMAX));
  word[0] = word[1] = 0;
  if (FMT == MXFP8) {
    // |x 2^-e| < 512: values above 448 saturate (448 converts exactly), the
    // rest go through the hardware E4M3 conversion (nearest even, sign kept
    // for values that round to zero)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = fmaxf(fminf(ldexpf(x[4 * h + i], -e), 448.0f), -448.0f);
      int w = 0;
      w = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], w, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w, true);
      word[h] = uint32_t(w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q = fminf(rintf(ldexpf(x[i], -e)), 127.0f);  // |v| < 128: only +128 clips
      word[i >> 2] |= (uint32_t(int(q)) & 255u) << (8 * (i & 3));
    }
  }
  sbyte = uint32_t(e + 127);
  if (bad) {
    word[0] = word[1] = 0;
    sbyte = 0xff;
  }
}

}  // namespace w4a4
