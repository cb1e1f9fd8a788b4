// NVFP4 block quantization of eight fp32 values per lane (a 16-block is a
// lane pair), shared by the activation quantizer and the weight solver so
// that both take the same decisions (Section 3 of the DualQuant paper: UE4M3
// block scale, E2M1 elements, nearest grid point; the fp32 tensor scale t is
// this library's reading of the NVFP4 per-tensor scale).
#pragma once

#include <math.h>

#include "common.h"

namespace w4a4 {

__device__ __forceinline__ double e4m3_value(int code) {
  const int e = code >> 3, m = code & 7;
  return e == 0 ? ldexp(double(m), -9) : ldexp(double(8 + m), e - 10);
}

// UE4M3 code of the exact quotient a / D (a >= 0 finite fp32, D > 0), round
// to nearest even, saturating at 448 (0x7E).  A first guess from the rounded
// fp64 quotient is settled by one exact comparison against the midpoint above
// it (a and midpoint * D are exact in fp64).
__device__ __forceinline__ int e4m3_rne_ratio(float a, double D) {
  if (!(a > 0.0f)) return 0;
  const double u = double(a) / D;
  if (u >= 448.0) return 0x7e;
  int c;
  if (u < 0.015625) {
    c = int(u * 512.0);  // subnormal codes 0..7
  } else {
    const uint64_t b = uint64_t(__double_as_longlong(u));
    const int E = int((b >> 52) & 0x7ff) - 1023;  // -6 .. 8
    c = ((E + 7) << 3) | int((b >> 49) & 7);
  }
  const double thr = 0.5 * (e4m3_value(c) + e4m3_value(c + 1)) * D;
  const double ad = double(a);
  if (ad > thr) return c + 1;
  if (ad == thr) return ((c + 1) & 1) ? c : c + 1;
  return c;
}

// Smallest fp32 >= T (T >= 0, exact double).  With strict = true: smallest
// fp32 > T.  Turns "|x| > T" / "|x| >= T" for fp32 |x| into "|x| >= result".
__device__ __forceinline__ float f32_threshold(double T, bool strict) {
  float f = float(T);
  if (double(f) < T || (strict && double(f) == T)) f = nextafterf(f, INFINITY);
  return f;
}

// Codes and the UE4M3 scale code of one 16-block from this lane's 8 elements
// (the block is spread over 2 consecutive lanes, which must both be present),
// for the fp32 tensor scale t: s = RNE_E4M3(amax / (6 t)), saturating; codes
// RNE_E2M1(x / (s t)) decided against exact midpoints; a block whose scale
// rounds to 0 keeps only the signs.
__device__ __forceinline__ void quant8_nv(const float (&x)[8], float t, uint32_t& word, int& s) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  s = e4m3_rne_ratio(amax, 6.0 * double(t));  // 6 t is exact in fp64
  word = 0;
  if (s == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= ((__float_as_uint(x[i]) >> 28) & 8u) << (4 * i);
    return;
  }
  const double unit = e4m3_value(s) * double(t);  // exact: 4 + 24 significant bits
  const float t0 = f32_threshold(0.25 * unit, true);
  const float t1 = f32_threshold(0.75 * unit, false);
  const float t2 = f32_threshold(1.25 * unit, true);
  const float t3 = f32_threshold(1.75 * unit, false);
  const float t4 = f32_threshold(2.5 * unit, true);
  const float t5 = f32_threshold(3.5 * unit, false);
  const float t6 = f32_threshold(5.0 * unit, true);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = fabsf(x[i]);
    const uint32_t idx = (a >= t0) + (a >= t1) + (a >= t2) + (a >= t3) + (a >= t4) +
                         (a >= t5) + (a >= t6);
    word |= (idx | ((__float_as_uint(x[i]) >> 28) & 8u)) << (4 * i);
  }
}

}  // namespace w4a4
