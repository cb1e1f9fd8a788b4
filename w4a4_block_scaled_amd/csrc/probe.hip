// Measurement aids: a plain streaming read of a buffer (what a kernel that
// reads a given number of bytes once, in one launch, can reach on this chip:
// the ceiling the weight-streaming decode GEMMs are compared with), an empty
// kernel (the cost of one launch in a HIP graph), and the scaled FP4 MFMA
// alone on register operands (what the matrix cores sustain at the clock the
// chip holds under that load: the ceiling the MXFP4 GEMMs are compared with
// beside the nominal peak).  None is part of the quantized linear.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace w4a4 {
namespace {

typedef uint32_t p_u32x4 __attribute__((ext_vector_type(4)));

// Every lane keeps four 16-byte non-temporal loads in flight (the decode
// kernels' access: each byte read once, straight from HBM) and folds them
// into an XOR; a workgroup writes its word only if it equals a value the
// data never gives in practice, so the loads cannot be dropped and nothing
// is written.
__global__ void __launch_bounds__(256) stream_read_kernel(const p_u32x4* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const p_u32x4 a = __builtin_nontemporal_load(&src[i]);
    const p_u32x4 b = __builtin_nontemporal_load(&src[i + stride]);
    const p_u32x4 c = __builtin_nontemporal_load(&src[i + 2 * stride]);
    const p_u32x4 d = __builtin_nontemporal_load(&src[i + 3 * stride]);
    x ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const p_u32x4 a = __builtin_nontemporal_load(&src[i]);
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (x == 0x9E3779B9u) sink[blockIdx.x & 255] = x;
}

__global__ void empty_kernel() {}

typedef int p_v8i __attribute__((ext_vector_type(8)));
typedef float p_v16f __attribute__((ext_vector_type(16)));

// A wave holds the 4 x 4 blocks of 32 x 32 fp32 accumulators of a 128 x 128
// output tile, as each wave of the persistent MXFP4 GEMM does, and runs
// `iters` rounds of its 16 scaled FP4 MFMAs (32 x 32 x 64, E8M0 scales 1.0),
// alternating two operand sets read once from `ops` (16 fragments of 64
// lanes x 16 bytes: weight and activation fragments of set 0, then of set
// 1), so that the operands change from round to round as a GEMM's K-steps
// do.  Nothing else runs in the loop.  The accumulators are folded into one
// value that is written only if it equals a constant the sums never reach.
__device__ __forceinline__ p_v16f probe_mfma(const p_u32x4& w, const p_u32x4& a, const p_v16f& acc) {
  const p_v8i A = {int(w.x), int(w.y), int(w.z), int(w.w), 0, 0, 0, 0};
  const p_v8i B = {int(a.x), int(a.y), int(a.z), int(a.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc, 4, 4, 0, 0x7F7F7F7F, 0, 0x7F7F7F7F);
}

__global__ void __launch_bounds__(256, 1) mfma_fp4_kernel(const p_u32x4* __restrict__ ops, int iters,
                                                          float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  p_u32x4 w0[4], a0[4], w1[4], a1[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    w0[f] = ops[f * 64 + lane];
    a0[f] = ops[(4 + f) * 64 + lane];
    w1[f] = ops[(8 + f) * 64 + lane];
    a1[f] = ops[(12 + f) * 64 + lane];
  }
  p_v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = probe_mfma(w0[i], a0[j], acc[i][j]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = probe_mfma(w1[i], a1[j], acc[i][j]);
  }
  float x = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) x += acc[i][j][e];
  if (x == 1.0e-30f) sink[blockIdx.x & 255] = x;
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, void* sink, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  int64_t blocks = (n16 + 256 * 4 - 1) / (256 * 4);
  blocks = blocks < 256 ? 256 : (blocks > 4096 ? 4096 : blocks);
  hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                     static_cast<const p_u32x4*>(src), n16, static_cast<uint32_t*>(sink));
  return hipGetLastError();
}

hipError_t launch_mfma_fp4(const void* ops, int iters, int workgroups, void* sink, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_fp4_kernel, dim3(unsigned(workgroups)), dim3(256), 0, stream,
                     static_cast<const p_u32x4*>(ops), iters, static_cast<float*>(sink));
  return hipGetLastError();
}

hipError_t launch_empty(hipStream_t stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
  return hipGetLastError();
}

}  // namespace w4a4
