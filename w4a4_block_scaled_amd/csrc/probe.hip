// Measurement aids for the decode roofline: a plain streaming read of a
// buffer (what a kernel that reads a given number of bytes once, in one
// launch, can reach on this chip: the ceiling the weight-streaming decode
// GEMMs are compared with) and an empty kernel (the cost of one launch in a
// HIP graph).  Neither is part of the quantized linear.
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

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, void* sink, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  int64_t blocks = (n16 + 256 * 4 - 1) / (256 * 4);
  blocks = blocks < 256 ? 256 : (blocks > 4096 ? 4096 : blocks);
  hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                     static_cast<const p_u32x4*>(src), n16, static_cast<uint32_t*>(sink));
  return hipGetLastError();
}

hipError_t launch_empty(hipStream_t stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
  return hipGetLastError();
}

}  // namespace w4a4
