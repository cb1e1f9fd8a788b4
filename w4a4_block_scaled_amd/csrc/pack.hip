// Offline packing of a quantized weight into the gfx950 GEMM layout.
//
// DualQuant Appendix I: quantized weights and their scales are packed
// offline into the GEMM backend's storage layout and stay packed during
// inference.  The layout chosen here follows the operand order of the
// 16x16x128 scaled MFMA: one 1 KiB tile per (16 output rows, 128 K), lane l
// owning 16 bytes of row l%16 (for FP4 the canonical bytes of K chunk l/16;
// for MXINT4 two 8-byte halves, see unit_dest).  A wave loads a
// tile with one coalesced 16-byte load per lane.  The block scales are
// regrouped per K-step so that one dword per lane carries the scale bytes of
// several 16-row groups (picked by the MFMA's byte select).
#include <string.h>

#include "common.h"
#include "kernels.h"

namespace w4a4 {
namespace {

constexpr int kThreads = 256;

// Destination of 8-byte unit u (16 codes) of a canonical row inside the
// fragment tiles, as (K-step, lane group, byte offset in the lane's 16 bytes).
// FP4 operands: lane group c holds block c of the K-step (bytes 16c..16c+15).
// MXINT4 (widened to FP8 in the GEMM): with FP8 operands the 16x16x128 MFMA
// takes K 16c..16c+15 from lane group c's first four dwords and K
// 64+16c..64+16c+15 from its last four, while the scale of block b still comes
// from lane group b.  So lane group c carries half (c & 1) of block (c >> 1)
// in bytes 0..7 and the same half of block 2 + (c >> 1) in bytes 8..15.
__device__ __forceinline__ void unit_dest(int fmt, int64_t u, int64_t* ks, int* c, int* off) {
  *ks = u >> 3;
  const int v = int(u & 7);
  const int b = v >> 1, hb = v & 1;
  if (fmt == MXINT4) {
    *c = 2 * (b & 1) + hb;
    *off = 8 * (b >> 1);
  } else {
    *c = b;
    *off = 8 * hb;
  }
}

__global__ __launch_bounds__(kThreads) void pack_codes_kernel(int fmt, const uint2* __restrict__ src,
                                                              uint2* __restrict__ dst,
                                                              int64_t n_units, int64_t K16,
                                                              int64_t KS) {
  const int64_t q = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (q >= n_units) return;
  const int64_t n = q / K16, u = q - n * K16;
  int64_t ks;
  int c, off;
  unit_dest(fmt, u, &ks, &c, &off);
  const int lane = int(n & 15) + 16 * c;
  dst[(((n >> 4) * KS + ks) * 64 + lane) * 2 + (off >> 3)] = src[q];
}

__global__ __launch_bounds__(kThreads) void unpack_codes_kernel(int fmt,
                                                                const uint2* __restrict__ src,
                                                                uint2* __restrict__ dst,
                                                                int64_t n_units, int64_t K16,
                                                                int64_t KS) {
  const int64_t q = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (q >= n_units) return;
  const int64_t n = q / K16, u = q - n * K16;
  int64_t ks;
  int c, off;
  unit_dest(fmt, u, &ks, &c, &off);
  const int lane = int(n & 15) + 16 * c;
  dst[q] = src[(((n >> 4) * KS + ks) * 64 + lane) * 2 + (off >> 3)];
}

// Canonical scale byte index for byte b of scale word (sg, ks, lane);
// *valid is false for bytes of row groups beyond N/16.
__device__ __forceinline__ int64_t scale_src(int fmt, int64_t sg, int64_t ks, int lane, int b,
                                             int64_t NG, int64_t KB, bool* valid) {
  const int cgrp = lane >> 4;
  int64_t ng, blk;
  if (fmt == NVFP4) {
    ng = sg * 2 + (b >> 1);
    blk = ks * 8 + 2 * cgrp + (b & 1);
  } else {
    ng = sg * 4 + b;
    blk = ks * 4 + cgrp;
  }
  *valid = ng < NG;
  return (ng * 16 + (lane & 15)) * KB + blk;
}

__global__ __launch_bounds__(kThreads) void pack_scales_kernel(
    int fmt, const uint8_t* __restrict__ src, uint32_t* __restrict__ dst, int64_t total,
    int64_t KS, int64_t NG, int64_t KB) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= total) return;
  const int lane = int(i & 63);
  const int64_t t = i >> 6;
  const int64_t sg = t / KS, ks = t - sg * KS;
  uint32_t w = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    bool valid;
    const int64_t s = scale_src(fmt, sg, ks, lane, b, NG, KB, &valid);
    if (valid) w |= uint32_t(src[s]) << (8 * b);
  }
  dst[i] = w;
}

__global__ __launch_bounds__(kThreads) void unpack_scales_kernel(
    int fmt, const uint32_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t total,
    int64_t KS, int64_t NG, int64_t KB) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= total) return;
  const int lane = int(i & 63);
  const int64_t t = i >> 6;
  const int64_t sg = t / KS, ks = t - sg * KS;
  const uint32_t w = src[i];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    bool valid;
    const int64_t s = scale_src(fmt, sg, ks, lane, b, NG, KB, &valid);
    if (valid) dst[s] = uint8_t(w >> (8 * b));
  }
}

__global__ __launch_bounds__(kThreads) void pack_tail_kernel(int fmt, int64_t N, int64_t K,
                                                             const float* __restrict__ t_w,
                                                             const float* __restrict__ r,
                                                             uint8_t* __restrict__ blob) {
  const BlobLayout L = blob_layout(fmt, N, K);
  float* rd = reinterpret_cast<float*>(blob + L.r_off);
  for (int64_t n = int64_t(blockIdx.x) * kThreads + threadIdx.x; n < N;
       n += int64_t(gridDim.x) * kThreads)
    rd[n] = r[n];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    BlobHeader* h = reinterpret_cast<BlobHeader*>(blob);
    const char magic[8] = {'W', '4', 'A', '4', 'P', 'K', '0', '1'};
    for (int i = 0; i < 8; ++i) h->magic[i] = magic[i];
    h->version = 1;
    h->format = uint32_t(fmt);
    h->N = N;
    h->K = K;
    h->layout = 1;
    h->t_w = t_w ? *t_w : 1.0f;
    h->code_off = uint64_t(L.code_off);
    h->scale_off = uint64_t(L.scale_off);
    h->r_off = uint64_t(L.r_off);
    h->total = uint64_t(L.total);
    for (int i = 0; i < int(sizeof(h->pad)); ++i) h->pad[i] = 0;
  }
}

__global__ __launch_bounds__(kThreads) void unpack_tail_kernel(int fmt, int64_t N, int64_t K,
                                                               const uint8_t* __restrict__ blob,
                                                               float* __restrict__ r,
                                                               float* __restrict__ t_w) {
  const BlobLayout L = blob_layout(fmt, N, K);
  const float* rs = reinterpret_cast<const float*>(blob + L.r_off);
  if (r)
    for (int64_t n = int64_t(blockIdx.x) * kThreads + threadIdx.x; n < N;
         n += int64_t(gridDim.x) * kThreads)
      r[n] = rs[n];
  if (t_w && blockIdx.x == 0 && threadIdx.x == 0)
    *t_w = reinterpret_cast<const BlobHeader*>(blob)->t_w;
}

inline unsigned blocks_for(int64_t n) { return unsigned((n + kThreads - 1) / kThreads); }

}  // namespace

hipError_t launch_pack_weight(int fmt, int64_t N, int64_t K, const void* codes,
                              const void* scales, const float* t_w, const float* r, void* blob,
                              hipStream_t stream) {
  const BlobLayout L = blob_layout(fmt, N, K);
  uint8_t* b = static_cast<uint8_t*>(blob);
  const int64_t n_units = N * K / 16;
  if (n_units)
    hipLaunchKernelGGL(pack_codes_kernel, dim3(blocks_for(n_units)), dim3(kThreads), 0, stream, fmt,
                       static_cast<const uint2*>(codes), reinterpret_cast<uint2*>(b + L.code_off),
                       n_units, K / 16, L.KS);
  const int64_t n_sw = L.NSG * L.KS * 64;
  if (n_sw)
    hipLaunchKernelGGL(pack_scales_kernel, dim3(blocks_for(n_sw)), dim3(kThreads), 0, stream, fmt,
                       static_cast<const uint8_t*>(scales),
                       reinterpret_cast<uint32_t*>(b + L.scale_off), n_sw, L.KS, L.NG,
                       K / block_size(fmt));
  hipLaunchKernelGGL(pack_tail_kernel, dim3(std::max(1u, std::min(64u, blocks_for(N)))),
                     dim3(kThreads), 0, stream, fmt, N, K, t_w, r, b);
  return hipGetLastError();
}

hipError_t launch_unpack_weight(int fmt, int64_t N, int64_t K, const void* blob, void* codes,
                                void* scales, float* r, float* t_w, hipStream_t stream) {
  const BlobLayout L = blob_layout(fmt, N, K);
  const uint8_t* b = static_cast<const uint8_t*>(blob);
  const int64_t n_units = N * K / 16;
  if (codes && n_units)
    hipLaunchKernelGGL(unpack_codes_kernel, dim3(blocks_for(n_units)), dim3(kThreads), 0, stream,
                       fmt, reinterpret_cast<const uint2*>(b + L.code_off),
                       static_cast<uint2*>(codes), n_units, K / 16, L.KS);
  const int64_t n_sw = L.NSG * L.KS * 64;
  if (scales && n_sw)
    hipLaunchKernelGGL(unpack_scales_kernel, dim3(blocks_for(n_sw)), dim3(kThreads), 0, stream,
                       fmt, reinterpret_cast<const uint32_t*>(b + L.scale_off),
                       static_cast<uint8_t*>(scales), n_sw, L.KS, L.NG, K / block_size(fmt));
  if (r || t_w)
    hipLaunchKernelGGL(unpack_tail_kernel, dim3(std::max(1u, std::min(64u, blocks_for(N)))),
                       dim3(kThreads), 0, stream, fmt, N, K, b, r, t_w);
  return hipGetLastError();
}

}  // namespace w4a4
