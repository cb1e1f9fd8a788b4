// Offline packing of a quantized weight into the gfx950 GEMM layout.
//
// DualQuant Appendix I: quantized weights and their scales are packed
// offline into the GEMM backend's storage layout and stay packed during
// inference.  The layouts chosen here follow the operand order of the MFMA
// that consumes them (see common.h): a wave loads a 1 KiB fragment tile with
// one coalesced 16-byte load per lane, and the block scales are regrouped
// per K tile so that one dword per lane carries the scale bytes of several
// row groups (picked by the MFMA's byte select).
#include <string.h>

#include "common.h"
#include "kernels.h"

namespace w4a4 {
namespace {

constexpr int kThreads = 256;

// Destination of 8-byte unit u (16 codes) of a canonical row n inside the
// fragment tiles, as (tile (g, h), lane, byte offset in the lane's 16 bytes).
//   MXFP4  : 64-K tiles of 32 rows; lane (n%32) + 32 c holds the 32-code chunk
//            c of the tile, so unit u goes to tile h = u/4, chunk (u%4)/2,
//            offset 8 (u%2).
//   NVFP4  : 128-K tiles of 16 rows; lane (n%16) + 16 c holds chunk c.
//   MXINT4 : (widened to FP8 in the GEMM) with FP8 operands the 16x16x128
//            MFMA takes K 16c..16c+15 from lane group c's first four dwords
//            and K 64+16c..64+16c+15 from its last four, while the scale of
//            block b still comes from lane group b.  So lane group c carries
//            half (c & 1) of block (c >> 1) in bytes 0..7 and the same half
//            of block 2 + (c >> 1) in bytes 8..15.
//   MXFP8, MXINT8: one byte per code, so unit u holds 8 codes; 2 KiB tiles of
//            16 rows x 128 K, lane (n%16) + 16 c owning 32 bytes: K 16c..16c+15
//            (units 0, 1 of the lane) and 64+16c..64+16c+15 (units 2, 3).
__device__ __forceinline__ int64_t unit_dest(int fmt, int64_t n, int64_t u, int64_t KT) {
  int64_t g, h;
  int lane, off;
  if (is_mx8(fmt)) {
    g = n >> 4;
    h = u >> 4;
    const int v = int(u & 15);             // 8-code unit within the 128-K step
    const int half = v >> 3, c = (v >> 1) & 3;
    lane = int(n & 15) + 16 * c;
    return ((g * KT + h) * 64 + lane) * 4 + 2 * half + (v & 1);
  }
  if (fmt == MXFP4) {
    g = n >> 5;
    h = u >> 2;
    const int v = int(u & 3);
    lane = int(n & 31) + 32 * (v >> 1);
    off = v & 1;
  } else {
    g = n >> 4;
    h = u >> 3;
    const int v = int(u & 7);
    const int b = v >> 1, hb = v & 1;
    const int c = fmt == MXINT4 ? 2 * (b & 1) + hb : b;
    lane = int(n & 15) + 16 * c;
    off = fmt == MXINT4 ? b >> 1 : hb;
  }
  return ((g * KT + h) * 64 + lane) * 2 + off;  // in 8-byte units
}

// Rows N .. NG*tile_rows-1 (padding of the last row group) are written as zero.
__global__ __launch_bounds__(kThreads) void pack_codes_kernel(int fmt, const uint2* __restrict__ src,
                                                              uint2* __restrict__ dst,
                                                              int64_t n_units, int64_t N,
                                                              int64_t K16, int64_t KT) {
  // K16: 8-byte units per canonical row
  const int64_t q = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (q >= n_units) return;
  const int64_t n = q / K16, u = q - n * K16;
  dst[unit_dest(fmt, n, u, KT)] = n < N ? src[q] : uint2{0u, 0u};
}

__global__ __launch_bounds__(kThreads) void unpack_codes_kernel(int fmt,
                                                                const uint2* __restrict__ src,
                                                                uint2* __restrict__ dst,
                                                                int64_t n_units, int64_t K16,
                                                                int64_t KT) {
  const int64_t q = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (q >= n_units) return;
  const int64_t n = q / K16, u = q - n * K16;
  dst[q] = src[unit_dest(fmt, n, u, KT)];
}

// Canonical scale byte index for byte b of scale word (sg, h, lane);
// *valid is false for bytes of rows beyond N.
__device__ __forceinline__ int64_t scale_src(int fmt, int64_t sg, int64_t h, int lane, int b,
                                             int64_t N, int64_t KB, bool* valid) {
  int64_t row, blk;
  if (fmt == MXFP4) {
    row = (sg * 4 + b) * 32 + (lane & 31);
    blk = h * 2 + (lane >> 5);
  } else if (fmt == NVFP4) {
    row = (sg * 2 + (b >> 1)) * 16 + (lane & 15);
    blk = h * 8 + 2 * (lane >> 4) + (b & 1);
  } else {
    row = (sg * 4 + b) * 16 + (lane & 15);
    blk = h * 4 + (lane >> 4);
  }
  *valid = row < N;
  return row * KB + blk;
}

__global__ __launch_bounds__(kThreads) void pack_scales_kernel(
    int fmt, const uint8_t* __restrict__ src, uint32_t* __restrict__ dst, int64_t total,
    int64_t KT, int64_t N, int64_t KB) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= total) return;
  const int lane = int(i & 63);
  const int64_t t = i >> 6;
  const int64_t sg = t / KT, h = t - sg * KT;
  uint32_t w = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    bool valid;
    const int64_t s = scale_src(fmt, sg, h, lane, b, N, KB, &valid);
    if (valid) w |= uint32_t(src[s]) << (8 * b);
  }
  dst[i] = w;
}

__global__ __launch_bounds__(kThreads) void unpack_scales_kernel(
    int fmt, const uint32_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t total,
    int64_t KT, int64_t N, int64_t KB) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= total) return;
  const int lane = int(i & 63);
  const int64_t t = i >> 6;
  const int64_t sg = t / KT, h = t - sg * KT;
  const uint32_t w = src[i];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    bool valid;
    const int64_t s = scale_src(fmt, sg, h, lane, b, N, KB, &valid);
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
    h->layout = uint32_t(blob_layout_id(fmt));
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
  const int64_t row_units = code_row_bytes(fmt, K) / 8;
  const int64_t n_units = L.NG * tile_rows(fmt) * row_units;  // padded rows included
  if (n_units)
    hipLaunchKernelGGL(pack_codes_kernel, dim3(blocks_for(n_units)), dim3(kThreads), 0, stream, fmt,
                       static_cast<const uint2*>(codes), reinterpret_cast<uint2*>(b + L.code_off),
                       n_units, N, row_units, L.KT);
  const int64_t n_sw = L.NSG * L.KT * 64;
  if (n_sw)
    hipLaunchKernelGGL(pack_scales_kernel, dim3(blocks_for(n_sw)), dim3(kThreads), 0, stream, fmt,
                       static_cast<const uint8_t*>(scales),
                       reinterpret_cast<uint32_t*>(b + L.scale_off), n_sw, L.KT, N,
                       K / block_size(fmt));
  hipLaunchKernelGGL(pack_tail_kernel, dim3(std::max(1u, std::min(64u, blocks_for(N)))),
                     dim3(kThreads), 0, stream, fmt, N, K, t_w, r, b);
  return hipGetLastError();
}

hipError_t launch_unpack_weight(int fmt, int64_t N, int64_t K, const void* blob, void* codes,
                                void* scales, float* r, float* t_w, hipStream_t stream) {
  const BlobLayout L = blob_layout(fmt, N, K);
  const uint8_t* b = static_cast<const uint8_t*>(blob);
  const int64_t row_units = code_row_bytes(fmt, K) / 8;
  const int64_t n_units = N * row_units;
  if (codes && n_units)
    hipLaunchKernelGGL(unpack_codes_kernel, dim3(blocks_for(n_units)), dim3(kThreads), 0, stream,
                       fmt, reinterpret_cast<const uint2*>(b + L.code_off),
                       static_cast<uint2*>(codes), n_units, row_units, L.KT);
  const int64_t n_sw = L.NSG * L.KT * 64;
  if (scales && n_sw)
    hipLaunchKernelGGL(unpack_scales_kernel, dim3(blocks_for(n_sw)), dim3(kThreads), 0, stream,
                       fmt, reinterpret_cast<const uint32_t*>(b + L.scale_off),
                       static_cast<uint8_t*>(scales), n_sw, L.KT, N, K / block_size(fmt));
  if (r || t_w)
    hipLaunchKernelGGL(unpack_tail_kernel, dim3(std::max(1u, std::min(64u, blocks_for(N)))),
                       dim3(kThreads), 0, stream, fmt, N, K, b, r, t_w);
  return hipGetLastError();
}

}  // namespace w4a4
