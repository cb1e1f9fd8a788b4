// Internal definitions shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

enum Fmt : int { MXFP4 = 0, NVFP4 = 1, MXINT4 = 2 };

__host__ __device__ constexpr int block_size(int fmt) { return fmt == NVFP4 ? 16 : 32; }

// ---------------------------------------------------------------------------
// Packed-weight blob.
//
//   [0, 256)            header (BlobHeader)
//   [code_off, ...)     codes, MFMA fragment order: tile (ng, ks) covers output
//                       rows 16*ng .. +16 and K range 128*ks .. +128 and is
//                       1 KiB: lane l (0..63) owns 16 bytes = the 32 canonical
//                       codes of row 16*ng + l%16, K = 128*ks + 32*(l/16) .. +32
//                       (same nibble order as the canonical layout).
//   [scale_off, ...)    block scales as "scale words": one dword per
//                       (row-group quad/pair sg, K-step ks, lane l), laid out
//                       [sg][ks][lane].  Each byte serves one 16-row group so
//                       that a single VGPR feeds the MFMA scale operand of
//                       several weight fragments (byte picked by op_sel).
//                         MX : 4 groups per word; byte j = scale of row
//                              16*(4 sg + j) + l%16, block 4 ks + l/16.
//                         NV : 2 groups per word; byte 2j+h = scale of row
//                              16*(2 sg + j) + l%16, block 8 ks + 2 (l/16) + h.
//                       Bytes of groups beyond N/16 are zero.
//   [r_off, ...)        fp32 row scales r[N].
// ---------------------------------------------------------------------------
struct BlobHeader {
  char magic[8];      // "W4A4PK01"
  uint32_t version;   // 1
  uint32_t format;
  int64_t N, K;
  uint32_t layout;    // 1: 16x128 fragment tiles
  float t_w;
  uint64_t code_off, scale_off, r_off, total;
  uint8_t pad[256 - 8 - 4 - 4 - 16 - 4 - 4 - 32];
};
static_assert(sizeof(BlobHeader) == 256, "blob header must be 256 bytes");

struct BlobLayout {
  int64_t N, K, NG, KS;
  int64_t NSG;  // scale-word row groups: ceil(NG / groups_per_word)
  int64_t code_off, scale_off, r_off, total;
};

__host__ __device__ constexpr int groups_per_scale_word(int fmt) { return fmt == NVFP4 ? 2 : 4; }

__host__ __device__ inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

__host__ __device__ inline BlobLayout blob_layout(int fmt, int64_t N, int64_t K) {
  BlobLayout L;
  L.N = N;
  L.K = K;
  L.NG = N / 16;
  L.KS = K / 128;
  const int gpw = groups_per_scale_word(fmt);
  L.NSG = (L.NG + gpw - 1) / gpw;
  L.code_off = 256;
  L.scale_off = align256(L.code_off + N * K / 2);
  L.r_off = align256(L.scale_off + L.NSG * L.KS * 64 * 4);
  L.total = align256(L.r_off + 4 * N);
  return L;
}

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t qnan = ((u >> 16) | 0x40u) & 0xffffu;
  return (u & 0x7fffffffu) > 0x7f800000u ? qnan : rounded;
}

}  // namespace w4a4
