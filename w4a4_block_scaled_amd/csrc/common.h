// Internal definitions shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

// MXFP8 and MXINT8 are the 8-bit MX variants (E4M3 or int8 elements, one
// byte each, blocks of 32 with E8M0 scales); value 3 is INT4 with G = 64,
// which has its own kernels (int4g64.hip).
enum Fmt : int { MXFP4 = 0, NVFP4 = 1, MXINT4 = 2, MXFP8 = 4, MXINT8 = 5 };

__host__ __device__ constexpr int block_size(int fmt) { return fmt == NVFP4 ? 16 : 32; }
__host__ __device__ constexpr bool is_mx8(int fmt) { return fmt == MXFP8 || fmt == MXINT8; }
// bytes of codes per row of K elements
__host__ __device__ constexpr int64_t code_row_bytes(int fmt, int64_t K) {
  return is_mx8(fmt) ? K : K / 2;
}

// ---------------------------------------------------------------------------
// Packed-weight blob.
//
//   [0, 256)            header (BlobHeader)
//   [code_off, ...)     codes in 1 KiB fragment tiles, the operand order of the
//                       MFMA that consumes them; rows beyond N are zero.
//     MXFP4  (layout 2): tile (g, h) covers rows 32 g .. +32 and K 64 h .. +64;
//                        lane l (0..63) owns 16 bytes = the 32 canonical codes
//                        of row 32 g + l%32, K = 64 h + 32 (l/32) .. +32
//                        (V_MFMA_SCALE_F32_32X32X64_F8F6F4 with FP4 operands).
//     NVFP4, MXINT4 (layout 1): tile (g, h) covers rows 16 g .. +16 and K
//                        128 h .. +128; lane l owns 16 bytes of row 16 g + l%16
//                        (K chunk l/16 for NVFP4; the FP8 arrangement of the
//                        16x16x128 MFMA for MXINT4, see pack.hip).
//     MXFP8, MXINT8 (layout 3): 2 KiB tiles of 16 rows x 128 K (one byte per
//                        code); lane l owns 32 bytes of row 16 g + l%16: the
//                        codes of K 16c .. +16 and 64 + 16c .. +16 with
//                        c = l/16, the FP8 operand order of the 16x16x128 MFMA.
//                       Tiles are ordered g-major: ((g * KT) + h) * tile bytes.
//   [scale_off, ...)    block scales as "scale words": one dword per
//                       (row-group set sg, K tile h, lane l), laid out
//                       [sg][h][lane].  Each byte serves one row group so that
//                       a single VGPR feeds the MFMA scale operand of several
//                       weight tiles (byte picked by op_sel).
//                         MXFP4 : byte j = scale of row 32 (4 sg + j) + l%32,
//                                 block 2 h + l/32.
//                         MXINT4, MXFP8, MXINT8: byte j = scale of row
//                                 16 (4 sg + j) + l%16, block 4 h + l/16.
//                         NVFP4 : byte 2j+b = scale of row 16 (2 sg + j) + l%16,
//                                 block 8 h + 2 (l/16) + b.
//                       Bytes of row groups beyond N are zero.
//   [r_off, ...)        fp32 row scales r[N].
// ---------------------------------------------------------------------------
struct BlobHeader {
  char magic[8];      // "W4A4PK01"
  uint32_t version;   // 1
  uint32_t format;
  int64_t N, K;
  uint32_t layout;    // 1: 16-row x 128-K tiles, 2: 32-row x 64-K tiles, 3: 8-bit 16 x 128,
                      // 4: INT4 G=64 512-byte tiles (int4g64.hip)
  float t_w;
  uint64_t code_off, scale_off, r_off, total;
  uint8_t pad[256 - 8 - 4 - 4 - 16 - 4 - 4 - 32];
};
static_assert(sizeof(BlobHeader) == 256, "blob header must be 256 bytes");

__host__ __device__ constexpr int blob_layout_id(int fmt) {
  return fmt == MXFP4 ? 2 : is_mx8(fmt) ? 3 : 1;
}
__host__ __device__ constexpr int tile_rows(int fmt) { return fmt == MXFP4 ? 32 : 16; }
__host__ __device__ constexpr int tile_k(int fmt) { return fmt == MXFP4 ? 64 : 128; }
__host__ __device__ constexpr int groups_per_scale_word(int fmt) { return fmt == NVFP4 ? 2 : 4; }

struct BlobLayout {
  int64_t N, K;
  int64_t NG;   // row groups of tile_rows(fmt) rows (N rounded up)
  int64_t KT;   // K tiles of tile_k(fmt)
  int64_t KS;   // 128-wide K-steps
  int64_t NSG;  // scale-word row-group sets: ceil(NG / groups_per_scale_word)
  int64_t code_off, scale_off, r_off, total;
};

__host__ __device__ inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

__host__ __device__ inline BlobLayout blob_layout(int fmt, int64_t N, int64_t K) {
  BlobLayout L;
  L.N = N;
  L.K = K;
  const int rows = tile_rows(fmt);
  L.NG = (N + rows - 1) / rows;
  L.KT = K / tile_k(fmt);
  L.KS = K / 128;
  const int gpw = groups_per_scale_word(fmt);
  L.NSG = (L.NG + gpw - 1) / gpw;
  L.code_off = 256;
  L.scale_off = align256(L.code_off + L.NG * rows * code_row_bytes(fmt, K));
  L.r_off = align256(L.scale_off + L.NSG * L.KT * 64 * 4);
  L.total = align256(L.r_off + 4 * N);
  return L;
}

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// The blob header must name the format and shape the GEMM is called with:
// every GEMM kernel checks it before it reads anything else of the blob, and
// on a mismatch writes Y as BF16 NaN instead of reading a blob laid out for
// another shape (which could run past its end).
constexpr uint64_t kBlobMagic = 0x31304B5034413457ull;  // "W4A4PK01", little-endian

__device__ __forceinline__ bool blob_header_ok(const uint8_t* blob, int fmt, int64_t N, int64_t K) {
  const BlobHeader* h = reinterpret_cast<const BlobHeader*>(blob);
  return *reinterpret_cast<const uint64_t*>(h->magic) == kBlobMagic && h->format == uint32_t(fmt) &&
         h->N == N && h->K == K;
}

// Y [M x N] bf16 (N % 16 == 0, 16-byte aligned) <- NaN, spread over the
// whole grid (1-D or 2-D): every workgroup writes its share.
__device__ inline void fill_y_nan(uint16_t* Y, int64_t M, int64_t N) {
  const int64_t chunks = M * N / 8;
  const int64_t step = int64_t(gridDim.x) * gridDim.y * blockDim.x;
  const int64_t first = (int64_t(blockIdx.y) * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
  const uint4 nan = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
  for (int64_t i = first; i < chunks; i += step) reinterpret_cast<uint4*>(Y)[i] = nan;
}

// The rows m0 .. m0+rows-1 and columns n0 .. n0+cols-1 of Y (clipped to
// M x N; n0 and cols multiples of 8) <- NaN, by the threads of one workgroup.
__device__ inline void fill_tile_nan(uint16_t* Y, int64_t M, int64_t N, int64_t m0, int64_t n0,
                                     int rows, int cols) {
  const uint4 nan = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
  const int per_row = cols / 8;
  for (int i = threadIdx.x; i < rows * per_row; i += blockDim.x) {
    const int64_t m = m0 + i / per_row, n = n0 + 8 * (i % per_row);
    if (m < M && n < N) *reinterpret_cast<uint4*>(Y + m * N + n) = nan;
  }
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t qnan = ((u >> 16) | 0x40u) & 0xffffu;
  return (u & 0x7fffffffu) > 0x7f800000u ? qnan : rounded;
}

}  // namespace w4a4
