// INT4 with blocks of 64 and BF16 block scales: the packed deployment format
// of DualQuant (Appendix I, "Real packed W4A4 deployment": INT4, G = 64, BF16
// group scales, weights packed offline).  Section 3 gives the symmetric block
// quantizer (Delta = max|x| / q_max, q_max = 7 on the INT4 grid) and Section
// 4.2 the BF16 admissible set for INT4 scales.
//
// gfx950's block-scaled MFMAs take only E8M0 scales, so BF16 scales cannot
// ride on the matrix core: the kernels below either fold them into exact
// fp16 operands or apply each block's scale product to its exact integer
// partial sum in fp32.
//
//   quantize  x~ = fp32(X) * c (one rounded fp32 multiply); per 64-block
//             Delta = BF16(amax / 7) rounded once from the fp64 quotient;
//             code = clip(RNE(x~ / Delta), -8, 7) from the fp64 quotient.
//   blob      256-byte header; codes in 512-byte fragment tiles, tile (g, b)
//             = rows 16 g .. +16, K 64 b .. +64, lane l owning the 8 canonical
//             bytes of row 16 g + l % 16 at K 64 b + 16 (l / 16) .. +16,
//             g-major; scales [N/16][K/64][16] BF16; r [N] fp32.
//   GEMM      M > 16 and K a multiple of 128: code x scale expanded exactly
//             into fp16 for the fp16 MFMA (gemm_int4g64_f16_kernel below);
//             M <= 3 (same K): block dot products on the VALU
//             (gemm_int4g64_dot_kernel); otherwise one integer MFMA per block,
//             int4 nibbles widened to int8 as (nibble << 4), which is 16 x
//             the signed code, so each block sum is 256 x the code dot
//             product (the 2^-8 goes into the epilogue, exact).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "kernels.h"

namespace w4a4 {
namespace {

constexpr int kG = 64;

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ inline float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Nearest BF16 (ties to even) to a non-negative finite double: 8 significant
// bits, spacing fixed at 2^-133 below 2^-126.  The result is a BF16 value, so
// its conversion to fp32 is exact and the top 16 bits are the pattern.
__device__ inline uint32_t bf16_bits_rne(double v) {
  if (v == 0.0) return 0;
  const int e = ilogb(v);                      // 2^e <= v < 2^(e+1)
  const int qe = e - 7 > -133 ? e - 7 : -133;  // exponent of one unit in the last place
  const double n = rint(ldexp(v, -qe));
  return __float_as_uint(float(ldexp(n, qe))) >> 16;
}

__device__ inline float bf16_round_f32(float y, uint16_t* out) {
  const uint32_t u = __float_as_uint(y);
  *out = uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
  return y;
}

// ---------------------------------------------------------------- quantize --
// One thread per 8 consecutive elements (one 16-byte load); the 8 threads of a
// 64-block are 8 consecutive lanes and exchange the block maximum and the
// non-finite flag through lane shuffles.  Total threads M*K/8 is a multiple
// of 8, so a block's lanes are all inside or all outside the range.
__global__ void __launch_bounds__(256)
quantize_int4g64_kernel(const uint16_t* __restrict__ X, const float* __restrict__ c, int64_t K,
                        int64_t total8, uint32_t* __restrict__ codes,
                        uint16_t* __restrict__ scales) {
  const int64_t k8 = K / 8;
  for (int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x; t < total8;
       t += int64_t(gridDim.x) * 256) {
    const int64_t row = t / k8;
    const int64_t kc = (t - row * k8) * 8;
    const uint4 raw = *reinterpret_cast<const uint4*>(X + row * K + kc);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
      x[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
    }
    if (c) {
      const float4 c0 = *reinterpret_cast<const float4*>(c + kc);
      const float4 c1 = *reinterpret_cast<const float4*>(c + kc + 4);
      const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = x[j] * cc[j];
    }
    float amax = 0.f;
    int bad = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bad |= !isfinite(x[j]);
      amax = fmaxf(amax, fabsf(x[j]));
    }
#pragma unroll
    for (int s = 1; s < 8; s <<= 1) {
      amax = fmaxf(amax, __shfl_xor(amax, s));
      bad |= __shfl_xor(bad, s);
    }
    uint32_t bits = bad ? 0u : bf16_bits_rne(double(amax) / 7.0);
    const double delta = double(bf16_bits_to_f32(bits));
    uint32_t packed = 0;
    if (!bad && bits) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        double q = rint(double(x[j]) / delta);
        q = q > 7.0 ? 7.0 : (q < -8.0 ? -8.0 : q);
        packed |= (uint32_t(int(q)) & 15u) << (4 * j);
      }
    }
    if (bad) bits = 0x7FC0u;
    codes[t] = packed;
    if ((threadIdx.x & 7) == 0) scales[t / 8] = uint16_t(bits);
  }
}

// -------------------------------------------------------------------- pack --
struct I4Layout {
  int64_t NG, KB, code_off, scale_off, r_off, total;
};

__host__ __device__ inline I4Layout i4_layout(int64_t N, int64_t K) {
  I4Layout L;
  L.NG = N / 16;
  L.KB = K / kG;
  L.code_off = 256;
  L.scale_off = align256(L.code_off + N * (K / 2));
  L.r_off = align256(L.scale_off + N * L.KB * 2);
  L.total = align256(L.r_off + N * 4);
  return L;
}

// One thread per 8-byte lane chunk: chunk t = (tile, lane), tile = g * KB + b;
// also one per scale and per row scale.  unpack = 1 copies the other way
// (canonical outputs that are NULL are skipped).
__global__ void __launch_bounds__(256)
pack_int4g64_kernel(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                    const float* __restrict__ r, int64_t N, int64_t K, uint8_t* __restrict__ blob,
                    int unpack, float* __restrict__ t_w) {
  const I4Layout L = i4_layout(N, K);
  const int64_t chunks = N * K / 16;
  const int64_t nscales = N * L.KB;
  const int64_t work = chunks > nscales ? chunks : nscales;
  for (int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x; t < work;
       t += int64_t(gridDim.x) * 256) {
    if (t < chunks) {
      const int64_t tile = t >> 6;
      const int lane = int(t & 63);
      const int64_t g = tile / L.KB, b = tile - g * L.KB;
      const int64_t src = (16 * g + (lane & 15)) * (K / 2) + b * 32 + (lane >> 4) * 8;
      uint64_t* packed = reinterpret_cast<uint64_t*>(blob + L.code_off) + t;
      const uint64_t* canon = reinterpret_cast<const uint64_t*>(codes + src);
      if (!unpack) *packed = *canon;
      else if (codes) *const_cast<uint64_t*>(canon) = *packed;
    }
    if (t < nscales) {
      const int64_t n = t / L.KB, b = t - n * L.KB;
      uint16_t* ps = reinterpret_cast<uint16_t*>(blob + L.scale_off) + ((n >> 4) * L.KB + b) * 16 + (n & 15);
      uint16_t* cs = const_cast<uint16_t*>(scales) + t;
      if (!unpack) *ps = *cs;
      else if (scales) *cs = *ps;
    }
    if (t < N) {
      float* pr = reinterpret_cast<float*>(blob + L.r_off) + t;
      if (!unpack) *pr = r[t];
      else if (r) const_cast<float*>(r)[t] = *pr;
    }
    if (unpack && t_w && t == 0) *t_w = 1.0f;   // no tensor scale in this format
  }
}

// The header is written field by field into the blob (the GEMM kernels check
// its magic, format, N and K before reading the blob).
__global__ void pack_int4g64_header_kernel(int64_t N, int64_t K, uint8_t* blob) {
  if (threadIdx.x != 0) return;
  const I4Layout L = i4_layout(N, K);
  BlobHeader* h = reinterpret_cast<BlobHeader*>(blob);
  const char m[8] = {'W', '4', 'A', '4', 'P', 'K', '0', '1'};
  for (int i = 0; i < 8; ++i) h->magic[i] = m[i];
  h->version = 1;
  h->format = 3;
  h->N = N;
  h->K = K;
  h->layout = 4;
  h->t_w = 1.0f;
  h->code_off = uint64_t(L.code_off);
  h->scale_off = uint64_t(L.scale_off);
  h->r_off = uint64_t(L.r_off);
  h->total = uint64_t(L.total);
  for (int i = 0; i < int(sizeof(h->pad)); ++i) h->pad[i] = 0;
}

// -------------------------------------------------------------------- GEMM --
// Widen 16 int4 codes (8 bytes) to 16 int8 bytes holding 16 x code: even
// elements from the low nibbles, odd from the high ones.  The activation and
// weight fragments use the same arrangement, so the MFMA pairs equal K.
__device__ inline v4i widen(uint2 d) {
  v4i o;
  o[0] = int((d.x << 4) & 0xF0F0F0F0u);
  o[1] = int(d.x & 0xF0F0F0F0u);
  o[2] = int((d.y << 4) & 0xF0F0F0F0u);
  o[3] = int(d.y & 0xF0F0F0F0u);
  return o;
}

__device__ inline v4i mfma_block(v4i a, v4i w) {
  const v4i zero = {0, 0, 0, 0};
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, w, zero, 0, 0, 0);
}

// Both GEMM kernels put the weight fragment in the MFMA's row operand and the
// activation fragment in its column operand, so lane l holds the outputs
// (activation row l % 16, weight columns 4 (l / 16) .. +4): one activation
// scale per fragment, the four weight scales in one 8-byte load and the four
// outputs in one 8-byte store.
__device__ inline void store4(uint16_t* y, const float* acc, const float* rn) {
  uint16_t o[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) bf16_round_f32(acc[v] * rn[v], &o[v]);
  *reinterpret_cast<uint2*>(y) = make_uint2(uint32_t(o[0]) | (uint32_t(o[1]) << 16),
                                            uint32_t(o[2]) | (uint32_t(o[3]) << 16));
}

// acc[v] += sum[v] * Delta_a * Delta_w[v]: the accumulators hold 2^8 times
// the output (every block sum is 256 x the code dot product); the epilogue's
// row scale carries the 2^-8 (power-of-two scalings, so the products and
// sums round exactly as with the factor applied per block).  The product
// Delta_a * Delta_w is exact (BF16 values keep at most 8 significant bits).
__device__ inline void scale_add4(float* acc, v4i s, float sa, const float* sw) {
#pragma unroll
  for (int v = 0; v < 4; ++v) acc[v] = fmaf(float(s[v]), sa * sw[v], acc[v]);
}

__device__ inline void unpack_sw(uint2 w, float* sw) {
  sw[0] = bf16_bits_to_f32(w.x & 0xFFFFu);
  sw[1] = bf16_bits_to_f32(w.x >> 16);
  sw[2] = bf16_bits_to_f32(w.y & 0xFFFFu);
  sw[3] = bf16_bits_to_f32(w.y >> 16);
}

// Tile kernel: 4 waves as 2 (M) x 2 (N); a wave owns FM x FN fragments of
// 16 x 16 outputs, the workgroup (2 FM 16) x (2 FN 16).  Operands come
// straight from global memory, two K blocks ahead of the one being
// multiplied (activation rows clamped to M - 1, weight row groups to NG - 1,
// so every load is in bounds); outputs outside M x N are not stored.
// Workgroups are dealt to the 8 XCDs round-robin; workgroup b takes tile
// number (b % 8) per_xcd + b / 8 of an order that runs through blocks of 8
// x 8 tiles (8 column tiles wide, then down the rows): each XCD works
// through a contiguous range of that order, so the 64 workgroups it runs at
// once (two per CU) cover 8 row tiles x 8 column tiles and fetch each of
// their activation rows and weight groups into its L2 once.
template <int FM, int FN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
gemm_int4g64_tile_kernel(const uint8_t* __restrict__ a_codes, const uint16_t* __restrict__ a_scales,
                         const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M,
                         int64_t N, int64_t K, int tiles_m, int tiles_n, int per_xcd) {
  if (!blob_header_ok(blob, 3, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  const int o = int(blockIdx.x % 8) * per_xcd + int(blockIdx.x / 8);
  if (o >= tiles_m * tiles_n) return;
  const int nb = o / (8 * tiles_m), ob = o - nb * 8 * tiles_m;
  const int nw = tiles_n - 8 * nb < 8 ? tiles_n - 8 * nb : 8;  // width of this column block
  const int tm = ob / nw, tn = 8 * nb + ob % nw;
  const I4Layout L = i4_layout(N, K);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m0 = int64_t(tm) * (2 * FM * 16) + (wave >> 1) * (FM * 16);
  const int64_t g0 = int64_t(tn) * (2 * FN) + (wave & 1) * FN;
  const uint8_t* wcodes = blob + L.code_off + lane * 8;
  const uint16_t* wscales = reinterpret_cast<const uint16_t*>(blob + L.scale_off) + 4 * (lane >> 4);

  const uint8_t* arow[FM];
  const uint16_t* srow[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + i * 16 + (lane & 15);
    const int64_t mc = m < M ? m : M - 1;
    arow[i] = a_codes + mc * (K / 2) + (lane >> 4) * 8;
    srow[i] = a_scales + mc * L.KB;
  }
  int64_t gbase[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) gbase[j] = (g0 + j < L.NG ? g0 + j : L.NG - 1) * L.KB;

  float acc[FM][FN][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.f;

  // two register sets: block b + 2's loads go out while block b + 1's are
  // still in flight, so the in-order load counter only waits for the older set
  struct Ops {
    uint2 a[FM], w[FN], sw[FN];
    uint16_t sa[FM];
  };
  auto load = [&](int64_t b, Ops& o) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      o.a[i] = *reinterpret_cast<const uint2*>(arow[i] + b * 32);
      o.sa[i] = srow[i][b];
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t tile = gbase[j] + b;
      o.w[j] = *reinterpret_cast<const uint2*>(wcodes + tile * 512);
      o.sw[j] = *reinterpret_cast<const uint2*>(wscales + tile * 16);
    }
  };
  // Per pair of weight fragments: their 2 FM integer MFMAs back to back,
  // then the scaling of the block sums, so that no sum is read right after
  // the MFMA that writes it (each would stall the wave for the MFMA's
  // latency).
  auto compute = [&](const Ops& o) {
    v4i A[FM];
    float sa[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      A[i] = widen(o.a[i]);
      sa[i] = bf16_bits_to_f32(o.sa[i]);
    }
#pragma unroll
    for (int j0 = 0; j0 < FN; j0 += 2) {
      v4i S[2][FM];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const v4i W = widen(o.w[j0 + jj]);
#pragma unroll
        for (int i = 0; i < FM; ++i) S[jj][i] = mfma_block(W, A[i]);
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        float sw[4];
        unpack_sw(o.sw[j0 + jj], sw);
#pragma unroll
        for (int i = 0; i < FM; ++i) scale_add4(acc[i][j0 + jj], S[jj][i], sa[i], sw);
      }
    }
  };
  const int64_t last = L.KB - 1;
  Ops p0, p1;
  load(0, p0);
  load(last < 1 ? last : 1, p1);
  // the scheduling barriers keep each set's unpacking (and so its load wait)
  // after the other set's loads have been issued
  for (int64_t b = 0; b < L.KB; b += 2) {
    compute(p0);
    load(b + 2 < last ? b + 2 : last, p0);
    __builtin_amdgcn_sched_barrier(0);
    if (b + 1 < L.KB) {
      compute(p1);
      load(b + 3 < last ? b + 3 : last, p1);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  const float* r = reinterpret_cast<const float*>(blob + L.r_off);
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    if (g0 + j >= L.NG) continue;
    const int64_t n = (g0 + j) * 16 + 4 * (lane >> 4);
    const float4 r4 = *reinterpret_cast<const float4*>(r + n);
    const float rn[4] = {r4.x * 0.00390625f, r4.y * 0.00390625f, r4.z * 0.00390625f, r4.w * 0.00390625f};
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t m = m0 + i * 16 + (lane & 15);
      if (m < M) store4(Y + m * N + n, acc[i][j], rn);
    }
  }
}

// Decode kernel (M <= 16): a workgroup owns one 16-column group g; its
// WAVES waves take the K blocks b = wave, wave + WAVES, ... with U blocks'
// loads in flight, and their partial sums are added through LDS in wave
// order, so results do not depend on timing.
template <int WAVES, int U>
__global__ void __launch_bounds__(64 * WAVES)
gemm_int4g64_decode_kernel(const uint8_t* __restrict__ a_codes,
                           const uint16_t* __restrict__ a_scales, const uint8_t* __restrict__ blob,
                           uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K) {
  if (!blob_header_ok(blob, 3, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  const I4Layout L = i4_layout(N, K);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t g = blockIdx.x;
  const int64_t ma = (lane & 15) < M ? (lane & 15) : M - 1;
  const uint8_t* arow = a_codes + ma * (K / 2) + (lane >> 4) * 8;
  const uint16_t* srow = a_scales + ma * L.KB;
  const uint8_t* wtile = blob + L.code_off + g * L.KB * 512 + lane * 8;
  const uint16_t* wsc = reinterpret_cast<const uint16_t*>(blob + L.scale_off) + g * L.KB * 16 +
                        4 * (lane >> 4);

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  int64_t b = wave;
  for (; b + WAVES * (U - 1) < L.KB; b += WAVES * U) {
    uint2 wa[U], aa[U], ws[U];
    uint16_t as[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t bb = b + WAVES * u;
      wa[u] = *reinterpret_cast<const uint2*>(wtile + bb * 512);
      ws[u] = *reinterpret_cast<const uint2*>(wsc + bb * 16);
      aa[u] = *reinterpret_cast<const uint2*>(arow + bb * 32);
      as[u] = srow[bb];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float sw[4];
      unpack_sw(ws[u], sw);
      scale_add4(acc, mfma_block(widen(wa[u]), widen(aa[u])), bf16_bits_to_f32(as[u]), sw);
    }
  }
  for (; b < L.KB; b += WAVES) {
    float sw[4];
    unpack_sw(*reinterpret_cast<const uint2*>(wsc + b * 16), sw);
    scale_add4(acc,
               mfma_block(widen(*reinterpret_cast<const uint2*>(wtile + b * 512)),
                          widen(*reinterpret_cast<const uint2*>(arow + b * 32))),
               bf16_bits_to_f32(srow[b]), sw);
  }

  __shared__ float part[WAVES - 1][64][4];
  if (wave > 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) part[wave - 1][lane][v] = acc[v];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < WAVES - 1; ++w)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] += part[w][lane][v];
    const int64_t n = g * 16 + 4 * (lane >> 4);
    const float4 r4 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(blob + L.r_off) + n);
    const float rn[4] = {r4.x * 0.00390625f, r4.y * 0.00390625f, r4.z * 0.00390625f, r4.w * 0.00390625f};
    if ((lane & 15) < M) store4(Y + int64_t(lane & 15) * N + n, acc, rn);
  }
}

typedef _Float16 i4h2 __attribute__((ext_vector_type(2)));
typedef _Float16 i4v8h __attribute__((ext_vector_type(8)));
typedef float i4v16f __attribute__((ext_vector_type(16)));
typedef uint32_t i4u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t i4u32x2 __attribute__((ext_vector_type(2)));
#define I4_LDS __attribute__((address_space(3)))

// Decode kernel for one to three activation rows (MD = M), K a multiple of
// 128: the MFMA's 16 activation columns would be 15/16 empty, so the block
// dot products run on the VALU instead (v_dot8_i32_i4: 8 signed int4
// products per lane per instruction).  A workgroup owns one 16-column group
// g and reads its blob tiles two blocks (1 KiB, contiguous) at a time with
// one 16-byte load per lane: lane l takes tile b + l / 32 at byte 16 (l %
// 32), which is the fragment chunk of columns n = 2 (l % 8) and n + 1 at
// K 64 b' + 16 c .. +16 with c = (l % 32) / 8, and the same 16 activation
// codes of each row.  Two dot instructions per column give the exact
// integer block sum, which joins the lane's fp32 sum once multiplied by the
// block's Delta_a * Delta_w (exact: two BF16 values).  The WAVES waves take
// the block pairs wave, wave + WAVES, ... with U pairs' loads in flight;
// the eight lanes of a column pair are added by three lane exchanges and
// the waves in wave order through LDS, so results do not depend on timing.
template <int WAVES, int U, int MD>
__global__ void __launch_bounds__(64 * WAVES)
gemm_int4g64_dot_kernel(const uint8_t* __restrict__ a_codes, const uint16_t* __restrict__ a_scales,
                        const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N,
                        int64_t K) {
  if (!blob_header_ok(blob, 3, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  const I4Layout L = i4_layout(N, K);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = lane >> 5, c = (lane & 31) >> 3, n0 = 2 * (lane & 7);
  const int64_t g = blockIdx.x, KP = L.KB / 2;
  // pair p: block 2 p + t of this lane
  const uint8_t* wtile = blob + L.code_off + (g * L.KB + t) * 512 + 16 * (lane & 31);
  const uint16_t* wsc = reinterpret_cast<const uint16_t*>(blob + L.scale_off) + (g * L.KB + t) * 16 + n0;
  const uint8_t* arow[MD];
  const uint16_t* srow[MD];
#pragma unroll
  for (int m = 0; m < MD; ++m) {
    arow[m] = a_codes + m * (K / 2) + t * 32 + 8 * c;
    srow[m] = a_scales + m * L.KB + t;
  }

  float acc[MD][2];
#pragma unroll
  for (int m = 0; m < MD; ++m) acc[m][0] = acc[m][1] = 0.f;
  auto pair = [&](const i4u32x4& w, uint32_t wsb, const uint2 (&a)[MD], const uint32_t (&asb)[MD]) {
    const float sw0 = bf16_bits_to_f32(wsb & 0xFFFFu), sw1 = bf16_bits_to_f32(wsb >> 16);
#pragma unroll
    for (int m = 0; m < MD; ++m) {
      const float sa = bf16_bits_to_f32(asb[m]);
      int d0 = __builtin_amdgcn_sdot8(int(w.x), int(a[m].x), 0, false);
      d0 = __builtin_amdgcn_sdot8(int(w.y), int(a[m].y), d0, false);
      int d1 = __builtin_amdgcn_sdot8(int(w.z), int(a[m].x), 0, false);
      d1 = __builtin_amdgcn_sdot8(int(w.w), int(a[m].y), d1, false);
      acc[m][0] = fmaf(float(d0), sa * sw0, acc[m][0]);
      acc[m][1] = fmaf(float(d1), sa * sw1, acc[m][1]);
    }
  };
  int64_t p = wave;
  for (; p + WAVES * (U - 1) < KP; p += WAVES * U) {
    i4u32x4 w[U];
    uint2 a[U][MD];
    uint32_t ws[U], as[U][MD];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t pp = p + WAVES * u;
      w[u] = __builtin_nontemporal_load(reinterpret_cast<const i4u32x4*>(wtile + pp * 1024));
      ws[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(wsc + pp * 32));
#pragma unroll
      for (int m = 0; m < MD; ++m) {
        a[u][m] = *reinterpret_cast<const uint2*>(arow[m] + pp * 64);
        as[u][m] = srow[m][2 * pp];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) pair(w[u], ws[u], a[u], as[u]);
  }
  for (; p < KP; p += WAVES) {
    uint2 a[MD];
    uint32_t as[MD];
#pragma unroll
    for (int m = 0; m < MD; ++m) {
      a[m] = *reinterpret_cast<const uint2*>(arow[m] + p * 64);
      as[m] = srow[m][2 * p];
    }
    pair(*reinterpret_cast<const i4u32x4*>(wtile + p * 1024), *reinterpret_cast<const uint32_t*>(wsc + p * 32), a,
         as);
  }

  // the column pair's eight lanes (c = 0..3, t = 0, 1), in every lane
#pragma unroll
  for (int m = 0; m < MD; ++m)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      acc[m][e] += __shfl_xor(acc[m][e], 8);
      acc[m][e] += __shfl_xor(acc[m][e], 16);
      acc[m][e] += __shfl_xor(acc[m][e], 32);
    }
  __shared__ float part[WAVES > 1 ? WAVES - 1 : 1][MD][16];
  if (wave > 0 && lane < 8) {
#pragma unroll
    for (int m = 0; m < MD; ++m) {
      part[wave - 1][m][n0] = acc[m][0];
      part[wave - 1][m][n0 + 1] = acc[m][1];
    }
  }
  __syncthreads();
  if (wave == 0 && lane < 8) {
    const float* r = reinterpret_cast<const float*>(blob + L.r_off) + g * 16 + n0;
#pragma unroll
    for (int m = 0; m < MD; ++m) {
      float y0 = acc[m][0], y1 = acc[m][1];
#pragma unroll
      for (int w = 0; w < WAVES - 1; ++w) {
        y0 += part[w][m][n0];
        y1 += part[w][m][n0 + 1];
      }
      uint16_t o0, o1;
      bf16_round_f32(y0 * r[0], &o0);
      bf16_round_f32(y1 * r[1], &o1);
      *reinterpret_cast<uint32_t*>(Y + int64_t(m) * N + g * 16 + n0) = uint32_t(o0) | (uint32_t(o1) << 16);
    }
  }
}

// ------------------------------------------------------ fp16 GEMM (M > 16) --
// The block scaling moves into the operands: every code times its block's
// scale becomes one exact fp16 value, and the fp16 MFMA (32 x 32 x 16,
// fp32 accumulation) adds the products of both operands with no per-block
// work on the accumulators.  An INT4 code q times a BF16 scale needs at most
// 3 + 8 significant bits, which fp16 holds, so the expansion is exact while
// the value stays in fp16's normal range.  That range is kept by a power of
// two per activation row and per weight column, taken from the largest scale
// of the row (column) over all of K and removed again in the epilogue:
//
//   g = Delta * 2^sh, sh = 147 - (largest biased exponent field of the row's
//   scales), so the largest scale becomes 2^(E+9) m with E = 11 (m in [1, 2),
//   8 significant bits) and the others E = 11 - (exponent distance).  A byte
//   u = q + 8 (0..15) is the E4M3 encoding of u * 2^-9, so the hardware
//   conversion with the power-of-two scale 2^(E+9) gives u * 2^E exactly,
//   and one fp16 fma, u 2^E * m - 8 * 2^E * m, gives q * 2^E * m in a single
//   rounding of an exact result (8 * 2^E * m has 8 significant bits).  For
//   E in [-14, 11] every intermediate and result is an fp16 normal number
//   (|q 2^E m| < 2^15), so blocks whose scales lie within 25 binades of the
//   row's (column's) largest are exact; smaller ones are rounded to fp16,
//   an error below 2^-36 of the largest block's values.
//   Y = (sum of products) * 2^(ea + ew - 276) * r, with ea, ew the exponent
//   fields of the row's and the column's largest scales.
//
// Workgroup: 4 waves as 2 (n) x 2 (m), wave tile 32 FN (n) x 32 FM (m) of
// 32 x 32 fragments; the weight fragment is the MFMA's row operand, so lane
// l holds outputs n = 32 i + 8 (e / 4) + 4 (l / 32) + e % 4 and m = 32 j + l % 32.
// Each 128-wide K-step (two blocks) is one stage of a DEPTH-deep LDS ring,
// filled by direct global -> LDS copies (equal counts per wave, so the load
// counter tells when a stage has landed):
//   A codes  per 32-row fragment, 2 KiB: block b, 16-byte half c of the
//            block's 32 bytes, row R at b 1024 + c 512 + 16 R (lane (R, c)
//            reads its 16 bytes of a block with one 16-byte read)
//   W codes  per pair of 16-row groups, 2 KiB: block b, 8-byte chunk c of
//            the blob's tile (K 16 c .. +16), row R of the pair at
//            b 1024 + c 256 + 8 R
//   A scales one dword per row (the two blocks' BF16 scales)
//   W scales the blob's 64 bytes per group (two blocks x 16 columns)
// Lane l takes, per block, the codes of K 32 (l / 32) .. +32 of its row
// (chunks 2 (l / 32) and 2 (l / 32) + 1); MFMA t of the block uses their
// dword t, in the same order for both operands.


struct F16Scale {
  float p2;       // 2^(E+9): the scale operand of the fp8 -> fp16 conversion
  i4h2 mm, cc;    // (m, m) and (-8 2^E m, -8 2^E m)
};

// BF16 scale bits and the row's (column's) shift -> the expansion constants.
// A zero scale gives zeros; a NaN scale gives NaN (cc is NaN).  The sign of
// a scale stays with m, so a negative scale expands correctly as well.
__device__ __forceinline__ F16Scale f16_scale(uint32_t bits, int sh) {
  const float g = ldexpf(bf16_bits_to_f32(bits), sh);
  const uint32_t gb = __float_as_uint(g);
  F16Scale s;
  s.p2 = __uint_as_float(gb & 0x7F800000u);
  const float m = __uint_as_float((gb & 0x807FFFFFu) | 0x3F800000u);
  const float c = g * -0.015625f;
  s.mm = __builtin_bit_cast(i4h2, __builtin_amdgcn_cvt_pkrtz(m, m));
  s.cc = __builtin_bit_cast(i4h2, __builtin_amdgcn_cvt_pkrtz(c, c));
  return s;
}

// 8 INT4 codes (one dword, code j in bits 4j..4j+3) -> 8 fp16 values of
// code x scale, in the order (0, 2, 4, 6, 1, 3, 5, 7).
__device__ __forceinline__ i4v8h expand8(uint32_t x, const F16Scale& s) {
  const uint32_t e = x ^ 0x88888888u;
  const uint32_t lo = e & 0x0F0F0F0Fu;
  const uint32_t hi = (e >> 4) & 0x0F0F0F0Fu;
#define I4_CVT(d, w) __builtin_bit_cast(i4h2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, s.p2, w))
  const i4h2 v0 = __builtin_elementwise_fma(I4_CVT(lo, false), s.mm, s.cc);
  const i4h2 v1 = __builtin_elementwise_fma(I4_CVT(lo, true), s.mm, s.cc);
  const i4h2 v2 = __builtin_elementwise_fma(I4_CVT(hi, false), s.mm, s.cc);
  const i4h2 v3 = __builtin_elementwise_fma(I4_CVT(hi, true), s.mm, s.cc);
#undef I4_CVT
  return i4v8h{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

template <int FN, int FM, int DEPTH>
struct F16Cfg {
  static constexpr int BN = 64 * FN, BM = 64 * FM;
  static constexpr int A_BYTES = BM * 64;
  static constexpr int W_BYTES = BN * 64;
  static constexpr int AS_BYTES = BM * 4;
  static constexpr int WS_BYTES = BN * 4;
  static constexpr int STAGE = A_BYTES + W_BYTES + AS_BYTES + WS_BYTES;
  static constexpr int COPIES = FM + FN + 2;  // per wave per stage
  static constexpr int EPI_WAVE = (32 * FM) * (64 * FN);  // bf16 outputs of a wave tile
  static_assert(FN >= 2 && FN <= 4 && FM >= 2 && FM <= 4, "one scale copy per wave");
  static_assert((DEPTH - 2) * COPIES < 64 && DEPTH >= 2, "load counter range");
  static_assert(DEPTH * STAGE + 4 * (BM + BN) <= 160 * 1024, "LDS");
  static_assert(4 * EPI_WAVE <= DEPTH * STAGE, "epilogue staging");
};

struct F16Args {
  const uint8_t* a_codes;
  const uint16_t* a_scales;
  const uint8_t* wcodes;
  const uint16_t* wscales;
  int64_t M, K2, KB, NG, m0, g0;
};

// Copy K-step ks (blocks 2 ks, 2 ks + 1) into stage buffer dst: FM + FN
// 16-byte copies and one 4-byte copy of each scale kind per wave.  Rows
// beyond M and groups beyond N/16 read clamped valid addresses; they feed
// only outputs that are not stored.
template <int FN, int FM, int DEPTH>
__device__ __forceinline__ void f16_issue(const F16Args& t, int64_t ks, I4_LDS uint8_t* dst, int wave,
                                          int lane) {
  using C = F16Cfg<FN, FM, DEPTH>;
#pragma unroll
  for (int x = 0; x < FM; ++x) {
    const int k = wave * FM + x, f = k >> 1, b = k & 1;
    int64_t row = t.m0 + 32 * f + (lane & 31);
    row = row < t.M ? row : t.M - 1;
    __builtin_amdgcn_global_load_lds(t.a_codes + row * t.K2 + (2 * ks + b) * 32 + 16 * (lane >> 5),
                                     dst + f * 2048 + b * 1024, 16, 0, 0);
  }
  I4_LDS uint8_t* wdst = dst + C::A_BYTES;
#pragma unroll
  for (int x = 0; x < FN; ++x) {
    const int k = wave * FN + x, p = k >> 1, b = k & 1;
    int64_t g = t.g0 + 2 * p + ((lane >> 3) & 1);
    g = g < t.NG ? g : t.NG - 1;
    __builtin_amdgcn_global_load_lds(t.wcodes + (g * t.KB + 2 * ks + b) * 512 + 16 * (lane & 7) + 128 * (lane >> 4),
                                     wdst + p * 2048 + b * 1024, 16, 0, 0);
  }
  I4_LDS uint8_t* asdst = wdst + C::W_BYTES;
  if (lane < C::BM / 4) {
    int64_t row = t.m0 + wave * (C::BM / 4) + lane;
    row = row < t.M ? row : t.M - 1;
    __builtin_amdgcn_global_load_lds(t.a_scales + row * t.KB + 2 * ks, asdst + wave * C::BM, 4, 0, 0);
  }
  I4_LDS uint8_t* wsdst = asdst + C::AS_BYTES;
  if (lane < C::BN / 4) {
    const int d = wave * (C::BN / 4) + lane;
    int64_t g = t.g0 + d / 16;
    g = g < t.NG ? g : t.NG - 1;
    __builtin_amdgcn_global_load_lds(t.wscales + (g * t.KB + 2 * ks) * 16 + 2 * (d & 15), wsdst + wave * C::BN, 4,
                                     0, 0);
  }
}

__device__ __forceinline__ constexpr int f16_wait_encoding(int v) {
  // s_waitcnt: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8] = 0, vmcnt[5:4] at [15:14]
  return (v & 15) | (7 << 4) | (((v >> 4) & 3) << 14);
}

// Wait until at most `after` stages of C copies are in flight for this wave
// and its LDS reads have completed, then barrier: the stage is in LDS for
// every wave, and the buffer read in the previous step is free.
template <int C, int DEPTH>
__device__ __forceinline__ void f16_stage_ready(int after) {
  switch (after) {
    case 0: __builtin_amdgcn_s_waitcnt(f16_wait_encoding(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(f16_wait_encoding(C)); break;
    case 2: __builtin_amdgcn_s_waitcnt(f16_wait_encoding(2 * C)); break;
    case 3: __builtin_amdgcn_s_waitcnt(f16_wait_encoding(3 * C)); break;
    default: __builtin_amdgcn_s_waitcnt(f16_wait_encoding(4 * C)); break;
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int FN, int FM, int DEPTH>
__device__ __forceinline__ void f16_step(const I4_LDS uint8_t* __restrict__ st, int wn, int wm, int lane,
                                         const int (&sha)[FM], const int (&shw)[FN],
                                         i4v16f (&acc)[FN][FM]) {
  using C = F16Cfg<FN, FM, DEPTH>;
  const int R = lane & 31, h = lane >> 5;
  const I4_LDS uint8_t* A = st;
  const I4_LDS uint8_t* W = st + C::A_BYTES;
  const I4_LDS uint8_t* AS = W + C::W_BYTES;
  const I4_LDS uint8_t* WS = AS + C::AS_BYTES;
  uint32_t asw[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j)
    asw[j] = *reinterpret_cast<const I4_LDS uint32_t*>(AS + 4 * (32 * (wm * FM + j) + R));
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    i4u32x4 af[FM], wf[FN];
    F16Scale sa[FM], sw[FN];
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      af[j] = *reinterpret_cast<const I4_LDS i4u32x4*>(A + (wm * FM + j) * 2048 + b * 1024 + h * 512 + 16 * R);
      sa[j] = f16_scale((asw[j] >> (16 * b)) & 0xFFFFu, sha[j]);
    }
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int p = wn * FN + i;
      const I4_LDS uint8_t* wp = W + p * 2048 + b * 1024 + h * 512 + 8 * R;
      const i4u32x2 lo = *reinterpret_cast<const I4_LDS i4u32x2*>(wp);
      const i4u32x2 hi = *reinterpret_cast<const I4_LDS i4u32x2*>(wp + 256);
      wf[i] = i4u32x4{lo.x, lo.y, hi.x, hi.y};
      const uint32_t bits =
          *reinterpret_cast<const I4_LDS uint16_t*>(WS + (2 * p + (R >> 4)) * 64 + b * 32 + 2 * (R & 15));
      sw[i] = f16_scale(bits, shw[i]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      i4v8h ah[FM];
#pragma unroll
      for (int j = 0; j < FM; ++j) ah[j] = expand8(af[j][t], sa[j]);
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const i4v8h wh = expand8(wf[i][t], sw[i]);
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wh, ah[j], acc[i][j], 0, 0, 0);
      }
    }
  }
}

// The same K-step for a tile whose rows or columns hold scales more than 25
// binades apart (or subnormal or non-finite ones), where one power of two
// per row and column cannot keep every expanded value in fp16's normal
// range: the operands are code x scale in fp32 (exact for any scale, 11
// significant bits) and the fp32 MFMA (32 x 32 x 2) multiplies them, each
// product exact (22 bits), into the same accumulators.  Sixteen times the
// MFMA time of the fp16 path; it serves only such tiles.  MFMA c of a block
// takes code c of each lane's 32 (K 32 (l / 32) + c), both operands alike.
template <int FN, int FM, int DEPTH>
__device__ __forceinline__ void f16_step_wide(const I4_LDS uint8_t* __restrict__ st, int wn, int wm, int lane,
                                              i4v16f (&acc)[FN][FM]) {
  using C = F16Cfg<FN, FM, DEPTH>;
  const int R = lane & 31, h = lane >> 5;
  const I4_LDS uint8_t* A = st;
  const I4_LDS uint8_t* W = st + C::A_BYTES;
  const I4_LDS uint8_t* AS = W + C::W_BYTES;
  const I4_LDS uint8_t* WS = AS + C::AS_BYTES;
  for (int b = 0; b < 2; ++b) {
    i4u32x4 af[FM], wf[FN];
    float sa[FM], sw[FN];
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      af[j] = *reinterpret_cast<const I4_LDS i4u32x4*>(A + (wm * FM + j) * 2048 + b * 1024 + h * 512 + 16 * R);
      const uint32_t asw = *reinterpret_cast<const I4_LDS uint32_t*>(AS + 4 * (32 * (wm * FM + j) + R));
      sa[j] = bf16_bits_to_f32((asw >> (16 * b)) & 0xFFFFu);
    }
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int p = wn * FN + i;
      const I4_LDS uint8_t* wp = W + p * 2048 + b * 1024 + h * 512 + 8 * R;
      const i4u32x2 lo = *reinterpret_cast<const I4_LDS i4u32x2*>(wp);
      const i4u32x2 hi = *reinterpret_cast<const I4_LDS i4u32x2*>(wp + 256);
      wf[i] = i4u32x4{lo.x, lo.y, hi.x, hi.y};
      sw[i] = bf16_bits_to_f32(
          *reinterpret_cast<const I4_LDS uint16_t*>(WS + (2 * p + (R >> 4)) * 64 + b * 32 + 2 * (R & 15)));
    }
    for (int c = 0; c < 32; ++c) {
      const int d = c >> 3, sh = 28 - 4 * (c & 7);
      float av[FM], wv[FN];
#pragma unroll
      for (int j = 0; j < FM; ++j) av[j] = float(int(af[j][d] << sh) >> 28) * sa[j];
#pragma unroll
      for (int i = 0; i < FN; ++i) wv[i] = float(int(wf[i][d] << sh) >> 28) * sw[i];
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(wv[i], av[j], acc[i][j], 0, 0, 0);
    }
  }
}

// Running range of the exponent fields (bits 7..14, kept in place) of BF16
// scales: the largest over all, the smallest over the nonzero ones.  A
// nonzero scale with a zero field (subnormal) enters the minimum as 0.
__device__ __forceinline__ void exp_range1(uint32_t& mx, uint32_t& mn, uint32_t bits) {
  const uint32_t e = bits & 0x7F80u;
  mx = mx > e ? mx : e;
  const uint32_t f = (bits & 0x7FFFu) ? e : 0xFFFFu;
  mn = mn < f ? mn : f;
}

__device__ __forceinline__ void exp_range2(uint32_t& mx, uint32_t& mn, uint32_t w) {
  exp_range1(mx, mn, w & 0xFFFFu);
  exp_range1(mx, mn, w >> 16);
}

// Whether one power of two cannot hold the row's (column's) scales in the
// exact window: nonzero scales more than 25 binades apart, a subnormal one,
// or a non-finite one.
__device__ __forceinline__ bool exp_wide(uint32_t mx, uint32_t mn) {
  if (mn == 0xFFFFu) return false;  // all scales zero
  return mx == 0x7F80u || mn == 0u || (mx >> 7) - (mn >> 7) > 25;
}

template <int FN, int FM, int DEPTH>
__global__ void __launch_bounds__(256, 1)
gemm_int4g64_f16_kernel(const uint8_t* __restrict__ a_codes, const uint16_t* __restrict__ a_scales,
                        const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N,
                        int64_t K, int tiles_m, int tiles_n, int per_xcd) {
  if (!blob_header_ok(blob, 3, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  using C = F16Cfg<FN, FM, DEPTH>;
  // tile order: each XCD walks a contiguous range of an order through
  // blocks of CW column tiles (down the rows of a block, CW wide), so the 32
  // workgroups an XCD runs at once cover CW column tiles x 32 / CW row tiles;
  // CW = 4 for the 256 (n) x 128 (m) tile makes that 1024 x 1024 outputs,
  // whose weight and activation rows are fetched in equal shares
  constexpr int CW = C::BN > C::BM ? 4 : 8;
  const int o = int(blockIdx.x % 8) * per_xcd + int(blockIdx.x / 8);
  if (o >= tiles_m * tiles_n) return;
  const int nb = o / (CW * tiles_m), ob = o - nb * CW * tiles_m;
  const int nw = tiles_n - CW * nb < CW ? tiles_n - CW * nb : CW;
  const int tm = ob / nw, tn = CW * nb + ob % nw;
  const I4Layout L = i4_layout(N, K);
  F16Args t;
  t.a_codes = a_codes;
  t.a_scales = a_scales;
  t.wcodes = blob + L.code_off;
  t.wscales = reinterpret_cast<const uint16_t*>(blob + L.scale_off);
  t.M = M;
  t.K2 = K / 2;
  t.KB = L.KB;
  t.NG = L.NG;
  t.m0 = int64_t(tm) * C::BM;
  t.g0 = int64_t(tn) * (C::BN / 16);

  __shared__ __attribute__((aligned(1024))) uint8_t smem[DEPTH * C::STAGE];
  __shared__ __attribute__((aligned(16))) int ea_s[C::BM];
  __shared__ __attribute__((aligned(16))) int ew_s[C::BN];
  __shared__ int wide_s;
  I4_LDS uint8_t* ring = (I4_LDS uint8_t*)smem;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t KS = K / 128;

#pragma unroll
  for (int s = 0; s < DEPTH - 1; ++s)
    if (s < KS) f16_issue<FN, FM, DEPTH>(t, s, ring + s * C::STAGE, wave, lane);

  // largest exponent field of each row's and column's scales (over all of K),
  // and whether any row or column needs the per-block scaling
  if (tid == 0) wide_s = 0;
  __syncthreads();
  {
    constexpr int TPR = 256 / C::BM;
    const int rl = tid / TPR, sub = tid % TPR;
    int64_t row = t.m0 + rl;
    row = row < M ? row : M - 1;
    const uint16_t* s = a_scales + row * t.KB;
    uint32_t mx = 0, mn = 0xFFFFu;
    if (t.KB % 8 == 0 && (reinterpret_cast<uintptr_t>(a_scales) & 15) == 0) {
      for (int64_t c = sub; c < t.KB / 8; c += TPR) {
        const uint4 v = reinterpret_cast<const uint4*>(s)[c];
        exp_range2(mx, mn, v.x);
        exp_range2(mx, mn, v.y);
        exp_range2(mx, mn, v.z);
        exp_range2(mx, mn, v.w);
      }
    } else {
      for (int64_t b = sub; b < t.KB; b += TPR) exp_range1(mx, mn, s[b]);
    }
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) {
      const uint32_t y = uint32_t(__shfl_xor(int(mx), off));
      const uint32_t z = uint32_t(__shfl_xor(int(mn), off));
      mx = mx > y ? mx : y;
      mn = mn < z ? mn : z;
    }
    if (sub == 0) {
      ea_s[rl] = int(mx >> 7);
      if (exp_wide(mx, mn)) wide_s = 1;
    }
  }
  {
    constexpr int TPO = 2048 / C::BN;  // threads per 8 columns
    const int oc = tid / TPO, sub = tid % TPO;
    int64_t g = t.g0 + (oc >> 1);
    g = g < t.NG ? g : t.NG - 1;
    const uint4* s = reinterpret_cast<const uint4*>(t.wscales) + g * t.KB * 2 + (oc & 1);
    uint32_t mx[8], mn[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      mx[c] = 0u;
      mn[c] = 0xFFFFu;
    }
    for (int64_t b = sub; b < t.KB; b += TPO) {
      const uint4 v = s[2 * b];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        exp_range1(mx[2 * d], mn[2 * d], w[d] & 0xFFFFu);
        exp_range1(mx[2 * d + 1], mn[2 * d + 1], w[d] >> 16);
      }
    }
#pragma unroll
    for (int off = 1; off < TPO; off <<= 1)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t y = uint32_t(__shfl_xor(int(mx[c]), off));
        const uint32_t z = uint32_t(__shfl_xor(int(mn[c]), off));
        mx[c] = mx[c] > y ? mx[c] : y;
        mn[c] = mn[c] < z ? mn[c] : z;
      }
    if (sub == 0) {
      bool wide = false;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        ew_s[8 * oc + c] = int(mx[c] >> 7);
        wide = wide || exp_wide(mx[c], mn[c]);
      }
      if (wide) wide_s = 1;
    }
  }
  __syncthreads();
  const bool wide_tile = wide_s != 0;

  const int wn = wave & 1, wm = wave >> 1, R = lane & 31, h = lane >> 5;
  int sha[FM], shw[FN];
#pragma unroll
  for (int j = 0; j < FM; ++j) sha[j] = 147 - ea_s[32 * (wm * FM + j) + R];
#pragma unroll
  for (int i = 0; i < FN; ++i) shw[i] = 147 - ew_s[32 * (wn * FN + i) + R];

  i4v16f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  if (!wide_tile) {
    for (int64_t s = 0; s < KS; ++s) {
      const int64_t after = KS - 1 - s < DEPTH - 2 ? KS - 1 - s : DEPTH - 2;
      f16_stage_ready<C::COPIES, DEPTH>(int(after));
      const int64_t nx = s + DEPTH - 1;
      if (nx < KS) f16_issue<FN, FM, DEPTH>(t, nx, ring + (nx % DEPTH) * C::STAGE, wave, lane);
      f16_step<FN, FM, DEPTH>(ring + (s % DEPTH) * C::STAGE, wn, wm, lane, sha, shw, acc);
    }
  } else {
    for (int64_t s = 0; s < KS; ++s) {
      const int64_t after = KS - 1 - s < DEPTH - 2 ? KS - 1 - s : DEPTH - 2;
      f16_stage_ready<C::COPIES, DEPTH>(int(after));
      const int64_t nx = s + DEPTH - 1;
      if (nx < KS) f16_issue<FN, FM, DEPTH>(t, nx, ring + (nx % DEPTH) * C::STAGE, wave, lane);
      f16_step_wide<FN, FM, DEPTH>(ring + (s % DEPTH) * C::STAGE, wn, wm, lane, acc);
    }
  }

  // epilogue: y = acc * 2^(ea + ew - 276) * r, rounded to BF16, staged
  // through LDS per wave (rows of 32 FN outputs in 16-byte chunks, chunk
  // position XOR-swizzled by row) and stored as whole 16-byte chunks
  __builtin_amdgcn_s_waitcnt(f16_wait_encoding(0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  const float* __restrict__ r = reinterpret_cast<const float*>(blob + L.r_off);
  constexpr int CH = 4 * FN, ROWB = 64 * FN;
  I4_LDS uint8_t* ep = ring + wave * C::EPI_WAVE;
  const int64_t nbase = t.g0 * 16 + wn * 32 * FN, mbase = t.m0 + wm * 32 * FM;
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nl = 32 * i + 8 * q + 4 * h;  // within the wave tile
      int64_t n = nbase + nl;
      n = n < N ? n : N - 4;
      const float4 r4 = *reinterpret_cast<const float4*>(r + n);
      const v4i ew4 = *reinterpret_cast<const v4i*>(&ew_s[32 * wn * FN + nl]);
      const float rr[4] = {r4.x, r4.y, r4.z, r4.w};
      const int ew[4] = {ew4[0], ew4[1], ew4[2], ew4[3]};
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int ml = 32 * j + R;
        const int ea = ea_s[32 * wm * FM + ml] - 276;
        uint16_t o4[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          bf16_round_f32((wide_tile ? acc[i][j][4 * q + v] : ldexpf(acc[i][j][4 * q + v], ea + ew[v])) * rr[v],
                         &o4[v]);
        const int chunk = 4 * i + q;
        *reinterpret_cast<I4_LDS i4u32x2*>(ep + ml * ROWB + ((chunk ^ (ml % CH)) * 16) + 8 * h) =
            i4u32x2{uint32_t(o4[0]) | (uint32_t(o4[1]) << 16), uint32_t(o4[2]) | (uint32_t(o4[3]) << 16)};
      }
    }
  __builtin_amdgcn_s_waitcnt(f16_wait_encoding(0));
  asm volatile("" ::: "memory");
#pragma unroll
  for (int qq = 0; qq < 32 * FM * CH / 64; ++qq) {
    const int idx = qq * 64 + lane;
    const int row = idx / CH, chunk = idx % CH;
    const i4u32x4 v = *reinterpret_cast<const I4_LDS i4u32x4*>(ep + row * ROWB + ((chunk ^ (row % CH)) * 16));
    const int64_t m = mbase + row, n = nbase + 8 * chunk;
    if (m < M && n < N) *reinterpret_cast<i4u32x4*>(Y + m * N + n) = v;
  }
}

unsigned grid_for(int64_t work) {
  const int64_t blocks = (work + 255) / 256;
  return unsigned(blocks < (int64_t(1) << 20) ? blocks : (int64_t(1) << 20));
}


// The fp16 kernel takes whole 128-wide K-steps; other K run the integer tile
// kernel.  (Its 16-byte copies and stores need the operand alignment the C
// ABI already requires: 16 bytes for codes, scales and Y, 256 for the blob.)
bool f16_eligible(int64_t K) { return K % 128 == 0; }

int64_t f16_rounds(int64_t M, int64_t N, int64_t bn, int64_t bm) {
  const int64_t tiles = (N + bn - 1) / bn * ((M + bm - 1) / bm);
  return (tiles + 255) / 256;
}

template <int FN, int FM, int DEPTH>
hipError_t launch_int4g64_f16(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint16_t* as,
                              const uint8_t* bl, uint16_t* y, hipStream_t stream) {
  using C = F16Cfg<FN, FM, DEPTH>;
  const int64_t tiles_n = (N + C::BN - 1) / C::BN, tiles_m = (M + C::BM - 1) / C::BM;
  if (tiles_n * tiles_m >= (int64_t(1) << 30)) return hipErrorInvalidValue;
  const int tiles = int(tiles_n * tiles_m), per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL((gemm_int4g64_f16_kernel<FN, FM, DEPTH>), dim3(unsigned(8 * per_xcd)), dim3(256), 0,
                     stream, ac, as, bl, y, M, N, K, int(tiles_m), int(tiles_n), per_xcd);
  return hipGetLastError();
}

}  // namespace

size_t int4g64_packed_weight_bytes(int64_t N, int64_t K) { return size_t(i4_layout(N, K).total); }

hipError_t launch_quantize_int4g64(int64_t M, int64_t K, const void* X, const float* c,
                                   void* codes, void* scales, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int64_t total8 = M * K / 8;
  hipLaunchKernelGGL(quantize_int4g64_kernel, dim3(grid_for(total8)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(X), c, K, total8, static_cast<uint32_t*>(codes),
                     static_cast<uint16_t*>(scales));
  return hipGetLastError();
}

hipError_t launch_pack_int4g64(int64_t N, int64_t K, const void* codes, const void* scales,
                               const float* r, void* blob, hipStream_t stream) {
  hipLaunchKernelGGL(pack_int4g64_header_kernel, dim3(1), dim3(1), 0, stream, N, K,
                     static_cast<uint8_t*>(blob));
  const int64_t work = N * K / 16;
  hipLaunchKernelGGL(pack_int4g64_kernel, dim3(grid_for(work)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(codes), static_cast<const uint16_t*>(scales), r,
                     N, K, static_cast<uint8_t*>(blob), 0, nullptr);
  return hipGetLastError();
}

hipError_t launch_unpack_int4g64(int64_t N, int64_t K, const void* blob, void* codes, void* scales,
                                 float* r, float* t_w, hipStream_t stream) {
  const int64_t work = N * K / 16;
  hipLaunchKernelGGL(pack_int4g64_kernel, dim3(grid_for(work)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(codes), static_cast<const uint16_t*>(scales), r,
                     N, K, const_cast<uint8_t*>(static_cast<const uint8_t*>(blob)), 1, t_w);
  return hipGetLastError();
}

hipError_t launch_linear_int4g64(int64_t M, int64_t N, int64_t K, const void* a_codes,
                                 const void* a_scales, const void* blob, void* Y,
                                 hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const auto* ac = static_cast<const uint8_t*>(a_codes);
  const auto* as = static_cast<const uint16_t*>(a_scales);
  const auto* bl = static_cast<const uint8_t*>(blob);
  auto* y = static_cast<uint16_t*>(Y);
  if (M <= 3 && K % 128 == 0) {
    // up to three rows: the dot-product kernel (one 16-column group per
    // workgroup); from four rows on the MFMA decode kernel is faster
    const dim3 grid(unsigned(N / 16)), block(512);
    if (M == 1)
      hipLaunchKernelGGL((gemm_int4g64_dot_kernel<8, 8, 1>), grid, block, 0, stream, ac, as, bl, y, M, N, K);
    else if (M == 2)
      hipLaunchKernelGGL((gemm_int4g64_dot_kernel<8, 8, 2>), grid, block, 0, stream, ac, as, bl, y, M, N, K);
    else
      hipLaunchKernelGGL((gemm_int4g64_dot_kernel<8, 8, 3>), grid, block, 0, stream, ac, as, bl, y, M, N, K);
  } else if (M <= 16) {
    constexpr int WAVES = 8, U = 8;
    hipLaunchKernelGGL((gemm_int4g64_decode_kernel<WAVES, U>), dim3(unsigned(N / 16)),
                       dim3(64 * WAVES), 0, stream, ac, as, bl, y, M, N, K);
  } else if (f16_eligible(K)) {
    // the tile with the least estimated time: rounds of 256 workgroups times
    // a K-step's cost (MFMA-bound for 256 x 256, expansion-bound below)
    const int64_t r44 = f16_rounds(M, N, 256, 256), r42 = f16_rounds(M, N, 256, 128),
                  r22 = f16_rounds(M, N, 128, 128);
    const int64_t c44 = r44 * 2048, c42 = r42 * 1320, c22 = r22 * 880;
    if (c44 <= c42 && c44 <= c22) return launch_int4g64_f16<4, 4, 4>(M, N, K, ac, as, bl, y, stream);
    if (c42 <= c22) return launch_int4g64_f16<4, 2, 5>(M, N, K, ac, as, bl, y, stream);
    return launch_int4g64_f16<2, 2, 6>(M, N, K, ac, as, bl, y, stream);
  } else {
    constexpr int FM = 4, FN = 4;
    const int64_t tiles_n = (N / 16 + 2 * FN - 1) / (2 * FN);
    const int64_t tiles_m = (M + 2 * FM * 16 - 1) / (2 * FM * 16);
    if (tiles_n * tiles_m >= (int64_t(1) << 30)) return hipErrorInvalidValue;
    const int tiles = int(tiles_n * tiles_m), per_xcd = (tiles + 7) / 8;
    hipLaunchKernelGGL((gemm_int4g64_tile_kernel<FM, FN>), dim3(unsigned(8 * per_xcd)), dim3(256), 0,
                       stream, ac, as, bl, y, M, N, K, int(tiles_m), int(tiles_n), per_xcd);
  }
  return hipGetLastError();
}

}  // namespace w4a4
