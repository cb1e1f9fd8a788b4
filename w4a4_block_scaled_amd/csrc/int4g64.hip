// INT4 with blocks of 64 and BF16 block scales: the packed deployment format
// of DualQuant (Appendix I, "Real packed W4A4 deployment": INT4, G = 64, BF16
// group scales, weights packed offline).  Section 3 gives the symmetric block
// quantizer (Delta = max|x| / q_max, q_max = 7 on the INT4 grid) and Section
// 4.2 the BF16 admissible set for INT4 scales.
//
// gfx950's block-scaled MFMAs take only E8M0 scales, so BF16 scales cannot
// ride on the matrix core.  A 64-block is exactly the K of
// V_MFMA_I32_16X16X64_I8: each block's codes go through one integer MFMA
// (exact) and the block's scale product is applied to that partial sum in
// fp32 before it joins the accumulator.
//
//   quantize  x~ = fp32(X) * c (one rounded fp32 multiply); per 64-block
//             Delta = BF16(amax / 7) rounded once from the fp64 quotient;
//             code = clip(RNE(x~ / Delta), -8, 7) from the fp64 quotient.
//   blob      256-byte header; codes in 512-byte fragment tiles, tile (g, b)
//             = rows 16 g .. +16, K 64 b .. +64, lane l owning the 8 canonical
//             bytes of row 16 g + l % 16 at K 64 b + 16 (l / 16) .. +16,
//             g-major; scales [N/16][K/64][16] BF16; r [N] fp32.
//   GEMM      int4 nibbles widened to int8 as (nibble << 4), which is 16 x the
//             signed code, so each MFMA block sum is 256 x the code dot
//             product; the 2^-8 goes into the weight scale (exact).
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

unsigned grid_for(int64_t work) {
  const int64_t blocks = (work + 255) / 256;
  return unsigned(blocks < (int64_t(1) << 20) ? blocks : (int64_t(1) << 20));
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
  if (M <= 16) {
    constexpr int WAVES = 8, U = 8;
    hipLaunchKernelGGL((gemm_int4g64_decode_kernel<WAVES, U>), dim3(unsigned(N / 16)),
                       dim3(64 * WAVES), 0, stream, ac, as, bl, y, M, N, K);
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
