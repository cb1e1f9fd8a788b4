// INT8 with blocks of 128 and BF16 block scales: the 8-bit integer W+A
// variant of DualQuant's Appendix G.2 (Table 9: INT8 weights and activations,
// groups of 128).  Section 3 gives the symmetric block quantizer (Delta =
// max|x| / q_max, q_max = 127 on the INT8 grid); the scales are BF16 as in
// the packed INT4 deployment of Appendix I.
//
// gfx950's block-scaled MFMAs take only E8M0 scales, so the BF16 scales are
// applied on the VALU, once per 128-block: each block's integer sum is exact
// (|sum| <= 128 * 128 * 128 = 2^21) and joins the fp32 accumulator times
// Delta_a * Delta_w (an exact product of two BF16 values).
//
//   quantize  x~ = fp32(X) * c (one rounded fp32 multiply); per 128-block
//             Delta = BF16(amax / 127) rounded once from the fp64 quotient;
//             code = clip(RNE(x~ / Delta), -128, 127) from the fp64 quotient.
//   blob      256-byte header; codes in 2 KiB tiles of 16 rows x 128 K, tile
//             (g, s) = rows 16 g .. +16, K 128 s .. +128, g-major; lane l owns
//             32 bytes of row 16 g + l % 16: K 128 s + 16 c .. +16 and
//             128 s + 64 + 16 c .. +16 with c = l / 16 (each half one operand
//             of v_mfma_i32_16x16x64_i8); scales [N/16][K/128][16] BF16;
//             r [N] fp32.
//   GEMM      M <= 3 while the rows fit 64 KiB of LDS: block dot products on
//             the VALU (v_dot4_i32_i8), the activation rows copied once per
//             workgroup into LDS; otherwise two integer MFMAs per block and
//             16 x 16 fragment pair, then the block's scale product: weight
//             streaming with one 16-feature group per workgroup for M <= 16,
//             tiles of 32 or 64 rows x 128 features above.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "kernels.h"

namespace w4a4 {
namespace {

constexpr int kFmt = 6;   // W4A4_INT8G128
constexpr int kG = 128;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef unsigned int u2 __attribute__((ext_vector_type(2)));

#define LDS __attribute__((address_space(3)))

__device__ inline float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Nearest BF16 (ties to even) to a non-negative finite double: 8 significant
// bits, spacing fixed at 2^-133 below 2^-126.  The result is a BF16 value, so
// its conversion to fp32 is exact and the top 16 bits are the pattern.
__device__ inline uint32_t bf16_rne_bits(double v) {
  if (v == 0.0) return 0;
  const int e = ilogb(v);                      // 2^e <= v < 2^(e+1)
  const int qe = e - 7 > -133 ? e - 7 : -133;  // exponent of one unit in the last place
  const double n = rint(ldexp(v, -qe));
  return __float_as_uint(float(ldexp(n, qe))) >> 16;
}

__device__ inline uint16_t bf16_rne_f32(float y) {
  const uint32_t u = __float_as_uint(y);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------------------- quantize --
// One thread per 8 consecutive elements (one 16-byte load, one 8-byte store);
// the 16 threads of a 128-block are 16 consecutive lanes and exchange the
// block maximum and the non-finite flag through lane shuffles.  Total threads
// M*K/8 is a multiple of 16, so a block's lanes are all inside or all
// outside the range.
__global__ void __launch_bounds__(256)
quantize_int8g128_kernel(const uint16_t* __restrict__ X, const float* __restrict__ c, int64_t K,
                         int64_t total8, uint2* __restrict__ codes, uint16_t* __restrict__ scales) {
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
      x[2 * j] = bf16_to_f32(w[j] & 0xFFFFu);
      x[2 * j + 1] = bf16_to_f32(w[j] >> 16);
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
    for (int s = 1; s < 16; s <<= 1) {
      amax = fmaxf(amax, __shfl_xor(amax, s));
      bad |= __shfl_xor(bad, s);
    }
    // amax / 127 in fp64, then one rounding to BF16: the fp64 quotient lands
    // on a BF16 midpoint only when the exact quotient is that midpoint
    uint32_t bits = bad ? 0u : bf16_rne_bits(double(amax) / 127.0);
    const double delta = double(bf16_to_f32(bits));
    uint32_t lo = 0, hi = 0;
    if (!bad && bits) {
      // x~ (24 bits) / Delta (8 bits) in fp64: a quotient that is not a
      // half-integer is much farther from one than the fp64 rounding, so
      // rint of it is the exact nearest-even decision
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        double q = rint(double(x[j]) / delta);
        q = q > 127.0 ? 127.0 : (q < -128.0 ? -128.0 : q);
        const uint32_t b = uint32_t(int(q)) & 0xFFu;
        if (j < 4) lo |= b << (8 * j);
        else hi |= b << (8 * (j - 4));
      }
    }
    if (bad) bits = 0x7FC0u;
    codes[t] = make_uint2(lo, hi);
    if ((threadIdx.x & 15) == 0) scales[t / 16] = uint16_t(bits);
  }
}

// -------------------------------------------------------------------- pack --
struct I8Layout {
  int64_t NG, KS, code_off, scale_off, r_off, total;
};

__host__ __device__ inline I8Layout i8_layout(int64_t N, int64_t K) {
  I8Layout L;
  L.NG = N / 16;
  L.KS = K / kG;
  L.code_off = 256;
  L.scale_off = align256(L.code_off + N * K);
  L.r_off = align256(L.scale_off + N * L.KS * 2);
  L.total = align256(L.r_off + N * 4);
  return L;
}

// One thread per 16-byte chunk of a tile: chunk t = tile * 128 + 2 * lane +
// half, tile = g * KS + s; also one per scale and per row scale.  unpack = 1
// copies the other way (canonical outputs that are NULL are skipped).
__global__ void __launch_bounds__(256)
pack_int8g128_kernel(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                     const float* __restrict__ r, int64_t N, int64_t K, uint8_t* __restrict__ blob,
                     int unpack, float* __restrict__ t_w) {
  const I8Layout L = i8_layout(N, K);
  const int64_t chunks = N * K / 16;
  const int64_t nscales = N * L.KS;
  const int64_t work = chunks > nscales ? chunks : nscales;
  for (int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x; t < work;
       t += int64_t(gridDim.x) * 256) {
    if (t < chunks) {
      const int64_t tile = t >> 7;
      const int lane = int((t >> 1) & 63), half = int(t & 1);
      const int64_t g = tile / L.KS, s = tile - g * L.KS;
      const int64_t src = (16 * g + (lane & 15)) * K + s * kG + 64 * half + 16 * (lane >> 4);
      uint4* packed = reinterpret_cast<uint4*>(blob + L.code_off) + t;
      uint4* canon = reinterpret_cast<uint4*>(const_cast<uint8_t*>(codes) + src);
      if (!unpack) *packed = *canon;
      else if (codes) *canon = *packed;
    }
    if (t < nscales) {
      const int64_t n = t / L.KS, s = t - n * L.KS;
      uint16_t* ps = reinterpret_cast<uint16_t*>(blob + L.scale_off) + ((n >> 4) * L.KS + s) * 16 + (n & 15);
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
__global__ void pack_int8g128_header_kernel(int64_t N, int64_t K, uint8_t* blob) {
  if (threadIdx.x != 0) return;
  const I8Layout L = i8_layout(N, K);
  BlobHeader* h = reinterpret_cast<BlobHeader*>(blob);
  const char m[8] = {'W', '4', 'A', '4', 'P', 'K', '0', '1'};
  for (int i = 0; i < 8; ++i) h->magic[i] = m[i];
  h->version = 1;
  h->format = kFmt;
  h->N = N;
  h->K = K;
  h->layout = 5;
  h->t_w = 1.0f;
  h->code_off = uint64_t(L.code_off);
  h->scale_off = uint64_t(L.scale_off);
  h->r_off = uint64_t(L.r_off);
  h->total = uint64_t(L.total);
  for (int i = 0; i < int(sizeof(h->pad)); ++i) h->pad[i] = 0;
}

// ------------------------------------------------------- dot-product GEMM --
// M = MD <= 3.  One workgroup per 16 output features (group ng = (b % 8) S +
// b / 8 for workgroup b, S groups per XCD); WAVES waves split the K-steps
// into contiguous ranges, each with the loads of U K-steps in flight (two
// 16-byte non-temporal loads of the lane's tile bytes and its row's BF16
// scale).  The MD activation rows (K bytes each) and their scales (K/128
// BF16 each) are copied once per workgroup into LDS.  Lane (n = l % 16, c =
// l / 16) takes v_dot4_i32_i8 products of its 32 bytes with the same K of
// each row (the block's integer part sum is exact), and adds it to the row's
// fp32 sum times Delta_w * Delta_a.  The four lanes of a feature are added by
// two lane exchanges, the waves in wave order through LDS.
template <int MD>
__host__ __device__ constexpr int64_t i8_dot_lds(int64_t K) {
  return MD * (K + 2 * (K / kG));
}

template <int WAVES, int U, int MD>
__global__ __launch_bounds__(64 * WAVES) void gemm_int8g128_dot_kernel(
    const uint8_t* __restrict__ a_codes, const uint16_t* __restrict__ a_scales,
    const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K) {
  if (!blob_header_ok(blob, kFmt, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  const I8Layout L = i8_layout(N, K);
  const int64_t F = L.NG, per_x = (F + 7) / 8;
  const int64_t ng = int64_t(blockIdx.x % 8) * per_x + blockIdx.x / 8;
  if (ng >= F) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane >> 4, n = lane & 15;
  const int64_t KS = L.KS;
  const int64_t per = (KS + WAVES - 1) / WAVES;
  const int64_t k_begin = wave * per;
  const int64_t k_end = k_begin + per < KS ? k_begin + per : KS;
  const u4* __restrict__ Wg = reinterpret_cast<const u4*>(blob + L.code_off) + (ng * KS * 64 + lane) * 2;
  const uint16_t* __restrict__ Sg = reinterpret_cast<const uint16_t*>(blob + L.scale_off) + ng * KS * 16 + n;
  const float* __restrict__ R = reinterpret_cast<const float*>(blob + L.r_off);

  // the first batch of weight loads goes out before the activation rows are
  // staged, so the staging's latency overlaps them
  u4 w0[U], w1[U];
  uint16_t ws[U];
  auto load_batch = [&](int64_t kb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      w0[u] = __builtin_nontemporal_load(&Wg[(kb + u) * 128]);
      w1[u] = __builtin_nontemporal_load(&Wg[(kb + u) * 128 + 1]);
      ws[u] = Sg[(kb + u) * 16];
    }
  };
  if (k_begin + U <= k_end) load_batch(k_begin);

  // LDS: MD rows of K code bytes, then MD rows of K/128 BF16 scales
  extern __shared__ __attribute__((aligned(16))) uint8_t i8_dyn[];
  for (int64_t d = tid; d < MD * (K / 16); d += 64 * WAVES)
    reinterpret_cast<u4*>(i8_dyn)[d] = reinterpret_cast<const u4*>(a_codes)[d];
  uint16_t* asc = reinterpret_cast<uint16_t*>(i8_dyn + MD * K);
  for (int64_t d = tid; d < MD * KS; d += 64 * WAVES) asc[d] = a_scales[d];
  __syncthreads();

  float acc[MD];
#pragma unroll
  for (int m = 0; m < MD; ++m) acc[m] = 0.f;
  auto step = [&](const u4& a_w, const u4& b_w, uint16_t sw, int64_t ks) {
    const float dw = bf16_to_f32(sw);
#pragma unroll
    for (int m = 0; m < MD; ++m) {
      const uint8_t* row = i8_dyn + m * K + ks * kG + 16 * c;
      const u4 alo = *reinterpret_cast<const u4*>(row);
      const u4 ahi = *reinterpret_cast<const u4*>(row + 64);
      int dl = 0, dh = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dl = __builtin_amdgcn_sdot4(int(a_w[i]), int(alo[i]), dl, false);
        dh = __builtin_amdgcn_sdot4(int(b_w[i]), int(ahi[i]), dh, false);
      }
      acc[m] = fmaf(float(dl + dh), dw * bf16_to_f32(asc[m * KS + ks]), acc[m]);
    }
  };
  int64_t k0 = k_begin;
  for (; k0 + U <= k_end; k0 += U) {
    if (k0 != k_begin) load_batch(k0);
#pragma unroll
    for (int u = 0; u < U; ++u) step(w0[u], w1[u], ws[u], k0 + u);
  }
  for (; k0 < k_end; ++k0) step(Wg[k0 * 128], Wg[k0 * 128 + 1], Sg[k0 * 16], k0);

#pragma unroll
  for (int m = 0; m < MD; ++m) {
    acc[m] += __shfl_xor(acc[m], 16);
    acc[m] += __shfl_xor(acc[m], 32);
  }
  __shared__ float red[WAVES > 1 ? WAVES - 1 : 1][MD][16];
  if (wave != 0 && c == 0) {
#pragma unroll
    for (int m = 0; m < MD; ++m) red[wave - 1][m][n] = acc[m];
  }
  __syncthreads();
  if (wave != 0 || c != 0) return;
  const float rn = R[ng * 16 + n];
#pragma unroll
  for (int m = 0; m < MD; ++m) {
    float y = acc[m];
#pragma unroll
    for (int w = 0; w < WAVES - 1; ++w) y += red[w][m][n];
    Y[int64_t(m) * N + ng * 16 + n] = bf16_rne_f32(y * rn);
  }
}

template <int WAVES, int U, int MD>
hipError_t launch_i8_dot_md(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint16_t* as,
                            const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_int8g128_dot_kernel<WAVES, U, MD>), dim3(unsigned((N / 16 + 7) / 8 * 8)),
                     dim3(64 * WAVES), size_t(i8_dot_lds<MD>(K)), stream, ac, as, blob, Y, M, N, K);
  return hipGetLastError();
}

template <int WAVES, int U>
hipError_t launch_i8_dot(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint16_t* as,
                         const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  if (M == 1) return launch_i8_dot_md<WAVES, U, 1>(M, N, K, ac, as, blob, Y, stream);
  if (M == 2) return launch_i8_dot_md<WAVES, U, 2>(M, N, K, ac, as, blob, Y, stream);
  return launch_i8_dot_md<WAVES, U, 3>(M, N, K, ac, as, blob, Y, stream);
}

// -------------------------------------------------------------- tile GEMM --
// The weight fragment is the MFMA's row operand and the activation fragment
// its column operand, so lane l holds the outputs (activation row l % 16,
// weight columns 4 (l / 16) .. +4): one activation scale per fragment, the
// four weight scales in one 8-byte load and the four outputs in one 8-byte
// store.  Per 128-block and fragment pair, two v_mfma_i32_16x16x64_i8 (the
// lane's two 16-byte halves, the same K on both operands) give the block's
// exact integer sums; acc[v] += sum[v] * Delta_a * Delta_w[v].
__device__ inline v4i mfma_i8(u4 w, u4 a, v4i acc) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, w), __builtin_bit_cast(v4i, a),
                                               acc, 0, 0, 0);
}

__device__ inline void store4(uint16_t* y, const float* acc, const float* rn) {
  uint16_t o[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) o[v] = bf16_rne_f32(acc[v] * rn[v]);
  *reinterpret_cast<uint2*>(y) = make_uint2(uint32_t(o[0]) | (uint32_t(o[1]) << 16),
                                            uint32_t(o[2]) | (uint32_t(o[3]) << 16));
}

// ------------------------------------------------------------ decode GEMM --
// M <= 16: one workgroup per 16 output features (as the dot kernel), WAVES
// waves splitting the K-steps into contiguous ranges, each issuing the loads
// of up to U K-steps at once: the lane's 32 weight bytes (the MFMA's row
// operand, feature l % 16), the four weight scales of its outputs, and the 32
// bytes of activation row l % 16 at the same K (the column operand; lanes of
// rows >= M load nothing and hold zeros).  Per K-step two
// v_mfma_i32_16x16x64_i8 give the block's exact integer sums for (feature
// 4 (l / 16) + v, row l % 16), which join the fp32 sums times Delta_a *
// Delta_w[v].  Partial sums meet in LDS in wave order; wave 0 applies r and
// stores four features per lane.
template <int WAVES, int U>
__global__ __launch_bounds__(64 * WAVES) void gemm_int8g128_decode_kernel(
    const uint8_t* __restrict__ a_codes, const uint16_t* __restrict__ a_scales,
    const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K) {
  if (!blob_header_ok(blob, kFmt, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  static_assert(U <= 8, "load batch");
  const I8Layout L = i8_layout(N, K);
  const int64_t F = L.NG, per_x = (F + 7) / 8;
  const int64_t ng = int64_t(blockIdx.x % 8) * per_x + blockIdx.x / 8;
  if (ng >= F) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane >> 4;
  const int64_t m = lane & 15;
  const bool mvalid = m < M;
  const int64_t KS = L.KS;
  const int64_t per = (KS + WAVES - 1) / WAVES;
  const int64_t k_begin = wave * per;
  const int64_t k_end = k_begin + per < KS ? k_begin + per : KS;
  const u4* __restrict__ Wg = reinterpret_cast<const u4*>(blob + L.code_off) + (ng * KS * 64 + lane) * 2;
  const uint16_t* __restrict__ Sg =
      reinterpret_cast<const uint16_t*>(blob + L.scale_off) + ng * KS * 16 + 4 * c;
  const uint8_t* __restrict__ arow = a_codes + (mvalid ? m : 0) * K + 16 * c;
  const uint16_t* __restrict__ srow = a_scales + (mvalid ? m : 0) * KS;

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = k_begin; k0 < k_end; k0 += U) {
    u4 w0[U], w1[U], a0[U], a1[U];
    uint2 sw[U];
    uint16_t sa[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t ks = k0 + u;
      const bool ok = ks < k_end;
      const int64_t kc = ok ? ks : k_end - 1;  // clamped: loads stay in range
      const u4 x0 = __builtin_nontemporal_load(&Wg[kc * 128]);
      const u4 x1 = __builtin_nontemporal_load(&Wg[kc * 128 + 1]);
      u4 y0 = {0u, 0u, 0u, 0u}, y1 = {0u, 0u, 0u, 0u};
      if (mvalid) {
        y0 = *reinterpret_cast<const u4*>(arow + kc * kG);
        y1 = *reinterpret_cast<const u4*>(arow + kc * kG + 64);
      }
      const u4 z = {0u, 0u, 0u, 0u};
      w0[u] = ok ? x0 : z;
      w1[u] = ok ? x1 : z;
      a0[u] = ok ? y0 : z;
      a1[u] = ok ? y1 : z;
      sw[u] = *reinterpret_cast<const uint2*>(Sg + kc * 16);
      sa[u] = mvalid ? srow[kc] : uint16_t(0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const v4i zero = {0, 0, 0, 0};
      v4i S = mfma_i8(w0[u], a0[u], zero);
      S = mfma_i8(w1[u], a1[u], S);
      const float da = bf16_to_f32(sa[u]);
      const float dw[4] = {bf16_to_f32(sw[u].x & 0xFFFFu), bf16_to_f32(sw[u].x >> 16),
                           bf16_to_f32(sw[u].y & 0xFFFFu), bf16_to_f32(sw[u].y >> 16)};
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] = fmaf(float(S[v]), da * dw[v], acc[v]);
    }
  }

  __shared__ float red[WAVES > 1 ? WAVES - 1 : 1][4][64];
  if (wave != 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave - 1][v][lane] = acc[v];
  }
  __syncthreads();
  if (wave != 0 || !mvalid) return;
#pragma unroll
  for (int w = 0; w < WAVES - 1; ++w)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] += red[w][v][lane];
  const int64_t n = ng * 16 + 4 * c;
  const float* R = reinterpret_cast<const float*>(blob + L.r_off);
  const float4 r4 = *reinterpret_cast<const float4*>(R + n);
  const float rn[4] = {r4.x, r4.y, r4.z, r4.w};
  store4(Y + m * N + n, acc, rn);
}

template <int WAVES, int U>
hipError_t launch_i8_decode(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint16_t* as,
                            const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_int8g128_decode_kernel<WAVES, U>), dim3(unsigned((N / 16 + 7) / 8 * 8)),
                     dim3(64 * WAVES), 0, stream, ac, as, blob, Y, M, N, K);
  return hipGetLastError();
}

// 4 waves as 2 (M) x 2 (N); a wave owns FM x FN fragments of 16 x 16
// outputs, the workgroup (2 FM 16) x (2 FN 16).  Operands come straight from
// global memory, two blocks ahead of the one being multiplied (activation
// rows clamped to M - 1, weight row groups to NG - 1, so every load is in
// bounds); outputs outside M x N are not stored.  Workgroups are dealt to the
// 8 XCDs round-robin; workgroup b takes tile number (b % 8) per_xcd + b / 8
// of an order that runs through blocks of 8 x 8 tiles (8 column tiles wide,
// then down the rows), so the workgroups an XCD runs at once share their
// activation rows and weight groups in its L2.
template <int FM, int FN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
gemm_int8g128_tile_kernel(const uint8_t* __restrict__ a_codes, const uint16_t* __restrict__ a_scales,
                          const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M,
                          int64_t N, int64_t K, int tiles_m, int tiles_n, int per_xcd) {
  if (!blob_header_ok(blob, kFmt, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  const int o = int(blockIdx.x % 8) * per_xcd + int(blockIdx.x / 8);
  if (o >= tiles_m * tiles_n) return;
  const int nb = o / (8 * tiles_m), ob = o - nb * 8 * tiles_m;
  const int nw = tiles_n - 8 * nb < 8 ? tiles_n - 8 * nb : 8;  // width of this column block
  const int tm = ob / nw, tn = 8 * nb + ob % nw;
  const I8Layout L = i8_layout(N, K);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m0 = int64_t(tm) * (2 * FM * 16) + (wave >> 1) * (FM * 16);
  const int64_t g0 = int64_t(tn) * (2 * FN) + (wave & 1) * FN;
  const u4* wcodes = reinterpret_cast<const u4*>(blob + L.code_off) + 2 * lane;
  const uint16_t* wscales = reinterpret_cast<const uint16_t*>(blob + L.scale_off) + 4 * (lane >> 4);

  const uint8_t* arow[FM];
  const uint16_t* srow[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + i * 16 + (lane & 15);
    const int64_t mc = m < M ? m : M - 1;
    arow[i] = a_codes + mc * K + 16 * (lane >> 4);
    srow[i] = a_scales + mc * L.KS;
  }
  int64_t gbase[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) gbase[j] = (g0 + j < L.NG ? g0 + j : L.NG - 1) * L.KS;

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
    u4 a0[FM], a1[FM], w0[FN], w1[FN];
    uint2 sw[FN];
    uint16_t sa[FM];
  };
  auto load = [&](int64_t b, Ops& p) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      p.a0[i] = *reinterpret_cast<const u4*>(arow[i] + b * kG);
      p.a1[i] = *reinterpret_cast<const u4*>(arow[i] + b * kG + 64);
      p.sa[i] = srow[i][b];
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t tile = gbase[j] + b;
      p.w0[j] = wcodes[tile * 128];
      p.w1[j] = wcodes[tile * 128 + 1];
      p.sw[j] = *reinterpret_cast<const uint2*>(wscales + tile * 16);
    }
  };
  // Per pair of weight fragments: the first halves' MFMAs for every
  // activation fragment, then the second halves' (each adding to the sum of
  // its first), then the scaling, so that no sum is read right after the
  // MFMA that writes it.
  auto compute = [&](const Ops& p) {
    float sa[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) sa[i] = bf16_to_f32(p.sa[i]);
#pragma unroll
    for (int j0 = 0; j0 < FN; j0 += 2) {
      v4i S[2][FM];
      const v4i zero = {0, 0, 0, 0};
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int i = 0; i < FM; ++i) S[jj][i] = mfma_i8(p.w0[j0 + jj], p.a0[i], zero);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int i = 0; i < FM; ++i) S[jj][i] = mfma_i8(p.w1[j0 + jj], p.a1[i], S[jj][i]);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const uint2 w = p.sw[j0 + jj];
        const float sw[4] = {bf16_to_f32(w.x & 0xFFFFu), bf16_to_f32(w.x >> 16),
                             bf16_to_f32(w.y & 0xFFFFu), bf16_to_f32(w.y >> 16)};
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            acc[i][j0 + jj][v] = fmaf(float(S[jj][i][v]), sa[i] * sw[v], acc[i][j0 + jj][v]);
      }
    }
  };
  const int64_t last = L.KS - 1;
  Ops p0, p1;
  load(0, p0);
  load(last < 1 ? last : 1, p1);
  // the scheduling barriers keep each set's use (and so its load wait) after
  // the other set's loads have been issued
  for (int64_t b = 0; b < L.KS; b += 2) {
    compute(p0);
    load(b + 2 < last ? b + 2 : last, p0);
    __builtin_amdgcn_sched_barrier(0);
    if (b + 1 < L.KS) {
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
    const float rn[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t m = m0 + i * 16 + (lane & 15);
      if (m < M) store4(Y + m * N + n, acc[i][j], rn);
    }
  }
}

// ------------------------------------------------------- LDS-staged tile --
// (64 WM) (rows) x 128 (features) workgroup tiles, 2 WM waves as WM (rows)
// x 2 (features) of 64 x 64 (4 x 4 fragments); one 128-wide K-step (one
// block) per stage, DEPTH stages in a ring, copied global -> LDS with
// direct-to-LDS loads, so each operand byte crosses the L2 once per
// workgroup instead of once per wave.  WM = 2: 128-row tiles, one wave per
// SIMD; WM = 4: 256-row tiles, two waves per SIMD, so that one wave's VALU
// work (the scale products) runs while the other's MFMAs do.
//   A codes   64 WM rows x 128 B; 16-byte chunk j of row r at chunk position
//             8 r + (j ^ i8_swz(r)), so a fragment read (16 rows, one chunk
//             each) touches 16 different 16-byte bank groups;
//   W codes   8 tiles of 2 KiB: the first 16 bytes of every lane's 32 (the
//             operand of the block's first MFMA), then the second 16, so
//             that a fragment read is 64 consecutive 16-byte chunks;
//   A scales  64 WM dwords, the low half of dword r the K-step's BF16 scale
//             of row r (a two-byte direct-to-LDS copy fills one dword per
//             lane);
//   W scales  8 x 16 BF16 (the K-step's scales of each 16-feature group).
// Every wave issues the same number of copies per stage (4 activation, 8 /
// WM weight, 1 scale) and one stage per K-step (past the last K-step a copy
// of the last stage, into a slot that is not read again), so a stage is
// complete for a wave when its vmcnt has dropped to copies x (DEPTH - 2); a
// barrier then makes it complete for the workgroup, and also orders the
// reads of the slot a new stage overwrites before its copy.  All copies have
// landed before the epilogue.  Rows beyond M and groups beyond N/16 are read
// from clamped valid addresses; they only feed outputs that are never
// stored.
// chunk swizzle of the staged activation rows: the rows r and r + 8 of a
// 16-row fragment read land in different bank groups
__device__ __forceinline__ int i8_swz(int r) { return ((r & 7) + ((r >> 3) & 1)) & 7; }

template <int WM>
struct I8Lds {
  static constexpr int ROWS = 64 * WM, WAVES = 2 * WM;
  static constexpr int A = ROWS * 128, W = 8 * 2048, AS = ROWS * 4, WS = 8 * 32;
  static constexpr int STAGE = A + W + AS + WS;
  static constexpr int W_COPIES = 16 / WAVES;
  static constexpr int COPIES = 4 + W_COPIES + 1;
  static_assert(ROWS / 8 == 4 * WAVES && W_COPIES * WAVES == 16, "copy split");
};

__device__ __forceinline__ constexpr int i8_vmcnt(int v) {
  // s_waitcnt simm16 on gfx9: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]
  return (v & 15) | (7 << 4) | (15 << 8) | (((v >> 4) & 3) << 14);
}

template <int WM, int DEPTH>
__device__ __forceinline__ void i8_stage_ready() {
  static_assert(DEPTH >= 2 && (DEPTH - 2) * I8Lds<WM>::COPIES < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(i8_vmcnt((DEPTH - 2) * I8Lds<WM>::COPIES));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int WM>
__device__ __forceinline__ void i8_issue(const uint8_t* __restrict__ a_codes,
                                         const uint16_t* __restrict__ a_scales,
                                         const uint8_t* __restrict__ wc, const uint16_t* __restrict__ wsc,
                                         int64_t M, int64_t K, int64_t KS, int64_t NG, int64_t m0,
                                         int64_t g0, int64_t ks, LDS uint8_t* dst, int wave, int lane) {
  using C = I8Lds<WM>;
  // activation rows: copy f covers rows 8 f .. 8 f + 7; lane L fills chunk
  // position L % 8 of row L / 8 with the chunk that belongs there
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = wave * 4 + i;
    const int rr = 8 * f + (lane >> 3);
    int64_t row = m0 + rr;
    row = row < M ? row : M - 1;
    const int j = (lane & 7) ^ i8_swz(rr);
    __builtin_amdgcn_global_load_lds(a_codes + row * K + ks * kG + 16 * j, dst + f * 1024, 16, 0, 0);
  }
  LDS uint8_t* wdst = dst + C::A;
#pragma unroll
  for (int i = 0; i < C::W_COPIES; ++i) {
    const int f = wave * C::W_COPIES + i;  // 16-byte half (f % 2) of every lane's 32 bytes of tile f / 2
    int64_t g = g0 + f / 2;
    g = g < NG ? g : NG - 1;
    __builtin_amdgcn_global_load_lds(wc + (g * KS + ks) * 2048 + 32 * lane + 16 * (f & 1), wdst + f * 1024,
                                     16, 0, 0);
  }
  if (wave < WM) {
    // rows 64 wave + lane: one scale per lane, one dword per lane in LDS
    int64_t row = m0 + 64 * wave + lane;
    row = row < M ? row : M - 1;
    __builtin_amdgcn_global_load_lds(a_scales + row * KS + ks, dst + C::A + C::W + wave * 256, 2, 0, 0);
  } else {
    // the other waves copy the same 256 bytes of weight scales (same copy
    // count on every wave); lane L: two scales of group L / 8
    int64_t g = g0 + (lane >> 3);
    g = g < NG ? g : NG - 1;
    __builtin_amdgcn_global_load_lds(wsc + (g * KS + ks) * 16 + 2 * (lane & 7), dst + C::A + C::W + C::AS, 4,
                                     0, 0);
  }
}

template <int WM, int DEPTH>
__global__ __launch_bounds__(128 * WM, 1) void gemm_int8g128_lds_kernel(
    const uint8_t* __restrict__ a_codes, const uint16_t* __restrict__ a_scales,
    const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int tiles_m, int tiles_n, int per_xcd) {
  using C = I8Lds<WM>;
  if (!blob_header_ok(blob, kFmt, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  const int o = int(blockIdx.x % 8) * per_xcd + int(blockIdx.x / 8);
  if (o >= tiles_m * tiles_n) return;
  const int nb = o / (8 * tiles_m), ob = o - nb * 8 * tiles_m;
  const int nw = tiles_n - 8 * nb < 8 ? tiles_n - 8 * nb : 8;  // width of this column block
  const int tm = ob / nw, tn = 8 * nb + ob % nw;
  const I8Layout L = i8_layout(N, K);
  const int64_t m0 = int64_t(tm) * C::ROWS, g0 = int64_t(tn) * 8;
  const uint8_t* wc = blob + L.code_off;
  const uint16_t* wsc = reinterpret_cast<const uint16_t*>(blob + L.scale_off);

  __shared__ __attribute__((aligned(1024))) uint8_t smem[DEPTH * C::STAGE];
  LDS uint8_t* base = (LDS uint8_t*)smem;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int c = lane >> 4;

  float acc[4][4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.f;

  const int64_t KS = L.KS;
#pragma unroll
  for (int s = 0; s < DEPTH - 1; ++s)
    i8_issue<WM>(a_codes, a_scales, wc, wsc, M, K, KS, L.NG, m0, g0, s < KS ? s : KS - 1, base + s * C::STAGE,
                 wave, lane);
  for (int64_t s = 0; s < KS; ++s) {
    i8_stage_ready<WM, DEPTH>();
    i8_issue<WM>(a_codes, a_scales, wc, wsc, M, K, KS, L.NG, m0, g0, s + DEPTH - 1 < KS ? s + DEPTH - 1 : KS - 1,
                 base + ((s + DEPTH - 1) % DEPTH) * C::STAGE, wave, lane);
    const LDS uint8_t* st = base + (s % DEPTH) * C::STAGE;
    const LDS uint8_t* A = st;
    const LDS uint8_t* W = st + C::A;
    const LDS uint32_t* AS = reinterpret_cast<const LDS uint32_t*>(st + C::A + C::W);
    const LDS uint16_t* WS = reinterpret_cast<const LDS uint16_t*>(st + C::A + C::W + C::AS);
    u4 a0[4], a1[4];
    float sa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int R = 64 * wm + 16 * i + (lane & 15);
      a0[i] = *reinterpret_cast<const LDS u4*>(A + R * 128 + 16 * (c ^ i8_swz(R)));
      a1[i] = *reinterpret_cast<const LDS u4*>(A + R * 128 + 16 * ((4 + c) ^ i8_swz(R)));
      sa[i] = bf16_to_f32(AS[R] & 0xFFFFu);
    }
#pragma unroll
    for (int j0 = 0; j0 < 4; j0 += 2) {
      u4 w0[2], w1[2];
      u2 swb[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int T = 4 * wn + j0 + jj;
        w0[jj] = *reinterpret_cast<const LDS u4*>(W + T * 2048 + 16 * lane);
        w1[jj] = *reinterpret_cast<const LDS u4*>(W + T * 2048 + 1024 + 16 * lane);
        swb[jj] = *reinterpret_cast<const LDS u2*>(WS + T * 16 + 4 * c);
      }
      v4i S[2][4];
      const v4i zero = {0, 0, 0, 0};
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[jj][i] = mfma_i8(w0[jj], a0[i], zero);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[jj][i] = mfma_i8(w1[jj], a1[i], S[jj][i]);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const float sw[4] = {bf16_to_f32(swb[jj].x & 0xFFFFu), bf16_to_f32(swb[jj].x >> 16),
                             bf16_to_f32(swb[jj].y & 0xFFFFu), bf16_to_f32(swb[jj].y >> 16)};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            acc[i][j0 + jj][v] = fmaf(float(S[jj][i][v]), sa[i] * sw[v], acc[i][j0 + jj][v]);
      }
    }
  }

  // the copies issued past the last K-step land before the workgroup's LDS
  // is released
  __builtin_amdgcn_s_waitcnt(i8_vmcnt(0));
  const float* r = reinterpret_cast<const float*>(blob + L.r_off);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t g = g0 + 4 * wn + j;
    if (g >= L.NG) continue;
    const int64_t n = g * 16 + 4 * c;
    const float4 r4 = *reinterpret_cast<const float4*>(r + n);
    const float rn[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + 64 * wm + 16 * i + (lane & 15);
      if (m < M) store4(Y + m * N + n, acc[i][j], rn);
    }
  }
}

template <int WM, int DEPTH>
hipError_t launch_i8_lds(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint16_t* as,
                         const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  using C = I8Lds<WM>;
  static_assert(DEPTH * C::STAGE <= 160 * 1024, "LDS");
  const int64_t tiles_n = (N / 16 + 7) / 8;
  const int64_t tiles_m = (M + C::ROWS - 1) / C::ROWS;
  if (tiles_n * tiles_m >= (int64_t(1) << 30)) return hipErrorInvalidValue;
  const int tiles = int(tiles_n * tiles_m), per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL((gemm_int8g128_lds_kernel<WM, DEPTH>), dim3(unsigned(8 * per_xcd)), dim3(128 * WM), 0,
                     stream, ac, as, blob, Y, M, N, K, int(tiles_m), int(tiles_n), per_xcd);
  return hipGetLastError();
}

template <int FM, int FN>
hipError_t launch_i8_tile(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint16_t* as,
                          const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  const int64_t tiles_n = (N / 16 + 2 * FN - 1) / (2 * FN);
  const int64_t tiles_m = (M + 2 * FM * 16 - 1) / (2 * FM * 16);
  if (tiles_n * tiles_m >= (int64_t(1) << 30)) return hipErrorInvalidValue;
  const int tiles = int(tiles_n * tiles_m), per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL((gemm_int8g128_tile_kernel<FM, FN>), dim3(unsigned(8 * per_xcd)), dim3(256), 0,
                     stream, ac, as, blob, Y, M, N, K, int(tiles_m), int(tiles_n), per_xcd);
  return hipGetLastError();
}

}  // namespace

size_t int8g128_packed_weight_bytes(int64_t N, int64_t K) { return size_t(i8_layout(N, K).total); }

hipError_t launch_quantize_int8g128(int64_t M, int64_t K, const void* X, const float* c, void* codes,
                                    void* scales, hipStream_t stream) {
  const int64_t total8 = M * K / 8;
  if (total8 == 0) return hipSuccess;
  int64_t blocks = (total8 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(quantize_int8g128_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(X), c, K, total8, static_cast<uint2*>(codes),
                     static_cast<uint16_t*>(scales));
  return hipGetLastError();
}

hipError_t launch_pack_int8g128(int64_t N, int64_t K, const void* codes, const void* scales,
                                const float* r, void* blob, hipStream_t stream) {
  auto* b = static_cast<uint8_t*>(blob);
  hipLaunchKernelGGL(pack_int8g128_header_kernel, dim3(1), dim3(64), 0, stream, N, K, b);
  const int64_t work = N * K / 16;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_int8g128_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(codes), static_cast<const uint16_t*>(scales), r, N, K,
                     b, 0, static_cast<float*>(nullptr));
  return hipGetLastError();
}

hipError_t launch_unpack_int8g128(int64_t N, int64_t K, const void* blob, void* codes, void* scales,
                                  float* r, float* t_w, hipStream_t stream) {
  const int64_t work = N * K / 16;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_int8g128_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(codes), static_cast<const uint16_t*>(scales), r, N, K,
                     const_cast<uint8_t*>(static_cast<const uint8_t*>(blob)), 1, t_w);
  return hipGetLastError();
}

hipError_t launch_linear_int8g128(int64_t M, int64_t N, int64_t K, const void* a_codes,
                                  const void* a_scales, const void* blob, void* Y,
                                  hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const auto* ac = static_cast<const uint8_t*>(a_codes);
  const auto* as = static_cast<const uint16_t*>(a_scales);
  const auto* bl = static_cast<const uint8_t*>(blob);
  auto* y = static_cast<uint16_t*>(Y);
  const int64_t groups = N / 16;
  if (M == 1 && i8_dot_lds<1>(K) <= 65536) {
    if (groups < 1024) return launch_i8_dot<16, 2>(M, N, K, ac, as, bl, y, stream);
    return launch_i8_dot<8, 2>(M, N, K, ac, as, bl, y, stream);
  }
  if (M == 2 && i8_dot_lds<2>(K) <= 65536) {
    if (groups < 1024) return launch_i8_dot<16, 2>(M, N, K, ac, as, bl, y, stream);
    return launch_i8_dot<8, 2>(M, N, K, ac, as, bl, y, stream);
  }
  if (M == 3 && i8_dot_lds<3>(K) <= 65536) {
    if (groups < 1024) return launch_i8_dot<16, 2>(M, N, K, ac, as, bl, y, stream);
    return launch_i8_dot<8, 2>(M, N, K, ac, as, bl, y, stream);
  }
  if (M <= 16) {
    // weight streaming with the MFMA taking up to 16 activation rows
    const int64_t KS = K / kG;
    if (KS > 32) return launch_i8_decode<8, 8>(M, N, K, ac, as, bl, y, stream);
    if (groups < 256) return launch_i8_decode<16, 2>(M, N, K, ac, as, bl, y, stream);
    if (groups < 1024) return launch_i8_decode<8, 4>(M, N, K, ac, as, bl, y, stream);
    return launch_i8_decode<4, 8>(M, N, K, ac, as, bl, y, stream);
  }
  if (M <= 32) return launch_i8_tile<1, 4>(M, N, K, ac, as, bl, y, stream);
  if (M <= 64) return launch_i8_tile<2, 4>(M, N, K, ac, as, bl, y, stream);
  if (M <= 128) return launch_i8_lds<2, 4>(M, N, K, ac, as, bl, y, stream);
  return launch_i8_lds<4, 3>(M, N, K, ac, as, bl, y, stream);
}

}  // namespace w4a4
