// DualQuant's offline dual-scale solver on gfx950 (MXFP4, MXINT4, NVFP4).
//
// Algorithm 1 of the DualQuant paper (Section 4.3, block coordinate descent
// with closed-form scale updates): starting from alpha_0 = 1 / row absmax and
// beta_0 = 1 / column l1 norm, each of T iterations
//   - quantizes W~ = Diag(alpha) W Diag(beta) row-wise (the format's block
//     quantizer, the same device code as the activation quantizer), forms
//     R = Q^ Diag(beta)^-1 and sets r_i = alpha_i^-1 to the power of two
//     nearest to <W_i, R_i> / ||R_i||^2 (the row's closed-form minimizer,
//     projected as in Appendix C, Remark 1);
//   - re-quantizes with the new alpha, forms S = Diag(alpha)^-1 Q^ and sets
//     c_j = beta_j^-1 likewise over the columns.
// A final pass emits Q(Diag(alpha) W Diag(beta)) as canonical codes and
// scales; W ~ Diag(r) Q Diag(c).  The scales are projected to powers of two
// (E8M0) for the MX formats and to positive E4M3 values (UE4M3) for NVFP4,
// whose quantizer also takes the fp32 tensor scale of the W~ it quantizes:
// an amax pass over W~ precedes each NVFP4 quantization, and the last one
// gives the returned t_w.
//
// The iterations stop early at a fixed point: after each iteration a small
// kernel compares (alpha, beta) with the previous iteration's and, if
// nothing changed, raises a flag on which the remaining passes return at
// once (every later iteration would repeat the same one exactly).
//
// Every projection is a discrete decision taken on fp64 sums, taken here in
// one fixed order (so results are deterministic; a correctly rounded sum
// differs from it only in the last bits, which changes a projection only
// when the minimizer lies within that distance of a projection midpoint):
//   rows:    a lane sums its 8 consecutive terms in order; the 4 lanes of a
//            32-block combine as ((p0 + p1) + p2) + p3; the row-finalize
//            thread adds the block sums in order;
//   columns: a thread sums its column over a chunk of 16 rows in order; the
//            column-finalize thread adds the chunk sums in order.
// Per pass each element is read once (fp32 W), one grid covering W: threads
// own 8 consecutive columns (one 32-byte read per row) of a 16-row chunk and
// issue the 16 reads before any arithmetic.  R = Q^ / beta and S = Q^ / alpha
// are fp64 quotients; once the scales are powers of two (every pass after the
// first row pass: alpha = 1/r, beta = 1/c) the quotient equals the product
// with the exact reciprocal, which the kernel uses instead of a division.
#include "common.h"
#include "kernels.h"
#include "mx_quant.h"
#include "nv_quant.h"

namespace w4a4 {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 16;  // rows per column partial sum (and per thread in those passes)
constexpr int kRowTile = 4;  // rows per thread in the row and emit passes

enum PassMode { kInit = 0, kRows = 1, kCols = 2, kEmit = 3 };

// value of 4-bit code `q` of the format (exact)
template <int FMT>
__device__ __forceinline__ double code_value(uint32_t q) {
  if (FMT == MXINT4) return double(int(q << 28) >> 28);
  // E2M1: exponent field e, mantissa bit m: 0.5 m (e = 0), (1 + m/2) 2^(e-1)
  const int e = int(q >> 1) & 3, m = int(q & 1);
  const double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return (q & 8) ? -v : v;
}

// Nearest power of two 2^e, e in [-127, 127], to u in linear distance; an
// exact tie 1.5 * 2^e goes up; non-positive (or NaN) u gives 2^-127.
__device__ __forceinline__ double project_e8m0(double u) {
  if (!(u > 0.0)) return 0x1p-127;
  int e;
  (void)frexp(u, &e);  // 2^(e-1) <= u < 2^e
  const double lo = ldexp(1.0, e - 1);
  const double near = u >= 1.5 * lo ? 2.0 * lo : lo;
  return fmin(fmax(near, 0x1p-127), 0x1p127);
}

// Nearest positive finite E4M3 value to u in linear distance, ties to the
// even code; saturating at 448; u at or below 2^-9 (or NaN) gives 2^-9.
__device__ __forceinline__ double project_ue4m3(double u) {
  if (!(u > 0x1p-9)) return 0x1p-9;
  if (u >= 448.0) return 448.0;
  int c;  // value(c) <= u < value(c + 1)
  if (u < 0.015625) {
    c = int(u * 512.0);  // subnormal codes 1..7
  } else {
    const uint64_t b = uint64_t(__double_as_longlong(u));
    const int E = int((b >> 52) & 0x7ff) - 1023;  // -6 .. 8
    c = ((E + 7) << 3) | int((b >> 49) & 7);
  }
  const double lo = e4m3_value(c), hi = e4m3_value(c + 1), mid = 0.5 * (lo + hi);
  if (u > mid) return hi;
  if (u < mid) return lo;
  return (c & 1) ? hi : lo;
}

template <int FMT>
__device__ __forceinline__ double project_scale(double u) {
  return FMT == NVFP4 ? project_ue4m3(u) : project_e8m0(u);
}

__device__ __forceinline__ double shfl_lane(double v, int src) {
  return __shfl(v, src, 64);
}

// One pass over W [N, K] fp32.  Grid x: chunks of ROWS rows (16 where column
// sums are formed, 4 otherwise), grid y: 256-wide runs of 8-column groups.  Rows: per (32-block, row) fp64 sums of W*R and R*R,
// block-major (lane 4q of the quad writes them).  Cols: per (chunk, column) fp64 sums of
// W*S and S*S.  Init: per (row, 32-block) max |W| and per (chunk, column)
// sum |W|.  Emit: codes and scales.
template <int FMT, int MODE, bool DIV, int ROWS>
__global__ __launch_bounds__(kThreads) void dq_pass_kernel(
    const float* __restrict__ W, const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* __restrict__ tsc, int64_t N, int64_t K8, double* __restrict__ row_a,
    double* __restrict__ row_b,
    double* __restrict__ col_a, double* __restrict__ col_b, uint32_t* __restrict__ codes,
    uint8_t* __restrict__ scales, const int* __restrict__ done) {
  if ((MODE == kRows || MODE == kCols) && *done) return;  // at a fixed point: nothing changes
  const int64_t col_raw = int64_t(blockIdx.y) * kThreads + threadIdx.x;
  const bool live_c = col_raw < K8;
  const int64_t col8 = live_c ? col_raw : K8 - 1;  // every lane joins the quad exchanges
  const int64_t K = K8 * 8, KB = K8 / 4;
  static_assert((MODE == kInit || MODE == kCols) == (ROWS == kChunk), "column sums per 16 rows");
  const int64_t r0 = int64_t(blockIdx.x) * ROWS;
  const int lane = threadIdx.x & 63;
  const int quad0 = lane & ~3;
  float b8[8];
  double ib8[8];  // exact reciprocals of the column scales (powers of two)
  if (MODE != kInit) {
    const float4 b0 = reinterpret_cast<const float4*>(beta)[2 * col8];
    const float4 b1 = reinterpret_cast<const float4*>(beta)[2 * col8 + 1];
    b8[0] = b0.x; b8[1] = b0.y; b8[2] = b0.z; b8[3] = b0.w;
    b8[4] = b1.x; b8[5] = b1.y; b8[6] = b1.z; b8[7] = b1.w;
#pragma unroll
    for (int e = 0; e < 8; ++e) ib8[e] = 1.0 / double(b8[e]);
  }
  double ca[8], cb[8];  // column sums over this chunk
  const int64_t rows = N - r0 < ROWS ? N - r0 : ROWS;
  // all reads of the chunk in flight at once (rows past N re-read row N-1)
  float4 wv[ROWS][2];
#pragma unroll
  for (int i = 0; i < ROWS; ++i) {
    const int64_t row = r0 + i < N ? r0 + i : N - 1;
    wv[i][0] = reinterpret_cast<const float4*>(W + row * K)[2 * col8];
    wv[i][1] = reinterpret_cast<const float4*>(W + row * K)[2 * col8 + 1];
  }
#pragma unroll
  for (int i = 0; i < ROWS; ++i) {
    if (i >= rows) break;
    const int64_t row = r0 + i;
    const float4 w0 = wv[i][0], w1 = wv[i][1];
    const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    if (MODE == kInit) {
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        m = fmaxf(m, fabsf(w[e]));
        const double a = fabs(double(w[e]));
        ca[e] = i == 0 ? a : ca[e] + a;
      }
      m = fmaxf(m, quad_xor1(m));
      m = fmaxf(m, quad_xor2(m));
      if (live_c && (col8 & 3) == 0) row_a[(col8 >> 2) * N + row] = double(m);
      continue;
    }
    const float a = alpha[row];
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = __fmul_rn(__fmul_rn(a, w[e]), b8[e]);
    uint32_t word, sbyte;
    double bscale;  // block scale (times t for NVFP4), exact
    if constexpr (FMT == NVFP4) {
      const float t = *tsc;
      int sc;
      quant8_nv(x, t, word, sc);
      sbyte = uint32_t(sc);
      bscale = e4m3_value(sc) * double(t);
    } else {
      quant8_mx<FMT>(x, word, sbyte);
      bscale = ldexp(1.0, int(sbyte) - 127);
    }
    if (MODE == kEmit) {
      if (live_c) {
        codes[row * K8 + col8] = word;
        if (FMT == NVFP4 && (col8 & 1) == 0) scales[row * (K8 / 2) + (col8 >> 1)] = uint8_t(sbyte);
        if (FMT != NVFP4 && (col8 & 3) == 0) scales[row * KB + (col8 >> 2)] = uint8_t(sbyte);
      }
      continue;
    }
    if (MODE == kRows) {
      double pa = 0.0, pb = 0.0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double q = code_value<FMT>((word >> (4 * e)) & 15u) * bscale;
        const double R = DIV ? q / double(b8[e]) : q * ib8[e];
        const double ta = double(w[e]) * R, tb = R * R;
        pa = e == 0 ? ta : pa + ta;
        pb = e == 0 ? tb : pb + tb;
      }
      const double a1 = shfl_lane(pa, quad0 + 1), a2 = shfl_lane(pa, quad0 + 2),
                   a3 = shfl_lane(pa, quad0 + 3);
      const double b1 = shfl_lane(pb, quad0 + 1), b2 = shfl_lane(pb, quad0 + 2),
                   b3 = shfl_lane(pb, quad0 + 3);
      if (live_c && (col8 & 3) == 0) {
        row_a[(col8 >> 2) * N + row] = ((pa + a1) + a2) + a3;
        row_b[(col8 >> 2) * N + row] = ((pb + b1) + b2) + b3;
      }
    } else {  // kCols
      const double ia = 1.0 / double(a);  // exact for MX: alpha = 1/r is a power of two
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double q = code_value<FMT>((word >> (4 * e)) & 15u) * bscale;
        const double S = DIV ? q / double(a) : q * ia;
        const double ta = double(w[e]) * S, tb = S * S;
        ca[e] = i == 0 ? ta : ca[e] + ta;
        cb[e] = i == 0 ? tb : cb[e] + tb;
      }
    }
  }
  if ((MODE == kInit || MODE == kCols) && live_c && rows > 0) {
    const int64_t off = int64_t(blockIdx.x) * K + col8 * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      col_a[off + e] = ca[e];
      if (MODE == kCols) col_b[off + e] = cb[e];
    }
  }
}

// NVFP4: per-block maxima of |W~| = |fp32(fp32(alpha_i W_ij) beta_j)|, then
// t = fp32(amax) / 2688 (t = 1 for an all-zero W~ or when that underflows),
// the activation quantizer's tensor scale rule applied to W~.
constexpr int kAmaxBlocks = 1024;

__global__ __launch_bounds__(kThreads) void dq_amax_kernel(
    const float* __restrict__ W, const float* __restrict__ alpha, const float* __restrict__ beta,
    int64_t N, int64_t K8, float* __restrict__ part, const int* __restrict__ done) {
  if (done && *done) return;
  float m = 0.0f;
  const int64_t n = N * K8;
  for (int64_t g = int64_t(blockIdx.x) * kThreads + threadIdx.x; g < n;
       g += int64_t(gridDim.x) * kThreads) {
    const int64_t row = g / K8, col8 = g - row * K8;
    const float a = alpha[row];
    const float4 w0 = reinterpret_cast<const float4*>(W + row * K8 * 8)[2 * col8];
    const float4 w1 = reinterpret_cast<const float4*>(W + row * K8 * 8)[2 * col8 + 1];
    const float4 b0 = reinterpret_cast<const float4*>(beta)[2 * col8];
    const float4 b1 = reinterpret_cast<const float4*>(beta)[2 * col8 + 1];
    const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(__fmul_rn(__fmul_rn(a, w[e]), b[e])));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
    part[blockIdx.x] = r;
  }
}

__global__ __launch_bounds__(kThreads) void dq_tscale_kernel(const float* __restrict__ part, int n,
                                                             float* __restrict__ t_out,
                                                             float* __restrict__ t_copy,
                                                             const int* __restrict__ done) {
  if (done && *done) return;
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += kThreads) m = fmaxf(m, part[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = red[0];
    for (int i = 1; i < kThreads / 64; ++i) a = fmaxf(a, red[i]);
    float t = __fdiv_rn(a, 2688.0f);
    if (a == 0.0f || t == 0.0f) t = 1.0f;
    *t_out = t;
    if (t_copy) *t_copy = t;
  }
}

// Sum of the n values p[0], p[stride], ... in order; loads go out kBatch at a
// time ahead of the (sequential) additions.
constexpr int kBatch = 16;

__device__ __forceinline__ double ordered_sum(const double* __restrict__ p, int64_t n,
                                              int64_t stride) {
  double s = p[0];
  int64_t k = 1;
  for (; k + kBatch <= n; k += kBatch) {
    double v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = p[(k + u) * stride];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) s = s + v[u];
  }
  for (; k < n; ++k) s = s + p[k * stride];
  return s;
}

// One thread per row.  Init: alpha_0 = 1 / max|W_i| (1 for a zero row).
// Update: r_i = Pi(sum W*R / sum R*R), alpha_i = 1 / r_i (r = alpha = 1 when
// the row's Q^ is all zero).
template <int FMT, bool INIT>
__global__ __launch_bounds__(kThreads) void dq_row_finalize_kernel(
    const double* __restrict__ row_a, const double* __restrict__ row_b, int64_t N, int64_t KB,
    float* __restrict__ r, float* __restrict__ alpha, float* __restrict__ alpha_prev,
    int* __restrict__ done) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (INIT && i == 0) *done = 0;
  if (!INIT && *done) return;
  if (i >= N) return;
  if (INIT) {
    alpha_prev[i] = __builtin_nanf("");  // never equal: the first iteration always runs
    double m = 0.0;
    for (int64_t b = 0; b < KB; ++b) m = fmax(m, row_a[b * N + i]);
    alpha[i] = m > 0.0 ? float(1.0 / m) : 1.0f;
    return;
  }
  const double num = ordered_sum(row_a + i, KB, N);
  const double den = ordered_sum(row_b + i, KB, N);
  const double ri = den > 0.0 ? project_scale<FMT>(num / den) : 1.0;
  r[i] = float(ri);
  alpha[i] = float(1.0 / ri);
}

// One thread per column, the same over the 16-row chunk sums.
template <int FMT, bool INIT>
__global__ __launch_bounds__(kThreads) void dq_col_finalize_kernel(
    const double* __restrict__ col_a, const double* __restrict__ col_b, int64_t chunks, int64_t K,
    float* __restrict__ c, float* __restrict__ beta, float* __restrict__ beta_prev,
    const int* __restrict__ done) {
  const int64_t j = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (!INIT && *done) return;
  if (j >= K) return;
  if (INIT) beta_prev[j] = __builtin_nanf("");
  const double num = ordered_sum(col_a + j, chunks, K);
  const double den = INIT ? 0.0 : ordered_sum(col_b + j, chunks, K);
  if (INIT) {
    beta[j] = num > 0.0 ? float(1.0 / num) : 1.0f;
    return;
  }
  const double cj = den > 0.0 ? project_scale<FMT>(num / den) : 1.0;
  c[j] = float(cj);
  beta[j] = float(1.0 / cj);
}

// After an iteration: if neither alpha nor beta changed, (alpha, beta) is a
// fixed point and every later iteration would repeat it exactly, so `done`
// is raised and the remaining passes return at once.  One workgroup; it also
// keeps this iteration's scales for the next comparison.
__global__ __launch_bounds__(1024) void dq_fixed_point_kernel(const float* __restrict__ alpha,
                                                               const float* __restrict__ beta,
                                                               float* __restrict__ alpha_prev,
                                                               float* __restrict__ beta_prev,
                                                               int64_t N, int64_t K,
                                                               int* __restrict__ done) {
  if (*done) return;
  int changed = 0;
  for (int64_t i = threadIdx.x; i < N; i += 1024) {
    const float a = alpha[i];
    changed |= __float_as_uint(a) != __float_as_uint(alpha_prev[i]);
    alpha_prev[i] = a;
  }
  for (int64_t j = threadIdx.x; j < K; j += 1024) {
    const float b = beta[j];
    changed |= __float_as_uint(b) != __float_as_uint(beta_prev[j]);
    beta_prev[j] = b;
  }
  changed = __syncthreads_or(changed);
  if (threadIdx.x == 0 && !changed) *done = 1;
}

struct SolverWs {
  float* alpha;
  float* beta;
  float* alpha_prev;
  float* beta_prev;
  int* done;
  float* amax;  // kAmaxBlocks partial maxima (NVFP4)
  float* t;     // tensor scale of the current W~ (NVFP4)
  double *row_a, *row_b, *col_a, *col_b;
};

SolverWs carve(void* ws, int64_t N, int64_t K) {
  const int64_t KB = K / 32, chunks = (N + kChunk - 1) / kChunk;
  uint8_t* p = static_cast<uint8_t*>(ws);
  SolverWs s;
  s.row_a = reinterpret_cast<double*>(p);
  p += align256(N * KB * 8);
  s.row_b = reinterpret_cast<double*>(p);
  p += align256(N * KB * 8);
  s.col_a = reinterpret_cast<double*>(p);
  p += align256(chunks * K * 8);
  s.col_b = reinterpret_cast<double*>(p);
  p += align256(chunks * K * 8);
  s.alpha = reinterpret_cast<float*>(p);
  p += align256(N * 4);
  s.beta = reinterpret_cast<float*>(p);
  p += align256(K * 4);
  s.alpha_prev = reinterpret_cast<float*>(p);
  p += align256(N * 4);
  s.beta_prev = reinterpret_cast<float*>(p);
  p += align256(K * 4);
  s.amax = reinterpret_cast<float*>(p);
  p += align256(kAmaxBlocks * 4);
  s.t = reinterpret_cast<float*>(p);
  s.done = reinterpret_cast<int*>(p + 64);
  return s;
}

template <int FMT, int MODE, bool DIV = false>
void pass(const float* W, const SolverWs& s, int64_t N, int64_t K, uint32_t* codes,
          uint8_t* scales, hipStream_t stream) {
  constexpr int ROWS = (MODE == kInit || MODE == kCols) ? kChunk : kRowTile;
  const int64_t K8 = K / 8;
  const dim3 grid(unsigned((N + ROWS - 1) / ROWS), unsigned((K8 + kThreads - 1) / kThreads));
  hipLaunchKernelGGL((dq_pass_kernel<FMT, MODE, DIV, ROWS>), grid, dim3(kThreads), 0, stream, W, s.alpha,
                     s.beta, s.t, N, K8, s.row_a, s.row_b, s.col_a, s.col_b, codes, scales, s.done);
}

// NVFP4: the tensor scale of W~ at the current scales (into s.t, and into
// t_copy when given); inside the iterations it is skipped at a fixed point,
// the final one (t_copy) always runs
void tensor_scale(const float* W, const SolverWs& s, int64_t N, int64_t K, float* t_copy,
                  hipStream_t stream) {
  const int64_t n = N * (K / 8);
  const int blocks = int(n / kThreads + 1 < kAmaxBlocks ? n / kThreads + 1 : kAmaxBlocks);
  const int* done = t_copy ? nullptr : s.done;
  hipLaunchKernelGGL(dq_amax_kernel, dim3(blocks), dim3(kThreads), 0, stream, W, s.alpha, s.beta, N,
                     K / 8, s.amax, done);
  hipLaunchKernelGGL(dq_tscale_kernel, dim3(1), dim3(kThreads), 0, stream, s.amax, blocks, s.t,
                     t_copy, done);
}

template <int FMT>
hipError_t solve(int64_t N, int64_t K, const float* W, int iters, float* r, float* c,
                 void* codes, void* scales, float* t_w, void* ws, hipStream_t stream) {
  constexpr bool NV = FMT == NVFP4;
  const SolverWs s = carve(ws, N, K);
  const int64_t KB = K / 32, chunks = (N + kChunk - 1) / kChunk;
  const dim3 gr(unsigned((N + kThreads - 1) / kThreads)), gc(unsigned((K + kThreads - 1) / kThreads));
  uint32_t* cw = static_cast<uint32_t*>(codes);
  uint8_t* sb = static_cast<uint8_t*>(scales);
  pass<FMT, kInit>(W, s, N, K, cw, sb, stream);
  hipLaunchKernelGGL((dq_row_finalize_kernel<FMT, true>), gr, dim3(kThreads), 0, stream, s.row_a,
                     s.row_b, N, KB, r, s.alpha, s.alpha_prev, s.done);
  hipLaunchKernelGGL((dq_col_finalize_kernel<FMT, true>), gc, dim3(kThreads), 0, stream, s.col_a,
                     s.col_b, chunks, K, c, s.beta, s.beta_prev, s.done);
  for (int t = 0; t < iters; ++t) {
    if (NV) tensor_scale(W, s, N, K, nullptr, stream);
    // beta_0 = 1 / l1 is not a power of two: the first row pass divides (and
    // every NVFP4 pass: UE4M3 scales are not powers of two)
    if (t == 0 || NV)
      pass<FMT, kRows, true>(W, s, N, K, cw, sb, stream);
    else
      pass<FMT, kRows>(W, s, N, K, cw, sb, stream);
    hipLaunchKernelGGL((dq_row_finalize_kernel<FMT, false>), gr, dim3(kThreads), 0, stream, s.row_a,
                       s.row_b, N, KB, r, s.alpha, s.alpha_prev, s.done);
    if (NV) tensor_scale(W, s, N, K, nullptr, stream);
    pass<FMT, kCols, NV>(W, s, N, K, cw, sb, stream);
    hipLaunchKernelGGL((dq_col_finalize_kernel<FMT, false>), gc, dim3(kThreads), 0, stream, s.col_a,
                       s.col_b, chunks, K, c, s.beta, s.beta_prev, s.done);
    hipLaunchKernelGGL(dq_fixed_point_kernel, dim3(1), dim3(1024), 0, stream, s.alpha, s.beta,
                       s.alpha_prev, s.beta_prev, N, K, s.done);
  }
  if (NV) tensor_scale(W, s, N, K, t_w, stream);
  pass<FMT, kEmit>(W, s, N, K, cw, sb, stream);
  return hipGetLastError();
}

}  // namespace

size_t solver_workspace_bytes(int64_t N, int64_t K) {
  const int64_t KB = K / 32, chunks = (N + kChunk - 1) / kChunk;
  return size_t(2 * align256(N * KB * 8) + 2 * align256(chunks * K * 8) + 2 * align256(N * 4) +
                2 * align256(K * 4) + align256(kAmaxBlocks * 4) + 256);
}

hipError_t launch_dualquant_solve(int fmt, int64_t N, int64_t K, const float* W, int iters,
                                  float* r, float* c, void* codes, void* scales, float* t_w,
                                  void* workspace, hipStream_t stream) {
  if (fmt == MXFP4) return solve<MXFP4>(N, K, W, iters, r, c, codes, scales, t_w, workspace, stream);
  if (fmt == NVFP4) return solve<NVFP4>(N, K, W, iters, r, c, codes, scales, t_w, workspace, stream);
  return solve<MXINT4>(N, K, W, iters, r, c, codes, scales, t_w, workspace, stream);
}

}  // namespace w4a4
