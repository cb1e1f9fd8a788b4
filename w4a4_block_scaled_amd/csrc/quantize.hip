// Fused activation rescale + block quantization for gfx950.
//
// DualQuant Section 4.4: the column scale is applied inside the activation
// quantization kernel (no separate launch) and the format-native per-row
// block scale is computed on the rescaled activations; eq. (3) gives the
// rescaling X~ = X diag(c).  Section 3 gives the formats (MXFP4 / MXINT4:
// blocks of 32 with an E8M0 scale; NVFP4: blocks of 16 with a UE4M3 scale)
// and the quantizer (nearest grid point, clipped).
//
// One thread owns 8 consecutive elements of a row (one 16-byte load of bf16,
// one 4-byte store of codes).  A block of 32 (16) elements is owned by 4 (2)
// consecutive lanes; its amax is reduced with cross-lane exchanges.  Every
// rounding decision is exact: MX scales come from exponent bits, elements
// are compared against exact midpoints, NVFP4 scale/element decisions are
// taken against thresholds computed exactly in fp64.
#include "common.h"
#include "kernels.h"
#include "mx_quant.h"
#include "nv_quant.h"

namespace w4a4 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void load8(const uint4* __restrict__ X, const float* __restrict__ c,
                                      int64_t g, int64_t col8, float (&x)[8]) {
  const uint4 v = X[g];
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
    x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
  if (c) {
    const float4 c0 = reinterpret_cast<const float4*>(c)[2 * col8];
    const float4 c1 = reinterpret_cast<const float4*>(c)[2 * col8 + 1];
    const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __fmul_rn(x[i], cc[i]);  // one rounded fp32 multiply
  }
}

// E2M1 magnitude index of v (>= 0) in units of the block scale: count of
// midpoints below v, ties to the even code.
__device__ __forceinline__ uint32_t e2m1_index(float v) {
  return (v > 0.25f) + (v >= 0.75f) + (v > 1.25f) + (v >= 1.75f) + (v > 2.5f) + (v >= 3.5f) +
         (v > 5.0f);
}

// Grid x: chunks of R rows, grid y: 256-wide runs of 8-column groups.  A
// thread owns 8 consecutive columns (one 16-byte load of bf16 per row, one
// 4-byte store of codes): it loads their column scales once and quantizes
// those columns of R rows, with all R loads in flight together.
template <int FMT, int R>
__global__ __launch_bounds__(kThreads) void quantize_mx_kernel(
    const uint4* __restrict__ X, const float* __restrict__ c, uint32_t* __restrict__ codes,
    uint8_t* __restrict__ scales, int64_t M, int64_t K8) {
  const int64_t col_raw = int64_t(blockIdx.y) * kThreads + threadIdx.x;
  const bool live_c = col_raw < K8;
  const int64_t col8 = live_c ? col_raw : K8 - 1;  // every lane joins the shuffles
  const int64_t r0 = int64_t(blockIdx.x) * R;
  float cc[8];
  if (c) {
    const float4 c0 = reinterpret_cast<const float4*>(c)[2 * col8];
    const float4 c1 = reinterpret_cast<const float4*>(c)[2 * col8 + 1];
    cc[0] = c0.x; cc[1] = c0.y; cc[2] = c0.z; cc[3] = c0.w;
    cc[4] = c1.x; cc[5] = c1.y; cc[6] = c1.z; cc[7] = c1.w;
  }
  // X is read once: non-temporal loads
  typedef unsigned ux4 __attribute__((ext_vector_type(4)));
  ux4 v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = r0 + r < M ? r0 + r : M - 1;
    v[r] = __builtin_nontemporal_load(reinterpret_cast<const ux4*>(X) + row * K8 + col8);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t w[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
      x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
    if (c) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __fmul_rn(x[i], cc[i]);  // one rounded fp32 multiply
    }
    uint32_t word, sbyte;
    quant8_mx<FMT>(x, word, sbyte);
    const int64_t row = r0 + r;
    if (live_c && row < M) {
      codes[row * K8 + col8] = word;
      if ((col8 & 3) == 0) scales[row * (K8 / 4) + (col8 >> 2)] = uint8_t(sbyte);
    }
  }
}

// ----------------------------------------------------------------- NVFP4 --

__global__ __launch_bounds__(kThreads) void absmax_partial_kernel(
    const uint4* __restrict__ X, const float* __restrict__ c, float* __restrict__ partial,
    int64_t n_groups, int64_t K8) {
  float m = 0.0f;
  for (int64_t g = int64_t(blockIdx.x) * kThreads + threadIdx.x; g < n_groups;
       g += int64_t(gridDim.x) * kThreads) {
    float x[8];
    load8(X, c, g, g % K8, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
    partial[blockIdx.x] = r;
  }
}

// t = fp32(A) / 2688 with A the tensor amax; t = 1 when A = 0 (or t underflows).
__global__ __launch_bounds__(kThreads) void tensor_scale_kernel(const float* __restrict__ partial,
                                                                int n, float* __restrict__ t_out) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += kThreads) m = fmaxf(m, partial[i]);
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
  }
}

__global__ __launch_bounds__(kThreads) void quantize_nv_kernel(
    const uint4* __restrict__ X, const float* __restrict__ c, const float* __restrict__ t_ptr,
    uint32_t* __restrict__ codes, uint8_t* __restrict__ scales, int64_t n_groups, int64_t K8) {
  const int64_t g_raw = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const bool live = g_raw < n_groups;
  const int64_t g = live ? g_raw : n_groups - 1;
  const int64_t row = g / K8;
  const int64_t col8 = g - row * K8;

  float x[8];
  load8(X, c, g, col8, x);
  uint32_t word;
  int s;
  quant8_nv(x, *t_ptr, word, s);
  if (!live) return;
  codes[g] = word;
  if ((col8 & 1) == 0) scales[row * (K8 / 2) + (col8 >> 1)] = uint8_t(s);
}

// Small NVFP4 tensors (decode: a few rows) in one launch: every workgroup
// takes the tensor amax over all of X itself (a few tens of KB, read from
// L2 after the first), forms t, and quantizes its own kThreads groups; the
// first writes t.  Same reduction result (a maximum does not depend on
// order), same t rounding and the same block quantizer as the three-kernel
// path, so codes, scales and t are identical, without the two extra
// launches and without one workgroup doing all the fp64 block decisions.
constexpr int64_t kNvSmallGroups = 8192;  // groups of 8 elements (<= 32 workgroups)

__global__ __launch_bounds__(kThreads) void quantize_nv_small_kernel(
    const uint4* __restrict__ X, const float* __restrict__ c, float* __restrict__ t_out,
    uint32_t* __restrict__ codes, uint8_t* __restrict__ scales, int64_t n_groups, int64_t K8) {
  float m = 0.0f;
  for (int64_t g = threadIdx.x; g < n_groups; g += kThreads) {
    float x[8];
    load8(X, c, g, g % K8, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float a = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) a = fmaxf(a, red[i]);
  float t = __fdiv_rn(a, 2688.0f);
  if (a == 0.0f || t == 0.0f) t = 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *t_out = t;
  // this workgroup's groups (a 16-block is an even group and the next one,
  // in adjacent lanes); lanes past the end quantize a clamped copy and
  // store nothing
  const int64_t g_raw = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const bool live = g_raw < n_groups;
  const int64_t g = live ? g_raw : n_groups - 1;
  const int64_t row = g / K8, col8 = g - row * K8;
  float x[8];
  load8(X, c, g, col8, x);
  uint32_t word;
  int sc;
  quant8_nv(x, t, word, sc);
  if (live) {
    codes[g] = word;
    if ((col8 & 1) == 0) scales[row * (K8 / 2) + (col8 >> 1)] = uint8_t(sc);
  }
}

// ------------------------------------------------ several column scales --
//
// One X, P column-scale vectors (per-projection c on a fused input, e.g. the
// q, k and v projections of one hidden state): X is read once and each of the
// P rescalings is quantized as quantize_act would quantize it.

struct MultiOut {
  const float* c[kMaxOutputs];
  uint32_t* codes[kMaxOutputs];
  uint8_t* scales[kMaxOutputs];
  float* t[kMaxOutputs];
  float* partial[kMaxOutputs];
};

__device__ __forceinline__ void load_c8(const float* __restrict__ c, int64_t col8, float (&cc)[8]) {
  const float4 c0 = reinterpret_cast<const float4*>(c)[2 * col8];
  const float4 c1 = reinterpret_cast<const float4*>(c)[2 * col8 + 1];
  cc[0] = c0.x; cc[1] = c0.y; cc[2] = c0.z; cc[3] = c0.w;
  cc[4] = c1.x; cc[5] = c1.y; cc[6] = c1.z; cc[7] = c1.w;
}

__device__ __forceinline__ void bf16x8(const uint4& v, float (&x)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
    x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
}

template <int FMT, int R, int P>
__global__ __launch_bounds__(kThreads) void quantize_mx_multi_kernel(const uint4* __restrict__ X,
                                                                     MultiOut o, int64_t M,
                                                                     int64_t K8) {
  const int64_t col_raw = int64_t(blockIdx.y) * kThreads + threadIdx.x;
  const bool live_c = col_raw < K8;
  const int64_t col8 = live_c ? col_raw : K8 - 1;
  const int64_t r0 = int64_t(blockIdx.x) * R;
  float cc[P][8];
#pragma unroll
  for (int p = 0; p < P; ++p) load_c8(o.c[p], col8, cc[p]);
  typedef unsigned ux4 __attribute__((ext_vector_type(4)));
  ux4 v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = r0 + r < M ? r0 + r : M - 1;
    v[r] = __builtin_nontemporal_load(reinterpret_cast<const ux4*>(X) + row * K8 + col8);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float x0[8];
    bf16x8(uint4{v[r].x, v[r].y, v[r].z, v[r].w}, x0);
    const int64_t row = r0 + r;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __fmul_rn(x0[i], cc[p][i]);
      uint32_t word, sbyte;
      quant8_mx<FMT>(x, word, sbyte);
      if (live_c && row < M) {
        o.codes[p][row * K8 + col8] = word;
        if ((col8 & 3) == 0) o.scales[p][row * (K8 / 4) + (col8 >> 2)] = uint8_t(sbyte);
      }
    }
  }
}

template <int P>
__global__ __launch_bounds__(kThreads) void absmax_multi_kernel(const uint4* __restrict__ X,
                                                                MultiOut o, int64_t n_groups,
                                                                int64_t K8) {
  float m[P];
#pragma unroll
  for (int p = 0; p < P; ++p) m[p] = 0.0f;
  for (int64_t g = int64_t(blockIdx.x) * kThreads + threadIdx.x; g < n_groups;
       g += int64_t(gridDim.x) * kThreads) {
    float x0[8];
    bf16x8(X[g], x0);
#pragma unroll
    for (int p = 0; p < P; ++p) {
      float cc[8];
      load_c8(o.c[p], g % K8, cc);
#pragma unroll
      for (int i = 0; i < 8; ++i) m[p] = fmaxf(m[p], fabsf(__fmul_rn(x0[i], cc[i])));
    }
  }
  __shared__ float red[P][kThreads / 64];
#pragma unroll
  for (int p = 0; p < P; ++p) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m[p] = fmaxf(m[p], __shfl_xor(m[p], off));
    if ((threadIdx.x & 63) == 0) red[p][threadIdx.x >> 6] = m[p];
  }
  __syncthreads();
  if (threadIdx.x < P) {
    const int p = threadIdx.x;
    float r = red[p][0];
    for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[p][i]);
    o.partial[p][blockIdx.x] = r;
  }
}

template <int P>
__global__ __launch_bounds__(kThreads) void quantize_nv_multi_kernel(const uint4* __restrict__ X,
                                                                     MultiOut o, int64_t n_groups,
                                                                     int64_t K8) {
  const int64_t g_raw = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const bool live = g_raw < n_groups;
  const int64_t g = live ? g_raw : n_groups - 1;
  const int64_t row = g / K8;
  const int64_t col8 = g - row * K8;
  float x0[8];
  bf16x8(X[g], x0);
#pragma unroll
  for (int p = 0; p < P; ++p) {
    float cc[8], x[8];
    load_c8(o.c[p], col8, cc);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __fmul_rn(x0[i], cc[i]);
    uint32_t word;
    int s;
    quant8_nv(x, *o.t[p], word, s);
    if (live) {
      o.codes[p][g] = word;
      if ((col8 & 1) == 0) o.scales[p][row * (K8 / 2) + (col8 >> 1)] = uint8_t(s);
    }
  }
}

// The 8-bit MX variants: as quantize_mx_kernel, with 8 code bytes per thread
// and row (one 8-byte store).
template <int FMT, int R>
__global__ __launch_bounds__(kThreads) void quantize_mx8_kernel(
    const uint4* __restrict__ X, const float* __restrict__ c, uint2* __restrict__ codes,
    uint8_t* __restrict__ scales, int64_t M, int64_t K8) {
  const int64_t col_raw = int64_t(blockIdx.y) * kThreads + threadIdx.x;
  const bool live_c = col_raw < K8;
  const int64_t col8 = live_c ? col_raw : K8 - 1;  // every lane joins the shuffles
  const int64_t r0 = int64_t(blockIdx.x) * R;
  float cc[8];
  if (c) {
    const float4 c0 = reinterpret_cast<const float4*>(c)[2 * col8];
    const float4 c1 = reinterpret_cast<const float4*>(c)[2 * col8 + 1];
    cc[0] = c0.x; cc[1] = c0.y; cc[2] = c0.z; cc[3] = c0.w;
    cc[4] = c1.x; cc[5] = c1.y; cc[6] = c1.z; cc[7] = c1.w;
  }
  typedef unsigned ux4 __attribute__((ext_vector_type(4)));
  ux4 v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = r0 + r < M ? r0 + r : M - 1;
    v[r] = __builtin_nontemporal_load(reinterpret_cast<const ux4*>(X) + row * K8 + col8);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t w[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
      x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
    if (c) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __fmul_rn(x[i], cc[i]);  // one rounded fp32 multiply
    }
    uint32_t word[2], sbyte;
    quant8_mx8<FMT>(x, word, sbyte);
    const int64_t row = r0 + r;
    if (live_c && row < M) {
      codes[row * K8 + col8] = uint2{word[0], word[1]};
      if ((col8 & 3) == 0) scales[row * (K8 / 4) + (col8 >> 2)] = uint8_t(sbyte);
    }
  }
}

template <int P>
hipError_t launch_multi(int fmt, int64_t M, int64_t K, const uint4* Xv, MultiOut o,
                        hipStream_t stream) {
  const int64_t K8 = K / 8, n_groups = M * K8;
  if (fmt == MXFP4 || fmt == MXINT4) {
    const dim3 grid(unsigned((M + 1) / 2), unsigned((K8 + kThreads - 1) / kThreads));
    if (fmt == MXFP4)
      hipLaunchKernelGGL((quantize_mx_multi_kernel<MXFP4, 2, P>), grid, dim3(kThreads), 0, stream, Xv, o, M, K8);
    else
      hipLaunchKernelGGL((quantize_mx_multi_kernel<MXINT4, 2, P>), grid, dim3(kThreads), 0, stream, Xv, o, M, K8);
    return hipGetLastError();
  }
  const int nparts = int(std::min<int64_t>(kNvAmaxBlocks, (n_groups + kThreads - 1) / kThreads));
  hipLaunchKernelGGL((absmax_multi_kernel<P>), dim3(nparts), dim3(kThreads), 0, stream, Xv, o,
                     n_groups, K8);
  for (int p = 0; p < P; ++p)
    hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(kThreads), 0, stream, o.partial[p], nparts,
                       o.t[p]);
  hipLaunchKernelGGL((quantize_nv_multi_kernel<P>), dim3(unsigned((n_groups + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, Xv, o, n_groups, K8);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_act(int fmt, int64_t M, int64_t K, const void* X, const float* c,
                               void* codes, void* scales, float* t_act, void* workspace,
                               hipStream_t stream) {
  const int64_t n_groups = M * K / 8;
  if (n_groups == 0) {
    if (fmt == NVFP4) {
      // an empty tensor has amax 0: t = 1
      hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(kThreads), 0, stream,
                         static_cast<const float*>(workspace), 0, t_act);
      return hipGetLastError();
    }
    return hipSuccess;
  }
  const int64_t K8 = K / 8;
  const dim3 grid(unsigned((n_groups + kThreads - 1) / kThreads));
  const uint4* Xv = static_cast<const uint4*>(X);
  uint32_t* cw = static_cast<uint32_t*>(codes);
  uint8_t* sb = static_cast<uint8_t*>(scales);
  if (is_mx8(fmt)) {
    const unsigned gy = unsigned((K8 + kThreads - 1) / kThreads);
    uint2* cw8 = static_cast<uint2*>(codes);
    if (M >= 256) {
      const dim3 g2(unsigned((M + 1) / 2), gy);
      if (fmt == MXFP8)
        hipLaunchKernelGGL((quantize_mx8_kernel<MXFP8, 2>), g2, dim3(kThreads), 0, stream, Xv, c, cw8, sb, M, K8);
      else
        hipLaunchKernelGGL((quantize_mx8_kernel<MXINT8, 2>), g2, dim3(kThreads), 0, stream, Xv, c, cw8, sb, M, K8);
    } else {
      const dim3 g1(unsigned(M), gy);
      if (fmt == MXFP8)
        hipLaunchKernelGGL((quantize_mx8_kernel<MXFP8, 1>), g1, dim3(kThreads), 0, stream, Xv, c, cw8, sb, M, K8);
      else
        hipLaunchKernelGGL((quantize_mx8_kernel<MXINT8, 1>), g1, dim3(kThreads), 0, stream, Xv, c, cw8, sb, M, K8);
    }
  } else if (fmt == MXFP4 || fmt == MXINT4) {
    // 2 rows per thread once there are enough rows to fill the chip (1, 4,
    // 8 or 16 rows per thread measured slower on 2048-row activations)
    const unsigned gy = unsigned((K8 + kThreads - 1) / kThreads);
    if (M >= 256) {
      const dim3 g2(unsigned((M + 1) / 2), gy);
      if (fmt == MXFP4)
        hipLaunchKernelGGL((quantize_mx_kernel<MXFP4, 2>), g2, dim3(kThreads), 0, stream, Xv, c, cw, sb, M, K8);
      else
        hipLaunchKernelGGL((quantize_mx_kernel<MXINT4, 2>), g2, dim3(kThreads), 0, stream, Xv, c, cw, sb, M, K8);
    } else {
      const dim3 g1(unsigned(M), gy);
      if (fmt == MXFP4)
        hipLaunchKernelGGL((quantize_mx_kernel<MXFP4, 1>), g1, dim3(kThreads), 0, stream, Xv, c, cw, sb, M, K8);
      else
        hipLaunchKernelGGL((quantize_mx_kernel<MXINT4, 1>), g1, dim3(kThreads), 0, stream, Xv, c, cw, sb, M, K8);
    }
  } else if (n_groups <= kNvSmallGroups) {
    hipLaunchKernelGGL(quantize_nv_small_kernel, grid, dim3(kThreads), 0, stream, Xv, c, t_act, cw, sb,
                       n_groups, K8);
  } else {
    float* partial = static_cast<float*>(workspace);
    const int nparts = int(std::min<int64_t>(kNvAmaxBlocks, (n_groups + kThreads - 1) / kThreads));
    hipLaunchKernelGGL(absmax_partial_kernel, dim3(nparts), dim3(kThreads), 0, stream, Xv, c,
                       partial, n_groups, K8);
    hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(kThreads), 0, stream, partial, nparts,
                       t_act);
    hipLaunchKernelGGL(quantize_nv_kernel, grid, dim3(kThreads), 0, stream, Xv, c, t_act, cw, sb,
                       n_groups, K8);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_act_multi(int fmt, int64_t M, int64_t K, const void* X, int P,
                                     const float* const* c, void* const* codes,
                                     void* const* scales, float* const* t_act, void* workspace,
                                     hipStream_t stream) {
  if (M == 0) return hipSuccess;
  MultiOut o{};
  for (int p = 0; p < P; ++p) {
    o.c[p] = c[p];
    o.codes[p] = static_cast<uint32_t*>(codes[p]);
    o.scales[p] = static_cast<uint8_t*>(scales[p]);
    o.t[p] = fmt == NVFP4 ? t_act[p] : nullptr;
    o.partial[p] = fmt == NVFP4 ? static_cast<float*>(workspace) + int64_t(p) * kNvAmaxBlocks : nullptr;
  }
  const uint4* Xv = static_cast<const uint4*>(X);
  switch (P) {
    case 1: return launch_multi<1>(fmt, M, K, Xv, o, stream);
    case 2: return launch_multi<2>(fmt, M, K, Xv, o, stream);
    case 3: return launch_multi<3>(fmt, M, K, Xv, o, stream);
    default: return launch_multi<4>(fmt, M, K, Xv, o, stream);
  }
}

}  // namespace w4a4
