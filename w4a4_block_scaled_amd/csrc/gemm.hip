// Block-scaled 4-bit x 4-bit GEMM with the row-scale epilogue, gfx950.
//
// DualQuant Section 4.4: Y = Q(X~) Q^T diag(r); Appendix I: the block scales
// are consumed inside the GEMM (no weight dequantization pass), the packed
// weights stay packed, and the entry point allocates nothing.
//
// Operand roles: the MFMA's first operand is the weight fragment (16 output
// features n) and its second the activation fragment (16 tokens m), so the
// accumulator of a lane holds 4 consecutive n of one m and the BF16 store of
// a lane is 8 contiguous bytes of a row of Y.
//
// Fragments: both operands are handled as 16-byte fragments = 32 consecutive
// K of one row (lane l: row l%16, K chunk l/16 of a 128-wide K-step), which
// is the operand layout of V_MFMA_SCALE_F32_16X16X128_F8F6F4.
//   MXFP4  : fragments go to the scaled MFMA as FP4 (E2M1) with the E8M0
//            block scales as the MFMA's per-lane scale bytes.
//   MXINT4 : each int4 code q is widened to the FP8 E4M3 byte that encodes
//            q * 2^-9 (|q| <= 8 lies in E4M3's linear subnormal/first-binade
//            range, so the widening is a byte table lookup), then the same
//            scaled MFMA runs in FP8 mode; the epilogue multiplies by 2^18.
//   NVFP4  : UE4M3 scales are not power-of-two, so the MFMA's E8M0 scale port
//            cannot apply them.  Each code is expanded to fp16 and multiplied
//            by its block scale in fp16 (code * scale has <= 6 significant
//            bits and lies in [2^-10, 2688]: exact), then the fp16 MFMA
//            (16x16x32) accumulates in fp32.  A lane feeds dword j of its
//            fragment to the j-th of four MFMAs; the same permutation of K
//            applies to both operands, so the dot products are unchanged.
#include "common.h"
#include "kernels.h"

namespace w4a4 {
namespace {

// ------------------------------------------------------------- MFMA ops --

__device__ __forceinline__ v4f mma_fp4(const uint4& w, const uint4& a, v4f acc, int sw, int sa) {
  const v8i A = {int(w.x), int(w.y), int(w.z), int(w.w), 0, 0, 0, 0};
  const v8i B = {int(a.x), int(a.y), int(a.z), int(a.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 4, 4, 0, sw, 0, sa);
}

// four int4 codes (low nibble of each byte) -> E4M3 bytes of q * 2^-9:
// q >= 0 -> byte q; q < 0 -> 0x80 | -q.
__device__ __forceinline__ uint32_t int4x4_to_e4m3(uint32_t nib) {
  const uint32_t neg_lo = 0x85868788u;  // nibbles 8..11 (q = -8..-5)
  const uint32_t neg_hi = 0x81828384u;  // nibbles 12..15 (q = -4..-1)
  const uint32_t neg = __builtin_amdgcn_perm(neg_hi, neg_lo, nib & 0x07070707u);
  const uint32_t sel = ((nib >> 1) & 0x04040404u) | 0x03020100u;
  return __builtin_amdgcn_perm(neg, nib, sel);
}

__device__ __forceinline__ v8i int4_frag_to_fp8(const uint4& f) {
  const uint32_t d[4] = {f.x, f.y, f.z, f.w};
  v8i r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = int(int4x4_to_e4m3(d[i] & 0x0f0f0f0fu));
    r[2 * i + 1] = int(int4x4_to_e4m3((d[i] >> 4) & 0x0f0f0f0fu));
  }
  return r;
}

__device__ __forceinline__ v4f mma_fp8(const v8i& w, const v8i& a, v4f acc, int sw, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, acc, 0, 0, 0, sw, 0, sa);
}

__device__ __forceinline__ v4f mma_int4(const uint4& w, const uint4& a, v4f acc, int sw, int sa) {
  return mma_fp8(int4_frag_to_fp8(w), int4_frag_to_fp8(a), acc, sw, sa);
}

// E4M3 byte -> its value as fp16 (exact)
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t b) {
  const int e = (b >> 3) & 15, m = b & 7;
  const float v = e == 0 ? ldexpf(float(m), -9) : ldexpf(float(8 + m), e - 10);
  return _Float16(v);
}

// 8 E2M1 codes (one dword) times an fp16 scale -> 8 fp16 values (exact)
__device__ __forceinline__ v8h e2m1x8_to_f16(uint32_t d, _Float16 s) {
  // high byte of the fp16 encoding of E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6
  // (the low byte is always 0)
  const uint32_t tlo = 0x3e3c3800u, thi = 0x46444240u;
  const uint32_t e = d & 0x0f0f0f0fu;
  const uint32_t o = (d >> 4) & 0x0f0f0f0fu;
  const uint32_t he = __builtin_amdgcn_perm(thi, tlo, e & 0x07070707u) | ((e & 0x08080808u) << 4);
  const uint32_t ho = __builtin_amdgcn_perm(thi, tlo, o & 0x07070707u) | ((o & 0x08080808u) << 4);
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 ss = {s, s};
  v8h out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t sel = 0x040c000cu + 0x01000100u * uint32_t(i);
    const uint32_t w = __builtin_amdgcn_perm(ho, he, sel);  // [0, he.b_i, 0, ho.b_i]
    const h2 v = __builtin_bit_cast(h2, w) * ss;
    out[2 * i] = v[0];
    out[2 * i + 1] = v[1];
  }
  return out;
}

__device__ __forceinline__ v4f mma_f16(const v8h& w, const v8h& a, v4f acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(w, a, acc, 0, 0, 0);
}

// --------------------------------------------------- activation fragments --

// 16-byte fragment of canonical activation codes for (row, K-step ks, lane
// group c), in the same arrangement as the packed weight tiles: FP4 formats
// take block c of the K-step; MXINT4 (FP8 MFMA operand order) takes half
// (c & 1) of block (c >> 1) and of block 2 + (c >> 1).
template <int FMT>
__device__ __forceinline__ uint4 load_act_frag(const uint8_t* __restrict__ rowp, int64_t ks, int c) {
  const uint8_t* p = rowp + ks * 64;
  if constexpr (FMT == MXINT4) {
    const int off = 16 * (c >> 1) + 8 * (c & 1);
    const uint2 lo = *reinterpret_cast<const uint2*>(p + off);
    const uint2 hi = *reinterpret_cast<const uint2*>(p + 32 + off);
    return uint4{lo.x, lo.y, hi.x, hi.y};
  } else {
    return *reinterpret_cast<const uint4*>(p + 16 * c);
  }
}

// ------------------------------------------------------- scale fetching --

// MX activation scale byte for (row m, K-step ks, chunk c): canonical [M x K/32]
__device__ __forceinline__ int act_scale_mx(const uint8_t* __restrict__ s, int64_t row, int64_t KB,
                                            int64_t ks, int c) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(s + row * KB + 4 * ks);
  return int(w >> (8 * c));
}

// NVFP4 activation scale pair for (row, ks, chunk c): bytes 8ks+2c, 8ks+2c+1 of [M x K/16]
__device__ __forceinline__ uint32_t act_scale_nv(const uint8_t* __restrict__ s, int64_t row,
                                                 int64_t KB, int64_t ks, int c) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(s + row * KB + 8 * ks + 4 * (c >> 1));
  return (w >> (16 * (c & 1))) & 0xffffu;
}

// ------------------------------------------------------------ epilogue --

// Y[m, n..n+3] = bf16(acc[i] * r[n+i] * f)
__device__ __forceinline__ void store4(uint16_t* __restrict__ Y, int64_t N, int64_t m, int64_t n,
                                       const v4f& acc, const float* __restrict__ R, float f) {
  const float4 r = *reinterpret_cast<const float4*>(R + n);
  const float rr[4] = {r.x, r.y, r.z, r.w};
  uint32_t b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = f32_to_bf16_rne(acc[i] * (rr[i] * f));
  uint2 v;
  v.x = b[0] | (b[1] << 16);
  v.y = b[2] | (b[3] << 16);
  *reinterpret_cast<uint2*>(Y + m * N + n) = v;
}

__device__ __forceinline__ float epilogue_factor(int fmt, const float* __restrict__ t_act,
                                                 const uint8_t* __restrict__ blob) {
  if (fmt == MXINT4) return 262144.0f;  // undo the 2^-9 of both FP8 widenings
  if (fmt == NVFP4) return *t_act * reinterpret_cast<const BlobHeader*>(blob)->t_w;
  return 1.0f;
}

// ======================================================== tiled kernel ==
//
// Workgroup tile: 128 n x 128 m, 4 waves as 2 (n) x 2 (m), wave tile 64 x 64
// (4 x 4 MFMA tiles).  K advances in stages of two 128-wide K-steps; both
// operands of a stage are staged through LDS in fragment order (16 KiB each,
// double-buffered), so every LDS read is one conflict-free 16-byte load per
// lane.  Global loads of stage s+1 are issued before the MFMAs of stage s.

constexpr int kTileThreads = 256;
constexpr int kTileM = 128, kTileN = 128;

// Global -> registers for one stage (two K-steps): 4 activation and 4 weight
// fragments per thread, indexed in LDS fragment order p = tid + 256 i:
// group g = p / 128 (16 rows), K-step p / 64 % 2, lane p % 64.
template <int FMT>
__device__ __forceinline__ void tile_load_stage(const uint8_t* __restrict__ a_codes,
                                                const uint4* __restrict__ Wc, int s, int tid,
                                                int64_t m0, int64_t ng0, int64_t M, int64_t NG,
                                                int64_t KS, int64_t K2, uint4 (&ra)[4],
                                                uint4 (&rw)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + 256 * i;
    const int g = p >> 7, ksl = (p >> 6) & 1, ln = p & 63;
    // out-of-range fragments load from a clamped valid address and are zeroed
    // afterwards (a select on the value, never on the address)
    const int64_t ks = 2 * int64_t(s) + ksl;
    const int64_t ksc = ks < KS ? ks : KS - 1;
    const int64_t row = m0 + g * 16 + (ln & 15);
    const int64_t rowc = row < M ? row : M - 1;
    const int64_t ng = ng0 + g;
    const int64_t ngc = ng < NG ? ng : NG - 1;
    const uint4 va = load_act_frag<FMT>(a_codes + rowc * K2, ksc, ln >> 4);
    const uint4 vw = Wc[(ngc * KS + ksc) * 64 + ln];
    const bool oka = row < M && ks < KS, okw = ng < NG && ks < KS;
    ra[i] = uint4{oka ? va.x : 0u, oka ? va.y : 0u, oka ? va.z : 0u, oka ? va.w : 0u};
    rw[i] = uint4{okw ? vw.x : 0u, okw ? vw.y : 0u, okw ? vw.z : 0u, okw ? vw.w : 0u};
  }
}

__device__ __forceinline__ void tile_store_stage(uint4 (*lds)[1024], int tid, const uint4 (&ra)[4],
                                                 const uint4 (&rw)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lds[0][tid + 256 * i] = ra[i];
    lds[1][tid + 256 * i] = rw[i];
  }
}

template <int FMT>
__device__ __forceinline__ void tile_load_scales(const uint8_t* __restrict__ a_scales,
                                                 const uint32_t* __restrict__ Ws, int s, int lane,
                                                 int64_t ng_base, int64_t NG, int64_t KG,
                                                 int64_t KS, int64_t KB, const int64_t (&arow)[4],
                                                 uint32_t (&sw)[4], uint32_t (&sa)[4][2]) {
  const int c = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t ng = ng_base + i;
    ng = ng < NG ? ng : NG - 1;
    const int64_t grp = FMT == NVFP4 ? int64_t(s) : int64_t(s) / 2;
    sw[i] = Ws[(ng * KG + grp) * 64 + lane];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int ksl = 0; ksl < 2; ++ksl) {
      const int64_t ks = 2 * int64_t(s) + ksl;
      if (ks < KS)
        sa[j][ksl] = FMT == NVFP4 ? act_scale_nv(a_scales, arow[j], KB, ks, c)
                                  : uint32_t(act_scale_mx(a_scales, arow[j], KB, ks, c));
      else
        sa[j][ksl] = 0;
    }
}

template <int FMT>
__global__ __launch_bounds__(kTileThreads) void gemm_tile_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ t_act, const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y,
    int64_t M, int64_t N, int64_t K, int tiles_n) {
  const BlobLayout L = blob_layout(FMT, N, K);
  const uint4* __restrict__ Wc = reinterpret_cast<const uint4*>(blob + L.code_off);
  const uint32_t* __restrict__ Ws = reinterpret_cast<const uint32_t*>(blob + L.scale_off);
  const float* __restrict__ R = reinterpret_cast<const float*>(blob + L.r_off);

  const int tn = blockIdx.x % tiles_n;
  const int tm = blockIdx.x / tiles_n;
  const int64_t m0 = int64_t(tm) * kTileM;
  const int64_t ng0 = int64_t(tn) * (kTileN / 16);

  __shared__ uint4 lds[2][2][1024];  // [buffer][0: activations, 1: weights][fragment]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int c = lane >> 4;
  const int64_t KS = L.KS, K2 = K / 2;
  const int64_t KB = K / block_size(FMT);
  const int nstages = int((KS + 1) / 2);

  uint4 ra[4], rw[4];
  uint32_t sw[4];     // weight scale dword per n-group (current stage)
  uint32_t sa[4][2];  // activation scale word per m-group and K-step (current stage)
  int64_t arow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t row = m0 + wm * 64 + j * 16 + (lane & 15);
    arow[j] = row < M ? row : M - 1;
  }

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  tile_load_stage<FMT>(a_codes, Wc, 0, tid, m0, ng0, M, L.NG, KS, K2, ra, rw);
  tile_store_stage(lds[0], tid, ra, rw);
  __syncthreads();

  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    tile_load_scales<FMT>(a_scales, Ws, s, lane, ng0 + wn * 4, L.NG, L.KG, KS, KB, arow, sw, sa);
    if (s + 1 < nstages) tile_load_stage<FMT>(a_codes, Wc, s + 1, tid, m0, ng0, M, L.NG, KS, K2, ra, rw);
#pragma unroll
    for (int ksl = 0; ksl < 2; ++ksl) {
      if (2 * int64_t(s) + ksl >= KS) break;
      uint4 wf[4], af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) wf[i] = lds[buf][1][(wn * 4 + i) * 128 + ksl * 64 + lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) af[j] = lds[buf][0][(wm * 4 + j) * 128 + ksl * 64 + lane];
      if (FMT == NVFP4) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          v8h wh[4], ah[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t d[4] = {wf[i].x, wf[i].y, wf[i].z, wf[i].w};
            const uint32_t sb = (sw[i] >> (8 * (2 * ksl + (jj >> 1)))) & 0xffu;
            wh[i] = e2m1x8_to_f16(d[jj], e4m3_to_f16(sb));
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t d[4] = {af[j].x, af[j].y, af[j].z, af[j].w};
            const uint32_t sb = (sa[j][ksl] >> (8 * (jj >> 1))) & 0xffu;
            ah[j] = e2m1x8_to_f16(d[jj], e4m3_to_f16(sb));
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mma_f16(wh[i], ah[j], acc[i][j]);
        }
      } else {
        const int shift = 8 * (((2 * s) & 3) + ksl);
        if (FMT == MXFP4) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[i][j] = mma_fp4(wf[i], af[j], acc[i][j], int(sw[i] >> shift), int(sa[j][ksl]));
        } else {
          v8i w8[4], a8[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            w8[i] = int4_frag_to_fp8(wf[i]);
            a8[i] = int4_frag_to_fp8(af[i]);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[i][j] = mma_fp8(w8[i], a8[j], acc[i][j], int(sw[i] >> shift), int(sa[j][ksl]));
        }
      }
    }
    if (s + 1 < nstages) tile_store_stage(lds[buf ^ 1], tid, ra, rw);
    __syncthreads();
  }

  const float f = epilogue_factor(FMT, t_act, blob);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t ng = ng0 + wn * 4 + i;
    if (ng >= L.NG) continue;
    const int64_t n = ng * 16 + 4 * c;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t m = m0 + wm * 64 + j * 16 + (lane & 15);
      if (m < M) store4(Y, N, m, n, acc[i][j], R, f);
    }
  }
}

// ====================================================== decode kernel ==
//
// M <= 16 (MX formats): weight streaming.  One workgroup per 16 output
// features; its waves split K into contiguous ranges and stream the weight
// fragments straight from HBM into registers (one coalesced 16-byte load
// per lane per 128-wide K-step, no LDS).  The activation rows (<= 16) are
// the MFMA's second operand; rows >= M are zero.  Partial sums of the waves
// are added through LDS and wave 0 runs the epilogue.

constexpr int kDecodeWaves = 4;
constexpr int kDecodeUnroll = 4;

template <int FMT>
__global__ __launch_bounds__(64 * kDecodeWaves) void gemm_decode_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K) {
  const BlobLayout L = blob_layout(FMT, N, K);
  const uint4* __restrict__ Wc = reinterpret_cast<const uint4*>(blob + L.code_off);
  const uint32_t* __restrict__ Ws = reinterpret_cast<const uint32_t*>(blob + L.scale_off);
  const float* __restrict__ R = reinterpret_cast<const float*>(blob + L.r_off);

  const int64_t ng = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane >> 4;
  const int64_t m = lane & 15;
  const bool mvalid = m < M;
  const int64_t row = mvalid ? m : 0;
  const int64_t KS = L.KS, K2 = K / 2, KB = K / 32;
  const int64_t per = (KS + kDecodeWaves - 1) / kDecodeWaves;
  const int64_t k_begin = wave * per;
  const int64_t k_end = k_begin + per < KS ? k_begin + per : KS;

  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = k_begin; k0 < k_end; k0 += kDecodeUnroll) {
    uint4 wf[kDecodeUnroll], af[kDecodeUnroll];
    uint32_t swd[kDecodeUnroll];
    int sab[kDecodeUnroll];
#pragma unroll
    for (int u = 0; u < kDecodeUnroll; ++u) {
      const int64_t ks = k0 + u;
      const bool ok = ks < k_end;
      const int64_t ksc = ok ? ks : k_end - 1;  // clamped: loads stay in range
      const uint4 w = Wc[(ng * KS + ksc) * 64 + lane];
      const uint4 a = load_act_frag<FMT>(a_codes + row * K2, ksc, c);
      const bool oka = ok && mvalid;
      wf[u] = uint4{ok ? w.x : 0u, ok ? w.y : 0u, ok ? w.z : 0u, ok ? w.w : 0u};
      af[u] = uint4{oka ? a.x : 0u, oka ? a.y : 0u, oka ? a.z : 0u, oka ? a.w : 0u};
      swd[u] = Ws[(ng * L.KG + ksc / 4) * 64 + lane] >> (8 * (ksc & 3));
      sab[u] = act_scale_mx(a_scales, row, KB, ksc, c);
    }
#pragma unroll
    for (int u = 0; u < kDecodeUnroll; ++u)
      acc = FMT == MXFP4 ? mma_fp4(wf[u], af[u], acc, int(swd[u]), sab[u])
                         : mma_int4(wf[u], af[u], acc, int(swd[u]), sab[u]);
  }

  __shared__ v4f red[kDecodeWaves][64];
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < kDecodeWaves; ++w) {
    const v4f o = red[w][lane];
    acc[0] += o[0];
    acc[1] += o[1];
    acc[2] += o[2];
    acc[3] += o[3];
  }
  if (mvalid) store4(Y, N, m, ng * 16 + 4 * c, acc, R, epilogue_factor(FMT, nullptr, blob));
}

template <int FMT>
hipError_t launch_fmt(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                      const float* t_act, const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  if constexpr (FMT != NVFP4) {
    if (M <= 16) {
      hipLaunchKernelGGL(gemm_decode_kernel<FMT>, dim3(unsigned(N / 16)), dim3(64 * kDecodeWaves),
                         0, stream, ac, as, blob, Y, M, N, K);
      return hipGetLastError();
    }
  }
  const int tiles_n = int((N + kTileN - 1) / kTileN);
  const int tiles_m = int((M + kTileM - 1) / kTileM);
  hipLaunchKernelGGL(gemm_tile_kernel<FMT>, dim3(unsigned(tiles_n * tiles_m)), dim3(kTileThreads),
                     0, stream, ac, as, t_act, blob, Y, M, N, K, tiles_n);
  return hipGetLastError();
}

}  // namespace

size_t linear_workspace_bytes(int, int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_linear(int fmt, int64_t M, int64_t N, int64_t K, const void* a_codes,
                         const void* a_scales, const float* t_act, const void* blob, void* Y,
                         void*, size_t, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const uint8_t* ac = static_cast<const uint8_t*>(a_codes);
  const uint8_t* as = static_cast<const uint8_t*>(a_scales);
  const uint8_t* b = static_cast<const uint8_t*>(blob);
  uint16_t* y = static_cast<uint16_t*>(Y);
  switch (fmt) {
    case MXFP4: return launch_fmt<MXFP4>(M, N, K, ac, as, t_act, b, y, stream);
    case MXINT4: return launch_fmt<MXINT4>(M, N, K, ac, as, t_act, b, y, stream);
    default: return launch_fmt<NVFP4>(M, N, K, ac, as, t_act, b, y, stream);
  }
}

}  // namespace w4a4
