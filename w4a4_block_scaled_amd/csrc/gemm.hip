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
// Fragments: both operands are handled as 16-byte fragments = 32 codes of one
// row for a 128-wide K-step (lane l: row l%16).
//   MXFP4  : fragments go to V_MFMA_SCALE_F32_16X16X128_F8F6F4 as FP4 (E2M1);
//            lane group c = l/16 holds block c of the K-step, and the E8M0
//            block scales are the MFMA's per-lane scale bytes.
//   MXINT4 : each int4 code q is widened to the FP8 E4M3 byte that encodes
//            q * 2^-9 (|q| <= 8 lies in E4M3's linear subnormal/first-binade
//            range, so the widening is a byte permutation), then the same
//            scaled MFMA runs in FP8 mode and the epilogue multiplies by 2^18.
//            With FP8 operands lane group c takes K 16c..16c+15 and
//            64+16c..64+16c+15, so its fragment carries half (c & 1) of blocks
//            c >> 1 and 2 + (c >> 1).
//   NVFP4  : UE4M3 scales are not powers of two, so the MFMA's E8M0 scale port
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

#define LDS __attribute__((address_space(3)))
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------- MFMA ops --

template <int OPW>
__device__ __forceinline__ v4f mfma_fp4_op(const u32x4& w, const u32x4& a, v4f acc, int sw,
                                           int sa) {
  const v8i A = {int(w.x), int(w.y), int(w.z), int(w.w), 0, 0, 0, 0};
  const v8i B = {int(a.x), int(a.y), int(a.z), int(a.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 4, 4, OPW, sw, 0, sa);
}

template <int OPW>
__device__ __forceinline__ v4f mfma_fp8_op(const v8i& w, const v8i& a, v4f acc, int sw, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, acc, 0, 0, OPW, sw, 0, sa);
}

// byte `opw` of the weight scale word selects the scale (folded after unrolling)
__device__ __forceinline__ v4f mfma_fp4(int opw, const u32x4& w, const u32x4& a, v4f acc, int sw,
                                        int sa) {
  switch (opw & 3) {
    case 0: return mfma_fp4_op<0>(w, a, acc, sw, sa);
    case 1: return mfma_fp4_op<1>(w, a, acc, sw, sa);
    case 2: return mfma_fp4_op<2>(w, a, acc, sw, sa);
    default: return mfma_fp4_op<3>(w, a, acc, sw, sa);
  }
}

__device__ __forceinline__ v4f mfma_fp8(int opw, const v8i& w, const v8i& a, v4f acc, int sw,
                                        int sa) {
  switch (opw & 3) {
    case 0: return mfma_fp8_op<0>(w, a, acc, sw, sa);
    case 1: return mfma_fp8_op<1>(w, a, acc, sw, sa);
    case 2: return mfma_fp8_op<2>(w, a, acc, sw, sa);
    default: return mfma_fp8_op<3>(w, a, acc, sw, sa);
  }
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

__device__ __forceinline__ v8i int4_frag_to_fp8(const u32x4& f) {
  v8i r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = int(int4x4_to_e4m3(f[i] & 0x0f0f0f0fu));
    r[2 * i + 1] = int(int4x4_to_e4m3((f[i] >> 4) & 0x0f0f0f0fu));
  }
  return r;
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

__device__ __forceinline__ v4f mfma_f16(const v8h& w, const v8h& a, v4f acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(w, a, acc, 0, 0, 0);
}

// --------------------------------------------------- activation fragments --

// 16-byte fragment of canonical activation codes for (row, K-step ks, lane
// group c) in the operand arrangement of the format (see the file header).
template <int FMT>
__device__ __forceinline__ u32x4 load_act_frag(const uint8_t* __restrict__ rowp, int64_t ks, int c) {
  const uint8_t* p = rowp + ks * 64;
  if constexpr (FMT == MXINT4) {
    const int off = 16 * (c >> 1) + 8 * (c & 1);
    const u32x2 lo = *reinterpret_cast<const u32x2*>(p + off);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 32 + off);
    return u32x4{lo.x, lo.y, hi.x, hi.y};
  } else {
    return *reinterpret_cast<const u32x4*>(p + 16 * c);
  }
}

// MX activation scale byte for (row, K-step ks, lane group c): canonical [M x K/32]
__device__ __forceinline__ int act_scale_mx(const uint8_t* __restrict__ s, int64_t row, int64_t KB,
                                            int64_t ks, int c) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(s + row * KB + 4 * ks);
  return int(w >> (8 * c));
}

// ------------------------------------------------------------ epilogue --

typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16, round to nearest even (one V_CVT_PK_BF16_F32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, bf2));
}

// bf16(acc[i] * rs[i]) for i = 0..3, packed
__device__ __forceinline__ u32x2 scale_pack4(const v4f& acc, const v4f& rs) {
  return u32x2{pack_bf16x2(acc[0] * rs[0], acc[1] * rs[1]),
               pack_bf16x2(acc[2] * rs[2], acc[3] * rs[3])};
}

// Y[m, n..n+3] = bf16(acc[i] * rs[i]) with rs = r[n..n+3] * f
__device__ __forceinline__ void store4(uint16_t* __restrict__ Y, int64_t N, int64_t m, int64_t n,
                                       const v4f& acc, const v4f& rs) {
  *reinterpret_cast<u32x2*>(Y + m * N + n) = scale_pack4(acc, rs);
}

__device__ __forceinline__ float epilogue_factor(int fmt, const float* __restrict__ t_act,
                                                 const uint8_t* __restrict__ blob) {
  if (fmt == MXINT4) return 262144.0f;  // undo the 2^-9 of both FP8 widenings
  if (fmt == NVFP4) return *t_act * reinterpret_cast<const BlobHeader*>(blob)->t_w;
  return 1.0f;
}

// ======================================================== tiled kernel ==
//
// Workgroup tile BN (n) x BM (m), WN x WM waves (n x m), wave tile
// BN/WN x BM/WM.  Each 128-wide K-step is one pipeline stage.  A stage's
// operands (activation fragments, weight tiles, activation scales, weight
// scale words) are copied global -> LDS by the waves' direct-to-LDS loads
// (global_load_lds, no VGPR staging) into a ring of DEPTH stage buffers; up
// to DEPTH-1 stages are in flight while the MFMAs consume the oldest one.
// Every wave issues the same number of copy instructions per stage, so a
// stage is complete for a wave when its vmcnt has dropped to (stages issued
// after it) x (copies per stage); an s_barrier then makes it complete for
// the workgroup and also frees the buffer computed in the previous step.
//
// LDS stage buffer layout:
//   [A codes: BM/16 fragments x 64 lanes x 16 B, FP4 fragment order]
//   [W codes: BN/16 tiles x 1 KiB, copied from the blob as is]
//   [A scales: BM rows x (4 B MX | 8 B NVFP4): this K-step's scale bytes]
//   [W scale words: groups x 64 lanes x 4 B]
// Rows beyond M and row groups beyond N/16 are loaded from clamped valid
// addresses; they only feed outputs that are never stored.

template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
struct TileCfg {
  static constexpr int WAVES = WN * WM;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int FN = BN / 16 / WN;  // weight fragments per wave
  static constexpr int FM = BM / 16 / WM;  // activation fragments per wave
  static constexpr int GPW = groups_per_scale_word(FMT);
  static constexpr int ASB = FMT == NVFP4 ? 8 : 4;  // activation scale bytes per row per K-step
  static constexpr int A_BYTES = BM * 64;
  static constexpr int W_BYTES = BN * 64;
  static constexpr int AS_BYTES = BM * ASB;
  static constexpr int WS_BYTES = (BN / 16 / GPW) * 256;
  static constexpr int STAGE = A_BYTES + W_BYTES + AS_BYTES + WS_BYTES;
  static constexpr int A_DMA = BM / 16 / WAVES;  // 1 KiB copies per wave
  static constexpr int W_DMA = BN / 16 / WAVES;
  static constexpr int AS_DW = AS_BYTES / 4 / WAVES;  // scale dwords per wave
  static constexpr int WS_DW = WS_BYTES / 4 / WAVES;
  static constexpr int AS_DMA = (AS_DW + 63) / 64;
  static constexpr int WS_DMA = (WS_DW + 63) / 64;
  static constexpr int COPIES = A_DMA + W_DMA + AS_DMA + WS_DMA;  // per wave per stage
  static_assert(A_DMA * WAVES * 16 == BM && W_DMA * WAVES * 16 == BN, "tile / wave split");
  static_assert(FN % GPW == 0, "scale words per wave");
  static_assert(AS_DW <= 64 || AS_DW % 64 == 0, "activation scale copy split");
  static_assert(WS_DW <= 64 || WS_DW % 64 == 0, "weight scale copy split");
  static_assert(DEPTH * STAGE <= 160 * 1024, "LDS");
};

__device__ __forceinline__ constexpr int vmcnt_encoding(int v) {
  // s_waitcnt simm16 on gfx9: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]
  return (v & 15) | (7 << 4) | (15 << 8) | (((v >> 4) & 3) << 14);
}

// Wait until at most `after` stages (of C copies each) are outstanding for
// this wave, then barrier.  The asm statement keeps LDS reads below it.
template <int C, int DEPTH>
__device__ __forceinline__ void stage_ready(int after) {
  static_assert((DEPTH - 2) * C < 64 && DEPTH <= 6, "vmcnt range");
  switch (after) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_encoding(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_encoding(C)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_encoding(2 * C)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_encoding(3 * C)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_encoding(4 * C)); break;
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct TileArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint4* Wc;
  const uint32_t* Ws;
  int64_t M, K2, KB, KS, NG, NSG;
  int64_t m0, ng0;
};

// Copy the operands of K-step ks into stage buffer `dst` (this wave's share).
template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
__device__ __forceinline__ void issue_stage(const TileArgs& t, int64_t ks, LDS uint8_t* dst,
                                            int wave, int lane) {
  using C = TileCfg<FMT, BN, BM, WN, WM, DEPTH>;
  const int r = lane & 15, c = lane >> 4;
  // activation fragments (FP4 fragment order for every format)
#pragma unroll
  for (int i = 0; i < C::A_DMA; ++i) {
    const int f = wave * C::A_DMA + i;
    int64_t row = t.m0 + 16 * f + r;
    row = row < t.M ? row : t.M - 1;
    __builtin_amdgcn_global_load_lds(t.a_codes + row * t.K2 + ks * 64 + 16 * c,
                                     dst + f * 1024, 16, 0, 0);
  }
  // weight tiles
  LDS uint8_t* wdst = dst + C::A_BYTES;
#pragma unroll
  for (int i = 0; i < C::W_DMA; ++i) {
    const int f = wave * C::W_DMA + i;
    int64_t ng = t.ng0 + f;
    ng = ng < t.NG ? ng : t.NG - 1;
    __builtin_amdgcn_global_load_lds(t.Wc + (ng * t.KS + ks) * 64 + lane, wdst + f * 1024, 16, 0, 0);
  }
  // activation scales: dword d of the strip = row d / (ASB/4), part d % (ASB/4)
  LDS uint8_t* asdst = wdst + C::W_BYTES;
#pragma unroll
  for (int i = 0; i < C::AS_DMA; ++i) {
    const int d = wave * C::AS_DW + i * 64 + lane;
    if (C::AS_DW >= 64 || lane < C::AS_DW) {
      constexpr int parts = C::ASB / 4;
      int64_t row = t.m0 + d / parts;
      row = row < t.M ? row : t.M - 1;
      __builtin_amdgcn_global_load_lds(t.a_scales + row * t.KB + ks * C::ASB + 4 * (d % parts),
                                       asdst + (wave * C::AS_DW + i * 64) * 4, 4, 0, 0);
    }
  }
  // weight scale words: dword d = group d / 64, lane d % 64
  LDS uint8_t* wsdst = asdst + C::AS_BYTES;
#pragma unroll
  for (int i = 0; i < C::WS_DMA; ++i) {
    const int d = wave * C::WS_DW + i * 64 + lane;
    if (C::WS_DW >= 64 || lane < C::WS_DW) {
      int64_t sg = t.ng0 / C::GPW + d / 64;
      sg = sg < t.NSG ? sg : t.NSG - 1;
      __builtin_amdgcn_global_load_lds(t.Ws + (sg * t.KS + ks) * 64 + (d & 63),
                                       wsdst + (wave * C::WS_DW + i * 64) * 4, 4, 0, 0);
    }
  }
}

// One pipeline step: start the copy of K-step `ks_next` into `nxt` (if any),
// then run the MFMAs of the stage held in `cur`.  The two buffers are
// distinct, which the restrict qualifiers state; the ordering against copies
// of earlier steps is enforced by stage_ready().
template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
__device__ __forceinline__ void tile_step(const TileArgs& t, const LDS uint8_t* __restrict__ cur,
                                          LDS uint8_t* __restrict__ nxt, int64_t ks_next,
                                          bool issue, int wave, int lane,
                                          v4f (&acc)[BN / 16 / WN][BM / 16 / WM]) {
  using C = TileCfg<FMT, BN, BM, WN, WM, DEPTH>;
  constexpr int FN = C::FN, FM = C::FM;
  if (issue) issue_stage<FMT, BN, BM, WN, WM, DEPTH>(t, ks_next, nxt, wave, lane);

  const int wn = wave % WN, wm = wave / WN;
  const int r = lane & 15, c = lane >> 4;
  const LDS u32x4* A = reinterpret_cast<const LDS u32x4*>(cur);
  const LDS u32x4* W = reinterpret_cast<const LDS u32x4*>(cur + C::A_BYTES);
  const LDS uint8_t* AS = cur + C::A_BYTES + C::W_BYTES;
  const LDS uint32_t* WS = reinterpret_cast<const LDS uint32_t*>(AS + C::AS_BYTES);

  u32x4 wf[FN];
#pragma unroll
  for (int i = 0; i < FN; ++i) wf[i] = W[(wn * FN + i) * 64 + lane];
  uint32_t sw[FN / C::GPW];
#pragma unroll
  for (int q = 0; q < FN / C::GPW; ++q) sw[q] = WS[(wn * FN / C::GPW + q) * 64 + lane];

  if constexpr (FMT == MXFP4) {
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int f = wm * FM + j;
      const u32x4 af = A[f * 64 + lane];
      const int sa = AS[(16 * f + r) * 4 + c];
#pragma unroll
      for (int i = 0; i < FN; ++i)
        acc[i][j] = mfma_fp4(i % 4, wf[i], af, acc[i][j], int(sw[i / 4]), sa);
    }
  } else if constexpr (FMT == MXINT4) {
    v8i w8[FN];
#pragma unroll
    for (int i = 0; i < FN; ++i) w8[i] = int4_frag_to_fp8(wf[i]);
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int f = wm * FM + j;
      // MXINT4 operand order from the FP4-ordered LDS copy: half (c & 1) of
      // blocks c >> 1 and 2 + (c >> 1) of row r
      const LDS u32x2* base = reinterpret_cast<const LDS u32x2*>(A + f * 64);
      const u32x2 lo = base[(r + 16 * (c >> 1)) * 2 + (c & 1)];
      const u32x2 hi = base[(r + 16 * (2 + (c >> 1))) * 2 + (c & 1)];
      const v8i a8 = int4_frag_to_fp8(u32x4{lo.x, lo.y, hi.x, hi.y});
      const int sa = AS[(16 * f + r) * 4 + c];
#pragma unroll
      for (int i = 0; i < FN; ++i)
        acc[i][j] = mfma_fp8(i % 4, w8[i], a8, acc[i][j], int(sw[i / 4]), sa);
    }
  } else {  // NVFP4: fp16 MFMA, four per K-step
    u32x4 af[FM];
    uint32_t sa[FM];
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int f = wm * FM + j;
      af[j] = A[f * 64 + lane];
      sa[j] = *reinterpret_cast<const LDS uint16_t*>(AS + (16 * f + r) * 8 + 2 * c);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      v8h wh[FN];
#pragma unroll
      for (int i = 0; i < FN; ++i)
        wh[i] = e2m1x8_to_f16(wf[i][jj],
                              e4m3_to_f16((sw[i / 2] >> (8 * (2 * (i % 2) + (jj >> 1)))) & 0xffu));
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const v8h ah = e2m1x8_to_f16(af[j][jj], e4m3_to_f16((sa[j] >> (8 * (jj >> 1))) & 0xffu));
#pragma unroll
        for (int i = 0; i < FN; ++i) acc[i][j] = mfma_f16(wh[i], ah, acc[i][j]);
      }
    }
  }
}

template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
__global__ __launch_bounds__(64 * WN * WM, 1) void gemm_tile_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ t_act, const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y,
    int64_t M, int64_t N, int64_t K, int tiles_m, int tiles_total, int per_xcd) {
  using C = TileCfg<FMT, BN, BM, WN, WM, DEPTH>;
  constexpr int FN = C::FN, FM = C::FM;
  // XCD-aware order: the hardware deals workgroups round-robin to the 8 XCDs;
  // give each XCD a contiguous run of tiles (m fastest), so the workgroups
  // sharing an L2 share weight tiles and sweep the activations.
  const int tile = int(blockIdx.x % 8) * per_xcd + int(blockIdx.x / 8);
  if (tile >= tiles_total) return;
  const int tm = tile % tiles_m, tn = tile / tiles_m;

  const BlobLayout L = blob_layout(FMT, N, K);
  TileArgs t;
  t.a_codes = a_codes;
  t.a_scales = a_scales;
  t.Wc = reinterpret_cast<const uint4*>(blob + L.code_off);
  t.Ws = reinterpret_cast<const uint32_t*>(blob + L.scale_off);
  t.M = M;
  t.K2 = K / 2;
  t.KB = K / block_size(FMT);
  t.KS = L.KS;
  t.NG = L.NG;
  t.NSG = L.NSG;
  t.m0 = int64_t(tm) * BM;
  t.ng0 = int64_t(tn) * (BN / 16);

  __shared__ __attribute__((aligned(1024))) uint8_t smem[DEPTH * C::STAGE];
  LDS uint8_t* base = (LDS uint8_t*)smem;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  v4f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int64_t KS = L.KS;
#pragma unroll
  for (int s = 0; s < DEPTH - 1; ++s)
    if (s < KS) issue_stage<FMT, BN, BM, WN, WM, DEPTH>(t, s, base + s * C::STAGE, wave, lane);

  for (int64_t s = 0; s < KS; ++s) {
    const int64_t after = KS - 1 - s < DEPTH - 2 ? KS - 1 - s : DEPTH - 2;
    stage_ready<C::COPIES, DEPTH>(int(after));
    const int64_t nx = s + DEPTH - 1;
    tile_step<FMT, BN, BM, WN, WM, DEPTH>(t, base + (s % DEPTH) * C::STAGE,
                                          base + (nx % DEPTH) * C::STAGE, nx, nx < KS, wave, lane,
                                          acc);
  }

  const float* __restrict__ R = reinterpret_cast<const float*>(blob + L.r_off);
  const float f = epilogue_factor(FMT, t_act, blob);
  const int wn = wave % WN, wm = wave / WN;
  v4f rs[FN];
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    int64_t ng = t.ng0 + wn * FN + i;
    ng = ng < L.NG ? ng : L.NG - 1;
    const float4 r = *reinterpret_cast<const float4*>(R + ng * 16 + 4 * (lane >> 4));
    rs[i] = v4f{r.x * f, r.y * f, r.z * f, r.w * f};
  }
  // Epilogue through LDS: every wave writes its BF16 tile (WMT rows x WNT
  // columns) into its own region of the now idle stage ring, 16-byte chunks of
  // a row XOR-swizzled by the row index (conflict-free writes of the MFMA
  // layout), then reads it back row-major and stores full 16-byte chunks.
  constexpr int WNT = BN / WN, WMT = BM / WM;  // wave tile: n x m
  constexpr int CH = WNT / 8;                  // 16-byte chunks per row
  constexpr int ROWB = 2 * WNT;
  static_assert(WN * WM * WMT * ROWB <= DEPTH * C::STAGE, "epilogue staging");
  __builtin_amdgcn_s_barrier();  // every wave is done with the stage buffers
  asm volatile("" ::: "memory");
  LDS uint8_t* ep = base + wave * (WMT * ROWB);
  const int c = lane >> 4;
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int m = 16 * j + (lane & 15);
      const int chunk = 2 * i + (c >> 1);
      const int off = m * ROWB + ((chunk ^ (m % CH)) * 16) + 8 * (c & 1);
      *reinterpret_cast<LDS u32x2*>(ep + off) = scale_pack4(acc[i][j], rs[i]);
    }
  const int64_t nbase = (t.ng0 + wn * FN) * 16;
  const int64_t mbase = t.m0 + wm * WMT;
#pragma unroll
  for (int q = 0; q < WMT * CH / 64; ++q) {
    const int idx = q * 64 + lane;
    const int row = idx / CH, chunk = idx % CH;
    const u32x4 v = *reinterpret_cast<const LDS u32x4*>(ep + row * ROWB + ((chunk ^ (row % CH)) * 16));
    const int64_t m = mbase + row, n = nbase + 8 * chunk;
    if (m < M && n < N) *reinterpret_cast<u32x4*>(Y + m * N + n) = v;
  }
}

// ====================================================== decode kernel ==
//
// M <= 16 (MX formats): weight streaming.  One workgroup per 16 output
// features; its waves split K into contiguous ranges and stream the weight
// tiles straight from HBM into registers (one coalesced 16-byte load per
// lane per K-step, no LDS).  The activation rows (<= 16) are the MFMA's second
// operand; rows >= M are zero.  Partial sums of the waves are added through
// LDS and wave 0 runs the epilogue.

constexpr int kDecodeWaves = 4;
constexpr int kDecodeUnroll = 4;

template <int FMT>
__global__ __launch_bounds__(64 * kDecodeWaves) void gemm_decode_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K) {
  const BlobLayout L = blob_layout(FMT, N, K);
  const u32x4* __restrict__ Wc = reinterpret_cast<const u32x4*>(blob + L.code_off);
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
  const int sw_shift = 8 * int(ng & 3);
  const uint32_t* __restrict__ Wsg = Ws + (ng >> 2) * KS * 64 + lane;

  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = k_begin; k0 < k_end; k0 += kDecodeUnroll) {
    u32x4 wf[kDecodeUnroll], af[kDecodeUnroll];
    uint32_t swd[kDecodeUnroll];
    int sab[kDecodeUnroll];
#pragma unroll
    for (int u = 0; u < kDecodeUnroll; ++u) {
      const int64_t ks = k0 + u;
      const bool ok = ks < k_end;
      const int64_t ksc = ok ? ks : k_end - 1;  // clamped: loads stay in range
      const u32x4 w = Wc[(ng * KS + ksc) * 64 + lane];
      const u32x4 a = load_act_frag<FMT>(a_codes + row * K2, ksc, c);
      const bool oka = ok && mvalid;
      wf[u] = ok ? w : u32x4{0u, 0u, 0u, 0u};
      af[u] = oka ? a : u32x4{0u, 0u, 0u, 0u};
      swd[u] = Wsg[ksc * 64] >> sw_shift;
      sab[u] = act_scale_mx(a_scales, row, KB, ksc, c);
    }
#pragma unroll
    for (int u = 0; u < kDecodeUnroll; ++u) {
      if constexpr (FMT == MXFP4)
        acc = mfma_fp4_op<0>(wf[u], af[u], acc, int(swd[u]), sab[u]);
      else
        acc = mfma_fp8_op<0>(int4_frag_to_fp8(wf[u]), int4_frag_to_fp8(af[u]), acc, int(swd[u]),
                             sab[u]);
    }
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
  const float f = epilogue_factor(FMT, nullptr, blob);
  const float4 r = *reinterpret_cast<const float4*>(R + ng * 16 + 4 * c);
  if (mvalid) store4(Y, N, m, ng * 16 + 4 * c, acc, v4f{r.x * f, r.y * f, r.z * f, r.w * f});
}

template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
hipError_t launch_tile(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                       const float* t_act, const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  const int tiles_n = int((N + BN - 1) / BN);
  const int tiles_m = int((M + BM - 1) / BM);
  const int total = tiles_n * tiles_m;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL((gemm_tile_kernel<FMT, BN, BM, WN, WM, DEPTH>), dim3(unsigned(per_xcd * 8)),
                     dim3(64 * WN * WM), 0, stream, ac, as, t_act, blob, Y, M, N, K, tiles_m, total,
                     per_xcd);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                      const float* t_act, const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  if constexpr (FMT == NVFP4) {
    // NVFP4 runs four fp16 MFMAs per fragment pair, so its K-step is long
    // enough for 64 x 64 wave tiles at any shape, and it holds expanded fp16
    // fragments that would not fit the register budget of a 128 x 64 tile.
    return launch_tile<FMT, 256, 128, 4, 2, 5>(M, N, K, ac, as, t_act, blob, Y, stream);
  } else {
    if (M <= 16) {
      hipLaunchKernelGGL(gemm_decode_kernel<FMT>, dim3(unsigned(N / 16)), dim3(64 * kDecodeWaves),
                         0, stream, ac, as, blob, Y, M, N, K);
      return hipGetLastError();
    }
    // 8 waves per workgroup (two per SIMD, so one wave's memory and barrier
    // stalls are covered by the other's MFMAs).  256x256 tiles (waves 2 x 4,
    // 128 x 64 each) unless that leaves more than ~30% of the 256 CUs idle;
    // then 256 (n) x 128 (m) tiles (waves 4 x 2, 64 x 64 each).
    const int64_t big = ((N + 255) / 256) * ((M + 255) / 256);
    if (big >= 180)
      return launch_tile<FMT, 256, 256, 2, 4, 4>(M, N, K, ac, as, t_act, blob, Y, stream);
    return launch_tile<FMT, 256, 128, 4, 2, 5>(M, N, K, ac, as, t_act, blob, Y, stream);
  }
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
