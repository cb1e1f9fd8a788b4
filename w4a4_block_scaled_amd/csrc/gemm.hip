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
#include "w4a4.h"
#include "common.h"
#include "kernels.h"

#include <mutex>

namespace w4a4 {
namespace {

#define LDS __attribute__((address_space(3)))
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// Direct-to-LDS copies: 16 (4) bytes per lane from `src`, lane l writing
// `dst` + 16 l (4 l); `dst` is wave-uniform.
// Activation tiles (16 rows x the 64 bytes of one 128-wide K-step) are
// copied with lane l taking row l / 4 and 16-byte chunk (l % 4) ^ fp4_swz(l
// / 4): four consecutive lanes read the 64 contiguous bytes of one row (one
// request per lane quad instead of four), and the LDS tile holds chunk c of
// row r at 16-byte position a_tile_pos(r, c) = 4 r + (c ^ fp4_swz(r)).  The
// swizzle keeps the fragment reads (16 consecutive rows, one chunk) free of
// bank conflicts for 32 and for 64 LDS banks.
__device__ __forceinline__ int fp4_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
__device__ __forceinline__ int a_tile_pos(int r, int c) { return 4 * r + (c ^ fp4_swz(r)); }

__device__ __forceinline__ void lds_copy16(const void* src, LDS void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}
__device__ __forceinline__ void lds_copy4(const void* src, LDS void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
}

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

// A constant in a VGPR that the compiler cannot see through.  Three-operand
// (VOP3) instructions take no literal here and at most one SGPR, so with the
// constants in VGPRs `(x & c) | c'` becomes one v_and_or_b32 and v_perm_b32
// reads both table words from registers; with literals the compiler splits
// them into two instructions.  Free of side effects, so the copies are hoisted
// out of loops and merged.
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
  uint32_t v;
  asm("v_mov_b32 %0, %1" : "=v"(v) : "i"(c));
  return v;
}

// four int4 codes (the low nibbles of the bytes of `d`; the high nibbles are
// ignored) -> E4M3 bytes of q * 2^-9: q >= 0 -> byte q; q < 0 -> 0x80 | -q.
// Five instructions: the low three bits index the table of negative codes,
// and bit 3 selects, per byte, that entry or the three bits themselves.
__device__ __forceinline__ uint32_t int4x4_to_e4m3(uint32_t d) {
  const uint32_t neg_lo = vgpr_const(0x85868788u);  // nibbles 8..11 (q = -8..-5)
  const uint32_t neg_hi = vgpr_const(0x81828384u);  // nibbles 12..15 (q = -4..-1)
  const uint32_t g = d & 0x07070707u;
  const uint32_t neg = __builtin_amdgcn_perm(neg_hi, neg_lo, g);
  const uint32_t sel = ((d >> 1) & vgpr_const(0x04040404u)) | vgpr_const(0x03020100u);
  return __builtin_amdgcn_perm(neg, g, sel);
}

// int4 codes biased by 8 (u = q + 8 in 0..15, the code with bit 3 flipped):
// the E4M3 byte u encodes u * 2^-9 exactly (subnormals 0..7 and the first
// binade 8..15 are evenly spaced), so no table is needed.  Same byte order
// as int4_frag_to_fp8.
__device__ __forceinline__ v8i int4_frag_biased_fp8(const u32x4& f) {
  v8i r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = f[i] ^ 0x88888888u;
    r[2 * i] = int(x & 0x0f0f0f0fu);
    r[2 * i + 1] = int((x >> 4) & 0x0f0f0f0fu);
  }
  return r;
}

__device__ __forceinline__ v8i int4_frag_to_fp8(const u32x4& f) {
  v8i r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = int(int4x4_to_e4m3(f[i]));
    r[2 * i + 1] = int(int4x4_to_e4m3(f[i] >> 4));
  }
  return r;
}

// 8 E2M1 codes (one dword) times the E4M3 scale byte `sb` -> 8 fp16 values
// (exact).  The scale, converted exactly to fp32, splits into 2^E (its
// exponent bits) and 1 + f/8 (its mantissa bits): the hardware conversion
// v_cvt_scalef32_pk_f16_fp4 takes only the power of two (code x 2^E, at most
// 2 significant bits, within fp16's normal range), and a packed fp16
// multiply by 1 + f/8 adds at most 4 more bits, so every product (at most
// 6 x 448) is an fp16 value.  A zero scale gives zeros.
__device__ __forceinline__ v8h e2m1x8_scaled_f16(uint32_t d, uint32_t sb) {
  const float sv = __builtin_amdgcn_cvt_f32_fp8(int(sb), 0);
  const float p2 = __uint_as_float(__float_as_uint(sv) & 0xff800000u);
  const _Float16 fr = _Float16(__uint_as_float((__float_as_uint(sv) & 0x007fffffu) | 0x3f800000u));
  const h2 ff = {fr, fr};
  const h2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, p2, 0) * ff;
  const h2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, p2, 1) * ff;
  const h2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, p2, 2) * ff;
  const h2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, p2, 3) * ff;
  return v8h{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
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

// ------------------------------------------------------- tile epilogue --
//
// Y = bf16(acc * r[n] * f) for a wave tile of FN x FM fragments.  Every wave
// writes its BF16 tile (16 FM rows x 16 FN columns) into its own region of the
// idle stage ring, 16-byte chunks of a row XOR-swizzled by the row index
// (conflict-free writes of the MFMA layout), then reads it back row-major and
// stores full 16-byte chunks.  The caller has passed a barrier after the last
// LDS read of the main loop.
struct TileArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint4* Wc;
  const uint32_t* Ws;
  int64_t M, K2, KB, KS, NG, NSG;
  int64_t m0, ng0;
};

// operands of the workgroup tile whose first activation row is m0 and first
// weight row group ng0
__device__ __forceinline__ TileArgs tile_args(int fmt, const uint8_t* a_codes,
                                              const uint8_t* a_scales, const uint8_t* blob,
                                              const BlobLayout& L, int64_t M, int64_t K, int64_t m0,
                                              int64_t ng0) {
  TileArgs t;
  t.a_codes = a_codes;
  t.a_scales = a_scales;
  t.Wc = reinterpret_cast<const uint4*>(blob + L.code_off);
  t.Ws = reinterpret_cast<const uint32_t*>(blob + L.scale_off);
  t.M = M;
  t.K2 = K / 2;
  t.KB = K / block_size(fmt);
  t.KS = L.KS;
  t.NG = L.NG;
  t.NSG = L.NSG;
  t.m0 = m0;
  t.ng0 = ng0;
  return t;
}

template <int FN, int FM, int WN, int WM>
__device__ __forceinline__ void tile_epilogue(const v4f (&acc)[FN][FM], LDS uint8_t* base,
                                              const TileArgs& t, const uint8_t* __restrict__ blob,
                                              const BlobLayout& L, float f,
                                              uint16_t* __restrict__ Y, int64_t M, int64_t N,
                                              int wave, int lane) {
  const float* __restrict__ R = reinterpret_cast<const float*>(blob + L.r_off);
  const int wn = wave % WN, wm = wave / WN;
  v4f rs[FN];
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    int64_t ng = t.ng0 + wn * FN + i;
    ng = ng < L.NG ? ng : L.NG - 1;
    const float4 r = *reinterpret_cast<const float4*>(R + ng * 16 + 4 * (lane >> 4));
    rs[i] = v4f{r.x * f, r.y * f, r.z * f, r.w * f};
  }
  constexpr int WNT = 16 * FN, WMT = 16 * FM;  // wave tile: n x m
  constexpr int CH = WNT / 8;                  // 16-byte chunks per row
  constexpr int ROWB = 2 * WNT;
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

// Tile order of the one-tile-per-workgroup kernels: the hardware deals
// workgroups round-robin to the 8 XCDs, and workgroup b takes number
// (b % 8) per_xcd + b / 8 of an order that walks blocks of (up to) 4 column
// tiles row by row, so each XCD runs through a contiguous range of it: the
// workgroups sharing an L2 at once cover 8 row tiles x 4 column tiles, and
// the activation rows are swept once per 4 column tiles rather than once per
// column tile.  A bijection onto the tiles_m x (tiles_total / tiles_m) grid.
__device__ __forceinline__ void col_block_tile(int tile, int tiles_m, int tiles_total, int& tm, int& tn) {
  const int tiles_n = tiles_total / tiles_m;
  const int nb = tile / (4 * tiles_m), ob = tile - nb * 4 * tiles_m;
  const int nw = tiles_n - 4 * nb < 4 ? tiles_n - 4 * nb : 4;  // width of this column block
  tm = ob / nw;
  tn = 4 * nb + ob % nw;
}

// ======================================================== tiled kernel ==
//
// NVFP4, all M.  Workgroup tile BN (n) x BM (m), WN x WM waves (n x m), wave tile
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
//   [A codes: BM/16 tiles of 16 rows x 64 B; chunk c of row r at 16-byte
//    position a_tile_pos(r, c)]
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

// Copy the operands of K-step ks into stage buffer `dst` (this wave's share).
template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
__device__ __forceinline__ void issue_stage(const TileArgs& t, int64_t ks, LDS uint8_t* dst,
                                            int wave, int lane) {
  using C = TileCfg<FMT, BN, BM, WN, WM, DEPTH>;
  // activation tiles, rows in lane quads (a_tile_pos)
#pragma unroll
  for (int i = 0; i < C::A_DMA; ++i) {
    const int f = wave * C::A_DMA + i;
    int64_t row = t.m0 + 16 * f + (lane >> 2);
    row = row < t.M ? row : t.M - 1;
    __builtin_amdgcn_global_load_lds(t.a_codes + row * t.K2 + ks * 64 + ((lane & 3) ^ fp4_swz(lane >> 2)) * 16,
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

  static_assert(FMT == NVFP4, "the tiled kernel serves NVFP4");
  {  // fp16 MFMA, four per K-step
    u32x4 af[FM];
    uint32_t sa[FM];
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int f = wm * FM + j;
      af[j] = A[f * 64 + a_tile_pos(r, c)];
      sa[j] = *reinterpret_cast<const LDS uint16_t*>(AS + (16 * f + r) * 8 + 2 * c);
    }
    // per 32-wide K part: the activation fragments expanded once and held,
    // the weight fragments expanded one at a time
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      v8h ah[FM];
#pragma unroll
      for (int j = 0; j < FM; ++j)
        ah[j] = e2m1x8_scaled_f16(af[j][jj], (sa[j] >> (8 * (jj >> 1))) & 0xffu);
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const v8h wh = e2m1x8_scaled_f16(wf[i][jj], (sw[i / 2] >> (8 * (2 * (i % 2) + (jj >> 1)))) & 0xffu);
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = mfma_f16(wh, ah[j], acc[i][j]);
      }
    }
  }
}

template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
__global__ __launch_bounds__(64 * WN * WM, 1) void gemm_tile_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ t_act, const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y,
    int64_t M, int64_t N, int64_t K, int tiles_m, int tiles_total, int per_xcd) {
  if (!blob_header_ok(blob, FMT, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  using C = TileCfg<FMT, BN, BM, WN, WM, DEPTH>;
  constexpr int FN = C::FN, FM = C::FM;
  // XCD-aware order (col_block_tile): 8 row tiles x 4 column tiles share an
  // XCD's L2 at once (2 MiB of activation rows and 2 MiB of weights at K =
  // 4096)
  const int tile = int(blockIdx.x % 8) * per_xcd + int(blockIdx.x / 8);
  if (tile >= tiles_total) return;
  int tm, tn;
  col_block_tile(tile, tiles_m, tiles_total, tm, tn);

  const BlobLayout L = blob_layout(FMT, N, K);
  const TileArgs t = tile_args(FMT, a_codes, a_scales, blob, L, M, K, int64_t(tm) * BM,
                               int64_t(tn) * (BN / 16));

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

  static_assert(WN * WM * (16 * FM) * (32 * FN) <= DEPTH * C::STAGE, "epilogue staging");
  __builtin_amdgcn_s_barrier();  // every wave is done with the stage buffers
  asm volatile("" ::: "memory");
  tile_epilogue<FN, FM, WN, WM>(acc, base, t, blob, L, epilogue_factor(FMT, t_act, blob), Y, M, N,
                                wave, lane);
}

// ===================================================== MX tiled kernel ==
//
// MXINT4 for M > 16.  Workgroup tile BN (n) x BM (m) with WN x WM
// waves, one 128-wide K-step per stage of a DEPTH-deep LDS ring filled by
// direct-to-LDS copies, as above, but software-pipelined inside each wave:
// while the MFMAs of K-step s run from registers, the wave already reads the
// fragments of K-step s+1 from LDS (weight fragment i is re-read right after
// its last MFMA; activation fragments, scales and scale words are double
// buffered).  Once every wave holds K-step s+1 in registers the barrier at the
// top of the next iteration releases its buffer, and the copy of K-step
// s+1+DEPTH goes there, so DEPTH-1 stages stay in flight.
//
// LDS stage buffer: [A codes: BM/16 x 1 KiB][W codes: BN/16 x 1 KiB]
// [scales: 256 B per wave, or 512 B when a wave's scale dwords exceed 64].
// One 4-byte copy per wave per stage fills that wave's scale chunk: dwords
// [0, AS_DW) are the activation scale dwords (the four blocks of one row) of
// rows wave*AS_DW.., dwords [AS_DW, AS_DW+WS_DW) the weight scale words
// wave*WS_DW.. of the tile (word d: group d/64, lane d%64); the remaining
// lanes copy a duplicate into padding.  With 512 B the activation dwords
// fill the first 256 B and the weight words the second, one copy each.
// (gemm_mx_lean_kernel below shares the ring, copies and fragment reads but
// keeps nothing of the next K-step in registers.)

template <int BN, int BM, int WN, int WM, int DEPTH>
struct MxCfg {
  static constexpr int WAVES = WN * WM;
  static constexpr int FN = BN / 16 / WN;
  static constexpr int FM = BM / 16 / WM;
  static constexpr int A_BYTES = BM * 64;
  static constexpr int W_BYTES = BN * 64;
  static constexpr int A_DMA = BM / 16 / WAVES;
  static constexpr int W_DMA = BN / 16 / WAVES;
  static constexpr int AS_DW = BM / WAVES;  // activation scale rows per wave
  static constexpr int WS_DW = BN / WAVES;  // weight scale words per wave (BN/64 groups x 64)
  // A wave copies its scale dwords with one 64-lane load (activation rows,
  // then weight words) or, when they are more than 64, with two (one each).
  static constexpr bool SC_SPLIT = AS_DW + WS_DW > 64;
  static constexpr int SC_LOADS = SC_SPLIT ? 2 : 1;
  static constexpr int SC_BYTES = WAVES * 256 * SC_LOADS;
  static constexpr int STAGE = A_BYTES + W_BYTES + SC_BYTES;
  static constexpr int COPIES = A_DMA + W_DMA + SC_LOADS;
  // byte offsets in the scale area: activation row R's scale dword, weight word d
  static constexpr int a_sc(int R) {
    return (R / AS_DW) * 256 * SC_LOADS + (R % AS_DW) * 4;
  }
  static constexpr int w_sc(int d) {
    return SC_SPLIT ? (d / WS_DW) * 512 + 256 + (d % WS_DW) * 4
                    : (d / WS_DW) * 256 + (AS_DW + d % WS_DW) * 4;
  }
  static_assert(A_DMA * WAVES * 16 == BM && W_DMA * WAVES * 16 == BN, "tile / wave split");
  static_assert(AS_DW <= 64 && WS_DW <= 64, "scale chunk");
  static_assert((AS_DW & (AS_DW - 1)) == 0 && (WS_DW & (WS_DW - 1)) == 0, "scale chunk split");
  static_assert(FN % 4 == 0 && BN % 64 == 0, "scale words");
  static_assert(DEPTH * STAGE <= 160 * 1024, "LDS");
  static_assert(WAVES * (16 * FM) * (32 * FN) <= DEPTH * STAGE, "epilogue staging");
};

// s_waitcnt vmcnt(v) lgkmcnt(0)
__device__ __forceinline__ constexpr int vm_lgkm0_encoding(int v) {
  return (v & 15) | (7 << 4) | (0 << 8) | (((v >> 4) & 3) << 14);
}

// Wait until this wave has at most `after` stages of copies outstanding and
// no LDS reads in flight, then barrier.
template <int C, int DEPTH>
__device__ __forceinline__ void mx_sync(int after) {
  static_assert((DEPTH - 1) * C < 64 && DEPTH <= 6, "vmcnt range");
  switch (after) {
    case 0: __builtin_amdgcn_s_waitcnt(vm_lgkm0_encoding(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vm_lgkm0_encoding(C)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vm_lgkm0_encoding(2 * C)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vm_lgkm0_encoding(3 * C)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vm_lgkm0_encoding(4 * C)); break;
    default: __builtin_amdgcn_s_waitcnt(vm_lgkm0_encoding(5 * C)); break;
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// (FMT only keeps the specializations of different kernels apart.)
template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
__device__ __forceinline__ void mx_issue(const TileArgs& t, int64_t ks, LDS uint8_t* dst, int wave,
                                         int lane) {
  using C = MxCfg<BN, BM, WN, WM, DEPTH>;
  // activation tiles, rows in lane quads (a_tile_pos)
#pragma unroll
  for (int i = 0; i < C::A_DMA; ++i) {
    const int f = wave * C::A_DMA + i;
    int64_t row = t.m0 + 16 * f + (lane >> 2);
    row = row < t.M ? row : t.M - 1;
    __builtin_amdgcn_global_load_lds(t.a_codes + row * t.K2 + ks * 64 + ((lane & 3) ^ fp4_swz(lane >> 2)) * 16,
                                     dst + f * 1024, 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < C::W_DMA; ++i) {
    const int f = wave * C::W_DMA + i;
    int64_t ng = t.ng0 + f;
    ng = ng < t.NG ? ng : t.NG - 1;
    __builtin_amdgcn_global_load_lds(t.Wc + (ng * t.KS + ks) * 64 + lane,
                                     dst + C::A_BYTES + f * 1024, 16, 0, 0);
  }
  LDS uint8_t* sc = dst + C::A_BYTES + C::W_BYTES + wave * 256 * C::SC_LOADS;
  const int wl = C::SC_SPLIT ? lane : lane - C::AS_DW;  // this lane's weight word, if any
  const bool is_a = lane < C::AS_DW;
  const bool is_w = wl >= 0 && wl < C::WS_DW;
  int64_t row = t.m0 + wave * C::AS_DW + (is_a ? lane : 0);
  row = row < t.M ? row : t.M - 1;
  const int d = wave * C::WS_DW + (is_w ? wl : 0);
  int64_t sg = t.ng0 / 4 + d / 64;
  sg = sg < t.NSG ? sg : t.NSG - 1;
  const uint8_t* wsrc = reinterpret_cast<const uint8_t*>(t.Ws + (sg * t.KS + ks) * 64 + (d & 63));
  const uint8_t* asrc = t.a_scales + row * t.KB + ks * 4;
  if constexpr (C::SC_SPLIT) {
    __builtin_amdgcn_global_load_lds(asrc, sc, 4, 0, 0);
    __builtin_amdgcn_global_load_lds(wsrc, sc + 256, 4, 0, 0);
  } else {
    __builtin_amdgcn_global_load_lds(is_a ? asrc : wsrc, sc, 4, 0, 0);
  }
}

// Register copies of one K-step's operands for a wave (besides the weight
// fragments, which live in their own array).
template <int FMT, int FN, int FM>
struct MxFrags {
  u32x4 a[FM];
  int sa[FM];
  uint32_t sw[FN / 4];
};

template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
__device__ __forceinline__ u32x4 mx_load_w(const LDS uint8_t* __restrict__ st, int wn, int i,
                                           int lane) {
  using C = MxCfg<BN, BM, WN, WM, DEPTH>;
  const LDS u32x4* W = reinterpret_cast<const LDS u32x4*>(st + C::A_BYTES);
  return W[(wn * C::FN + i) * 64 + lane];
}

template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
__device__ __forceinline__ void mx_load_rest(const LDS uint8_t* __restrict__ st, int wn, int wm,
                                             int lane, MxFrags<FMT, BN / 16 / WN, BM / 16 / WM>& fr) {
  using C = MxCfg<BN, BM, WN, WM, DEPTH>;
  const int r = lane & 15, c = lane >> 4;
  const LDS u32x4* A = reinterpret_cast<const LDS u32x4*>(st);
  const LDS uint8_t* SC = st + C::A_BYTES + C::W_BYTES;
#pragma unroll
  for (int j = 0; j < C::FM; ++j) {
    const int f = wm * C::FM + j;
    // MXINT4 operand order: half (c & 1) of blocks c >> 1 and 2 + (c >> 1) of row r
    const LDS u32x2* b = reinterpret_cast<const LDS u32x2*>(A + f * 64);
    const u32x2 lo = b[a_tile_pos(r, c >> 1) * 2 + (c & 1)];
    const u32x2 hi = b[a_tile_pos(r, 2 + (c >> 1)) * 2 + (c & 1)];
    fr.a[j] = u32x4{lo.x, lo.y, hi.x, hi.y};
    const int R = 16 * f + r;
    fr.sa[j] = SC[C::a_sc(R) + c];
  }
#pragma unroll
  for (int q = 0; q < C::FN / 4; ++q) {
    const int d = (wn * C::FN / 4 + q) * 64 + lane;
    fr.sw[q] = *reinterpret_cast<const LDS uint32_t*>(SC + C::w_sc(d));
  }
}

template <int FMT, int FN, int FM>
__device__ __forceinline__ void mx_mfma_row(v4f (&acc)[FN][FM], int i, const u32x4& wf,
                                            const MxFrags<FMT, FN, FM>& fr,
                                            const v8i (&a8)[FM]) {
  const v8i w8 = int4_frag_to_fp8(wf);
#pragma unroll
  for (int j = 0; j < FM; ++j)
    acc[i][j] = mfma_fp8(i % 4, w8, a8[j], acc[i][j], int(fr.sw[i / 4]), fr.sa[j]);
}

// MFMAs of the K-step held in registers, while the fragments of the next
// K-step are read from its stage buffer `nx`.
template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
__device__ __forceinline__ void mx_step(const LDS uint8_t* __restrict__ nx, int wn, int wm, int lane,
                                        v4f (&acc)[BN / 16 / WN][BM / 16 / WM],
                                        u32x4 (&wf)[BN / 16 / WN],
                                        MxFrags<FMT, BN / 16 / WN, BM / 16 / WM>& fr) {
  constexpr int FN = BN / 16 / WN, FM = BM / 16 / WM;
  static_assert(FMT == MXINT4, "the MX tiled kernel serves MXINT4");
  v8i a8[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) a8[j] = int4_frag_to_fp8(fr.a[j]);
  MxFrags<FMT, FN, FM> fn;
  mx_load_rest<FMT, BN, BM, WN, WM, DEPTH>(nx, wn, wm, lane, fn);
  // the last weight fragment is double-buffered so that no LDS read has to
  // wait for the final MFMA
  const u32x4 wlast = mx_load_w<FMT, BN, BM, WN, WM, DEPTH>(nx, wn, FN - 1, lane);
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    mx_mfma_row<FMT, FN, FM>(acc, i, wf[i], fr, a8);
    if (i < FN - 1) wf[i] = mx_load_w<FMT, BN, BM, WN, WM, DEPTH>(nx, wn, i, lane);
  }
  wf[FN - 1] = wlast;
  fr = fn;
}

// Instruction interleave of one loop iteration: the copies of the next stage
// and the reads of the next K-step's activation fragments and scales go
// between the first MFMAs, the weight-fragment reads after the MFMAs of the
// row they replace.
template <int FN, int FM, int COPIES>
__device__ __forceinline__ void mx_schedule() {
  constexpr int MFMA = 0x008, DS_READ = 0x100, VMEM = 0x020;
  constexpr int REST = FM + FM + FN / 4 + 1;  // A frags (up to 2 reads each), scales, last W
#pragma unroll
  for (int k = 0; k < COPIES; ++k) {
    __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(VMEM, 1, 0);
  }
#pragma unroll
  for (int k = 0; k < REST; ++k) {
    __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(DS_READ, 1, 0);
  }
#pragma unroll
  for (int i = 0; i < FN - 1; ++i) {
    __builtin_amdgcn_sched_group_barrier(MFMA, FM, 0);
    __builtin_amdgcn_sched_group_barrier(DS_READ, 1, 0);
  }
}

template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
__global__ __launch_bounds__(64 * WN * WM, 1) void gemm_mx_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int tiles_m, int tiles_total, int per_xcd) {
  if (!blob_header_ok(blob, FMT, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  using C = MxCfg<BN, BM, WN, WM, DEPTH>;
  constexpr int FN = C::FN, FM = C::FM;
  const int tile = int(blockIdx.x % 8) * per_xcd + int(blockIdx.x / 8);
  if (tile >= tiles_total) return;
  int tm, tn;
  col_block_tile(tile, tiles_m, tiles_total, tm, tn);

  const BlobLayout L = blob_layout(FMT, N, K);
  const TileArgs t = tile_args(FMT, a_codes, a_scales, blob, L, M, K, int64_t(tm) * BM,
                               int64_t(tn) * (BN / 16));

  __shared__ __attribute__((aligned(1024))) uint8_t smem[DEPTH * C::STAGE];
  LDS uint8_t* base = (LDS uint8_t*)smem;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wn = wave % WN, wm = wave / WN;

  v4f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int64_t KS = L.KS;
#pragma unroll
  for (int s = 0; s < DEPTH; ++s)
    if (s < KS) mx_issue<FMT, BN, BM, WN, WM, DEPTH>(t, s, base + s * C::STAGE, wave, lane);
  mx_sync<C::COPIES, DEPTH>(int((KS < DEPTH ? KS : DEPTH) - 1));

  u32x4 wf[FN];
  MxFrags<FMT, FN, FM> fr;
#pragma unroll
  for (int i = 0; i < FN; ++i) wf[i] = mx_load_w<FMT, BN, BM, WN, WM, DEPTH>(base, wn, i, lane);
  mx_load_rest<FMT, BN, BM, WN, WM, DEPTH>(base, wn, wm, lane, fr);

  // Main part: every iteration also starts the copy of K-step s+DEPTH (one
  // basic block, so the MFMAs, LDS reads and copies can be interleaved);
  // tail: the last DEPTH-1 iterations have nothing left to copy.
  int64_t s = 0;
  for (; s + DEPTH < KS; ++s) {
    mx_sync<C::COPIES, DEPTH>(DEPTH - 2);
    mx_issue<FMT, BN, BM, WN, WM, DEPTH>(t, s + DEPTH, base + (s % DEPTH) * C::STAGE, wave, lane);
    mx_step<FMT, BN, BM, WN, WM, DEPTH>(base + ((s + 1) % DEPTH) * C::STAGE, wn, wm, lane, acc, wf,
                                        fr);
    mx_schedule<FN, FM, C::COPIES>();
  }
  for (; s + 1 < KS; ++s) {
    mx_sync<C::COPIES, DEPTH>(int(KS - (s + 2)));
    mx_step<FMT, BN, BM, WN, WM, DEPTH>(base + ((s + 1) % DEPTH) * C::STAGE, wn, wm, lane, acc, wf,
                                        fr);
    mx_schedule<FN, FM, 0>();
  }
  {
    v8i a8[FMT == MXINT4 ? FM : 1];
    if constexpr (FMT == MXINT4) {
#pragma unroll
      for (int j = 0; j < FM; ++j) a8[j] = int4_frag_to_fp8(fr.a[j]);
    }
#pragma unroll
    for (int i = 0; i < FN; ++i) mx_mfma_row<FMT, FN, FM>(acc, i, wf[i], fr, a8);
  }

  __builtin_amdgcn_s_barrier();  // every wave is done with the stage buffers
  asm volatile("" ::: "memory");
  tile_epilogue<FN, FM, WN, WM>(acc, base, t, blob, L, epilogue_factor(FMT, nullptr, blob), Y, M,
                                N, wave, lane);
}

// Two waves per SIMD (8 waves of 128 x 64): a wave's widening, copies and
// LDS reads then overlap the other wave's MFMAs.  To fit 256 registers a
// wave keeps nothing of the next K-step in registers: after the barrier it
// reads the K-step's activation fragments and scales from the stage buffer,
// widens them, and walks the weight fragments one row ahead.  The copy of
// stage s + DEPTH - 1 goes out right after the barrier of K-step s, into the
// buffer that K-step s - 1 has just released.
template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
__device__ __forceinline__ void mx_lean_step(const LDS uint8_t* __restrict__ st, int wn, int wm,
                                             int lane, v4f (&acc)[BN / 16 / WN][BM / 16 / WM]) {
  constexpr int FN = BN / 16 / WN, FM = BM / 16 / WM;
  static_assert(FMT == MXINT4, "the MX tiled kernel serves MXINT4");
  MxFrags<FMT, FN, FM> fr;
  mx_load_rest<FMT, BN, BM, WN, WM, DEPTH>(st, wn, wm, lane, fr);
  u32x4 wcur = mx_load_w<FMT, BN, BM, WN, WM, DEPTH>(st, wn, 0, lane);
  v8i a8[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) a8[j] = int4_frag_to_fp8(fr.a[j]);
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    u32x4 wnext = wcur;
    if (i + 1 < FN) wnext = mx_load_w<FMT, BN, BM, WN, WM, DEPTH>(st, wn, i + 1, lane);
    mx_mfma_row<FMT, FN, FM>(acc, i, wcur, fr, a8);
    wcur = wnext;
  }
}

template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
__global__ __launch_bounds__(64 * WN * WM, 1) void gemm_mx_lean_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int tiles_m, int tiles_total, int per_xcd) {
  if (!blob_header_ok(blob, FMT, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  using C = MxCfg<BN, BM, WN, WM, DEPTH>;
  constexpr int FN = C::FN, FM = C::FM;
  const int tile = int(blockIdx.x % 8) * per_xcd + int(blockIdx.x / 8);
  if (tile >= tiles_total) return;
  int tm, tn;
  col_block_tile(tile, tiles_m, tiles_total, tm, tn);

  const BlobLayout L = blob_layout(FMT, N, K);
  const TileArgs t = tile_args(FMT, a_codes, a_scales, blob, L, M, K, int64_t(tm) * BM,
                               int64_t(tn) * (BN / 16));

  __shared__ __attribute__((aligned(1024))) uint8_t smem[DEPTH * C::STAGE];
  LDS uint8_t* base = (LDS uint8_t*)smem;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wn = wave % WN, wm = wave / WN;

  v4f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int64_t KS = L.KS;
#pragma unroll
  for (int s = 0; s < DEPTH - 1; ++s)
    if (s < KS) mx_issue<FMT, BN, BM, WN, WM, DEPTH>(t, s, base + s * C::STAGE, wave, lane);
  for (int64_t s = 0; s < KS; ++s) {
    // stages issued after s: min(DEPTH - 2, KS - 1 - s)
    const int64_t left = KS - 1 - s;
    mx_sync<C::COPIES, DEPTH>(int(left < DEPTH - 2 ? left : DEPTH - 2));
    if (s + DEPTH - 1 < KS)
      mx_issue<FMT, BN, BM, WN, WM, DEPTH>(t, s + DEPTH - 1, base + ((s + DEPTH - 1) % DEPTH) * C::STAGE,
                                           wave, lane);
    mx_lean_step<FMT, BN, BM, WN, WM, DEPTH>(base + (s % DEPTH) * C::STAGE, wn, wm, lane, acc);
  }

  __builtin_amdgcn_s_barrier();  // every wave is done with the stage buffers
  asm volatile("" ::: "memory");
  tile_epilogue<FN, FM, WN, WM>(acc, base, t, blob, L, epilogue_factor(FMT, nullptr, blob), Y, M,
                                N, wave, lane);
}

template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
hipError_t launch_mx_lean(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                          const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  const int tiles_n = int((N + BN - 1) / BN);
  const int tiles_m = int((M + BM - 1) / BM);
  const int total = tiles_n * tiles_m;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL((gemm_mx_lean_kernel<FMT, BN, BM, WN, WM, DEPTH>), dim3(unsigned(per_xcd * 8)),
                     dim3(64 * WN * WM), 0, stream, ac, as, blob, Y, M, N, K, tiles_m, total,
                     per_xcd);
  return hipGetLastError();
}

template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
hipError_t launch_mx(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                     const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  const int tiles_n = int((N + BN - 1) / BN);
  const int tiles_m = int((M + BM - 1) / BM);
  const int total = tiles_n * tiles_m;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL((gemm_mx_kernel<FMT, BN, BM, WN, WM, DEPTH>), dim3(unsigned(per_xcd * 8)),
                     dim3(64 * WN * WM), 0, stream, ac, as, blob, Y, M, N, K, tiles_m, total,
                     per_xcd);
  return hipGetLastError();
}

// ================================================ MXFP4, 32x32x64 MFMA ==
//
// MXFP4 runs on V_MFMA_SCALE_F32_32X32X64_F8F6F4: a single wave per SIMD
// keeps that instruction's pipeline full, so a workgroup is 4 waves (2 x 2),
// each with a 128 x 128 (or 128 x 64) output tile held in 256 (128)
// accumulator registers.  Operand fragments (1 KiB: 32 rows x 64 K, lane l
// holding the 32 codes of row l%32, K chunk l/32) come from the packed
// weight tiles as they are and from the canonical activation rows.  Scales:
// lane l of a fragment supplies the E8M0 scale of its row and block;
// weights take theirs from a scale word (byte = row group, op_sel), the
// activations from the row's scale dword shifted by 8 (l/32) (op_sel 0 or 2
// for the first or second 64-K half of the K-step).
//
// Pipeline: a DEPTH-deep LDS ring of 128-wide K-steps filled by
// direct-to-LDS copies; every wave holds the fragments of K-step s in
// registers while it reads those of K-step s+1 and runs the MFMAs of s.

template <int OPW, int OPA>
__device__ __forceinline__ v16f mfma32_fp4_op(const u32x4& w, const u32x4& a, const v16f& acc,
                                              int sw, int sa) {
  const v8i A = {int(w.x), int(w.y), int(w.z), int(w.w), 0, 0, 0, 0};
  const v8i B = {int(a.x), int(a.y), int(a.z), int(a.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc, 4, 4, OPW, sw, OPA, sa);
}

template <int BN, int BM, int DEPTH>
struct Fp4Cfg {
  static constexpr int WN = 2, WM = 2, WAVES = 4;
  static constexpr int FN = BN / WN / 32;  // 32-row weight groups per wave
  static constexpr int FM = BM / WM / 32;  // 32-row activation groups per wave
  // 1 KiB copies per K-step: activations 16 rows x 64 B, weights one fragment tile
  static constexpr int A_TILES = BM / 16, W_TILES = BN / 32 * 2;
  static constexpr int A_BYTES = A_TILES * 1024, W_BYTES = W_TILES * 1024;
  static constexpr int WS_DW = BN / 128 * 2 * 64 / WAVES;  // weight scale words per wave
  static constexpr int STAGE = A_BYTES + W_BYTES + WAVES * 256;
  static constexpr int A_DMA = A_TILES / WAVES, W_DMA = W_TILES / WAVES;
  // per wave per K-step: activation and weight tiles, one copy of weight
  // scale words, one quarter of an activation scale block
  static constexpr int COPIES = A_DMA + W_DMA + 2;
  // activation scale blocks: 4 K-steps x BM rows of scale dwords; a wave
  // owns ASR rows, copied as 4 quarters of 16 rows x 4 K-steps
  static constexpr int ASR = 64;
  static constexpr int ASB = WAVES * ASR * 16;  // bytes per block
  static constexpr int AS_OFF = DEPTH * STAGE;  // 3 blocks after the ring
  static constexpr int LDS_BYTES = AS_OFF + 3 * ASB;
  static constexpr int EPI_BYTES = WAVES * (32 * FM) * (64 * FN);
  static_assert(A_DMA * WAVES == A_TILES && W_DMA * WAVES == W_TILES, "tile / wave split");
  static_assert(BN % 128 == 0 && FN >= 1 && FN <= 4 && FM >= 1, "wave tile");
  static_assert(WS_DW <= 64 && BM <= WAVES * ASR, "scale copies");
  static_assert(LDS_BYTES <= 160 * 1024 && EPI_BYTES <= DEPTH * STAGE, "LDS");
  static_assert((DEPTH - 1) * COPIES + 4 < 64 && DEPTH <= 5, "vmcnt range / scale block reuse");
};

struct Fp4Args {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint4* Wc;
  const uint32_t* Ws;
  int64_t M, K2, KB, KT, NG, NSG;
  int64_t m0, g0;  // first activation row, first 32-row weight group
  int64_t KS;      // 128-wide K-steps
  LDS uint8_t* smem;
};

template <int FN, int FM>
struct Fp4Frags {
  u32x4 w[FN][2];
  u32x4 a[FM][2];
  int sa[FM];
  int sw[2];
};

// MFMAs of one K-step: weight group I (scale byte I of the word), 64-K half
// H (activation scale byte 2H), every activation group j.
template <int FN, int FM, int I, int H>
struct Fp4Row {
  static __device__ __forceinline__ void run(v16f (&acc)[FN][FM], const Fp4Frags<FN, FM>& fr) {
#pragma unroll
    for (int j = 0; j < FM; ++j)
      acc[I][j] = mfma32_fp4_op<I, 2 * H>(fr.w[I][H], fr.a[j][H], acc[I][j], fr.sw[H], fr.sa[j]);
    if constexpr (I + 1 < FN) Fp4Row<FN, FM, I + 1, H>::run(acc, fr);
    else if constexpr (H == 0) Fp4Row<FN, FM, 0, 1>::run(acc, fr);
  }
};

template <int FN, int FM>
__device__ __forceinline__ void fp4_mfmas(v16f (&acc)[FN][FM], const Fp4Frags<FN, FM>& fr) {
  Fp4Row<FN, FM, 0, 0>::run(acc, fr);
}

// s_waitcnt vmcnt(v) lgkmcnt(0), then barrier
template <int C, int DEPTH>
__device__ __forceinline__ void fp4_sync(int after) {
  switch (after) {
    case 0: __builtin_amdgcn_s_waitcnt(vm_lgkm0_encoding(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vm_lgkm0_encoding(C)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vm_lgkm0_encoding(2 * C)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vm_lgkm0_encoding(3 * C)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vm_lgkm0_encoding(4 * C)); break;
    default: __builtin_amdgcn_s_waitcnt(vm_lgkm0_encoding(5 * C)); break;
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Quarter q of activation scale block b (the scale dwords of K-steps
// 4b..4b+3): lane l of wave w copies the dword of row w*ASR + 16q + l/4,
// K-step 4b + l%4, so one copy touches 16 rows instead of 64.  Rows beyond
// M and K-steps beyond KS copy a valid duplicate.  Block b lives in buffer
// b % 3 after the stage ring; it is copied together with the stages of
// block b-1, one quarter per stage.
template <int BN, int BM, int DEPTH>
__device__ __forceinline__ void fp4_copy_scale_quarter(const Fp4Args& t, int64_t b, int q, int wave,
                                                       int lane) {
  using C = Fp4Cfg<BN, BM, DEPTH>;
  int64_t row = t.m0 + wave * C::ASR + 16 * q + (lane >> 2);
  row = row < t.M ? row : t.M - 1;
  int64_t ks = 4 * b + (lane & 3);
  ks = ks < t.KS ? ks : t.KS - 1;
  lds_copy4(t.a_scales + row * t.KB + 4 * ks,
            t.smem + C::AS_OFF + int(b % 3) * C::ASB + wave * (C::ASR * 16) + q * 256);
}

// LDS byte offset of the scale dword of local activation row R, K-step ks
// (NB scale block buffers)
template <int BN, int BM, int DEPTH, int NB = 3>
__device__ __forceinline__ int fp4_scale_offset(int R, int64_t ks) {
  using C = Fp4Cfg<BN, BM, DEPTH>;
  const int w = R / C::ASR, r = R % C::ASR;
  return C::AS_OFF + int((ks / 4) % NB) * C::ASB + w * (C::ASR * 16) + (r >> 4) * 256 + (r & 15) * 16 +
         int(ks & 3) * 4;
}

// Copy number k of a wave's share of K-step ks (activation copies, weight
// copies, then scale copies), so that the copies can be spread over a step.
template <int BN, int BM, int DEPTH>
__device__ __forceinline__ void fp4_copy(const Fp4Args& t, int64_t ks, LDS uint8_t* dst, int wave,
                                         int lane, int k) {
  using C = Fp4Cfg<BN, BM, DEPTH>;
  if (k < C::A_DMA) {
    // 16 rows x 64 contiguous bytes (one K-step), rows in lane quads (fp4_swz)
    const int f = wave * C::A_DMA + k;
    int64_t row = t.m0 + 16 * f + (lane >> 2);
    row = row < t.M ? row : t.M - 1;
    lds_copy16(t.a_codes + row * t.K2 + ks * 64 + ((lane & 3) ^ fp4_swz(lane >> 2)) * 16, dst + f * 1024);
  } else if (k < C::A_DMA + C::W_DMA) {
    const int f = wave * C::W_DMA + (k - C::A_DMA);
    int64_t g = t.g0 + (f >> 1);
    g = g < t.NG ? g : t.NG - 1;
    lds_copy16(t.Wc + (g * t.KT + 2 * ks + (f & 1)) * 64 + lane, dst + C::A_BYTES + f * 1024);
  } else if (k == C::A_DMA + C::W_DMA) {
    // weight scale words of K-step ks: word e = (sg local, half, lane)
    const int e = wave * C::WS_DW + (lane < C::WS_DW ? lane : 0);
    int64_t sg = t.g0 / 4 + (e >> 7);
    sg = sg < t.NSG ? sg : t.NSG - 1;
    lds_copy4(t.Ws + (sg * t.KT + 2 * ks + ((e >> 6) & 1)) * 64 + (e & 63),
              dst + C::A_BYTES + C::W_BYTES + wave * 256);
  } else {
    fp4_copy_scale_quarter<BN, BM, DEPTH>(t, ks / 4 + 1, int(ks & 3), wave, lane);
  }
}

// All copies of a wave's share of K-step ks.
template <int BN, int BM, int DEPTH>
__device__ __forceinline__ void fp4_issue(const Fp4Args& t, int64_t ks, LDS uint8_t* dst, int wave,
                                          int lane) {
#pragma unroll
  for (int k = 0; k < Fp4Cfg<BN, BM, DEPTH>::COPIES; ++k) fp4_copy<BN, BM, DEPTH>(t, ks, dst, wave, lane, k);
}

// activation scale byte of lane l: block 2 hh + l/32 is byte 2 hh of the shifted dword
template <int FM>
__device__ __forceinline__ void fp4_fix_scales(int (&sa)[FM], int lane) {
#pragma unroll
  for (int j = 0; j < FM; ++j) sa[j] = int(uint32_t(sa[j]) >> (8 * (lane >> 5)));
}

// LDS read number r of a wave's fragments of K-step kstep (stage buffer
// `st`): activation scale dwords (raw, from the scale block; fp4_fix_scales
// applies the lane's byte shift once the reads have landed), weight scale
// words, activation fragments, weight fragments.  FNE (<= FN) is the number
// of 32-row weight groups the wave uses: a tile whose waves cover only the
// first FNE groups each (the first 64 FNE of its BN rows) reads the same
// stage layout.
// With FNE = 3 the wave's 3 groups start at group goff + 3 wn of the two
// scale words copied for the tile (goff = first group's position in its
// scale word), so its scale word is cut from both.
template <int BN, int BM, int DEPTH, int NB = 3, int FNE = BN / 64>
__device__ __forceinline__ void fp4_read_item(const LDS uint8_t* __restrict__ st,
                                              const LDS uint8_t* __restrict__ base, int64_t kstep,
                                              int wn, int wm, int lane, Fp4Frags<BN / 64, BM / 64>& fr,
                                              int r, int goff = 0) {
  using C = Fp4Cfg<BN, BM, DEPTH>;
  if (r < C::FM) {
    const int j = r;
    const int R = 32 * (wm * C::FM + j) + (lane & 31);
    fr.sa[j] = *reinterpret_cast<const LDS int*>(base + fp4_scale_offset<BN, BM, DEPTH, NB>(R, kstep));
  } else if (r < C::FM + 2) {
    const int hh = r - C::FM;
    if constexpr (FNE == 3) {
      static_assert(C::WS_DW == 64, "one scale word per lane and wave slot");
      const LDS uint32_t* ws = reinterpret_cast<const LDS uint32_t*>(st + C::A_BYTES + C::W_BYTES);
      const uint64_t w2 = uint64_t(ws[hh * 64 + lane]) | (uint64_t(ws[(2 + hh) * 64 + lane]) << 32);
      fr.sw[hh] = int(uint32_t(w2 >> (8 * (goff + 3 * wn))));
    } else {
      const int e = ((wn * FNE / 4) * 2 + hh) * 64 + lane;
      const uint32_t wsw = *reinterpret_cast<const LDS uint32_t*>(st + C::A_BYTES + C::W_BYTES +
                                                                  (e / C::WS_DW) * 256 + (e % C::WS_DW) * 4);
      // byte i of the shifted word is the scale of the wave's weight group i
      fr.sw[hh] = int(FNE == 4 ? wsw : wsw >> (8 * ((wn * FNE) & 3)));
    }
  } else if (r < 3 * C::FM + 2) {
    const int q = r - C::FM - 2, j = q >> 1, hh = q & 1;
    // fragment lane l: row 32 g + l%32 (16-row tile 2 g + (l%32)/16, row
    // l%16 in it), 16-byte chunk 2 hh + l/32 of its K-step bytes (fp4_swz)
    fr.a[j][hh] = *reinterpret_cast<const LDS u32x4*>(
        st + (2 * (wm * C::FM + j) + ((lane >> 4) & 1)) * 1024 + a_tile_pos(lane & 15, 2 * hh + (lane >> 5)) * 16);
  } else {
    const int q = r - 3 * C::FM - 2, i = q >> 1, hh = q & 1;
    fr.w[i][hh] = *reinterpret_cast<const LDS u32x4*>(st + C::A_BYTES + ((wn * FNE + i) * 2 + hh) * 1024 +
                                                      lane * 16);
  }
}

template <int BN, int BM, int DEPTH, int NB = 3, int FNE = BN / 64>
__device__ __forceinline__ void fp4_read_all(const LDS uint8_t* __restrict__ st,
                                             const LDS uint8_t* __restrict__ base, int64_t kstep,
                                             int wn, int wm, int lane, Fp4Frags<BN / 64, BM / 64>& fr,
                                             int goff = 0) {
  using C = Fp4Cfg<BN, BM, DEPTH>;
#pragma unroll
  for (int r = 0; r < 3 * C::FM + 2 + 2 * FNE; ++r)
    fp4_read_item<BN, BM, DEPTH, NB, FNE>(st, base, kstep, wn, wm, lane, fr, r, goff);
  fp4_fix_scales<C::FM>(fr.sa, lane);
}


// One pipeline step as 2 FN groups of FM MFMAs (64-K half H, weight group I);
// after each group this wave issues its share of the copies of the stage
// DEPTH steps ahead and of the LDS reads of the next step, and a scheduling
// barrier keeps that order: the texture unit gets the copies at a rate it can
// take (a burst of them stalls the issuing wave and starves the MFMAs) and
// every read is in flight long before the step ends.
template <int BN, int BM, int DEPTH, bool ISSUE, int G>
struct Fp4Group {
  using C = Fp4Cfg<BN, BM, DEPTH>;
  static constexpr int FN = C::FN, FM = C::FM, NGRP = 2 * FN;
  static constexpr int READS = 3 * FM + 2 + 2 * FN;
  static __device__ __forceinline__ void run(v16f (&acc)[FN][FM], const Fp4Frags<FN, FM>& cur,
                                             Fp4Frags<FN, FM>& nxt, const Fp4Args& t, int64_t ks_copy,
                                             LDS uint8_t* dst, const LDS uint8_t* __restrict__ st,
                                             int64_t ks_read, int wave, int wn, int wm, int lane) {
    constexpr int H = G / FN, I = G % FN;
#pragma unroll
    for (int j = 0; j < FM; ++j)
      acc[I][j] = mfma32_fp4_op<I, 2 * H>(cur.w[I][H], cur.a[j][H], acc[I][j], cur.sw[H], cur.sa[j]);
    if constexpr (ISSUE) {
#pragma unroll
      for (int k = G * C::COPIES / NGRP; k < (G + 1) * C::COPIES / NGRP; ++k)
        fp4_copy<BN, BM, DEPTH>(t, ks_copy, dst, wave, lane, k);
    }
    // the reads go in the first RG groups, so that they have landed by the end of the step
    constexpr int RG = NGRP > 2 ? NGRP - 2 : NGRP;
    if constexpr (G < RG) {
#pragma unroll
      for (int r = G * READS / RG; r < (G + 1) * READS / RG; ++r)
        fp4_read_item<BN, BM, DEPTH>(st, t.smem, ks_read, wn, wm, lane, nxt, r);
    }
    if constexpr (G + 1 == NGRP) fp4_fix_scales<FM>(nxt.sa, lane);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (G + 1 < NGRP)
      Fp4Group<BN, BM, DEPTH, ISSUE, G + 1>::run(acc, cur, nxt, t, ks_copy, dst, st, ks_read, wave, wn,
                                                  wm, lane);
  }
};

// One BN x BM output tile (row tile tm, column tile tn) of one problem.
template <int BN, int BM, int DEPTH>
__device__ __forceinline__ void fp4_tile(const uint8_t* __restrict__ a_codes,
                                         const uint8_t* __restrict__ a_scales,
                                         const uint8_t* __restrict__ blob,
                                         uint16_t* __restrict__ Y, int64_t M, int64_t N,
                                         int64_t K, int tm, int tn) {
  if (!blob_header_ok(blob, MXFP4, N, K)) {
    fill_tile_nan(Y, M, N, int64_t(tm) * BM, int64_t(tn) * BN, BM, BN);
    return;
  }
  using C = Fp4Cfg<BN, BM, DEPTH>;
  constexpr int FN = C::FN, FM = C::FM;
  const BlobLayout L = blob_layout(MXFP4, N, K);
  Fp4Args t;
  t.a_codes = a_codes;
  t.a_scales = a_scales;
  t.Wc = reinterpret_cast<const uint4*>(blob + L.code_off);
  t.Ws = reinterpret_cast<const uint32_t*>(blob + L.scale_off);
  t.M = M;
  t.K2 = K / 2;
  t.KB = K / 32;
  t.KT = L.KT;
  t.NG = L.NG;
  t.NSG = L.NSG;
  t.m0 = int64_t(tm) * BM;
  t.g0 = int64_t(tn) * (BN / 32);
  t.KS = L.KS;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES];
  LDS uint8_t* base = (LDS uint8_t*)smem;
  t.smem = base;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wn = wave % C::WN, wm = wave / C::WN;

  v16f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int64_t KS = L.KS;
  // activation scale block 0 (the stages of block b-1 carry block b)
#pragma unroll
  for (int q = 0; q < 4; ++q) fp4_copy_scale_quarter<BN, BM, DEPTH>(t, 0, q, wave, lane);
#pragma unroll
  for (int s = 0; s < DEPTH; ++s)
    if (s < KS) fp4_issue<BN, BM, DEPTH>(t, s, base + s * C::STAGE, wave, lane);
  fp4_sync<C::COPIES, DEPTH>(int((KS < DEPTH ? KS : DEPTH) - 1));
  Fp4Frags<FN, FM> fa, fb;
  fp4_read_all<BN, BM, DEPTH>(base, base, 0, wn, wm, lane, fa);

  // Main part, two steps per iteration (the fragment buffers swap roles),
  // each step also copying K-step s+DEPTH into the buffer K-step s came
  // from; tail: nothing left to copy.
  int64_t s = 0;
  for (; s + 1 + DEPTH < KS; s += 2) {
    fp4_sync<C::COPIES, DEPTH>(DEPTH - 2);
    Fp4Group<BN, BM, DEPTH, true, 0>::run(acc, fa, fb, t, s + DEPTH, base + (s % DEPTH) * C::STAGE,
                                          base + ((s + 1) % DEPTH) * C::STAGE, s + 1, wave, wn, wm,
                                          lane);
    fp4_sync<C::COPIES, DEPTH>(DEPTH - 2);
    Fp4Group<BN, BM, DEPTH, true, 0>::run(acc, fb, fa, t, s + 1 + DEPTH,
                                          base + ((s + 1) % DEPTH) * C::STAGE,
                                          base + ((s + 2) % DEPTH) * C::STAGE, s + 2, wave, wn, wm,
                                          lane);
  }
  for (; s + 1 < KS; ++s) {
    const int64_t issued = KS < s + DEPTH ? KS : s + DEPTH;
    fp4_sync<C::COPIES, DEPTH>(int(issued - (s + 2)));
    if (s + DEPTH < KS)
      fp4_issue<BN, BM, DEPTH>(t, s + DEPTH, base + (s % DEPTH) * C::STAGE, wave, lane);
    fp4_read_all<BN, BM, DEPTH>(base + ((s + 1) % DEPTH) * C::STAGE, base, s + 1, wn, wm, lane, fb);
    fp4_mfmas<FN, FM>(acc, fa);
    fa = fb;
  }
  fp4_mfmas<FN, FM>(acc, fa);

  // epilogue: Y = bf16(acc * r) through LDS (see tile_epilogue), 32x32 blocks:
  // acc[i][j] element e of lane l is n = 32 i + 8 (e/4) + 4 (l/32) + e%4,
  // m = 32 j + l%32 within the wave tile
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  const float* __restrict__ R = reinterpret_cast<const float*>(blob + L.r_off);
  constexpr int WNT = 32 * FN, WMT = 32 * FM;
  constexpr int CH = WNT / 8, ROWB = 2 * WNT;
  LDS uint8_t* ep = base + wave * (WMT * ROWB);
  const int64_t nbase = (t.g0 + wn * FN) * 32;
  const int64_t mbase = t.m0 + wm * WMT;
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int64_t n = nbase + 32 * i + 8 * q + 4 * (lane >> 5);
      n = n < N ? n : N - 4;
      const float4 r = *reinterpret_cast<const float4*>(R + n);
      const v4f rs = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int m = 32 * j + (lane & 31);
        const int chunk = 4 * i + q;
        const int off = m * ROWB + ((chunk ^ (m % CH)) * 16) + 8 * (lane >> 5);
        const v4f a = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        *reinterpret_cast<LDS u32x2*>(ep + off) = scale_pack4(a, rs);
      }
    }
#pragma unroll
  for (int q = 0; q < WMT * CH / 64; ++q) {
    const int idx = q * 64 + lane;
    const int row = idx / CH, chunk = idx % CH;
    const u32x4 v = *reinterpret_cast<const LDS u32x4*>(ep + row * ROWB + ((chunk ^ (row % CH)) * 16));
    const int64_t m = mbase + row, n = nbase + 8 * chunk;
    if (m < M && n < N) *reinterpret_cast<u32x4*>(Y + m * N + n) = v;
  }
}

template <int BN, int BM, int DEPTH>
__global__ __launch_bounds__(256, 1) void gemm_fp4_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int tiles_m, int tiles_total, int per_xcd) {
  const int tile = int(blockIdx.x % 8) * per_xcd + int(blockIdx.x / 8);
  if (tile >= tiles_total) return;
  fp4_tile<BN, BM, DEPTH>(a_codes, a_scales, blob, Y, M, N, K, tile % tiles_m, tile / tiles_m);
}

// Several problems of one M and K in one launch (per-projection linears of a
// fused input): problem p owns tiles [first[p], first[p + 1]) of the launch;
// the XCD-contiguous tile order runs over the problems in turn.
struct Fp4Problems {
  const uint8_t* ac[kMaxGroup];
  const uint8_t* as[kMaxGroup];
  const uint8_t* blob[kMaxGroup];
  uint16_t* Y[kMaxGroup];
  int64_t N[kMaxGroup];
  int first[kMaxGroup + 1];
  int P;
};

template <int BN, int BM, int DEPTH>
__global__ __launch_bounds__(256, 1) void gemm_fp4_grouped_kernel(Fp4Problems g, int64_t M, int64_t K,
                                                                  int tiles_m, int per_xcd) {
  const int tile = int(blockIdx.x % 8) * per_xcd + int(blockIdx.x / 8);
  if (tile >= g.first[g.P]) return;
  int p = 0;
#pragma unroll
  for (int q = 1; q < kMaxGroup; ++q) p += (q < g.P && tile >= g.first[q]) ? 1 : 0;
  const int lt = tile - g.first[p];
  fp4_tile<BN, BM, DEPTH>(g.ac[p], g.as[p], g.blob[p], g.Y[p], M, g.N[p], K, lt % tiles_m,
                          lt / tiles_m);
}

template <int BN, int BM, int DEPTH>
hipError_t launch_fp4(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                      const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  const int tiles_n = int((N + BN - 1) / BN);
  const int tiles_m = int((M + BM - 1) / BM);
  const int total = tiles_n * tiles_m;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL((gemm_fp4_kernel<BN, BM, DEPTH>), dim3(unsigned(per_xcd * 8)), dim3(256), 0,
                     stream, ac, as, blob, Y, M, N, K, tiles_m, total, per_xcd);
  return hipGetLastError();
}

// ===================================== MXFP4, persistent ==
//
// Large MXFP4 GEMMs (256 x 256 tiles, K a multiple of 512) run one
// workgroup per CU.  Tiles go to the 8 XCDs in contiguous chunks, each chunk
// in the tile order of gemm_fp4_kernel (m fastest); within an XCD the 32
// workgroups take its tiles round-robin, so each round of 32 concurrent
// tiles shares activation rows and weight groups in that XCD's L2.  Where
// whole tiles would leave CUs idle, the items are narrower: 256 x 192 tiles
// (3 of the 4 weight groups per wave) when those fill at most one round,
// and with 96..128 tiles, the tiles' n halves of 128 output features.  A
// narrow item runs the same copy stream as a whole tile (the weight copies
// of rows it does not have read from an empty buffer range, which moves
// nothing), so every wait count holds, and fewer MFMAs.
//
// The tiles of a workgroup form one stream of K-steps, and the DEPTH-deep
// copy ring runs over that stream: the next tile's first K-steps are in
// flight while a tile finishes, so there is no per-tile pipeline fill.  The
// epilogue stores straight from registers (a lane swap gives each lane 8
// consecutive outputs of its row); its buffer stores drop rows beyond M and
// columns beyond N at the buffer's bounds.

struct Fp4P {
  static constexpr int BN = 256, BM = 256, DEPTH = 4, XCDS = 8, PER_XCD = 32;
  using C = Fp4Cfg<BN, BM, DEPTH>;
  static constexpr int NSB = 2;                      // activation scale block buffers
  static constexpr int R_OFF = C::AS_OFF + NSB * C::ASB;  // r of two items, 1 KiB each
  static constexpr int LDS_BYTES = R_OFF + 2 * 1024;
  // vector memory operations of a wave between the copies of one item's
  // last quad and the first K-step of the next: the epilogue's stores (two
  // per 32 x 32 block) and the copy of the following item's r
  static constexpr int EPI_STORES = 2 * C::FN * C::FM;
  static constexpr int ITEM_OPS = EPI_STORES + 1;
  // copies per wave with K-step j of a quad: activation and weight tiles,
  // weight scale words, and with j = 0 the 4 quarters of the quad's
  // activation scale block
  static constexpr int STAGE_COPIES = C::A_DMA + C::W_DMA + 1;
  static constexpr int copies(int j) { return STAGE_COPIES + (j == 0 ? 4 : 0); }
  // copies younger than the stage the step at quad position j reads next
  // (those of the two K-steps after it)
  static constexpr int younger(int j) { return copies((j + 2) & 3) + copies((j + 3) & 3); }
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(DEPTH == 4, "one quad of K-steps in flight");
};
static_assert(Fp4P::younger(1) + Fp4P::ITEM_OPS < 64 && Fp4P::younger(2) + Fp4P::ITEM_OPS < 64 &&
                  Fp4P::copies(1) + Fp4P::copies(2) + Fp4P::copies(3) + Fp4P::EPI_STORES < 64,
              "vmcnt range");

// The items of workgroup b: its XCD x = b % 8 and index i = b / 8 within it
// (workgroups are dealt to the XCDs round-robin) give items tb + i + 32 k of
// the XCD's chunk [tb, te) of the launch's items (tiles, or n halves).
struct Fp4PSched {
  int tiles_m, KS, tb, i, n_items;

  __device__ __forceinline__ void init(int T, int tiles_m_, int KS_, int b) {
    tiles_m = tiles_m_;
    KS = KS_;
    const int x = b % Fp4P::XCDS;
    i = b / Fp4P::XCDS;
    tb = int(int64_t(x) * T / Fp4P::XCDS);
    const int te = int(int64_t(x + 1) * T / Fp4P::XCDS);
    n_items = te - tb > i ? (te - tb - i + Fp4P::PER_XCD - 1) / Fp4P::PER_XCD : 0;
  }
  __device__ __forceinline__ int tile(int k) const { return tb + i + Fp4P::PER_XCD * k; }
};

// Where item k of the stream reads: its tile origin and K-steps [ks0, ks0 +
// len).  Past the last item it repeats the last item's last quad, so copies
// beyond the end of the stream read valid sources.  FNE is the item width
// in 64-feature units per wave: 4, a 256 x 256 tile; 3, a 256 x 192 tile
// (tiles of 192 features, 6 weight groups); 2, item h is n half h % 2 of
// 256 x 256 tile h / 2 (consecutive workgroups of an XCD take the two halves
// of a tile, which share its activation rows).
struct Fp4PDesc {
  int m0, g0;  // first activation row, first 32-row weight group
  int ks0, len;
};

template <int FNE>
__device__ __forceinline__ Fp4PDesc fp4p_desc(const Fp4PSched& S, int k) {
  const bool over = k >= S.n_items;
  const int it = S.tile(over ? S.n_items - 1 : k);
  const int t = FNE == 2 ? it / 2 : it;
  Fp4PDesc d;
  d.m0 = (t % S.tiles_m) * Fp4P::BM;
  d.g0 = FNE == 3 ? (t / S.tiles_m) * 6 : (t / S.tiles_m) * (Fp4P::BN / 32) + (FNE == 2 ? 4 * (it & 1) : 0);
  d.ks0 = over ? S.KS - 4 : 0;
  d.len = over ? 4 : S.KS;
  return d;
}

// Copies go straight into LDS as buffer loads (BUFFER_LOAD ... LDS): a scalar
// resource (base, size in bytes) and a per-lane 32-bit offset.  Lanes whose
// bytes lie beyond the size read zeros, which takes care of rows and weight
// groups past the end of an operand; lane l writes `dst` + size * l.
typedef int i32x4 __attribute__((ext_vector_type(4)));
extern "C" __device__ void llvm_amdgcn_raw_buffer_load_lds(i32x4 rsrc, LDS void* lds, int size,
                                                          int voffset, int soffset, int offset,
                                                          int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// resource for the bytes [off, n) of `base` (offsets fit 31 bits: checked
// on the host)
__device__ __forceinline__ i32x4 buf_rsrc(const uint8_t* base, int off, int n) {
  const uint64_t a = reinterpret_cast<uint64_t>(base) + uint32_t(off);
  return i32x4{int(uint32_t(a)), int(uint32_t(a >> 32) & 0xffff), n - off, 0x00020000};
}

// The operands as byte ranges.
struct Fp4PSrc {
  const uint8_t *ac, *as, *wc, *ws, *r;
  int ac_n, as_n, wc_n, ws_n, r_n;
  int K2, KB, KT;
};

// Per-lane offsets of the copies (fixed for the whole kernel): activation
// tile k and weight tile k of the wave, weight scale word, activation scale
// quarter (relative to its first row).
struct Fp4PLane {
  int a[4], w[4], ws, as;
};

__device__ __forceinline__ Fp4PLane fp4p_lane(const Fp4PSrc& b, int wave, int lane) {
  using C = Fp4P::C;
  static_assert(C::A_DMA == 4 && C::W_DMA == 4 && C::WS_DW == 64, "lane offsets");
  Fp4PLane o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int f = wave * 4 + k;
    // activation tile f: 16 rows x 64 B, rows in lane quads (fp4_swz)
    o.a[k] = (16 * f + (lane >> 2)) * b.K2 + ((lane & 3) ^ fp4_swz(lane >> 2)) * 16;
    // weight tile f: group f/2, 64-K half f%2, lane l's 16 bytes
    o.w[k] = ((f >> 1) * b.KT + (f & 1)) * 1024 + lane * 16;
  }
  const int e = wave * 64 + lane;  // weight scale word: (scale group, half, lane)
  o.ws = ((e >> 7) * b.KT * 64 + ((e >> 6) & 1) * 64 + (e & 63)) * 4;
  o.as = (wave * C::ASR + (lane >> 2)) * b.KB + 4 * (lane & 3);
  return o;
}

// The copies of one quad of 4 K-steps (all in one item): the stage copies of
// its K-step ks + j (tile at m0, g0) and the 4 quarters of its activation
// scale block, into scale buffer sbuf.
struct Fp4PQuad {
  int m0, g0, ks;
  int sbuf;
};

// Copy number k of a wave's share of K-step j of quad q (activation tiles,
// weight tiles, weight scale words, then with j = 0 the scale quarters).
template <int J, int FNE>
__device__ __forceinline__ void fp4p_copy(const Fp4PSrc& b, const Fp4PQuad& q, const Fp4PLane& o,
                                          LDS uint8_t* smem, LDS uint8_t* dst, int wave, int k) {
  using C = Fp4P::C;
  const int ks = q.ks + J;
  if (k < C::A_DMA) {
    llvm_amdgcn_raw_buffer_load_lds(buf_rsrc(b.ac, q.m0 * b.K2 + ks * 64, b.ac_n),
                                    dst + (wave * C::A_DMA + k) * 1024, 16, o.a[k], 0, 0, 0);
  } else if (k < C::A_DMA + C::W_DMA) {
    // (wave w copies weight tiles 4 w .. 4 w + 3, groups 2 w and 2 w + 1;
    // groups an item does not have come from an empty range)
    const int off = (q.g0 * b.KT + 2 * ks) * 1024;
    llvm_amdgcn_raw_buffer_load_lds(buf_rsrc(b.wc, off, FNE < 4 && wave >= FNE ? off : b.wc_n),
                                    dst + C::A_BYTES + (wave * C::W_DMA + k - C::A_DMA) * 1024, 16,
                                    o.w[k - C::A_DMA], 0, 0, 0);
  } else if (k == C::A_DMA + C::W_DMA) {
    llvm_amdgcn_raw_buffer_load_lds(buf_rsrc(b.ws, ((q.g0 / 4) * b.KT + 2 * ks) * 256, b.ws_n),
                                    dst + C::A_BYTES + C::W_BYTES + wave * 256, 4, o.ws, 0, 0, 0);
  } else {
    const int qq = k - (C::A_DMA + C::W_DMA + 1);
    llvm_amdgcn_raw_buffer_load_lds(buf_rsrc(b.as, (q.m0 + 16 * qq) * b.KB + 4 * q.ks, b.as_n),
                                    smem + C::AS_OFF + q.sbuf * C::ASB + wave * (C::ASR * 16) + qq * 256, 4,
                                    o.as, 0, 0, 0);
  }
}

// The lane index, read from the hardware where it is used.  Values derived
// from it for the per-item code (r copy, first reads, epilogue) are then
// computed there instead of being hoisted out of the item loop and held, or
// spilled, across it: reloading a spill would wait for every copy in flight.
__device__ __forceinline__ int fp4p_lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// r of an item (256 output features from n = 32 g0) into r buffer `rbuf`
__device__ __forceinline__ void fp4p_copy_r(const Fp4PSrc& b, LDS uint8_t* smem, int g0, int rbuf,
                                            int wave) {
  const int lane = fp4p_lane_id();
  llvm_amdgcn_raw_buffer_load_lds(buf_rsrc(b.r, g0 * 128, b.r_n),
                                  smem + Fp4P::R_OFF + rbuf * 1024 + wave * 256, 4, (wave * 64 + lane) * 4, 0,
                                  0, 0);
}

// One K-step of the stream, as Fp4Group: FNE x 2 groups of FM MFMAs (FNE =
// 2 for an n half), each followed by its share of the step's copies (K-step
// J of quad q) and of the reads of stream K-step pr.
template <int J, int G, int FNE>
struct Fp4PGroup {
  using C = Fp4P::C;
  static constexpr int FN = C::FN, FM = C::FM, NGRP = 2 * FNE, NC = Fp4P::copies(J);
  static constexpr int READS = 3 * FM + 2 + 2 * FNE;
  static __device__ __forceinline__ void run(v16f (&acc)[FN][FM], const Fp4Frags<FN, FM>& cur,
                                             Fp4Frags<FN, FM>& nxt, LDS uint8_t* smem,
                                             const Fp4PSrc& b, const Fp4PQuad& q, const Fp4PLane& o,
                                             LDS uint8_t* dst, const LDS uint8_t* __restrict__ st,
                                             int64_t pr, int wave, int wn, int wm, int lane, int goff) {
    constexpr int H = G / FNE, I = G % FNE;
#pragma unroll
    for (int j = 0; j < FM; ++j)
      acc[I][j] = mfma32_fp4_op<I, 2 * H>(cur.w[I][H], cur.a[j][H], acc[I][j], cur.sw[H], cur.sa[j]);
#pragma unroll
    for (int k = G * NC / NGRP; k < (G + 1) * NC / NGRP; ++k)
      fp4p_copy<J, FNE>(b, q, o, smem, dst, wave, k);
    constexpr int RG = NGRP - 2;
    if constexpr (G < RG) {
#pragma unroll
      for (int r = G * READS / RG; r < (G + 1) * READS / RG; ++r)
        fp4_read_item<Fp4P::BN, Fp4P::BM, Fp4P::DEPTH, Fp4P::NSB, FNE>(st, smem, pr, wn, wm, lane, nxt, r,
                                                                       goff);
    }
    if constexpr (G + 1 == NGRP) fp4_fix_scales<FM>(nxt.sa, lane);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (G + 1 < NGRP)
      Fp4PGroup<J, G + 1, FNE>::run(acc, cur, nxt, smem, b, q, o, dst, st, pr, wave, wn, wm, lane, goff);
  }
};

// Step p = 4 p4 + J of the stream (position J of its quad; quads start at
// multiples of 4, so K-step p is in stage J): wait for the stage of K-step
// p + 1 and barrier, then MFMAs of K-step p from `cur`, copies of stream
// K-step p + DEPTH (K-step J of quad q) into stage J, reads of K-step p + 1
// into `nxt`.  The wait leaves in flight the younger(J) copies this wave
// issued after that stage, plus X other operations issued after it (in the
// first quad of an item: the previous item's epilogue stores and the r
// copy); vector memory operations complete in issue order, so anything
// else issued later only makes the wait stricter.  The stage indices are
// compile-time, so the LDS reads use immediate offsets.
template <int J, int X, int FNE>
__device__ __forceinline__ void fp4p_step(v16f (&acc)[4][4], const Fp4Frags<4, 4>& cur,
                                          Fp4Frags<4, 4>& nxt, LDS uint8_t* smem, const Fp4PSrc& b,
                                          const Fp4PQuad& q, const Fp4PLane& o, int p4, int wave, int wn,
                                          int wm, int lane, int goff) {
  using C = Fp4P::C;
  __builtin_amdgcn_s_waitcnt(vm_lgkm0_encoding(Fp4P::younger(J) + X));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  Fp4PGroup<J, 0, FNE>::run(acc, cur, nxt, smem, b, q, o, smem + J * C::STAGE,
                            smem + ((J + 1) & 3) * C::STAGE, 4 * int64_t(p4) + J + 1, wave, wn, wm, lane,
                            goff);
}

// Y[m0.., n0..] = bf16(acc * r) for the wave's 128 x 128 block, straight
// from the accumulators.  In a 32 x 32 block, lane l holds row l % 32 and
// for g = 0..3 the 4 columns 8 g + 4 (l / 32) + 0..3.  Two lane exchanges
// give each lane 8 consecutive columns: swapping the upper lane half of the
// group-2p words with the lower lane half of the group-(2p+1) words leaves
// lane l with columns 16 p + 8 (l / 32) + 0..7 of row l % 32 (p = 0, 1);
// swapping 16-lane rows 1 and 3 of the p = 0 set with rows 0 and 2 of the
// p = 1 set then leaves the first set with rows 0..15 and the second with
// rows 16..31, lane l holding row l % 16, columns 8 c + 0..7 with
// c = 2 ((l / 16) % 2) + l / 32.  Each 16-byte-per-lane store thus writes
// 16 rows x 64 bytes.  Blocks go out row band by row band (j outer), so a
// band's rows are written as whole 256-byte segments back to back.  Exactly
// EPI_STORES buffer stores per wave (the first K-steps of the next item
// count them): an n half (FNE = 2) stores its 8 blocks and issues the
// other 8 blocks' stores at an offset past the buffer, where they write
// nothing.
template <int FNE>
__device__ __forceinline__ void fp4p_epilogue(const v16f (&acc)[4][4], LDS uint8_t* base, int rbuf,
                                              uint16_t* __restrict__ Y, int64_t M, int64_t N,
                                              int64_t m0, int64_t n0, int wn, int wm) {
  const int lane = fp4p_lane_id(), h = lane >> 5;
  const LDS uint8_t* rb = base + Fp4P::R_OFF + rbuf * 1024;
  const int64_t rows = M - m0 < Fp4P::BM ? M - m0 : Fp4P::BM;
  const __amdgpu_buffer_rsrc_t ys =
      __builtin_amdgcn_make_buffer_rsrc(Y + m0 * N, 0, int(rows * N * 2), 0x00020000);
  v4f rs[4][4];
#pragma unroll
  for (int i = 0; i < FNE; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      rs[i][g] = *reinterpret_cast<const LDS v4f*>(rb + (wn * 32 * FNE + 32 * i + 8 * g + 4 * h) * 4);
  // 32-bit offsets: the host checks 256 N * 2 < 2^31
  const int N32 = int(N), row = wm * 128 + (lane & 15);
  const int n32 = int(n0) + wn * 32 * FNE + 8 * (2 * ((lane >> 4) & 1) + h);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= FNE) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, ys, -1, 0, 0);
        continue;
      }
      // read this block's accumulators here, not all of them up front
      v16f av = acc[i][j];
      asm volatile("" : "+a"(av));
      u32x4 v[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const v4f a0 = {av[8 * p], av[8 * p + 1], av[8 * p + 2], av[8 * p + 3]};
        const v4f a1 = {av[8 * p + 4], av[8 * p + 5], av[8 * p + 6], av[8 * p + 7]};
        const u32x2 lo = scale_pack4(a0, rs[i][2 * p]), hi = scale_pack4(a1, rs[i][2 * p + 1]);
        const auto s0 = __builtin_amdgcn_permlane32_swap(lo.x, hi.x, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(lo.y, hi.y, false, false);
        v[p] = u32x4{s0[0], s1[0], s0[1], s1[1]};
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const auto t = __builtin_amdgcn_permlane16_swap(v[0][d], v[1][d], false, false);
        v[0][d] = t[0];
        v[1][d] = t[1];
      }
      // columns beyond N: offset -1 (beyond the buffer, dropped), formed
      // without a compare so that every store is issued (the wave counts them)
      const int n = n32 + 32 * i;
      const int past = (N32 - 1 - n) >> 31;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int m = row + 32 * j + 16 * hh;
        __builtin_amdgcn_raw_buffer_store_b128(v[hh], ys, ((m * N32 + n) * 2) | past, 0, 0);
      }
    }
}

// Prologue of a stream: r of its first item (buffer 0), the copies of its
// first quad, then EPI_STORES stores that write nothing (offsets beyond an
// empty buffer), so that the first item's first quad finds as many
// operations after its copies as every later item does (an epilogue's).
template <int FNE>
__device__ __forceinline__ void fp4p_prologue(const Fp4PSrc& b, const Fp4PLane& o, LDS uint8_t* base,
                                              const Fp4PDesc& d0, uint16_t* Y, int wave) {
  using C = Fp4P::C;
  fp4p_copy_r(b, base, d0.g0, 0, wave);
  const Fp4PQuad q{d0.m0, d0.g0, d0.ks0, 0};
#pragma unroll
  for (int k = 0; k < Fp4P::copies(0); ++k) fp4p_copy<0, FNE>(b, q, o, base, base, wave, k);
#pragma unroll
  for (int k = 0; k < Fp4P::copies(1); ++k) fp4p_copy<1, FNE>(b, q, o, base, base + C::STAGE, wave, k);
#pragma unroll
  for (int k = 0; k < Fp4P::copies(2); ++k) fp4p_copy<2, FNE>(b, q, o, base, base + 2 * C::STAGE, wave, k);
#pragma unroll
  for (int k = 0; k < Fp4P::copies(3); ++k) fp4p_copy<3, FNE>(b, q, o, base, base + 3 * C::STAGE, wave, k);
  const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(Y, 0, 0, 0x00020000);
  // (16-byte stores 32 bytes apart: nothing for the compiler to merge)
#pragma unroll
  for (int k = 0; k < Fp4P::EPI_STORES; ++k)
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, none, 32 * k, 0, 0);
  // stage 0 (and scale block 0) landed: 3 K-steps of copies and the stores
  // issued after it
  __builtin_amdgcn_s_waitcnt(vm_lgkm0_encoding(Fp4P::copies(1) + Fp4P::copies(2) + Fp4P::copies(3) +
                                               Fp4P::EPI_STORES));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The quad of an item starting at item position u (stream K-step p + u):
// its copies are of the next quad, in this item or (the item's last quad)
// the first of item d1.
__device__ __forceinline__ Fp4PQuad fp4p_quad(const Fp4PDesc& d0, const Fp4PDesc& d1, int64_t p, int u) {
  const bool nx = u + 4 >= d0.len;
  Fp4PQuad q;
  q.m0 = nx ? d1.m0 : d0.m0;
  q.g0 = nx ? d1.g0 : d0.g0;
  q.ks = nx ? d1.ks0 : d0.ks0 + u + 4;
  q.sbuf = int(((p + u) >> 2) + 1) & 1;
  return q;
}

// The K-steps of item d0 (stream K-steps p..p + d0.len - 1, p a multiple
// of 4), one quad at a time.  The first quad's waits for stages copied
// before the previous epilogue also leave that epilogue's stores and the r
// copy (ITEM_OPS) in flight.  FNE = 2 for an n half.
template <int FNE>
__device__ __forceinline__ void fp4p_item(v16f (&acc)[4][4], Fp4Frags<4, 4>& fa, Fp4Frags<4, 4>& fb,
                                          LDS uint8_t* base, const Fp4PSrc& b, const Fp4PLane& o,
                                          const Fp4PDesc& d0, const Fp4PDesc& d1, int64_t p, int wave,
                                          int wn, int wm, int lane) {
  constexpr int X = Fp4P::ITEM_OPS;
  const int goff = FNE == 3 ? d0.g0 & 3 : 0;
  {
    const Fp4PQuad q = fp4p_quad(d0, d1, p, 0);
    const int p4 = int(p >> 2);
    fp4p_step<0, X, FNE>(acc, fa, fb, base, b, q, o, p4, wave, wn, wm, lane, goff);
    fp4p_step<1, X, FNE>(acc, fb, fa, base, b, q, o, p4, wave, wn, wm, lane, goff);
    fp4p_step<2, X, FNE>(acc, fa, fb, base, b, q, o, p4, wave, wn, wm, lane, goff);
    fp4p_step<3, 0, FNE>(acc, fb, fa, base, b, q, o, p4, wave, wn, wm, lane, goff);
  }
  for (int u = 4; u < d0.len; u += 4) {
    const Fp4PQuad q = fp4p_quad(d0, d1, p, u);
    const int p4 = int((p + u) >> 2);
    fp4p_step<0, 0, FNE>(acc, fa, fb, base, b, q, o, p4, wave, wn, wm, lane, goff);
    fp4p_step<1, 0, FNE>(acc, fb, fa, base, b, q, o, p4, wave, wn, wm, lane, goff);
    fp4p_step<2, 0, FNE>(acc, fa, fb, base, b, q, o, p4, wave, wn, wm, lane, goff);
    fp4p_step<3, 0, FNE>(acc, fb, fa, base, b, q, o, p4, wave, wn, wm, lane, goff);
  }
}

// FNE: the items' width (see fp4p_desc); `items` of them in the launch.
template <int FNE>
__global__ __launch_bounds__(256, 1) void gemm_fp4_persistent_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int tiles_m, int items) {
  if (!blob_header_ok(blob, MXFP4, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  using C = Fp4P::C;
  constexpr int FN = C::FN, FM = C::FM, DEPTH = Fp4P::DEPTH;
  const BlobLayout L = blob_layout(MXFP4, N, K);
  Fp4PSched S;
  S.init(items, tiles_m, int(L.KS), int(blockIdx.x));
  if (S.n_items == 0) return;

  Fp4PSrc b;
  b.ac = a_codes;
  b.as = a_scales;
  b.wc = blob + L.code_off;
  b.ws = blob + L.scale_off;
  b.r = blob + L.r_off;
  b.K2 = int(K / 2);
  b.KB = int(K / 32);
  b.KT = int(L.KT);
  b.ac_n = int(M * b.K2);
  b.as_n = int(M * b.KB);
  b.wc_n = int(L.NG * L.KT * 1024);
  b.ws_n = int(L.NSG * L.KT * 256);
  b.r_n = int(N * 4);
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Fp4P::LDS_BYTES];
  LDS uint8_t* base = (LDS uint8_t*)smem;
  // the wave index as a scalar, so that wave-dependent LDS addresses are too
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int wn = wave % C::WN, wm = wave / C::WN;
  const Fp4PLane o = fp4p_lane(b, wave, lane);

  fp4p_prologue<FNE>(b, o, base, fp4p_desc<FNE>(S, 0), Y, wave);

  int64_t p = 0;  // stream K-step whose MFMAs run next
  for (int k = 0; k < S.n_items; ++k) {
    const Fp4PDesc d0 = fp4p_desc<FNE>(S, k), d1 = fp4p_desc<FNE>(S, k + 1);
    v16f acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    // The stage of K-step p has landed (the wait of the previous step, or of
    // the prologue), and every wave is past item k-1's epilogue: r of item
    // k+1 goes into the r buffer item k-1 used.
    __builtin_amdgcn_s_barrier();
    fp4p_copy_r(b, base, d1.g0, (k + 1) & 1, wave);
    // the item's first fragments (read here rather than carried from the
    // previous item's last step, so that none are live in its epilogue)
    Fp4Frags<FN, FM> fa, fb;
    fp4_read_all<Fp4P::BN, Fp4P::BM, DEPTH, Fp4P::NSB, FNE>(base, base, 4 * int64_t(p >> 2), wn, wm,
                                                            fp4p_lane_id(), fa, FNE == 3 ? d0.g0 & 3 : 0);
    fp4p_item<FNE>(acc, fa, fb, base, b, o, d0, d1, p, wave, wn, wm, lane);
    p += d0.len;

    const int64_t n0 = int64_t(d0.g0) * 32;
    fp4p_epilogue<FNE>(acc, base, k & 1, Y, M, N, d0.m0, n0, wn, wm);
  }
  // every copy (the last ones repeat valid sources) lands before the end
  __builtin_amdgcn_s_waitcnt(0);
}

// The persistent kernel's conditions: K in whole quads of 128-wide K-steps,
// operands and Y's tile rows addressable by 32-bit buffer offsets, and one of
//   * at least 256 tiles of 256 x 256 (whole tiles, FNE = 4), or 192..256
//     tiles when 256 x 192 tiles would need more than one round;
//   * 129..256 tiles with M >= 1024 (256-row tiles mostly full) whose 256 x
//     192 tiles fit one round (FNE = 3: the 6144 x 4096 projection at M =
//     2048, 192 tiles, runs as 256 tiles of 3/4 the work);
//   * 96..128 tiles with M >= 1024: n halves (FNE = 2), at most one per CU,
//     faster there than the 256 (n) x 128 (m) tile kernel (the 4096 x 4096
//     projection at M = 2048: 33.8 -> 30.3 us).
// Below that the one-tile-per-workgroup kernels do as well.  (Halves after
// whole rounds, for a last round of few tiles, gained nothing on the 28672 x
// 4096 projection: the CUs a short last round leaves idle give the busy ones
// power headroom.)
static bool fp4_persistent_limits(int64_t M, int64_t N, int64_t K) {
  return M > 32 && K % 512 == 0 && ((N + 255) / 256) * ((M + 255) / 256) < (int64_t(1) << 23) &&
         int64_t(Fp4P::BM) * N * 2 < (int64_t(1) << 31) && M * (K / 2) < (int64_t(1) << 31) &&
         ((N + 31) / 32) * 32 * (K / 2) < (int64_t(1) << 31);
}

// item width of the persistent kernel for the shape (0: not taken)
static int fp4_persistent_fne(int64_t M, int64_t N, int64_t K) {
  if (!fp4_persistent_limits(M, N, K)) return 0;
  const int64_t tm = (M + 255) / 256;
  const int64_t T = ((N + 255) / 256) * tm, T3 = ((N + 191) / 192) * tm;
  if (M >= 1024 && T > 128 && T <= 256 && T3 <= 256) return 3;
  if (T >= 192) return 4;
  if (M >= 1024 && T >= 96 && T <= 128) return 2;
  return 0;
}

bool fp4_persistent_fits(int64_t M, int64_t N, int64_t K) { return fp4_persistent_fne(M, N, K) != 0; }

hipError_t launch_fp4_persistent(int64_t M, int64_t N, int64_t K, const uint8_t* ac,
                                 const uint8_t* as, const uint8_t* blob, uint16_t* Y,
                                 hipStream_t stream) {
  const int tiles_m = int((M + 255) / 256);
  const dim3 grid(Fp4P::XCDS * Fp4P::PER_XCD);
  switch (fp4_persistent_fne(M, N, K)) {
    case 3:
      hipLaunchKernelGGL(gemm_fp4_persistent_kernel<3>, grid, dim3(256), 0, stream, ac, as, blob, Y, M, N, K,
                         tiles_m, int((N + 191) / 192) * tiles_m);
      break;
    case 2:
      hipLaunchKernelGGL(gemm_fp4_persistent_kernel<2>, grid, dim3(256), 0, stream, ac, as, blob, Y, M, N, K,
                         tiles_m, 2 * int((N + 255) / 256) * tiles_m);
      break;
    default:
      hipLaunchKernelGGL(gemm_fp4_persistent_kernel<4>, grid, dim3(256), 0, stream, ac, as, blob, Y, M, N, K,
                         tiles_m, int((N + 255) / 256) * tiles_m);
  }
  return hipGetLastError();
}

// ========================== MXFP4, K split in two across workgroups ==
//
// Shapes with too few 256 x 256 tiles to fill the chip (64..128 tiles) and a
// long K (such as the 4096 x 14336 down projection at M = 2048) split each
// tile's K-steps into two
// halves, run by two workgroups with the persistent kernel's prologue, copy
// ring and K loop (one item each; items are part-major, so each XCD works on
// one K half of its tiles).  The halves meet per wave slot, the 128 x 128
// block of wave (wm, wn) (64 KiB of fp32): of the two waves holding a slot,
// the one that takes the slot's ticket first writes its partial sums
// (agent-coherent write-through stores) and raises the slot's flag; the
// second waits for the flag, adds those sums to its own and runs the
// epilogue, then clears the ticket and the flag, so the synchronization
// words are zero again after every call.  The second wave only waits for a
// wave that is already past its K loop, so no wait depends on how the
// workgroups are scheduled.

// Workspace: the tickets and flags of up to MAX_TILES tiles at fixed places
// (one 4 KiB block, whatever the shape, so that shapes sharing a workspace
// never write partial sums over each other's synchronization words), a
// status word (non-zero once a wave gave up waiting for its partner; the
// block it owns is then written as NaN), then the partial-sum slots.
struct Fp4S {
  static constexpr int SLOTS = 4;                   // wave slots per tile
  static constexpr int MAX_TILES = 128;
  static constexpr int SLOT_BYTES = 64 * 1024;      // 128 x 128 fp32
  static constexpr int WORDS_BYTES = MAX_TILES * SLOTS * 8;
  static constexpr int STATUS_OFF = WORDS_BYTES;
  static constexpr int SYNC_BYTES = WORDS_BYTES + 256;
  static constexpr int CACHE_THROUGH = 16;          // sc1: agent-coherent, past the L2s
  static constexpr int SPIN_LIMIT = 1 << 20;        // polls of the partner's flag (~1 s)
};
static_assert(Fp4S::WORDS_BYTES == 4096 && Fp4S::SYNC_BYTES == W4A4_SPLITK_SYNC_BYTES &&
                  Fp4S::STATUS_OFF == W4A4_SPLITK_STATUS_OFFSET,
              "split-K workspace layout");
static_assert(kNoAllocScratchBytes ==
                  size_t(Fp4S::SYNC_BYTES) + size_t(Fp4S::MAX_TILES) * Fp4S::SLOTS * Fp4S::SLOT_BYTES,
              "the allocation-free scratch holds the largest split-K workspace");

// The partner's partial sums for the blocks in epilogue order e = 4 j + i:
// quarter q of block e is 1 KiB at (4 e + q) KiB, lane l's 16 bytes at 16 l
// (each store or load instruction moves one contiguous KiB; write-through
// of partial lines was 4x slower), 8 blocks in flight.
__device__ __forceinline__ v16f fp4s_load_block(__amdgpu_buffer_rsrc_t pr, int e, int lane) {
  v16f v;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(pr, ((e * 4 + q) * 64 + lane) * 16, 0,
                                                          Fp4S::CACHE_THROUGH);
    v[4 * q] = __uint_as_float(w.x);
    v[4 * q + 1] = __uint_as_float(w.y);
    v[4 * q + 2] = __uint_as_float(w.z);
    v[4 * q + 3] = __uint_as_float(w.w);
  }
  return v;
}

// As fp4p_epilogue, with the partner's partial sums added to each block.
// With met == false (the partner's flag never came) the wave's 128 x 128
// block of Y is written as BF16 NaN instead, and no partial sum is read.
__device__ __forceinline__ void fp4s_epilogue(const v16f (&acc)[4][4], __amdgpu_buffer_rsrc_t pr,
                                              LDS uint8_t* base, int rbuf, uint16_t* __restrict__ Y,
                                              int64_t M, int64_t N, int64_t m0, int64_t n0, int wn,
                                              int wm, bool met) {
  const int lane = fp4p_lane_id(), h = lane >> 5;
  const LDS uint8_t* rb = base + Fp4P::R_OFF + rbuf * 1024;
  const int64_t rows = M - m0 < Fp4P::BM ? M - m0 : Fp4P::BM;
  const __amdgpu_buffer_rsrc_t ys =
      __builtin_amdgcn_make_buffer_rsrc(Y + m0 * N, 0, int(rows * N * 2), 0x00020000);
  if (!met) {
    const int N32 = int(N), row = wm * 128 + (lane & 15);
    const int n32 = int(n0) + wn * 128 + 8 * (2 * ((lane >> 4) & 1) + h);
    const u32x4 nan = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n32 + 32 * i;
        const int past = (N32 - 1 - n) >> 31;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int m = row + 32 * j + 16 * hh;
          __builtin_amdgcn_raw_buffer_store_b128(nan, ys, ((m * N32 + n) * 2) | past, 0, 0);
        }
      }
    return;
  }
  v16f pb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) pb[e] = fp4s_load_block(pr, e, lane);
  v4f rs[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      rs[i][g] = *reinterpret_cast<const LDS v4f*>(rb + (wn * 128 + 32 * i + 8 * g + 4 * h) * 4);
  const int N32 = int(N), row = wm * 128 + (lane & 15);
  const int n32 = int(n0) + wn * 128 + 8 * (2 * ((lane >> 4) & 1) + h);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * j + i;
      v16f av = acc[i][j];
      asm volatile("" : "+a"(av));
      av += pb[e & 7];
      if (e + 8 < 16) pb[e & 7] = fp4s_load_block(pr, e + 8, lane);
      u32x4 v[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const v4f a0 = {av[8 * p], av[8 * p + 1], av[8 * p + 2], av[8 * p + 3]};
        const v4f a1 = {av[8 * p + 4], av[8 * p + 5], av[8 * p + 6], av[8 * p + 7]};
        const u32x2 lo = scale_pack4(a0, rs[i][2 * p]), hi = scale_pack4(a1, rs[i][2 * p + 1]);
        const auto s0 = __builtin_amdgcn_permlane32_swap(lo.x, hi.x, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(lo.y, hi.y, false, false);
        v[p] = u32x4{s0[0], s1[0], s0[1], s1[1]};
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const auto t = __builtin_amdgcn_permlane16_swap(v[0][d], v[1][d], false, false);
        v[0][d] = t[0];
        v[1][d] = t[1];
      }
      const int n = n32 + 32 * i;
      const int past = (N32 - 1 - n) >> 31;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int m = row + 32 * j + 16 * hh;
        __builtin_amdgcn_raw_buffer_store_b128(v[hh], ys, ((m * N32 + n) * 2) | past, 0, 0);
      }
    }
}

__global__ __launch_bounds__(256, 1) void gemm_fp4_splitk_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int tiles_m, int T, uint8_t* __restrict__ ws) {
  if (!blob_header_ok(blob, MXFP4, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  using C = Fp4P::C;
  constexpr int FN = C::FN, FM = C::FM, DEPTH = Fp4P::DEPTH;
  const BlobLayout L = blob_layout(MXFP4, N, K);
  // the 2T items (part-major) in the XCD chunks of Fp4PSched: one per workgroup
  Fp4PSched S;
  S.init(2 * T, tiles_m, int(L.KS), int(blockIdx.x));
  if (S.n_items == 0) return;
  const int item = S.tile(0), part = item / T, t = item % T;
  const int half = int(L.KS / 2);
  Fp4PDesc d0;
  d0.m0 = (t % tiles_m) * Fp4P::BM;
  d0.g0 = (t / tiles_m) * (Fp4P::BN / 32);
  d0.ks0 = part * half;
  d0.len = half;
  Fp4PDesc d1 = d0;  // nothing follows: the ring copies this item's last quad again
  d1.ks0 = d0.ks0 + half - 4;
  d1.len = 4;

  Fp4PSrc b;
  b.ac = a_codes;
  b.as = a_scales;
  b.wc = blob + L.code_off;
  b.ws = blob + L.scale_off;
  b.r = blob + L.r_off;
  b.K2 = int(K / 2);
  b.KB = int(K / 32);
  b.KT = int(L.KT);
  b.ac_n = int(M * b.K2);
  b.as_n = int(M * b.KB);
  b.wc_n = int(L.NG * L.KT * 1024);
  b.ws_n = int(L.NSG * L.KT * 256);
  b.r_n = int(N * 4);
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Fp4P::LDS_BYTES];
  LDS uint8_t* base = (LDS uint8_t*)smem;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int wn = wave % C::WN, wm = wave / C::WN;
  const Fp4PLane o = fp4p_lane(b, wave, lane);

  fp4p_prologue<4>(b, o, base, d0, Y, wave);
  v16f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  // as the persistent kernel's item start (its r copy goes to the unused
  // buffer 1, keeping the first quad's wait counts)
  __builtin_amdgcn_s_barrier();
  fp4p_copy_r(b, base, d0.g0, 1, wave);
  Fp4Frags<FN, FM> fa, fb;
  fp4_read_all<Fp4P::BN, Fp4P::BM, DEPTH, Fp4P::NSB>(base, base, 0, wn, wm, fp4p_lane_id(), fa);
  fp4p_item<4>(acc, fa, fb, base, b, o, d0, d1, 0, wave, wn, wm, lane);

  // the meeting of the two halves at this wave's slot
  const int slot = t * Fp4S::SLOTS + wm * 2 + wn;
  int* tickets = reinterpret_cast<int*>(ws);
  int* flags = tickets + Fp4S::MAX_TILES * Fp4S::SLOTS;
  uint8_t* pslot = ws + Fp4S::SYNC_BYTES + int64_t(slot) * Fp4S::SLOT_BYTES;
  const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(pslot, 0, Fp4S::SLOT_BYTES, 0x00020000);
  int first = 0;
  if (lane == 0) first = __hip_atomic_fetch_add(&tickets[slot], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0;
  first = __builtin_amdgcn_readfirstlane(first);
  if (first) {
    const int l = fp4p_lane_id();
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v16f av = acc[i][j];
        asm volatile("" : "+a"(av));
        const int e = 4 * j + i;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          __builtin_amdgcn_raw_buffer_store_b128(
              u32x4{__float_as_uint(av[4 * q]), __float_as_uint(av[4 * q + 1]), __float_as_uint(av[4 * q + 2]),
                    __float_as_uint(av[4 * q + 3])},
              pr, ((e * 4 + q) * 64 + l) * 16, 0, Fp4S::CACHE_THROUGH);
      }
    // The sums are device-scope write-through stores: once they have
    // completed (waitcnt) they are at the coherent level, and a
    // workgroup-scope release fence keeps the flag store behind them.  (An
    // agent-scope release would also write back this XCD's whole L2, none
    // of it ours: measured +11 us on the 4096 x 14336 projection.)
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) __hip_atomic_store(&flags[slot], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    // the other wave is past its K loop: it raises the flag after its
    // stores.  The poll is bounded; a wave that gives up (the partner never
    // raised the flag: synchronization words left non-zero by a caller, or
    // a partner that never arrived) records it in the status word and
    // writes its block as NaN rather than adding a slot nobody filled.
    // The partial sums are read with device-scope (sc1) loads, which see
    // the coherent level, so the acquire only has to keep them behind the
    // flag: the poll is an agent-scope load, then a workgroup-scope acquire
    // fence orders what follows.  (An agent-scope acquire would also
    // invalidate this XCD's L2, which cost the other workgroups' cached
    // tiles ~32 us on the 4096 x 14336 projection at M = 2048.)
    int met = 1;
    if (lane == 0) {
      met = 0;
      for (int n = 0; n < Fp4S::SPIN_LIMIT; ++n) {
        if (__hip_atomic_load(&flags[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
          met = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      if (!met)
        __hip_atomic_fetch_or(reinterpret_cast<int*>(ws + Fp4S::STATUS_OFF), 1, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
    }
    met = __builtin_amdgcn_readfirstlane(met);
    fp4s_epilogue(acc, pr, base, 0, Y, M, N, d0.m0, int64_t(d0.g0) * 32, wn, wm, met != 0);
    __builtin_amdgcn_s_waitcnt(0);
    if (lane == 0) {
      __hip_atomic_store(&flags[slot], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&tickets[slot], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// Split-K conditions: 64..128 tiles of 256 x 256 (2T <= 256 workgroups),
// each K half whole quads, offsets in 32 bits, and K >= 8192: the exchange
// of the halves costs about as much as 16 K-steps (at K = 4096 the
// 256 x 128 tile kernel is faster, at K = 14336 the split is 16% faster).
bool fp4_splitk_fits(int64_t M, int64_t N, int64_t K) {
  const int64_t T = ((N + 255) / 256) * ((M + 255) / 256);
  return M > 32 && K % 1024 == 0 && K >= 8192 && T >= 64 && T <= Fp4S::MAX_TILES &&
         int64_t(Fp4P::BM) * N * 2 < (int64_t(1) << 31) && M * (K / 2) < (int64_t(1) << 31) &&
         ((N + 31) / 32) * 32 * (K / 2) < (int64_t(1) << 31);
}

size_t fp4_splitk_workspace(int64_t M, int64_t N) {
  const int64_t T = ((N + 255) / 256) * ((M + 255) / 256);
  return size_t(Fp4S::SYNC_BYTES + T * Fp4S::SLOTS * int64_t(Fp4S::SLOT_BYTES));
}

hipError_t launch_fp4_splitk(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                             const uint8_t* blob, uint16_t* Y, void* workspace, hipStream_t stream) {
  const int tiles_m = int((M + 255) / 256);
  const int T = int((N + 255) / 256) * tiles_m;
  hipLaunchKernelGGL(gemm_fp4_splitk_kernel, dim3(Fp4P::XCDS * Fp4P::PER_XCD), dim3(256), 0, stream, ac, as,
                     blob, Y, M, N, K, tiles_m, T, static_cast<uint8_t*>(workspace));
  return hipGetLastError();
}

// MXFP4 weight streaming for M <= 32: one workgroup per 32 output features
// (groups run on XCD b % 8 in contiguous per-XCD ranges, as in the 16-feature
// kernel), WAVES waves splitting its 64-K tiles into contiguous ranges.  Each
// wave streams its tiles from HBM straight into registers in batches of U
// (U coalesced 1 KiB non-temporal loads in flight per wave, no LDS); the
// activation rows are the MFMA's second operand (rows >= M are zero, and
// their lanes load nothing), loaded as row-contiguous lane pairs and moved to
// the fragment lanes with a lane permutation.  Partial sums are added
// through LDS and wave 0 runs the epilogue.
template <int WAVES, int U>
__global__ __launch_bounds__(64 * WAVES) void gemm_fp4_decode_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K) {
  if (!blob_header_ok(blob, MXFP4, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  const BlobLayout L = blob_layout(MXFP4, N, K);
  const u32x4* __restrict__ Wc = reinterpret_cast<const u32x4*>(blob + L.code_off);
  const uint32_t* __restrict__ Ws = reinterpret_cast<const uint32_t*>(blob + L.scale_off);
  const float* __restrict__ R = reinterpret_cast<const float*>(blob + L.r_off);

  const int64_t G = (N + 31) / 32, per_x = (G + 7) / 8;
  const int64_t g = int64_t(blockIdx.x % 8) * per_x + blockIdx.x / 8;
  if (g >= G) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5;
  const int64_t m = lane & 31;
  const bool mvalid = m < M;
  const int64_t row = mvalid ? m : 0;
  const int64_t KT = L.KT, K2 = K / 2, KB = K / 32;
  const int64_t per = (KT + WAVES - 1) / WAVES;
  const int64_t k_begin = wave * per;
  const int64_t k_end = k_begin + per < KT ? k_begin + per : KT;
  const int sw_shift = 8 * int(g & 3);
  const uint32_t* __restrict__ Wsg = Ws + (g >> 2) * KT * 64 + lane;
  const u32x4* __restrict__ Wg = Wc + g * KT * 64 + lane;
  // activation codes: lane l loads row l / 2, 16-byte half l % 2 of the
  // tile's 32 bytes (only the lanes of rows < M load); fragment lane l
  // (row l % 32, half l / 32) reads it from lane 2 (l % 32) + l / 32
  const int lr = lane >> 1;
  const bool lvalid = lr < M;
  const uint8_t* __restrict__ arow = a_codes + (lvalid ? lr : 0) * K2 + 16 * (lane & 1);
  const int perm = 4 * (2 * int(m) + half);
  const uint8_t* __restrict__ srow = a_scales + row * KB + half;

  v16f acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  for (int64_t h0 = k_begin; h0 < k_end; h0 += U) {
    u32x4 wf[U], af[U];
    uint32_t swd[U];
    int sab[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t h = h0 + u;
      const bool ok = h < k_end;
      const int64_t hc = ok ? h : k_end - 1;  // clamped: loads stay in range
      wf[u] = __builtin_nontemporal_load(&Wg[hc * 64]);
      swd[u] = __builtin_nontemporal_load(&Wsg[hc * 64]);
      u32x4 a = {0u, 0u, 0u, 0u};
      if (lvalid) a = *reinterpret_cast<const u32x4*>(arow + hc * 32);
      af[u] = ok ? a : u32x4{0u, 0u, 0u, 0u};
      sab[u] = mvalid ? int(srow[hc * 2]) : 127;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      u32x4 a;
      a.x = uint32_t(__builtin_amdgcn_ds_bpermute(perm, int(af[u].x)));
      a.y = uint32_t(__builtin_amdgcn_ds_bpermute(perm, int(af[u].y)));
      a.z = uint32_t(__builtin_amdgcn_ds_bpermute(perm, int(af[u].z)));
      a.w = uint32_t(__builtin_amdgcn_ds_bpermute(perm, int(af[u].w)));
      acc = mfma32_fp4_op<0, 0>(wf[u], a, acc, int(swd[u] >> sw_shift), sab[u]);
    }
  }

  __shared__ v16f red[WAVES > 1 ? WAVES - 1 : 1][64];
  if (wave != 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll 1
  for (int w = 0; w < WAVES - 1; ++w) {
    const v16f o = red[w][lane];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] += o[e];
  }
  if (!mvalid) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t n = g * 32 + 8 * q + 4 * half;
    if (n < N) {
      const float4 r = *reinterpret_cast<const float4*>(R + n);
      store4(Y, N, m, n, v4f{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]},
             v4f{r.x, r.y, r.z, r.w});
    }
  }
}

template <int WAVES, int U>
hipError_t launch_fp4_decode(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                             const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_fp4_decode_kernel<WAVES, U>), dim3(unsigned(((N + 31) / 32 + 7) / 8 * 8)),
                     dim3(64 * WAVES), 0, stream, ac, as, blob, Y, M, N, K);
  return hipGetLastError();
}

// MXFP4 weight streaming for M <= 16: one workgroup per FS x 16 output
// features (FS = 1: one half of a 32-row weight group; FS = 2: the whole
// group, for large N), on the 16x16x128 scaled MFMA with the activation rows
// as its 16 columns (columns >= M are zero).  With FS = 1 there are twice as
// many workgroups as 32-row groups, so every CU streams even when N is only
// 4096; with FS = 2 each activation fragment (and its scale) serves two
// weight fragments, halving the activation loads per weight byte, which at
// M = 16 cost the texture unit as much as the weights.  Workgroup b takes
// slice (b % 8) S + b / 8 (S slices per XCD): consecutive slices, which
// share 1 KiB weight tiles and scale words, run on one XCD at about the same
// time.  The WAVES waves split the 128-wide K-steps into contiguous ranges;
// each wave issues the loads of up to U K-steps at once, then their MFMAs.
// Weight fragment lane l holds row l % 16 and 32-wide K chunk l / 16 of a
// K-step: the tile of 64-K half (l / 16) / 2 and, in it, tile lane 32 ((l /
// 16) % 2) + 16 h + l % 16 for group half h, so each 16-lane group reads
// 256 contiguous bytes; the weight stream is read once, with non-temporal
// loads.  Activation codes are loaded with lane l taking row l / 4, 16-byte
// chunk l % 4 (a row's 64 bytes per lane quad), then moved to the fragment
// lane (chunk l / 16 of row l % 16) with a lane permutation.  Partial sums
// of the waves are added through LDS and wave 0 runs the epilogue.
//
// SD (M > 4): the activation scale bytes come as dwords, lane (r, c) loading
// the four block scales of row r for K-step s + c, and reach the fragment
// lanes through a lane permutation: one scale load per 4 K-steps instead of
// one per K-step, each touching the same 16 rows.
template <int WAVES, int U, int FS = 1, bool SD = false>
__global__ __launch_bounds__(64 * WAVES) void gemm_fp4_decode16_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K) {
  static_assert(FS == 1 || FS == 2 || FS == 4, "one half, one or two 32-row groups");
  static_assert(!SD || U % 4 == 0, "scale dwords cover whole groups of 4 K-steps");
  if (!blob_header_ok(blob, MXFP4, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  const BlobLayout L = blob_layout(MXFP4, N, K);
  // slices of FS x 16 features (N % (16 FS) == 0 for FS > 1); slice h of
  // the workgroup is half h % 2 of 32-row group g0 + h / 2
  const int64_t F = N / (16 * FS), per_x = (F + 7) / 8;
  const int64_t f = int64_t(blockIdx.x % 8) * per_x + blockIdx.x / 8;
  if (f >= F) return;
  const int64_t g0 = FS == 1 ? f >> 1 : f * (FS / 2);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, c = lane >> 4;
  const int64_t KT = L.KT, KS = L.KS, K2 = K / 2, KB = K / 32;
  const u32x4* __restrict__ W[FS];
  const uint32_t* __restrict__ S[FS];
  int sw_shift[FS];
#pragma unroll
  for (int h = 0; h < FS; ++h) {
    const int64_t g = g0 + h / 2;
    const int tl = 32 * (c & 1) + 16 * (FS == 1 ? int(f & 1) : h % 2) + r;
    W[h] = reinterpret_cast<const u32x4*>(blob + L.code_off) + (g * KT + (c >> 1)) * 64 + tl;
    S[h] = reinterpret_cast<const uint32_t*>(blob + L.scale_off) + ((g >> 2) * KT + (c >> 1)) * 64 + tl;
    sw_shift[h] = 8 * int(g & 3);
  }
  const bool mvalid = r < M;
  // activation loads: lane l takes row l / 4, chunk l % 4 (only the lanes of
  // rows < M load); fragment lane l then reads it from lane 4 (l % 16) + l / 16
  const int lr = lane >> 2;
  const bool lvalid = lr < M;
  const uint8_t* __restrict__ arow = a_codes + (lvalid ? lr : 0) * K2 + 16 * (lane & 3);
  const int perm = 4 * (4 * r + c);
  const uint8_t* __restrict__ srow = a_scales + (mvalid ? r : 0) * KB + c;
  const int64_t per = (KS + WAVES - 1) / WAVES;
  const int64_t s_begin = wave * per;
  const int64_t s_end = s_begin + per < KS ? s_begin + per : KS;

  v4f acc[FS];
#pragma unroll
  for (int h = 0; h < FS; ++h) acc[h] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int64_t s0 = s_begin; s0 < s_end; s0 += U) {
    u32x4 wf[U][FS], af[U];
    uint32_t swd[U][FS];
    int sab[U];
    int sdw[SD ? U / 4 : 1];
    if constexpr (SD) {
#pragma unroll
      for (int j = 0; j < U / 4; ++j) {
        const int64_t s = s0 + 4 * j + c;
        const int64_t sc = s < s_end ? s : s_end - 1;  // clamped: loads stay in range
        sdw[j] = *reinterpret_cast<const int*>(srow - c + sc * 4);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t s = s0 + u;
      const bool ok = s < s_end;
      const int64_t sc = ok ? s : s_end - 1;  // clamped: loads stay in range
#pragma unroll
      for (int h = 0; h < FS; ++h) {
        wf[u][h] = __builtin_nontemporal_load(&W[h][sc * 128]);
        swd[u][h] = __builtin_nontemporal_load(&S[h][sc * 128]);
      }
      u32x4 a = {0u, 0u, 0u, 0u};
      if (lvalid) a = *reinterpret_cast<const u32x4*>(arow + sc * 64);
      af[u] = ok ? a : u32x4{0u, 0u, 0u, 0u};
      if constexpr (!SD) sab[u] = mvalid ? int(srow[sc * 4]) : 127;
    }
    if constexpr (SD) {
      // byte c of the dword lane (r, u % 4) loaded for K-step s0 + u
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int d = __builtin_amdgcn_ds_bpermute(4 * (r + 16 * (u & 3)), sdw[u >> 2]);
        sab[u] = mvalid ? int((uint32_t(d) >> (8 * c)) & 0xffu) : 127;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      u32x4 a;
      a.x = uint32_t(__builtin_amdgcn_ds_bpermute(perm, int(af[u].x)));
      a.y = uint32_t(__builtin_amdgcn_ds_bpermute(perm, int(af[u].y)));
      a.z = uint32_t(__builtin_amdgcn_ds_bpermute(perm, int(af[u].z)));
      a.w = uint32_t(__builtin_amdgcn_ds_bpermute(perm, int(af[u].w)));
#pragma unroll
      for (int h = 0; h < FS; ++h)
        acc[h] = mfma_fp4_op<0>(wf[u][h], a, acc[h], int(swd[u][h] >> sw_shift[h]), sab[u]);
    }
  }

  __shared__ v4f red[WAVES > 1 ? WAVES - 1 : 1][FS][64];
  if (wave != 0) {
#pragma unroll
    for (int h = 0; h < FS; ++h) red[wave - 1][h][lane] = acc[h];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < WAVES - 1; ++w)
#pragma unroll
    for (int h = 0; h < FS; ++h) {
      const v4f o = red[w][h][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[h][e] += o[e];
    }
  // lane l: activation row l % 16, features 4 (l / 16) + 0..3 of a 16-slice
  if (!mvalid) return;
#pragma unroll
  for (int h = 0; h < FS; ++h) {
    const int64_t n = (FS * f + h) * 16 + 4 * c;
    const float4 rv = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(blob + L.r_off) + n);
    store4(Y, N, r, n, acc[h], v4f{rv.x, rv.y, rv.z, rv.w});
  }
}

template <int WAVES, int U = 8, int FS = 1, bool SD = false>
hipError_t launch_fp4_decode16(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                               const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_fp4_decode16_kernel<WAVES, U, FS, SD>), dim3(unsigned((N / (16 * FS) + 7) / 8 * 8)),
                     dim3(64 * WAVES), 0, stream, ac, as, blob, Y, M, N, K);
  return hipGetLastError();
}

// ====================================================== decode kernel ==
//
// M <= 16, MXINT4: weight streaming.  One workgroup per 16 output features
// (one 16-row weight group); workgroup b takes group (b % 8) S + b / 8 (S
// groups per XCD), so neighbouring groups, which share scale words, run on
// one XCD at about the same time.  The WAVES waves split K into contiguous
// ranges of 128-wide K-steps and each issues the loads of up to U K-steps at
// once (the weight tiles straight from HBM into registers, one coalesced
// 16-byte load per lane per K-step, non-temporal: the stream is read once),
// then their MFMAs.  The activation rows (<= 16) are the MFMA's second
// operand; rows >= M are zero.  Partial sums of the waves are added through
// LDS and wave 0 runs the epilogue.
//
// Codes enter the FP8 MFMA biased by 8 (u = q + 8, one XOR and a nibble
// split instead of the sign-magnitude table), and the product is expanded as
// (u - 8)(v - 8) = u v - 8 v - 8 u + 64: four MFMAs per K-step instead of one
// but a third of the VALU work, which here bounds the rate.  Every product is
// exact; the fp32 accumulator rounds partial sums up to ~(15 * 15 * 128) per
// K-step and block-scale unit where the direct form rounds ~(8 * 8 * 128),
// well inside the output tolerance, and with equal block scales all partial
// sums are integers below 2^24 units, so the result is the same exact value.
template <int FMT, int WAVES, int U>
__global__ __launch_bounds__(64 * WAVES) void gemm_decode_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K) {
  if (!blob_header_ok(blob, FMT, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  const BlobLayout L = blob_layout(FMT, N, K);
  const u32x4* __restrict__ Wc = reinterpret_cast<const u32x4*>(blob + L.code_off);
  const uint32_t* __restrict__ Ws = reinterpret_cast<const uint32_t*>(blob + L.scale_off);
  const float* __restrict__ R = reinterpret_cast<const float*>(blob + L.r_off);

  const int64_t F = N / 16, per_x = (F + 7) / 8;
  const int64_t ng = int64_t(blockIdx.x % 8) * per_x + blockIdx.x / 8;
  if (ng >= F) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane >> 4;
  const int64_t m = lane & 15;
  const bool mvalid = m < M;
  const int64_t KS = L.KS, K2 = K / 2, KB = K / 32;
  const int64_t per = (KS + WAVES - 1) / WAVES;
  const int64_t k_begin = wave * per;
  const int64_t k_end = k_begin + per < KS ? k_begin + per : KS;
  const int sw_shift = 8 * int(ng & 3);
  const uint32_t* __restrict__ Wsg = Ws + (ng >> 2) * KS * 64 + lane;
  const u32x4* __restrict__ Wg = Wc + ng * KS * 64 + lane;
  // activation codes: lane l loads row l / 4, 16-byte chunk l % 4 of the
  // K-step; fragment lane l (row m = l % 16, group c = l / 16) takes half
  // c % 2 of chunks c / 2 and 2 + c / 2 of row m (see load_act_frag) from
  // lanes 4 m + c / 2 and 4 m + 2 + c / 2.  Lanes of rows >= M take zeros:
  // only the lanes of rows < M load (exec mask).  Batches stay at <= 8
  // K-steps: around longer batches that branch made the compiler drain the
  // whole batch at its join.
  static_assert(FMT == MXINT4, "activation fragment layout");
  static_assert(U <= 8, "masked activation loads");
  const int lr = lane >> 2;
  const bool lvalid = lr < M;
  const uint8_t* __restrict__ arow = a_codes + (lvalid ? lr : 0) * K2 + 16 * (lane & 3);
  const uint8_t* __restrict__ srow = a_scales + (mvalid ? m : 0) * KB + c;
  const int src_lo = 4 * (4 * int(m) + (c >> 1)), src_hi = src_lo + 8;
  const bool odd = c & 1;

  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = k_begin; k0 < k_end; k0 += U) {
    u32x4 wf[U], af[U];
    uint32_t swd[U];
    int sab[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t ks = k0 + u;
      const bool ok = ks < k_end;
      const int64_t ksc = ok ? ks : k_end - 1;  // clamped: loads stay in range
      const u32x4 w = __builtin_nontemporal_load(&Wg[ksc * 64]);
      u32x4 a = {0u, 0u, 0u, 0u};
      if (lvalid) a = *reinterpret_cast<const u32x4*>(arow + ksc * 64);
      sab[u] = mvalid ? int(srow[ksc * 4]) : 127;
      wf[u] = ok ? w : u32x4{0u, 0u, 0u, 0u};
      af[u] = ok ? a : u32x4{0u, 0u, 0u, 0u};
      swd[u] = __builtin_nontemporal_load(&Wsg[ksc * 64]) >> sw_shift;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // the halves of the two chunks this fragment lane takes
      const uint32_t l0 = uint32_t(__builtin_amdgcn_ds_bpermute(src_lo, int(af[u].x)));
      const uint32_t l1 = uint32_t(__builtin_amdgcn_ds_bpermute(src_lo, int(af[u].y)));
      const uint32_t l2 = uint32_t(__builtin_amdgcn_ds_bpermute(src_lo, int(af[u].z)));
      const uint32_t l3 = uint32_t(__builtin_amdgcn_ds_bpermute(src_lo, int(af[u].w)));
      const uint32_t h0 = uint32_t(__builtin_amdgcn_ds_bpermute(src_hi, int(af[u].x)));
      const uint32_t h1 = uint32_t(__builtin_amdgcn_ds_bpermute(src_hi, int(af[u].y)));
      const uint32_t h2 = uint32_t(__builtin_amdgcn_ds_bpermute(src_hi, int(af[u].z)));
      const uint32_t h3 = uint32_t(__builtin_amdgcn_ds_bpermute(src_hi, int(af[u].w)));
      const u32x4 a = odd ? u32x4{l2, l3, h2, h3} : u32x4{l0, l1, h0, h1};
      const int sw = int(swd[u]), sa = sab[u];
      // q_w q_a = (u - 8)(v - 8) = u v - 8 v - 8 u + 64 with the biased codes
      // u, v: four MFMAs into the same accumulator under the same block
      // scales, two of them against the constant -8 (E4M3 0x88 = -8 * 2^-9)
      const v8i m8 = {-0x77777778, -0x77777778, -0x77777778, -0x77777778,
                      -0x77777778, -0x77777778, -0x77777778, -0x77777778};
      const v8i wu = int4_frag_biased_fp8(wf[u]), av = int4_frag_biased_fp8(a);
      acc = mfma_fp8_op<0>(m8, av, acc, sw, sa);
      acc = mfma_fp8_op<0>(wu, av, acc, sw, sa);
      acc = mfma_fp8_op<0>(wu, m8, acc, sw, sa);
      acc = mfma_fp8_op<0>(m8, m8, acc, sw, sa);
    }
  }

  __shared__ v4f red[WAVES > 1 ? WAVES - 1 : 1][64];
  if (wave != 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < WAVES - 1; ++w) {
    const v4f o = red[w][lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += o[e];
  }
  const float f = epilogue_factor(FMT, nullptr, blob);
  const float4 r = *reinterpret_cast<const float4*>(R + ng * 16 + 4 * c);
  if (mvalid) store4(Y, N, m, ng * 16 + 4 * c, acc, v4f{r.x * f, r.y * f, r.z * f, r.w * f});
}

template <int FMT, int WAVES, int U>
hipError_t launch_decode(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                         const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_decode_kernel<FMT, WAVES, U>), dim3(unsigned((N / 16 + 7) / 8 * 8)), dim3(64 * WAVES), 0,
                     stream, ac, as, blob, Y, M, N, K);
  return hipGetLastError();
}

// ============================================= MXINT4 dot decode kernel ==
//
// M = 1, MXINT4: the workgroups, waves and K-step batches of the decode
// kernel above, but with one activation row the MFMA's 16 columns would be
// 15/16 empty; the block sums are integer dot products on the VALU
// (v_dot8_i32_i4: 8 signed int4 products per lane per instruction) and
// nothing is widened.  The workgroup first copies the activation row's codes
// and scale bytes into LDS (K/2 + K/32 bytes; the first batch of weight loads
// is issued before).  Lane (n = l % 16, c = l / 16) holds the weight tile's
// 16 bytes: half (c & 1) of block c >> 1 in bytes 0..7 and the same half of
// block 2 + (c >> 1) in bytes 8..15, canonical nibble order (see pack.hip);
// it reads the same two 8-byte pieces of the activation row from LDS, and
// those two blocks' weight scales from the scale words of lanes n + 16 (c >>
// 1) and n + 16 (2 + (c >> 1)) by lane permutation.  Each half's integer
// sum (16 products) is exact and joins the lane's fp32 sum times
// 2^(e_w + e_a - 254), exact; a 0xFF (NaN) scale gives NaN.  The four lanes
// of a feature are added by two lane exchanges and the waves in wave order
// through LDS.
__device__ __forceinline__ float mx_pair_factor(uint32_t ew, uint32_t ea) {
  return (ew == 0xFFu || ea == 0xFFu) ? __builtin_nanf("") : ldexpf(1.0f, int(ew + ea) - 254);
}

template <int WAVES, int U>
__global__ __launch_bounds__(64 * WAVES) void gemm_mxint4_dot_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K) {
  if (!blob_header_ok(blob, MXINT4, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  const BlobLayout L = blob_layout(MXINT4, N, K);
  const u32x4* __restrict__ Wc = reinterpret_cast<const u32x4*>(blob + L.code_off);
  const uint32_t* __restrict__ Ws = reinterpret_cast<const uint32_t*>(blob + L.scale_off);
  const float* __restrict__ R = reinterpret_cast<const float*>(blob + L.r_off);

  const int64_t F = N / 16, per_x = (F + 7) / 8;
  const int64_t ng = int64_t(blockIdx.x % 8) * per_x + blockIdx.x / 8;
  if (ng >= F) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane >> 4, n = lane & 15, half = c >> 1;
  const int64_t KS = L.KS, K2 = K / 2;
  const int64_t per = (KS + WAVES - 1) / WAVES;
  const int64_t k_begin = wave * per;
  const int64_t k_end = k_begin + per < KS ? k_begin + per : KS;
  const int sw_shift = 8 * int(ng & 3);
  const u32x4* __restrict__ Wg = Wc + ng * KS * 64 + lane;
  const uint32_t* __restrict__ Wsg = Ws + (ng >> 2) * KS * 64 + lane;
  const int src_lo = 4 * (n + 16 * half), src_hi = src_lo + 128;
  const int off = 16 * half + 8 * (c & 1);

  u32x4 wf[U];
  uint32_t wsw[U];
  auto load_batch = [&](int64_t kb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      wf[u] = __builtin_nontemporal_load(&Wg[(kb + u) * 64]);
      wsw[u] = __builtin_nontemporal_load(&Wsg[(kb + u) * 64]);
    }
  };
  if (k_begin + U <= k_end) load_batch(k_begin);

  // the activation row: codes (K/2 bytes) then scale bytes (K/32), copied
  extern __shared__ __attribute__((aligned(16))) uint8_t mx_dyn[];
  for (int64_t d = tid; d < K2 / 16; d += 64 * WAVES)
    reinterpret_cast<u32x4*>(mx_dyn)[d] = reinterpret_cast<const u32x4*>(a_codes)[d];
  for (int64_t d = tid; d < K / 128; d += 64 * WAVES)
    reinterpret_cast<uint32_t*>(mx_dyn + K2)[d] = reinterpret_cast<const uint32_t*>(a_scales)[d];
  __syncthreads();
  const uint8_t* act = mx_dyn;
  const uint32_t* asc = reinterpret_cast<const uint32_t*>(mx_dyn + K2);

  float acc = 0.f;
  auto step = [&](const u32x4& w, uint32_t sw_own, int64_t ks) {
    const uint32_t wl = uint32_t(__builtin_amdgcn_ds_bpermute(src_lo, int(sw_own)));
    const uint32_t wh = uint32_t(__builtin_amdgcn_ds_bpermute(src_hi, int(sw_own)));
    const u32x2 alo = *reinterpret_cast<const u32x2*>(act + ks * 64 + off);
    const u32x2 ahi = *reinterpret_cast<const u32x2*>(act + ks * 64 + 32 + off);
    const uint32_t asw = asc[ks];
    int dl = __builtin_amdgcn_sdot8(int(w.x), int(alo.x), 0, false);
    dl = __builtin_amdgcn_sdot8(int(w.y), int(alo.y), dl, false);
    int dh = __builtin_amdgcn_sdot8(int(w.z), int(ahi.x), 0, false);
    dh = __builtin_amdgcn_sdot8(int(w.w), int(ahi.y), dh, false);
    acc = fmaf(float(dl), mx_pair_factor((wl >> sw_shift) & 0xFFu, (asw >> (8 * half)) & 0xFFu), acc);
    acc = fmaf(float(dh), mx_pair_factor((wh >> sw_shift) & 0xFFu, (asw >> (8 * (2 + half))) & 0xFFu), acc);
  };
  int64_t k0 = k_begin;
  for (; k0 + U <= k_end; k0 += U) {
    if (k0 != k_begin) load_batch(k0);
#pragma unroll
    for (int u = 0; u < U; ++u) step(wf[u], wsw[u], k0 + u);
  }
  for (; k0 < k_end; ++k0) step(Wg[k0 * 64], Wsg[k0 * 64], k0);

  // the feature's four lanes (c = 0..3): (c0 + c1) + (c2 + c3) in every lane
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  __shared__ float red[WAVES > 1 ? WAVES - 1 : 1][16];
  if (wave != 0 && c == 0) red[wave - 1][n] = acc;
  __syncthreads();
  if (wave != 0 || c != 0) return;
  float y = acc;
#pragma unroll
  for (int w = 0; w < WAVES - 1; ++w) y += red[w][n];
  const uint32_t u = __float_as_uint(y * R[ng * 16 + n]);
  Y[ng * 16 + n] = uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <int WAVES, int U>
hipError_t launch_mxint4_dot(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                             const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  const size_t lds = size_t(K) / 2 + size_t(K) / 32;
  hipLaunchKernelGGL((gemm_mxint4_dot_kernel<WAVES, U>), dim3(unsigned((N / 16 + 7) / 8 * 8)), dim3(64 * WAVES),
                     lds, stream, ac, as, blob, Y, M, N, K);
  return hipGetLastError();
}

// ================================================= NVFP4 decode kernel ==
//
// M <= 16, NVFP4: weight streaming like the MXINT4 decode kernel (one
// workgroup per 16 output features, groups per XCD, the WAVES waves splitting
// K into contiguous ranges of K-steps loaded U at a time, weights
// non-temporal), on the 16x16x32 fp16 MFMA.  Both operands' lanes hold the
// same K positions, so no permutation is needed: lane (m = l % 16, c = l / 16)
// of the weight tile holds the 32 codes of K-chunk c (blocks 2c and 2c + 1)
// of row m, and the activation lane loads the same 16 bytes of row m with its
// two block-scale bytes.  Each 32-wide part is expanded exactly into fp16
// (code times E4M3 scale) on both sides; t_a t_w and r come in the epilogue.
template <int WAVES, int U>
__global__ __launch_bounds__(64 * WAVES) void gemm_nv_decode_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ t_act, const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y,
    int64_t M, int64_t N, int64_t K) {
  if (!blob_header_ok(blob, NVFP4, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  const BlobLayout L = blob_layout(NVFP4, N, K);
  const u32x4* __restrict__ Wc = reinterpret_cast<const u32x4*>(blob + L.code_off);
  const uint32_t* __restrict__ Ws = reinterpret_cast<const uint32_t*>(blob + L.scale_off);
  const float* __restrict__ R = reinterpret_cast<const float*>(blob + L.r_off);

  const int64_t F = N / 16, per_x = (F + 7) / 8;
  const int64_t ng = int64_t(blockIdx.x % 8) * per_x + blockIdx.x / 8;
  if (ng >= F) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane >> 4;
  const int64_t m = lane & 15;
  const bool mvalid = m < M;
  const int64_t KS = L.KS, K2 = K / 2, KB = K / 16;
  const int64_t per = (KS + WAVES - 1) / WAVES;
  const int64_t k_begin = wave * per;
  const int64_t k_end = k_begin + per < KS ? k_begin + per : KS;
  // scale word: bytes 2 (ng % 2) and 2 (ng % 2) + 1 hold blocks 2c and 2c + 1
  const int sw_shift = 16 * int(ng & 1);
  const uint32_t* __restrict__ Wsg = Ws + (ng >> 1) * KS * 64 + lane;
  const u32x4* __restrict__ Wg = Wc + ng * KS * 64 + lane;
  const uint8_t* __restrict__ arow = a_codes + (mvalid ? m : 0) * K2 + 16 * c;
  const uint8_t* __restrict__ srow = a_scales + (mvalid ? m : 0) * KB + 2 * c;
  static_assert(U <= 8, "masked activation loads");

  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = k_begin; k0 < k_end; k0 += U) {
    u32x4 wf[U], af[U];
    uint32_t swd[U], sad[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t ks = k0 + u;
      const bool ok = ks < k_end;
      const int64_t ksc = ok ? ks : k_end - 1;  // clamped: loads stay in range
      const u32x4 w = __builtin_nontemporal_load(&Wg[ksc * 64]);
      u32x4 a = {0u, 0u, 0u, 0u};
      uint32_t sa = 0;
      if (mvalid) {
        a = *reinterpret_cast<const u32x4*>(arow + ksc * 64);
        sa = *reinterpret_cast<const uint16_t*>(srow + ksc * 8);
      }
      wf[u] = ok ? w : u32x4{0u, 0u, 0u, 0u};
      af[u] = ok ? a : u32x4{0u, 0u, 0u, 0u};
      swd[u] = __builtin_nontemporal_load(&Wsg[ksc * 64]) >> sw_shift;
      sad[u] = sa;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const v8h wh = e2m1x8_scaled_f16(wf[u][jj], (swd[u] >> (8 * (jj >> 1))) & 0xffu);
        const v8h ah = e2m1x8_scaled_f16(af[u][jj], (sad[u] >> (8 * (jj >> 1))) & 0xffu);
        acc = mfma_f16(wh, ah, acc);
      }
    }
  }

  __shared__ v4f red[WAVES > 1 ? WAVES - 1 : 1][64];
  if (wave != 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < WAVES - 1; ++w) {
    const v4f o = red[w][lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += o[e];
  }
  const float f = epilogue_factor(NVFP4, t_act, blob);
  const float4 r = *reinterpret_cast<const float4*>(R + ng * 16 + 4 * c);
  if (mvalid) store4(Y, N, m, ng * 16 + 4 * c, acc, v4f{r.x * f, r.y * f, r.z * f, r.w * f});
}

template <int WAVES, int U>
hipError_t launch_nv_decode(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                            const float* t_act, const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_nv_decode_kernel<WAVES, U>), dim3(unsigned((N / 16 + 7) / 8 * 8)), dim3(64 * WAVES),
                     0, stream, ac, as, t_act, blob, Y, M, N, K);
  return hipGetLastError();
}

// =============================================== NVFP4 dot decode kernel ==
//
// M = 1, NVFP4: the workgroups, waves and K-step batches of the decode
// kernel above, but with one activation row 15 of the MFMA's 16 columns
// would be empty while every lane still expands its activation fragment.
// Here the workgroup first expands its activation row(s) (MD) once into
// LDS as exact fp16 (code times E4M3 scale, as e2m1x8_scaled_f16 does), and
// the products run on the VALU as fp16 dot products (v_dot2_f32_f16) with the
// weight codes converted under the power of two of their block scale alone
// (v_cvt_scalef32_pk_f16_fp4, exact); each 16-code block's fp32 partial sum
// is then multiplied by the scale's remaining mantissa factor (1 + f/8).
// Lane (n = l % 16, c = l / 16) holds the weight tile's 32 codes of K-chunk c
// (blocks 2c, 2c + 1) of feature 16 g + n; the activation pairs of the same
// codes come from LDS in the conversion's own order (both sides use the same
// instruction on canonical bytes), so every product pairs equal K.  The four
// lanes of a feature are added by two lane exchanges and the waves in wave
// order through LDS.
template <int WAVES, int U, int MD>
__global__ __launch_bounds__(64 * WAVES) void gemm_nv_dot_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ t_act, const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y,
    int64_t M, int64_t N, int64_t K) {
  if (!blob_header_ok(blob, NVFP4, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  const BlobLayout L = blob_layout(NVFP4, N, K);
  const u32x4* __restrict__ Wc = reinterpret_cast<const u32x4*>(blob + L.code_off);
  const uint32_t* __restrict__ Ws = reinterpret_cast<const uint32_t*>(blob + L.scale_off);
  const float* __restrict__ R = reinterpret_cast<const float*>(blob + L.r_off);

  const int64_t F = N / 16, per_x = (F + 7) / 8;
  const int64_t ng = int64_t(blockIdx.x % 8) * per_x + blockIdx.x / 8;
  if (ng >= F) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane >> 4, n = lane & 15;
  const int64_t KS = L.KS, K2 = K / 2, KB = K / 16;
  const int64_t per = (KS + WAVES - 1) / WAVES;
  const int64_t k_begin = wave * per;
  const int64_t k_end = k_begin + per < KS ? k_begin + per : KS;
  const int sw_shift = 16 * int(ng & 1);
  const uint32_t* __restrict__ Wsg = Ws + (ng >> 1) * KS * 64 + lane;
  const u32x4* __restrict__ Wg = Wc + ng * KS * 64 + lane;

  // the first batch of weight loads goes out before the activation rows are
  // staged, so the staging's latency overlaps them
  u32x4 wf[U];
  uint32_t swd[U];
  auto load_batch = [&](int64_t kb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      wf[u] = __builtin_nontemporal_load(&Wg[(kb + u) * 64]);
      swd[u] = __builtin_nontemporal_load(&Wsg[(kb + u) * 64]) >> sw_shift;
    }
  };
  if (k_begin + U <= k_end) load_batch(k_begin);

  // activation rows, expanded: pair p of row m = the two codes of byte p
  extern __shared__ __attribute__((aligned(16))) uint8_t nv_dyn[];
  h2* act = reinterpret_cast<h2*>(nv_dyn);
  const int64_t rowd = K / 8;  // code dwords per row
  for (int64_t d = tid; d < MD * rowd; d += 64 * WAVES) {
    const int64_t m = d / rowd, kd = d - m * rowd;
    const uint32_t code = reinterpret_cast<const uint32_t*>(a_codes + m * K2)[kd];
    const v8h v = e2m1x8_scaled_f16(code, a_scales[m * KB + kd / 2]);
    *reinterpret_cast<v8h*>(act + m * K2 + 4 * kd) = v;
  }
  __syncthreads();

  float acc[MD];
#pragma unroll
  for (int m = 0; m < MD; ++m) acc[m] = 0.f;
  auto step = [&](const u32x4& w, uint32_t swd, int64_t ks) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float sv = __builtin_amdgcn_cvt_f32_fp8(int((swd >> (8 * b)) & 0xffu), 0);
      const float p2 = __uint_as_float(__float_as_uint(sv) & 0xff800000u);
      const float fr = __uint_as_float((__float_as_uint(sv) & 0x007fffffu) | 0x3f800000u);
      h2 wv[8];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t d = w[2 * b + q];
        wv[4 * q + 0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, p2, 0);
        wv[4 * q + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, p2, 1);
        wv[4 * q + 2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, p2, 2);
        wv[4 * q + 3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, p2, 3);
      }
#pragma unroll
      for (int m = 0; m < MD; ++m) {
        // the 16 codes of block 2c + b: bytes 8b .. 8b + 7 of the lane's 16
        const h2* ap = act + m * K2 + ks * 64 + 16 * c + 8 * b;
        const v8h a0 = *reinterpret_cast<const v8h*>(ap);
        const v8h a1 = *reinterpret_cast<const v8h*>(ap + 4);
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) part = __builtin_amdgcn_fdot2(wv[i], h2{a0[2 * i], a0[2 * i + 1]}, part, false);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          part = __builtin_amdgcn_fdot2(wv[4 + i], h2{a1[2 * i], a1[2 * i + 1]}, part, false);
        acc[m] = fmaf(part, fr, acc[m]);
      }
    }
  };
  int64_t k0 = k_begin;
  for (; k0 + U <= k_end; k0 += U) {
    if (k0 != k_begin) load_batch(k0);
#pragma unroll
    for (int u = 0; u < U; ++u) step(wf[u], swd[u], k0 + u);
  }
  for (; k0 < k_end; ++k0) step(Wg[k0 * 64], Wsg[k0 * 64] >> sw_shift, k0);

  // the feature's four lanes (c = 0..3): (c0 + c1) + (c2 + c3) in every lane
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
  const float rf = R[ng * 16 + n] * epilogue_factor(NVFP4, t_act, blob);
#pragma unroll
  for (int m = 0; m < MD; ++m) {
    float y = acc[m];
#pragma unroll
    for (int w = 0; w < WAVES - 1; ++w) y += red[w][m][n];
    const uint32_t u = __float_as_uint(y * rf);
    Y[int64_t(m) * N + ng * 16 + n] = uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
  }
}

template <int WAVES, int U>
hipError_t launch_nv_dot(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                         const float* t_act, const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  const dim3 grid(unsigned((N / 16 + 7) / 8 * 8)), block(64 * WAVES);
  const size_t lds = size_t(M) * size_t(K) * 2;  // M = 1: at most 64 KiB
  hipLaunchKernelGGL((gemm_nv_dot_kernel<WAVES, U, 1>), grid, block, lds, stream, ac, as, t_act, blob, Y, M, N, K);
  return hipGetLastError();
}

// ================================================ 8-bit MX (MXFP8, MXINT8) ==
//
// Codes are one byte each.  A fragment lane l (row r = l % 16, group c =
// l / 16) holds 32 bytes of its row for a 128-wide K-step: K 16c..16c+15 in
// its first four dwords and 64+16c..64+16c+15 in the last four, the FP8
// operand order of V_MFMA_SCALE_F32_16X16X128_F8F6F4 (so the first half
// lies in block c/2 and the second in block 2 + c/2).
//   MXFP8 : the scaled FP8 MFMA does not add the 32 products of a block
//           exactly when their magnitudes spread: measured, a product 2^-6
//           next to 448 x 1 in the same group of eight is dropped (about 14
//           bits kept below the group's largest product), and E4M3 products
//           span 36 binades.  So each code is expanded with its block scale
//           into bf16 (v_cvt_scalef32_pk_bf16_fp8: code x 2^e has 4
//           significant bits, exact), and the bf16 MFMA (16x16x32, products
//           kept to ~26 bits, measured) runs four times per K-step, MFMA j
//           taking elements 8j..8j+7 of every lane on both operands (the same
//           K permutation on both sides, each element already carrying its
//           block scale).
//   MXINT8: q = 16 h + l with h = q >> 4 in [-8, 7] and l = q & 15.  h enters
//           as the E4M3 byte of h * 2^-5 and l as that of l * 2^-9 (bytes
//           0..15 encode u * 2^-9 exactly), so q * 2^-9 = h 2^-5 + l 2^-9 and
//           q_w q_a 2^-18 is the sum of four exact MFMA products under the
//           same block scales; the epilogue multiplies by 2^18.

// four int8 codes (the bytes of d) -> E4M3 bytes of (q >> 4) * 2^-5.  The low
// three bits of the high nibble index a table of positive and one of negative
// values; bit 7 of each byte picks, per byte, which.
__device__ __forceinline__ uint32_t int8x4_hi_e4m3(uint32_t d) {
  const uint32_t pos_lo = vgpr_const(0x1C181000u);  // h = 0..3
  const uint32_t pos_hi = vgpr_const(0x26242220u);  // h = 4..7
  const uint32_t neg_lo = vgpr_const(0xA2A4A6A8u);  // h = -8..-5
  const uint32_t neg_hi = vgpr_const(0x90989CA0u);  // h = -4..-1
  const uint32_t g = (d >> 4) & vgpr_const(0x07070707u);
  const uint32_t pos = __builtin_amdgcn_perm(pos_hi, pos_lo, g);
  const uint32_t neg = __builtin_amdgcn_perm(neg_hi, neg_lo, g);
  const uint32_t sel = ((d >> 5) & vgpr_const(0x04040404u)) | vgpr_const(0x03020100u);
  return __builtin_amdgcn_perm(neg, pos, sel);
}

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// E8M0 byte -> the fp32 scale 2^(b - 127) (only its exponent is used by the
// conversion)
__device__ __forceinline__ float e8m0_scale(uint32_t b) { return __uint_as_float((b & 0xffu) << 23); }

// 32 E4M3 codes of a fragment lane, the first 16 under scale s0 and the last
// 16 under s1, as four groups of 8 bf16 values (exact)
struct Bf16Frag {
  v8bf p[4];
};

__device__ __forceinline__ Bf16Frag e4m3_frag_bf16(const v8i& f, float s0, float s1) {
  Bf16Frag o;
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const float sc = d < 4 ? s0 : s1;
    const bf2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(uint32_t(f[d]), sc, false);
    const bf2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(uint32_t(f[d]), sc, true);
    o.p[d >> 1][4 * (d & 1) + 0] = lo[0];
    o.p[d >> 1][4 * (d & 1) + 1] = lo[1];
    o.p[d >> 1][4 * (d & 1) + 2] = hi[0];
    o.p[d >> 1][4 * (d & 1) + 3] = hi[1];
  }
  return o;
}

__device__ __forceinline__ v4f mfma_bf16x4(const Bf16Frag& w, const Bf16Frag& a, v4f acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w.p[j], a.p[j], acc, 0, 0, 0);
  return acc;
}

struct Mx8Split {
  v8i hi, lo;
};

__device__ __forceinline__ Mx8Split int8_frag_split(const v8i& f) {
  Mx8Split s;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s.hi[i] = int(int8x4_hi_e4m3(uint32_t(f[i])));
    s.lo[i] = int(uint32_t(f[i]) & 0x0f0f0f0fu);
  }
  return s;
}

// acc += w . a for one fragment pair (byte `OPW` of sw is the weight scale)
template <int FMT, int OPW>
__device__ __forceinline__ v4f mx8_mfma_op(const v8i& w, const Mx8Split& ws, const v8i& a,
                                           const Mx8Split& as, v4f acc, int sw, int sa) {
  if constexpr (FMT == MXFP8) {
    return mfma_fp8_op<OPW>(w, a, acc, sw, sa);
  } else {
    acc = mfma_fp8_op<OPW>(ws.hi, as.hi, acc, sw, sa);
    acc = mfma_fp8_op<OPW>(ws.hi, as.lo, acc, sw, sa);
    acc = mfma_fp8_op<OPW>(ws.lo, as.hi, acc, sw, sa);
    return mfma_fp8_op<OPW>(ws.lo, as.lo, acc, sw, sa);
  }
}

template <int FMT>
__device__ __forceinline__ v4f mx8_mfma(int opw, const v8i& w, const Mx8Split& ws, const v8i& a,
                                        const Mx8Split& as, v4f acc, int sw, int sa) {
  switch (opw & 3) {
    case 0: return mx8_mfma_op<FMT, 0>(w, ws, a, as, acc, sw, sa);
    case 1: return mx8_mfma_op<FMT, 1>(w, ws, a, as, acc, sw, sa);
    case 2: return mx8_mfma_op<FMT, 2>(w, ws, a, as, acc, sw, sa);
    default: return mx8_mfma_op<FMT, 3>(w, ws, a, as, acc, sw, sa);
  }
}

__device__ __forceinline__ v8i v8i_of(const u32x4& lo, const u32x4& hi) {
  return v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
}

__device__ __forceinline__ float mx8_epilogue_factor(int fmt) {
  return fmt == MXINT8 ? 262144.0f : 1.0f;  // undo 2^-9 on both operands (MXINT8)
}

// ---------------------------------------------------- 8-bit decode (M <= 16)
//
// Weight streaming, as the MXINT4 decode kernel: one workgroup per 16 output
// features, workgroup b taking group (b % 8) S + b / 8 (S groups per XCD),
// WAVES waves splitting the K-steps into contiguous ranges, each issuing the
// loads of up to U K-steps at once (the 2 KiB weight tile of a K-step with
// two coalesced 16-byte non-temporal loads per lane).  The activation rows
// (<= 16) are the MFMA's second operand: lane (m, c) loads its two 16-byte
// chunks of row m straight in fragment order (the four lanes of a row read
// 64 contiguous bytes per load); lanes of rows >= M load nothing and hold
// zeros.  Partial sums meet in LDS; wave 0 applies r and stores.
template <int FMT, int WAVES, int U>
__global__ __launch_bounds__(64 * WAVES) void gemm_mx8_decode_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K) {
  if (!blob_header_ok(blob, FMT, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  static_assert(FMT == MXFP8 || FMT == MXINT8, "8-bit MX formats");
  const BlobLayout L = blob_layout(FMT, N, K);
  const u32x4* __restrict__ Wc = reinterpret_cast<const u32x4*>(blob + L.code_off);
  const uint32_t* __restrict__ Ws = reinterpret_cast<const uint32_t*>(blob + L.scale_off);
  const float* __restrict__ R = reinterpret_cast<const float*>(blob + L.r_off);

  const int64_t F = N / 16, per_x = (F + 7) / 8;
  const int64_t ng = int64_t(blockIdx.x % 8) * per_x + blockIdx.x / 8;
  if (ng >= F) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane >> 4;
  const int64_t m = lane & 15;
  const bool mvalid = m < M;
  const int64_t KS = L.KS, KB = K / 32;
  const int64_t per = (KS + WAVES - 1) / WAVES;
  const int64_t k_begin = wave * per;
  const int64_t k_end = k_begin + per < KS ? k_begin + per : KS;
  const int sw_shift = 8 * int(ng & 3);
  const uint32_t* __restrict__ Wsg = Ws + (ng >> 2) * KS * 64 + lane;
  const u32x4* __restrict__ Wg = Wc + (ng * KS * 64 + lane) * 2;
  const uint8_t* __restrict__ arow = a_codes + (mvalid ? m : 0) * K + 16 * c;
  // MXINT8: this lane group's block scale (the MFMA's scale lane); MXFP8: the
  // scales of the two blocks this lane's halves lie in (c / 2 and 2 + c / 2)
  const int b0 = FMT == MXFP8 ? (c >> 1) : c;
  const uint8_t* __restrict__ srow = a_scales + (mvalid ? m : 0) * KB + b0;
  const uint32_t* __restrict__ Wsg0 = Wsg - lane + (lane & 15) + 16 * b0;  // lane group b0's word
  static_assert(U <= 8, "masked activation loads");

  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = k_begin; k0 < k_end; k0 += U) {
    u32x4 w0[U], w1[U], a0[U], a1[U];
    uint32_t swd[U], swd2[U];
    int sab[U], sab2[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t ks = k0 + u;
      const bool ok = ks < k_end;
      const int64_t ksc = ok ? ks : k_end - 1;  // clamped: loads stay in range
      const u32x4 x0 = __builtin_nontemporal_load(&Wg[ksc * 128]);
      const u32x4 x1 = __builtin_nontemporal_load(&Wg[ksc * 128 + 1]);
      u32x4 y0 = {0u, 0u, 0u, 0u}, y1 = {0u, 0u, 0u, 0u};
      if (mvalid) {
        y0 = *reinterpret_cast<const u32x4*>(arow + ksc * 128);
        y1 = *reinterpret_cast<const u32x4*>(arow + ksc * 128 + 64);
      }
      sab[u] = mvalid ? int(srow[ksc * 4]) : 127;
      w0[u] = ok ? x0 : u32x4{0u, 0u, 0u, 0u};
      w1[u] = ok ? x1 : u32x4{0u, 0u, 0u, 0u};
      a0[u] = ok ? y0 : u32x4{0u, 0u, 0u, 0u};
      a1[u] = ok ? y1 : u32x4{0u, 0u, 0u, 0u};
      swd[u] = __builtin_nontemporal_load(&Wsg0[ksc * 64]) >> sw_shift;
      if constexpr (FMT == MXFP8) {
        sab2[u] = mvalid ? int(srow[ksc * 4 + 2]) : 127;
        swd2[u] = __builtin_nontemporal_load(&Wsg0[ksc * 64 + 32]) >> sw_shift;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const v8i w = v8i_of(w0[u], w1[u]), a = v8i_of(a0[u], a1[u]);
      if constexpr (FMT == MXFP8) {
        const Bf16Frag wb = e4m3_frag_bf16(w, e8m0_scale(swd[u]), e8m0_scale(swd2[u]));
        const Bf16Frag ab = e4m3_frag_bf16(a, e8m0_scale(uint32_t(sab[u])), e8m0_scale(uint32_t(sab2[u])));
        acc = mfma_bf16x4(wb, ab, acc);
      } else {
        const Mx8Split ws = int8_frag_split(w), as = int8_frag_split(a);
        acc = mx8_mfma_op<FMT, 0>(w, ws, a, as, acc, int(swd[u]), sab[u]);
      }
    }
  }

  __shared__ v4f red[WAVES > 1 ? WAVES - 1 : 1][64];
  if (wave != 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < WAVES - 1; ++w) {
    const v4f o = red[w][lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += o[e];
  }
  // lane l: activation row l % 16, features 4 (l / 16) + 0..3 of the group
  if (!mvalid) return;
  const int64_t n = ng * 16 + 4 * c;
  const float f = mx8_epilogue_factor(FMT);
  const float4 rv = *reinterpret_cast<const float4*>(R + n);
  store4(Y, N, m, n, acc, v4f{rv.x * f, rv.y * f, rv.z * f, rv.w * f});
}

template <int FMT, int WAVES, int U>
hipError_t launch_mx8_decode(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                             const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_mx8_decode_kernel<FMT, WAVES, U>), dim3(unsigned((N / 16 + 7) / 8 * 8)),
                     dim3(64 * WAVES), 0, stream, ac, as, blob, Y, M, N, K);
  return hipGetLastError();
}

// M <= 3: the weight tile streamed as by gemm_mx8_decode_kernel, the sums on
// the VALU instead of the MFMA.  Lane (n = l % 16, c = l / 16) holds the
// tile's 32 bytes: K 16c .. +16 (in block c >> 1) and 64 + 16c .. +16 (in
// block 2 + (c >> 1)); the two blocks' weight scales come from the scale
// words of lanes n + 16 (c >> 1) and n + 16 (2 + (c >> 1)) by lane
// permutation.  The MD activation rows are copied once per workgroup into
// LDS, then their block scales:
//   MXINT8: the code bytes as they are; v_dot4_i32_i8 adds four products, so
//           each half's sum (16 products, |sum| < 2^19) is an exact integer;
//   MXFP8 : the codes expanded to fp16 (every E4M3 value is an fp16 value,
//           subnormals included); the weight codes expanded the same way and
//           v_dot2_f32_f16 adds two exact products into the fp32 sum.
// Each half's sum joins the fp32 sum of its row times 2^(e_w + e_a - 254)
// (NaN for a 0xFF scale).  The four lanes of a feature are added by two lane
// exchanges and the waves in wave order through LDS.
template <int FMT>
__host__ __device__ constexpr int64_t mx8_dot_row_bytes(int64_t K) {
  return (FMT == MXFP8 ? 2 * K : K) + K / 32;
}

template <int FMT, int WAVES, int U, int MD>
__global__ __launch_bounds__(64 * WAVES) void gemm_mx8_dot_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K) {
  static_assert(FMT == MXFP8 || FMT == MXINT8, "8-bit MX formats");
  if (!blob_header_ok(blob, FMT, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  const BlobLayout L = blob_layout(FMT, N, K);
  const u32x4* __restrict__ Wc = reinterpret_cast<const u32x4*>(blob + L.code_off);
  const uint32_t* __restrict__ Ws = reinterpret_cast<const uint32_t*>(blob + L.scale_off);
  const float* __restrict__ R = reinterpret_cast<const float*>(blob + L.r_off);

  const int64_t F = N / 16, per_x = (F + 7) / 8;
  const int64_t ng = int64_t(blockIdx.x % 8) * per_x + blockIdx.x / 8;
  if (ng >= F) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane >> 4, n = lane & 15, half = c >> 1;
  const int64_t KS = L.KS;
  const int64_t per = (KS + WAVES - 1) / WAVES;
  const int64_t k_begin = wave * per;
  const int64_t k_end = k_begin + per < KS ? k_begin + per : KS;
  const int sw_shift = 8 * int(ng & 3);
  const u32x4* __restrict__ Wg = Wc + (ng * KS * 64 + lane) * 2;   // the lane's two 16-byte halves
  const uint32_t* __restrict__ Wsg = Ws + (ng >> 2) * KS * 64 + lane;
  const int src_lo = 4 * (n + 16 * half), src_hi = src_lo + 128;

  // the first batch of weight loads goes out before the activation rows are
  // staged, so the staging's latency overlaps them
  u32x4 w0[U], w1[U];
  uint32_t wsw[U];
  auto load_batch = [&](int64_t kb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      w0[u] = __builtin_nontemporal_load(&Wg[(kb + u) * 128]);
      w1[u] = __builtin_nontemporal_load(&Wg[(kb + u) * 128 + 1]);
      wsw[u] = __builtin_nontemporal_load(&Wsg[(kb + u) * 64]);
    }
  };
  if (k_begin + U <= k_end) load_batch(k_begin);

  // LDS: MD rows of codes (MXINT8: K bytes each; MXFP8: K fp16 values), then
  // MD rows of K/32 scale bytes
  extern __shared__ __attribute__((aligned(16))) uint8_t mx8_dyn[];
  const int64_t code_row = FMT == MXFP8 ? 2 * K : K;
  for (int64_t d = tid; d < MD * (K / 16); d += 64 * WAVES) {
    const u32x4 v = reinterpret_cast<const u32x4*>(a_codes)[d];
    if constexpr (FMT == MXINT8) {
      reinterpret_cast<u32x4*>(mx8_dyn)[d] = v;
    } else {
      h2* dst = reinterpret_cast<h2*>(mx8_dyn) + 8 * d;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dst[2 * i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[i], 1.0f, false);
        dst[2 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[i], 1.0f, true);
      }
    }
  }
  for (int64_t d = tid; d < MD * (K / 128); d += 64 * WAVES)
    reinterpret_cast<uint32_t*>(mx8_dyn + MD * code_row)[d] = reinterpret_cast<const uint32_t*>(a_scales)[d];
  __syncthreads();
  const uint32_t* asc = reinterpret_cast<const uint32_t*>(mx8_dyn + MD * code_row);

  float acc[MD];
#pragma unroll
  for (int m = 0; m < MD; ++m) acc[m] = 0.f;
  auto step = [&](const u32x4& a_w, const u32x4& b_w, uint32_t sw_own, int64_t ks) {
    const uint32_t wl = uint32_t(__builtin_amdgcn_ds_bpermute(src_lo, int(sw_own)));
    const uint32_t wh = uint32_t(__builtin_amdgcn_ds_bpermute(src_hi, int(sw_own)));
    const uint32_t ewl = (wl >> sw_shift) & 0xFFu, ewh = (wh >> sw_shift) & 0xFFu;
    if constexpr (FMT == MXINT8) {
#pragma unroll
      for (int m = 0; m < MD; ++m) {
        const uint8_t* row = mx8_dyn + m * K + ks * 128 + 16 * c;
        const u32x4 alo = *reinterpret_cast<const u32x4*>(row);
        const u32x4 ahi = *reinterpret_cast<const u32x4*>(row + 64);
        const uint32_t asw = asc[m * (K / 128) + ks];
        int dl = 0, dh = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dl = __builtin_amdgcn_sdot4(int(a_w[i]), int(alo[i]), dl, false);
          dh = __builtin_amdgcn_sdot4(int(b_w[i]), int(ahi[i]), dh, false);
        }
        acc[m] = fmaf(float(dl), mx_pair_factor(ewl, (asw >> (8 * half)) & 0xFFu), acc[m]);
        acc[m] = fmaf(float(dh), mx_pair_factor(ewh, (asw >> (8 * (2 + half))) & 0xFFu), acc[m]);
      }
    } else {
      h2 wv[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wv[2 * i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a_w[i], 1.0f, false);
        wv[2 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a_w[i], 1.0f, true);
        wv[8 + 2 * i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b_w[i], 1.0f, false);
        wv[8 + 2 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b_w[i], 1.0f, true);
      }
#pragma unroll
      for (int m = 0; m < MD; ++m) {
        const h2* row = reinterpret_cast<const h2*>(mx8_dyn + m * code_row) + ks * 64 + 8 * c;
        const uint32_t asw = asc[m * (K / 128) + ks];
        float pl = 0.f, ph = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const v8h lo = *reinterpret_cast<const v8h*>(row + 4 * j);
          const v8h hi = *reinterpret_cast<const v8h*>(row + 32 + 4 * j);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pl = __builtin_amdgcn_fdot2(wv[4 * j + i], h2{lo[2 * i], lo[2 * i + 1]}, pl, false);
            ph = __builtin_amdgcn_fdot2(wv[8 + 4 * j + i], h2{hi[2 * i], hi[2 * i + 1]}, ph, false);
          }
        }
        acc[m] = fmaf(pl, mx_pair_factor(ewl, (asw >> (8 * half)) & 0xFFu), acc[m]);
        acc[m] = fmaf(ph, mx_pair_factor(ewh, (asw >> (8 * (2 + half))) & 0xFFu), acc[m]);
      }
    }
  };
  int64_t k0 = k_begin;
  for (; k0 + U <= k_end; k0 += U) {
    if (k0 != k_begin) load_batch(k0);
#pragma unroll
    for (int u = 0; u < U; ++u) step(w0[u], w1[u], wsw[u], k0 + u);
  }
  for (; k0 < k_end; ++k0) step(Wg[k0 * 128], Wg[k0 * 128 + 1], Wsg[k0 * 64], k0);

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
    const uint32_t u = __float_as_uint(y * rn);
    Y[int64_t(m) * N + ng * 16 + n] = uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
  }
}

// dynamic LDS the dot kernels may take (activation rows and their scales)
constexpr int64_t kMx8DotLds = 64 * 1024;

template <int FMT, int WAVES, int U, int MD>
hipError_t launch_mx8_dot_md(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                             const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  const size_t lds = size_t(MD * mx8_dot_row_bytes<FMT>(K));
  hipLaunchKernelGGL((gemm_mx8_dot_kernel<FMT, WAVES, U, MD>), dim3(unsigned((N / 16 + 7) / 8 * 8)),
                     dim3(64 * WAVES), lds, stream, ac, as, blob, Y, M, N, K);
  return hipGetLastError();
}

template <int FMT, int WAVES, int U>
hipError_t launch_mx8_dot(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                          const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  if (M == 1) return launch_mx8_dot_md<FMT, WAVES, U, 1>(M, N, K, ac, as, blob, Y, stream);
  if (M == 2) return launch_mx8_dot_md<FMT, WAVES, U, 2>(M, N, K, ac, as, blob, Y, stream);
  return launch_mx8_dot_md<FMT, WAVES, U, 3>(M, N, K, ac, as, blob, Y, stream);
}

// ------------------------------------------------------ 8-bit tiled (M > 16)
//
// Workgroup tile BN (n) x BM (m) with WN x WM waves; one 128-wide K-step per
// pipeline stage, DEPTH stages in a ring, copied global -> LDS with
// direct-to-LDS loads (16 bytes per lane, 1 KiB per instruction; every wave
// issues the same COPIES per stage, so a stage is complete for a wave when
// its vmcnt has dropped to COPIES x the stages issued after it, and a
// barrier makes it complete for the workgroup).
//
// Stage layout:
//   A codes   BM rows x 128 B; 16-byte chunk j of row r at chunk position
//             8 r + (j ^ mx8_swz(r)), so the fragment reads (16 rows, one
//             chunk each) touch 16 different 16-byte bank groups;
//   W codes   BN/16 tiles of 2 KiB: the first 16 bytes of every lane's 32
//             in the blob's tile, then the second 16, so that a fragment
//             read is 64 consecutive 16-byte chunks;
//   A scales  BM rows x 4 B (the K-step's four block scales of a row);
//   W scales  BN/64 scale-word sets x 64 lanes x 4 B.
// Rows beyond M and row groups beyond N/16 are read from clamped valid
// addresses; they only feed outputs that are never stored.
// chunk swizzle of the staged 8-bit activation rows: the rows r and r + 8
// of a 16-row fragment read land in different bank groups
__device__ __forceinline__ int mx8_swz(int r) { return ((r & 7) + ((r >> 3) & 1)) & 7; }

template <int BN, int BM, int WN, int WM, int DEPTH>
struct Mx8Cfg {
  static constexpr int WAVES = WN * WM;
  static constexpr int FN = BN / 16 / WN, FM = BM / 16 / WM;
  static constexpr int A_BYTES = BM * 128, W_BYTES = BN * 128;
  static constexpr int AS_BYTES = BM * 4, WS_BYTES = (BN / 64) * 256;
  static constexpr int STAGE = A_BYTES + W_BYTES + AS_BYTES + WS_BYTES;
  static constexpr int A_DMA = A_BYTES / 1024 / WAVES, W_DMA = W_BYTES / 1024 / WAVES;
  static constexpr int AS_DW = BM / WAVES;              // activation scale dwords per wave
  static constexpr int WS_SETS = BN / 64 / WAVES;       // scale-word sets per wave (0: shared)
  static constexpr int COPIES = A_DMA + W_DMA + 1 + 1;
  static_assert(A_DMA * WAVES * 1024 == A_BYTES && W_DMA * WAVES * 1024 == W_BYTES, "copy split");
  static_assert(AS_DW <= 64 && (BN / 64) <= WAVES, "scale copies: one instruction per wave each");
  static_assert(FN % 4 == 0, "weight scale words per wave");
  static_assert(DEPTH * STAGE <= 160 * 1024, "LDS");
  static_assert((DEPTH - 1) * COPIES < 64, "vmcnt range");
};

template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
__device__ __forceinline__ void mx8_issue(const uint8_t* __restrict__ a_codes,
                                          const uint8_t* __restrict__ a_scales,
                                          const uint8_t* __restrict__ wc,
                                          const uint32_t* __restrict__ wsw, int64_t M, int64_t K,
                                          int64_t KS, int64_t NG, int64_t NSG, int64_t m0,
                                          int64_t ng0, int64_t ks, LDS uint8_t* dst, int wave,
                                          int lane) {
  using C = Mx8Cfg<BN, BM, WN, WM, DEPTH>;
  // activation rows: copy f covers rows 8 f .. 8 f + 7; lane L fills chunk
  // position L % 8 of row L / 8 with the chunk that belongs there
#pragma unroll
  for (int i = 0; i < C::A_DMA; ++i) {
    const int f = wave * C::A_DMA + i;
    const int rr = 8 * f + (lane >> 3);
    int64_t row = m0 + rr;
    row = row < M ? row : M - 1;
    const int j = (lane & 7) ^ mx8_swz(rr);
    __builtin_amdgcn_global_load_lds(a_codes + row * K + ks * 128 + 16 * j, dst + f * 1024, 16, 0, 0);
  }
  LDS uint8_t* wdst = dst + C::A_BYTES;
#pragma unroll
  for (int i = 0; i < C::W_DMA; ++i) {
    const int f = wave * C::W_DMA + i;  // 16-byte half (f % 2) of every lane's 32 bytes of tile f / 2
    int64_t ng = ng0 + f / 2;
    ng = ng < NG ? ng : NG - 1;
    __builtin_amdgcn_global_load_lds(wc + (ng * KS + ks) * 2048 + 32 * lane + 16 * (f & 1), wdst + f * 1024, 16,
                                     0, 0);
  }
  LDS uint8_t* asdst = wdst + C::W_BYTES;
  if (lane < C::AS_DW) {
    int64_t row = m0 + wave * C::AS_DW + lane;
    row = row < M ? row : M - 1;
    __builtin_amdgcn_global_load_lds(a_scales + row * (K / 32) + ks * 4, asdst + wave * C::AS_DW * 4,
                                     4, 0, 0);
  }
  LDS uint8_t* wsdst = asdst + C::AS_BYTES;
  if (wave < BN / 64) {
    int64_t sg = ng0 / 4 + wave;
    sg = sg < NSG ? sg : NSG - 1;
    __builtin_amdgcn_global_load_lds(wsw + (sg * KS + ks) * 64 + lane, wsdst + wave * 256, 4, 0, 0);
  } else {
    // same copy count on every wave: the last set again (same bytes)
    int64_t sg = ng0 / 4 + (BN / 64 - 1);
    sg = sg < NSG ? sg : NSG - 1;
    __builtin_amdgcn_global_load_lds(wsw + (sg * KS + ks) * 64 + lane,
                                     wsdst + (BN / 64 - 1) * 256, 4, 0, 0);
  }
}

template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
__device__ __forceinline__ void mx8_step(const LDS uint8_t* __restrict__ st, int wn, int wm, int lane,
                                         v4f (&acc)[BN / 16 / WN][BM / 16 / WM]) {
  using C = Mx8Cfg<BN, BM, WN, WM, DEPTH>;
  constexpr int FN = C::FN, FM = C::FM;
  const int r = lane & 15, c = lane >> 4;
  const LDS uint8_t* A = st;
  const LDS uint8_t* W = st + C::A_BYTES;
  const LDS uint8_t* AS = W + C::W_BYTES;
  const LDS uint32_t* WS = reinterpret_cast<const LDS uint32_t*>(AS + C::AS_BYTES);
  if constexpr (FMT == MXFP8) {
    // bf16 expansion with the block scales folded in: the first half of a
    // lane's bytes lies in block c / 2, the second in block 2 + c / 2
    const int b0 = c >> 1;
    Bf16Frag ab[FM];
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int R = wm * (16 * FM) + 16 * j + r;
      const u32x4 lo = *reinterpret_cast<const LDS u32x4*>(A + R * 128 + 16 * (c ^ mx8_swz(R)));
      const u32x4 hi = *reinterpret_cast<const LDS u32x4*>(A + R * 128 + 16 * ((4 + c) ^ mx8_swz(R)));
      ab[j] = e4m3_frag_bf16(v8i_of(lo, hi), e8m0_scale(AS[R * 4 + b0]), e8m0_scale(AS[R * 4 + 2 + b0]));
    }
    uint32_t sw0[FN / 4], sw1[FN / 4];
#pragma unroll
    for (int q = 0; q < FN / 4; ++q) {
      sw0[q] = WS[(wn * (FN / 4) + q) * 64 + r + 16 * b0];
      sw1[q] = WS[(wn * (FN / 4) + q) * 64 + r + 16 * (2 + b0)];
    }
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const LDS uint8_t* wt = W + (wn * FN + i) * 2048 + 16 * lane;
      const u32x4 wlo = *reinterpret_cast<const LDS u32x4*>(wt);
      const u32x4 whi = *reinterpret_cast<const LDS u32x4*>(wt + 1024);
      const int sh = 8 * (i % 4);
      const Bf16Frag wb = e4m3_frag_bf16(v8i_of(wlo, whi), e8m0_scale(sw0[i / 4] >> sh),
                                         e8m0_scale(sw1[i / 4] >> sh));
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = mfma_bf16x4(wb, ab[j], acc[i][j]);
    }
  } else {
    v8i af[FM];
    Mx8Split as[FM];
    int sa[FM];
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int R = wm * (16 * FM) + 16 * j + r;
      const u32x4 lo = *reinterpret_cast<const LDS u32x4*>(A + R * 128 + 16 * (c ^ mx8_swz(R)));
      const u32x4 hi = *reinterpret_cast<const LDS u32x4*>(A + R * 128 + 16 * ((4 + c) ^ mx8_swz(R)));
      af[j] = v8i_of(lo, hi);
      sa[j] = AS[R * 4 + c];
      as[j] = int8_frag_split(af[j]);
    }
    uint32_t sw[FN / 4];
#pragma unroll
    for (int q = 0; q < FN / 4; ++q) sw[q] = WS[(wn * (FN / 4) + q) * 64 + lane];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const LDS uint8_t* wt = W + (wn * FN + i) * 2048 + 16 * lane;
      const u32x4 wlo = *reinterpret_cast<const LDS u32x4*>(wt);
      const u32x4 whi = *reinterpret_cast<const LDS u32x4*>(wt + 1024);
      const v8i w = v8i_of(wlo, whi);
      const Mx8Split ws = int8_frag_split(w);
#pragma unroll
      for (int j = 0; j < FM; ++j)
        acc[i][j] = mx8_mfma<FMT>(i % 4, w, ws, af[j], as[j], acc[i][j], int(sw[i / 4]), sa[j]);
    }
  }
}

template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
__global__ __launch_bounds__(64 * WN * WM, 1) void gemm_mx8_tile_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ blob, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int tiles_m, int tiles_total, int per_xcd) {
  if (!blob_header_ok(blob, FMT, N, K)) {
    fill_y_nan(Y, M, N);
    return;
  }
  static_assert(FMT == MXFP8 || FMT == MXINT8, "8-bit MX formats");
  using C = Mx8Cfg<BN, BM, WN, WM, DEPTH>;
  constexpr int FN = C::FN, FM = C::FM;
  const int tile = int(blockIdx.x % 8) * per_xcd + int(blockIdx.x / 8);
  if (tile >= tiles_total) return;
  int tm, tn;
  col_block_tile(tile, tiles_m, tiles_total, tm, tn);

  const BlobLayout L = blob_layout(FMT, N, K);
  const int64_t m0 = int64_t(tm) * BM, ng0 = int64_t(tn) * (BN / 16);
  const uint8_t* wc = blob + L.code_off;
  const uint32_t* wsw = reinterpret_cast<const uint32_t*>(blob + L.scale_off);

  __shared__ __attribute__((aligned(1024))) uint8_t smem[DEPTH * C::STAGE];
  LDS uint8_t* base = (LDS uint8_t*)smem;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int wn = wave % WN, wm = wave / WN;

  v4f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int64_t KS = L.KS;
#pragma unroll
  for (int s = 0; s < DEPTH - 1; ++s)
    if (s < KS)
      mx8_issue<FMT, BN, BM, WN, WM, DEPTH>(a_codes, a_scales, wc, wsw, M, K, KS, L.NG, L.NSG, m0,
                                            ng0, s, base + s * C::STAGE, wave, lane);
  for (int64_t s = 0; s < KS; ++s) {
    // stages issued after s: min(DEPTH - 2, KS - 1 - s)
    const int64_t left = KS - 1 - s;
    stage_ready<C::COPIES, DEPTH>(int(left < DEPTH - 2 ? left : DEPTH - 2));
    if (s + DEPTH - 1 < KS)
      mx8_issue<FMT, BN, BM, WN, WM, DEPTH>(a_codes, a_scales, wc, wsw, M, K, KS, L.NG, L.NSG, m0,
                                            ng0, s + DEPTH - 1,
                                            base + ((s + DEPTH - 1) % DEPTH) * C::STAGE, wave, lane);
    mx8_step<FMT, BN, BM, WN, WM, DEPTH>(base + (s % DEPTH) * C::STAGE, wn, wm, lane, acc);
  }

  __builtin_amdgcn_s_barrier();  // every wave is done with the stage buffers
  asm volatile("" ::: "memory");
  const TileArgs t = tile_args(FMT, a_codes, a_scales, blob, L, M, K, m0, ng0);
  tile_epilogue<FN, FM, WN, WM>(acc, base, t, blob, L, mx8_epilogue_factor(FMT), Y, M, N, wave, lane);
}

template <int FMT, int BN, int BM, int WN, int WM, int DEPTH>
hipError_t launch_mx8_tile(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                           const uint8_t* blob, uint16_t* Y, hipStream_t stream) {
  const int tiles_n = int((N + BN - 1) / BN);
  const int tiles_m = int((M + BM - 1) / BM);
  const int total = tiles_n * tiles_m;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL((gemm_mx8_tile_kernel<FMT, BN, BM, WN, WM, DEPTH>), dim3(unsigned(per_xcd * 8)),
                     dim3(64 * WN * WM), 0, stream, ac, as, blob, Y, M, N, K, tiles_m, total,
                     per_xcd);
  return hipGetLastError();
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
                      const float* t_act, const uint8_t* blob, uint16_t* Y, void* workspace,
                      hipStream_t stream) {
  if constexpr (FMT == MXFP8 || FMT == MXINT8) {
    if (M <= 16) {
      // weight streaming; waves enough for at most 8 K-steps each, more
      // waves when there are few groups
      const int64_t ks = K / 128, groups = N / 16;
      // up to three rows: dot products on the VALU (the rows in LDS)
      if (M <= 3 && M * mx8_dot_row_bytes<FMT>(K) <= kMx8DotLds) {
        if (groups < 1024) return launch_mx8_dot<FMT, 16, 2>(M, N, K, ac, as, blob, Y, stream);
        return launch_mx8_dot<FMT, 8, 2>(M, N, K, ac, as, blob, Y, stream);
      }
      if (ks <= 32 && groups < 256) return launch_mx8_decode<FMT, 16, 2>(M, N, K, ac, as, blob, Y, stream);
      if (ks <= 32 && groups < 1024) return launch_mx8_decode<FMT, 8, 4>(M, N, K, ac, as, blob, Y, stream);
      if (ks <= 32) return launch_mx8_decode<FMT, 4, 8>(M, N, K, ac, as, blob, Y, stream);
      // long K: 8 waves in batches of 8 K-steps (16 waves of 8 would not
      // fit their loads in the 128 registers a wave of 1024 threads has)
      return launch_mx8_decode<FMT, 8, 8>(M, N, K, ac, as, blob, Y, stream);
    }
    // 256 x 256 tiles with 8 waves (two per SIMD: one wave's operand
    // expansion runs beside the other's MFMAs) where they nearly fill the
    // CUs; otherwise 256 (n) x 128 (m) tiles with 4 waves, twice as many
    if (((N + 255) / 256) * ((M + 255) / 256) >= 160)
      return launch_mx8_tile<FMT, 256, 256, 2, 4, 2>(M, N, K, ac, as, blob, Y, stream);
    return launch_mx8_tile<FMT, 256, 128, 2, 2, 3>(M, N, K, ac, as, blob, Y, stream);
  } else if constexpr (FMT == NVFP4) {
    if (M <= 16) {
      // weight streaming; waves enough for at most 8 K-steps each, more
      // waves when there are few groups
      const int64_t ks = K / 128, groups = N / 16;
      // one row: the dot-product kernel, its activation row expanded once
      // per workgroup into LDS (2 K bytes); 16 waves in batches of 2 K-steps
      // when there are few groups (Llama QKV, O, down), 8 waves in batches
      // of 4 with many (gate+up): the fastest of the seven configurations
      // measured at each shape (four linears 37.3 us against 41.9 on the
      // MFMA decode kernel); from two rows the MFMA kernel wins
      if (M == 1 && K <= 32768) {
        if (groups < 1024) return launch_nv_dot<16, 2>(M, N, K, ac, as, t_act, blob, Y, stream);
        return launch_nv_dot<8, 4>(M, N, K, ac, as, t_act, blob, Y, stream);
      }
      if (ks <= 32 && groups < 256) return launch_nv_decode<16, 2>(M, N, K, ac, as, t_act, blob, Y, stream);
      if (ks <= 32 && groups < 1024) return launch_nv_decode<8, 4>(M, N, K, ac, as, t_act, blob, Y, stream);
      if (ks <= 32) return launch_nv_decode<4, 8>(M, N, K, ac, as, t_act, blob, Y, stream);
      if (ks <= 64) return launch_nv_decode<8, 8>(M, N, K, ac, as, t_act, blob, Y, stream);
      return launch_nv_decode<16, 8>(M, N, K, ac, as, t_act, blob, Y, stream);
    }
    // NVFP4 runs four fp16 MFMAs per fragment pair, so its K-step is long
    // enough for 64 x 64 wave tiles at any shape, and it holds expanded fp16
    // fragments that would not fit the register budget of a 128 x 64 tile.
    return launch_tile<FMT, 256, 128, 4, 2, 5>(M, N, K, ac, as, t_act, blob, Y, stream);
  } else if constexpr (FMT == MXFP4) {
    if (M <= 16) {
      // 16-feature workgroups; waves enough for at most 8 K-steps each
      const int64_t ks = K / 128;
      // two whole 32-row groups per workgroup when there are enough of them
      // to fill the CUs twice over, and more than 4 activation rows to
      // share (Llama gate+up at M = 16: 20.5 -> 15.6 us; batches of 4
      // K-steps keep the 16 fragments in flight that 8 of one slice had)
      // (activation scales as dwords there: -4%; on the 16-feature
      // workgroups of the smaller linears they gained nothing)
      if (M > 4 && N % 64 == 0 && N / 64 >= 256 && ks <= 32)
        return launch_fp4_decode16<4, 4, 4, true>(M, N, K, ac, as, blob, Y, stream);
      // one whole group per workgroup from 192 groups on (Llama QKV at M =
      // 16: 7.1 -> 6.2 us; with 128 groups, O and down, it is slower)
      if (M > 4 && N % 32 == 0 && N / 32 >= 192 && ks <= 32)
        return launch_fp4_decode16<4, 8, 2, true>(M, N, K, ac, as, blob, Y, stream);
      if (ks <= 32) return launch_fp4_decode16<4>(M, N, K, ac, as, blob, Y, stream);
      if (ks <= 64) return launch_fp4_decode16<8>(M, N, K, ac, as, blob, Y, stream);
      // one load batch per wave sized to its K-steps when they are <= 7
      // (Llama down, K = 14336: 7.9 -> 7.4 us against batches of 8 with
      // one masked slot)
      if ((ks + 15) / 16 <= 7) return launch_fp4_decode16<16, 7>(M, N, K, ac, as, blob, Y, stream);
      return launch_fp4_decode16<16>(M, N, K, ac, as, blob, Y, stream);
    }
    if (M <= 32) {
      // large grids: 4 waves streaming 8 tiles each per batch; small grids
      // (fewer groups than about two per CU): 8 waves of 4
      if ((N + 31) / 32 >= 512) return launch_fp4_decode<4, 8>(M, N, K, ac, as, blob, Y, stream);
      return launch_fp4_decode<8, 4>(M, N, K, ac, as, blob, Y, stream);
    }
    // few tiles and a long K: split-K; large problems: the persistent
    // kernel (256 x 256 tiles and halves); otherwise 256 x 256 tiles (4
    // waves of 128 x 128) unless that leaves more than ~30% of the 256 CUs
    // idle, then 256 (n) x 128 (m) tiles.
    if (fp4_splitk_fits(M, N, K)) return launch_fp4_splitk(M, N, K, ac, as, blob, Y, workspace, stream);
    if (fp4_persistent_fits(M, N, K)) return launch_fp4_persistent(M, N, K, ac, as, blob, Y, stream);
    const int64_t big = ((N + 255) / 256) * ((M + 255) / 256);
    if (big >= 180) return launch_fp4<256, 256, 4>(M, N, K, ac, as, blob, Y, stream);
    return launch_fp4<256, 128, 5>(M, N, K, ac, as, blob, Y, stream);
  } else {
    if (M <= 16) {
      // waves enough for at most 7 or 8 K-steps each; with K <= 4096, more
      // waves (shorter per-wave chains) when there are few groups; long K:
      // 16 waves taking their K-steps in batches of 5, so that the MFMAs of
      // one batch overlap the loads of the next (Qwen down, K = 18944: 12.5
      // -> 9.8 us against one batch of 10)
      const int64_t ks = K / 128, groups = N / 16;
      // one row: the dot-product kernel, K-steps in batches of 2; 16 waves
      // when there are few groups (Qwen QKV, O, down: 4.9, 4.3, 9.2 us), 8
      // with many (gate+up: 14.8 us); the six configurations measured put
      // these first at each shape
      if (M == 1 && K <= 65536) {
        if (groups < 1024) return launch_mxint4_dot<16, 2>(M, N, K, ac, as, blob, Y, stream);
        return launch_mxint4_dot<8, 2>(M, N, K, ac, as, blob, Y, stream);
      }
      if (ks <= 32 && groups < 256) return launch_decode<FMT, 16, 2>(M, N, K, ac, as, blob, Y, stream);
      if (ks <= 32 && groups < 1024) return launch_decode<FMT, 8, 4>(M, N, K, ac, as, blob, Y, stream);
      if (ks <= 28) return launch_decode<FMT, 4, 7>(M, N, K, ac, as, blob, Y, stream);
      if (ks <= 32) return launch_decode<FMT, 4, 8>(M, N, K, ac, as, blob, Y, stream);
      if (ks <= 64) return launch_decode<FMT, 8, 8>(M, N, K, ac, as, blob, Y, stream);
      return launch_decode<FMT, 16, 5>(M, N, K, ac, as, blob, Y, stream);
    }
    // MXINT4 on the 16x16x128 FP8 MFMA with wave tiles of 128 x 64.
    // Fragments are widened to FP8 in registers by every wave that uses them,
    // so the VALU work per MFMA falls as the wave tile grows: 12 widened
    // fragments per 32 MFMAs against 8 per 16 with 64 x 64 (22-28% faster on
    // the Qwen linears); 128 x 128 spills.  256 x 256 tiles with two waves per
    // SIMD run ~8% more per tile than 256 x 128 tiles with one, so they are
    // taken unless their coarser rounds over the 256 CUs cost more.
    const int64_t tn = (N + 255) / 256;
    const int64_t rounds_lean = (tn * ((M + 255) / 256) + 255) / 256;
    const int64_t rounds_one = (tn * ((M + 127) / 128) + 255) / 256;
    if (100 * rounds_lean <= 54 * rounds_one)
      return launch_mx_lean<FMT, 256, 256, 2, 4, 4>(M, N, K, ac, as, blob, Y, stream);
    // Fewer than 128 tiles of 256 x 128 would leave half the CUs idle: then
    // the most tiles that still fit one round, 128 x 64 (wave tiles 64 x 32)
    // or 128 x 128 (64 x 64), which gain more from the CUs they add than
    // they lose per tile (Qwen at M = 512: QKV 51.6 -> 36.3 us with 128 x
    // 128, O 50.6 -> 26.9 and down 241 -> 114 us with 128 x 64).
    const int64_t t1 = tn * ((M + 127) / 128);
    if (t1 < 128) {
      const int64_t tn2 = (N + 127) / 128;
      if (tn2 * ((M + 63) / 64) <= 256) return launch_mx<FMT, 128, 64, 2, 2, 4>(M, N, K, ac, as, blob, Y, stream);
      if (tn2 * ((M + 127) / 128) <= 256)
        return launch_mx<FMT, 128, 128, 2, 2, 4>(M, N, K, ac, as, blob, Y, stream);
    }
    return launch_mx<FMT, 256, 128, 2, 2, 4>(M, N, K, ac, as, blob, Y, stream);
  }
}

}  // namespace

size_t linear_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K) {
  if (fmt == MXFP4 && fp4_splitk_fits(M, N, K)) return fp4_splitk_workspace(M, N);
  return 0;
}

hipError_t launch_linear(int fmt, int64_t M, int64_t N, int64_t K, const void* a_codes,
                         const void* a_scales, const float* t_act, const void* blob, void* Y,
                         void* workspace, size_t, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const uint8_t* ac = static_cast<const uint8_t*>(a_codes);
  const uint8_t* as = static_cast<const uint8_t*>(a_scales);
  const uint8_t* b = static_cast<const uint8_t*>(blob);
  uint16_t* y = static_cast<uint16_t*>(Y);
  switch (fmt) {
    case MXFP4: return launch_fmt<MXFP4>(M, N, K, ac, as, t_act, b, y, workspace, stream);
    case MXINT4: return launch_fmt<MXINT4>(M, N, K, ac, as, t_act, b, y, workspace, stream);
    case MXFP8: return launch_fmt<MXFP8>(M, N, K, ac, as, t_act, b, y, workspace, stream);
    case MXINT8: return launch_fmt<MXINT8>(M, N, K, ac, as, t_act, b, y, workspace, stream);
    default: return launch_fmt<NVFP4>(M, N, K, ac, as, t_act, b, y, workspace, stream);
  }
}

// ------------------------------------------------ allocation-free linear --
//
// For callers that cannot allocate (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc): the split-K workspace comes from
// `scratch`, a device array of this library, one copy per device, that lives
// until the process ends.  Its address on a device is looked up once, with
// that device current, and kept per device; the array's name is only a host
// stand-in and never reaches a kernel.  Every call on a device shares that
// device's copy, so calls that overlap on one device race.

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// zero the synchronization words and the status of the split-K workspace
// (a kernel, not hipMemsetAsync, so that the call can be captured in a graph)
__global__ __launch_bounds__(256) void clear_sync_kernel(uint8_t* __restrict__ ws) {
  for (int i = int(threadIdx.x); i < Fp4S::SYNC_BYTES / 16; i += 256)
    reinterpret_cast<u32x4*>(ws)[i] = u32x4{0u, 0u, 0u, 0u};
}

}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot] {
    slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
    if (slot.err == hipSuccess && slot.ptr == nullptr) slot.err = hipErrorInvalidSymbol;
  });
  *out = slot.ptr;
  return slot.err;
}

hipError_t launch_linear_noalloc(int fmt, int64_t M, int64_t N, int64_t K, const void* a_codes,
                                 const void* a_scales, const float* t_act, const void* blob,
                                 void* Y, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const size_t need = linear_workspace_bytes(fmt, M, N, K);
  if (need == 0)
    return launch_linear(fmt, M, N, K, a_codes, a_scales, t_act, blob, Y, nullptr, 0, stream);
  if (need > kNoAllocScratchBytes) return hipErrorInvalidValue;  // rejected on the host first
  void* ws = nullptr;
  hipError_t e = noalloc_scratch(&ws);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(clear_sync_kernel, dim3(1), dim3(256), 0, stream, static_cast<uint8_t*>(ws));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_linear(fmt, M, N, K, a_codes, a_scales, t_act, blob, Y, ws, need, stream);
}

hipError_t launch_linear_grouped(int fmt, int P, int64_t M, int64_t K, const int64_t* N,
                                 const void* const* a_codes, const void* const* a_scales,
                                 const float* const* t_act, const void* const* blobs,
                                 void* const* Y, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  bool all_persistent = true;
  for (int p = 0; p < P; ++p) all_persistent &= fmt == MXFP4 && fp4_persistent_fits(M, N[p], K);
  if (fmt != MXFP4 || M <= 32 || all_persistent) {
    // one after another, each on its own kernel (none of these needs a workspace)
    for (int p = 0; p < P; ++p) {
      const hipError_t e = launch_linear(fmt, M, N[p], K, a_codes[p], a_scales[p],
                                         t_act ? t_act[p] : nullptr, blobs[p], Y[p], nullptr, 0,
                                         stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // 256 (n) x 128 (m) tiles of all problems in one launch
  Fp4Problems g{};
  const int tiles_m = int((M + 127) / 128);
  g.P = P;
  g.first[0] = 0;
  for (int p = 0; p < P; ++p) {
    g.ac[p] = static_cast<const uint8_t*>(a_codes[p]);
    g.as[p] = static_cast<const uint8_t*>(a_scales[p]);
    g.blob[p] = static_cast<const uint8_t*>(blobs[p]);
    g.Y[p] = static_cast<uint16_t*>(Y[p]);
    g.N[p] = N[p];
    g.first[p + 1] = g.first[p] + int((N[p] + 255) / 256) * tiles_m;
  }
  for (int p = P; p < kMaxGroup; ++p) g.first[p + 1] = g.first[P];
  const int per_xcd = (g.first[P] + 7) / 8;
  hipLaunchKernelGGL((gemm_fp4_grouped_kernel<256, 128, 5>), dim3(unsigned(per_xcd * 8)), dim3(256),
                     0, stream, g, M, K, tiles_m, per_xcd);
  return hipGetLastError();
}

}  // namespace w4a4
