/*
 * w4a4.h - C ABI of the MI355X (gfx950) packed W4A4 block-scaled linear.
 *
 * What the library computes (DualQuant, "Dual-scale Calibration-free
 * Weight-and-Activation Quantization for LLMs"):
 *
 *   Section 4.2, eq. (2)-(3): a weight is stored as W ~ diag(r) . Q . diag(c)
 *   with row scales r (the inverse alpha) and column scales c (the inverse
 *   beta); the column scales become an activation rescaling X~ = X diag(c).
 *   Section 4.4: at inference the layer computes Q(X~) . Q^T . diag(r), where
 *   Q(X~) is the format-native row-wise block quantization of X~, c is
 *   multiplied in inside the activation-quantization kernel and r is applied
 *   to the GEMM output.  Section 3: block formats MXFP4 (E2M1, blocks of 32,
 *   E8M0 scale), MXINT4 (int4, blocks of 32, E8M0 scale) and NVFP4 (E2M1,
 *   blocks of 16, UE4M3 scale) plus an FP32 tensor scale for NVFP4.
 *   Appendix I: weights are packed offline into the GEMM's storage layout
 *   and stay packed; group scales are consumed inside the GEMM; the GEMM
 *   entry allocates nothing, so a whole model can be captured in a graph.
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument named as device memory must point to memory
 *     of the device that owns `stream` (a hipStream_t; NULL = the null
 *     stream of the current device).  The caller owns all buffers; the
 *     library never allocates, frees or synchronizes, and keeps no pointer
 *     after a call returns (w4a4_linear_noalloc's scratch array is the
 *     library's own, see there).  Work is enqueued on `stream`; buffers must stay
 *     valid until the stream has executed it.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     non-OK status means nothing was enqueued.  w4a4_last_error() then
 *     returns a message (thread-local).  Launch failures return
 *     W4A4_ERR_HIP.  No entry point aborts the process.
 *   - Row-major everywhere; K is the reduction (input-feature) dimension.
 *   - Canonical code layout: [rows x K/2] bytes, element 2j of a row in the
 *     low nibble of byte j and element 2j+1 in the high nibble.  FP4 codes
 *     are E2M1 (sign bit 3), INT4 codes two's complement.  Canonical scale
 *     layout: [rows x K/G] bytes (E8M0 for MX formats, UE4M3 for NVFP4).
 *   - Calls are reentrant; the library has no mutable global state, apart
 *     from the per-device scratch array of w4a4_linear_noalloc.
 */
#ifndef W4A4_H_
#define W4A4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4A4_MXFP4 = 0,   /* E2M1 elements, G = 32, E8M0 block scale             */
  W4A4_NVFP4 = 1,   /* E2M1 elements, G = 16, UE4M3 block scale + fp32 t   */
  W4A4_MXINT4 = 2,  /* int4 elements, G = 32, E8M0 block scale             */
  W4A4_INT4G64 = 3, /* int4 elements, G = 64, BF16 block scale (see below)  */
  W4A4_MXFP8 = 4,   /* E4M3 elements, G = 32, E8M0 block scale (8-bit)     */
  W4A4_MXINT8 = 5,  /* int8 elements, G = 32, E8M0 block scale (8-bit)     */
  W4A4_INT8G128 = 6 /* int8 elements, G = 128, BF16 block scale (8-bit)    */
} w4a4_format;

/*
 * W4A4_MXFP8, W4A4_MXINT8 - the 8-bit MX variants of Appendix G.2 (Table 9:
 * MXFP8 and MXINT8 with G = 32), for the same quantize / pack / linear path.
 * Codes take one byte each: canonical codes are [rows x K] bytes (E4M3 bytes,
 * or two's-complement int8), scales [rows x K/32] E8M0 bytes.  The block
 * scale follows the OCP shared-exponent rule with the element grid's largest
 * binade: e = floor(log2 amax) - 8 for E4M3 (448 = 1.75 * 2^8; elements
 * RNE_E4M3(x~ * 2^-e) saturating at +-448, sign kept for -0), and
 * e = floor(log2 amax) - 6 for int8 (127 < 2^7; elements clamp(RNE(x~ *
 * 2^-e), -128, 127)).  Supported by the size queries, w4a4_quantize_act,
 * w4a4_pack_weight, w4a4_unpack_weight, w4a4_linear and w4a4_linear_noalloc
 * (no workspace); the multi-output quantizer, the grouped linear and the
 * solver return W4A4_ERR_FORMAT.  MXINT8 runs on the scaled FP8 MFMA
 * (16x16x128, E8M0 block scales in hardware) with each int8 code split into
 * 16 h + l (h = q >> 4 in [-8, 7], l = q & 15), both parts exact in E4M3,
 * four MFMAs per K-step.  MXFP8 codes are expanded with their block scales
 * into bf16 (exact) for the bf16 MFMA: the FP8 MFMA drops small products
 * next to large ones within a block (about 14 bits kept), which E4M3's 36
 * binades of product range would expose.
 */

/*
 * W4A4_INT4G64 - the paper's packed deployment format (Appendix I: INT4,
 * G = 64, BF16 group scales; Section 3's symmetric quantizer with q_max = 7;
 * Section 4.2's BF16 admissible set for INT4).  A block's scale is
 * Delta = BF16(amax / 7), rounded once to nearest even; codes are
 * clip(RNE(x~ / Delta), -8, 7); a zero block has Delta = 0 and zero codes; a
 * block with a non-finite value gets Delta = 0x7FC0 and zero codes.  Scales
 * are stored as BF16 bit patterns, [rows x K/64] uint16 (two bytes per block,
 * w4a4_act_scales_bytes counts bytes).  K % 64 == 0 and N % 16 == 0 (no K % 128
 * requirement); there is no tensor scale (t_act and t_w are ignored; unpack
 * writes t_w = 1).  Supported by the size queries, w4a4_quantize_act,
 * w4a4_pack_weight, w4a4_unpack_weight and w4a4_linear (no workspace); the
 * multi-output quantizer, w4a4_linear_noalloc, the grouped linear and the
 * solver return W4A4_ERR_FORMAT for it.  The GEMM expands code x scale
 * exactly into fp16 for the fp16 MFMA (M > 16, K % 128 == 0), takes int4 dot
 * products on the VALU for up to three rows, and otherwise runs one int8
 * MFMA (16x16x64) per 64-block and applies Delta_a * Delta_w to each block
 * sum in fp32.
 */

/*
 * W4A4_INT8G128 - the 8-bit integer W+A variant of Appendix G.2 (Table 9: INT8
 * weights and activations in groups of 128), with Section 3's symmetric
 * quantizer (q_max = 127) and BF16 block scales as for W4A4_INT4G64.  A
 * block's scale is Delta = BF16(amax / 127), rounded once to nearest even;
 * codes are RNE(x~ / Delta) on the INT8 grid, clip(., -128, 127) (only a
 * subnormal Delta can take a code past +-127); a zero block has Delta = 0
 * and zero codes; a block with a non-finite value gets Delta = 0x7FC0 and
 * zero codes.  Canonical codes are [rows x K] two's-complement bytes,
 * scales [rows x K/128] BF16 bit patterns (two bytes per block).  K % 128 ==
 * 0 and N % 16 == 0; no tensor scale (t_act and t_w are ignored; unpack
 * writes t_w = 1).  w4a4_quantize_act needs codes 8-byte aligned.  Supported
 * by the size queries, w4a4_quantize_act, w4a4_pack_weight,
 * w4a4_unpack_weight and w4a4_linear (no workspace); the multi-output
 * quantizer, w4a4_linear_noalloc, the grouped linear and the solver return
 * W4A4_ERR_FORMAT for it.  The GEMM takes each 128-block's exact integer sum
 * (int8 dot products on the VALU for up to three rows, two int8 MFMAs
 * (16x16x64) per block otherwise) and applies Delta_a * Delta_w to it in
 * fp32.
 */

typedef enum {
  W4A4_OK = 0,
  W4A4_ERR_NULL = 1,       /* a required pointer is NULL                        */
  W4A4_ERR_SHAPE = 2,      /* M < 0, N or K out of range, K % G, N % 16, K % 128 */
  W4A4_ERR_ALIGN = 3,      /* a pointer misses its documented alignment         */
  W4A4_ERR_FORMAT = 4,     /* unknown format, or not supported by this call    */
  W4A4_ERR_WORKSPACE = 5,  /* workspace missing or smaller than required        */
  W4A4_ERR_HIP = 6         /* a HIP call or kernel launch failed                */
} w4a4_status;

/* Split-K workspace of w4a4_linear: bytes of synchronization words and
 * status at its start, and the byte offset of the int32 status word. */
#define W4A4_SPLITK_SYNC_BYTES 4352
#define W4A4_SPLITK_STATUS_OFFSET 4096

/* Block size G of a format (32, 16 or 32); 0 for an unknown format. */
int w4a4_block_size(w4a4_format fmt);

/* Byte sizes, so that callers allocate every buffer.  Return 0 for invalid
 * arguments. */
size_t w4a4_act_codes_bytes(w4a4_format fmt, int64_t M, int64_t K);   /* M*K/2 (8-bit: M*K) */
size_t w4a4_act_scales_bytes(w4a4_format fmt, int64_t M, int64_t K);  /* M*K/G */
size_t w4a4_quantize_workspace_bytes(w4a4_format fmt, int64_t M, int64_t K);
size_t w4a4_packed_weight_bytes(w4a4_format fmt, int64_t N, int64_t K);
size_t w4a4_linear_workspace_bytes(w4a4_format fmt, int64_t M, int64_t N, int64_t K);

/*
 * w4a4_quantize_act - fused rescale + block quantization of activations.
 *
 * DualQuant Section 4.4 (beta applied inside the activation-quantization
 * kernel, no separate launch; the format-native per-row block scale is still
 * computed on X~) with eq. (3) (X~ = X diag(beta)^-1 = X diag(c)), and the
 * quantizer of Section 3 (nearest grid point, clipped).
 *
 *   X      device, bf16 [M x K], 16-byte aligned.
 *   c      device, fp32 [K], 16-byte aligned; NULL means c = 1 (this is how
 *          weights W / (r c^T) are quantized before packing).
 *   codes  device, out, [M x K/2] canonical codes, 4-byte aligned ([M x K]
 *          bytes, 8-byte aligned, for MXFP8 and MXINT8).
 *   scales device, out, [M x K/G] canonical scale bytes.
 *   t_act  device, out, one fp32: the NVFP4 tensor scale
 *          t = fp32(max|X~|) / 2688 (t = 1 for an all-zero tensor).  Ignored
 *          (may be NULL) for MX formats.
 *   workspace / ws_bytes: device scratch of at least
 *          w4a4_quantize_workspace_bytes() bytes (0 for MX formats; NVFP4
 *          uses it for the tensor-amax partial maxima), 4-byte aligned.
 *
 * Per row, per block of G along K, with x~ = fp32(x) * c[k] (one rounded
 * fp32 multiply) and a = max |x~| over the block:
 *   MX:    e = clamp(floor(log2 a) - 2, -127, 127), byte e + 127 (0 if a = 0);
 *          MXFP4 code = RNE_E2M1(x~ * 2^-e) saturating at +-6;
 *          MXINT4 code = clamp(RNE(x~ * 2^-e), -8, 7).
 *          A block holding Inf/NaN gets byte 0xFF and zero codes.
 *   NVFP4: byte s = RNE_E4M3(a / (6 t)) saturating at 448; code =
 *          RNE_E2M1(x~ / (s t)); a block whose scale is 0 keeps sign-only
 *          zero codes.  Inputs must be finite.
 * All rounding decisions are exact (ties to even, decided against exact
 * midpoints), so codes and scales are fully determined by X and c.
 * Requires M >= 0, K > 0, K % G == 0.
 */
w4a4_status w4a4_quantize_act(w4a4_format fmt, int64_t M, int64_t K,
                              const void* X, const float* c,
                              void* codes, void* scales, float* t_act,
                              void* workspace, size_t ws_bytes, void* stream);

/*
 * w4a4_quantize_act_multi - one activation X quantized under P column-scale
 * vectors (per-projection c on a fused input, e.g. the q, k and v
 * projections of one hidden state: DualQuant deploys one beta per linear,
 * Section 4.4 and Appendix I).  X is read once; output p is what
 * w4a4_quantize_act(fmt, M, K, X, c[p], codes[p], scales[p], t_act[p]) would
 * write, bit for bit.
 *
 *   P        1 .. 4.
 *   c        host array of P device pointers, fp32 [K] each, 16-byte aligned.
 *   codes    host array of P device pointers, [M x K/2] each, 4-byte aligned.
 *   scales   host array of P device pointers, [M x K/G] each.
 *   t_act    host array of P device pointers to one fp32 each (NVFP4 only;
 *            may be NULL for MX formats).
 *   workspace/ws_bytes: NVFP4 needs P times w4a4_quantize_workspace_bytes()
 *            (4-byte aligned); MX formats need none.
 */
w4a4_status w4a4_quantize_act_multi(w4a4_format fmt, int64_t M, int64_t K,
                                    const void* X, int P, const float* const* c,
                                    void* const* codes, void* const* scales,
                                    float* const* t_act, void* workspace,
                                    size_t ws_bytes, void* stream);

/*
 * w4a4_pack_weight - pack a quantized weight into the GEMM storage layout.
 *
 * DualQuant Appendix I: the per-layer artifacts (quantized weight Q, row
 * scales, column scales; Section 4.4) are packed offline into the target
 * storage layout and remain packed during inference.  Here Q arrives as
 * canonical codes and block scales (for instance from w4a4_quantize_act with
 * c = NULL on W / (r c^T)); the column scales c are not part of the blob,
 * they are passed to w4a4_quantize_act at run time.
 *
 *   codes  device, [N x K/2] canonical codes, 16-byte aligned.
 *   scales device, [N x K/G] canonical scale bytes.
 *   t_w    device, one fp32 NVFP4 weight tensor scale; NULL means 1.
 *   r      device, fp32 [N] row scales (multiplied into the output).
 *   blob   device, out, w4a4_packed_weight_bytes() bytes, 256-byte aligned.
 *
 * Blob contents (opaque to callers apart from this description): a 256-byte
 * header (magic "W4A4PK01", format, N, K, t_w), then the codes in MFMA
 * fragment order (1 KiB tiles, lane l holding 16 bytes of one row: 32 output
 * rows x 64 K for MXFP4, 16 rows x 128 K for NVFP4 and MXINT4), the block
 * scales regrouped per K tile and lane (one dword carries the scale bytes of
 * 4 row groups for the MX formats, of 2 groups x 2 blocks for NVFP4), and r.
 * Rows past N up to the last full row group are zero.  Requires
 * N % 16 == 0, K % 128 == 0.
 */
w4a4_status w4a4_pack_weight(w4a4_format fmt, int64_t N, int64_t K,
                             const void* codes, const void* scales,
                             const float* t_w, const float* r,
                             void* blob, void* stream);

/*
 * w4a4_unpack_weight - inverse of w4a4_pack_weight (round-trip checks,
 * serialization).  Writes canonical codes, scales, r (each may be NULL to
 * skip) and t_w (device fp32, may be NULL) from a blob packed with the same
 * fmt, N and K.
 */
w4a4_status w4a4_unpack_weight(w4a4_format fmt, int64_t N, int64_t K,
                               const void* blob, void* codes, void* scales,
                               float* r, float* t_w, void* stream);

/*
 * w4a4_linear - block-scaled 4-bit x 4-bit GEMM with the row-scale epilogue.
 *
 * DualQuant Section 4.4: Y = Q(X~) . Q^T . diag(r); Appendix I: the block
 * scales are applied inside the GEMM (no weight dequantization pass) and the
 * entry point allocates nothing.
 *
 *   Y[m, n] = bf16_rne( r[n] * t * sum_k a^[m,k] w^[n,k] )
 *
 * where a^ / w^ are code times block scale and t = t_act * t_w for NVFP4
 * (1 for MX formats).  Accumulation is fp32.
 *
 *   a_codes  device, [M x K/2] canonical activation codes, 16-byte aligned.
 *   a_scales device, [M x K/G] canonical activation scales, 16-byte aligned.
 *   t_act    device, one fp32 (NVFP4 only; may be NULL for MX formats).
 *   blob     device, a blob packed for the same fmt, N, K, 256-byte aligned.
 *   Y        device, out, bf16 [M x N], 16-byte aligned.
 *   workspace/ws_bytes: device scratch of at least
 *            w4a4_linear_workspace_bytes() bytes, 16-byte aligned.  The size
 *            is 0 (and NULL accepted) except for MXFP4 shapes that split K
 *            across two workgroups (M > 32, 64..128 tiles of 256 x 256,
 *            K % 1024 == 0, K >= 8192): W4A4_SPLITK_SYNC_BYTES of
 *            synchronization words and status, then 256 KiB of fp32 partial
 *            sums per tile.  The first W4A4_SPLITK_SYNC_BYTES must be zero
 *            before the first call that uses the buffer; every call leaves
 *            the synchronization words zero again.  The int32 at byte
 *            W4A4_SPLITK_STATUS_OFFSET is a sticky status: a workgroup whose
 *            partner half never signalled (the synchronization words were not
 *            zero at the call) gives up after a bounded wait (about a
 *            second), ORs 1 into it and writes its 128 x 128 block of Y as
 *            BF16 NaN; the caller clears the word to reset it.  Calls sharing
 *            a workspace must not run concurrently (issue them in order on
 *            one stream).
 *
 * Requires M >= 0, N % 16 == 0, K % 128 == 0.  The blob's header (magic,
 * format, N, K) is checked on the device by every GEMM kernel before it reads
 * anything else of the blob: a blob packed for another format or shape gives
 * Y = BF16 NaN everywhere (the status is W4A4_OK: the host does not read
 * device memory), never a read past the blob.
 */
w4a4_status w4a4_linear(w4a4_format fmt, int64_t M, int64_t N, int64_t K,
                        const void* a_codes, const void* a_scales,
                        const float* t_act, const void* blob, void* Y,
                        void* workspace, size_t ws_bytes, void* stream);

/*
 * w4a4_linear_noalloc - w4a4_linear for callers that cannot allocate: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments as w4a4_linear without the workspace; the same
 * kernels run and Y is bit for bit what w4a4_linear writes.
 *
 * Scratch: the split-K workspace (the only one w4a4_linear uses) is taken
 * from a device array inside the library, W4A4_NOALLOC_SCRATCH_BYTES
 * (32 MiB + 4352 B, the largest split-K workspace), one copy on every device
 * the library runs on, held until the process ends.  Its address on a device
 * is looked up on the first call on that device (with that device current).
 * Each split-K call first clears the array's synchronization words and
 * status with a small kernel on `stream`.  Every call on a device shares
 * that device's array: calls that overlap on one device (other streams,
 * other threads, other graphs) race and must be serialized by the caller.
 * A split-K wave that gives up waiting for its partner writes its 128 x 128
 * block of Y as BF16 NaN (see w4a4_linear); the status word stays inside the
 * library.  Shapes whose workspace would exceed the array return
 * W4A4_ERR_WORKSPACE (none does: split-K shapes have at most 128 tiles).
 * Nothing is allocated, freed or synchronized.  Not available for
 * W4A4_INT4G64 and W4A4_INT8G128 (W4A4_ERR_FORMAT).
 */
#define W4A4_NOALLOC_SCRATCH_BYTES (4352 + 128 * 4 * 65536)
w4a4_status w4a4_linear_noalloc(w4a4_format fmt, int64_t M, int64_t N, int64_t K,
                                const void* a_codes, const void* a_scales,
                                const float* t_act, const void* blob, void* Y,
                                void* stream);

/*
 * w4a4_linear_grouped - P linears of one M and K (the per-projection linears
 * of a fused input, e.g. q, k and v with their own column scales, after
 * w4a4_quantize_act_multi): output p is what w4a4_linear(fmt, M, N[p], K,
 * a_codes[p], a_scales[p], t_act[p], blobs[p], Y[p]) computes, within the
 * same accumulation-order tolerance.  For MXFP4 with M > 32 the problems'
 * 256 x 128 tiles run in one launch, unless each would take the persistent
 * kernel on its own; otherwise (and for the other formats) they run one
 * after another on their usual kernels.  No workspace is needed.
 *
 *   P        1 .. 4.
 *   N        host array of P output widths (each % 16 == 0).
 *   a_codes, a_scales, blobs, Y: host arrays of P device pointers, with the
 *            alignments of w4a4_linear.
 *   t_act    host array of P device pointers (NVFP4 only; may be NULL for MX).
 */
w4a4_status w4a4_linear_grouped(w4a4_format fmt, int P, int64_t M, int64_t K,
                                const int64_t* N, const void* const* a_codes,
                                const void* const* a_scales, const float* const* t_act,
                                const void* const* blobs, void* const* Y, void* stream);

/*
 * w4a4_dualquant_solve - the offline dual-scale solver.
 *
 * DualQuant Algorithm 1 (Section 4.3, block coordinate descent with
 * closed-form scale updates; initialization and T from Section 5): finds the
 * row scales r (= alpha^-1) and column scales c (= beta^-1) in the format's
 * admissible set (powers of two, E8M0, for MXFP4 / MXINT4; positive E4M3
 * values, UE4M3, for NVFP4) and the codes Q = Q(Diag(alpha) W Diag(beta)) so
 * that W ~ Diag(r) Q Diag(c).  r, t_w and the codes/scales go to
 * w4a4_pack_weight, c to w4a4_quantize_act.  Starting from alpha_0 = 1 / row absmax and
 * beta_0 = 1 / column l1 norm, each iteration sets r_i to the admissible value
 * nearest to <W_i, R_i> / ||R_i||^2 with R = Q^ Diag(beta)^-1 (Q^ the
 * quantized rescaled weight; for NVFP4 with the fp32 tensor scale of that
 * rescaled weight, as in w4a4_quantize_act), re-quantizes, then sets c_j likewise from
 * S = Diag(alpha)^-1 Q^ over the columns.  A row or column whose Q^ is all
 * zero gets scale 1.  The inner products and norms are fp64 sums in a fixed
 * order (rows: 8 terms, then ((p0 + p1) + p2) + p3 per 32-block, then the
 * blocks in order; columns: 16-row chunks in order, then the chunks), so
 * results are deterministic.  The iterations stop once one leaves (r, c)
 * unchanged (a fixed point: the rest would repeat it).
 *
 *   W        device, fp32 [N x K] row-major (N output rows, K inputs),
 *            16-byte aligned; finite values.
 *   iters    T >= 1 (the paper uses 15).
 *   r        device, out, fp32 [N], 4-byte aligned.
 *   c        device, out, fp32 [K], 4-byte aligned.
 *   codes    device, out, [N x K/2] canonical codes, 4-byte aligned.
 *   scales   device, out, [N x K/G] scale bytes (E8M0; UE4M3 for NVFP4).
 *   t_w      device, out, one fp32: the NVFP4 tensor scale of the returned
 *            codes (required for NVFP4, not written for MX formats; may be
 *            NULL there).
 *   workspace/ws_bytes: device scratch of at least
 *            w4a4_dualquant_workspace_bytes() bytes, 256-byte aligned
 *            (fp64 partial sums: 16 B per 32-block and per 16-row chunk and
 *            column, the current and previous scales, a flag); no initial
 *            contents needed.
 *
 * Requires N > 0, K % 32 == 0 (for every format), N*K <= 2^36.  Kernels are
 * enqueued on `stream`; nothing is allocated.
 */
size_t w4a4_dualquant_workspace_bytes(w4a4_format fmt, int64_t N, int64_t K);
w4a4_status w4a4_dualquant_solve(w4a4_format fmt, int64_t N, int64_t K,
                                 const float* W, int iters, float* r, float* c,
                                 void* codes, void* scales, float* t_w,
                                 void* workspace, size_t ws_bytes, void* stream);

/*
 * Measurement aids for the decode roofline (not part of the quantized
 * linear).  w4a4_probe_stream_read reads `bytes` of device memory once, in
 * one launch, with 16-byte non-temporal loads four in flight per lane (the
 * decode GEMMs' access): its duration is what any kernel reading that many
 * bytes once can reach, the ceiling the weight-streaming decode GEMMs are
 * compared with at their own sizes.  w4a4_probe_empty launches an empty
 * kernel (the cost of one launch).
 *
 *   src      device, 16-byte aligned, `bytes` readable.
 *   bytes    a positive multiple of 16.
 *   sink     device, 256 x 4 bytes, 4-byte aligned; written only in the
 *            (practically impossible) case that a workgroup's XOR of its
 *            data equals a fixed constant, which keeps the loads live.
 * Returns W4A4_ERR_NULL, W4A4_ERR_SHAPE or W4A4_ERR_ALIGN for bad arguments;
 * enqueued on `stream`.
 */
w4a4_status w4a4_probe_stream_read(const void* src, size_t bytes, void* sink, void* stream);
w4a4_status w4a4_probe_empty(void* stream);

/*
 * Measurement aid for the prefill roofline (not part of the quantized
 * linear): the scaled FP4 MFMA of the MXFP4 GEMMs (32 x 32 x 64, E8M0
 * scales) alone, on register operands.  Each of the 4 waves of each of
 * `workgroups` workgroups holds a 128 x 128 tile of fp32 accumulators (4 x 4
 * blocks of 32 x 32, as a wave of the persistent MXFP4 GEMM) and runs `iters`
 * rounds of its 16 MFMAs, alternating two operand sets, with no memory
 * traffic in the loop: 2 * 128 * 128 * 64 * iters * 4 * workgroups FP4
 * operations per launch.  Its rate is what the matrix cores sustain at the
 * clock the chip holds under that load, for the operand bits given (random
 * codes draw more power than zeros).
 *
 *   ops         device, 16-byte aligned, 16 KiB: 16 fragments of 64 lanes x
 *               16 bytes (32 FP4 codes a lane): weight fragments 0..3 and
 *               activation fragments 4..7 of set 0, then 8..15 of set 1.
 *   iters       even, 2 .. 2^20.
 *   workgroups  1 .. 4096 (one workgroup per CU at most: 256 fill the chip).
 *   sink        device, 256 x 4 bytes, 4-byte aligned; written only if a
 *               workgroup's sum of accumulators equals a fixed constant that
 *               the sums never reach, which keeps the MFMAs live.
 * Returns W4A4_ERR_NULL, W4A4_ERR_SHAPE or W4A4_ERR_ALIGN for bad arguments;
 * enqueued on `stream`.
 */
w4a4_status w4a4_probe_mfma_fp4(const void* ops, int iters, int workgroups, void* sink, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* w4a4_last_error(void);

/* Library version string. */
const char* w4a4_version(void);

#ifdef __cplusplus
}
#endif

#endif  /* W4A4_H_ */
