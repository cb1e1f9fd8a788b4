// C ABI of libw4a4 (declared in include/w4a4.h): argument validation,
// thread-local error messages and dispatch to the gfx950 kernels.  Nothing
// here allocates device memory or synchronizes.
#include "w4a4.h"

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include "common.h"
#include "kernels.h"

static_assert(W4A4_NOALLOC_SCRATCH_BYTES == w4a4::kNoAllocScratchBytes, "scratch size");

namespace {

thread_local char g_err[512] = "";

w4a4_status fail(w4a4_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

w4a4_status ok() {
  g_err[0] = 0;
  return W4A4_OK;
}

bool valid_fmt(w4a4_format f) {
  return f == W4A4_MXFP4 || f == W4A4_NVFP4 || f == W4A4_MXINT4 || f == W4A4_MXFP8 ||
         f == W4A4_MXINT8;
}

// the 8-bit MX variants (one byte per code) run through quantize, pack and
// linear only
bool is_mx8(w4a4_format f) { return f == W4A4_MXFP8 || f == W4A4_MXINT8; }

w4a4_status not_for_mx8(const char* what) {
  return fail(W4A4_ERR_FORMAT, "%s: not available for the 8-bit MX formats", what);
}

// The integer formats with BF16 block scales have their own kernels: INT4
// with G = 64 (int4g64.hip) and INT8 with G = 128 (int8g128.hip)
bool is_i4(w4a4_format f) { return f == W4A4_INT4G64; }
bool is_i8(w4a4_format f) { return f == W4A4_INT8G128; }
bool is_bf16_int(w4a4_format f) { return is_i4(f) || is_i8(f); }
int64_t bf16_int_block(w4a4_format f) { return is_i4(f) ? 64 : 128; }
const char* bf16_int_name(w4a4_format f) { return is_i4(f) ? "INT4 G=64" : "INT8 G=128"; }
// canonical code bytes of a row of K elements
int64_t bf16_int_row_bytes(w4a4_format f, int64_t K) { return is_i4(f) ? K / 2 : K; }

w4a4_status check_int_shape(w4a4_format fmt, int64_t N, int64_t K) {
  const int64_t G = bf16_int_block(fmt);
  if (N <= 0 || K <= 0 || N % 16 || K % G || N > (int64_t(1) << 31) || K > (int64_t(1) << 31))
    return fail(W4A4_ERR_SHAPE, "%s: N=%lld K=%lld (need N > 0, N %% 16 == 0, K > 0, K %% %lld == 0)",
                bf16_int_name(fmt), (long long)N, (long long)K, (long long)G);
  return W4A4_OK;
}

w4a4_status not_for_int(w4a4_format fmt, const char* what) {
  return fail(W4A4_ERR_FORMAT, "%s: not available for %s (MX and NVFP4 formats only)", what,
              bf16_int_name(fmt));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

w4a4_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(W4A4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// (K % 128, N % 16) shapes of the packed GEMM
w4a4_status check_gemm_shape(w4a4_format fmt, int64_t N, int64_t K) {
  if (!valid_fmt(fmt)) return fail(W4A4_ERR_FORMAT, "unknown format %d", int(fmt));
  if (N <= 0 || K <= 0) return fail(W4A4_ERR_SHAPE, "N=%lld K=%lld must be positive",
                                    (long long)N, (long long)K);
  if (N % 16) return fail(W4A4_ERR_SHAPE, "N=%lld must be a multiple of 16", (long long)N);
  if (K % 128) return fail(W4A4_ERR_SHAPE, "K=%lld must be a multiple of 128", (long long)K);
  if (N > (int64_t(1) << 31) || K > (int64_t(1) << 31))
    return fail(W4A4_ERR_SHAPE, "N or K too large");
  return W4A4_OK;
}

}  // namespace

extern "C" {

int w4a4_block_size(w4a4_format fmt) {
  if (is_bf16_int(fmt)) return int(bf16_int_block(fmt));
  return valid_fmt(fmt) ? w4a4::block_size(fmt) : 0;
}

size_t w4a4_act_codes_bytes(w4a4_format fmt, int64_t M, int64_t K) {
  if (is_bf16_int(fmt))
    return (M < 0 || K <= 0 || K % bf16_int_block(fmt)) ? 0 : size_t(M) * size_t(bf16_int_row_bytes(fmt, K));
  if (!valid_fmt(fmt) || M < 0 || K <= 0 || K % w4a4::block_size(fmt)) return 0;
  return size_t(M) * size_t(w4a4::code_row_bytes(fmt, K));
}

size_t w4a4_act_scales_bytes(w4a4_format fmt, int64_t M, int64_t K) {
  if (is_bf16_int(fmt)) {
    const int64_t G = bf16_int_block(fmt);
    return (M < 0 || K <= 0 || K % G) ? 0 : size_t(M) * size_t(K / G) * 2;
  }
  if (!valid_fmt(fmt) || M < 0 || K <= 0 || K % w4a4::block_size(fmt)) return 0;
  return size_t(M) * size_t(K / w4a4::block_size(fmt));
}

size_t w4a4_quantize_workspace_bytes(w4a4_format fmt, int64_t, int64_t) {
  return fmt == W4A4_NVFP4 ? size_t(w4a4::kNvAmaxBlocks) * sizeof(float) : 0;
}

size_t w4a4_packed_weight_bytes(w4a4_format fmt, int64_t N, int64_t K) {
  if (is_bf16_int(fmt)) {
    if (check_int_shape(fmt, N, K) != W4A4_OK) return 0;
    return is_i4(fmt) ? w4a4::int4g64_packed_weight_bytes(N, K) : w4a4::int8g128_packed_weight_bytes(N, K);
  }
  if (check_gemm_shape(fmt, N, K) != W4A4_OK) return 0;
  return size_t(w4a4::blob_layout(fmt, N, K).total);
}

size_t w4a4_linear_workspace_bytes(w4a4_format fmt, int64_t M, int64_t N, int64_t K) {
  if (!valid_fmt(fmt)) return 0;
  return w4a4::linear_workspace_bytes(fmt, M, N, K);
}

w4a4_status w4a4_quantize_act(w4a4_format fmt, int64_t M, int64_t K, const void* X,
                              const float* c, void* codes, void* scales, float* t_act,
                              void* workspace, size_t ws_bytes, void* stream) {
  if (is_bf16_int(fmt)) {
    const int64_t G = bf16_int_block(fmt);
    if (M < 0 || K <= 0 || K % G)
      return fail(W4A4_ERR_SHAPE, "quantize_act: M=%lld K=%lld (need M >= 0, K > 0, K %% %lld == 0)",
                  (long long)M, (long long)K, (long long)G);
    if (M * K / 8 > (int64_t(1) << 40)) return fail(W4A4_ERR_SHAPE, "quantize_act: tensor too large");
    if (M > 0 && (!X || !codes || !scales))
      return fail(W4A4_ERR_NULL, "quantize_act: X, codes and scales must be non-NULL");
    const uintptr_t ca = is_i4(fmt) ? 4 : 8;   // one 4- or 8-byte store per 8 elements
    if (!aligned(X, 16) || (c && !aligned(c, 16)) || !aligned(codes, ca) || !aligned(scales, 2))
      return fail(W4A4_ERR_ALIGN, "quantize_act: X and c need 16-byte, codes %d-byte, scales 2-byte alignment",
                  int(ca));
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(is_i4(fmt) ? w4a4::launch_quantize_int4g64(M, K, X, c, codes, scales, s)
                                 : w4a4::launch_quantize_int8g128(M, K, X, c, codes, scales, s),
                      "quantize_act launch");
  }
  if (!valid_fmt(fmt)) return fail(W4A4_ERR_FORMAT, "unknown format %d", int(fmt));
  const int G = w4a4::block_size(fmt);
  if (M < 0 || K <= 0 || K % G)
    return fail(W4A4_ERR_SHAPE, "quantize_act: M=%lld K=%lld (need M >= 0, K > 0, K %% %d == 0)",
                (long long)M, (long long)K, G);
  if (M * K / 8 > (int64_t(1) << 40)) return fail(W4A4_ERR_SHAPE, "quantize_act: tensor too large");
  if (M > 0 && (!X || !codes || !scales))
    return fail(W4A4_ERR_NULL, "quantize_act: X, codes and scales must be non-NULL");
  if (fmt == W4A4_NVFP4) {
    if (!t_act) return fail(W4A4_ERR_NULL, "quantize_act: NVFP4 needs t_act");
    if (!workspace || ws_bytes < w4a4_quantize_workspace_bytes(fmt, M, K))
      return fail(W4A4_ERR_WORKSPACE, "quantize_act: NVFP4 needs %zu workspace bytes, got %zu",
                  w4a4_quantize_workspace_bytes(fmt, M, K), workspace ? ws_bytes : size_t(0));
    if (!aligned(workspace, 4) || !aligned(t_act, 4))
      return fail(W4A4_ERR_ALIGN, "quantize_act: workspace and t_act must be 4-byte aligned");
  }
  if (!aligned(X, 16) || (c && !aligned(c, 16)) || !aligned(codes, is_mx8(fmt) ? 8 : 4))
    return fail(W4A4_ERR_ALIGN,
                "quantize_act: X and c need 16-byte, codes 4-byte (8-bit formats: 8-byte) alignment");
  return hip_status(w4a4::launch_quantize_act(fmt, M, K, X, c, codes, scales, t_act, workspace,
                                              static_cast<hipStream_t>(stream)),
                    "quantize_act launch");
}

w4a4_status w4a4_quantize_act_multi(w4a4_format fmt, int64_t M, int64_t K, const void* X, int P,
                                    const float* const* c, void* const* codes,
                                    void* const* scales, float* const* t_act, void* workspace,
                                    size_t ws_bytes, void* stream) {
  if (is_bf16_int(fmt)) return not_for_int(fmt, "quantize_act_multi");
  if (is_mx8(fmt)) return not_for_mx8("quantize_act_multi");
  if (!valid_fmt(fmt)) return fail(W4A4_ERR_FORMAT, "unknown format %d", int(fmt));
  const int G = w4a4::block_size(fmt);
  if (M < 0 || K <= 0 || K % G || P < 1 || P > w4a4::kMaxOutputs)
    return fail(W4A4_ERR_SHAPE,
                "quantize_act_multi: M=%lld K=%lld P=%d (need M >= 0, K > 0, K %% %d == 0, "
                "1 <= P <= %d)",
                (long long)M, (long long)K, P, G, w4a4::kMaxOutputs);
  if (M * K / 8 > (int64_t(1) << 40)) return fail(W4A4_ERR_SHAPE, "quantize_act_multi: tensor too large");
  if (!c || !codes || !scales || (fmt == W4A4_NVFP4 && !t_act))
    return fail(W4A4_ERR_NULL, "quantize_act_multi: the pointer arrays must be non-NULL");
  for (int p = 0; p < P; ++p) {
    if (!c[p] || (M > 0 && (!X || !codes[p] || !scales[p])) || (fmt == W4A4_NVFP4 && !t_act[p]))
      return fail(W4A4_ERR_NULL, "quantize_act_multi: output %d has a NULL pointer", p);
    if (!aligned(c[p], 16) || !aligned(codes[p], 4) || (fmt == W4A4_NVFP4 && !aligned(t_act[p], 4)))
      return fail(W4A4_ERR_ALIGN, "quantize_act_multi: c needs 16-byte, codes/t_act 4-byte alignment");
  }
  if (!aligned(X, 16)) return fail(W4A4_ERR_ALIGN, "quantize_act_multi: X needs 16-byte alignment");
  if (fmt == W4A4_NVFP4) {
    const size_t need = size_t(P) * w4a4_quantize_workspace_bytes(fmt, M, K);
    if (!workspace || ws_bytes < need)
      return fail(W4A4_ERR_WORKSPACE, "quantize_act_multi: NVFP4 needs %zu workspace bytes, got %zu",
                  need, workspace ? ws_bytes : size_t(0));
    if (!aligned(workspace, 4)) return fail(W4A4_ERR_ALIGN, "quantize_act_multi: workspace 4-byte alignment");
  }
  return hip_status(w4a4::launch_quantize_act_multi(fmt, M, K, X, P, c, codes, scales, t_act,
                                                    workspace, static_cast<hipStream_t>(stream)),
                    "quantize_act_multi launch");
}

w4a4_status w4a4_pack_weight(w4a4_format fmt, int64_t N, int64_t K, const void* codes,
                             const void* scales, const float* t_w, const float* r, void* blob,
                             void* stream) {
  if (is_bf16_int(fmt)) {
    w4a4_status st = check_int_shape(fmt, N, K);
    if (st != W4A4_OK) return st;
    if (!codes || !scales || !r || !blob)
      return fail(W4A4_ERR_NULL, "pack_weight: codes, scales, r and blob must be non-NULL");
    if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(blob, 256) || !aligned(r, 4))
      return fail(W4A4_ERR_ALIGN, "pack_weight: codes 16-byte, scales 2-byte, blob 256-byte, r 4-byte alignment");
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(is_i4(fmt) ? w4a4::launch_pack_int4g64(N, K, codes, scales, r, blob, s)
                                 : w4a4::launch_pack_int8g128(N, K, codes, scales, r, blob, s),
                      "pack_weight launch");
  }
  w4a4_status st = check_gemm_shape(fmt, N, K);
  if (st != W4A4_OK) return st;
  if (!codes || !scales || !r || !blob)
    return fail(W4A4_ERR_NULL, "pack_weight: codes, scales, r and blob must be non-NULL");
  if (!aligned(codes, 16) || !aligned(blob, 256) || !aligned(r, 4) || (t_w && !aligned(t_w, 4)))
    return fail(W4A4_ERR_ALIGN, "pack_weight: codes 16-byte, blob 256-byte, r/t_w 4-byte alignment");
  return hip_status(w4a4::launch_pack_weight(fmt, N, K, codes, scales, t_w, r, blob,
                                             static_cast<hipStream_t>(stream)),
                    "pack_weight launch");
}

w4a4_status w4a4_unpack_weight(w4a4_format fmt, int64_t N, int64_t K, const void* blob,
                               void* codes, void* scales, float* r, float* t_w, void* stream) {
  if (is_bf16_int(fmt)) {
    w4a4_status st = check_int_shape(fmt, N, K);
    if (st != W4A4_OK) return st;
    if (!blob) return fail(W4A4_ERR_NULL, "unpack_weight: blob must be non-NULL");
    if (!aligned(blob, 256) || (codes && !aligned(codes, 16)) || (scales && !aligned(scales, 2)) ||
        (r && !aligned(r, 4)) || (t_w && !aligned(t_w, 4)))
      return fail(W4A4_ERR_ALIGN, "unpack_weight: blob 256-byte, codes 16-byte, scales 2-byte, r/t_w 4-byte alignment");
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(is_i4(fmt) ? w4a4::launch_unpack_int4g64(N, K, blob, codes, scales, r, t_w, s)
                                 : w4a4::launch_unpack_int8g128(N, K, blob, codes, scales, r, t_w, s),
                      "unpack_weight launch");
  }
  w4a4_status st = check_gemm_shape(fmt, N, K);
  if (st != W4A4_OK) return st;
  if (!blob) return fail(W4A4_ERR_NULL, "unpack_weight: blob must be non-NULL");
  if (!aligned(blob, 256) || (codes && !aligned(codes, 16)) || (r && !aligned(r, 4)) ||
      (t_w && !aligned(t_w, 4)))
    return fail(W4A4_ERR_ALIGN, "unpack_weight: blob 256-byte, codes 16-byte, r/t_w 4-byte alignment");
  return hip_status(w4a4::launch_unpack_weight(fmt, N, K, blob, codes, scales, r, t_w,
                                               static_cast<hipStream_t>(stream)),
                    "unpack_weight launch");
}

w4a4_status w4a4_linear(w4a4_format fmt, int64_t M, int64_t N, int64_t K, const void* a_codes,
                        const void* a_scales, const float* t_act, const void* blob, void* Y,
                        void* workspace, size_t ws_bytes, void* stream) {
  if (is_bf16_int(fmt)) {
    w4a4_status st = check_int_shape(fmt, N, K);
    if (st != W4A4_OK) return st;
    if (M < 0 || M > (int64_t(1) << 31)) return fail(W4A4_ERR_SHAPE, "linear: M=%lld out of range", (long long)M);
    if (M == 0) return ok();
    if (!a_codes || !a_scales || !blob || !Y)
      return fail(W4A4_ERR_NULL, "linear: a_codes, a_scales, blob and Y must be non-NULL");
    if (!aligned(a_codes, 16) || !aligned(a_scales, 16) || !aligned(blob, 256) || !aligned(Y, 16))
      return fail(W4A4_ERR_ALIGN, "linear: a_codes/a_scales/Y need 16-byte, blob 256-byte alignment");
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(is_i4(fmt) ? w4a4::launch_linear_int4g64(M, N, K, a_codes, a_scales, blob, Y, s)
                                 : w4a4::launch_linear_int8g128(M, N, K, a_codes, a_scales, blob, Y, s),
                      "linear launch");
  }
  w4a4_status st = check_gemm_shape(fmt, N, K);
  if (st != W4A4_OK) return st;
  if (M < 0 || M > (int64_t(1) << 31)) return fail(W4A4_ERR_SHAPE, "linear: M=%lld out of range", (long long)M);
  if (M == 0) return ok();
  if (!a_codes || !a_scales || !blob || !Y)
    return fail(W4A4_ERR_NULL, "linear: a_codes, a_scales, blob and Y must be non-NULL");
  if (fmt == W4A4_NVFP4 && !t_act) return fail(W4A4_ERR_NULL, "linear: NVFP4 needs t_act");
  const size_t need = w4a4_linear_workspace_bytes(fmt, M, N, K);
  if (need && (!workspace || ws_bytes < need))
    return fail(W4A4_ERR_WORKSPACE, "linear: needs %zu workspace bytes, got %zu", need,
                workspace ? ws_bytes : size_t(0));
  if (!aligned(a_codes, 16) || !aligned(a_scales, 16) || !aligned(blob, 256) || !aligned(Y, 16) ||
      (t_act && !aligned(t_act, 4)) || (need && !aligned(workspace, 16)))
    return fail(W4A4_ERR_ALIGN,
                "linear: a_codes/a_scales/Y/workspace need 16-byte, blob 256-byte, t_act 4-byte "
                "alignment");
  return hip_status(w4a4::launch_linear(fmt, M, N, K, a_codes, a_scales, t_act, blob, Y, workspace,
                                        ws_bytes, static_cast<hipStream_t>(stream)),
                    "linear launch");
}

w4a4_status w4a4_linear_noalloc(w4a4_format fmt, int64_t M, int64_t N, int64_t K,
                                const void* a_codes, const void* a_scales, const float* t_act,
                                const void* blob, void* Y, void* stream) {
  if (is_bf16_int(fmt)) return not_for_int(fmt, "linear_noalloc");
  w4a4_status st = check_gemm_shape(fmt, N, K);
  if (st != W4A4_OK) return st;
  if (M < 0 || M > (int64_t(1) << 31))
    return fail(W4A4_ERR_SHAPE, "linear_noalloc: M=%lld out of range", (long long)M);
  if (M == 0) return ok();
  if (!a_codes || !a_scales || !blob || !Y)
    return fail(W4A4_ERR_NULL, "linear_noalloc: a_codes, a_scales, blob and Y must be non-NULL");
  if (fmt == W4A4_NVFP4 && !t_act) return fail(W4A4_ERR_NULL, "linear_noalloc: NVFP4 needs t_act");
  const size_t need = w4a4_linear_workspace_bytes(fmt, M, N, K);
  if (need > w4a4::kNoAllocScratchBytes)
    return fail(W4A4_ERR_WORKSPACE, "linear_noalloc: needs %zu scratch bytes, the maximum is %zu",
                need, w4a4::kNoAllocScratchBytes);
  if (!aligned(a_codes, 16) || !aligned(a_scales, 16) || !aligned(blob, 256) || !aligned(Y, 16) ||
      (t_act && !aligned(t_act, 4)))
    return fail(W4A4_ERR_ALIGN,
                "linear_noalloc: a_codes/a_scales/Y need 16-byte, blob 256-byte, t_act 4-byte "
                "alignment");
  return hip_status(w4a4::launch_linear_noalloc(fmt, M, N, K, a_codes, a_scales, t_act, blob, Y,
                                                static_cast<hipStream_t>(stream)),
                    "linear_noalloc");
}

w4a4_status w4a4_linear_grouped(w4a4_format fmt, int P, int64_t M, int64_t K, const int64_t* N,
                                const void* const* a_codes, const void* const* a_scales,
                                const float* const* t_act, const void* const* blobs,
                                void* const* Y, void* stream) {
  if (is_bf16_int(fmt)) return not_for_int(fmt, "linear_grouped");
  if (is_mx8(fmt)) return not_for_mx8("linear_grouped");
  if (!valid_fmt(fmt)) return fail(W4A4_ERR_FORMAT, "unknown format %d", int(fmt));
  if (P < 1 || P > w4a4::kMaxGroup || M < 0)
    return fail(W4A4_ERR_SHAPE, "linear_grouped: P=%d M=%lld (need 1 <= P <= %d, M >= 0)", P,
                (long long)M, w4a4::kMaxGroup);
  if (!N || !a_codes || !a_scales || !blobs || !Y || (fmt == W4A4_NVFP4 && !t_act))
    return fail(W4A4_ERR_NULL, "linear_grouped: the arrays must be non-NULL");
  for (int p = 0; p < P; ++p) {
    w4a4_status st = check_gemm_shape(fmt, N[p], K);
    if (st != W4A4_OK) return st;
    if (M == 0) continue;
    if (!a_codes[p] || !a_scales[p] || !blobs[p] || !Y[p] || (fmt == W4A4_NVFP4 && !t_act[p]))
      return fail(W4A4_ERR_NULL, "linear_grouped: problem %d has a NULL pointer", p);
    if (!aligned(a_codes[p], 16) || !aligned(a_scales[p], 16) || !aligned(Y[p], 16) ||
        !aligned(blobs[p], 256) || (fmt == W4A4_NVFP4 && !aligned(t_act[p], 4)))
      return fail(W4A4_ERR_ALIGN,
                  "linear_grouped: a_codes/a_scales/Y need 16-byte, blob 256-byte, t_act 4-byte "
                  "alignment");
  }
  return hip_status(w4a4::launch_linear_grouped(fmt, P, M, K, N, a_codes, a_scales, t_act, blobs,
                                                Y, static_cast<hipStream_t>(stream)),
                    "linear_grouped launch");
}

size_t w4a4_dualquant_workspace_bytes(w4a4_format fmt, int64_t N, int64_t K) {
  if (!valid_fmt(fmt) || is_mx8(fmt) || N <= 0 || K <= 0 || K % 32 ||
      N * K > (int64_t(1) << 36))
    return 0;
  return w4a4::solver_workspace_bytes(N, K);
}

w4a4_status w4a4_dualquant_solve(w4a4_format fmt, int64_t N, int64_t K, const float* W, int iters,
                                 float* r, float* c, void* codes, void* scales, float* t_w,
                                 void* workspace, size_t ws_bytes, void* stream) {
  if (is_bf16_int(fmt)) return not_for_int(fmt, "dualquant_solve");
  if (is_mx8(fmt)) return not_for_mx8("dualquant_solve");
  if (!valid_fmt(fmt)) return fail(W4A4_ERR_FORMAT, "unknown format %d", int(fmt));
  if (N <= 0 || K <= 0 || K % 32 || N * K > (int64_t(1) << 36) || iters < 1)
    return fail(W4A4_ERR_SHAPE,
                "dualquant_solve: N=%lld K=%lld iters=%d (need N > 0, K > 0, K %% 32 == 0, "
                "N*K <= 2^36, iters >= 1)",
                (long long)N, (long long)K, iters);
  if (!W || !r || !c || !codes || !scales || (fmt == W4A4_NVFP4 && !t_w))
    return fail(W4A4_ERR_NULL,
                "dualquant_solve: W, r, c, codes, scales (and t_w for NVFP4) must be non-NULL");
  const size_t need = w4a4::solver_workspace_bytes(N, K);
  if (!workspace || ws_bytes < need)
    return fail(W4A4_ERR_WORKSPACE, "dualquant_solve: needs %zu workspace bytes, got %zu", need,
                workspace ? ws_bytes : size_t(0));
  if (!aligned(W, 16) || !aligned(r, 4) || !aligned(c, 4) || !aligned(codes, 4) ||
      (t_w && !aligned(t_w, 4)) || !aligned(workspace, 256))
    return fail(W4A4_ERR_ALIGN,
                "dualquant_solve: W 16-byte, r/c/codes/t_w 4-byte, workspace 256-byte alignment");
  return hip_status(w4a4::launch_dualquant_solve(fmt, N, K, W, iters, r, c, codes, scales, t_w,
                                                 workspace, static_cast<hipStream_t>(stream)),
                    "dualquant_solve launch");
}

w4a4_status w4a4_probe_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return fail(W4A4_ERR_NULL, "probe_stream_read: src and sink must be non-NULL");
  if (bytes == 0 || bytes % 16) return fail(W4A4_ERR_SHAPE, "probe_stream_read: bytes must be a positive multiple of 16");
  if (!aligned(src, 16) || !aligned(sink, 4)) return fail(W4A4_ERR_ALIGN, "probe_stream_read: src 16-byte, sink 4-byte alignment");
  return hip_status(w4a4::launch_stream_read(src, int64_t(bytes), sink, static_cast<hipStream_t>(stream)),
                    "probe_stream_read launch");
}

w4a4_status w4a4_probe_mfma_fp4(const void* ops, int iters, int workgroups, void* sink, void* stream) {
  if (!ops || !sink) return fail(W4A4_ERR_NULL, "probe_mfma_fp4: ops and sink must be non-NULL");
  if (iters < 2 || iters > (1 << 20) || iters % 2) return fail(W4A4_ERR_SHAPE, "probe_mfma_fp4: iters must be even, 2 .. 2^20");
  if (workgroups < 1 || workgroups > 4096) return fail(W4A4_ERR_SHAPE, "probe_mfma_fp4: workgroups must be 1 .. 4096");
  if (!aligned(ops, 16) || !aligned(sink, 4)) return fail(W4A4_ERR_ALIGN, "probe_mfma_fp4: ops 16-byte, sink 4-byte alignment");
  return hip_status(w4a4::launch_mfma_fp4(ops, iters, workgroups, sink, static_cast<hipStream_t>(stream)),
                    "probe_mfma_fp4 launch");
}

w4a4_status w4a4_probe_empty(void* stream) {
  return hip_status(w4a4::launch_empty(static_cast<hipStream_t>(stream)), "probe_empty launch");
}

const char* w4a4_last_error(void) { return g_err; }

const char* w4a4_version(void) { return "w4a4 1.0 gfx950"; }

}  // extern "C"
