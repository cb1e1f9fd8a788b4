// Host-side launchers of the gfx950 kernels (internal to libw4a4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace w4a4 {

// NVFP4 tensor-amax pre-pass: at most this many partial maxima (4 bytes each)
// live in the quantize workspace.
constexpr int kNvAmaxBlocks = 1024;

hipError_t launch_quantize_act(int fmt, int64_t M, int64_t K, const void* X, const float* c,
                               void* codes, void* scales, float* t_act, void* workspace,
                               hipStream_t stream);

// One X quantized under up to kMaxOutputs column-scale vectors (X read once).
constexpr int kMaxOutputs = 4;

hipError_t launch_quantize_act_multi(int fmt, int64_t M, int64_t K, const void* X, int P,
                                     const float* const* c, void* const* codes,
                                     void* const* scales, float* const* t_act, void* workspace,
                                     hipStream_t stream);

hipError_t launch_pack_weight(int fmt, int64_t N, int64_t K, const void* codes,
                              const void* scales, const float* t_w, const float* r, void* blob,
                              hipStream_t stream);

hipError_t launch_unpack_weight(int fmt, int64_t N, int64_t K, const void* blob, void* codes,
                                void* scales, float* r, float* t_w, hipStream_t stream);

hipError_t launch_linear(int fmt, int64_t M, int64_t N, int64_t K, const void* a_codes,
                         const void* a_scales, const float* t_act, const void* blob, void* Y,
                         void* workspace, size_t ws_bytes, hipStream_t stream);

size_t linear_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K);

// The allocation-free linear: the split-K workspace (the only scratch of
// w4a4_linear) lives in a device array of the library of this many bytes,
// one per device (the largest split-K workspace: the status block plus 128
// tiles of 256 KiB).
constexpr size_t kNoAllocScratchBytes = size_t(4352) + size_t(128) * 4 * 65536;

hipError_t launch_linear_noalloc(int fmt, int64_t M, int64_t N, int64_t K, const void* a_codes,
                                 const void* a_scales, const float* t_act, const void* blob,
                                 void* Y, hipStream_t stream);

// Up to kMaxGroup linears of one M and K (per-projection linears of a fused
// input): one launch where that pays (MXFP4, M > 32, unless every problem
// takes the persistent kernel on its own), else one after another.
constexpr int kMaxGroup = 4;

hipError_t launch_linear_grouped(int fmt, int P, int64_t M, int64_t K, const int64_t* N,
                                 const void* const* a_codes, const void* const* a_scales,
                                 const float* const* t_act, const void* const* blobs,
                                 void* const* Y, hipStream_t stream);

// DualQuant's dual-scale solver: workspace bytes and launch.
size_t solver_workspace_bytes(int64_t N, int64_t K);

hipError_t launch_dualquant_solve(int fmt, int64_t N, int64_t K, const float* W, int iters,
                                  float* r, float* c, void* codes, void* scales, float* t_w,
                                  void* workspace, hipStream_t stream);

// INT4 with G = 64 and BF16 block scales (int4g64.hip): canonical codes
// [rows x K/2], scales [rows x K/64] BF16 bit patterns.
size_t int4g64_packed_weight_bytes(int64_t N, int64_t K);

hipError_t launch_quantize_int4g64(int64_t M, int64_t K, const void* X, const float* c,
                                   void* codes, void* scales, hipStream_t stream);

hipError_t launch_pack_int4g64(int64_t N, int64_t K, const void* codes, const void* scales,
                               const float* r, void* blob, hipStream_t stream);

hipError_t launch_unpack_int4g64(int64_t N, int64_t K, const void* blob, void* codes, void* scales,
                                 float* r, float* t_w, hipStream_t stream);

hipError_t launch_linear_int4g64(int64_t M, int64_t N, int64_t K, const void* a_codes,
                                 const void* a_scales, const void* blob, void* Y,
                                 hipStream_t stream);

// INT8 with G = 128 and BF16 block scales (int8g128.hip): canonical codes
// [rows x K] int8, scales [rows x K/128] BF16 bit patterns.
size_t int8g128_packed_weight_bytes(int64_t N, int64_t K);

hipError_t launch_quantize_int8g128(int64_t M, int64_t K, const void* X, const float* c,
                                    void* codes, void* scales, hipStream_t stream);

hipError_t launch_pack_int8g128(int64_t N, int64_t K, const void* codes, const void* scales,
                                const float* r, void* blob, hipStream_t stream);

hipError_t launch_unpack_int8g128(int64_t N, int64_t K, const void* blob, void* codes, void* scales,
                                  float* r, float* t_w, hipStream_t stream);

hipError_t launch_linear_int8g128(int64_t M, int64_t N, int64_t K, const void* a_codes,
                                  const void* a_scales, const void* blob, void* Y,
                                  hipStream_t stream);

// Measurement aids (probe.hip): a streaming read of `bytes` (a multiple of
// 16), an empty kernel, and `iters` (even) rounds of 16 scaled FP4 MFMAs per
// wave on register operands from `ops` (16 KiB) over `workgroups` workgroups
// of 4 waves.
hipError_t launch_stream_read(const void* src, int64_t bytes, void* sink, hipStream_t stream);
hipError_t launch_empty(hipStream_t stream);
hipError_t launch_mfma_fp4(const void* ops, int iters, int workgroups, void* sink, hipStream_t stream);

}  // namespace w4a4
