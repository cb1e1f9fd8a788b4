"""C-ABI checks that need no GPU: the library loads, exports every function
include/w4a4.h declares, answers size queries, and rejects invalid arguments
on the host before anything is enqueued."""
import ctypes
import os
import re

import pytest

import w4a4_block_scaled_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a4.h")

pytestmark = pytest.mark.skipif(not os.path.exists(w4.library_path()),
                                reason="libw4a4.so not built (python -m w4a4_block_scaled_amd.build)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a4_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("w4a4_quantize_act", "w4a4_pack_weight", "w4a4_linear"):
        assert n in names


def test_library_exports_every_declared_function():
    L = w4.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_version_and_block_sizes():
    L = w4.lib()
    assert L.w4a4_version().decode().startswith("w4a4")
    assert [L.w4a4_block_size(f) for f in (0, 1, 2, 7)] == [32, 16, 32, 0]


def test_size_queries():
    L = w4.lib()
    assert L.w4a4_act_codes_bytes(0, 2048, 4096) == 2048 * 2048
    assert L.w4a4_act_scales_bytes(0, 2048, 4096) == 2048 * 128
    assert L.w4a4_act_scales_bytes(1, 2048, 4096) == 2048 * 256
    assert L.w4a4_act_codes_bytes(0, 3, 33) == 0                 # K % G
    assert L.w4a4_quantize_workspace_bytes(1, 16, 256) >= 4
    assert L.w4a4_quantize_workspace_bytes(0, 16, 256) == 0
    for fmt, G in ((0, 32), (1, 16), (2, 32)):
        N, K = 28672, 4096
        total = L.w4a4_packed_weight_bytes(fmt, N, K)
        payload = N * K // 2 + N * K // G + 4 * N
        assert payload <= total <= payload + 4 * 256 + (N // 16) * 64 * 4 * 1
    assert L.w4a4_packed_weight_bytes(0, 100, 4096) == 0          # N % 16
    assert L.w4a4_packed_weight_bytes(0, 128, 4000) == 0          # K % 128


def split_k(M, N, K):
    """The host-side condition of the MXFP4 split-K GEMM: 64..128 tiles of
    256 x 256 and K a multiple of 1024, at least 8192."""
    T = ((N + 255) // 256) * ((M + 255) // 256)
    return M > 32 and K % 1024 == 0 and K >= 8192 and 64 <= T <= 128


def test_linear_workspace_sizes():
    """Only the MXFP4 split-K GEMM needs scratch: a fixed 4 KiB block of
    tickets and flags (8 bytes per wave slot of up to 128 tiles) and a
    256-byte status block, then per tile 4 wave slots of 64 KiB of fp32
    partial sums."""
    L = w4.lib()
    shapes = ((2048, 28672, 4096), (2048, 4096, 14336), (2048, 4096, 4096), (16, 4096, 4096),
              (2048, 6144, 4096), (300, 8208, 8192), (2048, 4096, 9216))
    for fmt in (0, 1, 2):
        for M, N, K in shapes:
            got = L.w4a4_linear_workspace_bytes(fmt, M, N, K)
            if fmt == 0 and split_k(M, N, K):
                T = ((N + 255) // 256) * ((M + 255) // 256)
                assert got == 4096 + 256 + T * 4 * 65536, (M, N, K)
            else:
                assert got == 0, (fmt, M, N, K)
    assert split_k(2048, 4096, 14336) and not split_k(2048, 4096, 4096) and not split_k(2048, 6144, 14336)


def test_table12_scale_bytes_from_the_library():
    """Llama-3.1-8B's 224 linears: the MXFP4 blob payload is 3.49 GB of codes
    plus 0.22 GB of scales (Appendix I, Table 12 byte counts)."""
    L = w4.lib()
    shapes = [(6144, 4096), (4096, 4096), (28672, 4096), (4096, 14336)]
    total = sum(L.w4a4_packed_weight_bytes(0, N, K) for N, K in shapes) * 32
    codes = sum(L.w4a4_act_codes_bytes(0, N, K) for N, K in shapes) * 32
    scales = sum(L.w4a4_act_scales_bytes(0, N, K) for N, K in shapes) * 32
    assert round(codes / 1e9, 2) == 3.49 and round(scales / 1e9, 2) == 0.22
    assert total - codes - scales < 0.01e9      # header, r and padding stay small


FAKE = ctypes.c_void_p(1 << 20)        # never dereferenced: validation fails first
FAKE_MIS = ctypes.c_void_p((1 << 20) + 2)


@pytest.mark.parametrize("args,status", [
    ((9, 16, 256, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, None), 4),       # format
    ((0, -1, 256, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None), 2),          # M < 0
    ((0, 16, 250, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None), 2),          # K % 32
    ((1, 16, 264, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None), 2),          # K % 16
    ((0, 16, 256, None, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None), 1),          # X NULL
    ((0, 16, 256, FAKE_MIS, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None), 3),      # X misaligned
    ((1, 16, 256, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None), 5),          # NVFP4 workspace
    ((1, 16, 256, FAKE, FAKE, FAKE, FAKE, None, FAKE, 4096, None), 1),       # NVFP4 t_act
])
def test_quantize_act_rejects(args, status):
    L = w4.lib()
    assert L.w4a4_quantize_act(*args) == status
    assert L.w4a4_last_error().decode()


@pytest.mark.parametrize("args,status", [
    ((0, 100, 256, FAKE, FAKE, None, FAKE, FAKE, None), 2),     # N % 16
    ((0, 128, 200, FAKE, FAKE, None, FAKE, FAKE, None), 2),     # K % 128
    ((0, 128, 256, None, FAKE, None, FAKE, FAKE, None), 1),
    ((0, 128, 256, FAKE, FAKE, None, FAKE, ctypes.c_void_p((1 << 20) + 16), None), 3),  # blob 256-B
    ((9, 128, 256, FAKE, FAKE, None, FAKE, FAKE, None), 4),
])
def test_pack_weight_rejects(args, status):
    assert w4.lib().w4a4_pack_weight(*args) == status


@pytest.mark.parametrize("args,status", [
    ((0, -2, 128, 256, FAKE, FAKE, None, FAKE, FAKE, None, 0, None), 2),
    ((0, 4, 120, 256, FAKE, FAKE, None, FAKE, FAKE, None, 0, None), 2),
    ((0, 4, 128, 200, FAKE, FAKE, None, FAKE, FAKE, None, 0, None), 2),
    ((0, 4, 128, 256, FAKE, None, None, FAKE, FAKE, None, 0, None), 1),
    ((1, 4, 128, 256, FAKE, FAKE, None, FAKE, FAKE, None, 0, None), 1),     # NVFP4 t_act
    ((0, 4, 128, 256, FAKE, FAKE, None, FAKE, FAKE_MIS, None, 0, None), 3),
])
def test_linear_rejects(args, status):
    assert w4.lib().w4a4_linear(*args) == status


def test_linear_split_k_workspace_checks():
    """The split-K MXFP4 shape (2048 x 4096 x 14336) needs its workspace: a
    missing or short one is rejected (W4A4_ERR_WORKSPACE), a misaligned one
    too (W4A4_ERR_ALIGN), before anything is launched."""
    L = w4.lib()
    M, N, K = 2048, 4096, 14336
    need = L.w4a4_linear_workspace_bytes(0, M, N, K)
    assert need > 0
    base = (0, M, N, K, FAKE, FAKE, None, FAKE, FAKE)
    assert L.w4a4_linear(*base, None, need, None) == 5
    assert L.w4a4_linear(*base, FAKE, need - 1, None) == 5
    assert "workspace" in L.w4a4_last_error().decode()
    assert L.w4a4_linear(*base, FAKE_MIS, need, None) == 3


def test_empty_linear_is_a_no_op():
    # M = 0 returns OK without touching the pointers or the device
    assert w4.lib().w4a4_linear(0, 0, 128, 256, None, None, None, None, None, None, 0, None) == 0


def test_dualquant_workspace_bytes():
    """fp64 partial sums per (row, 32-block) and per (16-row chunk, column),
    two of each, the current and the previous iteration's fp32 scales, 1024
    partial maxima, the tensor scale (NVFP4) and the fixed-point flag, each
    256-byte aligned."""
    L = w4.lib()

    def a256(x):
        return (x + 255) // 256 * 256

    for N, K in [(64, 256), (100, 4096), (4096, 14336)]:
        want = (2 * a256(N * (K // 32) * 8) + 2 * a256((N + 15) // 16 * K * 8) + 2 * a256(4 * N) +
                2 * a256(4 * K) + 4096 + 256)
        for fmt in (0, 1, 2):
            assert L.w4a4_dualquant_workspace_bytes(fmt, N, K) == want
    assert L.w4a4_dualquant_workspace_bytes(9, 64, 256) == 0      # unknown format
    assert L.w4a4_dualquant_workspace_bytes(0, 64, 48) == 0       # K % 32
    assert L.w4a4_dualquant_workspace_bytes(0, 0, 256) == 0


@pytest.mark.parametrize("args,status", [
    ((9, 64, 256, FAKE, 15, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None), 4),      # format
    ((0, 64, 48, FAKE, 15, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None), 2),       # K % 32
    ((1, 64, 48, FAKE, 15, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None), 2),       # NVFP4 K % 32
    ((0, 64, 256, FAKE, 0, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None), 2),       # iters < 1
    ((0, 64, 256, None, 15, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None), 1),      # W NULL
    ((1, 64, 256, FAKE, 15, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None), 1),      # NVFP4 t_w
    ((0, 64, 256, FAKE, 15, FAKE, FAKE, FAKE, FAKE, None, None, 1 << 30, None), 5),      # no workspace
    ((0, 64, 256, FAKE, 15, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1024, None), 5),         # short
    ((0, 64, 256, FAKE_MIS, 15, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None), 3),  # W 16-byte
])
def test_dualquant_solve_rejects(args, status):
    L = w4.lib()
    assert L.w4a4_dualquant_solve(*args) == status
    assert L.w4a4_last_error().decode()


def test_quantize_act_multi_rejects():
    L = w4.lib()
    arr = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    nul = (ctypes.c_void_p * 4)(FAKE, None, FAKE, FAKE)
    base = (0, 16, 256, FAKE)
    assert L.w4a4_quantize_act_multi(*base, 0, arr, arr, arr, None, None, 0, None) == 2    # P < 1
    assert L.w4a4_quantize_act_multi(*base, 5, arr, arr, arr, None, None, 0, None) == 2    # P > 4
    assert L.w4a4_quantize_act_multi(*base, 2, None, arr, arr, None, None, 0, None) == 1   # arrays
    assert L.w4a4_quantize_act_multi(*base, 2, nul, arr, arr, None, None, 0, None) == 1    # c[1]
    assert L.w4a4_quantize_act_multi(9, 16, 256, FAKE, 2, arr, arr, arr, None, None, 0, None) == 4
    nv = (1, 16, 256, FAKE, 2, arr, arr, arr)
    assert L.w4a4_quantize_act_multi(*nv, None, FAKE, 1 << 20, None) == 1                  # t_act
    assert L.w4a4_quantize_act_multi(*nv, arr, None, 0, None) == 5                         # workspace
    need = 2 * L.w4a4_quantize_workspace_bytes(1, 16, 256)
    assert L.w4a4_quantize_act_multi(*nv, arr, FAKE, need - 1, None) == 5
    mis = (ctypes.c_void_p * 4)(FAKE_MIS, FAKE, FAKE, FAKE)
    assert L.w4a4_quantize_act_multi(*base, 2, mis, arr, arr, None, None, 0, None) == 3    # c align


def test_linear_grouped_rejects():
    L = w4.lib()
    arr = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    Ns = (ctypes.c_int64 * 4)(256, 128, 128, 64)
    bad_n = (ctypes.c_int64 * 4)(256, 100, 128, 64)
    assert L.w4a4_linear_grouped(0, 0, 64, 256, Ns, arr, arr, None, arr, arr, None) == 2   # P < 1
    assert L.w4a4_linear_grouped(0, 5, 64, 256, Ns, arr, arr, None, arr, arr, None) == 2   # P > 4
    assert L.w4a4_linear_grouped(0, 2, 64, 256, None, arr, arr, None, arr, arr, None) == 1
    assert L.w4a4_linear_grouped(0, 2, 64, 256, bad_n, arr, arr, None, arr, arr, None) == 2  # N % 16
    assert L.w4a4_linear_grouped(1, 2, 64, 256, Ns, arr, arr, None, arr, arr, None) == 1   # NVFP4 t_act
    assert L.w4a4_linear_grouped(7, 2, 64, 256, Ns, arr, arr, None, arr, arr, None) == 4


def test_int4g64_size_queries():
    """INT4 G=64 with BF16 scales: G = 64, two scale bytes per block (as many
    as E8M0 at G = 32), K % 64 suffices, no workspaces."""
    L = w4.lib()
    assert L.w4a4_block_size(3) == 64
    assert L.w4a4_act_codes_bytes(3, 5, 192) == 5 * 96
    assert L.w4a4_act_scales_bytes(3, 5, 192) == 5 * 3 * 2
    assert L.w4a4_act_scales_bytes(3, 7, 4096) == L.w4a4_act_scales_bytes(0, 7, 4096)
    assert L.w4a4_act_scales_bytes(3, 5, 96) == 0                  # K % 64
    assert L.w4a4_quantize_workspace_bytes(3, 5, 192) == 0
    assert L.w4a4_linear_workspace_bytes(3, 2048, 4096, 4096) == 0

    def a256(x):
        return (x + 255) // 256 * 256

    for N, K in [(16, 64), (48, 192), (4096, 14336)]:
        assert L.w4a4_packed_weight_bytes(3, N, K) == a256(a256(256 + N * K // 2) + N * K // 64 * 2) + a256(4 * N)
    assert L.w4a4_packed_weight_bytes(3, 24, 192) == 0              # N % 16
    assert L.w4a4_packed_weight_bytes(3, 16, 96) == 0               # K % 64
    assert L.w4a4_dualquant_workspace_bytes(3, 64, 256) == 0        # no solver for this format


def test_int4g64_rejects():
    L = w4.lib()
    arr = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    n = (ctypes.c_int64 * 4)(64, 64, 64, 64)
    # quantize_act: K % 64, NULL X, misaligned X
    assert L.w4a4_quantize_act(3, 4, 96, FAKE, None, FAKE, FAKE, None, None, 0, None) == 2
    assert L.w4a4_quantize_act(3, 4, 128, None, None, FAKE, FAKE, None, None, 0, None) == 1
    assert L.w4a4_quantize_act(3, 4, 128, FAKE_MIS, None, FAKE, FAKE, None, None, 0, None) == 3
    # pack / linear: N % 16, K % 64, NULL r, misaligned blob
    assert L.w4a4_pack_weight(3, 24, 128, FAKE, FAKE, None, FAKE, FAKE, None) == 2
    assert L.w4a4_pack_weight(3, 16, 96, FAKE, FAKE, None, FAKE, FAKE, None) == 2
    assert L.w4a4_pack_weight(3, 16, 128, FAKE, FAKE, None, None, FAKE, None) == 1
    assert L.w4a4_linear(3, 4, 16, 96, FAKE, FAKE, None, FAKE, FAKE, None, 0, None) == 2
    assert L.w4a4_linear(3, 4, 16, 128, FAKE, FAKE, None, FAKE_MIS, FAKE, None, 0, None) == 3
    assert L.w4a4_linear(3, 0, 16, 128, None, None, None, None, None, None, 0, None) == 0
    # the multi-output quantizer, grouped linear and solver do not take this format
    assert L.w4a4_quantize_act_multi(3, 4, 128, FAKE, 1, arr, arr, arr, None, None, 0, None) == 4
    assert L.w4a4_linear_grouped(3, 1, 4, 128, n, arr, arr, None, arr, arr, None) == 4
    assert L.w4a4_dualquant_solve(3, 64, 256, FAKE, 15, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                  1 << 30, None) == 4
    assert "INT4 G=64" in L.w4a4_last_error().decode()


def test_linear_noalloc_validation():
    """w4a4_linear_noalloc checks its arguments on the host like w4a4_linear
    (no workspace argument: the split-K scratch is the library's own)."""
    L = w4.lib()
    base = (FAKE, FAKE, None, FAKE, FAKE, None)
    assert L.w4a4_linear_noalloc(0, 0, 128, 256, None, None, None, None, None, None) == 0  # M = 0
    assert L.w4a4_linear_noalloc(0, 4, 100, 256, *base) == 2        # N % 16
    assert L.w4a4_linear_noalloc(0, 4, 128, 200, *base) == 2        # K % 128
    assert L.w4a4_linear_noalloc(9, 4, 128, 256, *base) == 4        # unknown format
    assert L.w4a4_linear_noalloc(3, 4, 128, 256, *base) == 4        # INT4 G=64
    assert L.w4a4_linear_noalloc(1, 4, 128, 256, *base) == 1        # NVFP4 without t_act
    assert L.w4a4_linear_noalloc(0, 4, 128, 256, None, FAKE, None, FAKE, FAKE, None) == 1
    assert L.w4a4_linear_noalloc(0, 4, 128, 256, FAKE_MIS, FAKE, None, FAKE, FAKE, None) == 3
    # the largest split-K workspace fits the scratch array
    assert L.w4a4_linear_workspace_bytes(0, 2048, 4096, 8192) == 4352 + 128 * 4 * 65536


def test_mx8_size_queries_and_unsupported_calls():
    """The 8-bit MX formats (4 = MXFP8, 5 = MXINT8): one byte per code,
    32-blocks, a blob of N*K code bytes + N*K/32 scale bytes + r; the
    multi-output quantizer, the grouped linear and the solver reject them."""
    L = w4.lib()
    for f in (4, 5):
        assert L.w4a4_block_size(f) == 32
        assert L.w4a4_act_codes_bytes(f, 2048, 4096) == 2048 * 4096
        assert L.w4a4_act_scales_bytes(f, 2048, 4096) == 2048 * 128
        assert L.w4a4_quantize_workspace_bytes(f, 2048, 4096) == 0
        assert L.w4a4_linear_workspace_bytes(f, 2048, 4096, 14336) == 0
        N, K = 4096, 14336
        got = L.w4a4_packed_weight_bytes(f, N, K)
        assert N * K + N * K // 32 + 4 * N <= got < N * K + N * K // 32 + 4 * N + 1024
        assert L.w4a4_dualquant_workspace_bytes(f, 64, 256) == 0
        arr = (ctypes.c_void_p * 1)(FAKE)
        assert L.w4a4_quantize_act_multi(f, 4, 256, FAKE, 1, arr, arr, arr, None, None, 0, None) == 4
        Ns = (ctypes.c_int64 * 1)(256)
        assert L.w4a4_linear_grouped(f, 1, 4, 256, Ns, arr, arr, None, arr, arr, None) == 4
        # 8-byte code alignment for the 8-bit quantizer
        assert L.w4a4_quantize_act(f, 4, 256, FAKE, None, ctypes.c_void_p((1 << 20) + 4), FAKE, None,
                                   None, 0, None) == 3


def test_probe_rejects_bad_arguments():
    """The measurement probe validates its arguments on the host."""
    L = w4.lib()
    fake = ctypes.c_void_p(4096)
    assert L.w4a4_probe_stream_read(None, 1024, fake, None) == 1           # NULL src
    assert L.w4a4_probe_stream_read(fake, 1024, None, None) == 1           # NULL sink
    assert L.w4a4_probe_stream_read(fake, 1000, fake, None) == 2           # bytes % 16
    assert L.w4a4_probe_stream_read(fake, 0, fake, None) == 2
    assert L.w4a4_probe_stream_read(ctypes.c_void_p(4100), 1024, fake, None) == 3  # alignment
    assert L.w4a4_probe_mfma_fp4(None, 2, 1, fake, None) == 1              # NULL ops
    assert L.w4a4_probe_mfma_fp4(fake, 2, 1, None, None) == 1              # NULL sink
    assert L.w4a4_probe_mfma_fp4(fake, 3, 1, fake, None) == 2              # odd iters
    assert L.w4a4_probe_mfma_fp4(fake, 0, 1, fake, None) == 2
    assert L.w4a4_probe_mfma_fp4(fake, (1 << 20) + 2, 1, fake, None) == 2
    assert L.w4a4_probe_mfma_fp4(fake, 2, 0, fake, None) == 2              # workgroups
    assert L.w4a4_probe_mfma_fp4(fake, 2, 4097, fake, None) == 2
    assert L.w4a4_probe_mfma_fp4(ctypes.c_void_p(4104), 2, 1, fake, None) == 3  # alignment



def test_int8g128_size_queries():
    """INT8 G=128 with BF16 scales (6): one byte per code, two scale bytes per
    128-block, K % 128 and N % 16, a blob of N*K code bytes + N*K/64 scale
    bytes + r, no workspaces."""
    L = w4.lib()
    assert L.w4a4_block_size(6) == 128
    assert L.w4a4_act_codes_bytes(6, 5, 384) == 5 * 384
    assert L.w4a4_act_scales_bytes(6, 5, 384) == 5 * 3 * 2
    assert L.w4a4_act_scales_bytes(6, 5, 192) == 0                  # K % 128
    assert L.w4a4_act_codes_bytes(6, 5, 64) == 0
    assert L.w4a4_quantize_workspace_bytes(6, 5, 384) == 0
    assert L.w4a4_linear_workspace_bytes(6, 2048, 4096, 4096) == 0

    def a256(x):
        return (x + 255) // 256 * 256

    for N, K in [(16, 128), (48, 384), (4096, 14336)]:
        assert L.w4a4_packed_weight_bytes(6, N, K) == a256(a256(256 + N * K) + N * (K // 128) * 2) + a256(4 * N)
    assert L.w4a4_packed_weight_bytes(6, 24, 256) == 0              # N % 16
    assert L.w4a4_packed_weight_bytes(6, 16, 192) == 0              # K % 128
    assert L.w4a4_dualquant_workspace_bytes(6, 64, 256) == 0        # no solver for this format


def test_int8g128_rejects():
    L = w4.lib()
    arr = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    n = (ctypes.c_int64 * 4)(64, 64, 64, 64)
    # quantize_act: K % 128, NULL X, misaligned X, codes not 8-byte aligned
    assert L.w4a4_quantize_act(6, 4, 192, FAKE, None, FAKE, FAKE, None, None, 0, None) == 2
    assert L.w4a4_quantize_act(6, 4, 256, None, None, FAKE, FAKE, None, None, 0, None) == 1
    assert L.w4a4_quantize_act(6, 4, 256, FAKE_MIS, None, FAKE, FAKE, None, None, 0, None) == 3
    assert L.w4a4_quantize_act(6, 4, 256, FAKE, None, ctypes.c_void_p((1 << 20) + 4), FAKE, None,
                               None, 0, None) == 3
    # pack / unpack / linear: N % 16, K % 128, NULL r, misaligned blob
    assert L.w4a4_pack_weight(6, 24, 128, FAKE, FAKE, None, FAKE, FAKE, None) == 2
    assert L.w4a4_pack_weight(6, 16, 192, FAKE, FAKE, None, FAKE, FAKE, None) == 2
    assert L.w4a4_pack_weight(6, 16, 128, FAKE, FAKE, None, None, FAKE, None) == 1
    assert L.w4a4_unpack_weight(6, 16, 128, None, FAKE, FAKE, None, None, None) == 1
    assert L.w4a4_linear(6, 4, 16, 192, FAKE, FAKE, None, FAKE, FAKE, None, 0, None) == 2
    assert L.w4a4_linear(6, 4, 16, 128, FAKE, FAKE, None, FAKE_MIS, FAKE, None, 0, None) == 3
    assert L.w4a4_linear(6, 0, 16, 128, None, None, None, None, None, None, 0, None) == 0
    # the multi-output quantizer, noalloc and grouped linear and the solver do not take it
    assert L.w4a4_quantize_act_multi(6, 4, 128, FAKE, 1, arr, arr, arr, None, None, 0, None) == 4
    assert L.w4a4_linear_noalloc(6, 4, 128, 256, FAKE, FAKE, None, FAKE, FAKE, None) == 4
    assert L.w4a4_linear_grouped(6, 1, 4, 128, n, arr, arr, None, arr, arr, None) == 4
    assert L.w4a4_dualquant_solve(6, 64, 256, FAKE, 15, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                  1 << 30, None) == 4
    assert "INT8 G=128" in L.w4a4_last_error().decode()
