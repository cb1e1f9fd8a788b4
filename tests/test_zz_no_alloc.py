"""The allocation-free linear (w4a4_linear_noalloc) against w4a4_linear.

w4a4_linear_noalloc runs the same kernels as w4a4_linear, taking the MXFP4
split-K workspace from the library's own per-device scratch array instead of
a caller buffer.  Two calls in a row on split-K shapes, the second smaller
(128 then 66 tiles, so the second call reuses slots the first filled), must
each equal w4a4_linear's output bit for bit (the two halves of a tile are
added in either order, a + b = b + a exactly), and the oracle's gates on
sampled rows; a shape without a workspace (decode) and the other formats go
through unchanged.  Every call goes through the C ABI (ctypes)."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_common import device, say, bf16_bits, check_linear
from test_gpu_linear import gpu_layer, oracle_layer
from w4a4_block_scaled_amd import inputs
import w4a4_block_scaled_amd as w4

pytestmark = pytest.mark.gpu


def noalloc(case_gpu, fmt, N, K):
    Y, blob, (ac, sc, ta), _ = case_gpu
    L = w4.lib()
    out = torch.full_like(Y, float("nan"))
    st = L.w4a4_linear_noalloc(w4.FORMATS[fmt], ac.shape[0], N, K, ctypes.c_void_p(ac.data_ptr()),
                               ctypes.c_void_p(sc.data_ptr()),
                               None if ta is None else ctypes.c_void_p(ta.data_ptr()),
                               ctypes.c_void_p(blob.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                               ctypes.c_void_p(torch.cuda.current_stream(Y.device).cuda_stream))
    assert st == 0, L.w4a4_last_error().decode()
    return out


def test_noalloc_two_split_k_calls_match_linear():
    dev = device()
    L = w4.lib()
    for M, N, K, seed in ((2048, 4096, 8192, 41), (300, 8208, 8192, 42)):
        need = L.w4a4_linear_workspace_bytes(0, M, N, K)
        assert 0 < need <= 4352 + 128 * 4 * 65536, "the shape takes the split-K kernel"
        say(f"[noalloc] mxfp4 M={M} N={N} K={K} (split-K workspace {need} B)")
        case = inputs.adhoc_case("mxfp4", M, N, K, seed=seed)
        g = gpu_layer(case, dev)
        Y = noalloc(g, "mxfp4", N, K)
        torch.cuda.synchronize()
        assert torch.equal(Y, g[0]), "noalloc output differs from w4a4_linear's"
        rows = np.unique(np.r_[0:3, M // 2, M - 3:M])
        y, S, _, _ = oracle_layer(case, rows=rows)
        check_linear(bf16_bits(Y)[rows], y, S, K, f"noalloc {M}x{N}x{K}")


@pytest.mark.parametrize("fmt,M,N,K", [("mxfp4", 4, 4096, 4096), ("mxint4", 64, 512, 1024),
                                       ("nvfp4", 17, 256, 512)])
def test_noalloc_without_workspace_matches_linear(fmt, M, N, K):
    dev = device()
    assert w4.lib().w4a4_linear_workspace_bytes(w4.FORMATS[fmt], M, N, K) == 0
    say(f"[noalloc] {fmt} M={M} N={N} K={K} (no workspace)")
    case = inputs.adhoc_case(fmt, M, N, K, seed=M + N)
    g = gpu_layer(case, dev)
    Y = noalloc(g, fmt, N, K)
    torch.cuda.synchronize()
    assert torch.equal(Y, g[0])
