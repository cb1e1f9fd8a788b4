"""GPU parity of the MXINT4 tiled kernels against the oracle.

M > 16 runs either 256 x 128 tiles with one wave per SIMD or 256 x 256
tiles with two waves per SIMD (8 waves of 128 x 64), whichever takes fewer
estimated rounds over the 256 CUs; with fewer than 128 tiles of 256 x 128,
128 x 64 or 128 x 128 tiles (the most that fit one round).  All four are
covered here on ragged and exact tile grids, with the oracle computing
sampled outputs, and bit for bit where the accumulation is exact."""
import numpy as np
import pytest

import oracle
from gpu_common import device, say, to_dev, bf16_bits, check_linear
from test_gpu_linear import gpu_layer, oracle_layer, _sample
from w4a4_block_scaled_amd import inputs
import w4a4_block_scaled_amd as w4

pytestmark = pytest.mark.gpu


def tile_config(M, N):
    """The host-side choice among the MXINT4 tiled kernels (M > 16)."""
    tn = (N + 255) // 256
    rounds_lean = (tn * ((M + 255) // 256) + 255) // 256
    rounds_one = (tn * ((M + 127) // 128) + 255) // 256
    if 100 * rounds_lean <= 54 * rounds_one:
        return "256x256 lean"
    if tn * ((M + 127) // 128) < 128:
        tn2 = (N + 127) // 128
        if tn2 * ((M + 63) // 64) <= 256:
            return "128x64"
        if tn2 * ((M + 127) // 128) <= 256:
            return "128x128"
    return "256x128"


def two_waves_per_simd(M, N):
    return tile_config(M, N) == "256x256 lean"


# (M, N, K, kernel): ragged M and N, exact grids, one K-step and several
SHAPES = [
    (4000, 3504, 1024, "256x256 lean"),
    (4096, 3584, 512, "256x256 lean"),
    (4096, 4608, 384, "256x128"),
    (1000, 2000, 640, "128x64"),
    (300, 3536, 640, "128x64"),
    (512, 4608, 1024, "128x128"),
    (520, 4560, 384, "128x128"),
]


@pytest.mark.parametrize("M,N,K,config", SHAPES)
def test_mxint4_tiled_kernels_match_oracle(M, N, K, config):
    dev = device()
    assert tile_config(M, N) == config
    say(f"[mxint4 tiles] M={M} N={N} K={K} tiles: {config}")
    rng = np.random.default_rng(M + N + K)
    case = inputs.adhoc_case("mxint4", M, N, K, seed=M + 3 * N + K)
    Y, *_ = gpu_layer(case, dev)
    rows = np.unique(np.concatenate([np.arange(130), _sample(M, 40, rng), np.arange(M - 130, M)]))
    cols = np.unique(np.concatenate([np.arange(260), _sample(N, 96, rng), np.arange(N - 260, N)]))
    y, S, _, _ = oracle_layer(case, rows, cols)
    elem, row = check_linear(bf16_bits(Y)[np.ix_(rows, cols)], y, S, K, f"mxint4 {M}x{N}x{K}")
    say(f"    max elementwise rel err {elem:.2e}, max row rel-L2 {row:.2e}")


@pytest.mark.parametrize("M,N,K,config", [(4096, 3584, 1024, "256x256 lean"), (512, 4608, 512, "128x128"),
                                           (300, 3536, 512, "128x64")])
def test_mxint4_tiled_bit_exact(M, N, K, config):
    """Equal block scales per operand: every fp32 partial sum is exact, so
    the output equals the oracle's BF16 rounding bit for bit."""
    dev = device()
    assert tile_config(M, N) == config
    say(f"[mxint4 tiles bit-exact] M={M} N={N} K={K} tiles: {config}")
    rng = np.random.default_rng(17)
    w_codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    w_scales = np.full((N, K // 32), 124, np.uint8)
    r = np.ldexp(1.0, rng.integers(-3, 4, N)).astype(np.float32)
    a_codes = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    a_scales = np.full((M, K // 32), 130, np.uint8)
    blob = w4.pack_weight(to_dev(w_codes, dev), to_dev(w_scales, dev), None, to_dev(r, dev), "mxint4")
    Y = w4.linear(to_dev(a_codes, dev), to_dev(a_scales, dev), None, blob, "mxint4", N, K)
    bits, _ = oracle.linear_bf16(a_codes, a_scales, None, w_codes, w_scales, 1.0, r, "mxint4")
    got = bf16_bits(Y)
    assert np.array_equal(got, bits), f"{(got != bits).sum()} of {bits.size} outputs differ"
