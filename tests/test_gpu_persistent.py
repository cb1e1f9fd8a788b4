"""GPU parity of the MXFP4 persistent GEMM against the oracle.

MXFP4 shapes with enough 256 x 256 tiles and K a multiple of 512 run one
workgroup per CU that walks its items as one stream of K-steps (the copy
ring crosses item boundaries).  The items are whole tiles, 256 x 192 tiles
(3 of the 4 weight groups of a wave) where those fill one round, or n halves
of 128 features with 96..128 tiles.  Covered here, all outputs compared:
several tiles per workgroup, tile counts that are not a multiple of the 8
XCDs, ragged M and N, one-quad tiles (K = 512: every tile's only quad also
copies the next tile's first), 192-wide tiles (their first weight group at
either position of its scale word, and a last tile partly past N), halves
(one per workgroup, and fewer halves than workgroups, with ragged M and N
and a half past N), bit-exactness where accumulation is exact, and repeated
calls."""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import device, say, to_dev, bf16_bits, check_linear
from test_gpu_linear import gpu_layer, oracle_layer
from w4a4_block_scaled_amd import inputs
import w4a4_block_scaled_amd as w4

pytestmark = pytest.mark.gpu


def fne(M, N, K):
    """Item width the host picks for the persistent kernel (0: not taken);
    mirrors the library's rule."""
    if not (M > 32 and K % 512 == 0):
        return 0
    tm = (M + 255) // 256
    T, T3 = (N + 255) // 256 * tm, (N + 191) // 192 * tm
    if M >= 1024 and 128 < T <= 256 and T3 <= 256:
        return 3
    if T >= 192:
        return 4
    if M >= 1024 and 96 <= T <= 128:
        return 2
    return 0


def persistent(M, N, K):
    """The host-side condition for the persistent kernel (MXFP4)."""
    return fne(M, N, K) != 0


# (M, N, K): what the tile walk does with it (256 workgroups, 32 per XCD)
PERSIST = [
    (512, 40960, 1024),    # 320 tiles: 40 per XCD, 8 workgroups take two
    (300, 24592, 1024),    # 194 tiles (24 or 25 per XCD), ragged M and N
    (1100, 16400, 2048),   # 325 tiles, ragged M and N, 4 quads per tile
    (512, 49152, 512),     # 384 tiles of one quad each
    (1024, 8192, 1024),    # 128 tiles: 256 halves, one per workgroup
    (2000, 4000, 1024),    # 128 tiles: halves, ragged M and N (the last half past N)
    (1100, 6000, 512),     # 120 tiles: 240 halves, ragged M and N, one quad each
    (2048, 6144, 1024),    # 192 tiles: 256 tiles of 256 x 192
    (1100, 7024, 512),     # 185 tiles of 256 x 192, ragged M, the last tile 112 features wide
]


def test_shapes_take_the_intended_path():
    assert [fne(*s) for s in PERSIST] == [4, 4, 4, 4, 2, 2, 2, 3, 3]
    assert fne(2048, 4096, 4096) == 2 and fne(2048, 6144, 4096) == 3 and fne(2048, 28672, 4096) == 4


@pytest.mark.parametrize("M,N,K", PERSIST)
def test_persistent_matches_oracle(M, N, K):
    dev = device()
    assert persistent(M, N, K)
    say(f"[persistent] mxfp4 M={M} N={N} K={K}")
    case = inputs.adhoc_case("mxfp4", M, N, K, seed=M + 7 * N + K)
    Y, *_ = gpu_layer(case, dev)
    y, S, _, _ = oracle_layer(case)
    elem, row = check_linear(bf16_bits(Y), y, S, K, f"persistent {M}x{N}x{K}")
    say(f"    max elementwise rel err {elem:.2e}, max row rel-L2 {row:.2e}")


def test_persistent_bit_exact_when_accumulation_is_exact():
    """All block scales of an operand equal: every fp32 partial sum is
    exact, so Y equals the oracle's BF16 rounding bit for bit."""
    dev = device()
    M, N, K = 512, 24576, 1024
    assert persistent(M, N, K)
    say(f"[persistent bit-exact] M={M} N={N} K={K}")
    rng = np.random.default_rng(11)
    w_codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    w_scales = np.full((N, K // 32), 126, np.uint8)
    r = np.ldexp(1.0, rng.integers(-3, 4, N)).astype(np.float32)
    a_codes = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    a_scales = np.full((M, K // 32), 128, np.uint8)
    blob = w4.pack_weight(to_dev(w_codes, dev), to_dev(w_scales, dev), None, to_dev(r, dev), "mxfp4")
    Y = w4.linear(to_dev(a_codes, dev), to_dev(a_scales, dev), None, blob, "mxfp4", N, K)
    bits, _ = oracle.linear_bf16(a_codes, a_scales, None, w_codes, w_scales, 1.0, r, "mxfp4")
    got = bf16_bits(Y)
    assert np.array_equal(got, bits), f"{(got != bits).sum()} of {bits.size} outputs differ"


def test_persistent_repeated_calls():
    """Same inputs twice around a call of another shape: identical results."""
    dev = device()
    a = inputs.adhoc_case("mxfp4", 512, 40960, 1024, seed=5)
    b = inputs.adhoc_case("mxfp4", 300, 24592, 1024, seed=6)
    say("[persistent repeat] 512x40960x1024 / 300x24592x1024")
    Y1, blob, (ac, as_, ta), _ = gpu_layer(a, dev)
    Yb1, blob_b, (bc, bs, bt), _ = gpu_layer(b, dev)
    Y2 = w4.linear(ac, as_, ta, blob, "mxfp4", a.N, a.K)
    Yb2 = w4.linear(bc, bs, bt, blob_b, "mxfp4", b.N, b.K)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(Yb1, Yb2)
