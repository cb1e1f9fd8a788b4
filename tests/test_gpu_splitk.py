"""GPU parity of the MXFP4 split-K GEMM against the oracle.

MXFP4 shapes with 64..128 tiles of 256 x 256 (too few to fill 256 CUs) and
K a multiple of 1024, at least 8192, split each tile's K-steps in two halves
run by two workgroups; the halves meet per wave slot through the workspace
(partial sums, a ticket and a flag per slot).  Covered here: every output
against the oracle with ragged M and N and tile counts not a multiple of 8;
all 256 workgroups busy, checked on sampled column bands (first, middle and
last tile) with every row; bit-exactness where accumulation is exact;
repeated calls (the tickets and flags must be back at zero after each call)
around calls of other shapes sharing the workspace."""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import device, say, to_dev, bf16_bits, check_linear
from test_gpu_linear import gpu_layer, oracle_layer
from w4a4_block_scaled_amd import inputs
import w4a4_block_scaled_amd as w4

pytestmark = pytest.mark.gpu


def split_k(M, N, K):
    """The host-side condition for the split-K kernel (MXFP4)."""
    T = ((N + 255) // 256) * ((M + 255) // 256)
    return M > 32 and K % 1024 == 0 and K >= 8192 and 64 <= T <= 128


# (M, N, K): tiles (256 x 256), what the test reaches
SPLIT = [
    (300, 8208, 8192),     # 2 x 33 = 66 tiles, ragged M and N, 32 K-steps per half
    (520, 5632, 9216),     # 3 x 22 = 66 tiles, ragged M, 36 K-steps per half
]


@pytest.mark.parametrize("M,N,K", SPLIT)
def test_splitk_matches_oracle(M, N, K):
    dev = device()
    assert split_k(M, N, K)
    say(f"[split-k] mxfp4 M={M} N={N} K={K}")
    case = inputs.adhoc_case("mxfp4", M, N, K, seed=M + 5 * N + K)
    Y, *_ = gpu_layer(case, dev)
    y, S, _, _ = oracle_layer(case)
    elem, row = check_linear(bf16_bits(Y), y, S, K, f"split-k {M}x{N}x{K}")
    say(f"    max elementwise rel err {elem:.2e}, max row rel-L2 {row:.2e}")


def test_splitk_all_workgroups_sampled():
    """128 tiles (256 workgroups): every row of three 256-column bands."""
    dev = device()
    M, N, K = 64, 32768, 8192
    assert split_k(M, N, K)
    say(f"[split-k sampled] mxfp4 M={M} N={N} K={K}")
    case = inputs.adhoc_case("mxfp4", M, N, K, seed=77, weights="codes")
    Y, *_ = gpu_layer(case, dev)
    cols = np.concatenate([np.arange(0, 256), np.arange(16384, 16640), np.arange(N - 256, N)])
    y, S, _, _ = oracle_layer(case, cols=cols)
    elem, row = check_linear(bf16_bits(Y)[:, cols], y, S, K, f"split-k {M}x{N}x{K} sampled")
    say(f"    max elementwise rel err {elem:.2e}, max row rel-L2 {row:.2e}")


def test_splitk_bit_exact_when_accumulation_is_exact():
    """All block scales of an operand equal: every fp32 partial sum, and the
    sum of the two halves, is exact, so Y equals the oracle's BF16 rounding
    bit for bit."""
    dev = device()
    M, N, K = 512, 16384, 8192
    assert split_k(M, N, K)
    say(f"[split-k bit-exact] M={M} N={N} K={K}")
    rng = np.random.default_rng(12)
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


def test_splitk_repeated_calls_and_clean_workspace():
    """Same inputs three times around calls of another split-K shape and of
    a persistent shape: identical results, and the workspace's tickets and
    flags are zero after every call."""
    dev = device()
    a = inputs.adhoc_case("mxfp4", 300, 8208, 8192, seed=21)
    b = inputs.adhoc_case("mxfp4", 64, 32768, 8192, seed=22, weights="codes")
    c = inputs.adhoc_case("mxfp4", 512, 49152, 512, seed=23)
    say("[split-k repeat] 300x8208x8192 / 64x32768x8192 / 512x49152x512")
    Ya, blob_a, (aa, sa, ta), _ = gpu_layer(a, dev)
    Yb, blob_b, (ab, sb, tb), _ = gpu_layer(b, dev)
    gpu_layer(c, dev)
    nb = w4.lib().w4a4_linear_workspace_bytes(0, 64, 32768, 8192)
    ws = w4.linear_workspace(dev, nb)
    for _ in range(3):
        Y2 = w4.linear(aa, sa, ta, blob_a, "mxfp4", a.N, a.K)
        Yb2 = w4.linear(ab, sb, tb, blob_b, "mxfp4", b.N, b.K, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(Ya, Y2) and torch.equal(Yb, Yb2)
        sync_words = ws[:4352].view(torch.int32)
        assert int(sync_words.abs().sum()) == 0, "tickets/flags not cleared"


def test_splitk_dirty_sync_word_is_reported_not_silent():
    """A ticket left non-zero before the call (the documented precondition
    broken on purpose from the host): both halves of that wave slot find a
    non-zero ticket, neither writes partial sums, and each gives up after
    its bounded wait.  The call must not return a silently wrong Y: that
    slot's 128 x 128 block of Y is BF16 NaN, the status word is set, the
    synchronization words are zero again, every other output equals the
    clean run, and the next call (status cleared) is clean."""
    dev = device()
    M, N, K = 300, 8208, 8192
    assert split_k(M, N, K)
    say(f"[split-k dirty ticket] mxfp4 M={M} N={N} K={K}")
    case = inputs.adhoc_case("mxfp4", M, N, K, seed=31)
    Ya, blob, (ac, sc, ta), _ = gpu_layer(case, dev)
    nb = w4.lib().w4a4_linear_workspace_bytes(0, M, N, K)
    ws = torch.zeros(nb, dtype=torch.uint8, device=dev)
    words = ws[:4352].view(torch.int32)
    words[0] = 1                                  # ticket of tile 0, wave slot 0 (rows 0..127, cols 0..127)
    torch.cuda.synchronize()
    Y = w4.linear(ac, sc, ta, blob, "mxfp4", N, K, workspace=ws)
    torch.cuda.synchronize()
    got = bf16_bits(Y)
    ref = bf16_bits(Ya)
    assert np.all(got[:128, :128] == 0x7FC0), "the abandoned block is not NaN"
    mask = np.ones_like(got, bool)
    mask[:128, :128] = False
    assert np.array_equal(got[mask], ref[mask]), "outputs outside the abandoned block changed"
    w = words.cpu().numpy()
    assert w[4096 // 4] == 1, "status word not set"
    assert np.all(w[:4096 // 4] == 0), "tickets/flags not cleared after the timeout"
    words[4096 // 4] = 0
    Y2 = w4.linear(ac, sc, ta, blob, "mxfp4", N, K, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(Y2, Ya)
    assert int(words.abs().sum()) == 0
