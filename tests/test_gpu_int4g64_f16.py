"""GPU parity of the INT4 G=64 fp16-expansion GEMM (M > 16) against the oracle.

The kernel turns every code times its BF16 block scale into one fp16 value
(exact within 25 binades of the largest scale of the activation row or the
weight column, a power of two per row and column keeping the values in
fp16's normal range) and runs the fp16 MFMA.  Covered here, through the C
ABI: each of its three tile shapes (chosen by the host from the shape), one
K-step (fewer K-steps than pipeline stages) and several, ragged M and N,
bit-exactness where every fp32 partial sum is exact, scales spread over more
binades than the exact window, zero and negative scales, a non-finite
activation block (its row is NaN, the others unaffected), the integer
kernel that K not a multiple of 128 takes, and the Llama-3.1-8B shapes at
full size on sampled outputs."""
import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from gpu_common import device, say, bf16_bits, check_linear
import w4a4_block_scaled_amd as w4
from w4a4_block_scaled_amd import inputs

pytestmark = pytest.mark.gpu
FMT = "int4g64"


def tile_choice(M, N, K):
    """GEMM kernel the host picks for an INT4 G=64 linear; mirrors the
    library's rule ("decode", "int" or the fp16 kernel's n x m tile)."""
    if M <= 16:
        return "decode"
    if K % 128:
        return "int"

    def rounds(bn, bm):
        return ((N + bn - 1) // bn * ((M + bm - 1) // bm) + 255) // 256

    c44, c42, c22 = rounds(256, 256) * 2048, rounds(256, 128) * 1320, rounds(128, 128) * 880
    if c44 <= c42 and c44 <= c22:
        return "256x256"
    return "256x128" if c42 <= c22 else "128x128"


def bits16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_dev(bits_u16, dev):
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).view(torch.bfloat16).to(dev)


def bf16_of(x64):
    """float64 array -> BF16 bit patterns (round to nearest even)."""
    return F.bf16_from_f64(np.asarray(x64, np.float64))


def run_codes(a_codes, a_bits, w_codes, w_bits, r, dev, a_dev=None):
    """GEMM on given codes and scale bit patterns; returns (Y bits, oracle y, S)."""
    N, K = w_codes.shape[0], 2 * w_codes.shape[1]
    blob = w4.pack_weight(torch.from_numpy(w_codes).to(dev), bf16_dev(w_bits, dev), None,
                          torch.from_numpy(r).to(dev), FMT)
    ac = torch.from_numpy(a_codes).to(dev) if a_dev is None else a_dev
    Y = w4.linear(ac, bf16_dev(a_bits, dev), None, blob, FMT, N, K)
    torch.cuda.synchronize()
    _, y = oracle.linear_bf16(a_codes, a_bits, None, w_codes, w_bits, 1.0, r, FMT)
    S = oracle.linear.linear_abs_sum(a_codes, a_bits, None, w_codes, w_bits, 1.0, r, FMT)
    return bf16_bits(Y), y, S


def random_codes(rng, R, K):
    return rng.integers(0, 256, (R, K // 2), dtype=np.uint8)


# (M, N, K, tile): ragged M and N, one K-step (K = 128, below the pipeline
# depth) up to many
SHAPES = [
    (17, 48, 128, "128x128"),
    (130, 528, 256, "128x128"),
    (300, 2000, 640, "128x128"),
    (1000, 5008, 256, "256x128"),
    (1000, 5008, 128, "256x128"),
    (1100, 8000, 256, "256x256"),
    (1100, 8000, 384, "256x256"),
]


def test_shapes_take_the_intended_tile():
    assert [tile_choice(M, N, K) for M, N, K, _ in SHAPES] == [s[3] for s in SHAPES]
    # the Llama-3.1-8B linears at M = 2048: qkv, o, gate+up, down
    assert [tile_choice(2048, N, K) for N, K in [(6144, 4096), (4096, 4096), (28672, 4096), (4096, 14336)]] \
        == ["256x256", "256x128", "256x256", "256x128"]
    assert tile_choice(64, 272, 1088) == "int" and tile_choice(16, 4096, 4096) == "decode"


@pytest.mark.parametrize("M,N,K,tile", SHAPES)
def test_f16_kernel_matches_oracle(M, N, K, tile):
    dev = device()
    label = f"int4g64 f16 {tile} M={M} N={N} K={K}"
    say(label)
    case = inputs.adhoc_case(FMT, M, N, K, seed=3 * M + N + K)
    wc, ws, _ = oracle.quantize_weight(case.w_prescaled.float().numpy(), FMT)
    blob = w4.pack_weight(torch.from_numpy(wc).to(dev), bf16_dev(ws, dev), None,
                          torch.from_numpy(case.r).to(dev), FMT)
    ac, asc, _ = w4.quantize_act(case.x.to(dev), torch.from_numpy(case.c).to(dev), FMT)
    Y = w4.linear(ac, asc, None, blob, FMT, N, K)
    torch.cuda.synchronize()
    a_o, as_o, _ = oracle.quantize_act(case.x.float().numpy(), case.c, FMT)
    assert np.array_equal(ac.cpu().numpy(), a_o) and np.array_equal(bits16(asc), as_o)
    _, y = oracle.linear_bf16(a_o, as_o, None, wc, ws, 1.0, case.r, FMT)
    S = oracle.linear.linear_abs_sum(a_o, as_o, None, wc, ws, 1.0, case.r, FMT)
    elem, row = check_linear(bf16_bits(Y), y, S, K, label)
    say(f"    max elementwise rel err {elem:.2e}, max row rel-L2 {row:.2e}")


@pytest.mark.parametrize("M,N,K", [(40, 160, 1024), (1000, 5008, 256), (1100, 8000, 256)])
def test_f16_kernel_bit_exact_with_power_of_two_scales(M, N, K):
    """Scales and r powers of two in a narrow range: every expanded value,
    product and fp32 partial sum is exact, so Y equals the oracle's single
    BF16 rounding bit for bit (G0), on each tile shape."""
    dev = device()
    say(f"[int4g64 f16 G0] {tile_choice(M, N, K)} M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    a_codes, w_codes = random_codes(rng, M, K), random_codes(rng, N, K)
    pow2 = np.array([0x3E80, 0x3F00, 0x3F80, 0x4000, 0x4080], np.uint16)  # 0.25 .. 4
    a_bits = pow2[rng.integers(0, 5, (M, K // 64))]
    w_bits = pow2[rng.integers(0, 5, (N, K // 64))]
    r = np.ldexp(1.0, rng.integers(-2, 3, N)).astype(np.float32)
    got, y, _ = run_codes(a_codes, a_bits, w_codes, w_bits, r, dev)
    want = F.bf16_from_f64(y)
    assert np.array_equal(got, want), f"{(got != want).sum()} of {want.size} outputs differ"


@pytest.mark.parametrize("spread", [24, 60])
def test_f16_kernel_wide_scale_range(spread):
    """Block scales of each activation row and weight column spread over
    `spread` binades (24: all inside the exact window; 60: far outside it,
    the smallest blocks rounded): the outputs stay within G1 and G2.  Zero
    and negative weight scales are mixed in."""
    dev = device()
    M, N, K = 300, 2000, 1024
    say(f"[int4g64 f16 scale spread {spread}] M={M} N={N} K={K}")
    rng = np.random.default_rng(spread)
    a_codes, w_codes = random_codes(rng, M, K), random_codes(rng, N, K)
    mant = rng.uniform(1.0, 2.0, (M, K // 64))
    a_bits = bf16_of(mant * np.ldexp(1.0, rng.integers(-spread // 2, spread - spread // 2, (M, K // 64))))
    wm = rng.uniform(1.0, 2.0, (N, K // 64)) * rng.choice([-1.0, 1.0], (N, K // 64))
    w_bits = bf16_of(wm * np.ldexp(1.0, rng.integers(-spread // 2 - 10, spread - spread // 2 - 10, (N, K // 64))))
    w_bits[rng.random((N, K // 64)) < 0.05] = 0
    r = rng.uniform(0.5, 2.0, N).astype(np.float32)
    got, y, S = run_codes(a_codes, a_bits, w_codes, w_bits, r, dev)
    elem, row = check_linear(got, y, S, K, f"spread {spread}")
    say(f"    max elementwise rel err {elem:.2e}, max row rel-L2 {row:.2e}")


def test_f16_kernel_zero_row_and_nonfinite_block():
    """An all-zero activation row gives an exactly zero output row; an
    activation row with a non-finite block (its scale quantizes to NaN) gives
    NaN across its output row and leaves every other row as the oracle has
    it (the NaN does not enter other rows' exponent shifts)."""
    dev = device()
    M, N, K = 200, 1040, 512
    say(f"[int4g64 f16 zero / NaN rows] M={M} N={N} K={K}")
    case = inputs.adhoc_case(FMT, M, N, K, seed=77)
    x = case.x.clone()
    x[3] = 0
    x[150, 70] = float("inf")
    wc, ws, _ = oracle.quantize_weight(case.w_prescaled.float().numpy(), FMT)
    blob = w4.pack_weight(torch.from_numpy(wc).to(dev), bf16_dev(ws, dev), None,
                          torch.from_numpy(case.r).to(dev), FMT)
    ac, asc, _ = w4.quantize_act(x.to(dev), torch.from_numpy(case.c).to(dev), FMT)
    Y = bf16_bits(w4.linear(ac, asc, None, blob, FMT, N, K))
    a_o, as_o, _ = oracle.quantize_act(x.float().numpy(), case.c, FMT)
    assert np.array_equal(ac.cpu().numpy(), a_o) and np.array_equal(bits16(asc), as_o)
    assert np.isnan(F.bf16_value(Y[150])).all()
    assert np.all((Y[3] & 0x7FFF) == 0)
    keep = np.array([m for m in range(M) if m != 150])
    _, y = oracle.linear_bf16(a_o[keep], as_o[keep], None, wc, ws, 1.0, case.r, FMT)
    S = oracle.linear.linear_abs_sum(a_o[keep], as_o[keep], None, wc, ws, 1.0, case.r, FMT)
    check_linear(Y[keep], y, S, K, "rows without the non-finite block")


def test_k_not_a_multiple_of_128_takes_the_integer_kernel():
    """An odd number of 64-blocks runs the integer tile kernel; it meets the
    gates on the same kind of inputs, scales over 60 binades included."""
    dev = device()
    M, N, K = 300, 2000, 576
    assert tile_choice(M, N, K) == "int"
    say(f"[int4g64 integer kernel] M={M} N={N} K={K}")
    rng = np.random.default_rng(5)
    a_codes, w_codes = random_codes(rng, M, K), random_codes(rng, N, K)
    a_bits = bf16_of(rng.uniform(1, 2, (M, K // 64)) * np.ldexp(1.0, rng.integers(-30, 30, (M, K // 64))))
    w_bits = bf16_of(rng.uniform(1, 2, (N, K // 64)) * np.ldexp(1.0, rng.integers(-40, 20, (N, K // 64))))
    r = rng.uniform(0.5, 2.0, N).astype(np.float32)
    got, y, S = run_codes(a_codes, a_bits, w_codes, w_bits, r, dev)
    check_linear(got, y, S, K, "integer kernel")


@pytest.mark.parametrize("name", ["qkv", "o", "gate_up", "down"])
def test_full_size_llama_int4g64_sampled(name):
    """Llama-3.1-8B linears at M = 2048, the benchmark's launch
    configuration; the oracle computes sampled rows and columns."""
    dev = device()
    M = 2048
    case = inputs.workload_cases("llama_int4g64", M=M, linears=[name])[0]
    say(f"[int4g64 f16 full] {name} M={M} N={case.N} K={case.K} tile {tile_choice(M, case.N, case.K)}")
    blob = w4.pack_weight(torch.from_numpy(case.w_codes).to(dev), bf16_dev(case.w_scales, dev), None,
                          torch.from_numpy(case.r).to(dev), FMT)
    ac, asc, _ = w4.quantize_act(case.x.to(dev), torch.from_numpy(case.c).to(dev), FMT)
    Y = w4.linear(ac, asc, None, blob, FMT, case.N, case.K)
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], rng.choice(M, 6, replace=False)]))
    cols = np.unique(np.concatenate([np.arange(32), np.arange(case.N - 32, case.N),
                                     rng.choice(case.N, 32, replace=False)]))
    a_o, as_o, _ = oracle.quantize_act(case.x[torch.from_numpy(rows)].float().numpy(), case.c, FMT)
    assert np.array_equal(ac.cpu().numpy()[rows], a_o) and np.array_equal(bits16(asc)[rows], as_o)
    wc, ws, r = case.w_codes[cols], case.w_scales[cols], case.r[cols]
    _, y = oracle.linear_bf16(a_o, as_o, None, wc, ws, 1.0, r, FMT)
    S = oracle.linear.linear_abs_sum(a_o, as_o, None, wc, ws, 1.0, r, FMT)
    check_linear(bf16_bits(Y)[np.ix_(rows, cols)], y, S, case.K, f"full {name}")
