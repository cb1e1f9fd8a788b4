"""GPU parity of the INT4 G=64 format with BF16 block scales (the paper's
packed deployment format, Appendix I), through the C ABI.

Codes and scale bit patterns are compared with the oracle bit for bit; GEMM
outputs pass gates G1 (every element within the fp32-accumulation bound) and
G2 (row relative L2 error <= 1e-3), and are bit-exact where every partial
sum is exact (power-of-two scales).  Shapes reach every GEMM kernel (M <= 3
and K a multiple of 128 the dot-product decode kernel, M <= 16 the MFMA
decode kernel, M > 16 the tile kernels) with ragged M, N and K-block counts."""
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


def bits16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_dev(bits_u16, dev):
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).view(torch.bfloat16).to(dev)


def gpu_quantize(x, c, dev):
    codes, scales, _ = w4.quantize_act(x.to(dev), None if c is None else torch.from_numpy(c).to(dev), FMT)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), bits16(scales)


def oracle_quantize(x, c):
    K = x.shape[1]
    codes, scales, _ = oracle.quantize_act(x.float().numpy(), np.ones(K, np.float32) if c is None else c, FMT)
    return codes, scales


@pytest.mark.parametrize("M,K", [(1, 64), (3, 192), (37, 576), (300, 4096), (5, 18944)])
@pytest.mark.parametrize("with_c", [False, True])
def test_quantize_matches_oracle(M, K, with_c):
    dev = device()
    say(f"[int4g64 quantize] M={M} K={K} c={with_c}")
    case = inputs.adhoc_case(FMT, M, 16, K, seed=M * 31 + K, weights="none")
    c = case.c if with_c else None
    gc, gs = gpu_quantize(case.x, c, dev)
    oc, os_ = oracle_quantize(case.x, c)
    assert np.array_equal(gs, os_), f"{(gs != os_).sum()} scales differ"
    assert np.array_equal(gc, oc), f"{(gc != oc).sum()} code bytes differ"


def test_quantize_edge_values():
    """Half-integer ties, a scale tie (7 (1 + 2^-8) / 7 is a BF16 midpoint),
    subnormals, an underflowing scale, zeros, the largest BF16, -8 after
    clipping never arising, and the non-finite convention."""
    dev = device()
    K = 64 * 8
    x = np.zeros((4, K), np.float32)
    x[0, :16] = np.arange(-8, 8) + 0.5
    x[0, 16] = 7.0
    x[0, 64] = 7.0                               # block 1: scale tie after c
    x[0, 65:70] = [1.5, -2.5, 3.5, -0.5, 6.5]
    x[1, 128:136] = np.ldexp(1.0, -130) * np.arange(1, 9)    # subnormal inputs
    x[1, 192] = np.ldexp(1.0, -133)              # amax / 7 underflows to 0
    x[1, 256:260] = [3.3895314e38, -1e38, 1.0, -3.0]
    x[2, 320] = np.inf
    x[2, 384] = np.nan
    x[3] = np.linspace(-5, 5, K)
    xb = inputs.to_bf16(x)
    c = np.ones(K, np.float32)
    c[64] = np.float32(1.0 + 2.0 ** -8)
    for cc in (None, c):
        gc, gs = gpu_quantize(xb, cc, dev)
        oc, os_ = oracle_quantize(xb, cc)
        assert np.array_equal(gs, os_) and np.array_equal(gc, oc)
    assert os_[0, 1] == 0x3F80                   # the scale tie went to the even pattern (1.0)
    assert os_[2, 5] == 0x7FC0 and os_[2, 6] == 0x7FC0


def test_pack_unpack_round_trip():
    dev = device()
    rng = np.random.default_rng(3)
    for N, K in ((48, 192), (4096, 4096)):
        codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
        sbits = rng.integers(0x3000, 0x4800, (N, K // 64)).astype(np.uint16)
        r = rng.uniform(0.5, 2, N).astype(np.float32)
        blob = w4.pack_weight(torch.from_numpy(codes).to(dev), bf16_dev(sbits, dev), None,
                              torch.from_numpy(r).to(dev), FMT)
        c2, s2, r2, t2 = w4.unpack_weight(blob, FMT, N, K)
        torch.cuda.synchronize()
        assert np.array_equal(c2.cpu().numpy(), codes)
        assert np.array_equal(bits16(s2), sbits)
        assert np.array_equal(r2.cpu().numpy(), r) and float(t2.item()) == 1.0
        assert blob.numel() == w4.packed_weight_bytes(FMT, N, K)


def run_case(case, dev, label):
    """Quantize (checked against the oracle), pack, GEMM; oracle on every output."""
    wc, ws, _ = oracle.quantize_weight(case.w_prescaled.float().numpy(), FMT) \
        if case.w_prescaled is not None else (case.w_codes, case.w_scales, None)
    blob = w4.pack_weight(torch.from_numpy(wc).to(dev), bf16_dev(ws, dev), None,
                          torch.from_numpy(case.r).to(dev), FMT)
    ac, asc, ta = w4.quantize_act(case.x.to(dev), torch.from_numpy(case.c).to(dev), FMT)
    Y = w4.linear(ac, asc, ta, blob, FMT, case.N, case.K)
    torch.cuda.synchronize()
    a_o, as_o, _ = oracle.quantize_act(case.x.float().numpy(), case.c, FMT)
    assert np.array_equal(ac.cpu().numpy(), a_o) and np.array_equal(bits16(asc), as_o)
    bits, y = oracle.linear_bf16(a_o, as_o, None, wc, ws, 1.0, case.r, FMT)
    S = oracle.linear.linear_abs_sum(a_o, as_o, None, wc, ws, 1.0, case.r, FMT)
    return check_linear(bf16_bits(Y), y, S, case.K, label), bf16_bits(Y), bits


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 16, 17, 64, 130, 300])
@pytest.mark.parametrize("N,K", [(48, 192), (272, 1088), (528, 4096)])
def test_linear_matches_oracle(M, N, K):
    dev = device()
    label = f"int4g64 linear M={M} N={N} K={K}"
    say(label)
    case = inputs.adhoc_case(FMT, M, N, K, seed=M + 7 * N + K)
    run_case(case, dev, label)


@pytest.mark.parametrize("M,N,K", [(1, 96, 1024), (2, 160, 1088), (8, 96, 1024), (40, 160, 1024)])
def test_linear_bit_exact_with_power_of_two_scales(M, N, K):
    """Activation blocks whose amax is 7 * 2^e (Delta = 2^e exactly), weight
    scales and r powers of two in a narrow range: every fp32 step is exact,
    so the BF16 output equals the oracle's single rounding bit for bit (G0)."""
    dev = device()
    rng = np.random.default_rng(M + N)
    q = rng.integers(-7, 8, (M, K)).astype(np.float64)
    q[:, ::64] = 7 * rng.choice([-1, 1], (M, K // 64))
    e = rng.integers(-1, 2, (M, K // 64))
    x = (q.reshape(M, K // 64, 64) * np.ldexp(1.0, e)[..., None]).reshape(M, K).astype(np.float32)
    case = inputs.LinearCase("g0", "g0", FMT, M, N, K, inputs.to_bf16(x),
                             np.ones(K, np.float32), np.ldexp(1.0, rng.integers(-1, 2, N)).astype(np.float32))
    case.w_codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    case.w_scales = np.array([0x3F00, 0x3F80, 0x4000], np.uint16)[rng.integers(0, 3, (N, K // 64))]
    _, got, want = run_case(case, dev, f"int4g64 G0 M={M}")
    assert np.array_equal(got, want), f"{(got != want).sum()} outputs differ"


@pytest.mark.parametrize("M", [1, 2048])
@pytest.mark.parametrize("name", ["qkv", "down"])
def test_full_size_llama_sampled(M, name):
    """Llama shapes at their full size, in the launch configuration the
    benchmark times; the oracle computes sampled rows and columns."""
    dev = device()
    case = inputs.workload_cases("llama_int4g64", M=M, linears=[name])[0]
    say(f"[int4g64 full] {name} M={M} N={case.N} K={case.K}")
    blob = w4.pack_weight(torch.from_numpy(case.w_codes).to(dev), bf16_dev(case.w_scales, dev), None,
                          torch.from_numpy(case.r).to(dev), FMT)
    ac, asc, ta = w4.quantize_act(case.x.to(dev), torch.from_numpy(case.c).to(dev), FMT)
    Y = w4.linear(ac, asc, ta, blob, FMT, case.N, case.K)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 6), replace=False)]))
    cols = np.unique(np.concatenate([np.arange(16), np.arange(case.N - 16, case.N),
                                     rng.choice(case.N, 32, replace=False)]))
    xs = case.x[torch.from_numpy(rows)]
    a_o, as_o, _ = oracle.quantize_act(xs.float().numpy(), case.c, FMT)
    assert np.array_equal(ac.cpu().numpy()[rows], a_o) and np.array_equal(bits16(asc)[rows], as_o)
    wc, ws, r = case.w_codes[cols], case.w_scales[cols], case.r[cols]
    bits, y = oracle.linear_bf16(a_o, as_o, None, wc, ws, 1.0, r, FMT)
    S = oracle.linear.linear_abs_sum(a_o, as_o, None, wc, ws, 1.0, r, FMT)
    check_linear(bf16_bits(Y)[np.ix_(rows, cols)], y, S, case.K, f"full {name} M={M}")


def test_dot_and_mfma_decode_kernels_agree():
    """M = 3 runs the dot-product kernel and M = 4 the MFMA decode kernel;
    on the same first three rows both meet the bound against each other and
    repeated calls are identical."""
    dev = device()
    case = inputs.adhoc_case(FMT, 4, 528, 4096, seed=8)
    (_, y4, _) = run_case(case, dev, "mfma decode")
    case3 = inputs.adhoc_case(FMT, 4, 528, 4096, seed=8)
    case3.M = 3
    case3.x = case3.x[:3]
    (_, y3, _) = run_case(case3, dev, "dot decode")
    (_, y3b, _) = run_case(case3, dev, "dot decode again")
    assert np.array_equal(y3, y3b)
    diff = np.abs(F.bf16_value(y3) - F.bf16_value(y4[:3]))
    assert diff.max() <= 2.0 ** -6 * np.abs(F.bf16_value(y4[:3])).max()


def test_decode_and_tile_kernels_agree():
    """M = 16 runs the decode kernel and M = 17 the tile kernel; the first 16
    rows see the same inputs, so both must meet the bound against each other's
    oracle values and stay deterministic over repeated calls."""
    dev = device()
    case = inputs.adhoc_case(FMT, 17, 272, 1088, seed=5)
    (_, y17, _) = run_case(case, dev, "tile")
    case16 = inputs.adhoc_case(FMT, 17, 272, 1088, seed=5)
    case16.M = 16
    case16.x = case16.x[:16]
    (_, y16, _) = run_case(case16, dev, "decode")
    (_, y16b, _) = run_case(case16, dev, "decode again")
    assert np.array_equal(y16, y16b)
    diff = np.abs(F.bf16_value(y16) - F.bf16_value(y17[:16]))
    assert diff.max() <= 2.0 ** -6 * np.abs(F.bf16_value(y17[:16])).max()


def test_empty_batch_and_rejected_calls():
    dev = device()
    blob = w4.pack_weight(torch.zeros((16, 32), dtype=torch.uint8, device=dev),
                          torch.ones((16, 1), dtype=torch.bfloat16, device=dev), None,
                          torch.ones(16, device=dev), FMT)
    ac = torch.empty((0, 32), dtype=torch.uint8, device=dev)
    asc = torch.empty((0, 1), dtype=torch.bfloat16, device=dev)
    Y = w4.linear(ac, asc, None, blob, FMT, 16, 64)
    assert Y.shape == (0, 16)
    with pytest.raises(w4.W4A4Error):
        w4.quantize_act_multi(torch.zeros((2, 64), dtype=torch.bfloat16, device=dev),
                              [torch.ones(64, device=dev)], FMT)
