"""GPU parity of the INT8 G=128 format with BF16 block scales (Appendix G.2,
Table 9's 8-bit integer W+A variant), through the C ABI.

Codes and scale bit patterns are compared with the oracle bit for bit; GEMM
outputs pass gates G1 (every element within the fp32-accumulation bound) and
G2 (row relative L2 error <= 1e-3), and are bit-exact where every partial
sum is exact (equal scales per operand).  Shapes reach every GEMM kernel:
M <= 3 the dot-product kernel while the rows fit 64 KiB of LDS (and the K on
either side of that bound, beyond it the MFMA decode kernel), M <= 16 the
MFMA decode kernel, 16 < M <= 32 the tile kernel with 32-row workgroup
tiles, larger M the 64-row tiles, with ragged M, N and K-block counts."""
import numpy as np
import pytest
import torch

from conftest import golden
import oracle
from oracle import formats as F
from gpu_common import device, say, bf16_bits, check_linear
import w4a4_block_scaled_amd as w4
from w4a4_block_scaled_amd import inputs

pytestmark = pytest.mark.gpu
FMT = "int8g128"


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


@pytest.mark.parametrize("M,K", [(1, 128), (3, 384), (37, 1152), (300, 4096), (5, 18944)])
@pytest.mark.parametrize("with_c", [False, True])
def test_quantize_matches_oracle(M, K, with_c):
    dev = device()
    say(f"[int8g128 quantize] M={M} K={K} c={with_c}")
    case = inputs.adhoc_case(FMT, M, 16, K, seed=M * 29 + K, weights="none")
    c = case.c if with_c else None
    gc, gs = gpu_quantize(case.x, c, dev)
    oc, os_ = oracle_quantize(case.x, c)
    assert np.array_equal(gs, os_), f"{(gs != os_).sum()} scales differ"
    assert np.array_equal(gc, oc), f"{(gc != oc).sum()} code bytes differ"


def test_quantize_continuous_column_scales():
    """c off the BF16 grid: x * c is a rounded fp32 product, and codes and
    scales still match the oracle's decisions on that product."""
    dev = device()
    rng = np.random.default_rng(6)
    case = inputs.adhoc_case(FMT, 64, 16, 2048, seed=6, weights="none")
    c = np.exp(rng.normal(0, 0.5, 2048)).astype(np.float32)
    gc, gs = gpu_quantize(case.x, c, dev)
    oc, os_ = oracle_quantize(case.x, c)
    assert np.array_equal(gs, os_) and np.array_equal(gc, oc)


def test_quantize_edge_values():
    """Half-integer ties, a scale tie (127 (1 + 2^-8) / 127 is a BF16
    midpoint), a subnormal scale that takes codes to -128 and 127, an
    underflowing scale, zeros, the largest values, and the non-finite
    convention."""
    dev = device()
    K = 128 * 6
    x = np.zeros((4, K), np.float32)
    x[0, :40] = (np.arange(-20, 20) + 0.5)
    x[0, 40] = 127.0
    x[0, 128] = 127.0                            # block 1: scale tie after c
    x[0, 129:134] = [1.5, -2.5, 3.5, -0.5, 126.5]
    x[1, 256] = np.float32(1.4 * 127 * 2.0 ** -133)   # Delta = 2^-133, codes past +-127
    x[1, 257] = -np.float32(1.4 * 127 * 2.0 ** -133)
    x[1, 384] = np.ldexp(1.0, -133)              # amax / 127 underflows to 0
    x[1, 512:516] = [3.3895314e38, -1e38, 1.0, -3.0]
    x[2, 640] = np.inf
    x[2, 700] = np.nan
    x[3] = np.linspace(-5, 5, K)
    xb = inputs.to_bf16(x)
    c = np.ones(K, np.float32)
    c[128] = np.float32(1.0 + 2.0 ** -8)
    for cc in (None, c):
        gc, gs = gpu_quantize(xb, cc, dev)
        oc, os_ = oracle_quantize(xb, cc)
        assert np.array_equal(gs, os_) and np.array_equal(gc, oc)
    assert os_[0, 1] == 0x3F80                   # the scale tie went to the even pattern (1.0)
    assert F.int8_value(oc[1, 257]) == -128 and F.int8_value(oc[1, 256]) == 127
    assert os_[2, 5] == 0x7FC0 and not oc[2, 640:768].any()


def test_golden_blocks_on_gpu():
    """The hand-worked blocks, whose values are fp32 but not all BF16: X is 1
    (BF16) where the block is nonzero and c carries the value, so x~ = 1 * c
    is the block's value exactly."""
    dev = device()
    g = golden("int8g128_blocks.json")
    for blk in g["blocks"]:
        x = np.zeros((1, 128), np.float32)
        c = np.ones(128, np.float32)
        for k, v in blk["x"].items():
            x[0, int(k)] = 1.0
            c[int(k)] = v
        codes, scales = gpu_quantize(inputs.to_bf16(x), c, dev)
        want = np.zeros(128, int)
        for k, v in blk["codes"].items():
            want[int(k)] = v
        assert int(scales[0, 0]) == blk["delta_bits"], blk["name"]
        assert np.array_equal(F.int8_value(codes[0]).astype(int), want), blk["name"]


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (4096, 14336)])
def test_pack_unpack_round_trip(N, K):
    dev = device()
    rng = np.random.default_rng(N + K)
    codes, sbits = inputs.random_codes(rng, N, K, 128, -20, 20, FMT)
    r = rng.uniform(0.5, 2, N).astype(np.float32)
    blob = w4.pack_weight(torch.from_numpy(codes).to(dev), bf16_dev(sbits, dev), None,
                          torch.from_numpy(r).to(dev), FMT)
    c2, s2, r2, t2 = w4.unpack_weight(blob, FMT, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(c2.cpu().numpy(), codes)
    assert np.array_equal(bits16(s2), sbits)
    assert np.array_equal(r2.cpu().numpy(), r) and float(t2.item()) == 1.0
    assert blob.numel() == w4.packed_weight_bytes(FMT, N, K)


def test_pack_fragment_order():
    """Lane l of the 2 KiB tile (g, s) holds row 16 g + l % 16, K 128 s + 16 c
    .. +16 and 128 s + 64 + 16 c .. +16 with c = l / 16; the scales sit at
    [g][s][row % 16] (checked against these index formulas on codes and
    scales whose values encode their position)."""
    dev = device()
    N, K = 32, 384
    rows = np.arange(N)[:, None]
    cols = np.arange(K)[None, :]
    codes = ((rows * 7 + cols * 13) % 251).astype(np.uint8)
    KS = K // 128
    sbits = (0x3F00 + np.arange(N)[:, None] * KS + np.arange(KS)[None, :]).astype(np.uint16)
    blob = w4.pack_weight(torch.from_numpy(codes).to(dev), bf16_dev(sbits, dev), None,
                          torch.ones(N, device=dev), FMT).cpu().numpy()
    tiles = blob[256:256 + N * K].reshape(N // 16, KS, 64, 32)
    for g in range(N // 16):
        for s in range(KS):
            for l in range(64):
                r, c = 16 * g + l % 16, l // 16
                want = np.concatenate([codes[r, 128 * s + 16 * c:128 * s + 16 * c + 16],
                                       codes[r, 128 * s + 64 + 16 * c:128 * s + 64 + 16 * c + 16]])
                assert np.array_equal(tiles[g, s, l], want), (g, s, l)
    off = (256 + N * K + 255) // 256 * 256
    packed = blob[off:off + N * KS * 2].view(np.uint16).reshape(N // 16, KS, 16)
    for n in range(N):
        for s in range(KS):
            assert packed[n // 16, s, n % 16] == sbits[n, s]


def run_case(case, dev, label):
    """Quantize (checked against the oracle), pack, GEMM; oracle on every output."""
    if case.w_prescaled is not None:
        wc, ws, _ = oracle.quantize_weight(case.w_prescaled.float().numpy(), FMT)
    else:
        wc, ws = case.w_codes, case.w_scales
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


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 9, 16, 17, 32, 33, 64, 100, 130, 300])
@pytest.mark.parametrize("N,K", [(48, 384), (272, 1152), (528, 4096)])
def test_linear_matches_oracle(M, N, K):
    dev = device()
    say(f"[int8g128 linear] M={M} N={N} K={K}")
    case = inputs.adhoc_case(FMT, M, N, K, seed=M * 7 + N + K)
    (elem, row), _, _ = run_case(case, dev, f"int8g128 {M}x{N}x{K}")
    say(f"    max elementwise rel err {elem:.2e}, max row rel-L2 {row:.2e}")


# many 16-feature groups (the dot kernel's 8-wave workgroups), a long K, and
# the K on either side of the dot kernel's 64 KiB LDS bound for 1, 2, 3 rows
@pytest.mark.parametrize("M,N,K", [(1, 16400, 640), (3, 16384, 512), (2, 64, 14336), (8, 16400, 640),
                                   (12, 64, 14336), (16, 4096, 4096), (1, 16, 64512),
                                   (1, 16, 64640), (2, 16, 32256), (2, 16, 32384), (3, 16, 21504),
                                   (3, 16, 21632), (40, 16400, 256)])
def test_linear_kernel_bounds(M, N, K):
    dev = device()
    say(f"[int8g128 bounds] M={M} N={N} K={K}")
    case = inputs.adhoc_case(FMT, M, N, K, seed=M + N + K)
    run_case(case, dev, f"int8g128 {M}x{N}x{K}")


@pytest.mark.parametrize("M", [1, 3, 7, 150])
def test_linear_random_codes(M):
    """Weight codes uniform over all 256 bytes (-128 included) with BF16 block
    scales spread over 2^-6 .. 2^1 with random mantissas."""
    dev = device()
    say(f"[int8g128 random codes] M={M}")
    case = inputs.adhoc_case(FMT, M, 272, 1024, seed=60 + M, weights="codes")
    run_case(case, dev, f"int8g128 random codes M={M}")


@pytest.mark.parametrize("M,N,K", [(1, 1040, 1024), (3, 16400, 512), (5, 272, 1024), (16, 16400, 512),
                                   (20, 272, 1024), (70, 528, 1024)])
def test_linear_bit_exact_with_equal_scales(M, N, K):
    """All activation scales equal and all weight scales equal (powers of
    two), r a power of two: every block sum is an integer below 2^21 and every
    fp32 partial sum an integer below 2^24 times one factor, so the output
    equals the oracle's bit for bit (gate G0)."""
    dev = device()
    say(f"[int8g128 G0] M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    case = inputs.LinearCase("adhoc", "g0", FMT, M, N, K, inputs.to_bf16(np.zeros((M, K), np.float32)),
                             np.ones(K, np.float32), np.ldexp(1.0, rng.integers(-2, 3, N)).astype(np.float32))
    a_codes = rng.integers(0, 256, (M, K), dtype=np.uint8)
    a_sc = np.full((M, K // 128), 0x3E80, np.uint16)            # 0.25
    w_codes = rng.integers(0, 256, (N, K), dtype=np.uint8)
    w_sc = np.full((N, K // 128), 0x4000, np.uint16)            # 2
    blob = w4.pack_weight(torch.from_numpy(w_codes).to(dev), bf16_dev(w_sc, dev), None,
                          torch.from_numpy(case.r).to(dev), FMT)
    Y = w4.linear(torch.from_numpy(a_codes).to(dev), bf16_dev(a_sc, dev), None, blob, FMT, N, K)
    bits, _ = oracle.linear_bf16(a_codes, a_sc, None, w_codes, w_sc, 1.0, case.r, FMT)
    got = bf16_bits(Y)
    assert np.array_equal(got, bits), f"{(got != bits).sum()} of {bits.size} outputs differ"


def test_dot_and_decode_kernels_agree():
    """M = 3 runs the dot-product kernel and M = 4 the MFMA decode kernel: on
    the same first three rows both pass the gates and repeated calls are
    identical."""
    dev = device()
    case = inputs.adhoc_case(FMT, 4, 528, 4096, seed=8)
    (_, y4, _) = run_case(case, dev, "decode")
    case3 = inputs.adhoc_case(FMT, 4, 528, 4096, seed=8)
    case3.M = 3
    case3.x = case3.x[:3]
    (_, y3, _) = run_case(case3, dev, "dot")
    (_, y3b, _) = run_case(case3, dev, "dot again")
    assert np.array_equal(y3, y3b)
    diff = np.abs(F.bf16_value(y3) - F.bf16_value(y4[:3]))
    assert diff.max() <= 2.0 ** -6 * np.abs(F.bf16_value(y4[:3])).max()


def test_decode_and_tile_kernels_agree():
    """M = 16 runs the MFMA decode kernel and M = 17 the tile kernel: on the
    same first 16 rows both pass the gates and repeated calls are
    identical."""
    dev = device()
    case = inputs.adhoc_case(FMT, 17, 272, 1152, seed=5)
    (_, y17, _) = run_case(case, dev, "tile")
    case16 = inputs.adhoc_case(FMT, 17, 272, 1152, seed=5)
    case16.M = 16
    case16.x = case16.x[:16]
    (_, y16, _) = run_case(case16, dev, "decode")
    (_, y16b, _) = run_case(case16, dev, "decode again")
    assert np.array_equal(y16, y16b)
    diff = np.abs(F.bf16_value(y16) - F.bf16_value(y17[:16]))
    assert diff.max() <= 2.0 ** -6 * np.abs(F.bf16_value(y17[:16])).max()


def test_lds_kernels_agree():
    """M = 128 runs the 128-row LDS-staged kernel (one wave per SIMD) and
    M = 200 the 256-row one (two waves per SIMD): both add every output's
    block sums in the same order with the same operations, so the first 128
    rows are bit-identical, and both pass the gates."""
    dev = device()
    case = inputs.adhoc_case(FMT, 200, 528, 4096, seed=11)
    (_, y200, _) = run_case(case, dev, "lds 256-row tiles")
    case128 = inputs.adhoc_case(FMT, 200, 528, 4096, seed=11)
    case128.M = 128
    case128.x = case128.x[:128]
    (_, y128, _) = run_case(case128, dev, "lds 128-row tiles")
    assert np.array_equal(y128, y200[:128])


@pytest.mark.parametrize("M", [1, 3, 16, 2048])
@pytest.mark.parametrize("name", ["qkv", "gate_up", "down"])
def test_full_size_llama_sampled(M, name):
    """Llama shapes at their full size, in the launch configuration the
    benchmark times: the weight codes and scales the GPU quantizer made from
    the prescaled weights equal the oracle's on sampled rows, so do the
    activation codes and scales, and the sampled outputs pass the gates."""
    dev = device()
    case = inputs.workload_cases("llama_int8g128", M=M, linears=[name])[0]
    say(f"[int8g128 full] {name} M={M} N={case.N} K={case.K}")
    wc, ws, _ = w4.quantize_act(case.w_prescaled.to(dev), None, FMT)
    blob = w4.pack_weight(wc, ws, None, torch.from_numpy(case.r).to(dev), FMT)
    ac, asc, ta = w4.quantize_act(case.x.to(dev), torch.from_numpy(case.c).to(dev), FMT)
    Y = w4.linear(ac, asc, ta, blob, FMT, case.N, case.K)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 6), replace=False)]))
    cols = np.unique(np.concatenate([np.arange(16), np.arange(case.N - 16, case.N),
                                     rng.choice(case.N, 48, replace=False)]))
    xs = case.x[torch.from_numpy(rows)]
    a_o, as_o, _ = oracle.quantize_act(xs.float().numpy(), case.c, FMT)
    assert np.array_equal(ac.cpu().numpy()[rows], a_o) and np.array_equal(bits16(asc)[rows], as_o)
    wo, wso, _ = oracle.quantize_weight(case.w_prescaled[torch.from_numpy(cols)].float().numpy(), FMT)
    assert np.array_equal(wc.cpu().numpy()[cols], wo) and np.array_equal(bits16(ws)[cols], wso)
    bits, y = oracle.linear_bf16(a_o, as_o, None, wo, wso, 1.0, case.r[cols], FMT)
    S = oracle.linear.linear_abs_sum(a_o, as_o, None, wo, wso, 1.0, case.r[cols], FMT)
    check_linear(bf16_bits(Y)[np.ix_(rows, cols)], y, S, case.K, f"full {name} M={M}")
    del Y, blob


def test_empty_batch_and_rejected_calls():
    dev = device()
    blob = w4.pack_weight(torch.zeros((16, 128), dtype=torch.uint8, device=dev),
                          torch.ones((16, 1), dtype=torch.bfloat16, device=dev), None,
                          torch.ones(16, device=dev), FMT)
    ac = torch.empty((0, 128), dtype=torch.uint8, device=dev)
    asc = torch.empty((0, 1), dtype=torch.bfloat16, device=dev)
    Y = w4.linear(ac, asc, None, blob, FMT, 16, 128)
    assert Y.shape == (0, 16)
    with pytest.raises(w4.W4A4Error):
        w4.quantize_act_multi(torch.zeros((2, 128), dtype=torch.bfloat16, device=dev),
                              [torch.ones(128, device=dev)], FMT)
    with pytest.raises(w4.W4A4Error):
        w4.linear_noalloc(torch.zeros((2, 128), dtype=torch.uint8, device=dev),
                          torch.ones((2, 1), dtype=torch.bfloat16, device=dev), None, blob, FMT, 16, 128)
