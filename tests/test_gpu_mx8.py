"""GPU parity of the 8-bit MX variants (MXFP8, MXINT8; DualQuant Appendix
G.2, Table 9) through the C ABI: activation codes and scales bit-exact
against the oracle (ragged shapes, with and without column scales, edge
values, the golden blocks, full Llama activations), pack/unpack round trips,
every output of small shapes that reach the decode and the tiled kernels
under gates G1/G2, bit-exactness where accumulation is exact, decode/tile
agreement, and the Llama workloads at full size on sampled outputs."""
import numpy as np
import pytest
import torch

from conftest import golden
import oracle
from oracle import formats as F
from gpu_common import device, say, to_dev, bf16_bits, check_linear, gpu_quantize
from test_gpu_linear import gpu_layer, oracle_layer, _sample
from w4a4_block_scaled_amd import inputs
import w4a4_block_scaled_amd as w4

pytestmark = pytest.mark.gpu
FMTS = ["mxfp8", "mxint8"]


def _compare_quant(x, c, fmt, label):
    dev = device()
    codes, scales, _ = gpu_quantize(x, c, fmt, dev)
    xf = x.float().numpy()
    cc = np.ones(xf.shape[1], np.float32) if c is None else c
    oc, os_, _ = oracle.quantize_act(xf, cc, fmt)
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    assert gc.shape == oc.shape and gs.shape == os_.shape
    if not np.array_equal(gs, os_):
        i = np.argwhere(gs != os_)[0]
        raise AssertionError(f"{label}: scale mismatch at {tuple(i)}: gpu {gs[tuple(i)]} oracle {os_[tuple(i)]}")
    if not np.array_equal(gc, oc):
        i = np.argwhere(gc != oc)[0]
        raise AssertionError(f"{label}: code mismatch at {tuple(i)}: gpu {gc[tuple(i)]:#04x} "
                             f"oracle {oc[tuple(i)]:#04x} x={xf[tuple(i)]!r} ({(gc != oc).sum()} total)")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,K", [(1, 32), (5, 96), (37, 1024), (300, 4096), (17, 14336)])
def test_mx8_quantize_matches_oracle(fmt, M, K):
    say(f"[mx8 quantize] {fmt} M={M} K={K}")
    case = inputs.adhoc_case(fmt, M, 16, K, seed=200 + M + K, weights="none")
    _compare_quant(case.x, case.c, fmt, f"{fmt} {M}x{K}")
    _compare_quant(case.x, None, fmt, f"{fmt} {M}x{K} c=None")


@pytest.mark.parametrize("fmt", FMTS)
def test_mx8_quantize_continuous_column_scales(fmt):
    """c not on the E8M0 grid: x * c is a rounded fp32 product, and the codes
    still match the oracle's decision on that product."""
    rng = np.random.default_rng(5)
    case = inputs.adhoc_case(fmt, 64, 16, 2048, seed=5, weights="none")
    c = np.exp(rng.normal(0, 0.5, 2048)).astype(np.float32)
    _compare_quant(case.x, c, fmt, f"{fmt} continuous c")


@pytest.mark.parametrize("fmt", FMTS)
def test_mx8_quantize_edge_values(fmt):
    """E4M3 ties and saturation, int8 ties and the +128 clip, subnormals,
    signed zeros, all-zero blocks, huge and tiny blocks."""
    x = np.zeros((4, 128), np.float32)
    x[0, :12] = [17.0, 19.0, 1.0625, -3.0, 448.0, 464.0, 500.0, -0.0, 0.0009765625,
                 -0.000732421875, 240.0, -496.0]
    x[1, :8] = [127.5, -127.5, 2.5, 3.5, -0.5, 64.0, 100.5, -0.25]
    x[1, 32:36] = [2.0 ** -130, -(2.0 ** -133), 2.0 ** -126, 0.0]
    x[2, :4] = [3.0e38, -1.0e38, 1.0, -2.0]
    x[2, 64:68] = [1e-30, -3e-31, 5e-32, 0.0]
    x[3, 96:128] = -0.0
    xb = torch.from_numpy(x).to(torch.bfloat16)
    _compare_quant(xb, None, fmt, f"{fmt} edges")


@pytest.mark.parametrize("fmt", FMTS)
def test_mx8_golden_block_on_gpu(fmt):
    g = golden(f"{fmt}_block.json")
    x = torch.tensor([g["x"]], dtype=torch.float32).to(torch.bfloat16)
    codes, scales, _ = gpu_quantize(x, np.ones(32, np.float32), fmt, device())
    assert codes.cpu().numpy()[0].tolist() == g["codes"]
    assert scales.cpu().numpy()[0].tolist() == [g["scale"]]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (4096, 14336)])
def test_mx8_pack_round_trip(fmt, N, K):
    dev = device()
    rng = np.random.default_rng(N + K)
    codes, scales = inputs.random_codes(rng, N, K, 32, -20, 20, fmt)
    r = rng.standard_normal(N).astype(np.float32)
    blob = w4.pack_weight(to_dev(codes, dev), to_dev(scales, dev), None, to_dev(r, dev), fmt)
    c2, s2, r2, t2 = w4.unpack_weight(blob, fmt, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(c2.cpu().numpy(), codes)
    assert np.array_equal(s2.cpu().numpy(), scales)
    assert np.array_equal(r2.cpu().numpy(), r)


def test_mx8_pack_fragment_order():
    """Lane l of the 2 KiB tile (g, h) holds row 16 g + l % 16, K 128 h + 16 c
    .. +16 and 128 h + 64 + 16 c .. +16 with c = l / 16 (checked against this
    index formula on a code matrix whose bytes encode their position)."""
    dev = device()
    N, K = 32, 256
    rows = np.arange(N)[:, None]
    cols = np.arange(K)[None, :]
    codes = ((rows * 7 + cols * 13) % 251).astype(np.uint8)
    scales = np.full((N, K // 32), 127, np.uint8)
    blob = w4.pack_weight(to_dev(codes, dev), to_dev(scales, dev), None,
                          to_dev(np.ones(N, np.float32), dev), "mxfp8").cpu().numpy()
    KT = K // 128
    tiles = blob[256:256 + N * K].reshape(N // 16, KT, 64, 32)
    for g in range(N // 16):
        for h in range(KT):
            for l in range(64):
                r, c = 16 * g + l % 16, l // 16
                want = np.concatenate([codes[r, 128 * h + 16 * c:128 * h + 16 * c + 16],
                                       codes[r, 128 * h + 64 + 16 * c:128 * h + 64 + 16 * c + 16]])
                assert np.array_equal(tiles[g, h, l], want), (g, h, l)


SMALL = [(1, 16, 128), (5, 272, 640), (16, 512, 1152), (17, 144, 384), (129, 272, 640),
         (300, 400, 1152), (64, 1024, 4096), (3, 528, 6144), (2, 64, 14336),
         (1, 1040, 1152), (2, 528, 1152), (3, 1040, 1152)]

# one to three rows take the dot-product kernel while the rows (MXINT8: K
# bytes, MXFP8: 2K) and their K/32 scale bytes fit 64 KiB of LDS, the MFMA
# decode kernel beyond: the K on either side of that bound
LDS_BOUND = {"mxfp8": [(1, 32, 32256), (1, 32, 32384), (3, 32, 10752), (3, 32, 10880)],
             "mxint8": [(1, 16, 63488), (1, 16, 63616), (3, 16, 21120), (3, 16, 21248)]}


@pytest.mark.parametrize("fmt,M,N,K", [(f,) + s for f in FMTS for s in LDS_BOUND[f]])
def test_mx8_dot_kernel_lds_bound(fmt, M, N, K):
    dev = device()
    say(f"[mx8 lds bound] {fmt} M={M} N={N} K={K}")
    case = inputs.adhoc_case(fmt, M, N, K, seed=M + N + K)
    Y, *_ = gpu_layer(case, dev)
    y, S, _, _ = oracle_layer(case)
    check_linear(bf16_bits(Y), y, S, K, f"{fmt} {M}x{N}x{K}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", SMALL)
def test_mx8_linear_matches_oracle(fmt, M, N, K):
    dev = device()
    say(f"[mx8 linear] {fmt} M={M} N={N} K={K}")
    case = inputs.adhoc_case(fmt, M, N, K, seed=M * 31 + N + K)
    Y, *_ = gpu_layer(case, dev)
    y, S, _, _ = oracle_layer(case)
    elem, row = check_linear(bf16_bits(Y), y, S, K, f"{fmt} {M}x{N}x{K}")
    say(f"    max elementwise rel err {elem:.2e}, max row rel-L2 {row:.2e}")


@pytest.mark.parametrize("fmt", FMTS)
def test_mx8_linear_random_codes(fmt):
    """Codes uniform over the whole byte range (every E4M3 value incl.
    subnormals and +-448; every int8 incl. -128) and widely spread block
    scales, through both kernels."""
    dev = device()
    for M in (1, 3, 7, 150):
        say(f"[mx8 random codes] {fmt} M={M}")
        case = inputs.adhoc_case(fmt, M, 272, 1024, seed=40 + M, weights="codes")
        Y, *_ = gpu_layer(case, dev)
        y, S, _, _ = oracle_layer(case)
        check_linear(bf16_bits(Y), y, S, case.K, f"{fmt} random codes M={M}")


E4M3_INTS = [0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50, 0x51, 0x52, 0x53, 0x54, 0x55,
             0x56, 0x57, 0x58]          # E4M3 bytes of the integers 0..16


@pytest.mark.parametrize("fmt,M,N,K", [("mxfp8", 16, 256, 4096), ("mxfp8", 200, 272, 4096),
                                       ("mxint8", 5, 64, 512), ("mxint8", 130, 272, 512),
                                       ("mxfp8", 1, 1040, 4096), ("mxfp8", 3, 16400, 1152),
                                       ("mxint8", 1, 1040, 512), ("mxint8", 3, 16400, 640)])
def test_mx8_bit_exact_when_accumulation_is_exact(fmt, M, N, K):
    """Equal block scales per operand and element values that keep every
    partial sum an integer below 2^24 (MXFP8: the integers -16..16, so
    |sum| <= 256 K; MXINT8: |q| <= 128 and K = 512, so |sum| <= 2^23, also for
    the four split products): the fp32 accumulation is exact in any order and
    the output equals the oracle bit for bit."""
    dev = device()
    say(f"[mx8 bit-exact] {fmt} M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)

    def codes(rows):
        if fmt == "mxfp8":
            c = np.array(E4M3_INTS, np.uint8)[rng.integers(0, 17, (rows, K))]
            return (c | (rng.integers(0, 2, (rows, K)) << 7)).astype(np.uint8)
        return rng.integers(0, 256, (rows, K), dtype=np.uint8)

    w_codes, a_codes = codes(N), codes(M)
    w_scales = np.full((N, K // 32), 125, np.uint8)
    a_scales = np.full((M, K // 32), 129, np.uint8)
    r = np.ldexp(1.0, rng.integers(-3, 4, N)).astype(np.float32)
    blob = w4.pack_weight(to_dev(w_codes, dev), to_dev(w_scales, dev), None, to_dev(r, dev), fmt)
    Y = w4.linear(to_dev(a_codes, dev), to_dev(a_scales, dev), None, blob, fmt, N, K)
    bits, _ = oracle.linear_bf16(a_codes, a_scales, None, w_codes, w_scales, 1.0, r, fmt)
    got = bf16_bits(Y)
    assert np.array_equal(got, bits), f"{(got != bits).sum()} of {bits.size} outputs differ"


@pytest.mark.parametrize("fmt", FMTS)
def test_mx8_decode_and_tile_kernels_agree(fmt):
    dev = device()
    case = inputs.adhoc_case(fmt, 40, 1024, 4096, seed=9)
    Y40, blob, (ac, as_, ta), _ = gpu_layer(case, dev)
    Y16 = w4.linear(ac[:16].contiguous(), as_[:16].contiguous(), ta, blob, fmt, case.N, case.K)
    torch.cuda.synchronize()
    y, S, _, _ = oracle_layer(case, rows=np.arange(16))
    check_linear(bf16_bits(Y16), y, S, case.K, "decode")
    check_linear(bf16_bits(Y40[:16]), y, S, case.K, "tile")


@pytest.mark.parametrize("fmt", FMTS)
def test_mx8_dot_and_decode_kernels_agree(fmt):
    """Three activation rows go through the VALU dot-product kernel, four
    through the MFMA decode kernel: the first three rows' outputs of both
    pass G1/G2 against the oracle."""
    dev = device()
    case = inputs.adhoc_case(fmt, 4, 4096, 4096, seed=12)
    Y4, blob, (ac, as_, ta), _ = gpu_layer(case, dev)
    Y3 = w4.linear(ac[:3].contiguous(), as_[:3].contiguous(), ta, blob, fmt, case.N, case.K)
    torch.cuda.synchronize()
    y, S, _, _ = oracle_layer(case, rows=np.arange(3))
    check_linear(bf16_bits(Y3), y, S, case.K, "dot")
    check_linear(bf16_bits(Y4[:3]), y, S, case.K, "decode")


@pytest.mark.parametrize("workload,M", [("llama_mxfp8", 2048), ("llama_mxfp8", 1),
                                        ("llama_mxint8", 2048), ("llama_mxint8", 1),
                                        ("llama_mxfp8", 3), ("llama_mxint8", 3)])
def test_mx8_workload_full_size(workload, M):
    """Every Llama linear at full size in the launch configuration the
    benchmark times: the weight codes and scales the GPU quantizer made from
    the prescaled weights equal the oracle's on sampled rows, the activation
    codes of the sampled rows equal the oracle's, and the sampled outputs
    pass G1/G2."""
    dev = device()
    rng = np.random.default_rng(M + 8)
    for case in inputs.workload_cases(workload, M=M):
        say(f"[mx8 workload] {workload} {case.name} M={case.M} N={case.N} K={case.K}")
        Y, blob, (ac, as_, ta), (wc, ws, tw) = gpu_layer(case, dev)
        rows = _sample(case.M, 12, rng)
        cols = np.unique(np.concatenate([np.arange(min(272, case.N)), _sample(case.N, 96, rng),
                                         np.arange(case.N - 16, case.N)]))
        y, S, (oa, osc, _), (owc, ows, _) = oracle_layer(case, rows, cols)
        assert np.array_equal(ac.cpu().numpy()[rows], oa)
        assert np.array_equal(as_.cpu().numpy()[rows], osc)
        assert np.array_equal(wc.cpu().numpy()[cols], owc)
        assert np.array_equal(ws.cpu().numpy()[cols], ows)
        elem, row = check_linear(bf16_bits(Y)[np.ix_(rows, cols)], y, S, case.K, f"{workload}/{case.name}")
        say(f"    max elementwise rel err {elem:.2e}, max row rel-L2 {row:.2e}")
        del Y, blob


@pytest.mark.parametrize("fmt", FMTS)
def test_mx8_large_tiles_ragged(fmt):
    """A shape with at least 160 tiles of 256 x 256 takes the 8-wave
    256 x 256 tile kernel: M and N end inside a tile (the last row tile has
    20 rows, the last column tile 16 features); sampled outputs including the
    first and last 40 rows and 272 columns pass G1/G2, and the activation
    codes of the sampled rows equal the oracle's."""
    dev = device()
    M, N, K = 1300, 6928, 384
    assert ((N + 255) // 256) * ((M + 255) // 256) >= 160
    case = inputs.adhoc_case(fmt, M, N, K, seed=77)
    Y, blob, (ac, as_, ta), _ = gpu_layer(case, dev)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(40), _sample(M, 24, rng), np.arange(M - 40, M)]))
    cols = np.unique(np.concatenate([np.arange(272), _sample(N, 64, rng), np.arange(N - 272, N)]))
    y, S, (oa, osc, _), _ = oracle_layer(case, rows, cols)
    assert np.array_equal(ac.cpu().numpy()[rows], oa)
    assert np.array_equal(as_.cpu().numpy()[rows], osc)
    elem, row = check_linear(bf16_bits(Y)[np.ix_(rows, cols)], y, S, K, f"{fmt} {M}x{N}x{K}")
    say(f"    max elementwise rel err {elem:.2e}, max row rel-L2 {row:.2e}")


@pytest.mark.parametrize("fmt", FMTS)
def test_mx8_empty_and_noalloc(fmt):
    dev = device()
    case = inputs.adhoc_case(fmt, 9, 256, 512, seed=2)
    Y, blob, (ac, as_, ta), _ = gpu_layer(case, dev)
    assert w4.linear(ac[:0], as_[:0], ta, blob, fmt, case.N, case.K).shape == (0, 256)
    Y2 = w4.linear_noalloc(ac, as_, ta, blob, fmt, case.N, case.K)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)
