"""GPU parity of the whole hot path (quantize_act -> pack_weight -> linear)
against the oracle: small shapes spanning several tiles with ragged tails
(all outputs compared), bit-exact cases, the golden block, every workload at
its full size on sampled outputs, decode-vs-tile agreement, determinism."""
import numpy as np
import pytest
import torch

from conftest import golden
import oracle
from oracle import formats as F
from oracle.quant import quantize_rows, rescale, nv_tensor_scale, pack_nibbles, pack_codes
from gpu_common import device, say, to_dev, bf16_bits, check_linear
from w4a4_block_scaled_amd import inputs
import w4a4_block_scaled_amd as w4

pytestmark = pytest.mark.gpu
FMTS = ["mxfp4", "nvfp4", "mxint4"]


def gpu_layer(case, dev):
    """Run the hot path on the GPU for one case; returns (Y bits, blob, act tensors)."""
    if case.w_codes is not None:
        wc, ws = to_dev(case.w_codes, dev), to_dev(case.w_scales, dev)
        tw = torch.tensor([case.t_w], dtype=torch.float32, device=dev)
    else:
        wc, ws, tw = w4.quantize_act(to_dev(case.w_prescaled, dev), None, case.fmt)
    blob = w4.pack_weight(wc, ws, tw, to_dev(case.r, dev), case.fmt)
    ac, as_, ta = w4.quantize_act(to_dev(case.x, dev), to_dev(case.c, dev), case.fmt)
    Y = w4.linear(ac, as_, ta, blob, case.fmt, case.N, case.K)
    torch.cuda.synchronize()
    return Y, blob, (ac, as_, ta), (wc, ws, tw)


def oracle_layer(case, rows=None, cols=None):
    """Oracle on the selected output rows/cols; returns (y fp64, S, act codes/scales, w codes/scales)."""
    fmt = case.fmt
    x = case.x.float().numpy()
    rows = np.arange(case.M) if rows is None else np.asarray(rows)
    cols = np.arange(case.N) if cols is None else np.asarray(cols)
    xt_full = rescale(x, case.c)
    t_a = nv_tensor_scale(xt_full) if fmt == "nvfp4" else None
    a_codes, a_scales, _ = quantize_rows(xt_full[rows], fmt, t=t_a)
    a_codes = pack_codes(a_codes, fmt)
    if case.w_codes is not None:
        w_codes, w_scales, t_w = case.w_codes[cols], case.w_scales[cols], np.float32(case.t_w)
    else:
        w = case.w_prescaled.float().numpy()
        t_w = nv_tensor_scale(w) if fmt == "nvfp4" else np.float32(1.0)
        wc, w_scales, _ = quantize_rows(w[cols], fmt, t=t_w if fmt == "nvfp4" else None)
        w_codes = pack_codes(wc, fmt)
    r = case.r[cols]
    y = oracle.linear_f64(a_codes, a_scales, t_a, w_codes, w_scales, t_w, r, fmt)
    S = oracle.linear.linear_abs_sum(a_codes, a_scales, t_a, w_codes, w_scales, t_w, r, fmt)
    return y, S, (a_codes, a_scales, t_a), (w_codes, w_scales, t_w)


SMALL = [(1, 16, 128), (5, 272, 640), (16, 512, 1152), (17, 144, 384), (129, 272, 640),
         (300, 400, 1152), (64, 1024, 4096), (3, 528, 6144), (9, 1040, 7168), (12, 528, 14336),
         (9, 16448, 640), (16, 16384, 4096), (7, 6176, 512), (2, 1040, 1152), (2, 16448, 640)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", SMALL)
def test_linear_matches_oracle(fmt, M, N, K):
    dev = device()
    say(f"[linear] {fmt} M={M} N={N} K={K}")
    case = inputs.adhoc_case(fmt, M, N, K, seed=M * 31 + N + K)
    Y, *_ = gpu_layer(case, dev)
    y, S, _, _ = oracle_layer(case)
    elem, row = check_linear(bf16_bits(Y), y, S, K, f"{fmt} {M}x{N}x{K}")
    say(f"    max elementwise rel err {elem:.2e}, max row rel-L2 {row:.2e}")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxint4"])
@pytest.mark.parametrize("M,N,K", [(16, 256, 4096), (200, 272, 18944), (1, 64, 14336)])
def test_linear_bit_exact_when_accumulation_is_exact(fmt, M, N, K):
    """All block scales of an operand equal: every fp32 partial sum is exact
    (|sum| < 2^24 units), so the output must equal the oracle bit for bit."""
    dev = device()
    say(f"[bit-exact] {fmt} M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    G = 32
    case = inputs.adhoc_case(fmt, M, N, K, seed=3, weights="none")
    case.w_codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    case.w_scales = np.full((N, K // G), 125, np.uint8)
    case.r = np.ldexp(1.0, rng.integers(-3, 4, N)).astype(np.float32)
    a_codes = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    a_scales = np.full((M, K // G), 129, np.uint8)
    blob = w4.pack_weight(to_dev(case.w_codes, dev), to_dev(case.w_scales, dev), None,
                          to_dev(case.r, dev), fmt)
    Y = w4.linear(to_dev(a_codes, dev), to_dev(a_scales, dev), None, blob, fmt, N, K)
    bits, _ = oracle.linear_bf16(a_codes, a_scales, None, case.w_codes, case.w_scales, 1.0, case.r, fmt)
    got = bf16_bits(Y)
    assert np.array_equal(got, bits), f"{(got != bits).sum()} of {bits.size} outputs differ"


def test_golden_single_block_on_gpu():
    """K = 32 is below the GEMM's 128 granularity: pad the block with three
    all-zero blocks (zero codes add nothing)."""
    dev = device()
    g = golden("linear_single_block.json")
    a = np.zeros((1, 128), np.uint8)
    w = np.zeros((16, 128), np.uint8)
    a[0, :32] = g["a_codes"]
    w[0, :32] = g["w_codes"]
    a_s = np.full((1, 4), 127, np.uint8)
    a_s[0, 0] = g["a_scale"]
    w_s = np.full((16, 4), 127, np.uint8)
    w_s[0, 0] = g["w_scale"]
    r = np.ones(16, np.float32)
    r[0] = g["r"]
    blob = w4.pack_weight(to_dev(pack_nibbles(w), dev), to_dev(w_s, dev), None, to_dev(r, dev), "mxfp4")
    Y = w4.linear(to_dev(pack_nibbles(a), dev), to_dev(a_s, dev), None, blob, "mxfp4", 16, 128)
    assert int(bf16_bits(Y)[0, 0]) == g["y_bf16_bits"]


def _sample(n, count, rng):
    base = [i for i in (0, 1, n - 1) if i < n]
    extra = rng.choice(n, size=min(count, n), replace=False).tolist()
    return np.array(sorted(set(base + extra)))


WORKLOADS = [("single", 16), ("llama_decode", 1), ("llama_decode", 4), ("llama_decode", 16),
             ("llama_prefill", 2048), ("llama_nvfp4", 16), ("llama_nvfp4", 4096), ("qwen_mxint4", 1),
             ("qwen_mxint4", 512), ("qwen_mxint4", 4096)]


@pytest.mark.parametrize("workload,M", WORKLOADS)
def test_workload_full_size(workload, M):
    """Every linear of the workload at its full size, in the launch
    configuration the benchmark times; the oracle computes sampled outputs
    (rows incl. the first and last, columns incl. a whole tile and the last
    one) from its own quantization of the same seeded inputs.  The
    activation codes of the sampled rows, and the weight codes, scales (and
    t_w) of the sampled weight rows, must equal the oracle's bit for bit."""
    dev = device()
    rng = np.random.default_rng(M)
    for case in inputs.workload_cases(workload, M=M):
        say(f"[workload] {workload} {case.name} M={case.M} N={case.N} K={case.K}")
        Y, blob, (ac, as_, ta), gpu_weights = gpu_layer(case, dev)
        rows = _sample(case.M, 12, rng)
        cols = np.unique(np.concatenate([np.arange(min(144, case.N)), _sample(case.N, 96, rng),
                                         np.arange(case.N - 16, case.N)]))
        y, S, (oa, osc, ota), (owc, ows, otw) = oracle_layer(case, rows, cols)
        # the GPU's activation codes of the sampled rows are the oracle's
        assert np.array_equal(ac.cpu().numpy()[rows], oa)
        assert np.array_equal(as_.cpu().numpy()[rows], osc)
        if case.w_prescaled is not None:
            # and so are the weight codes and scales the GPU quantizer made
            # from the prescaled weights (sampled weight rows), and t_w
            wc, ws, tw = gpu_weights
            assert np.array_equal(wc.cpu().numpy()[cols], owc), "weight codes differ from the oracle"
            assert np.array_equal(ws.cpu().numpy()[cols], ows), "weight scales differ from the oracle"
            if case.fmt == "nvfp4":
                assert float(tw.cpu().numpy()[0]) == float(otw)
        Yb = bf16_bits(Y)[np.ix_(rows, cols)]
        elem, row = check_linear(Yb, y, S, case.K, f"{workload}/{case.name}")
        say(f"    max elementwise rel err {elem:.2e}, max row rel-L2 {row:.2e}")
        del Y, blob


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_and_tile_kernels_agree(fmt):
    """M <= 16 runs the weight-streaming kernel, larger M the tiled one; the
    first 16 rows of an M = 40 call equal an M = 16 call within G1."""
    dev = device()
    case = inputs.adhoc_case(fmt, 40, 1024, 4096, seed=9)
    Y40, blob, (ac, as_, ta), _ = gpu_layer(case, dev)
    Y16 = w4.linear(ac[:16].contiguous(), as_[:16].contiguous(), ta, blob, fmt, case.N, case.K)
    torch.cuda.synchronize()
    a = F.bf16_value(bf16_bits(Y16))
    b = F.bf16_value(bf16_bits(Y40[:16]))
    y, S, _, _ = oracle_layer(case, rows=np.arange(16))
    check_linear(bf16_bits(Y16), y, S, case.K, "decode")
    check_linear(bf16_bits(Y40[:16]), y, S, case.K, "tile")
    assert np.max(np.abs(a - b)) <= np.max(2.0 ** -7 * np.abs(y) + 2 * (case.K + 2) * 2.0 ** -23 * S)


@pytest.mark.parametrize("fmt", FMTS)
def test_linear_deterministic(fmt):
    dev = device()
    case = inputs.adhoc_case(fmt, 70, 512, 2048, seed=21)
    Y1, blob, (ac, as_, ta), _ = gpu_layer(case, dev)
    Y2 = w4.linear(ac, as_, ta, blob, fmt, case.N, case.K)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)


@pytest.mark.parametrize("fmt", FMTS)
def test_linear_empty_batch(fmt):
    dev = device()
    case = inputs.adhoc_case(fmt, 3, 32, 256, seed=1)
    _, blob, (ac, as_, ta), _ = gpu_layer(case, dev)
    Y = w4.linear(ac[:0], as_[:0], ta, blob, fmt, case.N, case.K)
    assert Y.shape == (0, 32)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxint4", "mxfp8", "mxint8"])
@pytest.mark.parametrize("M,N,K", [(3, 528, 640), (17, 272, 1152), (130, 400, 384)])
def test_linear_writes_only_its_output(fmt, M, N, K):
    """Y lives inside a larger buffer whose surroundings hold a sentinel: the
    GEMM (decode and tiled kernels, ragged M and N) writes exactly M x N bf16
    values and no byte around them."""
    dev = device()
    case = inputs.adhoc_case(fmt, M, N, K, seed=M + N + K + 3)
    Y, blob, (ac, as_, ta), _ = gpu_layer(case, dev)
    guard = 4096
    buf = torch.full((guard + M * N * 2 + guard,), 0xA5, dtype=torch.uint8, device=dev)
    out = buf[guard:guard + M * N * 2].view(torch.bfloat16).view(M, N)
    w4.linear(ac, as_, ta, blob, fmt, N, K, out=out)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(b[:guard] == 0xA5) and np.all(b[guard + M * N * 2:] == 0xA5), "write outside Y"
    assert torch.equal(out, Y)


def _pack_into(buf, fmt, N, K, seed):
    """Pack random codes for (fmt, N, K) into the front of `buf` (a buffer
    larger than that blob) through the C ABI."""
    import ctypes
    dev = buf.device
    rng = np.random.default_rng(seed)
    cols = K if fmt in ("mxfp8", "mxint8") else K // 2
    codes = to_dev(rng.integers(0, 112, (N, cols), dtype=np.uint8), dev)
    scales = to_dev(np.full((N, K // oracle.BLOCK[fmt]), 120, np.uint8), dev)
    r = torch.ones(N, dtype=torch.float32, device=dev)
    L = w4.lib()
    st = L.w4a4_pack_weight(w4.FORMATS[fmt], N, K, ctypes.c_void_p(codes.data_ptr()),
                            ctypes.c_void_p(scales.data_ptr()), None, ctypes.c_void_p(r.data_ptr()),
                            ctypes.c_void_p(buf.data_ptr()),
                            ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    assert st == 0
    torch.cuda.synchronize()


# (format the blob is packed for, its N, K) -> (format, M, N, K of the call):
# other shape or other format; the calls reach the decode, tiled,
# persistent and split-K kernels
MISMATCH = [
    (("mxfp4", 256, 512), ("mxfp4", 4, 512, 1024)),
    (("mxfp4", 256, 512), ("mxfp4", 300, 256, 1024)),
    (("mxfp4", 12288, 512), ("mxfp4", 1024, 12288, 1024)),
    (("mxfp4", 8208, 4096), ("mxfp4", 300, 8208, 8192)),
    (("mxfp4", 256, 512), ("mxint4", 40, 256, 512)),
    (("mxint4", 256, 512), ("nvfp4", 3, 256, 512)),
    (("nvfp4", 256, 512), ("mxfp8", 70, 256, 512)),
    (("mxfp8", 256, 512), ("mxint8", 5, 256, 512)),
    (("mxfp8", 256, 512), ("mxint8", 1, 256, 512)),
    (("mxint8", 256, 512), ("mxfp8", 3, 256, 512)),
    (("mxint8", 256, 512), ("int8g128", 1, 256, 512)),
    (("mxfp8", 256, 512), ("int8g128", 40, 256, 1024)),
    (("mxint4", 256, 512), ("mxint4", 1, 256, 1024)),
    (("mxint4", 256, 512), ("nvfp4", 1, 256, 512)),
    (("mxint4", 256, 512), ("int4g64", 33, 256, 512)),
]


@pytest.mark.parametrize("packed,call", MISMATCH)
def test_blob_of_another_format_or_shape_gives_nan(packed, call):
    """The GEMM kernels check the blob header (magic, format, N, K) against
    their arguments before reading anything else of it: a blob packed for
    another format or shape yields an all-NaN Y, not a read past the blob.
    The blob sits at the front of a buffer as large as the call's own blob,
    so no read could leave it even if the check were missing."""
    dev = device()
    pf, pN, pK = packed
    fmt, M, N, K = call
    say(f"[blob mismatch] packed {pf} {pN}x{pK}, called {fmt} M={M} N={N} K={K}")
    size = max(w4.packed_weight_bytes(f, N, K) for f in ("mxfp8", fmt))
    buf = torch.zeros(size + 256, dtype=torch.uint8, device=dev)
    _pack_into(buf, pf, pN, pK, seed=M + N)
    x = torch.randn((M, K)).to(torch.bfloat16).to(dev)
    ac, as_, ta = w4.quantize_act(x, None, fmt)
    Y = torch.zeros((M, N), dtype=torch.bfloat16, device=dev)
    w4.linear(ac, as_, ta, buf, fmt, N, K, out=Y)
    torch.cuda.synchronize()
    assert torch.isnan(Y.float()).all(), "a mismatched blob did not give NaN"
