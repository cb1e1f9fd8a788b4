"""GPU parity of w4a4_quantize_act (codes, scales, tensor scale) against the
oracle: bit-exact, on seeded inputs of several shapes, the hand-worked golden
blocks, edge values and the full activation tensors of every workload."""
import numpy as np
import pytest
import torch

from conftest import golden
import oracle
from oracle import formats as F
from gpu_common import device, say, to_dev, gpu_quantize
from w4a4_block_scaled_amd import inputs
import w4a4_block_scaled_amd as w4

pytestmark = pytest.mark.gpu
FMTS = ["mxfp4", "nvfp4", "mxint4"]


def _compare(x, c, fmt, label):
    dev = device()
    codes, scales, t = gpu_quantize(x, c, fmt, dev)
    xf = x.float().numpy()
    cc = np.ones(xf.shape[1], np.float32) if c is None else c
    oc, os_, ot = oracle.quantize_act(xf, cc, fmt)
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    if fmt == "nvfp4":
        gt = float(t.cpu().numpy()[0])
        assert gt == float(ot), f"{label}: tensor scale {gt!r} != {float(ot)!r}"
    if not np.array_equal(gs, os_):
        i = np.argwhere(gs != os_)[0]
        raise AssertionError(f"{label}: scale mismatch at {tuple(i)}: gpu {gs[tuple(i)]} oracle {os_[tuple(i)]} "
                             f"({(gs != os_).sum()} total)")
    if not np.array_equal(gc, oc):
        i = np.argwhere(gc != oc)[0]
        raise AssertionError(f"{label}: code mismatch at {tuple(i)}: gpu {gc[tuple(i)]:#04x} oracle {oc[tuple(i)]:#04x} "
                             f"({(gc != oc).sum()} total)")
    return codes, scales, t


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,K", [(1, 32), (5, 96), (16, 256), (37, 1024), (300, 4096), (64, 18944)])
def test_quantize_matches_oracle(fmt, M, K):
    if K % oracle.BLOCK[fmt]:
        pytest.skip("K not a multiple of the block")
    say(f"[quantize] {fmt} M={M} K={K}")
    case = inputs.adhoc_case(fmt, M, 16, K, seed=100 + M + K, weights="none")
    _compare(case.x, case.c, fmt, f"{fmt} {M}x{K}")


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_without_column_scales(fmt):
    case = inputs.adhoc_case(fmt, 33, 16, 512, seed=7, weights="none")
    _compare(case.x, None, fmt, f"{fmt} c=None")


def test_golden_blocks_on_gpu():
    dev = device()
    g = golden("mxfp4_block.json")
    for cs in g["cases"]:
        x = torch.tensor([g["x"]], dtype=torch.float32).to(torch.bfloat16)
        codes, scales, _ = gpu_quantize(x, np.full(32, cs["c"], np.float32), "mxfp4", dev)
        assert codes.cpu().numpy()[0].tolist() == g["packed"]
        assert scales.cpu().numpy()[0].tolist() == [cs["scale"]]
    g = golden("mxint4_block.json")
    x = torch.tensor([g["x"]], dtype=torch.float32).to(torch.bfloat16)
    codes, scales, _ = gpu_quantize(x, np.ones(32, np.float32), "mxint4", dev)
    assert oracle.unpack_nibbles(codes.cpu().numpy())[0].tolist() == g["codes"]
    assert scales.cpu().numpy()[0].tolist() == [g["scale"]]
    g = golden("nvfp4_blocks.json")
    x = torch.tensor([g["x"]], dtype=torch.float32).to(torch.bfloat16)
    codes, scales, t = gpu_quantize(x, np.ones(32, np.float32), "nvfp4", dev)
    assert float(t.cpu()[0]) == g["t"]
    assert scales.cpu().numpy()[0].tolist() == g["scales"]
    assert oracle.unpack_nibbles(codes.cpu().numpy())[0].tolist() == g["codes"]


def _edge_tensor(fmt, rng):
    G = oracle.BLOCK[fmt]
    K = 16 * G
    x = (rng.standard_normal((8, K)) * 3).astype(np.float32)
    x[0, :G] = 0.0                                             # all-zero block
    x[0, G:2 * G] = -0.0                                       # negative zeros
    x[1, :G] = np.float32(2.0 ** -133) * rng.integers(-3, 4, G)   # bf16 subnormals
    x[1, G:2 * G] = np.float32(2.0 ** -126) * rng.integers(-100, 100, G)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.5, -0.25, -2.5, -5.0, 0.5, 3.0, 4.0, -6.0])
    x[2, :16] = ties
    x[2, 16:G] = 0.0
    x[3, :G] = 3.0e38 * np.sign(rng.standard_normal(G))       # near the bf16 maximum
    x[4, :G] = np.float32(2.0 ** 100)                          # constant block
    x[5, :] = x[5, :] * np.float32(2.0 ** -60)
    return torch.from_numpy(x).to(torch.bfloat16)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_edge_values(fmt):
    x = _edge_tensor(fmt, np.random.default_rng(11))
    if fmt == "nvfp4":
        x[3] = x[3] * 0  # keep the tensor amax moderate so that ties stay ties
    _compare(x, np.ones(x.shape[1], np.float32), fmt, f"{fmt} edge")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxint4"])
def test_quantize_nonfinite_convention(fmt):
    x = torch.randn(4, 128).to(torch.bfloat16)
    x[0, 5] = float("inf")
    x[1, 70] = float("nan")
    x[2, 127] = float("-inf")
    _compare(x, np.ones(128, np.float32), fmt, f"{fmt} nonfinite")


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_empty(fmt):
    dev = device()
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=dev)
    codes, scales, t = w4.quantize_act(x, None, fmt)
    torch.cuda.synchronize()
    assert codes.shape == (0, 128)
    if fmt == "nvfp4":
        assert float(t.cpu()[0]) == 1.0


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_deterministic(fmt):
    dev = device()
    case = inputs.adhoc_case(fmt, 129, 16, 2048, seed=5, weights="none")
    a = gpu_quantize(case.x, case.c, fmt, dev)
    b = gpu_quantize(case.x, case.c, fmt, dev)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


FULL = [("llama_prefill", 2048, ("qkv", "down")), ("llama_nvfp4", 4096, ("qkv", "down")),
        ("qwen_mxint4", 4096, ("qkv", "down")), ("llama_decode", 16, ("qkv", "down")),
        ("single", 16, ("single",))]


@pytest.mark.parametrize("workload,M,lins", FULL)
def test_quantize_full_activation_tensors(workload, M, lins):
    """Full activation tensors of each workload (the two distinct K of each
    model), compared bit for bit."""
    for case in inputs.workload_cases(workload, M=M, linears=lins, build_weights=False):
        say(f"[quantize full] {workload} {case.name} M={case.M} K={case.K}")
        _compare(case.x, case.c, case.fmt, f"{workload}/{case.name}")


def test_mxfp4_ties_at_many_scales():
    """Every E2M1 midpoint (and its negative) at block exponents from -100 to
    +100: codes and scales bit-exact against the oracle (ties to the even
    code, saturation at 6, sign kept on values that round to zero)."""
    dev = device()
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 0.125, 7.0, 1.0, 3.0], np.float64)
    rows = []
    for k in range(-100, 101, 7):
        blk = np.zeros(32, np.float64)
        blk[:12] = mids
        blk[12:24] = -mids
        blk[24] = 7.5                      # fixes the block exponent at 0 before scaling
        rows.append(blk * 2.0 ** k)
    x = torch.from_numpy(np.array(rows, np.float32)).to(torch.bfloat16)
    _compare(x, np.ones(32, np.float32), "mxfp4", "mxfp4 ties")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxint4", "mxfp8", "mxint8"])
@pytest.mark.parametrize("M,K", [(1, 96), (17, 1024), (300, 4096)])
def test_quantize_writes_only_its_outputs(fmt, M, K):
    """codes and scales live inside larger buffers holding a sentinel: the
    quantizer writes exactly their bytes (ragged M, K not a multiple of 256)."""
    if K % oracle.BLOCK[fmt]:
        pytest.skip("K not a multiple of the block")
    dev = device()
    case = inputs.adhoc_case(fmt, M, 16, K, seed=300 + M + K, weights="none")
    ref_codes, ref_scales, ref_t = gpu_quantize(case.x, case.c, fmt, dev)
    guard = 1024
    nc, ns = ref_codes.numel(), ref_scales.numel()
    cbuf = torch.full((guard + nc + guard,), 0xA5, dtype=torch.uint8, device=dev)
    sbuf = torch.full((guard + ns + guard,), 0xA5, dtype=torch.uint8, device=dev)
    codes = cbuf[guard:guard + nc].view(ref_codes.shape)
    scales = sbuf[guard:guard + ns].view(ref_scales.shape)
    t = torch.ones(1, dtype=torch.float32, device=dev)
    w4.quantize_act(to_dev(case.x, dev), to_dev(case.c, dev), fmt, out=(codes, scales, t))
    torch.cuda.synchronize()
    for b, n in ((cbuf.cpu().numpy(), nc), (sbuf.cpu().numpy(), ns)):
        assert np.all(b[:guard] == 0xA5) and np.all(b[guard + n:] == 0xA5), "write outside the outputs"
    assert torch.equal(codes, ref_codes) and torch.equal(scales, ref_scales)


def _midpoint_products(fmt, rng, n=64):
    """(x bf16 values, c fp32) pairs whose exact product is off an
    element-grid midpoint (E2M1 midpoints 0.25, 0.75, ..., 5, or integer + 0.5
    for INT4, with the block scale at 2^0) but whose fp32 product rounds onto
    it: the rescale's single fp32 rounding decides a tie.  c = fp32(t / x)
    for a bf16 x and a midpoint t."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] if fmt == "mxfp4" else
                    [0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5])
    trials = 4096
    x = torch.from_numpy(np.exp(rng.normal(0, 0.7, trials)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    x = x * rng.choice([-1.0, 1.0], trials).astype(np.float32)
    tgt = (mids[rng.integers(0, len(mids), trials)] * np.sign(x)).astype(np.float32)
    c = (tgt / x).astype(np.float32)
    hit = ((x * c).astype(np.float32) == tgt) & (x.astype(np.float64) * c.astype(np.float64) != tgt)
    assert hit.sum() >= n
    return x[hit][:n], c[hit][:n]


@pytest.mark.parametrize("fmt", ["mxfp4", "mxint4"])
def test_quantize_continuous_column_scales(fmt):
    """c off the E8M0 grid (lognormal fp32 values): x~ = fp32(x * c) is a
    rounded product, and codes must still equal the oracle's bit for bit,
    including products that round onto an element-grid midpoint (ties)."""
    rng = np.random.default_rng(17)
    case = inputs.adhoc_case(fmt, 64, 16, 2048, seed=17, weights="none")
    c = np.exp(rng.normal(0, 0.5, 2048)).astype(np.float32)
    _compare(case.x, c, fmt, f"{fmt} continuous c")
    xs, cs = _midpoint_products(fmt, rng)
    K = 32 * len(xs)
    x = np.zeros((1, K), np.float32)
    cc = np.ones(K, np.float32)
    for i, (xv, cv) in enumerate(zip(xs, cs)):
        x[0, 32 * i] = xv
        x[0, 32 * i + 1] = 6.0            # the block amax is 6 (or the tie itself, <= 6.5): scale 2^0
        cc[32 * i] = cv
    xb = torch.from_numpy(x).to(torch.bfloat16)
    _compare(xb, cc, fmt, f"{fmt} midpoint ties")
