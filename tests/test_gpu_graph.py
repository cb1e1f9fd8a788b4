"""The hot path captured as a HIP graph: every replay equals the eager result.

The benchmark replays a captured step (quantize_act + linear per linear), so
the kernels must behave the same under replay: no memset nodes, no state
kept between calls.  Each case runs the path eagerly, captures the same
launches into preallocated outputs, then replays the graph several times
with other eager work and synchronizations in between, clearing the outputs
before each replay, and compares every replay bit for bit with the eager
run (all kernels are deterministic)."""
import pytest
import torch

from gpu_common import device, say, to_dev
from w4a4_block_scaled_amd import inputs
import w4a4_block_scaled_amd as w4

pytestmark = pytest.mark.gpu

# (format, M, N, K): the persistent MXFP4 GEMM (256 x 256 tiles, 256 x 192
# tiles, n halves), the split-K GEMM (with its workspace), the tile GEMM,
# the decode kernels (16-feature, one-group and two-group workgroups), the
# MXINT4 decode (M = 1 and 16), tile and small-tile GEMMs, the NVFP4 path (tensor amax pre-pass with
# its workspace, or the one-launch quantizer; tile, MFMA decode and dot-product
# decode GEMMs), the
# 8-bit MX formats (with the 8-wave 256x256 tiles of the large shapes),
# INT4 G=64 (dot-product and MFMA decode kernels, the fp16-expansion GEMM's
# 128x128 and 256x256 tiles) and INT8 G=128 (the LDS-staged 128-row and
# 256-row tiles)
CASES = [
    ("mxfp4", 512, 49152, 512),
    ("mxfp4", 2048, 6144, 512),
    ("mxfp4", 1024, 8192, 1024),
    ("mxfp4", 300, 8208, 8192),
    ("mxfp4", 300, 1024, 1024),
    ("mxfp4", 4, 4096, 4096),
    ("mxfp4", 8, 6144, 1024),
    ("mxfp4", 16, 16384, 1024),
    ("mxint4", 16, 2048, 1024),
    ("mxint4", 1, 4608, 3584),
    ("mxint4", 300, 3536, 640),
    ("nvfp4", 260, 1024, 1024),
    ("nvfp4", 3, 1024, 1024),
    ("nvfp4", 1, 4096, 4096),
    ("nvfp4", 16, 4096, 4096),
    ("mxfp8", 300, 1024, 512),
    ("mxint8", 8, 1024, 512),
    ("mxint8", 1, 4096, 4096),
    ("mxfp8", 3, 4096, 4096),
    ("int4g64", 1, 2048, 1024),
    ("int4g64", 8, 1024, 1024),
    ("int4g64", 300, 1040, 1024),
    ("int4g64", 1100, 8000, 256),
    ("int8g128", 1, 4096, 4096),
    ("int8g128", 8, 1024, 1024),
    ("int8g128", 300, 1040, 1024),
    ("int8g128", 100, 1040, 1024),
    ("mxfp8", 1024, 10240, 256),
    ("mxint8", 1300, 6928, 256),
]


def build(case, dev):
    if case.w_codes is not None:
        wc, ws = to_dev(case.w_codes, dev), to_dev(case.w_scales, dev)
        tw = torch.tensor([case.t_w], dtype=torch.float32, device=dev)
    else:
        wc, ws, tw = w4.quantize_act(to_dev(case.w_prescaled, dev), None, case.fmt)
    blob = w4.pack_weight(wc, ws, tw, to_dev(case.r, dev), case.fmt)
    x, c = to_dev(case.x, dev), to_dev(case.c, dev)
    G = w4.block_size(case.fmt)
    codes = torch.empty((case.M, w4.code_cols(case.fmt, case.K)), dtype=torch.uint8, device=dev)
    scales = torch.empty((case.M, case.K // G), dtype=w4.scale_dtype(case.fmt), device=dev)
    t = torch.ones(1, dtype=torch.float32, device=dev)
    qws = torch.zeros(max(16, w4.lib().w4a4_quantize_workspace_bytes(w4.FORMATS[case.fmt], case.M, case.K)),
                      dtype=torch.uint8, device=dev)
    y = torch.empty((case.M, case.N), dtype=torch.bfloat16, device=dev)

    def step():
        w4.quantize_act(x, c, case.fmt, out=(codes, scales, t), workspace=qws)
        w4.linear(codes, scales, t, blob, case.fmt, case.N, case.K, out=y)

    return step, (codes, scales, t, y)


@pytest.mark.parametrize("fmt,M,N,K", CASES)
def test_graph_replays_match_eager(fmt, M, N, K):
    dev = device()
    say(f"[graph] {fmt} M={M} N={N} K={K}")
    case = inputs.adhoc_case(fmt, M, N, K, seed=3 * M + N + K)
    step, outs = build(case, dev)
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    # other eager work to interleave with the replays
    other = inputs.adhoc_case("mxfp4", 64, 512, 512, seed=1)
    other_step, _ = build(other, dev)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    # t is an output of the NVFP4 quantizer only (MX formats leave it alone)
    names = ("codes", "scales", "t", "y") if fmt == "nvfp4" else ("codes", "scales", "y")
    checked = [o for o, n in zip(outs, ("codes", "scales", "t", "y")) if n in names]
    expect = [r for r, n in zip(ref, ("codes", "scales", "t", "y")) if n in names]
    for rep in range(4):
        for o in checked:
            o.zero_()
        other_step()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, o, r in zip(names, checked, expect):
            assert torch.equal(o, r), f"replay {rep}: {name} differs from the eager run"
