"""GPU checks of w4a4_pack_weight / w4a4_unpack_weight: bitwise round trips
(codes, scales, r, t_w) over shapes with partial scale groups and the full
Llama gate+up weight."""
import numpy as np
import pytest
import torch

from gpu_common import device, say, to_dev
import w4a4_block_scaled_amd as w4

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxint4"])
@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (272, 1152), (4096, 14336), (28672, 4096)])
def test_pack_round_trip(fmt, N, K):
    dev = device()
    say(f"[pack] {fmt} N={N} K={K}")
    G = w4.block_size(fmt)
    g = torch.Generator(device="cpu").manual_seed(N * 7 + K)
    codes = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, generator=g).to(dev)
    scales = torch.randint(0, 256, (N, K // G), dtype=torch.uint8, generator=g).to(dev)
    r = torch.rand(N, generator=g).to(dev)
    t_w = torch.tensor([0.37], dtype=torch.float32, device=dev)
    blob = w4.pack_weight(codes, scales, t_w, r, fmt)
    c2, s2, r2, t2 = w4.unpack_weight(blob, fmt, N, K)
    torch.cuda.synchronize()
    assert torch.equal(codes, c2)
    assert torch.equal(scales, s2)
    assert torch.equal(r, r2)
    assert float(t2.cpu()[0]) == np.float32(0.37)
    hdr = blob[:8].cpu().numpy().tobytes()
    assert hdr == b"W4A4PK01"


def test_pack_layout_is_fragment_order():
    """Tile (ng, ks) lane l holds the 16 canonical bytes of row 16 ng + l%16,
    K chunk 4 ks + l/16."""
    dev = device()
    N, K = 32, 256
    codes = torch.arange(N * K // 2, dtype=torch.int64).remainder(251).to(torch.uint8).reshape(N, K // 2)
    scales = torch.zeros((N, K // 32), dtype=torch.uint8)
    blob = w4.pack_weight(codes.to(dev), scales.to(dev), None, torch.ones(N).to(dev), "mxfp4").cpu()
    frag = blob[256:256 + N * K // 2].reshape(N // 16, K // 128, 64, 16)
    for ng in range(N // 16):
        for ks in range(K // 128):
            for l in range(64):
                row, chunk = 16 * ng + l % 16, 4 * ks + l // 16
                assert torch.equal(frag[ng, ks, l], codes[row, 16 * chunk:16 * chunk + 16])
