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
    """MXFP4: tile (g, h) lane l holds the 16 canonical bytes of row 32 g + l%32,
    K chunk 2 h + l/32 (32 codes each); rows of a partial last group are zero.
    NVFP4: tile (g, h) lane l holds row 16 g + l%16, K chunk 4 h + l/16."""
    dev = device()
    for fmt, rows, kt, N in (("mxfp4", 32, 64, 48), ("nvfp4", 16, 128, 48)):
        K = 256
        G = w4.block_size(fmt)
        codes = torch.arange(N * K // 2, dtype=torch.int64).remainder(251).to(torch.uint8).reshape(N, K // 2)
        scales = torch.zeros((N, K // G), dtype=torch.uint8)
        blob = w4.pack_weight(codes.to(dev), scales.to(dev), None, torch.ones(N).to(dev), fmt).cpu()
        NG = -(-N // rows)
        frag = blob[256:256 + NG * rows * K // 2].reshape(NG, K // kt, 64, 16)
        per = 64 // rows  # 32-code chunks per lane group
        for g in range(NG):
            for h in range(K // kt):
                for l in range(64):
                    row, chunk = rows * g + l % rows, (kt // 32) * h + l // rows
                    want = codes[row, 16 * chunk:16 * chunk + 16] if row < N else torch.zeros(16, dtype=torch.uint8)
                    assert torch.equal(frag[g, h, l], want), (fmt, g, h, l)
        assert per in (2, 4)
