"""One activation quantized under several column-scale vectors
(w4a4_quantize_act_multi, per-projection c on a fused input): every output
equals, bit for bit, the oracle's quantize_act under that c and the
single-output GPU quantizer's."""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import device, say
from w4a4_block_scaled_amd import inputs
import w4a4_block_scaled_amd as w4

pytestmark = pytest.mark.gpu


def column_scales(rng, K, fmt):
    """Inverse column scales on the format's admissible set (lognormal law)."""
    e = np.rint(rng.normal(0, 0.5 / np.log(2), K)).astype(np.int64)
    if fmt == "nvfp4":
        return (np.ldexp(1.0, e) * (1 + rng.integers(0, 8, K) / 8)).astype(np.float32)
    return np.ldexp(1.0, e).astype(np.float32)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxint4", "nvfp4"])
@pytest.mark.parametrize("P", [1, 2, 3, 4])
@pytest.mark.parametrize("M,K", [(1, 256), (37, 1024), (300, 4096)])
def test_multi_matches_oracle_and_single(fmt, P, M, K):
    dev = device()
    say(f"[quantize multi] {fmt} P={P} M={M} K={K}")
    rng = np.random.default_rng(M * 10 + P + K)
    x = inputs.outlier_activations(rng, M, K, max(1, K // 128), 30.0)
    xd = x.to(dev)
    cs = [column_scales(rng, K, fmt) for _ in range(P)]
    outs = w4.quantize_act_multi(xd, [torch.from_numpy(c).to(dev) for c in cs], fmt)
    torch.cuda.synchronize()
    for p in range(P):
        codes, scales, t = outs[p]
        oc, osc, ot = oracle.quantize_act(x.float().numpy(), cs[p], fmt)
        assert np.array_equal(codes.cpu().numpy(), oc), f"output {p}: codes differ"
        assert np.array_equal(scales.cpu().numpy(), osc), f"output {p}: scales differ"
        if fmt == "nvfp4":
            assert np.float32(t.item()) == ot
        sc, ss, st = w4.quantize_act(xd, torch.from_numpy(cs[p]).to(dev), fmt)
        assert torch.equal(sc, codes) and torch.equal(ss, scales)
