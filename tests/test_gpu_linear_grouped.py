"""Per-projection linears of one M and K in one call (w4a4_linear_grouped):
each output against the oracle, and equal to a separate w4a4_linear call.
MXFP4 with M > 32 runs the problems' 256 x 128 tiles in one launch (the
separate calls of these shapes use the same tiles, so outputs are equal bit
for bit); shapes whose problems all take the persistent kernel, decode
sizes and the other formats run one after another."""
import numpy as np
import pytest
import torch

from gpu_common import device, say, to_dev, bf16_bits, check_linear
from test_gpu_linear import gpu_layer, oracle_layer
from w4a4_block_scaled_amd import inputs
import w4a4_block_scaled_amd as w4

pytestmark = pytest.mark.gpu


def problems(fmt, M, Ns, K, dev, seed):
    out = []
    for i, N in enumerate(Ns):
        case = inputs.adhoc_case(fmt, M, N, K, seed=seed + 31 * i)
        Y, blob, (ac, as_, ta), _ = gpu_layer(case, dev)
        out.append((case, Y, blob, ac, as_, ta))
    return out


CASES = [
    ("mxfp4", 300, (512, 144, 144), 1024, True),     # one launch, ragged M and N
    ("mxfp4", 2048, (4096, 1024, 1024), 512, True),  # the Llama QKV split, one launch
    ("mxfp4", 64, (1040,), 640, True),
    ("mxfp4", 512, (24576, 24576), 512, False),      # both persistent: one after another
    ("mxfp4", 16, (512, 256), 1024, False),          # decode sizes
    ("mxint4", 300, (512, 144), 1024, False),
    ("nvfp4", 300, (512, 144, 256), 1024, False),
]


@pytest.mark.parametrize("fmt,M,Ns,K,one_launch", CASES)
def test_grouped_matches_separate_and_oracle(fmt, M, Ns, K, one_launch):
    dev = device()
    say(f"[grouped] {fmt} M={M} N={Ns} K={K} one launch: {one_launch}")
    ps = problems(fmt, M, Ns, K, dev, seed=M + K)
    Ys = w4.linear_grouped([(ac, as_, ta, blob, case.N) for case, _, blob, ac, as_, ta in ps], fmt, K)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M)
    for (case, Y, blob, ac, as_, ta), Yg in zip(ps, Ys):
        assert torch.equal(Yg, Y), f"N={case.N}: grouped output differs from the separate call"
        rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 20), replace=False)]))
        y, S, _, _ = oracle_layer(case, rows)
        check_linear(bf16_bits(Yg)[rows], y, S, K, f"grouped {fmt} N={case.N}")
