"""CPU oracle for the packed W4A4 block-scaled linear.

TEST INFRASTRUCTURE ONLY.  A plain, slow, fp64 restatement of DualQuant's
inference-time computation (Section 4.4 with the formats of Section 3):
rescale the activations by the column scales, quantize them to MXFP4 /
NVFP4 / MXINT4 blocks (or INT4 blocks of 64 with BF16 scales, or the 8-bit
MXFP8 / MXINT8 blocks and INT8 blocks of 128 with BF16 scales), multiply
with the quantized weights and apply the row scales, rounding the result
once to BF16.

Only tests/, the smoke check in __graft_entry__.py and the CPU-baseline leg
of bench.py may import this package.  It shares no code with the HIP path
and does not import it; the two meet only through the seeded input
generator (w4a4_block_scaled_amd.inputs), which holds no method arithmetic.

Parity pins for every function live in tests/test_oracle_*.py: torch's own
float8 codecs, exact rational brute force (fractions.Fraction), scaling and
sign invariances, hand-worked golden blocks, a closed-form single block, and
the packed-size arithmetic of the paper's Table 12.
"""
from . import formats, quant, linear, solver  # noqa: F401
from .quant import (BLOCK, quantize_act, quantize_weight, quantize_rows,  # noqa: F401
                    pack_nibbles, unpack_nibbles, pack_codes, unpack_codes, dequantize, rescale,
                    nv_tensor_scale)
from .linear import linear as linear_bf16, linear_f64, layer, layer_prescaled  # noqa: F401
