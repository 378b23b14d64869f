"""CPU oracle for the 4-bit-weight GEMM hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``gemm_bit_weight_amd``) and never imports it.

Two implementations of the same definitions:
  * ``oracle.native`` -- plain C++17 (``oracle/native/oracle.cpp``): every
    operand decoded to double from its format's closed form, every output
    one term-by-term Neumaier-compensated sum, std::thread over outputs.  The
    GPU parity tests and the bench's CPU baseline use it for the
    contractions.
  * this package's numpy modules, the cross-check: each C++ function is
    held bit for bit (or to the last ulp where the summation order differs)
    to its numpy twin, and both are pinned by the same closed forms, brute
    force and special cases.

The numpy side decodes to float64 and accumulates in float64.  Where the method is an encoding (the block-scaled FP4 quantizers,
routing), the functions follow the steps in the order the pages describe
them; where the method reaches a result with a plain definition (every GEMM,
the LUT kernel, the VQ decode) the oracle is that definition written out with
a float64 matmul as the contraction step.

Sources (page titles as printed on the pages):
  * "MXCode: MX-Native Codebook Quantization" -- Table 1 (block formats),
    abstract (PreScale, PostScale, PreScale+, MX-native operand
    reconstruction), Fig. 2/3 and Table 4 (VQ d=4, K=256, QBlock sizes,
    scale VQ Ks=256, ds=8), Table 2 (bits per element of each method).
  * "PRQuant: Permutation Residual Quantization for Low-Overhead Inference" --
    §4 Eq. (1) (scaled/permuted FFN), Eq. (2) (offline weight residual),
    §4 "Kernel design for efficient inference" (augmented MXFP4 GEMM and the
    online tail copy).
  * "CodeQuant: Unified Clustering and Quantization for Enhanced Outlier
    Smoothing in Low-Precision Mixture-of-Experts" -- Fig. 1 (clustered
    weights, LUT kernel), Fig. 4 (LUT precompute + lookup per tile).

Parity status of each function is recorded in its docstring; every function
has at least one pin in ``tests/test_oracle_*.py``.
"""

from . import formats, gemm, moe, rotation  # noqa: F401
from .formats import (  # noqa: F401
    E2M1_MAGNITUDES,
    e2m1_decode,
    e8m0_decode,
    e4m3_decode,
    e2m1_round_magnitude,
    e4m3_round,
    quantize_e8m0_b32,
    quantize_e4m3_b16,
    ue5m3_decode,
    ue5m3_round,
    quantize_e5m3_b16,
    dequantize,
    pack_nibbles,
    unpack_nibbles,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
)
from .gemm import (  # noqa: F401
    mx_gemm,
    residual_weight,
    residual_tail_gemm,
    tail_copy,
    lut_decode,
    lut_gemm,
    vq_decode_codes,
    vq_dequantize,
    postscale_block_scales,
    prescale_plus_block_scales,
    mxcode_bpe,
)
from .rotation import fwht32_fp32  # noqa: F401
from .moe import (  # noqa: F401
    moe_route,
    moe_gateup,
    swiglu_bf16,
    moe_down_combine,
    moe_down_combine_residual,
)
