"""Block Walsh-Hadamard rotation of activations and weights before MXFP4
quantization.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sources (page titles as printed on the pages):
  * "CodeQuant: Unified Clustering and Quantization for Enhanced Outlier
    Smoothing in Low-Precision Mixture-of-Experts", Table 2 and its caption:
    the "had" variants enable online Hadamard transforms during quantization.
  * "PRQuant: Permutation Residual Quantization for Low-Overhead Inference",
    §2 "Rotation and block-aware FP4 quantization": global rotations spread
    outliers across MXFP4 blocks, so format-aware methods rotate within the
    microscaling blocks (block-wise rotations, MXFP4-aligned transforms).

Reading (the pages give no formula): every 32-element MXFP4 block along K is
multiplied by the normalized Sylvester-Hadamard matrix of order 32,
H32[i][j] = (-1)^popcount(i & j) / sqrt(32), which is symmetric and
orthonormal, so X W^T = (X H)(W H)^T with W rotated the same way offline.
Because the rotated values decide quantization codes, the transform is
written in the precision a GPU computes it in: fp32, by the fast transform in
stages of span 1, 2, 4, 8, 16 (each a pair (a, b) -> (a + b, a - b), one fp32
operation each), then one fp32 multiply by fp32(1/sqrt(32)).
"""

import numpy as np

INV_SQRT32 = np.float32(1.0 / np.sqrt(np.float64(32.0)))   # 0x3E3504F3


def fwht32_fp32(x, normalize=True):
    """x [rows][K] -> float32 [rows][K], each 32-block transformed as above."""
    x = np.asarray(x, dtype=np.float32)
    rows, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    v = x.reshape(rows, K // 32, 32).copy()
    h = 1
    while h < 32:
        idx = np.arange(32)
        lo = idx[(idx & h) == 0]
        a = v[..., lo].copy()
        b = v[..., lo + h].copy()
        v[..., lo] = (a + b).astype(np.float32)
        v[..., lo + h] = (a - b).astype(np.float32)
        h *= 2
    if normalize:
        v = (v * INV_SQRT32).astype(np.float32)
    return v.reshape(rows, K)
