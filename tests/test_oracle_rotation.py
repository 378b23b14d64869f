"""Pins for the oracle's block Walsh-Hadamard rotation (fwht32_fp32).

Checked against scipy's Sylvester-Hadamard matrix (a library routine), the
orthogonality of the transform, float64 matrix products, and the GEMM
invariance X W^T = (X H)(W H)^T that makes the rotation usable.
"""

import numpy as np
import pytest
from scipy.linalg import hadamard

import oracle
import synth


def _block_matmul(x, H):
    rows, K = x.shape
    return (x.reshape(rows, K // 32, 32).astype(np.float64) @ H.T).reshape(rows, K)


def test_unnormalized_transform_is_sylvester_hadamard_exactly():
    """Integer inputs keep every fp32 butterfly exact: the fast transform must
    equal the block product with scipy's order-32 Hadamard matrix."""
    rng = np.random.default_rng(30)
    x = rng.integers(-1000, 1000, (7, 256)).astype(np.float32)
    got = oracle.fwht32_fp32(x, normalize=False).astype(np.float64)
    assert np.array_equal(got, _block_matmul(x, hadamard(32)))


def test_transform_twice_is_32_times_identity():
    rng = np.random.default_rng(31)
    x = rng.integers(-1000, 1000, (5, 128)).astype(np.float32)
    twice = oracle.fwht32_fp32(oracle.fwht32_fp32(x, normalize=False), normalize=False)
    assert np.array_equal(twice, 32 * x)


def test_normalized_transform_close_to_float64_orthonormal_product():
    rng = np.random.default_rng(32)
    x = (rng.standard_normal((9, 512)) * np.exp(rng.uniform(-5, 5, (9, 1)))).astype(np.float32)
    got = oracle.fwht32_fp32(x).astype(np.float64)
    ref = _block_matmul(x, hadamard(32) / np.sqrt(32.0))
    l1 = np.abs(x.astype(np.float64)).reshape(9, 16, 32).sum(-1).repeat(32, axis=1)
    assert np.all(np.abs(got - ref) <= 8 * 2.0 ** -24 * l1)
    # orthonormal: block norms are preserved
    n0 = np.linalg.norm(x.reshape(9, 16, 32).astype(np.float64), axis=-1)
    n1 = np.linalg.norm(got.reshape(9, 16, 32), axis=-1)
    assert np.allclose(n0, n1, rtol=1e-6)


def test_blocks_are_independent_and_k_must_be_a_multiple_of_32():
    rng = np.random.default_rng(33)
    x = rng.standard_normal((2, 96)).astype(np.float32)
    y = x.copy()
    y[:, 32:64] += 1.0
    a, b = oracle.fwht32_fp32(x), oracle.fwht32_fp32(y)
    assert np.array_equal(a[:, :32], b[:, :32]) and np.array_equal(a[:, 64:], b[:, 64:])
    assert not np.array_equal(a[:, 32:64], b[:, 32:64])
    with pytest.raises(ValueError):
        oracle.fwht32_fp32(np.zeros((1, 48), np.float32))


def test_rotated_gemm_equals_plain_gemm():
    rng = np.random.default_rng(34)
    x = rng.standard_normal((6, 256)).astype(np.float32)
    w = (rng.standard_normal((10, 256)) * 0.02).astype(np.float32)
    y = oracle.fwht32_fp32(x).astype(np.float64) @ oracle.fwht32_fp32(w).astype(np.float64).T
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.allclose(y, ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max())


def test_rotation_reduces_mxfp4_error_on_outlier_channels():
    """Sanity for the reason the pages rotate: with 1% of channels x50 (the
    tail-residual workload's activations), quantizing the rotated operands
    gives a smaller output error than quantizing the plain ones."""
    p = synth.tail_residual_problem(64, 96, 1024, tail=256, seed=0, device="cpu")
    x = p["x"].float().numpy()
    w = p["w"].numpy()
    ref = x.astype(np.float64) @ w.astype(np.float64).T

    def err(xa, wa):
        ac, as_ = oracle.quantize_e8m0_b32(xa)
        wc, ws = oracle.quantize_e8m0_b32(wa)
        y = oracle.mx_gemm(ac, as_, wc, ws)
        return np.linalg.norm(y - ref) / np.linalg.norm(ref)

    plain = err(x, w)
    rot = err(oracle.fwht32_fp32(x), oracle.fwht32_fp32(w))
    assert rot < plain, (rot, plain)
