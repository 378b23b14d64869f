"""Pins for the MXCode PostScale and PreScale+ scale layouts in the oracle.

* Table 2's bits per element (tests/golden/mxcode_bpe.json): the storage
  accounting of each method, under the layout readings the oracle decodes
  (one E8M0 scale per QBlock codebook for PostScale; ds = 8 block scales
  along K per 8-bit index into a 256-entry scale codebook per matrix for
  PreScale+), reproduces all eight printed values, and the nearby
  alternative readings do not.
* Lossless round trips: weights built directly in a block-scaled FP4
  format (E8M0-B32, E4M3-B16 or E5M3-B16) so that the compression loses
  nothing (at most 256 distinct 4-vectors per QBlock, one
  scale per QBlock, at most 256 distinct scale vectors per matrix) are
  encoded here by a brute-force dictionary encoder written from the
  definitions; the oracle's decode must give back the original codes and
  scales bit for bit, hence the same dequantized weights.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle.formats import FMT_E4M3_B16, FMT_E5M3_B16, FMT_E8M0_B32

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mxcode_bpe.json")))


@pytest.mark.parametrize("fmt", ["E4M3-B16-FP4", "E8M0-B32-FP4"])
def test_table2_bits_per_element(fmt):
    rd = GOLD["readings"]
    N, K = rd["expert_matrix"]
    for method, printed in GOLD["bpe"][fmt].items():
        got = oracle.mxcode_bpe(method, rd["block"][fmt], rd["qblock"][fmt], N, K)
        assert round(float(got), 2) == printed, (fmt, method, got)


def test_table2_rejects_alternative_scale_layouts():
    # PostScale with an MX scale per 32 (or 16) codebook values instead of one
    # per codebook, and a PreScale+ scale codebook per QBlock instead of per
    # matrix: neither reproduces Table 2
    gold = GOLD["bpe"]
    for fmt, blk, qb in (("E8M0-B32-FP4", 32, 128), ("E4M3-B16-FP4", 16, 256)):
        per_block_cb_scales = 2.0 + 4096 / qb ** 2 + (1024 // blk) * 8 / qb ** 2
        assert round(per_block_cb_scales, 2) != gold[fmt]["postscale"]
        per_qblock_scale_cb = 2.0 + 4096 / qb ** 2 + 8 / (8 * blk) + 256 * 8 * 8 / qb ** 2
        assert round(per_qblock_scale_cb, 2) != gold[fmt]["prescale_plus"]


def test_config_qblock_bits_per_element():
    # at the 64x64 QBlocks the kernels are measured on: 1024 B of indices,
    # 512 B of table per QBlock, plus the scales
    N, K = 1536, 4096
    assert oracle.mxcode_bpe("prescale", 32, 64, N, K) == (1024 + 512 + 128) * 8 / 4096
    assert oracle.mxcode_bpe("postscale", 32, 64, N, K) == (1024 + 512 + 1) * 8 / 4096
    assert abs(oracle.mxcode_bpe("prescale_plus", 32, 64, N, K)
               - ((1024 + 512 + 16) * 8 / 4096 + 2048 * 8 / (N * K))) < 1e-12


# ---------------------------------------------------------------------------
# brute-force encoders (definitions written out with dictionaries and loops)
# ---------------------------------------------------------------------------

def _encode_vq(codes_unpacked, qblock):
    """Codes [N][K] (E2M1 nibbles) -> idx [N][K/4], codebook [N/qb][K/qb][256]
    with one table entry per distinct 4-vector of each QBlock."""
    N, K = codes_unpacked.shape
    idx = np.zeros((N, K // 4), np.uint8)
    cb = np.zeros((N // qblock, K // qblock, 256), np.uint16)
    for qr in range(N // qblock):
        for qc in range(K // qblock):
            table = {}
            for n in range(qr * qblock, (qr + 1) * qblock):
                for j in range(qc * qblock // 4, (qc + 1) * qblock // 4):
                    v = codes_unpacked[n, 4 * j:4 * j + 4]
                    key = int(v[0]) | int(v[1]) << 4 | int(v[2]) << 8 | int(v[3]) << 12
                    if key not in table:
                        table[key] = len(table)
                        cb[qr, qc, table[key]] = key
                    idx[n, j] = table[key]
            assert len(table) <= 256
    return idx, cb


def _mx_codes_with_few_vectors(rng, N, K, qblock, pool):
    """E2M1 nibbles [N][K] whose 4-vectors take at most `pool` values per QBlock."""
    out = np.zeros((N, K), np.uint8)
    for qr in range(N // qblock):
        for qc in range(K // qblock):
            vecs = rng.integers(0, 16, size=(pool, 4), dtype=np.uint8)
            pick = rng.integers(0, pool, size=(qblock, qblock // 4))
            out[qr * qblock:(qr + 1) * qblock, qc * qblock:(qc + 1) * qblock] = vecs[pick].reshape(qblock, qblock)
    return out


# (format, block, scale codes drawn from [lo, hi)): the three block-scaled formats
_SCALE_FMTS = [(FMT_E8M0_B32, 32, 110, 135), (FMT_E4M3_B16, 16, 0x30, 0x7F), (FMT_E5M3_B16, 16, 0x60, 0xFF)]


@pytest.mark.parametrize("fmt,block,lo,hi", _SCALE_FMTS, ids=["e8m0", "e4m3", "e5m3"])
@pytest.mark.parametrize("N,K,qblock", [(128, 192, 64), (128, 256, 128), (256, 512, 256)])
def test_postscale_lossless_round_trip(N, K, qblock, fmt, block, lo, hi):
    rng = np.random.default_rng(N + K + qblock + block)
    nib = _mx_codes_with_few_vectors(rng, N, K, qblock, pool=200)
    qscales = rng.integers(lo, hi, size=(N // qblock, K // qblock), dtype=np.uint8)
    # the block-scaled weight: every block of a QBlock carries that QBlock's scale
    scales = np.zeros((N, K // block), np.uint8)
    for n in range(N):
        for b in range(K // block):
            scales[n, b] = qscales[n // qblock, (block * b) // qblock]
    idx, cb = _encode_vq(nib, qblock)
    codes = oracle.vq_decode_codes(idx, cb, qblock)
    assert np.array_equal(codes, oracle.pack_nibbles(nib))
    got = oracle.postscale_block_scales(qscales, K, qblock, block)
    assert got.dtype == np.uint8 and np.array_equal(got, scales)
    ts = None if fmt == FMT_E8M0_B32 else 3.0e-5
    w = oracle.dequantize(codes, got, fmt, ts)
    assert np.array_equal(w, oracle.dequantize(oracle.pack_nibbles(nib), scales, fmt, ts))


def _encode_scale_vq(scales, ds):
    """Block scales [N][K/32] -> sidx [N][K/(32 ds)], table [256][ds]: one entry
    per distinct vector of ds consecutive scales of a row."""
    N, nb = scales.shape
    sidx = np.zeros((N, nb // ds), np.uint8)
    table = {}
    scb = np.zeros((256, ds), np.uint8)
    for n in range(N):
        for j in range(nb // ds):
            v = tuple(int(c) for c in scales[n, ds * j:ds * (j + 1)])
            if v not in table:
                table[v] = len(table)
                scb[table[v]] = v
            sidx[n, j] = table[v]
    assert len(table) <= 256
    return sidx, scb


@pytest.mark.parametrize("fmt,block,lo,hi", _SCALE_FMTS, ids=["e8m0", "e4m3", "e5m3"])
@pytest.mark.parametrize("N,K,pool", [(64, 256, 5), (96, 1024, 256), (128, 768, 40)])
def test_prescale_plus_lossless_round_trip(N, K, pool, fmt, block, lo, hi):
    rng = np.random.default_rng(7 * N + K + block)
    ds = 8
    vecs = rng.integers(lo, hi, size=(pool, ds), dtype=np.uint8)
    pick = rng.integers(0, pool, size=(N, K // (block * ds)))
    scales = vecs[pick].reshape(N, K // block)
    sidx, scb = _encode_scale_vq(scales, ds)
    got = oracle.prescale_plus_block_scales(sidx, scb, ds)
    assert got.dtype == np.uint8 and np.array_equal(got, scales)
    nib = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    codes = oracle.pack_nibbles(nib)
    ts = None if fmt == FMT_E8M0_B32 else 3.0e-5
    assert np.array_equal(oracle.dequantize(codes, got, fmt, ts), oracle.dequantize(codes, scales, fmt, ts))


def test_prescale_plus_vector_order_along_k():
    # scale b of row n comes from vector b // 8, element b % 8: a table whose
    # entry i holds (8i, 8i+1, ..) exposes a transposed or mis-strided decode
    scb = (np.arange(256 * 8) % 256).astype(np.uint8).reshape(256, 8)
    sidx = np.array([[0, 3], [5, 1]], np.uint8)
    got = oracle.prescale_plus_block_scales(sidx, scb)
    want = np.array([[(8 * int(i) + e) % 256 for i in row for e in range(8)] for row in sidx], np.uint8)
    assert np.array_equal(got, want)


def test_postscale_unit_scale_decodes_to_e2m1_values():
    # scale code 127 (2^0): the decoded weights are the E2M1 values of the keys
    qblock, N, K = 64, 64, 128
    cb = np.zeros((1, 2, 256), np.uint16)
    cb[0, 0, 1] = 0x7A21          # elements 0.5, 1, -1 (0xA), 6 (0x7)
    cb[0, 1, 0] = 0x0F00          # 0, 0, -6, 0
    idx = np.zeros((N, K // 4), np.uint8)
    idx[:, :16] = 1
    w = oracle.dequantize(oracle.vq_decode_codes(idx, cb, qblock),
                          oracle.postscale_block_scales(np.full((1, 2), 127, np.uint8), K, qblock), FMT_E8M0_B32)
    assert np.array_equal(w[:, :64], np.tile([0.5, 1.0, -1.0, 6.0], (N, 16)))
    assert np.array_equal(w[:, 64:], np.tile([0.0, 0.0, -6.0, 0.0], (N, 16)))
