"""Helpers shared by the GPU parity tests: tolerance checks and host copies.

The output tolerance is the one the library is held to: for every output row
m, max_n |y_gpu - y_ref| <= 1e-3 * ||y_ref[m, :]||_2, with y_ref the oracle's
float64 result.
"""

import numpy as np
import torch

REL_ROW_TOL = 1e-3


def to_np(t):
    return t.detach().cpu().numpy()


def u16(t):
    """bf16/fp16/int16 tensor -> numpy uint16 bit patterns."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def row_tol_ratio(y, ref):
    """max over rows of max_n |y - ref| / ||ref_row||_2 (0 for exact rows)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(y - ref).max(axis=1)
    nrm = np.linalg.norm(ref, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(err == 0, 0.0, err / nrm)
    return float(r.max()) if r.size else 0.0


def assert_rows_close(y, ref, tol=REL_ROW_TOL, what=""):
    r = row_tol_ratio(y, ref)
    assert r <= tol, f"{what}: max row error ratio {r:.3e} > {tol:.1e}"
    return r


def banner(msg):
    print(f"[case] {msg}", flush=True)


def vq_ref_block_scales(v, e, scales, K, qblock=64, block=32):
    """The oracle's block scale codes [N][K/block] of expert e of a
    synth.vq_weight dict, for its scale layout ``scales``."""
    import oracle
    sc = v["scales"][e].cpu().numpy()
    if scales == "prescale":
        return sc
    if scales == "postscale":
        return oracle.postscale_block_scales(sc, K, qblock, block)
    return oracle.prescale_plus_block_scales(sc, v["scale_codebook"][e].cpu().numpy())
