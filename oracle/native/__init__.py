"""The C++ oracle (oracle.cpp) behind the same calls as the numpy oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``): it shares nothing with
the HIP library.  The C++ side decodes every operand to double from the
formats' closed forms and sums each output term by term with a compensated
(Neumaier) sum on std::thread workers; these wrappers only move numpy arrays
in and out.  Functions that contract return their result and keep the number
of outputs whose plain double sum differed from the compensated one in
``last_inexact`` (0 means every output is the exact value of its sum).

The library is built by ``oracle/native/build.py`` (g++); it is built here on
first use when it is missing.
"""

import ctypes as _c
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
if not os.path.exists(_LIB_PATH):
    from . import build as _build
    _build.build()
_lib = _c.CDLL(_LIB_PATH)

_vp, _i64, _int, _dbl = _c.c_void_p, _c.c_int64, _c.c_int, _c.c_double
_lib.gbwo_threads.restype = _int
_lib.gbwo_dequantize.argtypes = [_i64, _i64, _int, _vp, _vp, _dbl, _vp]
_lib.gbwo_block_gemm.restype = _i64
_lib.gbwo_block_gemm.argtypes = [_i64, _i64, _i64, _int, _vp, _vp, _vp, _dbl, _vp, _vp, _dbl, _vp]
_lib.gbwo_residual_tail_gemm.restype = _i64
_lib.gbwo_residual_tail_gemm.argtypes = [_i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.gbwo_lut_gemm.restype = _i64
_lib.gbwo_lut_gemm.argtypes = [_i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp]
_lib.gbwo_vq_decode_codes.argtypes = [_i64, _i64, _i64, _vp, _vp, _vp]
_lib.gbwo_quantize_e8m0_b32.argtypes = [_i64, _i64, _vp, _vp, _vp]
_lib.gbwo_quantize_b16.restype = _c.c_float
_lib.gbwo_quantize_b16.argtypes = [_int, _i64, _i64, _vp, _dbl, _vp, _vp]
_lib.gbwo_swiglu_bf16.argtypes = [_i64, _vp, _vp, _vp]
_lib.gbwo_combine.argtypes = [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.gbwo_route.argtypes = [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.gbwo_e2m1_rne.argtypes = [_i64, _vp, _vp]

_FMT = {"e8m0_b32": 0, "e4m3_b16": 1, "e5m3_b16": 2}
TENSOR_SCALED = ("e4m3_b16", "e5m3_b16")

last_inexact = 0


def threads():
    """Worker threads the C++ oracle runs on (hardware threads, or GBWO_THREADS)."""
    return int(_lib.gbwo_threads())


def _arr(a, dtype):
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def _p(a):
    return None if a is None else a.ctypes.data_as(_vp)


def _ts(v):
    return 1.0 if v is None else float(np.float32(v))


def dequantize(codes, scales, fmt, tensor_scale=None):
    codes, scales = _arr(codes, np.uint8), _arr(scales, np.uint8)
    rows, K = codes.shape[0], codes.shape[1] * 2
    out = np.empty((rows, K))
    _lib.gbwo_dequantize(rows, K, _FMT[fmt], _p(codes), _p(scales), _ts(tensor_scale), _p(out))
    return out


def mx_gemm(a_codes, a_scales, w_codes, w_scales, fmt="e8m0_b32", a_ts=None, w_ts=None, a_rows=None):
    """Y = S_Ta S_Tw deq(A) deq(W)^T (rows a_rows of A if given)."""
    global last_inexact
    a_codes, a_scales = _arr(a_codes, np.uint8), _arr(a_scales, np.uint8)
    w_codes, w_scales = _arr(w_codes, np.uint8), _arr(w_scales, np.uint8)
    rows = None if a_rows is None else _arr(a_rows, np.int64)
    M = a_codes.shape[0] if rows is None else len(rows)
    N, K = w_codes.shape[0], w_codes.shape[1] * 2
    assert a_codes.shape[1] * 2 == K
    y = np.empty((M, N))
    if M and N:
        last_inexact = int(_lib.gbwo_block_gemm(M, N, K, _FMT[fmt], _p(a_codes), _p(a_scales), _p(rows), _ts(a_ts),
                                                _p(w_codes), _p(w_scales), _ts(w_ts), _p(y)))
    return y


def residual_tail_gemm(a_codes, a_scales, w_codes, w_scales, r_codes, r_scales, tail):
    """PRQuant augmented GEMM over K + tail (E8M0-B32)."""
    global last_inexact
    a_codes, a_scales = _arr(a_codes, np.uint8), _arr(a_scales, np.uint8)
    w_codes, w_scales = _arr(w_codes, np.uint8), _arr(w_scales, np.uint8)
    r_codes, r_scales = _arr(r_codes, np.uint8), _arr(r_scales, np.uint8)
    M, K, N = a_codes.shape[0], a_codes.shape[1] * 2, w_codes.shape[0]
    y = np.empty((M, N))
    last_inexact = int(_lib.gbwo_residual_tail_gemm(M, N, K, tail, _p(a_codes), _p(a_scales), _p(w_codes),
                                                    _p(w_scales), _p(r_codes), _p(r_scales), _p(y)))
    return y


def lut_gemm(x_bf16_bits, idx_packed, centroids_f16, group):
    """Y = bf16(X) fp16(C[idx])^T; centroids as float16 values or their bits."""
    global last_inexact
    x = _arr(x_bf16_bits, np.uint16)
    idx = _arr(idx_packed, np.uint8)
    c = np.asarray(centroids_f16)
    c = _arr(c.view(np.uint16) if c.dtype == np.float16 else c, np.uint16)
    M, K = x.shape
    N = idx.shape[0]
    y = np.empty((M, N))
    last_inexact = int(_lib.gbwo_lut_gemm(M, N, K, group, _p(x), _p(idx), _p(c), _p(y)))
    return y


def vq_decode_codes(idx, codebook, qblock=64):
    idx = _arr(idx, np.uint8)
    cb = np.asarray(codebook)
    cb = _arr(cb.view(np.uint16) if cb.dtype == np.int16 else cb, np.uint16)
    N, K = idx.shape[0], idx.shape[1] * 4
    out = np.empty((N, K // 2), np.uint8)
    _lib.gbwo_vq_decode_codes(N, K, qblock, _p(idx), _p(cb), _p(out))
    return out


def quantize_e8m0_b32(x):
    x = _arr(x, np.float32)
    rows, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    codes = np.empty((rows, K // 2), np.uint8)
    scales = np.empty((rows, K // 32), np.uint8)
    _lib.gbwo_quantize_e8m0_b32(rows, K, _p(x), _p(codes), _p(scales))
    return codes, scales


def _quantize_b16(fmt, x, tensor_amax):
    x = _arr(x, np.float32)
    rows, K = x.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    codes = np.empty((rows, K // 2), np.uint8)
    scales = np.empty((rows, K // 16), np.uint8)
    amax = -1.0 if tensor_amax is None else float(np.float32(tensor_amax))
    st = _lib.gbwo_quantize_b16(_FMT[fmt], rows, K, _p(x), amax, _p(codes), _p(scales))
    return codes, scales, np.float32(st)


def quantize_e4m3_b16(x, tensor_amax=None):
    return _quantize_b16("e4m3_b16", x, tensor_amax)


def quantize_e5m3_b16(x, tensor_amax=None):
    return _quantize_b16("e5m3_b16", x, tensor_amax)


def swiglu_bf16(g, u):
    g, u = _arr(g, np.float64), _arr(u, np.float64)
    h = np.empty(g.shape, np.uint16)
    _lib.gbwo_swiglu_bf16(g.size, _p(g), _p(u), _p(h))
    return h


def moe_route(logits, topk):
    logits = _arr(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, topk), np.int32)
    w = np.empty((T, topk))
    off = np.empty(E + 1, np.int32)
    pt = np.empty(T * topk, np.int32)
    pp = np.empty((T, topk), np.int32)
    _lib.gbwo_route(T, E, topk, _p(logits), _p(ids), _p(w), _p(off), _p(pt), _p(pp))
    return dict(topk_ids=ids, topk_w=w, expert_offsets=off, pair_token=pt, pair_pos=pp)


def moe_gateup(a_codes, a_scales, fmt, route, wgu_codes, wgu_scales, a_ts=None, wgu_ts=None, pairs=None):
    """g, u [P][I] in pair order (or for ``pairs``): the gathered GEMM of each
    pair's token row against its expert's fused [2I][H] gate/up weight.  The
    weights may be any indexable per-expert container; only experts that own
    requested pairs are touched."""
    global last_inexact
    off = np.asarray(route["expert_offsets"])
    pt = np.asarray(route["pair_token"])
    P = len(pt)
    want = np.arange(P) if pairs is None else np.asarray(pairs)
    E = len(off) - 1
    first = wgu_codes[int(np.searchsorted(off, want[0], side="right") - 1)] if len(want) else None
    I = (first.shape[0] // 2) if first is not None else 0
    g = np.zeros((len(want), I))
    u = np.zeros((len(want), I))
    inexact = 0
    for e in range(E):
        sel = np.nonzero((want >= off[e]) & (want < off[e + 1]))[0]
        if len(sel) == 0:
            continue
        ts = (wgu_ts[e][0], wgu_ts[e][1]) if fmt in TENSOR_SCALED else (None, None)
        wc, ws = np.asarray(wgu_codes[e]), np.asarray(wgu_scales[e])
        rows = pt[want[sel]]
        g[sel] = mx_gemm(a_codes, a_scales, wc[:I], ws[:I], fmt, a_ts, ts[0], a_rows=rows)
        inexact += last_inexact
        u[sel] = mx_gemm(a_codes, a_scales, wc[I:], ws[I:], fmt, a_ts, ts[1], a_rows=rows)
        inexact += last_inexact
    last_inexact = inexact
    return g, u


def moe_down_combine(h_codes, h_scales, fmt, route, wd_codes, wd_scales, h_ts=None, wd_ts=None, tokens=None):
    """Y[t] = sum_j w[t][j] deq(Hq[pair_pos[t][j]]) deq(W_down,e)^T, the slots
    of each token summed in slot order (or only the rows in ``tokens``)."""
    global last_inexact
    ids = np.asarray(route["topk_ids"])
    T, topk = ids.shape
    pp = _arr(route["pair_pos"], np.int32)
    off = np.asarray(route["expert_offsets"])
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    need = np.unique(pp[toks].reshape(-1))               # pairs of the requested tokens
    E = len(off) - 1
    H = np.asarray(wd_codes[int(np.searchsorted(off, need[0], side="right") - 1)]).shape[0] if len(need) else 0
    o = np.zeros((len(need), H))
    o_row = np.full(len(route["pair_token"]), -1, np.int64)
    o_row[need] = np.arange(len(need))
    inexact = 0
    for e in range(E):
        sel = np.nonzero((need >= off[e]) & (need < off[e + 1]))[0]
        if len(sel) == 0:
            continue
        o[sel] = mx_gemm(h_codes, h_scales, wd_codes[e], wd_scales[e], fmt, h_ts,
                         wd_ts[e] if fmt in TENSOR_SCALED else None, a_rows=need[sel])
        inexact += last_inexact
    last_inexact = inexact
    y = np.empty((len(toks), H))
    w = _arr(route["topk_w"], np.float64)
    tk = _arr(toks, np.int64)
    if len(toks) and H:
        _lib.gbwo_combine(len(toks), topk, H, _p(tk), _p(pp), _p(w), _p(o_row), _p(o), _p(y))
    return y


def moe_down_combine_residual(h_codes, h_scales, route, wd_codes, wd_scales, r_codes, r_scales, tail, tokens=None):
    """PRQuant on the expert down projections (E8M0-B32): the down GEMM over
    I + tail of [Hq, Hq_tail] against [W_down,e | R_e]."""
    h_codes, h_scales = np.asarray(h_codes), np.asarray(h_scales)
    I = h_codes.shape[1] * 2
    ac = np.concatenate([h_codes, h_codes[:, (I - tail) // 2:]], axis=1)
    as_ = np.concatenate([h_scales, h_scales[:, (I - tail) // 32:]], axis=1)

    class _Aug:
        def __init__(self, a, b):
            self.a, self.b = a, b

        def __getitem__(self, e):
            return np.concatenate([np.asarray(self.a[e]), np.asarray(self.b[e])], axis=1)

    return moe_down_combine(ac, as_, "e8m0_b32", route, _Aug(wd_codes, r_codes), _Aug(wd_scales, r_scales),
                            tokens=tokens)
