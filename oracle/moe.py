"""MoE expert FFN references: top-k routing, grouped gate/up + SwiGLU, grouped
down projection + weighted combine.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The FFN form is the gated MLP of PRQuant §4 Eq. (1):
MLP(X) = (X W_up^T * sigma(X W_gate^T)) W_down^T, applied per routed expert
(CodeQuant Fig. 1 / Fig. 2 place the quantized weights in the MoE FFN
experts).  Readings taken here, where the pages leave a step open:
  * routing selects the top-k logits of a token, ties to the lower expert id,
    and weights the k chosen experts by a softmax renormalised over them;
  * the gated activation is silu(g) * u (sigma(z) * z with the logistic
    sigma), rounded to bf16 before it is quantized again;
  * the fused gate/up weight of an expert stacks gate rows [0, I) on top of
    up rows [I, 2I);
  * the pair list is ordered by expert, then token; slot j of a token is its
    j-th largest logit.
"""

import numpy as np

from .formats import (
    FMT_E4M3_B16,
    FMT_E8M0_B32,
    TENSOR_SCALED,
    bf16_bits_to_f32,
    dequantize,
    f32_to_bf16_bits,
)


def moe_route(logits, topk):
    """logits fp32 [T][E] -> dict(topk_ids, topk_w, expert_offsets, pair_token, pair_pos).

    topk_ids[t][j]: the j-th largest logit's expert (ties -> lower id).
    topk_w[t][j] = exp(l_j - l_max) / sum_i exp(l_i - l_max) over the chosen k.
    Pairs are sorted by (expert, token); expert_offsets[e] = #pairs with a
    smaller expert id; pair_token[p] = token of pair p; pair_pos[t][j] = p.
    """
    l = np.asarray(logits, dtype=np.float32)
    T, E = l.shape
    # stable sort on the negated logits: descending value, ties keep lower id first
    order = np.argsort(-l.astype(np.float64), axis=1, kind="stable")
    ids = order[:, :topk].astype(np.int32)
    sel = np.take_along_axis(l, ids, axis=1).astype(np.float64)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    flat_e = ids.reshape(-1).astype(np.int64)
    flat_t = np.repeat(np.arange(T), topk)
    flat_j = np.tile(np.arange(topk), T)
    perm = np.lexsort((flat_t, flat_e))               # primary: expert, then token
    counts = np.bincount(flat_e, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    pair_token = flat_t[perm].astype(np.int32)
    pair_pos = np.empty((T, topk), dtype=np.int32)
    pair_pos[flat_t[perm], flat_j[perm]] = np.arange(T * topk, dtype=np.int32)
    return dict(topk_ids=ids, topk_w=w, expert_offsets=offsets,
                pair_token=pair_token, pair_pos=pair_pos)


def moe_gateup(a_codes, a_scales, fmt, route, wgu_codes, wgu_scales, a_ts=None, wgu_ts=None,
               pairs=None):
    """Per pair p = (token t, expert e): g = deq(A[t]) deq(W_gate,e)^T,
    u = deq(A[t]) deq(W_up,e)^T in float64.  Returns (g, u) [P][I] in pair
    order (or only for the pair indices in ``pairs``, in that order).

    a_codes [T][H/2] etc. is the quantized X; wgu_codes [E][2I][H/2].
    For E4M3-B16, a_ts is the activation tensor scale and wgu_ts [E][2] the
    (gate, up) weight tensor scales.
    """
    E = wgu_codes.shape[0]
    I = wgu_codes.shape[1] // 2
    P = len(route["pair_token"])
    want = np.arange(P) if pairs is None else np.asarray(pairs)
    g = np.zeros((len(want), I))
    u = np.zeros((len(want), I))
    pt = route["pair_token"]
    off = route["expert_offsets"]
    for e in range(E):
        sel = np.nonzero((want >= off[e]) & (want < off[e + 1]))[0]
        if len(sel) == 0:
            continue
        toks = pt[want[sel]]
        a = dequantize(a_codes[toks], a_scales[toks], fmt)
        w = dequantize(wgu_codes[e], wgu_scales[e], fmt)
        out = a @ w.T
        if fmt in TENSOR_SCALED:
            sa = float(np.float32(a_ts))
            out[:, :I] *= sa * float(np.float32(wgu_ts[e][0]))
            out[:, I:] *= sa * float(np.float32(wgu_ts[e][1]))
        g[sel] = out[:, :I]
        u[sel] = out[:, I:]
    return g, u


def swiglu_bf16(g, u):
    """h = bf16_RNE(silu(g) * u), silu(z) = z / (1 + exp(-z)), evaluated in
    float64 and rounded once to bf16.  Returns bf16 bit patterns."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    with np.errstate(over="ignore"):             # e^-g = inf for g < -709: h = -0 * u
        h = g / (1.0 + np.exp(-g)) * u
    # float64 -> bf16 RNE: go through float32 only when that is exact enough
    return _f64_to_bf16_bits(h)


def _f64_to_bf16_bits(h):
    """Round float64 to the nearest bf16 (ties to even) without double rounding."""
    h = np.asarray(h, dtype=np.float64)
    f = h.astype(np.float32)                     # RNE to fp32 (24 bits)
    bits = f32_to_bf16_bits(f)                   # RNE to 8 bits
    # double rounding can only go wrong when the fp32 value sits exactly on a
    # bf16 midpoint; decide those from the float64 value directly.
    fu = f.view(np.uint32)
    mid = (fu & 0xFFFF) == 0x8000
    if np.any(mid):
        lo = (fu & 0xFFFF0000).view(np.float32).astype(np.float64)
        hi_bits = ((fu >> 16) + 1).astype(np.uint32) << 16
        hi = hi_bits.view(np.float32).astype(np.float64)
        # distance measured in magnitude; sign shared by lo/hi
        d_lo = np.abs(h - lo)
        d_hi = np.abs(hi - h)
        up = (d_hi < d_lo) | ((d_hi == d_lo) & (((fu >> 16) & 1) == 1))
        fixed = np.where(up, (fu >> 16) + 1, fu >> 16).astype(np.uint16)
        bits = np.where(mid, fixed, bits)
    return bits.astype(np.uint16)


def moe_down_combine(h_codes, h_scales, fmt, route, wd_codes, wd_scales, h_ts=None, wd_ts=None,
                     tokens=None):
    """Y[t] = sum_j topk_w[t][j] * deq(Hq[pair_pos[t][j]]) deq(W_down,e)^T in float64.

    h_codes [P][I/2] is the quantized SwiGLU output in pair order;
    wd_codes [E][H][I/2].  Returns Y [T][H] (or only the rows in ``tokens``,
    in that order).  Experts are visited one at a time so that only one
    decoded weight is held at once.
    """
    ids = route["topk_ids"]
    w = route["topk_w"]
    pt = route["pair_token"]
    off = route["expert_offsets"]
    T, topk = ids.shape
    E = wd_codes.shape[0]
    H = wd_codes.shape[1]
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    row_of = np.full(T, -1, dtype=np.int64)
    row_of[toks] = np.arange(len(toks))
    y = np.zeros((len(toks), H))
    for e in range(E):
        p = np.arange(off[e], off[e + 1])
        p = p[row_of[pt[p]] >= 0]
        if len(p) == 0:
            continue
        t = pt[p]
        j = np.argmax(ids[t] == e, axis=1)          # the slot that chose e
        a = dequantize(h_codes[p], h_scales[p], fmt)
        out = a @ dequantize(wd_codes[e], wd_scales[e], fmt).T
        if fmt in TENSOR_SCALED:
            out = out * (float(np.float32(h_ts)) * float(np.float32(wd_ts[e])))
        np.add.at(y, row_of[t], w[t, j][:, None] * out)
    return y


def bf16_to_f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def moe_down_combine_residual(h_codes, h_scales, route, wd_codes, wd_scales, r_codes, r_scales, tail,
                              tokens=None):
    """PRQuant on the expert down-projections (E8M0-B32 / MXFP4):

    Y[t] = sum_j w[t][j] * (deq(Hq_p) deq(W_down,e)^T + deq(Hq_p[:, I-tail:]) deq(R_e)^T)

    with R_e = W_down,e[:, I-tail:] - deq(Q(W_down,e))[:, I-tail:] quantized
    (PRQuant §4 Eq. (2) per expert; the augmented GEMM of §4 "Kernel design"
    over I + tail).  h_codes [P][I/2]; r_codes [E][H][tail/2].
    """
    y = moe_down_combine(h_codes, h_scales, FMT_E8M0_B32, route, wd_codes, wd_scales, tokens=tokens)
    if tail:
        I = h_codes.shape[1] * 2
        y = y + moe_down_combine(h_codes[:, (I - tail) // 2:], h_scales[:, (I - tail) // 32:], FMT_E8M0_B32, route,
                                 r_codes, r_scales, tokens=tokens)
    return y
