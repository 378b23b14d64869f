"""Pins for the oracle's MoE routing and expert FFN stages.

Routing is checked against a pure-Python full sort per token; the FFN stages
are checked against the special cases that reduce to a dense SwiGLU FFN
(one expert, top-1), against routing-independence when all experts are
identical, and the SwiGLU rounding against torch's bf16 cast.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import moe as M


def _brute_route(logits, topk):
    T, E = logits.shape
    ids, ws = [], []
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:topk]
        mx = float(logits[t, order[0]])
        ex = [math.exp(float(logits[t, e]) - mx) for e in order]
        s = sum(ex)
        ids.append(order)
        ws.append([v / s for v in ex])
    return np.array(ids), np.array(ws)


@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (17, 8, 2), (64, 128, 8), (5, 16, 16)])
def test_route_brute_force(T, E, k):
    rng = np.random.default_rng(T + E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[0, :3] = logits[0, 3] if E > 3 else logits[0, 0]        # ties
    r = oracle.moe_route(logits, k)
    ids, ws = _brute_route(logits, k)
    assert np.array_equal(r["topk_ids"], ids)
    assert np.allclose(r["topk_w"], ws, rtol=1e-14, atol=0)
    # pair list: every (token, slot) once, sorted by (expert, token)
    off = r["expert_offsets"]
    assert off[0] == 0 and off[-1] == T * k and np.all(np.diff(off) >= 0)
    pt = r["pair_token"]
    for e in range(E):
        seg = pt[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert sorted(seg.tolist()) == sorted(t for t in range(T) if e in ids[t])
    for t in range(T):
        for j in range(k):
            p = r["pair_pos"][t, j]
            assert pt[p] == t and off[ids[t, j]] <= p < off[ids[t, j] + 1]


def test_route_known_permutation():
    E = 128
    rng = np.random.default_rng(0)
    perm = rng.permutation(E)
    logits = perm[None, :].astype(np.float32)            # logit of expert e is perm[e]
    r = oracle.moe_route(logits, 8)
    want = [int(np.nonzero(perm == v)[0][0]) for v in range(127, 119, -1)]
    assert r["topk_ids"][0].tolist() == want
    ref = np.exp(np.arange(0, -8, -1.0))
    assert np.allclose(r["topk_w"][0], ref / ref.sum(), rtol=1e-15)


def test_route_ties_go_to_lower_id():
    logits = np.zeros((2, 8), np.float32)
    logits[1, 5] = -0.0
    r = oracle.moe_route(logits, 3)
    assert r["topk_ids"].tolist() == [[0, 1, 2], [0, 1, 2]]
    assert np.allclose(r["topk_w"], 1 / 3)


def test_route_special_values_order():
    """Infinities order as numbers, -0 ties +0 (lower id first) and NaN
    ranks after every number (lower id first among NaNs): the order written
    out by hand for one row."""
    with np.errstate(invalid="ignore"):
        r = oracle.moe_route(np.array([[np.nan, -0.0, 0.0, 1.0, -np.inf, np.inf, 1.0, np.nan]], np.float32), 8)
    assert r["topk_ids"][0].tolist() == [5, 3, 6, 1, 2, 4, 0, 7]


def test_swiglu_bf16_rounding():
    g = np.array([0.0, 1.0, -1.0, 20.0, -30.0, 0.5])
    u = np.array([3.0, 2.0, 2.0, 1.5, 1.0, -7.25])
    h = oracle.swiglu_bf16(g, u)
    ref = g / (1 + np.exp(-g)) * u
    want = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(h, want)
    # double rounding guard: values just above a bf16 midpoint
    mid = np.float64(1.0 + 2.0 ** -8)                  # exact bf16 midpoint of 1 and 1+2^-7
    hh = M._f64_to_bf16_bits(np.array([mid, mid + 2.0 ** -40, mid - 2.0 ** -40]))
    assert hh.tolist() == [0x3F80, 0x3F81, 0x3F80]


def _quant_moe_weights(w_gu, w_d, fmt):
    E = w_gu.shape[0]
    out = dict(gu_c=[], gu_s=[], gu_t=[], d_c=[], d_s=[], d_t=[])
    I = w_gu.shape[1] // 2
    for e in range(E):
        if fmt == "e8m0_b32":
            c, s = oracle.quantize_e8m0_b32(w_gu[e])
            out["gu_c"].append(c); out["gu_s"].append(s)
            c, s = oracle.quantize_e8m0_b32(w_d[e])
            out["d_c"].append(c); out["d_s"].append(s)
        else:
            q = oracle.quantize_e4m3_b16 if fmt == "e4m3_b16" else oracle.quantize_e5m3_b16
            cg, sg, tg = q(w_gu[e][:I])
            cu, su, tu = q(w_gu[e][I:])
            out["gu_c"].append(np.concatenate([cg, cu])); out["gu_s"].append(np.concatenate([sg, su]))
            out["gu_t"].append([tg, tu])
            c, s, t = q(w_d[e])
            out["d_c"].append(c); out["d_s"].append(s); out["d_t"].append(t)
    return {k: np.array(v) for k, v in out.items()}


def _quant_act(x, fmt):
    if fmt == "e8m0_b32":
        c, s = oracle.quantize_e8m0_b32(x)
        return c, s, None
    return (oracle.quantize_e4m3_b16 if fmt == "e4m3_b16" else oracle.quantize_e5m3_b16)(x)


def _ffn(x, logits, w_gu, w_d, topk, fmt, tokens=None):
    W = _quant_moe_weights(w_gu, w_d, fmt)
    route = oracle.moe_route(logits, topk)
    ac, as_, at = _quant_act(x, fmt)
    g, u = oracle.moe_gateup(ac, as_, fmt, route, W["gu_c"], W["gu_s"], at, W["gu_t"] if len(W["gu_t"]) else None)
    h = oracle.bf16_bits_to_f32(oracle.swiglu_bf16(g, u))
    hc, hs, ht = _quant_act(h, fmt)
    y = oracle.moe_down_combine(hc, hs, fmt, route, W["d_c"], W["d_s"], ht,
                                W["d_t"] if len(W["d_t"]) else None, tokens=tokens)
    return y, dict(W=W, route=route, g=g, u=u, h=h, hc=hc, hs=hs, ht=ht, ac=ac, as_=as_, at=at)


@pytest.mark.parametrize("fmt", ["e8m0_b32", "e4m3_b16", "e5m3_b16"])
def test_one_expert_top1_is_dense_swiglu_ffn(fmt):
    rng = np.random.default_rng(20)
    T, H, I = 9, 64, 96
    x = rng.standard_normal((T, H)).astype(np.float32)
    w_gu = (rng.standard_normal((1, 2 * I, H)) * 0.05).astype(np.float32)
    w_d = (rng.standard_normal((1, H, I)) * 0.05).astype(np.float32)
    y, st = _ffn(x, np.zeros((T, 1), np.float32), w_gu, w_d, 1, fmt)
    W = st["W"]
    if fmt == "e8m0_b32":
        gu = oracle.mx_gemm(st["ac"], st["as_"], W["gu_c"][0], W["gu_s"][0])
        g, u = gu[:, :I], gu[:, I:]
        y_ref = oracle.mx_gemm(st["hc"], st["hs"], W["d_c"][0], W["d_s"][0])
    else:
        g = oracle.mx_gemm(st["ac"], st["as_"], W["gu_c"][0][:I], W["gu_s"][0][:I], fmt, st["at"], W["gu_t"][0][0])
        u = oracle.mx_gemm(st["ac"], st["as_"], W["gu_c"][0][I:], W["gu_s"][0][I:], fmt, st["at"], W["gu_t"][0][1])
        y_ref = oracle.mx_gemm(st["hc"], st["hs"], W["d_c"][0], W["d_s"][0], fmt, st["ht"], W["d_t"][0])
    # one pair per token, in token order
    assert np.array_equal(st["route"]["pair_token"], np.arange(T))
    assert np.array_equal(st["g"], g) and np.array_equal(st["u"], u)
    assert np.array_equal(y, y_ref)


def test_identical_experts_make_routing_irrelevant():
    rng = np.random.default_rng(21)
    T, H, I, E = 12, 64, 64, 6
    x = rng.standard_normal((T, H)).astype(np.float32)
    w_gu = np.repeat((rng.standard_normal((1, 2 * I, H)) * 0.05).astype(np.float32), E, axis=0)
    w_d = np.repeat((rng.standard_normal((1, H, I)) * 0.05).astype(np.float32), E, axis=0)
    y1, _ = _ffn(x, rng.standard_normal((T, E)).astype(np.float32), w_gu, w_d, 3, "e8m0_b32")
    y2, _ = _ffn(x, rng.standard_normal((T, E)).astype(np.float32), w_gu, w_d, 2, "e8m0_b32")
    assert np.allclose(y1, y2, rtol=1e-12, atol=1e-12)


def test_token_subset_matches_full():
    rng = np.random.default_rng(22)
    T, H, I, E = 20, 64, 64, 4
    x = rng.standard_normal((T, H)).astype(np.float32)
    w_gu = (rng.standard_normal((E, 2 * I, H)) * 0.05).astype(np.float32)
    w_d = (rng.standard_normal((E, H, I)) * 0.05).astype(np.float32)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    y, _ = _ffn(x, logits, w_gu, w_d, 2, "e4m3_b16")
    ys, _ = _ffn(x, logits, w_gu, w_d, 2, "e4m3_b16", tokens=[3, 0, 19])
    assert np.array_equal(ys, y[[3, 0, 19]])


# ---------------------------------------------------------------------------
# PRQuant tail residual on the expert down-projections
# ---------------------------------------------------------------------------

def _residual_problem(seed, T=10, H=64, I=128, E=3, topk=2, tail=64, on_grid=False):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((T * topk, I)).astype(np.float32)
    w_d = (rng.standard_normal((E, H, I)) * 0.05).astype(np.float32)
    if on_grid:   # weights that MXFP4 represents exactly: R = 0
        w_d = np.stack([oracle.dequantize(*oracle.quantize_e8m0_b32(w_d[e]), "e8m0_b32").astype(np.float32)
                        for e in range(E)])
    route = oracle.moe_route(rng.standard_normal((T, E)).astype(np.float32), topk)
    hc, hs = oracle.quantize_e8m0_b32(h)
    wc, ws, rc, rs = [], [], [], []
    for e in range(E):
        c, s = oracle.quantize_e8m0_b32(w_d[e])
        r = oracle.residual_weight(w_d[e], c, s, tail)
        r_c, r_s = oracle.quantize_e8m0_b32(r)
        wc.append(c); ws.append(s); rc.append(r_c); rs.append(r_s)
    return hc, hs, route, np.array(wc), np.array(ws), np.array(rc), np.array(rs), w_d, h


def test_residual_down_is_the_augmented_gemm():
    """Y with the residual term equals the plain down GEMM over [H, H_tail] x
    [W, R] (the online tail copy of the activation, the concatenated weight)."""
    hc, hs, route, wc, ws, rc, rs, _, _ = _residual_problem(40)
    y = oracle.moe_down_combine_residual(hc, hs, route, wc, ws, rc, rs, 64)
    ac, as_ = oracle.tail_copy(hc, hs, 64)
    y_aug = oracle.moe_down_combine(ac, as_, "e8m0_b32", route, np.concatenate([wc, rc], axis=2),
                                    np.concatenate([ws, rs], axis=2))
    assert np.allclose(y, y_aug, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_residual_down_special_cases():
    hc, hs, route, wc, ws, rc, rs, _, _ = _residual_problem(41)
    plain = oracle.moe_down_combine(hc, hs, "e8m0_b32", route, wc, ws)
    assert np.array_equal(oracle.moe_down_combine_residual(hc, hs, route, wc, ws, rc[..., :0], rs[..., :0], 0), plain)
    # weights already on the MXFP4 grid: the residual quantizes to zero codes and changes nothing
    hc, hs, route, wc, ws, rc, rs, _, _ = _residual_problem(42, on_grid=True)
    assert np.all((oracle.unpack_nibbles(rc) & 7) == 0)
    plain = oracle.moe_down_combine(hc, hs, "e8m0_b32", route, wc, ws)
    assert np.array_equal(oracle.moe_down_combine_residual(hc, hs, route, wc, ws, rc, rs, 64), plain)


def test_residual_down_reduces_weight_error():
    """Sanity for the method: the residual term moves the output toward the
    unquantized weights (same quantized activations on both sides)."""
    hc, hs, route, wc, ws, rc, rs, w_d, _ = _residual_problem(43, tail=64)
    hd = oracle.dequantize(hc, hs, "e8m0_b32")
    exact = np.zeros((10, 64))
    for e in range(3):
        p = np.arange(route["expert_offsets"][e], route["expert_offsets"][e + 1])
        t = route["pair_token"][p]
        j = np.argmax(route["topk_ids"][t] == e, axis=1)
        np.add.at(exact, t, route["topk_w"][t, j][:, None] * (hd[p] @ w_d[e].astype(np.float64).T))
    plain = oracle.moe_down_combine(hc, hs, "e8m0_b32", route, wc, ws)
    res = oracle.moe_down_combine_residual(hc, hs, route, wc, ws, rc, rs, 64)
    assert np.linalg.norm(res - exact) < np.linalg.norm(plain - exact)


# ---------------------------------------------------------------------------
# Distinct experts: the grouped stages against scalar loops over the pairs
# ---------------------------------------------------------------------------
#
# The gated MLP of the PRQuant page (§4 Eq. (1)) applied to each routed
# expert: for token t and its j-th chosen expert e,
#   g = a_t . W_gate,e rows, u = a_t . W_up,e rows, h = bf16(silu(g) * u),
#   y_t = sum_j w_tj * deq(hq_(t,j)) . W_down,e rows.
# The loops below walk tokens and slots (not the pair list), decode every
# element from the format's closed form with a local table (the E2M1 value set
# of the golden file; E8M0 2^(s-127); E4M3 (1 + m/8) 2^(e-7), (m/8) 2^-6) and
# sum products one at a time in float64.  Every expert's weights are drawn
# independently, so an oracle that contracts a pair with the wrong expert's
# weight, or shifts a segment by one expert, disagrees with them.

import json
import os

import oracle.native

# both oracles (numpy, C++) are held to the same loops
IMPLS = pytest.mark.parametrize("impl", [oracle, oracle.native], ids=["numpy", "cpp"])

_GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mx_formats.json")))
_E2M1 = _GOLD["e2m1_values"]["magnitudes"]


def _nib(packed_row, k):
    b = int(packed_row[k // 2])
    return (b >> 4) & 15 if k & 1 else b & 15


def _e2m1(c):
    return -_E2M1[c & 7] if c & 8 else _E2M1[c & 7]


def _scale(code, fmt):
    c = int(code)
    if fmt == "e8m0_b32":
        return math.ldexp(1.0, c - 127)
    e, m = (c >> 3) & 15, c & 7
    return (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * math.ldexp(1.0, e - 7)


def _elem(codes, scales, r, k, fmt):
    bs = 32 if fmt == "e8m0_b32" else 16
    return _e2m1(_nib(codes[r], k)) * _scale(scales[r][k // bs], fmt)


def _dot(ac, as_, ar, wc, ws, wr, K, fmt):
    s = 0.0
    for k in range(K):
        s += _elem(ac, as_, ar, k, fmt) * _elem(wc, ws, wr, k, fmt)
    return s


def _bf16(v):
    """float64 -> nearest bf16 value (ties to even); below bf16's normal
    range (2^-126) the spacing is that of its subnormals, 2^-133."""
    if v == 0.0:
        return v
    if abs(v) < 2.0 ** -126:
        return math.ldexp(round(math.ldexp(v, 133)), -133)   # round(): ties to even on floats
    m, e = math.frexp(v)                 # v = m 2^e, 0.5 <= |m| < 1
    return math.ldexp(round(m * 256.0), e - 8)


def _rand_codes(rng, shape):
    return rng.integers(0, 256, size=shape, dtype=np.uint8)


def _rand_scales(rng, shape, fmt):
    if fmt == "e8m0_b32":
        return rng.integers(118, 131, size=shape).astype(np.uint8)
    return rng.integers(0x28, 0x48, size=shape).astype(np.uint8)      # E4M3 codes around 1


def _distinct_problem(fmt, seed, T=7, H=64, I=32, E=3, k=2):
    rng = np.random.default_rng(seed)
    bs = 32 if fmt == "e8m0_b32" else 16
    logits = rng.standard_normal((T, E)).astype(np.float32)
    route = oracle.moe_route(logits, k)
    d = dict(route=route, T=T, H=H, I=I, E=E, k=k, bs=bs,
             ac=_rand_codes(rng, (T, H // 2)), as_=_rand_scales(rng, (T, H // bs), fmt),
             gc=_rand_codes(rng, (E, 2 * I, H // 2)), gs=_rand_scales(rng, (E, 2 * I, H // bs), fmt),
             hc=_rand_codes(rng, (T * k, I // 2)), hs=_rand_scales(rng, (T * k, I // bs), fmt),
             dc=_rand_codes(rng, (E, H, I // 2)), ds=_rand_scales(rng, (E, H, I // bs), fmt))
    if fmt != "e8m0_b32":
        d.update(a_ts=np.float32(0.375), g_ts=np.array([[0.5 + e, 1.25 * (e + 1)] for e in range(E)], np.float32),
                 h_ts=np.float32(1.5), d_ts=np.array([2.0 ** -e + 0.25 for e in range(E)], np.float32))
    return d


def _loop_gateup(d, fmt):
    """g, u [P][I] in pair order, from token/slot loops."""
    r = d["route"]
    I, H = d["I"], d["H"]
    P = d["T"] * d["k"]
    g = np.zeros((P, I))
    u = np.zeros((P, I))
    for t in range(d["T"]):
        for j in range(d["k"]):
            e = int(r["topk_ids"][t, j])
            p = int(r["pair_pos"][t, j])
            for i in range(I):
                gv = _dot(d["ac"], d["as_"], t, d["gc"][e], d["gs"][e], i, H, fmt)
                uv = _dot(d["ac"], d["as_"], t, d["gc"][e], d["gs"][e], I + i, H, fmt)
                if fmt != "e8m0_b32":
                    gv *= float(d["a_ts"]) * float(d["g_ts"][e][0])
                    uv *= float(d["a_ts"]) * float(d["g_ts"][e][1])
                g[p, i], u[p, i] = gv, uv
    return g, u


def _loop_down(d, fmt, hc, hs, dc, ds, I):
    """y [T][H]: for each token, its slots in order, weighted by topk_w."""
    r = d["route"]
    y = np.zeros((d["T"], d["H"]))
    for t in range(d["T"]):
        for j in range(d["k"]):
            e = int(r["topk_ids"][t, j])
            p = int(r["pair_pos"][t, j])
            w = float(r["topk_w"][t, j])
            for n in range(d["H"]):
                o = _dot(hc, hs, p, dc[e], ds[e], n, I, fmt)
                if fmt != "e8m0_b32":
                    o *= float(d["h_ts"]) * float(d["d_ts"][e])
                y[t, n] += w * o
    return y


@IMPLS
@pytest.mark.parametrize("fmt", ["e8m0_b32", "e4m3_b16"])
def test_gateup_distinct_experts_scalar_loop(fmt, impl):
    d = _distinct_problem(fmt, 50)
    assert len(set(d["route"]["topk_ids"].reshape(-1).tolist())) == d["E"]   # every expert owns pairs
    g_ref, u_ref = _loop_gateup(d, fmt)
    g, u = impl.moe_gateup(d["ac"], d["as_"], fmt, d["route"], d["gc"], d["gs"], d.get("a_ts"), d.get("g_ts"))
    # every product has <= 12 significant bits and the sums span far fewer than
    # 53 bits: both sides hold the exact value
    assert np.array_equal(g, g_ref) and np.array_equal(u, u_ref)
    # a subset of pairs, in a scrambled order
    pairs = np.array([5, 0, 13, 2])
    gs, us = impl.moe_gateup(d["ac"], d["as_"], fmt, d["route"], d["gc"], d["gs"], d.get("a_ts"), d.get("g_ts"),
                             pairs=pairs)
    assert np.array_equal(gs, g_ref[pairs]) and np.array_equal(us, u_ref[pairs])
    # the loop tells experts apart: with experts 0 and 1 swapped it disagrees
    sw = dict(d, gc=d["gc"][[1, 0, 2]], gs=d["gs"][[1, 0, 2]])
    if fmt != "e8m0_b32":
        sw["g_ts"] = d["g_ts"][[1, 0, 2]]
    g_sw, _ = _loop_gateup(sw, fmt)
    assert not np.array_equal(g_sw, g)


@IMPLS
def test_swiglu_of_gateup_scalar_loop(impl):
    """h = bf16(silu(g) u) element by element against a scalar frexp/round."""
    d = _distinct_problem("e8m0_b32", 51)
    g, u = impl.moe_gateup(d["ac"], d["as_"], "e8m0_b32", d["route"], d["gc"], d["gs"])
    h = oracle.bf16_bits_to_f32(impl.swiglu_bf16(g, u)).astype(np.float64)
    for p in range(g.shape[0]):
        for i in range(g.shape[1]):
            z = g[p, i]
            # z e^z / (1 + e^z) where e^-z would overflow (the result is then far below bf16's range)
            s = z / (1.0 + math.exp(-z)) if z > -700.0 else z * math.exp(z) / (1.0 + math.exp(z))
            assert h[p, i] == _bf16(s * u[p, i])


@IMPLS
@pytest.mark.parametrize("fmt", ["e8m0_b32", "e4m3_b16"])
def test_down_combine_distinct_experts_scalar_loop(fmt, impl):
    d = _distinct_problem(fmt, 52)
    y_ref = _loop_down(d, fmt, d["hc"], d["hs"], d["dc"], d["ds"], d["I"])
    y = impl.moe_down_combine(d["hc"], d["hs"], fmt, d["route"], d["dc"], d["ds"], d.get("h_ts"), d.get("d_ts"))
    # per-pair outputs are exact; the weighted sums of k terms round in a
    # different order
    assert np.allclose(y, y_ref, rtol=1e-13, atol=1e-13 * np.abs(y_ref).max())
    toks = [6, 1, 3]
    ys = impl.moe_down_combine(d["hc"], d["hs"], fmt, d["route"], d["dc"], d["ds"], d.get("h_ts"),
                               d.get("d_ts"), tokens=toks)
    assert np.allclose(ys, y_ref[toks], rtol=1e-13, atol=1e-13 * np.abs(y_ref).max())
    # a mistaken oracle -- the pairs of expert 1 contracted with expert 2's
    # down weight -- fails this comparison
    bad = d["dc"].copy()
    bad[1] = d["dc"][2]
    bad_s = d["ds"].copy()
    bad_s[1] = d["ds"][2]
    y_bad = impl.moe_down_combine(d["hc"], d["hs"], fmt, d["route"], bad, bad_s, d.get("h_ts"), d.get("d_ts"))
    assert not np.allclose(y_bad, y_ref, rtol=1e-6, atol=1e-6 * np.abs(y_ref).max())


@IMPLS
def test_down_combine_residual_distinct_experts_scalar_loop(impl):
    """PRQuant residual on the down projections: the loop over I + tail with
    the activation's last `tail` columns read a second time against R_e."""
    fmt, tail = "e8m0_b32", 32
    d = _distinct_problem(fmt, 53, I=64)
    rng = np.random.default_rng(54)
    rc = _rand_codes(rng, (d["E"], d["H"], tail // 2))
    rs = _rand_scales(rng, (d["E"], d["H"], tail // 32), fmt)
    I = d["I"]
    hc_aug = np.concatenate([d["hc"], d["hc"][:, (I - tail) // 2:]], axis=1)
    hs_aug = np.concatenate([d["hs"], d["hs"][:, (I - tail) // 32:]], axis=1)
    y_ref = _loop_down(d, fmt, hc_aug, hs_aug, np.concatenate([d["dc"], rc], axis=2),
                       np.concatenate([d["ds"], rs], axis=2), I + tail)
    y = impl.moe_down_combine_residual(d["hc"], d["hs"], d["route"], d["dc"], d["ds"], rc, rs, tail)
    assert np.allclose(y, y_ref, rtol=1e-13, atol=1e-13 * np.abs(y_ref).max())
