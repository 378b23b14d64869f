"""GPU parity: MoE routing and the grouped expert GEMMs (MXFP4, VQ->MX and
E4M3-B16 weights) against the oracle, stage by stage.

The oracle always runs from the synthetic inputs alone (its own
quantization of x, the weights and h); GPU outputs are compared with it and
are never fed into it.
* routing: expert ids, offsets and pair lists bit-exact; weights to 2e-6.
* x and weight encodings: bit-exact.
* gate/up: the GPU's bf16 h against the oracle's bf16(silu(g)u) within one
  bf16 rounding step (2^-8 relative) plus the 1e-3 row tolerance (the GPU
  accumulates g, u in fp32, the oracle exactly).
* requantized h: every 32/16-element block whose h the two sides rounded to
  the same bf16 values must carry the same codes and scale (bit-exact);
  blocks whose h differs by a bf16 step may differ and are counted.
* down/combine on the oracle's own quantized h (uploaded to the GPU): every
  sampled token within the 1e-3 row tolerance, in all three combine modes;
* the whole GPU pipeline: tokens whose h rows were requantized identically
  within 1e-3 * ||row||; a token whose h carries legitimately flipped codes
  within 1e-3 * ||row|| plus the exact effect of those code differences
  through its down weights (see _run_and_check).
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.native as on
import synth
from parity import assert_rows_close, banner, to_np, u16, vq_ref_block_scales

pytestmark = pytest.mark.gpu

try:
    import gemm_bit_weight_amd as gbw
except ImportError as e:
    gbw = None
    _IMPORT_ERROR = e

DEV = "cuda"


def setup_module():
    assert gbw is not None, f"HIP library missing: {_IMPORT_ERROR}"
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def _route_np(r):
    return {k: to_np(v) for k, v in r.items()}


def _check_route(logits, topk):
    r = gbw.moe_route(logits, topk)
    ref = oracle.moe_route(to_np(logits), topk)
    g = _route_np(r)
    assert np.array_equal(g["topk_ids"], ref["topk_ids"])
    assert np.array_equal(g["expert_offsets"], ref["expert_offsets"])
    assert np.array_equal(g["pair_token"], ref["pair_token"])
    assert np.array_equal(g["pair_pos"], ref["pair_pos"])
    assert np.allclose(g["topk_w"], ref["topk_w"], rtol=2e-6, atol=1e-7)
    return r, ref


@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (37, 16, 4), (200, 64, 6), (4096, 128, 8), (8192, 128, 8),
                                   (130, 1000, 16), (20000, 128, 8), (1100, 1000, 8)])
def test_route(T, E, k):
    banner(f"route T={T} E={E} k={k}")
    logits = synth.normal((T, E), 1.0, T + E, "route.l", DEV)
    _check_route(logits, k)


def test_route_ties_and_permutation():
    banner("route ties")
    T, E = 70, 32
    logits = torch.zeros((T, E), dtype=torch.float32, device=DEV)
    logits[1] = torch.arange(E, dtype=torch.float32).flip(0)
    logits[2, 5] = -0.0
    logits[3, ::3] = 1.0
    _check_route(logits, 8)


@pytest.mark.parametrize("E,k", [(128, 8), (200, 6), (300, 8)])
def test_route_special_values(E, k):
    """Logits drawn from {+-0, +-1, +-inf, NaN}: -0 ties +0 and NaN ranks
    below every number, as in the oracle's stable sort of the negated logits
    (E = 128 and 200 run the lane-group kernel, 300 the per-token one)."""
    banner(f"route special values E={E} k={k}")
    vals = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan, -np.nan], dtype=np.float32)
    rng = np.random.default_rng(E * 31 + k)
    logits = torch.from_numpy(vals[rng.integers(0, 8, size=(300, E))]).to(DEV)
    r = gbw.moe_route(logits, k)
    with np.errstate(invalid="ignore"):  # inf - inf in the weights of tokens led by +inf
        ref = oracle.moe_route(to_np(logits), k)
    g = _route_np(r)
    for key in ("topk_ids", "expert_offsets", "pair_token", "pair_pos"):
        assert np.array_equal(g[key], ref[key]), key
    assert np.allclose(g["topk_w"], ref["topk_w"], rtol=2e-6, atol=1e-7, equal_nan=True)


def _bf16_ulp(v):
    """Spacing of bf16 numbers at |v| (float64 array)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def _check_h(h_gpu_bits, h_ref):
    h_gpu = oracle.bf16_bits_to_f32(h_gpu_bits).astype(np.float64)
    err = np.abs(h_gpu - h_ref)
    bound = _bf16_ulp(h_ref) + 1e-3 * np.linalg.norm(h_ref, axis=1, keepdims=True)
    assert np.all(err <= bound), f"h outside tolerance: worst {np.max(err / bound):.3f}"


def _check_requant(h_gpu_bits, h_ref_bits, codes_gpu, scales_gpu, codes_ref, scales_ref, bs):
    """Blocks with identical h on both sides must quantize identically."""
    P, I = h_ref_bits.shape
    same = (h_gpu_bits.reshape(P, I // bs, bs) == h_ref_bits.reshape(P, I // bs, bs)).all(axis=2)
    c_eq = (oracle.unpack_nibbles(codes_gpu).reshape(P, I // bs, bs) ==
            oracle.unpack_nibbles(codes_ref).reshape(P, I // bs, bs)).all(axis=2)
    s_eq = scales_gpu == scales_ref
    blk_eq = c_eq & s_eq
    assert np.all(blk_eq[same]), f"{int((~blk_eq[same]).sum())} blocks with identical h quantized differently"
    frac = float((~blk_eq).mean())
    assert frac < 0.05, f"too many blocks differ ({frac:.3%})"
    return blk_eq.all(axis=1)   # rows requantized identically


class _LazyExperts:
    """Per-expert arrays materialized on first use (the oracle only touches
    the experts that own the pairs it is asked about)."""

    def __init__(self, shape, make):
        self.shape = shape
        self._make = make
        self._cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self._cache:
            self._cache[e] = self._make(e)
        return self._cache[e]


class _Problem:
    """One MoE FFN problem: synthetic inputs, the oracle's view of them, and
    the GPU weight descriptors built from the same inputs."""

    # VQ weights by scale layout (MXCode PreScale, PostScale, PreScale+) and
    # scale format: (layout, library format, the oracle's format name)
    VQ = {"vq": ("prescale", gbw.FMT_VQ4_E8M0, "e8m0_b32"), "vq_post": ("postscale", gbw.FMT_VQ4_POST, "e8m0_b32"),
          "vq_plus": ("prescale_plus", gbw.FMT_VQ4_PLUS, "e8m0_b32"),
          "vq_e4m3": ("prescale", gbw.FMT_VQ4_E4M3, "e4m3_b16"),
          "vq_e4m3_post": ("postscale", gbw.FMT_VQ4_E4M3_POST, "e4m3_b16"),
          "vq_e4m3_plus": ("prescale_plus", gbw.FMT_VQ4_E4M3_PLUS, "e4m3_b16"),
          "vq_e5m3": ("prescale", gbw.FMT_VQ4_E5M3, "e5m3_b16"),
          "vq_e5m3_post": ("postscale", gbw.FMT_VQ4_E5M3_POST, "e5m3_b16"),
          "vq_e5m3_plus": ("prescale_plus", gbw.FMT_VQ4_E5M3_PLUS, "e5m3_b16")}

    def __init__(self, fmt, x, logits, topk, gate_up, down, I, qblock=64):
        self.fmt, self.x, self.logits, self.topk, self.I = fmt, x, logits, topk, I
        self.ofmt = self.VQ[fmt][2] if fmt in self.VQ else fmt   # the activation / oracle format
        T, H = x.shape
        self.T, self.H = T, H
        E = (gate_up["w"] if fmt not in self.VQ else gate_up["idx"]).shape[0]
        self.E = E
        if fmt in self.VQ:
            mode, gfmt, ofmt = self.VQ[fmt]
            b16 = ofmt != "e8m0_b32"
            bs = 16 if b16 else 32

            def weight(v, N, K, nts):
                return gbw.Weight(gfmt, N, K, v["idx"].to(DEV), v["scales"].to(DEV), v["codebook"].to(DEV),
                                  v["tensor_scale"].to(DEV) if b16 else None, nts, E, qblock=qblock,
                                  scale_codebook=v["scale_codebook"].to(DEV) if "scale_codebook" in v else None)
            self.Wgu = weight(gate_up, 2 * I, H, 2)
            self.Wd = weight(down, H, I, 1)
            gcpu = {k: v.cpu() for k, v in gate_up.items()}
            dcpu = {k: v.cpu() for k, v in down.items()}
            self.ref_gu = (_LazyExperts((E, 2 * I, H // 2), lambda e: oracle.vq_decode_codes(
                gcpu["idx"][e].numpy(), gcpu["codebook"][e].numpy().view(np.uint16), qblock)),
                _LazyExperts((E, 2 * I, H // bs), lambda e: vq_ref_block_scales(gcpu, e, mode, H, qblock, bs)),
                _LazyExperts((E, 2), lambda e: list(gcpu["tensor_scale"][e].numpy())) if b16 else None)
            self.ref_d = (_LazyExperts((E, H, I // 2), lambda e: oracle.vq_decode_codes(
                dcpu["idx"][e].numpy(), dcpu["codebook"][e].numpy().view(np.uint16), qblock)),
                _LazyExperts((E, H, I // bs), lambda e: vq_ref_block_scales(dcpu, e, mode, I, qblock, bs)),
                _LazyExperts((E,), lambda e: dcpu["tensor_scale"][e].numpy()[0]) if b16 else None)
            return
        wgu, wd = gate_up["w"], down["w"]          # fp32 [E][2I][H], [E][H][I] (on the GPU)
        if fmt == "e8m0_b32":
            q = gbw.mx_quantize(wgu.reshape(E * 2 * I, H), gbw.FMT_E8M0_B32)
            self.Wgu = gbw.Weight(gbw.FMT_E8M0_B32, 2 * I, H, q.codes.view(E, 2 * I, H // 2),
                                  q.scales.view(E, 2 * I, H // 32), n_experts=E)
            q = gbw.mx_quantize(wd.reshape(E * H, I), gbw.FMT_E8M0_B32)
            self.Wd = gbw.Weight(gbw.FMT_E8M0_B32, H, I, q.codes.view(E, H, I // 2), q.scales.view(E, H, I // 32),
                                 n_experts=E)
            cache = {}

            def qe(which, e):
                key = (which, e)
                if key not in cache:
                    w = (wgu if which == "gu" else wd)[e].cpu().numpy()
                    cache[key] = oracle.quantize_e8m0_b32(w)
                return cache[key]
            self.ref_gu = (_LazyExperts((E, 2 * I, H // 2), lambda e: qe("gu", e)[0]),
                           _LazyExperts((E, 2 * I, H // 32), lambda e: qe("gu", e)[1]), None)
            self.ref_d = (_LazyExperts((E, H, I // 2), lambda e: qe("d", e)[0]),
                          _LazyExperts((E, H, I // 32), lambda e: qe("d", e)[1]), None)
            return
        # E4M3-B16 / E5M3-B16: every (expert, matrix) has its own dynamic tensor scale; gate and up separately
        gfmt = gbw.FMT_E4M3_B16 if fmt == "e4m3_b16" else gbw.FMT_E5M3_B16
        oq = oracle.quantize_e4m3_b16 if fmt == "e4m3_b16" else oracle.quantize_e5m3_b16
        gc = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=DEV)
        gs = torch.empty((E, 2 * I, H // 16), dtype=torch.uint8, device=DEV)
        gt = torch.empty((E, 2), dtype=torch.float32, device=DEV)
        dc = torch.empty((E, H, I // 2), dtype=torch.uint8, device=DEV)
        ds = torch.empty((E, H, I // 16), dtype=torch.uint8, device=DEV)
        dt = torch.empty((E, 1), dtype=torch.float32, device=DEV)
        for e in range(E):
            for half in range(2):
                rows = slice(half * I, (half + 1) * I)
                out = gbw.Act(gfmt, gc[e, rows], gs[e, rows])
                gbw.mx_quantize(wgu[e, rows].contiguous(), gfmt, out=out, tensor_scale=gt[e, half:half + 1],
                                dynamic=True)
            out = gbw.Act(gfmt, dc[e], ds[e])
            gbw.mx_quantize(wd[e].contiguous(), gfmt, out=out, tensor_scale=dt[e], dynamic=True)
        self.Wgu = gbw.Weight(gfmt, 2 * I, H, gc, gs, None, gt, 2, E)
        self.Wd = gbw.Weight(gfmt, H, I, dc, ds, None, dt, 1, E)
        cache = {}

        def q4(which, e):
            key = (which, e)
            if key not in cache:
                if which == "gu":
                    w = wgu[e].cpu().numpy()
                    a = oq(w[:I])
                    b = oq(w[I:])
                    cache[key] = (np.concatenate([a[0], b[0]]), np.concatenate([a[1], b[1]]), [a[2], b[2]])
                else:
                    cache[key] = oq(wd[e].cpu().numpy())
            return cache[key]
        self.ref_gu = (_LazyExperts((E, 2 * I, H // 2), lambda e: q4("gu", e)[0]),
                       _LazyExperts((E, 2 * I, H // 16), lambda e: q4("gu", e)[1]),
                       _LazyExperts((E, 2), lambda e: q4("gu", e)[2]))
        self.ref_d = (_LazyExperts((E, H, I // 2), lambda e: q4("d", e)[0]),
                      _LazyExperts((E, H, I // 16), lambda e: q4("d", e)[1]),
                      _LazyExperts((E,), lambda e: q4("d", e)[2]))

    def check_weight_encodings(self, experts):
        if self.fmt in self.VQ:
            return
        for e in experts:
            assert np.array_equal(to_np(self.Wgu.codes[e]), self.ref_gu[0][e])
            assert np.array_equal(to_np(self.Wgu.scales[e]), self.ref_gu[1][e])
            assert np.array_equal(to_np(self.Wd.codes[e]), self.ref_d[0][e])
            assert np.array_equal(to_np(self.Wd.scales[e]), self.ref_d[1][e])
            if self.fmt in ("e4m3_b16", "e5m3_b16"):
                assert np.array_equal(to_np(self.Wgu.tensor_scale[e]), np.array(self.ref_gu[2][e], np.float32))
                assert to_np(self.Wd.tensor_scale[e])[0] == self.ref_d[2][e]


def _deq_rows(codes, scales, fmt, ts=None):
    """Decode packed FP4 rows for the flip bound (a local closed-form table,
    not the oracle: these are the GPU's codes)."""
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    b = np.asarray(codes)
    nib = np.stack([b & 15, b >> 4], axis=-1).reshape(b.shape[0], -1).astype(np.int64)
    el = np.where(nib & 8, -mags[nib & 7], mags[nib & 7])
    sc = np.asarray(scales).astype(np.int64)
    if fmt == "e8m0_b32":
        s = np.ldexp(1.0, sc - 127)
        bs = 32
    else:
        bias = 7 if fmt == "e4m3_b16" else 15
        e, m = (sc >> 3) & (15 if fmt == "e4m3_b16" else 31), sc & 7
        s = np.where(e == 0, (m / 8.0) * np.ldexp(1.0, 1 - bias), (1 + m / 8.0) * np.ldexp(1.0, e - bias))
        bs = 16
    out = el * np.repeat(s, bs, axis=1)
    return out * (1.0 if ts is None else float(np.float32(ts)))


def _run_and_check(pb, tokens=None, experts=None, h_amax=None, exact=True):
    """Run the FFN on the GPU and check it against the oracle stage by stage.

    1. routing, Q(x) and the weight encodings bit-exact;
    2. gate/up: the GPU's bf16 h within one bf16 step (+ the row tolerance)
       of the oracle's bf16(silu(g) u), g and u exact;
    3. requantized h: blocks with identical bf16 h on both sides carry
       identical codes and scales;
    4. down + combine on the oracle's own quantized h (uploaded to the GPU):
       every sampled token within 1e-3 * ||row|| in all three combine modes
       (bf16 slots, fp32 slots, fp32 atomics);
    5. the whole GPU pipeline (the GPU's own h): tokens whose pairs were
       requantized identically within 1e-3 * ||row||; a token carrying code
       differences within 1e-3 * ||row|| plus the exact effect of those
       differences, sum_j w_tj sum_i |deq(hq_gpu) - deq(hq_ref)|_i |W_down,e[n, i]|.

    ``h_amax`` (tensor-scaled formats only): quantize h with the static
    tensor scale amax / (6 * top scale) on both sides instead of the dynamic
    one, so the oracle needs h only for the sampled pairs.  ``exact``: the
    E8M0 problem's dot products span fewer than 53 bits, so the oracle's sums
    must be exact (false for scale codes spread over the whole E8M0 range).
    """
    T, H, I, topk = pb.T, pb.H, pb.I, pb.topk
    fmt = pb.ofmt
    e4 = fmt in ("e4m3_b16", "e5m3_b16")          # tensor-scaled formats: h quantized by mx_quantize
    e5 = fmt == "e5m3_b16"
    afmt = (gbw.FMT_E5M3_B16 if e5 else gbw.FMT_E4M3_B16) if e4 else gbw.FMT_E8M0_B32
    oq = on.quantize_e5m3_b16 if e5 else on.quantize_e4m3_b16
    ots = oracle.formats.tensor_scale_e5m3 if e5 else oracle.formats.tensor_scale_e4m3
    bs = 16 if e4 else 32
    route, ref_route = _check_route(pb.logits, topk)
    P = T * topk
    # ---- GPU pipeline ----
    xq = gbw.mx_quantize(pb.x, afmt)
    hb = torch.empty((P, I), dtype=torch.bfloat16, device=DEV)
    if not e4:
        hc = torch.empty((P, I // 2), dtype=torch.uint8, device=DEV)
        hs = torch.empty((P, I // 32), dtype=torch.uint8, device=DEV)
        gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, pb.Wgu, h_bf16=hb, h_codes=hc, h_scales=hs)
        hq = gbw.Act(afmt, hc, hs)
    else:
        gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, pb.Wgu, h_bf16=hb)
        if h_amax is None:
            hq = gbw.mx_quantize(hb, afmt)
        else:
            st = torch.tensor([ots(np.float32(h_amax))], dtype=torch.float32, device=DEV)
            hq = gbw.mx_quantize(hb, afmt, tensor_scale=st, dynamic=False)
    y = torch.empty((T, H), dtype=torch.float32, device=DEV)
    gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, hq, pb.Wd, y=y)                 # bf16 slots
    y2 = torch.empty_like(y)
    gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, hq, pb.Wd, y=y2)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "slot combine differs between runs"
    # one workspace shared by several calls, as a serving loop passes it:
    # the bits of a fresh workspace each time
    wsd = torch.zeros(gbw.workspace_size(gbw.OP_MOE_GEMM, route["topk_ids"].numel(), H, 0), dtype=torch.uint8,
                      device=DEV)
    for _ in range(3):
        y3 = torch.empty_like(y)
        gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, hq, pb.Wd, y=y3, ws=wsd)
        torch.cuda.synchronize()
        assert torch.equal(y, y3), "a reused workspace changes the result"

    # ---- oracle pipeline, from the synthetic inputs only ----
    xn = pb.x.float().cpu().numpy()
    if e4:
        ac, as_, ats = oq(xn)
        assert to_np(xq.tensor_scale)[0] == ats
    else:
        ac, as_ = on.quantize_e8m0_b32(xn)
        ats = None
    assert np.array_equal(to_np(xq.codes), ac) and np.array_equal(to_np(xq.scales), as_)
    off = ref_route["expert_offsets"]
    if experts is None:
        experts = list(range(pb.E))
    pb.check_weight_encodings(experts[:4])
    if tokens is None:
        tokens = np.arange(T)
    tokens = np.asarray(tokens)
    whole = len(experts) == pb.E and len(tokens) == T

    def oracle_h(pairs):
        g, u = on.moe_gateup(ac, as_, fmt, ref_route, pb.ref_gu[0], pb.ref_gu[1], ats, pb.ref_gu[2], pairs=pairs)
        if not e4 and exact:
            assert on.last_inexact == 0
        return g, u, on.swiglu_bf16(g, u)

    def oracle_q(h_bits):
        hf = oracle.bf16_bits_to_f32(h_bits)
        if not e4:
            c, s = on.quantize_e8m0_b32(hf)
            return c, s, None
        return oq(hf, tensor_amax=h_amax)

    # gate/up + SwiGLU on every pair of the chosen experts
    pairs = np.concatenate([np.arange(off[e], off[e + 1]) for e in experts])
    g, u, h_ref_bits = oracle_h(pairs)
    _check_h(u16(hb)[pairs], g / (1.0 + np.exp(-g)) * u)

    # requantization of h
    if e4 and h_amax is None:
        assert whole, "a dynamic tensor scale needs the whole h"
        qc, qs, qts = oracle_q(h_ref_bits)
        same_ts = to_np(hq.tensor_scale)[0] == qts
        if same_ts:
            _check_requant(u16(hb), h_ref_bits, to_np(hq.codes), to_np(hq.scales), qc, qs, bs)
        full_c, full_s, hts = qc, qs, qts
    else:
        qc, qs, qts = oracle_q(h_ref_bits)
        if e4:
            assert to_np(hq.tensor_scale)[0] == qts
        _check_requant(u16(hb)[pairs], h_ref_bits, to_np(hq.codes)[pairs], to_np(hq.scales)[pairs], qc, qs, bs)
        # the sampled tokens' pairs, requantized by the oracle from its own h
        tp = np.sort(ref_route["pair_pos"][tokens].reshape(-1))
        _, _, hb_t = oracle_h(tp)
        qc_t, qs_t, hts = oracle_q(hb_t)
        full_c = np.zeros((P, I // 2), np.uint8)
        full_s = np.full((P, I // bs), 127 if not e4 else 0x38, np.uint8)
        full_c[tp], full_s[tp] = qc_t, qs_t

    # ---- stage: down + combine on the oracle's quantized h ----
    y_ref = on.moe_down_combine(full_c, full_s, fmt, ref_route, pb.ref_d[0], pb.ref_d[1], hts,
                                pb.ref_d[2] if e4 else None, tokens=tokens)
    if not e4 and exact:
        assert on.last_inexact == 0
    hq_o = gbw.Act(afmt, torch.from_numpy(full_c).to(DEV), torch.from_numpy(full_s).to(DEV),
                   torch.tensor([hts], dtype=torch.float32, device=DEV) if e4 else None)
    for name, kw in (("bf16 slots", {}), ("fp32 slots", dict(flags=gbw.FP32_COMBINE)), ("atomic", dict(ws=False))):
        yo = torch.empty((T, H), dtype=torch.float32, device=DEV)
        gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, hq_o, pb.Wd, y=yo, **kw)
        r = assert_rows_close(to_np(yo)[tokens], y_ref, what=f"moe down + combine on the oracle's h ({name})")
        print(f"[stats] down+combine ({name}) max row error ratio {r:.2e}", flush=True)

    # ---- the whole GPU pipeline: tokens with code differences get their exact effect as slack ----
    gc, gs = to_np(hq.codes), to_np(hq.scales)
    gts = to_np(hq.tensor_scale)[0] if e4 else None
    pp = ref_route["pair_pos"][tokens]                         # [n_tok][k]
    row_same = (gc[pp] == full_c[pp]).all(axis=2) & (gs[pp] == full_s[pp]).all(axis=2)
    clean = row_same.all(axis=1) & (not e4 or gts == hts)
    yv = to_np(y)[tokens].astype(np.float64)
    nrm = np.linalg.norm(y_ref, axis=1)
    err = np.abs(yv - y_ref)
    for i in np.nonzero(clean)[0]:
        assert err[i].max() <= 1e-3 * nrm[i], f"clean token {tokens[i]}: {err[i].max() / nrm[i]:.2e}"
    for i in np.nonzero(~clean)[0]:
        t = tokens[i]
        slack = np.zeros(H)
        for j in range(topk):
            p = int(pp[i, j])
            d = np.abs(_deq_rows(gc[p:p + 1], gs[p:p + 1], fmt, gts) - _deq_rows(full_c[p:p + 1], full_s[p:p + 1], fmt, hts))[0]
            if not d.any():
                continue
            e = int(ref_route["topk_ids"][t, j])
            wd = np.abs(on.dequantize(np.asarray(pb.ref_d[0][e]), np.asarray(pb.ref_d[1][e]), fmt,
                                      pb.ref_d[2][e] if e4 else None))
            slack += float(ref_route["topk_w"][t, j]) * (wd @ d)
        assert np.all(err[i] <= 1e-3 * nrm[i] + slack * (1 + 1e-6)), f"token {t}: error beyond its code differences"
    print(f"[stats] tokens whose pairs requantized identically: {clean.mean():.1%} of {len(tokens)}", flush=True)


def _mx_problem(T, H, I, E, k, seed=1):
    d = synth.moe_problem(T, H, I, E, seed=seed, device=DEV)
    return _Problem("e8m0_b32", d["x"], d["logits"], k, dict(w=d["w_gate_up"]), dict(w=d["w_down"]), I)


@pytest.mark.parametrize("T,H,I,E,k", [(300, 512, 256, 8, 2), (97, 256, 128, 5, 3), (64, 1024, 384, 16, 8)])
def test_moe_mxfp4_small(T, H, I, E, k):
    banner(f"moe mxfp4 T={T} H={H} I={I} E={E} k={k}")
    _run_and_check(_mx_problem(T, H, I, E, k))


@pytest.mark.parametrize("T,H,I,E,k", [(300, 512, 256, 8, 2), (97, 256, 128, 5, 3), (64, 1024, 384, 16, 8)])
def test_moe_e4m3_small(T, H, I, E, k):
    banner(f"moe e4m3 T={T} H={H} I={I} E={E} k={k}")
    d = synth.moe_problem(T, H, I, E, seed=3, device=DEV)
    pb = _Problem("e4m3_b16", d["x"], d["logits"], k, dict(w=d["w_gate_up"]), dict(w=d["w_down"]), I)
    _run_and_check(pb)
    _run_and_check(pb, h_amax=1.5)


@pytest.mark.parametrize("T,H,I,E,k", [(300, 512, 256, 8, 2), (513, 256, 384, 3, 2)])
def test_moe_vq_small(T, H, I, E, k):
    banner(f"moe vq T={T} H={H} I={I} E={E} k={k}")
    d = synth.moe_vq_problem(T, H, I, E, seed=2, device="cpu")
    _run_and_check(_Problem("vq", d["x"].to(DEV), d["logits"].to(DEV), k, d["gate_up"], d["down"], I))


@pytest.mark.parametrize("fmt,qblock,T,H,I,E,k", [("vq_post", 64, 300, 512, 256, 8, 2),
                                                  ("vq_plus", 64, 300, 512, 256, 8, 2),
                                                  ("vq_post", 128, 200, 768, 384, 6, 3),
                                                  ("vq_plus", 256, 260, 1024, 512, 5, 2),
                                                  ("vq", 128, 150, 512, 256, 4, 2)])
def test_moe_vq_scale_layouts_small(fmt, qblock, T, H, I, E, k):
    """MXCode PostScale and PreScale+ experts, and QBlocks above 64."""
    banner(f"moe {fmt} qblock={qblock} T={T} H={H} I={I} E={E} k={k}")
    mode = _Problem.VQ[fmt][0]
    d = synth.moe_vq_problem(T, H, I, E, seed=3, device="cpu", scales=mode, qblock=qblock)
    _run_and_check(_Problem(fmt, d["x"].to(DEV), d["logits"].to(DEV), k, d["gate_up"], d["down"], I, qblock))


@pytest.mark.parametrize("fmt", ["vq_post", "vq_plus"])
def test_moe_vq_scale_layouts_full_size_sampled(fmt):
    """The VQ->MX FFN shape (8192 tokens, H 4096, I 1536, 128 experts, top-8)
    with PostScale / PreScale+ scales; sampled experts and tokens."""
    banner(f"moe {fmt} full T=8192 H=4096 I=1536 E=128 k=8")
    mode = _Problem.VQ[fmt][0]
    d = synth.moe_vq_problem(8192, 4096, 1536, 128, seed=0, device=DEV, scales=mode)
    _run_and_check(_Problem(fmt, d["x"], d["logits"], 8, d["gate_up"], d["down"], 1536),
                   tokens=[0, 2049, 4097, 8191], experts=[0, 77, 127])


@pytest.mark.parametrize("fmt,qblock,T,H,I,E,k", [("vq_e4m3", 64, 300, 512, 256, 8, 2),
                                                  ("vq_e4m3_post", 64, 300, 512, 256, 8, 2),
                                                  ("vq_e4m3_plus", 128, 200, 768, 384, 6, 3),
                                                  ("vq_e5m3", 128, 260, 512, 256, 5, 2),
                                                  ("vq_e5m3_post", 256, 150, 1024, 512, 4, 2),
                                                  ("vq_e5m3_plus", 64, 300, 512, 256, 8, 2)])
def test_moe_vq_b16_small(fmt, qblock, T, H, I, E, k):
    """VQ experts with 16-element E4M3 / UE5M3 block scales (PreScale,
    PostScale, PreScale+) on the fp16 / bf16 MFMA kernel."""
    banner(f"moe {fmt} qblock={qblock} T={T} H={H} I={I} E={E} k={k}")
    mode = _Problem.VQ[fmt][0]
    sf = "e4m3" if "e4m3" in fmt else "e5m3"
    d = synth.moe_vq_problem(T, H, I, E, seed=4, device="cpu", scales=mode, qblock=qblock, scale_fmt=sf)
    _run_and_check(_Problem(fmt, d["x"].to(DEV), d["logits"].to(DEV), k, d["gate_up"], d["down"], I, qblock))


@pytest.mark.parametrize("fmt", ["vq_e4m3_post", "vq_e4m3_plus"])
def test_moe_vq_b16_e4m3_shape_sampled(fmt):
    """The E4M3-B16 MoE shape (4096 tokens, H 2048, I 768, 128 experts,
    top-8) with VQ weights; every pair of three experts, sampled tokens (h is
    quantized with a static tensor scale on both sides)."""
    banner(f"moe {fmt} T=4096 H=2048 I=768 E=128 k=8")
    mode = _Problem.VQ[fmt][0]
    d = synth.moe_vq_problem(4096, 2048, 768, 128, seed=0, device=DEV, scales=mode, scale_fmt="e4m3")
    _run_and_check(_Problem(fmt, d["x"], d["logits"], 8, d["gate_up"], d["down"], 768),
                   tokens=[0, 1, 2049, 4095], experts=[0, 64, 127], h_amax=4.0)


@pytest.mark.parametrize("fmt", ["e8m0_b32", "e4m3_b16", "vq", "vq_e5m3_plus"])
@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (3, 64, 2), (5, 1, 1), (40, 200, 3)])
def test_moe_edge_shapes(fmt, T, E, k):
    """One token, one expert, top-1, and most experts without a pair (every
    kernel then walks tiles of empty and one-row experts)."""
    banner(f"moe edge {fmt} T={T} E={E} k={k}")
    H, I = 256, 128
    if fmt.startswith("vq"):
        mode = _Problem.VQ[fmt][0]
        sf = "e8m0" if fmt == "vq" else "e5m3"
        d = synth.moe_vq_problem(T, H, I, E, seed=5, device="cpu", scales=mode, scale_fmt=sf)
        pb = _Problem(fmt, d["x"].to(DEV), d["logits"].to(DEV), k, d["gate_up"], d["down"], I)
    else:
        d = synth.moe_problem(T, H, I, E, seed=5, device=DEV)
        pb = _Problem(fmt, d["x"], d["logits"], k, dict(w=d["w_gate_up"]), dict(w=d["w_down"]), I)
    _run_and_check(pb)


def test_moe_mxfp4_wide_scale_codes():
    """MXFP4 experts with E8M0 codes far from the Gaussian band: x at 2^-120
    (activation scale codes near 1 .. 10), gate/up weights at 2^+120 (codes up
    to about 245), down weights at 2^-40: every product of scales stays a
    finite fp32, and the scaled MFMA's scale operands see both ends."""
    banner("moe mxfp4 wide scale codes T=300 H=512 I=256 E=8 k=2")
    d = synth.moe_problem(300, 512, 256, 8, seed=11, device=DEV)
    x = (d["x"].float() * 2.0 ** -120).to(torch.bfloat16)
    pb = _Problem("e8m0_b32", x, d["logits"], 2, dict(w=d["w_gate_up"] * 2.0 ** 120), dict(w=d["w_down"] * 2.0 ** -40),
                  256)
    sa = to_np(gbw.mx_quantize(x, gbw.FMT_E8M0_B32).scales)
    sw = to_np(pb.Wgu.scales)
    print(f"[stats] activation scale codes {sa.min()}..{sa.max()}, gate/up {sw.min()}..{sw.max()}", flush=True)
    assert sa.max() <= 12 and sw.max() >= 240
    _run_and_check(pb)


def test_moe_vq_wide_prescale_codes():
    """VQ->MX experts whose E8M0 prescales are drawn over 100 .. 253, against
    activations at 2^-100 (codes near 20 .. 30)."""
    banner("moe vq wide prescale codes T=300 H=512 I=256 E=8 k=2")
    d = synth.moe_vq_problem(300, 512, 256, 8, seed=12, device="cpu", x_log2=-100, gate_up_e8m0_range=(100, 253))
    pb = _Problem("vq", d["x"].to(DEV), d["logits"].to(DEV), 2, d["gate_up"], d["down"], 256)
    _run_and_check(pb, exact=False)


def test_moe_no_tokens():
    """T = 0: routing zeroes the expert offsets, both GEMM stages return OK
    and write nothing."""
    banner("moe T=0")
    E, H, I = 8, 256, 128
    logits = torch.empty((0, E), dtype=torch.float32, device=DEV)
    route = gbw.moe_route(logits, 2)
    torch.cuda.synchronize()
    assert to_np(route["expert_offsets"]).tolist() == [0] * (E + 1)
    d = synth.moe_problem(1, H, I, E, seed=6, device=DEV)
    pb = _Problem("e8m0_b32", d["x"], d["logits"], 2, dict(w=d["w_gate_up"]), dict(w=d["w_down"]), I)
    xq = gbw.Act(gbw.FMT_E8M0_B32, torch.empty((0, H // 2), dtype=torch.uint8, device=DEV),
                 torch.empty((0, H // 32), dtype=torch.uint8, device=DEV))
    hc = torch.empty((0, I // 2), dtype=torch.uint8, device=DEV)
    hs = torch.empty((0, I // 32), dtype=torch.uint8, device=DEV)
    gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, pb.Wgu, h_codes=hc, h_scales=hs)
    y = torch.full((0, H), 7.0, dtype=torch.float32, device=DEV)
    gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, gbw.Act(gbw.FMT_E8M0_B32, hc, hs), pb.Wd, y=y)
    torch.cuda.synchronize()


def test_moe_vq_full_size_sampled():
    """The measured prefill shape: T=8192, H=4096, I=1536, 128 experts,
    top-8; gate/up checked on every pair of two experts, y on sampled tokens."""
    banner("moe vq full T=8192 H=4096 I=1536 E=128 k=8")
    d = synth.moe_vq_problem(8192, 4096, 1536, 128, seed=0, device=DEV)
    _run_and_check(_Problem("vq", d["x"], d["logits"], 8, d["gate_up"], d["down"], 1536),
                   tokens=[0, 4097, 8191], experts=[0, 77])


@pytest.mark.parametrize("T,H,I,E,k", [(300, 512, 256, 8, 2), (64, 1024, 384, 16, 8)])
def test_moe_e5m3_small(T, H, I, E, k):
    banner(f"moe e5m3 T={T} H={H} I={I} E={E} k={k}")
    d = synth.moe_problem(T, H, I, E, seed=4, device=DEV)
    pb = _Problem("e5m3_b16", d["x"], d["logits"], k, dict(w=d["w_gate_up"]), dict(w=d["w_down"]), I)
    _run_and_check(pb)
    _run_and_check(pb, h_amax=1.5)


def test_moe_e5m3_full_size_sampled():
    """E5M3-B16 at the E4M3-B16 shape: T=4096, H=2048, I=768, 128 experts, top-8."""
    banner("moe e5m3 full T=4096 H=2048 I=768 E=128 k=8")
    d = synth.moe_problem(4096, 2048, 768, 128, seed=0, device=DEV)
    _run_and_check(_Problem("e5m3_b16", d["x"], d["logits"], 8, dict(w=d["w_gate_up"]), dict(w=d["w_down"]), 768),
                   tokens=[1, 2048, 4095], experts=[3, 100], h_amax=2.0)


def test_moe_e4m3_full_size_sampled():
    """The E4M3-B16 shape: T=4096, H=2048, I=768, 128 experts, top-8."""
    banner("moe e4m3 full T=4096 H=2048 I=768 E=128 k=8")
    d = synth.moe_problem(4096, 2048, 768, 128, seed=0, device=DEV)
    _run_and_check(_Problem("e4m3_b16", d["x"], d["logits"], 8, dict(w=d["w_gate_up"]), dict(w=d["w_down"]), 768),
                   tokens=[1, 2048, 4095], experts=[3, 100], h_amax=2.0)


def _prquant_weights(wd, tail):
    """Per expert: E8M0 down weight, its tail residual (mx_residual) quantized,
    and the augmented [W | R] rows the down stage reads over I + tail."""
    E, H, I = wd.shape
    qc = torch.empty((E, H, (I + tail) // 2), dtype=torch.uint8, device=DEV)
    qs = torch.empty((E, H, (I + tail) // 32), dtype=torch.uint8, device=DEV)
    plain_c = torch.empty((E, H, I // 2), dtype=torch.uint8, device=DEV)
    plain_s = torch.empty((E, H, I // 32), dtype=torch.uint8, device=DEV)
    for e in range(E):
        wq = gbw.mx_quantize(wd[e].contiguous(), gbw.FMT_E8M0_B32)
        r = gbw.mx_residual(wd[e].contiguous(), wq.codes, wq.scales, tail)
        rq = gbw.mx_quantize(r, gbw.FMT_E8M0_B32)
        qc[e] = torch.cat([wq.codes, rq.codes], dim=1)
        qs[e] = torch.cat([wq.scales, rq.scales], dim=1)
        plain_c[e], plain_s[e] = wq.codes, wq.scales
    return (gbw.Weight(gbw.FMT_E8M0_B32, H, I + tail, qc, qs, n_experts=E),
            gbw.Weight(gbw.FMT_E8M0_B32, H, I, plain_c, plain_s, n_experts=E))


@pytest.mark.parametrize("T,H,I,E,k,tail", [(300, 512, 256, 8, 2, 128), (64, 1024, 384, 16, 8, 128),
                                            (97, 256, 640, 5, 3, 256)])
def test_moe_prquant_down_residual(T, H, I, E, k, tail):
    """PRQuant on the expert down-projections: the gate/up stage appends the
    tail copy of the quantized h, the down stage runs over I + tail with
    [W_down | R] rows; checked against the oracle's residual formula."""
    banner(f"moe prquant T={T} H={H} I={I} E={E} k={k} tail={tail}")
    d = synth.moe_problem(T, H, I, E, seed=6, device=DEV)
    route, ref_route = _check_route(d["logits"], k)
    P = T * k
    wgu = d["w_gate_up"]
    q = gbw.mx_quantize(wgu.reshape(E * 2 * I, H), gbw.FMT_E8M0_B32)
    Wgu = gbw.Weight(gbw.FMT_E8M0_B32, 2 * I, H, q.codes.view(E, 2 * I, H // 2), q.scales.view(E, 2 * I, H // 32),
                     n_experts=E)
    Waug, Wplain = _prquant_weights(d["w_down"], tail)
    xq = gbw.mx_quantize(d["x"], gbw.FMT_E8M0_B32)
    hc = torch.empty((P, I // 2), dtype=torch.uint8, device=DEV)
    hs = torch.empty((P, I // 32), dtype=torch.uint8, device=DEV)
    gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, Wgu, h_codes=hc, h_scales=hs)
    hca = torch.empty((P, (I + tail) // 2), dtype=torch.uint8, device=DEV)
    hsa = torch.empty((P, (I + tail) // 32), dtype=torch.uint8, device=DEV)
    gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, Wgu, h_codes=hca, h_scales=hsa, h_tail=tail)
    # the appended columns are the online tail copy of the same quantized h
    assert torch.equal(hca[:, :I // 2], hc) and torch.equal(hca[:, I // 2:], hc[:, (I - tail) // 2:])
    assert torch.equal(hsa[:, :I // 32], hs) and torch.equal(hsa[:, I // 32:], hs[:, (I - tail) // 32:])
    # oracle weights from the fp32 down weights: Q(W), R = W_tail - Q(W)_tail, Q(R)
    wd = d["w_down"].cpu().numpy()
    wc, ws, rc, rs = [], [], [], []
    for e in range(E):
        c, s = on.quantize_e8m0_b32(wd[e])
        rq_c, rq_s = on.quantize_e8m0_b32(oracle.residual_weight(wd[e], c, s, tail))
        wc.append(c); ws.append(s); rc.append(rq_c); rs.append(rq_s)
    wc, ws, rc, rs = (np.array(v) for v in (wc, ws, rc, rs))
    assert np.array_equal(to_np(Waug.codes), np.concatenate([wc, rc], axis=2))
    assert np.array_equal(to_np(Waug.scales), np.concatenate([ws, rs], axis=2))
    # the oracle's own h: Q(x), gate/up, SwiGLU, Q(h)
    ac, as_ = on.quantize_e8m0_b32(d["x"].float().cpu().numpy())
    gq = [on.quantize_e8m0_b32(wgu[e].cpu().numpy()) for e in range(E)]
    g, u = on.moe_gateup(ac, as_, "e8m0_b32", ref_route, [c for c, _ in gq], [s for _, s in gq])
    h_ref = on.swiglu_bf16(g, u)
    qc, qs = on.quantize_e8m0_b32(oracle.bf16_bits_to_f32(h_ref))
    hb = torch.empty((P, I), dtype=torch.bfloat16, device=DEV)
    gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, Wgu, h_bf16=hb, h_codes=hc, h_scales=hs)
    _check_requant(u16(hb), h_ref, to_np(hc), to_np(hs), qc, qs, 32)
    # the down stage over I + tail, run on the oracle's quantized h (with its tail copy)
    hqa = gbw.Act(gbw.FMT_E8M0_B32, torch.from_numpy(np.concatenate([qc, qc[:, (I - tail) // 2:]], 1)).to(DEV),
                  torch.from_numpy(np.concatenate([qs, qs[:, (I - tail) // 32:]], 1)).to(DEV))
    y = torch.empty((T, H), dtype=torch.float32, device=DEV)
    gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, hqa, Waug, y=y)
    y_ref = on.moe_down_combine_residual(qc, qs, ref_route, wc, ws, rc, rs, tail)
    assert on.last_inexact == 0
    assert_rows_close(to_np(y), y_ref, what="moe down with the tail residual")
    # the residual moves the output toward the unquantized down weights
    y_plain = torch.empty_like(y)
    gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, gbw.Act(gbw.FMT_E8M0_B32, hqa.codes[:, :I // 2].contiguous(),
                                                              hqa.scales[:, :I // 32].contiguous()), Wplain, y=y_plain)
    hd = on.dequantize(qc, qs, "e8m0_b32")
    exact = np.zeros((T, H))
    off, pt = ref_route["expert_offsets"], ref_route["pair_token"]
    for e in range(E):
        p = np.arange(off[e], off[e + 1])
        t = pt[p]
        j = np.argmax(ref_route["topk_ids"][t] == e, axis=1)
        np.add.at(exact, t, ref_route["topk_w"][t, j][:, None] * (hd[p] @ wd[e].astype(np.float64).T))
    e_res = np.linalg.norm(to_np(y) - exact) / np.linalg.norm(exact)
    e_plain = np.linalg.norm(to_np(y_plain) - exact) / np.linalg.norm(exact)
    print(f"[stats] down-weight error with residual {e_res:.4f}, plain {e_plain:.4f}", flush=True)
    assert e_res < e_plain


def _offline_copy_weight(codes, scales, I, tail):
    """PRQuant offline copy: the gate and up weights with their last `tail`
    rows (output channels) duplicated, [E][2(I + tail)][...]: gate rows
    [0, I + tail), then up rows.  Rows are quantized along K on their own, so
    duplicating quantized rows is quantizing the duplicated weight."""
    g, u = codes[:, :I], codes[:, I:]
    gs, us = scales[:, :I], scales[:, I:]
    c = torch.cat([g, g[:, I - tail:], u, u[:, I - tail:]], dim=1).contiguous()
    sc = torch.cat([gs, gs[:, I - tail:], us, us[:, I - tail:]], dim=1).contiguous()
    return c, sc


@pytest.mark.parametrize("T,H,I,E,k,tail", [(300, 512, 256, 8, 2, 128), (64, 1024, 384, 16, 8, 128),
                                            (200, 256, 768, 6, 4, 128)])
def test_moe_prquant_offline_copy(T, H, I, E, k, tail):
    """PRQuant's offline copy (§4 "Activation tail construction"): gate/up
    run over I + tail intermediate columns whose last `tail` are copies of
    columns I - tail .. I - 1, so the FFN itself emits [h, h_tail] and no tail
    copy runs.  Its h codes equal the online copy's bit for bit (the tail
    starts on a 32-block boundary), and the down stage over I + tail matches
    the oracle's residual formula."""
    banner(f"moe prquant offline copy T={T} H={H} I={I} E={E} k={k} tail={tail}")
    d = synth.moe_problem(T, H, I, E, seed=7, device=DEV)
    route, ref_route = _check_route(d["logits"], k)
    P = T * k
    q = gbw.mx_quantize(d["w_gate_up"].reshape(E * 2 * I, H), gbw.FMT_E8M0_B32)
    gc, gs = q.codes.view(E, 2 * I, H // 2), q.scales.view(E, 2 * I, H // 32)
    Wgu = gbw.Weight(gbw.FMT_E8M0_B32, 2 * I, H, gc, gs, n_experts=E)
    oc, os_ = _offline_copy_weight(gc, gs, I, tail)
    Woff = gbw.Weight(gbw.FMT_E8M0_B32, 2 * (I + tail), H, oc, os_, n_experts=E)
    xq = gbw.mx_quantize(d["x"], gbw.FMT_E8M0_B32)
    W2 = (I + tail) // 2
    on_c = torch.empty((P, W2), dtype=torch.uint8, device=DEV)
    on_s = torch.empty((P, (I + tail) // 32), dtype=torch.uint8, device=DEV)
    gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, Wgu, h_codes=on_c, h_scales=on_s, h_tail=tail)
    off_c = torch.empty_like(on_c)
    off_s = torch.empty_like(on_s)
    gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, Woff, h_codes=off_c, h_scales=off_s)
    torch.cuda.synchronize()
    assert torch.equal(off_c, on_c) and torch.equal(off_s, on_s), "offline copy h differs from the online copy"
    Waug, _ = _prquant_weights(d["w_down"], tail)
    y = torch.empty((T, H), dtype=torch.float32, device=DEV)
    gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, gbw.Act(gbw.FMT_E8M0_B32, off_c, off_s), Waug, y=y)
    # the oracle's own chain: Q(x), gate/up, SwiGLU, Q(h), residual down
    ac, as_ = on.quantize_e8m0_b32(d["x"].float().cpu().numpy())
    gq = [on.quantize_e8m0_b32(d["w_gate_up"][e].cpu().numpy()) for e in range(E)]
    g, u = on.moe_gateup(ac, as_, "e8m0_b32", ref_route, [c for c, _ in gq], [s_ for _, s_ in gq])
    h_ref = on.swiglu_bf16(g, u)
    qc, qs = on.quantize_e8m0_b32(oracle.bf16_bits_to_f32(h_ref))
    wd = d["w_down"].cpu().numpy()
    wc, ws, rc, rs = [], [], [], []
    for e in range(E):
        c, s_ = on.quantize_e8m0_b32(wd[e])
        r_c, r_s = on.quantize_e8m0_b32(oracle.residual_weight(wd[e], c, s_, tail))
        wc.append(c); ws.append(s_); rc.append(r_c); rs.append(r_s)
    y_ref = on.moe_down_combine_residual(qc, qs, ref_route, np.array(wc), np.array(ws), np.array(rc), np.array(rs),
                                         tail)
    assert on.last_inexact == 0
    # the down stage on the oracle's h with its tail columns: every token within 1e-3
    hqa = gbw.Act(gbw.FMT_E8M0_B32, torch.from_numpy(np.concatenate([qc, qc[:, (I - tail) // 2:]], 1)).to(DEV),
                  torch.from_numpy(np.concatenate([qs, qs[:, (I - tail) // 32:]], 1)).to(DEV))
    yo = torch.empty((T, H), dtype=torch.float32, device=DEV)
    gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, hqa, Waug, y=yo)
    assert_rows_close(to_np(yo), y_ref, what="offline-copy down on the oracle's h")
    # pipeline: tokens whose h requantized identically within 1e-3
    gcn, gsn = to_np(off_c)[:, :I // 2], to_np(off_s)[:, :I // 32]
    same = (gcn == qc).all(axis=1) & (gsn == qs).all(axis=1)
    pp = ref_route["pair_pos"]
    clean = same[pp].all(axis=1)
    yv = to_np(y).astype(np.float64)
    nrm = np.linalg.norm(y_ref, axis=1)
    err = np.abs(yv - y_ref).max(axis=1)
    assert np.all(err[clean] <= 1e-3 * nrm[clean]), "clean tokens outside 1e-3"
    print(f"[stats] offline copy: tokens with identically requantized h {clean.mean():.1%}", flush=True)
    assert clean.mean() > 0.5
