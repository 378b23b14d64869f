"""GPU parity: MoE routing and the grouped FP4 expert GEMMs (MXFP4 and
VQ->MX weights) against the oracle, stage by stage.

* routing: expert ids, offsets and pair lists bit-exact; weights to 1e-6.
* gate/up: the GPU's bf16 h against bf16(silu(g)u) of the oracle's exact g, u
  within one bf16 rounding (2^-8 relative) plus the 1e-3 row tolerance; the
  GPU's requantized h bit-exact against the oracle's quantizer applied to the
  GPU's own h (the two sides share data, not code).
* down/combine: y against the oracle (fed the GPU's quantized h, which the
  previous check proved equal to the oracle's quantization) within the 1e-3
  row tolerance, for the atomic and the deterministic combine.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_rows_close, banner, to_np, u16

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
                                   (130, 1000, 16)])
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


def _mx_weights(w_f32):
    """E8M0-B32 quantization of [E][N][K] weights with the library's quantizer."""
    E, N, K = w_f32.shape
    q = gbw.mx_quantize(w_f32.reshape(E * N, K).contiguous(), gbw.FMT_E8M0_B32)
    return gbw.Weight(gbw.FMT_E8M0_B32, N, K, q.codes.view(E, N, K // 2), q.scales.view(E, N, K // 32),
                      n_experts=E)


def _vq_weights(v, N, K):
    E = v["idx"].shape[0]
    return gbw.Weight(gbw.FMT_VQ4_E8M0, N, K, v["idx"].to(DEV), v["scales"].to(DEV), v["codebook"].to(DEV),
                      n_experts=E)


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


def _w_codes_np(W):
    """[E][N][K/2] E2M1 codes + [E][N][K/32] scales of a weight, as numpy."""
    E, N, K = W.n_experts, W.N, W.K
    scales = _LazyExperts((E, N, K // 32), lambda e: to_np(W.scales[e]))
    if W.fmt == gbw.FMT_E8M0_B32:
        return _LazyExperts((E, N, K // 2), lambda e: to_np(W.codes[e])), scales
    return _LazyExperts((E, N, K // 2), lambda e: oracle.vq_decode_codes(
        to_np(W.codes[e]), W.codebook[e].cpu().numpy().view(np.uint16))), scales


def _run_and_check(x, logits, topk, Wgu, Wd, tokens=None, experts=None):
    T, H = x.shape
    I = Wgu.N // 2
    route, ref_route = _check_route(logits, topk)
    P = T * topk
    xq = gbw.mx_quantize(x, gbw.FMT_E8M0_B32)
    hb = torch.empty((P, I), dtype=torch.bfloat16, device=DEV)
    hc = torch.empty((P, I // 2), dtype=torch.uint8, device=DEV)
    hs = torch.empty((P, I // 32), dtype=torch.uint8, device=DEV)
    gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, Wgu, h_bf16=hb, h_codes=hc, h_scales=hs)
    y = torch.empty((T, H), dtype=torch.float32, device=DEV)
    hq = gbw.Act(gbw.FMT_E8M0_B32, hc, hs)
    gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, hq, Wd, y=y)
    yd = torch.empty_like(y)
    gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, hq, Wd, y=yd, flags=gbw.DETERMINISTIC)
    yd2 = torch.empty_like(y)
    gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, hq, Wd, y=yd2, flags=gbw.DETERMINISTIC)
    torch.cuda.synchronize()
    assert torch.equal(yd, yd2), "deterministic combine differs between runs"

    # activation quantization (bit-exact)
    ac, as_ = oracle.quantize_e8m0_b32(x.float().cpu().numpy())
    assert np.array_equal(to_np(xq.codes), ac) and np.array_equal(to_np(xq.scales), as_)
    # gate/up + SwiGLU on the chosen pairs
    off = ref_route["expert_offsets"]
    if experts is None:
        pairs = np.arange(P)
    else:
        pairs = np.concatenate([np.arange(off[e], off[e + 1]) for e in experts])
    gu_c, gu_s = _w_codes_np(Wgu)
    g, u = oracle.moe_gateup(ac, as_, "e8m0_b32", ref_route, gu_c, gu_s, pairs=pairs)
    h_ref = g / (1.0 + np.exp(-g)) * u
    h_gpu = oracle.bf16_bits_to_f32(u16(hb)[pairs]).astype(np.float64)
    err = np.abs(h_gpu - h_ref)
    bound = 2.0 ** -8 * np.abs(h_ref) + 1e-3 * np.linalg.norm(h_ref, axis=1, keepdims=True)
    assert np.all(err <= bound), f"h outside tolerance: worst {np.max(err / bound):.3f}"
    # requantization of the GPU's h: bit-exact
    qc, qs = oracle.quantize_e8m0_b32(h_gpu.astype(np.float32))
    assert np.array_equal(to_np(hc)[pairs], qc) and np.array_equal(to_np(hs)[pairs], qs)
    # down + combine from the GPU's quantized h
    d_c, d_s = _w_codes_np(Wd)
    y_ref = oracle.moe_down_combine(to_np(hc), to_np(hs), "e8m0_b32", ref_route, d_c, d_s, tokens=tokens)
    sel = np.arange(T) if tokens is None else np.asarray(tokens)
    assert_rows_close(to_np(y)[sel], y_ref, what="moe down (atomic)")
    assert_rows_close(to_np(yd)[sel], y_ref, what="moe down (deterministic)")


@pytest.mark.parametrize("T,H,I,E,k", [(300, 512, 256, 8, 2), (97, 256, 128, 5, 3), (64, 1024, 384, 16, 8)])
def test_moe_mxfp4_small(T, H, I, E, k):
    banner(f"moe mxfp4 T={T} H={H} I={I} E={E} k={k}")
    d = synth.moe_problem(T, H, I, E, seed=1, device=DEV)
    Wgu = _mx_weights(d["w_gate_up"])
    Wd = _mx_weights(d["w_down"])
    _run_and_check(d["x"], d["logits"], k, Wgu, Wd)


@pytest.mark.parametrize("T,H,I,E,k", [(300, 512, 256, 8, 2), (513, 256, 384, 3, 2)])
def test_moe_vq_small(T, H, I, E, k):
    banner(f"moe vq T={T} H={H} I={I} E={E} k={k}")
    d = synth.moe_vq_problem(T, H, I, E, seed=2, device="cpu")
    Wgu = _vq_weights(d["gate_up"], 2 * I, H)
    Wd = _vq_weights(d["down"], H, I)
    _run_and_check(d["x"].to(DEV), d["logits"].to(DEV), k, Wgu, Wd)


def test_moe_vq_full_size_sampled():
    """The measured shape: T=8192, H=4096, I=1536, 128 experts, top-8; gate/up
    checked on every pair of two experts, y on a sample of tokens."""
    banner("moe vq full T=8192 H=4096 I=1536 E=128 k=8")
    d = synth.moe_vq_problem(8192, 4096, 1536, 128, seed=0, device=DEV)
    Wgu = _vq_weights(d["gate_up"], 3072, 4096)
    Wd = _vq_weights(d["down"], 4096, 1536)
    _run_and_check(d["x"], d["logits"], 8, Wgu, Wd, tokens=[0, 4097, 8191], experts=[0, 77])
