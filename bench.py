#!/usr/bin/env python3
"""Throughput of the 4-bit-weight GEMM hot path on one MI355X.

Headline (the JSON line's ``value``): the routed MoE expert FFN in prefill,
T=8192 tokens, hidden 4096, intermediate 1536, 128 experts, top-8, weights in
the VQ->MX format (8-bit indices into a 256-entry table of four E2M1 codes per
64x64 QBlock plus E8M0 prescales), activations MXFP4 online.  One step is one
pass of the whole path over that batch: routing, activation quantization, the
grouped gate/up GEMM with fused SwiGLU and requantization, the grouped down
GEMM with the weighted combine.  Inputs are resident in HBM before timing.

Also measured in the same run (the ``decode`` and ``extra`` objects):
  * codebook/LUT weight-only GEMM, K = N = 4096, M in {1, 8, 64}, weight GB/s;
  * MXFP4 down projection with the PRQuant tail residual, M=128, K=9728,
    N=2560, tail 256, weight GB/s;
  * the E4M3-B16 MoE FFN, T=4096, hidden 2048, intermediate 768, 128 experts,
    top-8, TFLOP/s;
  * the single 16x512x512 MXFP4 linear, microseconds per call.
Decode-shaped calls rotate over enough weight replicas that every call reads
its weights from HBM rather than the 256 MB Infinity Cache, and are captured
in one HIP graph so host launch overhead stays out of the measurement.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--headline-only]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized GEMM TFLOP/s (prefill) + weight GB/s (decode) at 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MXFP4_PEAK_TFLOPS = 10100.0    # dense MFMA, fp4 / fp6
F16_PEAK_TFLOPS = 2500.0       # dense MFMA, fp16 / bf16
# HBM bytes per gate/up launch of the headline workload: rocprofv3 FETCH_SIZE and
# WRITE_SIZE of k_moe_fp4<VQ,256>, scaled by a 1 GiB copy (factors 2.0 and 1.0);
# profiles/k_moe_fp4_vq_prefill_T8192_H4096_I1536_E128_top8.md.  Must be
# measured again (or set to None) whenever that kernel changes.
GATEUP_HBM_BYTES = 431005.2 * 2 * 1024 + 62916.5 * 1024   # FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 (calibrated KiB per launch)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only copy BYTES between two device buffers 3 times (scale for the HBM byte counters)")
    return ap.parse_args()


def copy_calibration(torch, nbytes):
    """A plain device copy of known size: what FETCH_SIZE / WRITE_SIZE read for
    it converts those counters into bytes for the other kernels."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "calls": 3}), flush=True)


# ---------------------------------------------------------------------------
# headline: VQ->MX MoE prefill
# ---------------------------------------------------------------------------

VQ_SCALE_FMT = {"prescale": "FMT_VQ4_E8M0", "postscale": "FMT_VQ4_POST", "prescale_plus": "FMT_VQ4_PLUS"}


def moe_vq_prefill(gbw, synth, torch, steps, warmup, scales="prescale"):
    """The VQ->MX MoE FFN; ``scales`` picks the MXCode block-scale layout
    (PreScale for the headline, PostScale / PreScale+ as extra lines)."""
    T, H, I, E, K = 8192, 4096, 1536, 128, 8
    dev = "cuda"
    d = synth.moe_vq_problem(T, H, I, E, seed=0, device=dev, scales=scales)
    fmt = getattr(gbw, VQ_SCALE_FMT[scales])

    def weight(v, N, Kd):
        return gbw.Weight(fmt, N, Kd, v["idx"], v["scales"], v["codebook"], n_experts=E,
                          scale_codebook=v.get("scale_codebook"))
    Wgu = weight(d["gate_up"], 2 * I, H)
    Wd = weight(d["down"], H, I)
    P = T * K
    route = dict(topk_ids=torch.empty((T, K), dtype=torch.int32, device=dev),
                 topk_w=torch.empty((T, K), dtype=torch.float32, device=dev),
                 expert_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                 pair_token=torch.empty(P, dtype=torch.int32, device=dev),
                 pair_pos=torch.empty((T, K), dtype=torch.int32, device=dev))
    rws = torch.empty(gbw.workspace_size(gbw.OP_MOE_ROUTE, T, E), dtype=torch.uint8, device=dev)
    xq = gbw.Act(gbw.FMT_E8M0_B32, torch.empty((T, H // 2), dtype=torch.uint8, device=dev),
                 torch.empty((T, H // 32), dtype=torch.uint8, device=dev))
    hc = torch.empty((P, I // 2), dtype=torch.uint8, device=dev)
    hs = torch.empty((P, I // 32), dtype=torch.uint8, device=dev)
    hq = gbw.Act(gbw.FMT_E8M0_B32, hc, hs)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(marks=None):
        gbw.moe_route(d["logits"], K, out=route, ws=rws)
        gbw.mx_quantize(d["x"], gbw.FMT_E8M0_B32, out=xq)
        if marks is not None:
            marks[0].record()
        gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, Wgu, h_codes=hc, h_scales=hs)
        if marks is not None:
            marks[1].record()
        gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, hq, Wd, y=y)
        if marks is not None:
            marks[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    marks = [[ev(), ev(), ev()] for _ in range(steps)]
    t0, t1 = ev(), ev()
    torch.cuda.synchronize()
    t0.record()
    for s in range(steps):
        step(marks[s])
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    gu_ms = sum(m[0].elapsed_time(m[1]) for m in marks) / steps
    dn_ms = sum(m[1].elapsed_time(m[2]) for m in marks) / steps
    flops_gu = 2.0 * P * (2 * I) * H
    flops_dn = 2.0 * P * H * I
    weight_bytes = sum(t.numel() * t.element_size() for t in
                       (Wgu.codes, Wgu.scales, Wgu.codebook, Wd.codes, Wd.scales, Wd.codebook)
                       + tuple(w.scale_codebook for w in (Wgu, Wd) if w.scale_codebook is not None))
    return dict(ms_step=ms_step, gu_ms=gu_ms, dn_ms=dn_ms, flops=flops_gu + flops_dn, flops_gu=flops_gu,
                flops_dn=flops_dn, weight_bytes=weight_bytes, data=d, route=route, T=T, H=H, I=I, E=E, K=K)


CPU_SAMPLE_EXPERTS = 32   # about 10-15 s of oracle work on the host cores


def moe_vq_scale_layouts(gbw, synth, torch, steps=5, warmup=2):
    """The headline FFN with MXCode PostScale and PreScale+ weight scales:
    same shapes and kernels, fewer stored scale bytes."""
    out = {}
    for scales in ("postscale", "prescale_plus"):
        r = moe_vq_prefill(gbw, synth, torch, steps, warmup, scales=scales)
        n_w = 3 * r["E"] * r["H"] * r["I"]
        out[scales] = {"ms_per_step": r["ms_step"], "gate_up_ms": r["gu_ms"], "down_combine_ms": r["dn_ms"],
                       "tflops": r["flops"] / (r["ms_step"] * 1e-3) / 1e12,
                       "weight_bytes": r["weight_bytes"], "bits_per_weight": 8.0 * r["weight_bytes"] / n_w}
        r.clear()
        torch.cuda.empty_cache()
    return out


def cpu_baseline(oracle, synth, torch, np, res):
    """The oracle on a bounded sample of the headline workload: every pair
    routed to the first CPU_SAMPLE_EXPERTS experts through gate/up, SwiGLU,
    requantization and the down GEMM (float64 numpy on the host)."""
    import threadpoolctl
    d = res["data"]
    T, H, I = res["T"], res["H"], res["I"]
    route = {k: v.cpu().numpy() for k, v in res["route"].items()}
    off = route["expert_offsets"]
    experts = list(range(CPU_SAMPLE_EXPERTS))
    pairs = np.concatenate([np.arange(off[e], off[e + 1]) for e in experts])
    x = d["x"].float().cpu().numpy()
    gcpu = {k: v[experts].cpu() for k, v in d["gate_up"].items()}
    dcpu = {k: v[experts].cpu() for k, v in d["down"].items()}
    t0 = time.perf_counter()
    ac, as_ = oracle.quantize_e8m0_b32(x)
    n_out = 0
    for i, e in enumerate(experts):
        cb = gcpu["codebook"][i].numpy().view(np.uint16)
        wgu_codes = oracle.vq_decode_codes(gcpu["idx"][i].numpy(), cb)
        sel = np.arange(off[e], off[e + 1])
        toks = route["pair_token"][sel]
        g = oracle.mx_gemm(ac[toks], as_[toks], wgu_codes[:I], gcpu["scales"][i].numpy()[:I])
        u = oracle.mx_gemm(ac[toks], as_[toks], wgu_codes[I:], gcpu["scales"][i].numpy()[I:])
        h = oracle.bf16_bits_to_f32(oracle.swiglu_bf16(g, u))
        hc, hs = oracle.quantize_e8m0_b32(h)
        wd_codes = oracle.vq_decode_codes(dcpu["idx"][i].numpy(), dcpu["codebook"][i].numpy().view(np.uint16))
        out = oracle.mx_gemm(hc, hs, wd_codes, dcpu["scales"][i].numpy())
        n_out += out.shape[0]
    secs = time.perf_counter() - t0
    flops = 2.0 * len(pairs) * 3 * I * H
    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] + [1])
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"all {len(pairs)} pairs routed to experts 0-{experts[-1]} of the headline batch "
                      f"(quantize x, gate/up, SwiGLU, requantize, down; no combine), {secs:.1f} s"}


# ---------------------------------------------------------------------------
# decode-shaped GEMMs (weights streamed from HBM)
# ---------------------------------------------------------------------------

def _graph_time(torch, fn, calls, reps=10):
    fn()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * calls)  # us per call


def lut_decode(gbw, synth, torch, M):
    N = K = 4096
    w_bytes = N * K // 2 + N * (K // 128) * 16 * 2
    R = max(2, int(2 * 256e6 // w_bytes) + 1)
    base = synth.lut_problem(M, N=N, K=K, group=128, seed=0, device="cuda", iters=10)
    reps = [(base["idx"], base["centroids"])]
    for r in range(1, R):  # replicas: same statistics, distinct memory
        g = torch.Generator(device="cuda")
        g.manual_seed(r)
        perm = torch.randperm(N, generator=g, device="cuda")
        reps.append((base["idx"][perm].contiguous(), base["centroids"][perm].contiguous()))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, gbw.workspace_size(gbw.OP_LUT_GEMM, M, N, K)), dtype=torch.uint8, device="cuda")

    def fn():
        for idx, cent in reps:
            gbw.lut_gemm(base["x"], idx, cent, 128, out=y, ws=ws)
    us = _graph_time(torch, fn, len(reps))
    return {"M": M, "us_per_call": us, "weight_bytes": w_bytes, "GB_s": w_bytes / us / 1e3,
            "frac_hbm": w_bytes / us / 1e3 / HBM_PEAK_GBS, "replicas": len(reps)}


def tail_decode(gbw, synth, torch):
    M, N, K, tail = 128, 2560, 9728, 256
    p = synth.tail_residual_problem(M, N, K, tail=tail, seed=0, device="cuda")
    a = gbw.mx_quantize(p["x"], gbw.FMT_E8M0_B32)
    w_bytes = N * K // 2 + N * K // 32 + N * tail // 2 + N * tail // 32
    R = int(2 * 256e6 // w_bytes) + 1
    reps = []
    for r in range(R):
        w = p["w"] if r == 0 else synth.normal((N, K), 0.02, r, "bench.tail.w", "cuda")
        wq = gbw.mx_quantize(w, gbw.FMT_E8M0_B32)
        rq = gbw.mx_quantize(gbw.mx_residual(w, wq.codes, wq.scales, tail), gbw.FMT_E8M0_B32)
        reps.append((gbw.weight_from_act(wq), gbw.weight_from_act(rq)))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, gbw.workspace_size(gbw.OP_MX_GEMM, M, N, K + tail)), dtype=torch.uint8, device="cuda")

    def fn():
        for w, r in reps:
            gbw.residual_tail_gemm(a, w, r, tail, out=y, ws=ws)
    us = _graph_time(torch, fn, len(reps))
    flops = 2.0 * M * N * (K + tail)
    return {"M": M, "N": N, "K": K, "tail": tail, "us_per_call": us, "weight_bytes": w_bytes,
            "GB_s": w_bytes / us / 1e3, "frac_hbm": w_bytes / us / 1e3 / HBM_PEAK_GBS,
            "TFLOP_s": flops / us / 1e6, "replicas": R}


def moe_mxfp4_prquant(gbw, synth, torch, steps=5, tail=128):
    """MXFP4 experts at the E4M3-B16 workload's shape (T=4096, H=2048, I=768,
    128 experts, top-8), plain and with PRQuant's tail residual on the
    down-projections (gate/up appends the tail copy of h; the down stage runs
    over I + tail against [W_down | R]).  Overhead of the residual in %."""
    T, H, I, E, K = 4096, 2048, 768, 128, 8
    d = synth.moe_problem(T, H, I, E, seed=0, device="cuda")
    q = gbw.mx_quantize(d["w_gate_up"].reshape(E * 2 * I, H), gbw.FMT_E8M0_B32)
    Wgu = gbw.Weight(gbw.FMT_E8M0_B32, 2 * I, H, q.codes.view(E, 2 * I, H // 2), q.scales.view(E, 2 * I, H // 32),
                     n_experts=E)
    wd = d["w_down"]
    qc = torch.empty((E, H, (I + tail) // 2), dtype=torch.uint8, device="cuda")
    qs = torch.empty((E, H, (I + tail) // 32), dtype=torch.uint8, device="cuda")
    for e in range(E):
        wq = gbw.mx_quantize(wd[e].contiguous(), gbw.FMT_E8M0_B32)
        rq = gbw.mx_quantize(gbw.mx_residual(wd[e].contiguous(), wq.codes, wq.scales, tail), gbw.FMT_E8M0_B32)
        qc[e] = torch.cat([wq.codes, rq.codes], dim=1)
        qs[e] = torch.cat([wq.scales, rq.scales], dim=1)
    Wd = {0: gbw.Weight(gbw.FMT_E8M0_B32, H, I, qc[:, :, :I // 2].contiguous(), qs[:, :, :I // 32].contiguous(),
                        n_experts=E),
          tail: gbw.Weight(gbw.FMT_E8M0_B32, H, I + tail, qc, qs, n_experts=E)}
    del d["w_gate_up"], d["w_down"]
    P = T * K
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    res = {"T": T, "hidden": H, "intermediate": I, "experts": E, "topk": K, "tail": tail}
    for tl in (0, tail):
        hc = torch.empty((P, (I + tl) // 2), dtype=torch.uint8, device="cuda")
        hs = torch.empty((P, (I + tl) // 32), dtype=torch.uint8, device="cuda")

        def step(tl=tl, hc=hc, hs=hs):
            route = gbw.moe_route(d["logits"], K)
            xq = gbw.mx_quantize(d["x"], gbw.FMT_E8M0_B32)
            gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, Wgu, h_codes=hc, h_scales=hs, h_tail=tl)
            gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, gbw.Act(gbw.FMT_E8M0_B32, hc, hs), Wd[tl], y=y)
        step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        res["ms_per_step_tail%d" % tl] = e0.elapsed_time(e1) / steps
    res["overhead_pct"] = 100.0 * (res["ms_per_step_tail%d" % tail] / res["ms_per_step_tail0"] - 1.0)
    res["added_down_flop_pct"] = 100.0 * tail / I
    return res


def quantize_rate(gbw, synth, torch):
    """Online activation quantization (E8M0-B32) at the headline activation
    shape, plain and with the block Hadamard rotation, over four distinct
    64 MB inputs so every call reads its input from HBM."""
    rows, K = 8192, 4096
    xs = [synth.normal((rows, K), 1.0, 40 + r, "bench.q.x", "cuda").to(torch.bfloat16) for r in range(4)]
    out = gbw.Act(gbw.FMT_E8M0_B32, torch.empty((rows, K // 2), dtype=torch.uint8, device="cuda"),
                  torch.empty((rows, K // 32), dtype=torch.uint8, device="cuda"))
    nbytes = rows * K * 2 + rows * K // 2 + rows * K // 32
    res = {"rows": rows, "K": K, "dtype": "bf16", "bytes_per_call": nbytes}
    for name, rot in (("plain", False), ("block_hadamard", True)):
        def fn(rot=rot):
            for x in xs:
                gbw.mx_quantize(x, gbw.FMT_E8M0_B32, out=out, rotate=rot)
        us = _graph_time(torch, fn, len(xs))
        res[name] = {"us_per_call": us, "GB_s": nbytes / us / 1e3, "frac_hbm": nbytes / us / 1e3 / HBM_PEAK_GBS}
    return res


def dense_small(gbw, synth, torch):
    d = synth.dense_linear(16, 512, 512, seed=0, device="cuda")
    a = gbw.mx_quantize(d["x"], gbw.FMT_E8M0_B32)
    w = gbw.weight_from_act(gbw.mx_quantize(d["w"], gbw.FMT_E8M0_B32))
    y = torch.empty((16, 512), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, gbw.workspace_size(gbw.OP_MX_GEMM, 16, 512, 512)), dtype=torch.uint8, device="cuda")

    def fn():
        for _ in range(50):
            gbw.mx_gemm(a, w, out=y, ws=ws)
    return {"M": 16, "N": 512, "K": 512, "us_per_call": _graph_time(torch, fn, 50)}


def moe_e4m3(gbw, synth, torch, steps=5, fmt=None):
    """The tensor-scaled MoE workload (E4M3-B16 by default; E5M3-B16 with
    fmt=gbw.FMT_E5M3_B16, decoded to bf16 instead of fp16)."""
    fmt = gbw.FMT_E4M3_B16 if fmt is None else fmt
    T, H, I, E, K = 4096, 2048, 768, 128, 8
    d = synth.moe_problem(T, H, I, E, seed=0, device="cuda")
    dev = "cuda"
    gc = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=dev)
    gs = torch.empty((E, 2 * I, H // 16), dtype=torch.uint8, device=dev)
    gt = torch.empty((E, 2), dtype=torch.float32, device=dev)
    dc = torch.empty((E, H, I // 2), dtype=torch.uint8, device=dev)
    ds = torch.empty((E, H, I // 16), dtype=torch.uint8, device=dev)
    dt = torch.empty((E, 1), dtype=torch.float32, device=dev)
    for e in range(E):
        for half in range(2):
            rows = slice(half * I, (half + 1) * I)
            gbw.mx_quantize(d["w_gate_up"][e, rows].contiguous(), fmt,
                            out=gbw.Act(fmt, gc[e, rows], gs[e, rows]), tensor_scale=gt[e, half:half + 1], dynamic=True)
        gbw.mx_quantize(d["w_down"][e].contiguous(), fmt, out=gbw.Act(fmt, dc[e], ds[e]),
                        tensor_scale=dt[e], dynamic=True)
    del d["w_gate_up"], d["w_down"]
    Wgu = gbw.Weight(fmt, 2 * I, H, gc, gs, None, gt, 2, E)
    Wd = gbw.Weight(fmt, H, I, dc, ds, None, dt, 1, E)
    P = T * K
    hb = torch.empty((P, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)

    def step():
        route = gbw.moe_route(d["logits"], K)
        xq = gbw.mx_quantize(d["x"], fmt)
        gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, Wgu, h_bf16=hb)
        hq = gbw.mx_quantize(hb, fmt)
        gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, hq, Wd, y=y)
    step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 2.0 * P * 3 * H * I
    return {"T": T, "hidden": H, "intermediate": I, "experts": E, "topk": K, "ms_per_step": ms,
            "TFLOP_s": flops / ms / 1e9,
            ("frac_bf16_mfma" if fmt == gbw.FMT_E5M3_B16 else "frac_f16_mfma"): flops / ms / 1e9 / F16_PEAK_TFLOPS,
            "frac_mxfp4_mfma": flops / ms / 1e9 / MXFP4_PEAK_TFLOPS}


def moe_vq_b16(gbw, synth, torch, steps=5):
    """The E4M3-B16 MoE workload with VQ weights (MXCode PreScale, PostScale,
    PreScale+ with E4M3 block scales per 16): activations E4M3-B16 online."""
    T, H, I, E, K = 4096, 2048, 768, 128, 8
    fmts = {"prescale": gbw.FMT_VQ4_E4M3, "postscale": gbw.FMT_VQ4_E4M3_POST,
            "prescale_plus": gbw.FMT_VQ4_E4M3_PLUS}
    out = {"T": T, "hidden": H, "intermediate": I, "experts": E, "topk": K}
    for scales, fmt in fmts.items():
        d = synth.moe_vq_problem(T, H, I, E, seed=0, device="cuda", scales=scales, scale_fmt="e4m3")

        def weight(v, N, Kd, nts):
            return gbw.Weight(fmt, N, Kd, v["idx"], v["scales"], v["codebook"], v["tensor_scale"], nts, E,
                              scale_codebook=v.get("scale_codebook"))
        Wgu, Wd = weight(d["gate_up"], 2 * I, H, 2), weight(d["down"], H, I, 1)
        P = T * K
        hb = torch.empty((P, I), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((T, H), dtype=torch.float32, device="cuda")

        def step():
            route = gbw.moe_route(d["logits"], K)
            xq = gbw.mx_quantize(d["x"], gbw.FMT_E4M3_B16)
            gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, Wgu, h_bf16=hb)
            hq = gbw.mx_quantize(hb, gbw.FMT_E4M3_B16)
            gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, hq, Wd, y=y)
        step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        flops = 2.0 * P * 3 * H * I
        wbytes = sum(t.numel() * t.element_size() for w in (Wgu, Wd)
                     for t in (w.codes, w.scales, w.codebook, w.scale_codebook) if t is not None)
        out[scales] = {"ms_per_step": ms, "TFLOP_s": flops / ms / 1e9,
                       "frac_f16_mfma": flops / ms / 1e9 / F16_PEAK_TFLOPS,
                       "bits_per_weight": 8.0 * wbytes / (3 * E * H * I)}
        del d, Wgu, Wd
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import gemm_bit_weight_amd as gbw
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
        return

    log("headline: VQ->MX MoE prefill T=8192 H=4096 I=1536 E=128 top-8")
    res = moe_vq_prefill(gbw, synth, torch, args.steps, args.warmup)
    value = res["flops"] / (res["ms_step"] * 1e-3) / 1e12
    gu_tflops = res["flops_gu"] / (res["gu_ms"] * 1e-3) / 1e12
    log(f"step {res['ms_step']:.3f} ms -> {value:.1f} TFLOP/s; gate/up {res['gu_ms']:.3f} ms "
        f"({gu_tflops:.1f} TFLOP/s), down {res['dn_ms']:.3f} ms")
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "moe_ffn_prefill_vq_mx", "tokens": res["T"], "hidden": res["H"],
                   "intermediate": res["I"], "experts": res["E"], "topk": res["K"],
                   "weights": "VQ d=4, 256 E2M1 keys per 64x64 QBlock, 8-bit indices, E8M0-B32 prescale",
                   "activations": "E8M0-B32 FP4, quantized online", "routed_flops": res["flops"]},
        "roofline": {"kernel": "k_moe_fp4<VQ> gate/up (fused SwiGLU + requantization)", "bound": "mfma",
                     "achieved": gu_tflops, "peak": MXFP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": gu_tflops / MXFP4_PEAK_TFLOPS, "traffic": GATEUP_HBM_BYTES,
                     "traffic_unit": "bytes per launch (HBM, calibrated counters)",
                     "flops_per_launch": res["flops_gu"], "avg_launch_ms": res["gu_ms"]},
        "stages_ms": {"gate_up": res["gu_ms"], "down_combine": res["dn_ms"],
                      "route_quant_other": res["ms_step"] - res["gu_ms"] - res["dn_ms"]},
    }
    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline (oracle, bounded sample)")
        out["cpu_baseline"] = cpu_baseline(oracle, synth, torch, np, res)
    else:
        out["cpu_baseline"] = None
    res.clear()
    torch.cuda.empty_cache()
    if not args.headline_only:
        log("decode: LUT GEMM M=1/8/64, tail-residual MXFP4 GEMM")
        out["decode"] = {"lut_gemm": [lut_decode(gbw, synth, torch, M) for M in (1, 8, 64)],
                         "residual_tail_gemm": tail_decode(gbw, synth, torch)}
        torch.cuda.empty_cache()
        log("extra: E4M3-B16 MoE, 16x512x512 linear")
        out["extra"] = {"moe_e4m3_b16": moe_e4m3(gbw, synth, torch),
                        "moe_e5m3_b16": moe_e4m3(gbw, synth, torch, fmt=gbw.FMT_E5M3_B16),
                        "mx_gemm_16x512x512": dense_small(gbw, synth, torch),
                        "quantize_e8m0_8192x4096": quantize_rate(gbw, synth, torch),
                        "moe_mxfp4_prquant_down": moe_mxfp4_prquant(gbw, synth, torch),
                        "moe_vq_scale_layouts": moe_vq_scale_layouts(gbw, synth, torch),
                        "moe_vq_e4m3_b16": moe_vq_b16(gbw, synth, torch)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
