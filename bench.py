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
HOT_CALLS = 16                 # calls per graph for the cache-resident decode figures
F16_PEAK_TFLOPS = 2500.0       # dense MFMA, fp16 / bf16
# HBM bytes per gate/up launch of the headline workload: rocprofv3 FETCH_SIZE and
# WRITE_SIZE of k_moe_fp4<VQ,256>, scaled by a 1 GiB copy (factors 2.0 and 1.0);
# profiles/k_moe_fp4_vq_prefill_T8192_H4096_I1536_E128_top8.md.  Must be
# measured again (or set to None) whenever that kernel changes.
GATEUP_HBM_BYTES = 434482.4 * 2 * 1024 + 60940.7 * 1024   # FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 (calibrated KiB per launch)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--part", choices=("decode", "e4m3", "mfma", "tiletrace"), default=None,
                    help="profiling aid: run only the decode GEMMs, only the E4M3-B16 MoE or only the MFMA rate "
                         "probe and print their measurements (not the benchmark line); tiletrace: the per-tile "
                         "timeline of one headline gate/up and one down launch, with GBW_LIBRARY naming "
                         "libgbw_tiletrace.so (python gemm_bit_weight_amd/build.py --tile-trace)")
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
    # the down stage's workspace (slot buffer), allocated and zeroed once as
    # a caller would; every call overwrites every slot
    wsd = torch.zeros(gbw.workspace_size(gbw.OP_MOE_GEMM, P, H, 0), dtype=torch.uint8, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(marks=None):
        gbw.moe_route(d["logits"], K, out=route, ws=rws)
        gbw.mx_quantize(d["x"], gbw.FMT_E8M0_B32, out=xq)
        if marks is not None:
            marks[0].record()
        gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, Wgu, h_codes=hc, h_scales=hs)
        if marks is not None:
            marks[1].record()
        gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, hq, Wd, y=y, ws=wsd)
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


def tile_timeline(gbw, synth, torch, np):
    """Per-tile timeline of one gate/up and one down launch of the headline
    MoE step, from the wall-clock stamps of the tile-trace build (100 MHz):
    median lookup / prologue / K-loop / epilogue times of full tiles and of
    tiles holding 1-32 pairs, the CUs' finish times, the gaps between a CU's
    tiles and how many tiles are in their epilogue at once."""
    import ctypes
    lib = gbw._lib
    if not hasattr(lib, "gbw_tile_trace"):
        raise SystemExit("--part tiletrace needs GBW_LIBRARY=<repo>/gemm_bit_weight_amd/libgbw_tiletrace.so "
                         "(built by: python gemm_bit_weight_amd/build.py --tile-trace)")
    lib.gbw_tile_trace.restype = ctypes.c_int
    lib.gbw_tile_trace.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    res = moe_vq_prefill(gbw, synth, torch, steps=2, warmup=2)
    route, d, T, H, I, E, K = res["route"], res["data"], res["T"], res["H"], res["I"], res["E"], res["K"]
    fmt = getattr(gbw, VQ_SCALE_FMT["prescale"])
    W = lambda v, N, Kd: gbw.Weight(fmt, N, Kd, v["idx"], v["scales"], v["codebook"], n_experts=E)  # noqa: E731
    Wgu, Wd = W(d["gate_up"], 2 * I, H), W(d["down"], H, I)
    P = T * K
    xq = gbw.mx_quantize(d["x"], gbw.FMT_E8M0_B32)
    hc = torch.empty((P, I // 2), dtype=torch.uint8, device="cuda")
    hs = torch.empty((P, I // 32), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    wsd = torch.zeros(gbw.workspace_size(gbw.OP_MOE_GEMM, P, H, 0), dtype=torch.uint8, device="cuda")
    stages = {"gate_up": lambda: gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, Wgu, h_codes=hc, h_scales=hs),
              "down": lambda: gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, gbw.Act(gbw.FMT_E8M0_B32, hc, hs),
                                                   Wd, y=y, ws=wsd)}
    for fn in stages.values():
        fn()
    torch.cuda.synchronize()
    buf = np.zeros(16384 * 8, dtype=np.uint64)
    us = lambda t: t * 10 / 1000  # noqa: E731  (100 MHz ticks -> us)
    out = {}
    for name, fn in stages.items():
        assert lib.gbw_tile_trace(None, 0, 1) == 0
        torch.cuda.synchronize()
        fn()
        torch.cuda.synchronize()
        assert lib.gbw_tile_trace(buf.ctypes.data, buf.nbytes, 0) == 0
        a = buf.reshape(16384, 8).astype(np.int64)
        v = a[a[:, 1] > 0]
        t0, t1, t2, t3, t4, cu = (v[:, i] for i in range(6))
        rows = v[:, 6] & 0xFFFF
        base = t0.min()

        def phases(m):
            med = lambda x: float(us(np.median(x[m])))  # noqa: E731
            return {"tiles": int(m.sum()), "lookup_us": med(t1 - t0), "prologue_us": med(t2 - t1),
                    "kloop_us": med(t3 - t2), "epilogue_us": med(t4 - t3), "tile_us": med(t4 - t0)}
        ends, gaps = [], []
        for c in np.unique(cu):
            m = cu == c
            o = np.argsort(t0[m])
            ends.append(t4[m].max())
            gaps.extend((t0[m][o][1:] - t4[m][o][:-1]).tolist())
        ends = us(np.array(ends) - base)
        e3, e4 = us(t3 - base), us(t4 - base)
        span = float(us(t4.max() - base))
        inepi = np.array([((e3 <= g) & (e4 > g)).sum() for g in np.arange(0.0, span, 1.0)])
        out[name] = {"span_us": span, "full_tiles": phases(rows == 256), "tiles_1_32_pairs": phases(rows <= 32),
                     "cu_finish_us": {"min": float(ends.min()), "median": float(np.median(ends)),
                                      "max": float(ends.max())},
                     "gap_between_tiles_us": {"median": float(us(np.median(gaps))),
                                              "per_cu_total": float(us(np.sum(gaps)) / len(ends))},
                     "tiles_in_epilogue": {"median": float(np.median(inepi)), "p90": float(np.percentile(inepi, 90)),
                                           "max": int(inepi.max())}}
    return out


CPU_SAMPLE_EXPERTS = 24   # about 10-30 s of oracle work on 16 host threads (5 s per 8 experts)


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


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(synth, torch, np, res):
    """The C++ oracle (double, compensated sums, std::thread) on a bounded
    sample of the headline workload: every pair routed to the first
    CPU_SAMPLE_EXPERTS experts through quantization of x, gate/up, SwiGLU,
    requantization of h, the down GEMM and the weighted accumulation into y."""
    import oracle
    import oracle.native as on
    d = res["data"]
    I = res["I"]
    route = {k: v.cpu().numpy() for k, v in res["route"].items()}
    off = route["expert_offsets"]
    experts = list(range(CPU_SAMPLE_EXPERTS))
    pairs = np.concatenate([np.arange(off[e], off[e + 1]) for e in experts])
    x = d["x"].float().cpu().numpy()
    gcpu = {k: v[experts].cpu().numpy() for k, v in d["gate_up"].items()}
    dcpu = {k: v[experts].cpu().numpy() for k, v in d["down"].items()}
    y = np.zeros((res["T"], res["H"]))
    t0 = time.perf_counter()
    ac, as_ = on.quantize_e8m0_b32(x)
    for i, e in enumerate(experts):
        sel = np.arange(off[e], off[e + 1])
        toks = route["pair_token"][sel]
        wgu_codes = on.vq_decode_codes(gcpu["idx"][i], gcpu["codebook"][i].view(np.uint16))
        g = on.mx_gemm(ac, as_, wgu_codes[:I], gcpu["scales"][i][:I], a_rows=toks)
        u = on.mx_gemm(ac, as_, wgu_codes[I:], gcpu["scales"][i][I:], a_rows=toks)
        hc, hs = on.quantize_e8m0_b32(oracle.bf16_bits_to_f32(on.swiglu_bf16(g, u)))
        wd_codes = on.vq_decode_codes(dcpu["idx"][i], dcpu["codebook"][i].view(np.uint16))
        o = on.mx_gemm(hc, hs, wd_codes, dcpu["scales"][i])
        j = np.argmax(route["topk_ids"][toks] == e, axis=1)
        np.add.at(y, toks, route["topk_w"][toks, j][:, None] * o)
    secs = time.perf_counter() - t0
    flops = 2.0 * len(pairs) * 3 * I * res["H"]
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": on.threads(), "kind": "oracle",
            "cpu_model": _cpu_model(), "nproc": os.cpu_count(),
            "sample": f"all {len(pairs)} pairs routed to experts 0-{experts[-1]} of the headline batch "
                      f"(quantize x, gate/up, SwiGLU, requantize h, down, weighted accumulation), C++ oracle "
                      f"with compensated double sums, {secs:.1f} s"}


def cpu_oracle_1core(synth, torch, np):
    """The C++ oracle on one host thread for the dense and decode-shaped
    configurations (inputs generated first, not timed): the 16x512x512
    MXFP4 linear, the LUT GEMM at M = 1, 8 and 64 (K = N = 4096), and the
    tail-residual GEMM (M = 128, N = 2560, K = 9728 + 256).  The larger
    ones run on a leading slice of their rows and are scaled to the whole
    call; every entry states its sample.  Milliseconds per call."""
    import oracle
    import oracle.native as on
    out = {}

    def timed(fn):  # the timed call alone runs on one thread; the set-up uses them all
        prev = os.environ.get("GBWO_THREADS")
        os.environ["GBWO_THREADS"] = "1"
        try:
            t0 = time.perf_counter()
            fn()
            return (time.perf_counter() - t0) * 1e3
        finally:
            if prev is None:
                os.environ.pop("GBWO_THREADS", None)
            else:
                os.environ["GBWO_THREADS"] = prev

    if True:  # (one block, so the inputs of one configuration are freed before the next)
        d = synth.dense_linear(16, 512, 512, seed=0, device="cpu")
        ac, as_ = on.quantize_e8m0_b32(d["x"].float().numpy())
        wc, ws = on.quantize_e8m0_b32(d["w"].numpy())
        out["mx_gemm_16x512x512"] = {"ms_per_call": timed(lambda: on.mx_gemm(ac, as_, wc, ws)),
                                     "sample": "whole call (activation quantized beforehand)"}
        lut = []
        for M, rows in ((1, 1), (8, 8), (64, 8)):
            w = synth.lut_problem(M, N=4096, K=4096, group=128, seed=0, device="cuda", iters=10)
            xb = w["x"][:rows].cpu().view(torch.int16).numpy().view(np.uint16)
            idx, cent = w["idx"].cpu().numpy(), w["centroids"].cpu().numpy()
            ms = timed(lambda: on.lut_gemm(xb, idx, cent, 128)) * M / rows
            lut.append({"M": M, "ms_per_call": ms,
                        "sample": "whole call" if rows == M else f"{rows} of {M} rows, scaled by {M // rows}"})
        out["lut_gemm"] = lut
        M, N, K, tail, rows = 128, 2560, 9728, 256, 8
        p = synth.tail_residual_problem(M, N, K, tail=tail, seed=0, device="cpu")
        ac, as_ = on.quantize_e8m0_b32(p["x"][:rows].float().numpy())
        wn = p["w"].numpy()
        wc, ws = on.quantize_e8m0_b32(wn)
        rc, rs = on.quantize_e8m0_b32(oracle.residual_weight(wn, wc, ws, tail))
        ms = timed(lambda: on.residual_tail_gemm(ac, as_, wc, ws, rc, rs, tail)) * M / rows
        out["residual_tail_gemm"] = {"ms_per_call": ms, "sample": f"{rows} of {M} rows, scaled by {M // rows}"}
    out["threads"] = 1
    out["cpu_model"] = _cpu_model()
    return out


# ---------------------------------------------------------------------------
# decode-shaped GEMMs (weights streamed from HBM)
# ---------------------------------------------------------------------------

def _graph_time(torch, fn, calls, reps=5, min_calls=200):
    """Microseconds per call of ``fn`` (``calls`` launches) captured in one
    HIP graph: two warm-up replays, then ``reps`` repetitions of enough
    back-to-back replays for at least ``min_calls`` calls, each timed with
    events; the median repetition."""
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
    per = -(-min_calls // calls)  # replays per repetition
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(per):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / (per * calls))
    return sorted(times)[reps // 2]


_FLOOR = None


def _floor_lib():
    """The streaming-read measurement aid built beside the library (a plain
    read of a buffer, and an empty kernel); None if it was not built."""
    global _FLOOR
    if _FLOOR is None:
        import ctypes
        path = os.path.join(ROOT, "gemm_bit_weight_amd", "libgbw_floor.so")
        if not os.path.exists(path):
            return None
        lib = ctypes.CDLL(path)
        lib.gbw_floor_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        lib.gbw_floor_empty.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _FLOOR = lib
    return _FLOOR


def read_floor(torch, regions):
    """Microseconds per call of a plain streaming read of each (address,
    bytes) region in turn, one kernel per region, timed like the kernels
    (one graph, cold caches): what merely reading the same bytes costs."""
    lib = _floor_lib()
    if lib is None:
        return None
    import ctypes
    out = torch.zeros(1024, dtype=torch.int32, device="cuda")

    def fn():
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for addr, nbytes in regions:
            assert lib.gbw_floor_stream_read(ctypes.c_void_p(addr), nbytes, ctypes.c_void_p(out.data_ptr()), st) == 0
    return _graph_time(torch, fn, len(regions))


def empty_kernel_floor(torch, calls=64):
    """Microseconds per launch of an empty one-wave kernel in a graph."""
    lib = _floor_lib()
    if lib is None:
        return None
    import ctypes
    out = torch.zeros(1, dtype=torch.int32, device="cuda")

    def fn():
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for _ in range(calls):
            assert lib.gbw_floor_empty(ctypes.c_void_p(out.data_ptr()), st) == 0
    return _graph_time(torch, fn, calls)


def mfma_rate_probe(torch, iters=4096):
    """TFLOP/s that each MFMA shape sustains with nothing else running (the
    measurement aid's register-only MFMA loop, two waves per SIMD), next to
    the published dense peak of its type: the matrix cores' rate under load,
    clock behaviour included."""
    lib = _floor_lib()
    if lib is None:
        return None
    import ctypes
    lib.gbw_floor_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    blocks = 2 * torch.cuda.get_device_properties(0).multi_processor_count  # 4-wave workgroups
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    shapes = (("fp4_32x32x64", 0, 32 * 32 * 64, MXFP4_PEAK_TFLOPS), ("fp4_16x16x128", 1, 16 * 16 * 128, MXFP4_PEAK_TFLOPS),
              ("fp16_32x32x16", 2, 32 * 32 * 16, F16_PEAK_TFLOPS), ("fp16_16x16x32", 3, 16 * 16 * 32, F16_PEAK_TFLOPS))
    res = {}
    for name, kind, mnk, peak in shapes:
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

        def launch():
            assert lib.gbw_floor_mfma_rate(kind, blocks, iters, ctypes.c_void_p(out.data_ptr()), st) == 0
        launch()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            launch()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 3
        flops = blocks * 4 * iters * 8 * 2 * mnk
        tf = flops / ms / 1e9
        res[name] = {"TFLOP_s": tf, "frac_of_peak": tf / peak, "peak_TFLOP_s": peak, "ms_per_launch": ms}
    return res


def lut_decode(gbw, synth, torch, M):
    N = K = 4096
    w_bytes = N * K // 2 + N * (K // 128) * 16 * 2
    R = max(2, int(2 * 256e6 // w_bytes) + 1)
    base = synth.lut_problem(M, N=N, K=K, group=128, seed=0, device="cuda", iters=10)
    # replicas (same statistics, distinct memory) carved from one allocation,
    # so their placement does not depend on the caching allocator's history
    ib, cb = N * K // 2, N * (K // 128) * 16 * 2
    pool = torch.empty(R * (ib + cb), dtype=torch.uint8, device="cuda")
    reps = []
    for r in range(R):
        g = torch.Generator(device="cuda")
        g.manual_seed(r)
        perm = torch.randperm(N, generator=g, device="cuda") if r else torch.arange(N, device="cuda")
        idx = pool[r * (ib + cb):r * (ib + cb) + ib].view(N, K // 2)
        cent = pool[r * (ib + cb) + ib:(r + 1) * (ib + cb)].view(torch.float16).view(N, K // 128, 16)
        idx.copy_(base["idx"][perm])
        cent.copy_(base["centroids"][perm])
        reps.append((idx, cent))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    # zeroed once: the split-K arrival counters at its front start at zero and every call leaves them so
    ws = torch.zeros(max(1, gbw.workspace_size(gbw.OP_LUT_GEMM, M, N, K)), dtype=torch.uint8, device="cuda")

    def fn():
        for idx, cent in reps:
            gbw.lut_gemm(base["x"], idx, cent, 128, out=y, ws=ws)
    us = _graph_time(torch, fn, len(reps))
    floor = read_floor(torch, [(pool.data_ptr() + r * (ib + cb), ib + cb) for r in range(R)])

    def fn_hot():  # one replica, re-read by every call: its weights stay in the on-chip caches
        for _ in range(HOT_CALLS):
            gbw.lut_gemm(base["x"], reps[0][0], reps[0][1], 128, out=y, ws=ws)
    hot = _graph_time(torch, fn_hot, HOT_CALLS)
    all_bytes = w_bytes + M * K * 2 + M * N * 4  # weights + bf16 x + fp32 y
    return {"M": M, "us_per_call": us, "weight_bytes": w_bytes, "GB_s": w_bytes / us / 1e3,
            "frac_hbm": w_bytes / us / 1e3 / HBM_PEAK_GBS, "frac_hbm_all_bytes": all_bytes / us / 1e3 / HBM_PEAK_GBS,
            "replicas": len(reps), "read_floor_us": floor, "frac_of_read_floor": floor / us if floor else None,
            "hot_us_per_call": hot}


def tail_decode(gbw, synth, torch):
    M, N, K, tail = 128, 2560, 9728, 256
    p = synth.tail_residual_problem(M, N, K, tail=tail, seed=0, device="cuda")
    a = gbw.mx_quantize(p["x"], gbw.FMT_E8M0_B32)
    parts = (N * K // 2, N * K // 32, N * tail // 2, N * tail // 32)  # W codes, scales; R codes, scales
    w_bytes = sum(parts)
    R = int(2 * 256e6 // w_bytes) + 1
    # replicas carved from one allocation (placement independent of the
    # caching allocator's history), each one contiguous region
    stride = (w_bytes + 4095) // 4096 * 4096
    pool = torch.empty(R * stride, dtype=torch.uint8, device="cuda")
    reps = []
    for r in range(R):
        w = p["w"] if r == 0 else synth.normal((N, K), 0.02, r, "bench.tail.w", "cuda")
        wq = gbw.mx_quantize(w, gbw.FMT_E8M0_B32)
        rq = gbw.mx_quantize(gbw.mx_residual(w, wq.codes, wq.scales, tail), gbw.FMT_E8M0_B32)
        views, o = [], r * stride
        for t, nb in zip((wq.codes, wq.scales, rq.codes, rq.scales), parts):
            v = pool[o:o + nb].view(t.shape)
            v.copy_(t)
            views.append(v)
            o += nb
        reps.append((gbw.weight_from_act(gbw.Act(gbw.FMT_E8M0_B32, views[0], views[1])),
                     gbw.weight_from_act(gbw.Act(gbw.FMT_E8M0_B32, views[2], views[3]))))
        del w, wq, rq
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(1, gbw.workspace_size(gbw.OP_MX_GEMM, M, N, K + tail)), dtype=torch.uint8, device="cuda")

    def fn():
        for w, r in reps:
            gbw.residual_tail_gemm(a, w, r, tail, out=y, ws=ws)
    us = _graph_time(torch, fn, len(reps))
    floor = read_floor(torch, [(pool.data_ptr() + r * stride, w_bytes) for r in range(R)])

    def fn_hot():  # one replica, re-read by every call: its weights stay in the on-chip caches
        for _ in range(HOT_CALLS):
            gbw.residual_tail_gemm(a, reps[0][0], reps[0][1], tail, out=y, ws=ws)
    hot = _graph_time(torch, fn_hot, HOT_CALLS)
    flops = 2.0 * M * N * (K + tail)
    all_bytes = w_bytes + M * (K + tail) // 2 + M * (K + tail) // 32 + M * N * 4  # weights + codes/scales + y
    return {"M": M, "N": N, "K": K, "tail": tail, "us_per_call": us, "weight_bytes": w_bytes,
            "GB_s": w_bytes / us / 1e3, "frac_hbm": w_bytes / us / 1e3 / HBM_PEAK_GBS,
            "frac_hbm_all_bytes": all_bytes / us / 1e3 / HBM_PEAK_GBS,
            "TFLOP_s": flops / us / 1e6, "frac_mxfp4_mfma": flops / us / 1e6 / MXFP4_PEAK_TFLOPS, "replicas": R,
            "read_floor_us": floor, "frac_of_read_floor": floor / us if floor else None, "hot_us_per_call": hot}


def moe_mxfp4_prquant(gbw, synth, torch, steps=5, tail=128):
    """MXFP4 experts at the E4M3-B16 workload's shape (T=4096, H=2048, I=768,
    128 experts, top-8): plain, with PRQuant's tail residual on the
    down-projections through the online tail copy (gate/up appends the copy
    of h's last `tail` columns), and through the offline copy (gate/up
    weights with their last `tail` rows duplicated, so the FFN itself emits
    I + tail columns); the down stage then runs over I + tail against
    [W_down | R].  Overheads in % of the plain step."""
    T, H, I, E, K = 4096, 2048, 768, 128, 8
    d = synth.moe_problem(T, H, I, E, seed=0, device="cuda")
    q = gbw.mx_quantize(d["w_gate_up"].reshape(E * 2 * I, H), gbw.FMT_E8M0_B32)
    gc, gs = q.codes.view(E, 2 * I, H // 2), q.scales.view(E, 2 * I, H // 32)
    Wgu = gbw.Weight(gbw.FMT_E8M0_B32, 2 * I, H, gc, gs, n_experts=E)

    def dup(t):  # gate rows + copies of the last `tail`, then up rows + copies
        return torch.cat([t[:, :I], t[:, I - tail:I], t[:, I:], t[:, 2 * I - tail:]], dim=1).contiguous()
    Woff = gbw.Weight(gbw.FMT_E8M0_B32, 2 * (I + tail), H, dup(gc), dup(gs), n_experts=E)
    wd = d["w_down"]
    qc = torch.empty((E, H, (I + tail) // 2), dtype=torch.uint8, device="cuda")
    qs = torch.empty((E, H, (I + tail) // 32), dtype=torch.uint8, device="cuda")
    for e in range(E):
        wq = gbw.mx_quantize(wd[e].contiguous(), gbw.FMT_E8M0_B32)
        rq = gbw.mx_quantize(gbw.mx_residual(wd[e].contiguous(), wq.codes, wq.scales, tail), gbw.FMT_E8M0_B32)
        qc[e] = torch.cat([wq.codes, rq.codes], dim=1)
        qs[e] = torch.cat([wq.scales, rq.scales], dim=1)
    Wd0 = gbw.Weight(gbw.FMT_E8M0_B32, H, I, qc[:, :, :I // 2].contiguous(), qs[:, :, :I // 32].contiguous(),
                     n_experts=E)
    Wda = gbw.Weight(gbw.FMT_E8M0_B32, H, I + tail, qc, qs, n_experts=E)
    del d["w_gate_up"], d["w_down"]
    P = T * K
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    wsd = torch.zeros(gbw.workspace_size(gbw.OP_MOE_GEMM, P, H, 0), dtype=torch.uint8, device="cuda")
    res = {"T": T, "hidden": H, "intermediate": I, "experts": E, "topk": K, "tail": tail}
    # (name, gate/up weight, h columns, h_tail of the gate/up call, down weight)
    variants = (("tail0", Wgu, I, 0, Wd0), ("tail%d" % tail, Wgu, I + tail, tail, Wda),
                ("offline%d" % tail, Woff, I + tail, 0, Wda))
    for name, wg, hw, ht, wdn in variants:
        hc = torch.empty((P, hw // 2), dtype=torch.uint8, device="cuda")
        hs = torch.empty((P, hw // 32), dtype=torch.uint8, device="cuda")

        def step(wg=wg, ht=ht, wdn=wdn, hc=hc, hs=hs):
            route = gbw.moe_route(d["logits"], K)
            xq = gbw.mx_quantize(d["x"], gbw.FMT_E8M0_B32)
            gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, wg, h_codes=hc, h_scales=hs, h_tail=ht)
            gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, gbw.Act(gbw.FMT_E8M0_B32, hc, hs), wdn, y=y, ws=wsd)
        step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        res["ms_per_step_" + name] = e0.elapsed_time(e1) / steps
    base = res["ms_per_step_tail0"]
    res["overhead_pct"] = 100.0 * (res["ms_per_step_tail%d" % tail] / base - 1.0)
    res["overhead_pct_offline"] = 100.0 * (res["ms_per_step_offline%d" % tail] / base - 1.0)
    res["added_down_flop_pct"] = 100.0 * tail / I
    res["added_gate_up_flop_pct_offline"] = 100.0 * tail / I
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
    ws = torch.zeros(max(1, gbw.workspace_size(gbw.OP_MX_GEMM, 16, 512, 512)), dtype=torch.uint8, device="cuda")

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
    wsd = torch.zeros(gbw.workspace_size(gbw.OP_MOE_GEMM, P, H, 0), dtype=torch.uint8, device=dev)

    def step():
        route = gbw.moe_route(d["logits"], K)
        xq = gbw.mx_quantize(d["x"], fmt)
        gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, Wgu, h_bf16=hb)
        hq = gbw.mx_quantize(hb, fmt)
        gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, hq, Wd, y=y, ws=wsd)
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
        wsd = torch.zeros(gbw.workspace_size(gbw.OP_MOE_GEMM, P, H, 0), dtype=torch.uint8, device="cuda")

        def step():
            route = gbw.moe_route(d["logits"], K)
            xq = gbw.mx_quantize(d["x"], gbw.FMT_E4M3_B16)
            gbw.moe_grouped_gemm(gbw.MOE_GATEUP_SWIGLU, route, xq, Wgu, h_bf16=hb)
            hq = gbw.mx_quantize(hb, gbw.FMT_E4M3_B16)
            gbw.moe_grouped_gemm(gbw.MOE_DOWN_COMBINE, route, hq, Wd, y=y, ws=wsd)
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
        print("bench.py measures one GPU: the library has no multi-GPU path "
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
    if args.part == "decode":
        print(json.dumps({"lut_gemm": [lut_decode(gbw, synth, torch, M) for M in (1, 8, 64)],
                          "residual_tail_gemm": tail_decode(gbw, synth, torch)}), flush=True)
        return
    if args.part == "e4m3":
        print(json.dumps({"moe_e4m3_b16": moe_e4m3(gbw, synth, torch, steps=args.steps)}), flush=True)
        return
    if args.part == "tiletrace":
        print(json.dumps(tile_timeline(gbw, synth, torch, np)), flush=True)
        return
    if args.part == "mfma":
        print(json.dumps({"mfma_rate_probe": mfma_rate_probe(torch)}), flush=True)
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
    # what the FP4 matrix cores sustain on this device with nothing else
    # running (clock under load included), beside the published peak
    probe = mfma_rate_probe(torch)
    if probe:
        ceil = probe["fp4_32x32x64"]["TFLOP_s"]
        out["roofline"]["mfma_only_ceiling"] = ceil
        out["roofline"]["frac_of_mfma_only_ceiling"] = gu_tflops / ceil
        out["roofline"]["mfma_only_ceiling_note"] = ("v_mfma_scale_f32_32x32x64_f8f6f4 in a register-only loop, "
                                                     "two waves per SIMD on every CU")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle, bounded sample)")
        out["cpu_baseline"] = cpu_baseline(synth, torch, np, res)
    else:
        out["cpu_baseline"] = None
    res.clear()
    torch.cuda.empty_cache()
    if not args.headline_only:
        log("decode: LUT GEMM M=1/8/64, tail-residual MXFP4 GEMM")
        out["decode"] = {"lut_gemm": [lut_decode(gbw, synth, torch, M) for M in (1, 8, 64)],
                         "residual_tail_gemm": tail_decode(gbw, synth, torch),
                         "empty_kernel_us": empty_kernel_floor(torch),
                         "read_floor_note": "read_floor_us: a plain streaming read of the same weight bytes, "
                                            "one kernel per call, timed the same way",
                         "hot_note": "hot_us_per_call: one weight replica re-read by every call, so the weights "
                                     "come from the on-chip caches (a cache-resident figure, not an HBM one)"}
        if not args.no_cpu_baseline:
            log("oracle on one host thread: dense and decode-shaped configurations")
            out["decode"]["cpu_oracle_1core"] = cpu_oracle_1core(synth, torch, np)
        torch.cuda.empty_cache()
        log("extra: E4M3-B16 MoE, 16x512x512 linear")
        out["extra"] = {"moe_e4m3_b16": moe_e4m3(gbw, synth, torch),
                        "moe_e5m3_b16": moe_e4m3(gbw, synth, torch, fmt=gbw.FMT_E5M3_B16),
                        "mx_gemm_16x512x512": dense_small(gbw, synth, torch),
                        "quantize_e8m0_8192x4096": quantize_rate(gbw, synth, torch),
                        "moe_mxfp4_prquant_down": moe_mxfp4_prquant(gbw, synth, torch),
                        "moe_vq_scale_layouts": moe_vq_scale_layouts(gbw, synth, torch),
                        "moe_vq_e4m3_b16": moe_vq_b16(gbw, synth, torch),
                        "mfma_rate_probe": probe}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
