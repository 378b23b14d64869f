"""Seeded synthetic inputs for the 4-bit-weight GEMM path.

This module is shared by the oracle side (tests, CPU baseline) and the HIP
side (tests, bench).  It holds none of the method's arithmetic: it draws
random tensors, permutes columns, and builds codebook-format weights from
random draws.  Quantization to the block-scaled FP4 formats is never done
here -- each side does it with its own quantizer.

Every tensor is drawn from its own torch.Generator seeded from (seed, name),
so one tensor's recipe does not shift another's.  Values are generated on the
requested device (CPU for the oracle-sized cases, the GPU for large bench
inputs); the oracle always works on a host copy of the very same arrays.

Workload recipes (sizes follow the configurations the library is measured
on; the distributions stand in for trained weights and calibration
activations, which are not available):
  * dense linear: X ~ N(0,1) rounded to bf16, W ~ N(0, 0.02^2) fp32;
  * codebook/LUT weights: W ~ N(0, 0.02^2) with 0.5% of entries x20, one
    16-entry fp16 codebook per (output row, 128-wide K group) from a plain
    1-D Lloyd clustering, 4-bit indices;
  * tail-residual down projection: X ~ N(0,1) with 1% of its channels x50,
    rounded to bf16, W ~ N(0, 0.02^2); the outlier channels are moved to the
    end of K by a stable partition applied to the columns of both;
  * MoE: X ~ N(0,1) bf16, router logits ~ N(0,1) fp32, per-expert
    W_gate, W_up, W_down ~ N(0, 0.02^2) fp32;
  * VQ->MX MoE weights: per QBlock (64x64 unless stated) a 256-entry table
    of 4-element E2M1 keys, 8-bit indices, and E8M0 scales stored per 32
    along K (PreScale), per QBlock table (PostScale) or as 8-vectors of
    scales quantized against a 256-entry table per matrix (PreScale+) --
    drawn directly in that format (codebook learning is offline and out of
    scope).
"""

import zlib

import torch

GATE_UP_STACK = "gate rows [0, I), up rows [I, 2I)"


def seed_for(seed, name):
    return (int(seed) * 1_000_003 + zlib.crc32(name.encode())) & 0x7FFF_FFFF_FFFF


def _gen(seed, name, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(seed, name))
    return g


def normal(shape, std, seed, name, device="cpu", dtype=torch.float32):
    g = _gen(seed, name, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(dtype)


def uniform(shape, seed, name, device="cpu"):
    g = _gen(seed, name, device)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32)


# ----------------------------------------------------------------------------
# Dense linear (block-scaled FP4 weights are quantized by each side)
# ----------------------------------------------------------------------------

def dense_linear(M, N, K, seed=0, device="cpu"):
    """X bf16 [M][K] ~ N(0,1); W fp32 [N][K] ~ N(0, 0.02^2)."""
    x = normal((M, K), 1.0, seed, "dense.x", device).to(torch.bfloat16)
    w = normal((N, K), 0.02, seed, "dense.w", device)
    return dict(x=x, w=w)


def random_codes(rows, K, seed, name, device="cpu"):
    """Packed E2M1 codes [rows][K/2]: every byte uniform over 0 .. 255."""
    g = _gen(seed, name, device)
    return torch.randint(0, 256, (rows, K // 2), generator=g, device=device, dtype=torch.uint8)


def paired_scale_codes(M, N, K, seed, name, device="cpu", block=32):
    """E8M0 block scale codes over 1 .. 253 for an [M][K] activation and an
    [N][K] weight: per K block a base b drawn from 1 .. 119, activation codes
    b + (0 .. 7) and weight codes 254 - b - (0 .. 7), so a low activation scale
    meets a high weight scale in every block and each product of two scales
    stays within 2^-7 .. 2^7."""
    nb = K // block
    base = 1 + (uniform((nb,), seed, f"{name}.base", device) * 119).to(torch.int32).clamp(max=118)
    da = (uniform((M, 1), seed, f"{name}.da", device) * 8).to(torch.int32).clamp(max=7)
    dw = (uniform((N, 1), seed, f"{name}.dw", device) * 8).to(torch.int32).clamp(max=7)
    return (base[None, :] + da).to(torch.uint8), (254 - base[None, :] - dw).to(torch.uint8)


# ----------------------------------------------------------------------------
# Tail-residual down projection
# ----------------------------------------------------------------------------

def tail_residual_problem(M, N, K, tail=256, outlier_frac=0.01, outlier_gain=50.0, seed=0,
                          device="cpu"):
    """Activations with injected outlier channels moved to the end of K.

    Returns x bf16 [M][K] and w fp32 [N][K], both already permuted, plus the
    permutation (new column c holds old channel perm[c]) and the outlier
    channel ids.
    """
    n_out = int(outlier_frac * K)
    assert n_out <= tail <= K
    x = normal((M, K), 1.0, seed, "tail.x", device)
    g = _gen(seed, "tail.channels", "cpu")
    chans = torch.randperm(K, generator=g)[:n_out].sort().values
    if n_out:
        x[:, chans.to(device)] *= outlier_gain
    x = x.to(torch.bfloat16)
    w = normal((N, K), 0.02, seed, "tail.w", device)
    is_out = torch.zeros(K, dtype=torch.bool)
    is_out[chans] = True
    perm = torch.cat([torch.nonzero(~is_out).flatten(), torch.nonzero(is_out).flatten()])
    pd = perm.to(device)
    return dict(x=x[:, pd].contiguous(), w=w[:, pd].contiguous(), perm=perm, outlier_channels=chans)


# ----------------------------------------------------------------------------
# Codebook (CodeQuant-style clustered) weights
# ----------------------------------------------------------------------------

def clustered_weight(N, K, group=128, n_centroids=16, outlier_frac=0.005, outlier_gain=20.0,
                     iters=10, seed=0, device="cpu", rows_per_chunk=512):
    """W ~ N(0, 0.02^2) with outliers, clustered per (row, K group) into
    ``n_centroids`` fp16 centroids by 1-D Lloyd iterations.

    Initial centroid j is the mean of the j-th equal-count slice of the
    sorted group; each iteration assigns every value to the nearest centroid
    (ties to the lower index) and moves each non-empty centroid to the mean of
    its members.  Centroids are then rounded to fp16 and every value is
    assigned to its nearest fp16 centroid.

    Returns idx uint8 [N][K/2] (two 4-bit indices per byte, element 2i in
    bits 3:0), centroids fp16 [N][K/group][n_centroids], and the fp32 weight.
    """
    assert K % group == 0 and group % n_centroids == 0 and n_centroids <= 16
    w = normal((N, K), 0.02, seed, "lut.w", device)
    mask = uniform((N, K), seed, "lut.outliers", device) < outlier_frac
    w = torch.where(mask, w * outlier_gain, w)
    G = K // group
    idx_all = torch.empty((N, K), dtype=torch.uint8, device=device)
    cent_all = torch.empty((N, G, n_centroids), dtype=torch.float16, device=device)
    for r0 in range(0, N, rows_per_chunk):
        r1 = min(N, r0 + rows_per_chunk)
        v = w[r0:r1].view(r1 - r0, G, group)
        s = v.sort(dim=-1).values
        c = s.view(r1 - r0, G, n_centroids, group // n_centroids).mean(dim=-1)
        prev = None
        for _ in range(iters):
            a = (v.unsqueeze(-1) - c.unsqueeze(-2)).abs().argmin(dim=-1)
            if prev is not None and torch.equal(a, prev):
                break
            prev = a
            oh = torch.nn.functional.one_hot(a, n_centroids).to(torch.float32)
            cnt = oh.sum(dim=-2)
            tot = (oh * v.unsqueeze(-1)).sum(dim=-2)
            c = torch.where(cnt > 0, tot / cnt.clamp(min=1), c)
        c16 = c.to(torch.float16)
        a = (v.unsqueeze(-1) - c16.float().unsqueeze(-2)).abs().argmin(dim=-1)
        idx_all[r0:r1] = a.view(r1 - r0, K).to(torch.uint8)
        cent_all[r0:r1] = c16
    packed = (idx_all[:, 0::2] & 0xF) | ((idx_all[:, 1::2] & 0xF) << 4)
    return dict(idx=packed.contiguous(), centroids=cent_all, w=w)


def lut_problem(M, N=4096, K=4096, group=128, seed=0, device="cpu", iters=10):
    x = normal((M, K), 1.0, seed, "lut.x", device).to(torch.bfloat16)
    d = clustered_weight(N, K, group=group, seed=seed, device=device, iters=iters)
    d["x"] = x
    return d


# ----------------------------------------------------------------------------
# MoE inputs
# ----------------------------------------------------------------------------

def moe_problem(T, H, I, E, seed=0, device="cpu"):
    """X bf16 [T][H], logits fp32 [T][E], fused gate/up fp32 [E][2I][H]
    (gate rows first), down fp32 [E][H][I]."""
    x = normal((T, H), 1.0, seed, "moe.x", device).to(torch.bfloat16)
    logits = normal((T, E), 1.0, seed, "moe.logits", device)
    w_gu = torch.empty((E, 2 * I, H), dtype=torch.float32, device=device)
    w_d = torch.empty((E, H, I), dtype=torch.float32, device=device)
    for e in range(E):
        w_gu[e] = normal((2 * I, H), 0.02, seed, f"moe.w_gate_up.{e}", device)
        w_d[e] = normal((H, I), 0.02, seed, f"moe.w_down.{e}", device)
    return dict(x=x, logits=logits, w_gate_up=w_gu, w_down=w_d)


# Magnitude distribution used to draw E2M1 keys for synthetic VQ codebooks:
# probabilities of the 8 magnitude codes (0, 0.5, 1, 1.5, 2, 3, 4, 6), a
# shape typical of Gaussian weights after a per-32 power-of-two prescale.
_E2M1_MAG_PROBS = [0.08, 0.15, 0.15, 0.14, 0.18, 0.16, 0.10, 0.04]


def _scale_codes(shape, seed, name, device, scale_fmt="e8m0", e8m0_range=None):
    """Block scale codes.  E8M0: {119, 120, 121} (weights of magnitude
    ~0.02), 1:2:1, or uniform over e8m0_range = (lo, hi) inclusive.  E4M3 /
    UE5M3 (beside an FP32 tensor scale that maps the largest block to the top
    of the scale range): uniform over the codes of the upper three binades,
    64 .. 448 (E4M3 0x68-0x7E) and 16384 .. 114688 (UE5M3 0xE8-0xFE)."""
    u = uniform(shape, seed, name, device)
    if scale_fmt == "e8m0" and e8m0_range is not None:
        lo, hi = e8m0_range
        return (lo + torch.clamp((u * (hi - lo + 1)).to(torch.int32), max=hi - lo)).to(torch.uint8)
    if scale_fmt == "e8m0":
        return (119 + (u >= 0.25).to(torch.uint8) + (u >= 0.75).to(torch.uint8)).to(torch.uint8)
    lo = {"e4m3": 0x68, "e5m3": 0xE8}[scale_fmt]
    return (lo + torch.clamp((u * 23).to(torch.int32), max=22)).to(torch.uint8)


# FP32 tensor scales of the synthetic 16-element-block VQ weights: about
# amax / (6 * top scale) for N(0, 0.02^2) weights (amax ~ 0.1)
VQ_TENSOR_SCALE = {"e4m3": 0.1 / 2688.0, "e5m3": 0.1 / 688128.0}


def vq_weight(E, N, K, qblock=64, n_entries=256, seed=0, name="vq", device="cpu", scales="prescale",
              scale_fmt="e8m0", ts_segments=1, e8m0_range=None):
    """Codebook->MX weights drawn directly in the VQ format.

    idx uint8 [E][N][K/4]; codebook 16-bit [E][N/qblock][K/qblock][256]
    (4 E2M1 codes per entry, element i in bits 4i+3:4i); and the scales, by
    ``scales``, with block b = 32 for scale_fmt "e8m0", 16 for "e4m3" and
    "e5m3":
      "prescale":      scale codes uint8 [E][N][K/b];
      "postscale":     one scale code per QBlock table, uint8 [E][N/qblock][K/qblock];
      "prescale_plus": 8-bit scale-vector indices uint8 [E][N][K/(8 b)] into a
                       per-matrix table ``scale_codebook`` uint8 [E][256][8] of
                       scale codes (8 consecutive block scales along K each).
    "e4m3" / "e5m3" also give ``tensor_scale`` fp32 [E][ts_segments].
    ``e8m0_range`` = (lo, hi): E8M0 scale codes uniform over lo .. hi instead
    of the {119, 120, 121} of N(0, 0.02^2) weights.
    """
    assert N % qblock == 0 and K % qblock == 0
    probs = torch.tensor(_E2M1_MAG_PROBS, dtype=torch.float64)
    cdf = (probs.cumsum(0) / probs.sum()).to(torch.float32)[:-1].to(device)
    nb = (E, N // qblock, K // qblock, n_entries, 4)
    mag = torch.bucketize(uniform(nb, seed, f"{name}.cb.mag", device), cdf).to(torch.int32)
    sign = (uniform(nb, seed, f"{name}.cb.sign", device) < 0.5).to(torch.int32)
    nib = mag | (sign << 3)
    key = nib[..., 0] | (nib[..., 1] << 4) | (nib[..., 2] << 8) | (nib[..., 3] << 12)
    # stored as int16 bit patterns (torch has no general uint16 arithmetic)
    codebook = torch.where(key >= 32768, key - 65536, key).to(torch.int16)
    g = _gen(seed, f"{name}.idx", device)
    idx = torch.randint(0, n_entries, (E, N, K // 4), generator=g, device=device, dtype=torch.uint8)
    out = dict(idx=idx, codebook=codebook.contiguous())
    b = 32 if scale_fmt == "e8m0" else 16
    if scales == "prescale":
        out["scales"] = _scale_codes((E, N, K // b), seed, f"{name}.scale", device, scale_fmt, e8m0_range)
    elif scales == "postscale":
        out["scales"] = _scale_codes((E, N // qblock, K // qblock), seed, f"{name}.qscale", device, scale_fmt,
                                     e8m0_range)
    elif scales == "prescale_plus":
        assert K % (8 * b) == 0
        g = _gen(seed, f"{name}.sidx", device)
        out["scales"] = torch.randint(0, 256, (E, N, K // (8 * b)), generator=g, device=device, dtype=torch.uint8)
        out["scale_codebook"] = _scale_codes((E, 256, 8), seed, f"{name}.scb", device, scale_fmt, e8m0_range)
    else:
        raise ValueError(scales)
    if scale_fmt != "e8m0":
        u = uniform((E, ts_segments), seed, f"{name}.ts", device)
        out["tensor_scale"] = (VQ_TENSOR_SCALE[scale_fmt] * (0.75 + 0.5 * u)).to(torch.float32)
    return out


def moe_vq_problem(T, H, I, E, seed=0, device="cpu", scales="prescale", qblock=64, scale_fmt="e8m0",
                   x_log2=0, gate_up_e8m0_range=None):
    """X bf16 [T][H] (times 2^x_log2), logits [T][E], VQ gate/up weights
    (N = 2I, K = H; with 16-element blocks, tensor scales per gate and up
    half; E8M0 scale codes over gate_up_e8m0_range if given) and VQ down
    weights (N = H, K = I); ``scales``, ``qblock``, ``scale_fmt`` as in
    vq_weight."""
    x = normal((T, H), 1.0, seed, "moevq.x", device)
    x = (x * 2.0 ** x_log2 if x_log2 else x).to(torch.bfloat16)
    logits = normal((T, E), 1.0, seed, "moevq.logits", device)
    gu = vq_weight(E, 2 * I, H, qblock=qblock, seed=seed, name="moevq.gate_up", device=device, scales=scales,
                   scale_fmt=scale_fmt, ts_segments=2, e8m0_range=gate_up_e8m0_range)
    dn = vq_weight(E, H, I, qblock=qblock, seed=seed, name="moevq.down", device=device, scales=scales,
                   scale_fmt=scale_fmt)
    return dict(x=x, logits=logits, gate_up=gu, down=dn)
