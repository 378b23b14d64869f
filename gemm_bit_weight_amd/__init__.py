"""Python binding for libgbw.so: 4-bit-weight GEMMs on MI355X (gfx950).

Argument marshalling only.  Every step of the hot path runs in the HIP
kernels behind the C ABI declared in include/gbw.h; torch supplies device
memory (tensors) and the current stream.  The names match the C entry points.

The library is loaded from this directory (GBW_LIBRARY may name another build
of the same sources, such as the tile-trace measurement build); importing this
package when it has not been built raises ImportError -- there is no fallback
implementation.
"""

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("GBW_LIBRARY") or os.path.join(_HERE, "libgbw.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run gemm_bit_weight_amd.build.build() "
                      "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)

# status / enums (mirror include/gbw.h)
GBW_OK = 0
STATUS_NAMES = {0: "GBW_OK", 1: "GBW_E_ARG", 2: "GBW_E_SHAPE", 3: "GBW_E_ALIGN", 4: "GBW_E_UNSUPPORTED",
                5: "GBW_E_WORKSPACE", 6: "GBW_E_LAUNCH"}
FMT_E8M0_B32 = 0
FMT_E4M3_B16 = 1
FMT_VQ4_E8M0 = 2
FMT_E5M3_B16 = 3
FMT_VQ4_POST = 4
FMT_VQ4_PLUS = 5
FMT_VQ4_E4M3 = 6
FMT_VQ4_E4M3_POST = 7
FMT_VQ4_E4M3_PLUS = 8
FMT_VQ4_E5M3 = 9
FMT_VQ4_E5M3_POST = 10
FMT_VQ4_E5M3_PLUS = 11
DTYPE_BF16 = 0
DTYPE_F32 = 1
TS_DYNAMIC = 1
DETERMINISTIC = 2
FP32_COMBINE = 4
ROTATE_H32 = 8
MOE_GATEUP_SWIGLU = 0
MOE_DOWN_COMBINE = 1
OP_QUANTIZE = 0
OP_MX_GEMM = 1
OP_LUT_GEMM = 2
OP_MOE_ROUTE = 3
OP_MOE_GEMM = 4

EXPORTED = ["gbw_status_string", "gbw_last_error", "gbw_workspace_size", "mx_quantize", "mx_dequantize",
            "mx_residual", "mx_gemm", "residual_tail_gemm", "lut_gemm", "moe_route", "moe_route_noalloc",
            "moe_grouped_gemm"]

_c = ctypes
_vp = _c.c_void_p
_i32 = _c.c_int32
_i64 = _c.c_int64


class _Weight(_c.Structure):
    _fields_ = [("fmt", _i32), ("n_experts", _i32), ("N", _i64), ("K", _i64), ("codes", _vp), ("scales", _vp),
                ("codebook", _vp), ("tensor_scale", _vp), ("ts_per_expert", _i32), ("qblock", _i32),
                ("scale_codebook", _vp)]


class _Act(_c.Structure):
    _fields_ = [("fmt", _i32), ("rows", _i64), ("K", _i64), ("codes", _vp), ("scales", _vp),
                ("tensor_scale", _vp)]


class _MoeOut(_c.Structure):
    _fields_ = [("h_bf16", _vp), ("h_codes", _vp), ("h_scales", _vp), ("y", _vp), ("h_tail", _c.c_int64)]


_lib.gbw_status_string.restype = _c.c_char_p
_lib.gbw_status_string.argtypes = [_c.c_int]
_lib.gbw_last_error.restype = _c.c_char_p
_lib.gbw_last_error.argtypes = []
_lib.gbw_workspace_size.restype = _c.c_size_t
_lib.gbw_workspace_size.argtypes = [_i32, _i64, _i64, _i64, _i32]
_lib.mx_quantize.restype = _c.c_int
_lib.mx_quantize.argtypes = [_vp, _i32, _i64, _i64, _i32, _i64, _vp, _vp, _vp, _i32, _vp, _c.c_size_t, _vp]
_lib.mx_dequantize.restype = _c.c_int
_lib.mx_dequantize.argtypes = [_c.POINTER(_Weight), _i32, _vp, _vp]
_lib.mx_residual.restype = _c.c_int
_lib.mx_residual.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp]
_lib.mx_gemm.restype = _c.c_int
_lib.mx_gemm.argtypes = [_i64, _c.POINTER(_Act), _c.POINTER(_Weight), _vp, _i32, _vp, _c.c_size_t, _vp]
_lib.residual_tail_gemm.restype = _c.c_int
_lib.residual_tail_gemm.argtypes = [_i64, _c.POINTER(_Act), _c.POINTER(_Weight), _c.POINTER(_Weight), _i64, _vp,
                                    _i32, _vp, _c.c_size_t, _vp]
_lib.lut_gemm.restype = _c.c_int
_lib.lut_gemm.argtypes = [_i64, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _c.c_size_t, _vp]
_lib.moe_route.restype = _c.c_int
_lib.moe_route.argtypes = [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _c.c_size_t, _vp]
_lib.moe_route_noalloc.restype = _c.c_int
_lib.moe_route_noalloc.argtypes = [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.moe_grouped_gemm.restype = _c.c_int
_lib.moe_grouped_gemm.argtypes = [_i32, _i64, _i32, _vp, _vp, _vp, _vp, _c.POINTER(_Act), _c.POINTER(_Weight),
                                  _c.POINTER(_MoeOut), _i32, _vp, _c.c_size_t, _vp]


class GbwError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


def _check(code):
    if code != GBW_OK:
        raise GbwError(code, _lib.gbw_last_error().decode())


def _ptr(t):
    return None if t is None else _c.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is not None:
        return _c.c_void_p(stream)
    if torch.cuda.is_available():
        return _c.c_void_p(torch.cuda.current_stream().cuda_stream)
    return None


def library_path():
    return LIB_PATH


def status_string(code):
    return _lib.gbw_status_string(code).decode()


def workspace_size(op, d0=0, d1=0, d2=0, fmt=0):
    return int(_lib.gbw_workspace_size(op, d0, d1, d2, fmt))


# ---------------------------------------------------------------------------
# tensor bundles
# ---------------------------------------------------------------------------

@dataclass
class Act:
    """A quantized activation [rows][K]: codes uint8 [rows][K/2], scales uint8."""
    fmt: int
    codes: torch.Tensor
    scales: torch.Tensor
    tensor_scale: Optional[torch.Tensor] = None

    @property
    def rows(self):
        return self.codes.shape[0]

    @property
    def K(self):
        return self.codes.shape[1] * 2

    def c(self):
        return _Act(self.fmt, self.rows, self.K, self.codes.data_ptr(), self.scales.data_ptr(),
                    self.tensor_scale.data_ptr() if self.tensor_scale is not None else None)


@dataclass
class Weight:
    """A quantized weight of n_experts [N][K] matrices."""
    fmt: int
    N: int
    K: int
    codes: torch.Tensor
    scales: torch.Tensor
    codebook: Optional[torch.Tensor] = None
    tensor_scale: Optional[torch.Tensor] = None
    ts_per_expert: int = 1
    n_experts: int = 1
    qblock: int = 0                                # VQ formats: QBlock edge (0 = 64)
    scale_codebook: Optional[torch.Tensor] = None  # FMT_VQ4_PLUS: [E][256][8] E8M0 codes

    def c(self):
        return _Weight(self.fmt, self.n_experts, self.N, self.K, self.codes.data_ptr(), self.scales.data_ptr(),
                       self.codebook.data_ptr() if self.codebook is not None else None,
                       self.tensor_scale.data_ptr() if self.tensor_scale is not None else None,
                       self.ts_per_expert, self.qblock,
                       self.scale_codebook.data_ptr() if self.scale_codebook is not None else None)


def _dev(t):
    return t.device


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def mx_quantize(x, fmt=FMT_E8M0_B32, tail_copy=0, tensor_scale=None, dynamic=None, out=None, ws=None,
                stream=None, rotate=False):
    """Quantize x [rows][K] (bf16 or fp32, on the GPU) -> Act.

    E4M3-B16 / E5M3-B16: the tensor scale is computed from x unless
    ``tensor_scale`` (a 1-element fp32 device tensor) is given.
    ``rotate`` (E8M0-B32): block Hadamard rotation of every 32-block first.
    """
    assert x.dim() == 2 and x.is_contiguous()
    rows, K = x.shape
    dtype = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32}[x.dtype]
    bs = 32 if fmt == FMT_E8M0_B32 else 16
    W = K + tail_copy
    dev = x.device
    if out is None:
        codes = torch.empty((rows, W // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, W // bs), dtype=torch.uint8, device=dev)
    else:
        codes, scales = out.codes, out.scales
    flags = ROTATE_H32 if rotate else 0
    ts = None
    if fmt in (FMT_E4M3_B16, FMT_E5M3_B16):
        if dynamic is None:
            dynamic = tensor_scale is None
        if dynamic:
            flags |= TS_DYNAMIC
            ts = tensor_scale if tensor_scale is not None else torch.empty(1, dtype=torch.float32, device=dev)
        else:
            ts = tensor_scale
        if ws is None and dynamic:
            ws = torch.empty(workspace_size(OP_QUANTIZE, rows, K, 0, fmt), dtype=torch.uint8, device=dev)
    wsb = ws.numel() if ws is not None else 0
    _check(_lib.mx_quantize(_ptr(x), dtype, rows, K, fmt, tail_copy, _ptr(codes), _ptr(scales), _ptr(ts), flags,
                            _ptr(ws), wsb, _stream(stream)))
    return Act(fmt, codes, scales, ts)


def mx_dequantize(w: Weight, expert=0, out=None, stream=None):
    if out is None:
        out = torch.empty((w.N, w.K), dtype=torch.float32, device=w.codes.device)
    cw = w.c()
    _check(_lib.mx_dequantize(_c.byref(cw), expert, _ptr(out), _stream(stream)))
    return out


def mx_residual(w_f32, codes, scales, tail, out=None, stream=None):
    N, K = w_f32.shape
    if out is None:
        out = torch.empty((N, tail), dtype=torch.float32, device=w_f32.device)
    _check(_lib.mx_residual(_ptr(w_f32), N, K, tail, _ptr(codes), _ptr(scales), _ptr(out), _stream(stream)))
    return out


def weight_from_act(a: Act) -> Weight:
    """View a quantized [N][K] matrix (E8M0-B32, E4M3-B16 or E5M3-B16) as a one-expert weight."""
    return Weight(a.fmt, a.rows, a.K, a.codes, a.scales, None, a.tensor_scale, 1, 1)


def _ws(ws, nbytes, device):
    """A GEMM workspace: zeroed when made here, as split-K GEMMs need their
    arrival counters (its first 64 KiB) zero; calls leave them zero."""
    if ws is None and nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    return ws, (ws.numel() if ws is not None else 0)


def mx_gemm(a: Act, w: Weight, M=None, out=None, flags=0, ws=None, stream=None):
    """y = deq(a) deq(w)^T.  ``ws=False`` runs without a workspace."""
    M = a.rows if M is None else M
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.float32, device=a.codes.device)
    if ws is False:
        ws, wsb = None, 0
    else:
        ws, wsb = _ws(ws, workspace_size(OP_MX_GEMM, M, w.N, w.K), a.codes.device)
    ca, cw = a.c(), w.c()
    _check(_lib.mx_gemm(M, _c.byref(ca), _c.byref(cw), _ptr(out), flags, _ptr(ws), wsb, _stream(stream)))
    return out


def residual_tail_gemm(a: Act, w: Weight, r: Optional[Weight], tail, M=None, out=None, flags=0, ws=None,
                       stream=None):
    M = a.rows if M is None else M
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.float32, device=a.codes.device)
    if ws is False:
        ws, wsb = None, 0
    else:
        ws, wsb = _ws(ws, workspace_size(OP_MX_GEMM, M, w.N, w.K + tail), a.codes.device)
    ca, cw = a.c(), w.c()
    cr = r.c() if r is not None else None
    _check(_lib.residual_tail_gemm(M, _c.byref(ca), _c.byref(cw), _c.byref(cr) if cr is not None else None, tail,
                                   _ptr(out), flags, _ptr(ws), wsb, _stream(stream)))
    return out


def lut_gemm(x_bf16, idx, centroids_f16, group=128, out=None, ws=None, flags=0, stream=None):
    """y = bf16(x) fp16(C[idx])^T.  ``ws``: a workspace whose first bytes
    (the tile arrival counters) are zero before its first use; every call
    leaves them zero, so one zeroed workspace serves any number of calls.
    ``ws=False`` runs without one (one workgroup per tile over all of K)."""
    M, K = x_bf16.shape
    N = idx.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x_bf16.device)
    need = workspace_size(OP_LUT_GEMM, M, N, K)
    if ws is False:
        ws = None
    elif ws is None and need:
        ws = torch.zeros(need, dtype=torch.uint8, device=x_bf16.device)
    _check(_lib.lut_gemm(M, N, K, group, _ptr(x_bf16), _ptr(idx), _ptr(centroids_f16), _ptr(out), flags, _ptr(ws),
                         ws.numel() if ws is not None else 0, _stream(stream)))
    return out


def moe_route(logits, topk, out=None, ws=None, stream=None):
    T, E = logits.shape
    dev = logits.device
    if out is None:
        out = dict(topk_ids=torch.empty((T, topk), dtype=torch.int32, device=dev),
                   topk_w=torch.empty((T, topk), dtype=torch.float32, device=dev),
                   expert_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                   pair_token=torch.empty(T * topk, dtype=torch.int32, device=dev),
                   pair_pos=torch.empty((T, topk), dtype=torch.int32, device=dev))
    need = workspace_size(OP_MOE_ROUTE, T, E)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(_lib.moe_route(_ptr(logits), T, E, topk, _ptr(out["topk_ids"]), _ptr(out["topk_w"]),
                          _ptr(out["expert_offsets"]), _ptr(out["pair_token"]), _ptr(out["pair_pos"]), _ptr(ws),
                          ws.numel() if ws is not None else 0, _stream(stream)))
    return out


def moe_route_noalloc(logits, topk, out=None, stream=None):
    """moe_route with its scratch in the library's fixed per-GPU array (no
    workspace; ceil(T / 64) * E <= 131072).  Calls that overlap in time on
    one GPU share that array and race."""
    T, E = logits.shape
    dev = logits.device
    if out is None:
        out = dict(topk_ids=torch.empty((T, topk), dtype=torch.int32, device=dev),
                   topk_w=torch.empty((T, topk), dtype=torch.float32, device=dev),
                   expert_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                   pair_token=torch.empty(T * topk, dtype=torch.int32, device=dev),
                   pair_pos=torch.empty((T, topk), dtype=torch.int32, device=dev))
    _check(_lib.moe_route_noalloc(_ptr(logits), T, E, topk, _ptr(out["topk_ids"]), _ptr(out["topk_w"]),
                                  _ptr(out["expert_offsets"]), _ptr(out["pair_token"]), _ptr(out["pair_pos"]),
                                  _stream(stream)))
    return out


def moe_grouped_gemm(stage, route, a: Act, w: Weight, h_bf16=None, h_codes=None, h_scales=None, y=None, flags=0,
                     ws=None, stream=None, h_tail=0):
    """One stage of the routed expert FFN (see include/gbw.h).

    GATEUP: fills h_bf16 [P][I] and/or h_codes [P][(I+h_tail)/2] + h_scales
            [P][(I+h_tail)/32] (h_tail > 0: the quantized last h_tail columns
            are appended again, PRQuant's online tail copy).
    DOWN:   overwrites y [T][H] through a bf16 (flags=FP32_COMBINE: fp32)
            slot buffer in the workspace and a fixed-order combine; ws=False
            adds into y with fp32 atomics instead (no workspace).  With
            ws=None each call allocates and zero-fills a workspace (P x H
            x 2 bytes); repeated calls should pass one made once with
            torch.zeros(workspace_size(OP_MOE_GEMM, P, H, fp32_combine)).
    """
    T, topk = route["topk_ids"].shape
    P = T * topk
    need = 0
    if stage == MOE_DOWN_COMBINE and ws is not False:
        need = workspace_size(OP_MOE_GEMM, P, w.N, 1 if flags & FP32_COMBINE else 0)
    if ws is False:
        ws, wsb = None, 0
    else:
        ws, wsb = _ws(ws, need, a.codes.device)
    o = _MoeOut(h_bf16.data_ptr() if h_bf16 is not None else None,
                h_codes.data_ptr() if h_codes is not None else None,
                h_scales.data_ptr() if h_scales is not None else None,
                y.data_ptr() if y is not None else None, h_tail)
    ca, cw = a.c(), w.c()
    _check(_lib.moe_grouped_gemm(stage, T, topk, _ptr(route["expert_offsets"]), _ptr(route["pair_token"]),
                                 _ptr(route["pair_pos"]), _ptr(route["topk_w"]), _c.byref(ca), _c.byref(cw),
                                 _c.byref(o), flags, _ptr(ws), wsb, _stream(stream)))


def moe_ffn_mx(x, route, w_gate_up: Weight, w_down: Weight, out=None, h_bf16=None, flags=0, bufs=None,
               stream=None):
    """The whole routed FFN on MXFP4 activations: quantize x, gate/up with the
    fused SwiGLU + requantization, down with the weighted combine."""
    T, H = x.shape
    topk = route["topk_ids"].shape[1]
    P = T * topk
    I = w_gate_up.N // 2
    dev = x.device
    if bufs is None:
        bufs = dict(xq=Act(FMT_E8M0_B32, torch.empty((T, H // 2), dtype=torch.uint8, device=dev),
                           torch.empty((T, H // 32), dtype=torch.uint8, device=dev)),
                    hc=torch.empty((P, I // 2), dtype=torch.uint8, device=dev),
                    hs=torch.empty((P, I // 32), dtype=torch.uint8, device=dev))
    xq = mx_quantize(x, FMT_E8M0_B32, out=bufs["xq"], stream=stream)
    moe_grouped_gemm(MOE_GATEUP_SWIGLU, route, xq, w_gate_up, h_bf16=h_bf16, h_codes=bufs["hc"],
                     h_scales=bufs["hs"], stream=stream)
    if out is None:
        out = torch.empty((T, w_down.N), dtype=torch.float32, device=dev)
    moe_grouped_gemm(MOE_DOWN_COMBINE, route, Act(FMT_E8M0_B32, bufs["hc"], bufs["hs"]), w_down, y=out,
                     flags=flags, stream=stream)
    return out
