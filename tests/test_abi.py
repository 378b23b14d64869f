"""CPU checks of the C ABI: the library loads, exports every function that
include/gbw.h declares, and rejects bad arguments before touching a device
(no compute call is made here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gbw.h")
LIB = os.path.join(ROOT, "gemm_bit_weight_amd", "libgbw.so")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s+\**([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def gbw():
    if not os.path.exists(LIB):
        pytest.fail("libgbw.so is not built (run __graft_entry__.build())")
    import gemm_bit_weight_amd as m
    return m


def test_header_declares_the_boundary():
    names = _declared()
    for n in ["mx_quantize", "mx_gemm", "lut_gemm", "moe_grouped_gemm", "residual_tail_gemm", "moe_route",
              "mx_dequantize", "mx_residual", "gbw_workspace_size", "gbw_status_string", "gbw_last_error"]:
        assert n in names, n


def test_library_exports_every_declared_symbol(gbw):
    lib = ctypes.CDLL(LIB)
    for n in _declared():
        assert hasattr(lib, n), f"libgbw.so does not export {n}"
    assert sorted(gbw.EXPORTED) == _declared()


def test_status_strings(gbw):
    assert gbw.status_string(0) == "ok"
    assert gbw.status_string(2) == "invalid shape"
    assert gbw.status_string(99) == "unknown status"


def test_workspace_sizes(gbw):
    assert gbw.workspace_size(gbw.OP_QUANTIZE, 100, 64, 0, gbw.FMT_E8M0_B32) == 0
    assert gbw.workspace_size(gbw.OP_QUANTIZE, 100, 64, 0, gbw.FMT_E4M3_B16) > 0
    assert gbw.workspace_size(gbw.OP_MX_GEMM, 128, 2560, 9728 + 256) > 0
    assert gbw.workspace_size(gbw.OP_MX_GEMM, 0, 2560, 9728) == 0


def test_validation_before_any_device_work(gbw):
    L = gbw._lib
    # mx_quantize: K not a multiple of 32 -> GBW_E_SHAPE, bad dtype -> GBW_E_ARG
    assert L.mx_quantize(None, 0, 4, 33, 0, 0, None, None, None, 0, None, 0, None) == 2
    assert L.mx_quantize(None, 7, 4, 64, 0, 0, None, None, None, 0, None, 0, None) == 1
    assert L.mx_quantize(None, 0, 4, 64, 9, 0, None, None, None, 0, None, 0, None) == 1
    assert L.mx_quantize(None, 0, -1, 64, 0, 0, None, None, None, 0, None, 0, None) == 1
    # tail copy must be block aligned
    assert L.mx_quantize(None, 0, 4, 64, 0, 16, None, None, None, 0, None, 0, None) == 2
    # E4M3 without a tensor scale pointer
    assert L.mx_quantize(None, 0, 4, 64, 1, 0, None, None, None, 0, None, 0, None) == 1
    # null pointers with a real shape
    assert L.mx_quantize(None, 0, 4, 64, 0, 0, None, None, None, 0, None, 0, None) == 1
    assert b"null" in L.gbw_last_error()
    # misaligned pointers are rejected before launching
    assert L.mx_quantize(ctypes.c_void_p(0x1001), 0, 4, 64, 0, 0, ctypes.c_void_p(0x2000),
                         ctypes.c_void_p(0x3000), None, 0, None, 0, None) == 3
    # E4M3 dynamic scale needs a workspace
    assert L.mx_quantize(ctypes.c_void_p(0x1000), 0, 4, 64, 1, 0, ctypes.c_void_p(0x2000),
                         ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000), 1, None, 0, None) == 5
    # zero rows is a no-op that never touches the device
    assert L.mx_quantize(None, 0, 0, 64, 0, 0, None, None, None, 0, None, 0, None) == 0


def test_gemm_validation(gbw):
    L = gbw._lib
    a = gbw._Act(0, 16, 48, 0x1000, 0x2000, None)        # K = 48: not a multiple of 32
    w = gbw._Weight(0, 1, 8, 48, 0x3000, 0x4000, None, None, 1)
    assert L.mx_gemm(16, ctypes.byref(a), ctypes.byref(w), ctypes.c_void_p(0x5000), 0, None, 0, None) == 2
    a = gbw._Act(1, 16, 64, 0x1000, 0x2000, None)        # E4M3 activation on the MXFP4 GEMM
    assert L.mx_gemm(16, ctypes.byref(a), ctypes.byref(w), ctypes.c_void_p(0x5000), 0, None, 0, None) == 4
    a = gbw._Act(0, 16, 64, 0x1000, 0x2000, None)
    w = gbw._Weight(0, 1, 8, 96, 0x3000, 0x4000, None, None, 1)   # K mismatch
    assert L.mx_gemm(16, ctypes.byref(a), ctypes.byref(w), ctypes.c_void_p(0x5000), 0, None, 0, None) == 2
    w = gbw._Weight(0, 1, 8, 64, 0x3000, 0x4000, None, None, 1)
    assert L.mx_gemm(32, ctypes.byref(a), ctypes.byref(w), ctypes.c_void_p(0x5000), 0, None, 0, None) == 2  # M > rows
    assert L.mx_gemm(0, ctypes.byref(a), ctypes.byref(w), None, 0, None, 0, None) == 0                   # empty
    # residual tail not a multiple of 32
    r = gbw._Weight(0, 1, 8, 48, 0x3000, 0x4000, None, None, 1)
    assert L.residual_tail_gemm(16, ctypes.byref(a), ctypes.byref(w), ctypes.byref(r), 48,
                                ctypes.c_void_p(0x5000), 0, None, 0, None) == 2


def test_moe_validation(gbw):
    """moe_grouped_gemm: format pairs, QBlock edges and the scale-table
    requirements are checked on the host; T = 0 is a no-op (NULL outputs
    allowed) that never touches the device."""
    L = gbw._lib
    off = ctypes.c_void_p(0x1000)
    ptr = ctypes.c_void_p(0x2000)

    def call(stage, T, a, w, out):
        return L.moe_grouped_gemm(stage, T, 2, off, ptr, ptr, ptr, ctypes.byref(a), ctypes.byref(w),
                                  ctypes.byref(out), 0, None, 0, None)
    H, I, E = 256, 128, 4
    a = gbw._Act(0, 8, H, 0x3000, 0x4000, None)
    out = gbw._MoeOut(None, None, None, None, 0)
    w = gbw._Weight(gbw.FMT_VQ4_E8M0, E, 2 * I, H, 0x5000, 0x6000, 0x7000, None, 1, 0, None)
    assert call(0, 0, a, w, out) == 0                              # no tokens, no outputs: OK
    assert call(0, 4, a, w, out) == 1                              # tokens but no h buffers
    w.qblock = 96
    assert call(0, 0, a, w, out) == 1                              # QBlock edge not 64/128/256
    w.qblock = 256
    assert call(0, 0, a, w, out) == 0                              # N = 256, K = 256: fine
    w = gbw._Weight(gbw.FMT_VQ4_PLUS, E, 2 * I, H, 0x5000, 0x6000, 0x7000, None, 1, 0, None)
    assert call(0, 0, a, w, out) == 1                              # PreScale+ without a scale table
    w.scale_codebook = 0x8001
    assert call(0, 0, a, w, out) == 3                              # scale table not 4-byte aligned
    w = gbw._Weight(gbw.FMT_VQ4_E4M3, E, 2 * I, H, 0x5000, 0x6000, 0x7000, 0x9000, 2, 0, None)
    assert call(0, 0, a, w, out) == 4                              # E4M3 VQ weights need E4M3 activations
    a16 = gbw._Act(gbw.FMT_E4M3_B16, 8, H, 0x3000, 0x4000, 0xA000)
    assert call(0, 0, a16, w, out) == 0
    a16.fmt = gbw.FMT_E5M3_B16
    assert call(0, 0, a16, w, out) == 4                            # scale formats must agree
    # E4M3-B16 down weights: one tensor scale per expert (two segments would
    # give the lower output rows the wrong scale)
    a16.fmt = gbw.FMT_E4M3_B16
    wd = gbw._Weight(gbw.FMT_E4M3_B16, E, H, I, 0x5000, 0x6000, None, 0x9000, 2, 0, None)
    a16.K = I
    a16.rows = 16
    assert call(1, 0, a16, wd, out) == 1
    wd.ts_per_expert = 1
    assert call(1, 0, a16, wd, out) == 0


def test_descriptor_layouts_match_the_header(gbw, tmp_path):
    """The ctypes descriptors have the C structs' field offsets and sizes
    (compiled from include/gbw.h by the host C compiler)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    structs = {"gbw_weight": gbw._Weight, "gbw_act": gbw._Act, "gbw_moe_out": gbw._MoeOut}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "gbw.h"', 'int main(void) {']
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ['  return 0;', '}']
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)
