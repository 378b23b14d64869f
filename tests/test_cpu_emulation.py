"""The HIP kernels compiled as host C++ against an emulation header
(tests/cpu_emu/hip/hip_runtime.h) and run under AddressSanitizer on small,
ragged cases: an out-of-bounds access aborts with an ASan report, a
barrier-count mismatch deadlocks and hits the timeout.  Routing is also
checked for its values (its cross-lane steps are emulated exactly); the
other kernels' arithmetic is checked on the GPU against the oracle.

Test infrastructure only; skipped where the ROCm host compiler is absent.
"""
import concurrent.futures
import os
import subprocess
import threading

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(HERE)
EMU = os.path.join(HERE, "cpu_emu")
CLANG = "/opt/rocm/llvm/bin/clang++"
CSRC = os.path.join(REPO, "gemm_bit_weight_amd", "csrc")

pytestmark = pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not available")


@pytest.fixture(scope="module")
def build_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("cpu_emu")


def _build(build_dir, src, drv, name):
    out = os.path.join(str(build_dir), name)
    if not os.path.exists(out):
        cmd = [CLANG, "-std=c++20", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-Wno-unused-value",
               "-I", EMU, "-I", os.path.join(REPO, "include"), "-I", CSRC,
               "-x", "c++", os.path.join(CSRC, src), "-x", "c++", os.path.join(EMU, drv), "-o", out, "-lpthread"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
    return out


def _run(exe, *args, timeout=600):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=timeout, env=env)
    assert "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stderr[-4000:]
    return r.stdout


# The emulated workgroups spend most of their time at barriers, so several
# cases run side by side: the first test of a kernel starts all of that
# kernel's cases (at most _JOBS at a time) and each test waits for its own.
_JOBS = 4
_POOL = concurrent.futures.ThreadPoolExecutor(max_workers=_JOBS)
_RUNS = {}
_LOCK = threading.Lock()


def _run_all(exe, cases, args):
    """Start every case of `cases` (argument tuples) for `exe` once, then wait
    for the one with arguments `args` and return its output."""
    with _LOCK:
        for c in cases:
            key = (exe, *map(str, c))
            if key not in _RUNS:
                _RUNS[key] = _POOL.submit(_run, exe, *c)
    return _RUNS[(exe, *map(str, args))].result()


_MOE_FMTS = [0, 2, 1, 3]
_MOE_LAYOUTS = [(4, 64), (4, 128), (5, 64), (5, 256), (6, 128), (7, 64), (8, 64), (11, 256)]
_MOE_CASES = ([(200, 512, 256, 6, 2, f) for f in _MOE_FMTS] +
              [(90, 512, 256, 3, 2, f, 0, 0, q) for f, q in _MOE_LAYOUTS] + [(200, 512, 256, 6, 2, 0, 1, 128)])


def _moe(build_dir, *args):
    return _run_all(_build(build_dir, "moe_gemm.hip", "drv_moe.cpp", "emu_moe"), _MOE_CASES, args)


@pytest.mark.parametrize("fmt", _MOE_FMTS, ids=["mxfp4", "vq", "e4m3", "e5m3"])
def test_moe_grouped_gemm_in_bounds(build_dir, fmt):
    out = _moe(build_dir, 200, 512, 256, 6, 2, fmt)
    assert "gateup status 0" in out and all(f"down mode {m} status 0" in out for m in range(3)), out


@pytest.mark.parametrize("fmt,qblock", _MOE_LAYOUTS,
                         ids=["postscale-q64", "postscale-q128", "prescale_plus-q64", "prescale_plus-q256",
                              "e4m3-prescale-q128", "e4m3-postscale-q64", "e4m3-prescale_plus-q64",
                              "e5m3-prescale_plus-q256"])
def test_moe_vq_scale_layouts_in_bounds(build_dir, fmt, qblock):
    """VQ weights (E8M0-B32, E4M3-B16 and E5M3-B16 scales) with PreScale /
    PostScale / PreScale+ scales and larger QBlocks: gate/up (2I = 512 rows,
    K = 512) and down (K = I = 256), 3 experts."""
    out = _moe(build_dir, 90, 512, 256, 3, 2, fmt, 0, 0, qblock)
    assert "gateup status 0" in out and all(f"down mode {m} status 0" in out for m in range(3)), out


def test_moe_prquant_tail_copy_in_bounds(build_dir):
    """MXFP4 gate/up writing h with a 128-column tail copy (I + 128 code
    columns), then the down stage over I + 128."""
    out = _moe(build_dir, 200, 512, 256, 6, 2, 0, 1, 128)
    assert "gateup status 0" in out and all(f"down mode {m} status 0" in out for m in range(3)), out


@pytest.mark.parametrize("T,E,K,mode", [(37, 16, 4, ""), (300, 128, 8, ""), (70, 32, 8, "ties"), (50, 300, 5, ""),
                                        (90, 128, 8, "special"), (40, 200, 6, "special"), (30, 300, 8, "special"),
                                        (1100, 1000, 8, ""), (700, 16, 4, ""),
                                        (100, 7, 2, "")])
def test_moe_route_in_bounds_and_exact(build_dir, T, E, K, mode):
    """Ids against a stable sort (descending; -0 ties +0; NaN after every
    number): 'ties' draws from {0, 1, 2}, 'special' from {+-0, +-1, +-inf,
    NaN}; E = 128, 200 and 300 run the 8- and 16-entry lane-group kernels
    and the one-thread-per-token kernel.  Offsets and the pair list are
    checked against the (expert, token) order.  Count tables of at most 16384
    entries (chunks of 64 tokens x experts) take the fused scan + scatter
    kernel (700 tokens: 11 chunks, more than one eight-chunk step of its
    per-expert pass); 1100 tokens x 1000 experts (18000) the separate scan
    and scatter; 7 experts: an odd expert count (14 counts)."""
    exe = _build(build_dir, "moe_route.hip", "drv_route.cpp", "emu_route")
    out = _run(exe, T, E, K, *([mode] if mode else []))
    assert "status 0 mismatched ids 0 mismatched pairs 0" in out, out
    # the allocation-free entry point gives the same outputs (every case here fits its scratch)
    assert "noalloc status 0 differing outputs 0" in out, out


_LUT_CASES = [(1, 40, 384, 32), (5, 256, 1024, 128), (17, 40, 384, 32), (64, 128, 2048, 128), (70, 100, 1024, 64),
              (33, 64, 512, 32), (3, 20, 4608, 64), (16, 33, 2176, 32)]


@pytest.mark.parametrize("M,N,K,group", _LUT_CASES)
def test_lut_gemm_in_bounds(build_dir, M, N, K, group):
    """Ragged M and N, every group size; for M > 16 the split-K path twice (its
    arrival counters must be left at zero) and the no-workspace path."""
    out = _run_all(_build(build_dir, "lut_gemm.hip", "drv_lut.cpp", "emu_lut"), _LUT_CASES, (M, N, K, group))
    assert out.count("status 0 counters left 0") == 2, out
    if M > 16 and " ws=0 " not in out:
        assert "short workspace status 0" in out, out


_MX_CASES = [(16, 512, 512, 0), (1, 40, 96, 0), (130, 72, 640, 64), (33, 40, 2048, 32), (128, 64, 9728, 256),
             (130, 72, 640, 128), (40, 100, 1024, 0), (200, 70, 512, 0), (64, 33, 256, 128), (17, 64, 128, 0),
             (8, 64, 2048, 0)]


@pytest.mark.parametrize("M,N,K,tail", _MX_CASES)
def test_mx_gemm_in_bounds(build_dir, M, N, K, tail):
    out = _run_all(_build(build_dir, "mx_gemm.hip", "drv_mx.cpp", "emu_mx"), _MX_CASES, (M, N, K, tail))
    assert out.count("status 0 counters left 0") == 3, out
