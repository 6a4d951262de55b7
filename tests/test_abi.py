"""C-ABI checks that need no GPU: the library loads, exports every function
include/s5.h declares, and host-side validation returns the documented
status codes before anything is enqueued (fake, aligned pointers are never
dereferenced on these paths)."""

import ctypes
import os
import re
import subprocess
import sys

import pytest

import diagonal_state_space_amd as s5

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "s5.h")

OK, INVALID, UNSUPPORTED, OOM, HIPERR = 0, 1, 2, 3, 4
FAKE = 0x10000  # aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(s5_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("s5_discretize", "s5_forward", "s5_forward_timevarying", "s5_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol():
    L = s5.lib()
    for name in declared_functions():
        assert hasattr(L, name), f"{name} not exported by {s5.lib_path}"
    out = subprocess.run(["nm", "-D", "--defined-only", s5.lib_path], capture_output=True, text=True)
    exported = set(re.findall(r"\bT (s5_[a-z_]+)", out.stdout))
    assert set(declared_functions()) <= exported


def test_peak_library_exports_its_probes():
    """libs5_peak.so (the roofline report's peak-rate probes) exports what
    include/s5_peak.h declares, and refuses bad arguments on the host."""
    from diagonal_state_space_amd import build_lib
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "s5_peak.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(s5_[a-z_0-9]+)\s*\(", text)))
    assert names == ["s5_peak_copy", "s5_peak_mfma_bf16"]
    L = ctypes.CDLL(build_lib.PEAK_LIB_PATH)
    for name in names:
        assert hasattr(L, name)
    L.s5_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    L.s5_peak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert L.s5_peak_copy(FAKE, FAKE + 0x100000, 24, 0, None) == -1       # not a multiple of 16
    assert L.s5_peak_copy(FAKE, FAKE + 16, 64, 0, None) == -1             # overlapping
    assert L.s5_peak_copy(None, FAKE, 64, 1, None) == -1
    assert L.s5_peak_mfma_bf16(0, 10, FAKE, None) == -1
    assert L.s5_peak_mfma_bf16(4, 12, None, None) == -1
    assert L.s5_peak_mfma_bf16(4, 10, FAKE, None) == -1                  # not a multiple of 4


def test_status_strings():
    assert s5.status_string(OK) == "S5_OK"
    assert s5.status_string(INVALID) == "S5_ERR_INVALID_ARGUMENT"
    assert s5.status_string(UNSUPPORTED) == "S5_ERR_UNSUPPORTED"
    assert s5.status_string(OOM) == "S5_ERR_OUT_OF_MEMORY"
    assert s5.status_string(HIPERR) == "S5_ERR_HIP"
    assert s5.status_string(99) == "S5_ERR_UNKNOWN"


def _fwd(B=2, L=8, H=4, P=3, io=0, u=FAKE, lam=FAKE + 0x1000, bt=FAKE + 0x2000, ct=FAKE + 0x3000,
         d=FAKE + 0x4000, logd=FAKE + 0x5000, y=FAKE + 0x100000):
    return s5.lib().s5_forward(B, L, H, P, io, u, lam, bt, ct, d, logd, y, None)


def _fwd_tv(B=2, L=8, H=4, P=3, io=0, u=FAKE, delta=FAKE + 0x6000, y=FAKE + 0x100000, **kw):
    return s5.lib().s5_forward_timevarying(B, L, H, P, io, u, FAKE + 0x1000, FAKE + 0x2000,
                                           FAKE + 0x3000, FAKE + 0x4000, delta, y, None)


def test_forward_validation():
    assert _fwd(u=None) == INVALID
    assert _fwd(y=None) == INVALID
    assert _fwd(lam=None) == INVALID
    assert _fwd(bt=None) == INVALID
    assert _fwd(ct=None) == INVALID
    assert _fwd(d=None) == INVALID
    assert _fwd(logd=None) == INVALID
    assert _fwd(B=-1) == INVALID
    assert _fwd(L=-5) == INVALID
    assert _fwd(P=0) == INVALID
    assert _fwd(H=0) == INVALID
    assert _fwd(P=s5.S5_MAX_P + 1) == UNSUPPORTED
    assert _fwd(H=s5.S5_MAX_H + 1) == UNSUPPORTED
    assert _fwd(io=7) == UNSUPPORTED
    assert _fwd(u=FAKE + 4) == UNSUPPORTED           # misaligned
    assert _fwd(y=FAKE + 0x100008) == UNSUPPORTED
    # y overlapping u / a parameter
    assert _fwd(y=FAKE + 16) == INVALID
    assert _fwd(y=FAKE + 0x3000) == INVALID


def test_empty_is_noop():
    # B*L == 0 validates and returns before touching the device
    assert _fwd(B=0) == OK
    assert _fwd(L=0) == OK
    assert _fwd(B=0, u=None, y=None) == OK
    assert _fwd_tv(L=0, delta=None) == OK


def test_timevarying_validation():
    assert _fwd_tv(delta=None) == INVALID
    assert _fwd_tv(delta=FAKE + 0x6004) == UNSUPPORTED
    assert _fwd_tv(y=FAKE + 0x6000) == INVALID   # y overlaps delta


def test_discretize_validation():
    f = s5.lib().s5_discretize
    a = [FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000, FAKE + 0x4000]
    assert f(4, 3, None, a[1], a[2], a[3], a[4], None) == INVALID
    assert f(0, 3, *a, None) == INVALID
    assert f(4, 0, *a, None) == INVALID
    assert f(s5.S5_MAX_P + 1, 3, *a, None) == UNSUPPORTED
    assert f(4, 3, a[0], a[1], a[2], a[0], a[4], None) == INVALID   # output overlaps input
    assert f(4, 3, a[0], a[1], a[2] + 4, a[3], a[4], None) == UNSUPPORTED


def test_profiling_events_validation():
    L = s5.lib()
    arr = (ctypes.c_void_p * 14)(*([FAKE] * 14))
    assert L.s5_set_profiling_events(arr, 3) == INVALID           # odd count
    assert L.s5_set_profiling_events(arr, 14) == INVALID          # beyond the maximum (12)
    assert L.s5_set_profiling_events(None, 2) == INVALID          # no array
    holes = (ctypes.c_void_p * 2)(FAKE, None)
    assert L.s5_set_profiling_events(holes, 2) == INVALID         # NULL handle
    assert L.s5_set_profiling_events(arr, 6) == OK
    assert L.s5_set_profiling_events(arr, 12) == OK
    assert L.s5_set_profiling_events(None, 0) == OK


def test_alloc_failure_hook():
    # forced from the host in a child process; returns before any HIP call
    code = (
        "import diagonal_state_space_amd as s5;"
        "r = s5.lib().s5_forward(2, 8, 4, 3, 0, 0x10000, 0x11000, 0x12000, 0x13000, 0x14000,"
        " 0x15000, 0x110000, None); print(r)"
    )
    env = dict(os.environ, S5_TEST_FAIL_ALLOC="1")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                         cwd=ROOT, timeout=120)
    assert out.stdout.strip() == str(OOM), out.stderr


def test_binding_refuses_cpu_tensors():
    import torch
    u = torch.zeros(1, 4, 2)
    with pytest.raises(ValueError):
        s5.forward(u, torch.zeros(3, dtype=torch.complex64), torch.zeros(3, 2, dtype=torch.complex64),
                   torch.zeros(2, 3, dtype=torch.complex64), torch.zeros(2), torch.zeros(3))


def _fwd_state(B=2, L=8, H=4, P=3, io=0, u=FAKE, y=FAKE + 0x100000, x0=FAKE + 0x7000,
               xl=FAKE + 0x8000, tv=False):
    L_ = s5.lib()
    if tv:
        return L_.s5_forward_timevarying_stateful(B, L, H, P, io, u, FAKE + 0x1000, FAKE + 0x2000,
                                                  FAKE + 0x3000, FAKE + 0x4000, FAKE + 0x6000, x0, y,
                                                  xl, None)
    return L_.s5_forward_stateful(B, L, H, P, io, u, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000,
                                  FAKE + 0x4000, FAKE + 0x5000, x0, y, xl, None)


@pytest.mark.parametrize("tv", [False, True])
def test_stateful_validation(tv):
    assert _fwd_state(x0=FAKE + 0x7004, tv=tv) == UNSUPPORTED       # misaligned state
    assert _fwd_state(xl=FAKE + 0x8008, tv=tv) == UNSUPPORTED
    assert _fwd_state(xl=FAKE + 16, tv=tv) == INVALID               # final state overlaps u
    assert _fwd_state(xl=FAKE + 0x100000, tv=tv) == INVALID         # ... y
    assert _fwd_state(xl=FAKE + 0x7000, tv=tv) == INVALID           # ... x0 (no in-place update)
    assert _fwd_state(xl=FAKE + 0x1000, tv=tv) == INVALID           # ... a parameter
    assert _fwd_state(y=FAKE + 0x7000 - 32, tv=tv) == INVALID       # y overlaps x0
    assert _fwd_state(B=-1, tv=tv) == INVALID
    assert _fwd_state(B=0, tv=tv) == OK                              # nothing to do
    assert _fwd_state(L=0, x0=None, xl=None, tv=tv) == OK           # nothing asked for


def _fwd_ex(flags=0, B=2, L=8, H=4, P=3, io=0, ct=FAKE + 0x3000, logd=FAKE + 0x5000, delta=None,
            x0=None, x_last=None, y=FAKE + 0x100000, size=None, glu_w=None, glu_bias=None, glu_variant=0):
    desc = s5.ForwardDesc(ctypes.sizeof(s5.ForwardDesc) if size is None else size, flags, io, B, L, H, P,
                          FAKE, FAKE + 0x1000, FAKE + 0x2000, ct, FAKE + 0x4000, logd, delta, x0, y, x_last,
                          glu_w, glu_bias, glu_variant)
    return s5.lib().s5_forward_ex(ctypes.byref(desc), None)


def test_forward_ex_validation():
    assert s5.lib().s5_forward_ex(None, None) == INVALID
    assert _fwd_ex(size=64) == INVALID                                   # wrong struct size
    assert _fwd_ex(flags=1 << 7) == INVALID                              # unknown option bit
    assert _fwd_ex(logd=None) == INVALID                                 # no intervals
    assert _fwd_ex(delta=FAKE + 0x6000) == INVALID                       # both kinds of intervals
    bidir = s5.FLAG_BIDIRECTIONAL
    assert _fwd_ex(flags=bidir, logd=None, delta=FAKE + 0x6000) == INVALID   # backward scan: time-invariant
    assert _fwd_ex(flags=bidir, x0=FAKE + 0x7000) == INVALID             # ... and stateless
    assert _fwd_ex(flags=bidir, x_last=FAKE + 0x7000) == INVALID
    # C~ of 2P columns ending inside y (P columns would end before it)
    H, P = 4, 3
    y = FAKE + 0x100000
    ct = y - H * P * 8 - 16
    assert _fwd_ex(flags=bidir, ct=ct, y=y) == INVALID
    assert _fwd_ex(flags=bidir, ct=FAKE + 0x3004) == UNSUPPORTED         # misaligned
    assert _fwd_ex(flags=bidir | s5.FLAG_GELU | s5.FLAG_HALF_SPECTRUM, B=0) == OK   # empty: no-op
    assert _fwd_ex(flags=s5.FLAG_BILINEAR, L=0) == OK
    assert _fwd_ex(P=0) == INVALID and _fwd_ex(H=1000) == UNSUPPORTED
    # the gated activation
    glu = s5.FLAG_GLU
    w = FAKE + 0x9000
    assert _fwd_ex(flags=glu, glu_variant=1) == INVALID                      # no W
    assert _fwd_ex(flags=glu, glu_w=w, glu_variant=3) == INVALID             # no such variant
    assert _fwd_ex(flags=glu | s5.FLAG_GELU, glu_w=w, glu_variant=1) == INVALID   # a GELU beside the gate's
    assert _fwd_ex(flags=glu, glu_w=FAKE + 0x100000 - 32, glu_variant=2) == INVALID   # W overlaps y
    assert _fwd_ex(flags=glu, glu_w=w, glu_bias=FAKE + 0x100000, glu_variant=1) == INVALID   # bias in y
    assert _fwd_ex(flags=glu, glu_w=w + 4, glu_variant=1) == UNSUPPORTED     # misaligned
    assert _fwd_ex(flags=glu, H=300, glu_w=w, glu_variant=1) == UNSUPPORTED  # beyond the gate's H
    assert _fwd_ex(flags=glu, B=0, glu_w=w, glu_variant=2) == OK             # empty: no-op
    # a caller built before the gate fields: the first version's size, no gate
    v1 = s5.ForwardDesc.glu_w.offset
    assert _fwd_ex(size=v1, B=0) == OK
    assert _fwd_ex(size=v1, flags=glu, B=0, glu_w=w, glu_variant=1) == INVALID


def _step(B=2, H=4, P=3, io=0, flags=0, logd=FAKE + 0x5000, delta=None, x=FAKE + 0x8000, y=FAKE + 0x9000,
          u=FAKE):
    return s5.lib().s5_step(B, H, P, io, flags, u, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000,
                            FAKE + 0x4000, logd, delta, x, y, None)


def test_step_validation():
    assert _step(flags=s5.FLAG_BIDIRECTIONAL) == INVALID      # no backward scan in one step
    assert _step(flags=1 << 9) == INVALID
    assert _step(logd=None) == INVALID                        # neither interval array
    assert _step(delta=FAKE + 0x6000) == INVALID              # both
    assert _step(x=FAKE + 0x9000) == INVALID                  # x overlaps y
    assert _step(x=FAKE + 0x2000) == INVALID                  # x overlaps B~
    assert _step(y=FAKE) == INVALID                           # y overlaps u
    assert _step(x=None) == INVALID and _step(u=None) == INVALID
    assert _step(B=-1) == INVALID and _step(P=0) == INVALID
    assert _step(H=1000) == UNSUPPORTED and _step(io=5) == UNSUPPORTED
    assert _step(x=FAKE + 0x8008) == UNSUPPORTED              # misaligned
    assert _step(B=0) == OK                                   # no-op


def _glu(T=4, H=8, io=0, variant=1, y=FAKE, w=FAKE + 0x1000, bias=FAKE + 0x2000, out=FAKE + 0x3000):
    return s5.lib().s5_glu(T, H, io, variant, y, w, bias, out, None)


def test_glu_validation():
    assert _glu(variant=3) == INVALID
    assert _glu(H=0) == INVALID and _glu(T=-1) == INVALID
    assert _glu(H=300) == UNSUPPORTED and _glu(io=7) == UNSUPPORTED
    assert _glu(w=None) == INVALID and _glu(y=None) == INVALID and _glu(out=None) == INVALID
    assert _glu(out=FAKE + 16) == INVALID          # partial overlap with y
    assert _glu(out=FAKE + 0x1000) == INVALID      # out overlaps W
    assert _glu(out=FAKE + 0x2000) == INVALID      # out overlaps the bias
    assert _glu(y=FAKE + 8) == UNSUPPORTED         # misaligned
    assert _glu(T=0) == OK                         # no-op


@pytest.mark.parametrize("lang,std", [("c", "-std=c99"), ("c++", "-std=c++17")])
def test_header_compiles_standalone(tmp_path, lang, std):
    """include/s5.h needs no HIP headers: plain C and C++ callers can include it."""
    import shutil
    cc = shutil.which("gcc" if lang == "c" else "g++")
    if cc is None:
        pytest.skip("no host compiler")
    src = tmp_path / "use.c"
    src.write_text('#include "s5.h"\nint s5_probe(void) { s5_forward_desc d; d.size = sizeof d; '
                   'return (int)d.size + (int)S5_FORWARD_DESC_SIZE_V1 + S5_FLAG_GLU + S5_GLU_MAX_H; }\n')
    r = subprocess.run([cc, "-x", lang, std, "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{os.path.dirname(HEADER)}",
                        "-c", str(src), "-o", str(tmp_path / "use.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_missing_library_fails_loudly(tmp_path):
    # a copy of the package with no libs5.so: the first call raises, there is
    # no other code path to fall back on
    import shutil
    pkg = os.path.join(ROOT, "diagonal_state_space_amd")
    shutil.copytree(pkg, tmp_path / "diagonal_state_space_amd",
                    ignore=shutil.ignore_patterns("*.so", "csrc", "__pycache__", "_build"))
    code = ("import diagonal_state_space_amd as s5, torch\n"
            "try:\n"
            "    s5.lib()\n"
            "except ImportError as e:\n"
            "    print('raised', e)\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True,
                         env=dict(os.environ, PYTHONPATH=str(tmp_path)), timeout=300)
    assert out.returncode == 0, out.stderr
    assert "raised" in out.stdout and "libs5.so not found" in out.stdout


_SWEEP = r"""
import ctypes, json, sys
import diagonal_state_space_amd as s5
base, gap = 1 << 36, 1 << 26          # fake, aligned, disjoint device ranges (never dereferenced)
ptr = [base + i * gap for i in range(12)]
opts = [(0, False), (s5.FLAG_HALF_SPECTRUM, False), (s5.FLAG_BILINEAR, False), (s5.FLAG_GELU, False),
        (s5.FLAG_GELU_TANH, False), (0, True), (s5.FLAG_BILINEAR | s5.FLAG_GELU, True),
        (s5.FLAG_BIDIRECTIONAL, False), (s5.FLAG_BIDIRECTIONAL | s5.FLAG_GELU, False),
        (s5.FLAG_GLU, False), (s5.FLAG_GLU | s5.FLAG_BILINEAR, True)]
Ps = [1, 63, 64, 65, 128, 129, 192, 193, 255, 256]
Hs = sorted({1, 2, 31, 96, 257, 511} | {32 * k + e for k in range(1, 17) for e in (0, 1) if 32 * k + e <= 512})
bad, n = [], 0
for io in (0, 1):
    for tv in (False, True):
        for flags, state in opts:
            if tv and flags & s5.FLAG_BIDIRECTIONAL:
                continue
            glu = bool(flags & s5.FLAG_GLU)
            for P in Ps:
                for H in Hs:
                    if glu and H > 256:
                        continue
                    d = s5.ForwardDesc(ctypes.sizeof(s5.ForwardDesc), flags, io, 2, 64, H, P,
                                       ptr[0], ptr[1], ptr[2], ptr[3], ptr[4],
                                       None if tv else ptr[5], ptr[6] if tv else None,
                                       ptr[7] if state else None, ptr[8], ptr[9] if state else None,
                                       ptr[10] if glu else None, None, 1 if glu else 0)
                    r = s5.lib().s5_forward_ex(ctypes.byref(d), None)
                    n += 1
                    if r != 3:
                        bad.append((io, tv, flags, state, P, H, r))
print(json.dumps({"n": n, "bad": bad[:20], "nbad": len(bad)}))
"""


def test_every_supported_call_has_kernels():
    """Every size within the limits, with every option, I/O type and interval
    kind, passes validation and finds a compiled kernel instance for each of
    its launches: with allocation forced to fail from the host, each call
    ends at the scratch allocation (S5_ERR_OUT_OF_MEMORY), which comes after
    the dispatch walk, and never at S5_ERR_UNSUPPORTED or S5_ERR_HIP."""
    import json
    env = dict(os.environ, S5_TEST_FAIL_ALLOC="1")
    out = subprocess.run([sys.executable, "-c", _SWEEP], capture_output=True, text=True, env=env,
                         cwd=ROOT, timeout=300)
    assert out.returncode == 0, out.stderr
    res = json.loads(out.stdout.strip().splitlines()[-1])
    assert res["n"] > 10000
    assert res["nbad"] == 0, res["bad"]
