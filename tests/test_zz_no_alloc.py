"""s5_forward_noalloc (the entry point that allocates nothing: scratch from a
fixed per-device array) against s5_forward (the same kernels, scratch from
the library's allocated buffers), through the C ABI: bitwise equal outputs on
two calls in a row, the second smaller than the first (the array keeps the
first call's contents), and a call needing more scratch than the array holds
refused before anything is enqueued."""

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diagonal_state_space_amd  # noqa: F401  (fails loudly if libs5.so is missing)


def _dev(w, cuda):
    t = {k: torch.from_numpy(np.ascontiguousarray(getattr(w, k))).to(cuda)
         for k in ("lam", "b_tilde", "c_tilde", "d", "log_delta")}
    if w.io == "bf16":
        t["u"] = torch.from_numpy(w.u_bf16.view(np.int16)).view(torch.bfloat16).to(cuda)
    else:
        t["u"] = torch.from_numpy(w.u).to(cuda)
    return t


def _abi_call(fn, w, t, y):
    import diagonal_state_space_amd as s5
    io = 1 if w.io == "bf16" else 0
    stream = torch.cuda.current_stream().cuda_stream
    return fn(w.B, w.L, w.H, w.P, io, t["u"].data_ptr(), t["lam"].data_ptr(), t["b_tilde"].data_ptr(),
              t["c_tilde"].data_ptr(), t["d"].data_ptr(), t["log_delta"].data_ptr(), y.data_ptr(), stream)


@pytest.mark.parametrize("first,second", [
    ((16, 16384, 128, 256, "bf16"), (2, 1000, 64, 64, "bf16")),   # the long workload, then a small one
    ((8, 4096, 96, 128, "f32"), (1, 300, 24, 40, "f32")),
    # bf16 with at most 8 features: the float32-operand path, with the
    # widened u and y in the array beside the aggregates
    ((16, 4096, 4, 256, "bf16"), (3, 700, 1, 65, "bf16")),
])
def test_noalloc_matches_allocating_entry_point(first, second):
    import diagonal_state_space_amd as s5
    L = s5.lib()
    cuda = torch.device("cuda:0")
    for k, (B, Lq, H, P, io) in enumerate((first, second)):
        w = wl.make_random(B, Lq, H, P, io=io, seed=60 + k)
        t = _dev(w, cuda)
        y_ref = torch.full_like(t["u"], float("nan"))
        y_fix = torch.full_like(t["u"], float("nan"))
        print(f"[noalloc] call {k}: B={B} L={Lq} H={H} P={P} {io}", flush=True)
        assert _abi_call(L.s5_forward, w, t, y_ref) == 0
        assert _abi_call(L.s5_forward_noalloc, w, t, y_fix) == 0
        torch.cuda.synchronize()
        assert torch.isfinite(y_fix.float()).all()
        assert torch.equal(y_fix, y_ref), f"call {k}: outputs differ"


def test_noalloc_refuses_scratch_beyond_the_array():
    import diagonal_state_space_amd as s5
    L = s5.lib()
    cuda = torch.device("cuda:0")
    # 4096 sequences of one token at P = 256: one range per sequence, whose
    # aggregates alone need 4096 * 16 * 256 * 8 bytes (134 MB) > 32 MiB
    w = wl.make_random(4096, 1, 128, 256, io="bf16", seed=70)
    t = _dev(w, cuda)
    y = torch.zeros_like(t["u"])
    torch.cuda.synchronize()
    st = _abi_call(L.s5_forward_noalloc, w, t, y)
    assert st == 2, s5.status_string(st)   # S5_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.count_nonzero(y.float()) == 0   # nothing was enqueued
    # the allocating entry point serves the same call
    assert _abi_call(L.s5_forward, w, t, y) == 0
    torch.cuda.synchronize()
