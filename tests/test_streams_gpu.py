"""Forward calls from several host threads on several streams at once give
the bits of the same calls run one after another: the library's reusable
scratch buffers (each taken by one call at a time and reused only by later
calls on the stream of its last use) keep concurrent calls apart; past 64
streams a call waits for the device and takes over another stream's buffer."""

import threading

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


def _inputs(w, cuda):
    t = {k: torch.from_numpy(np.ascontiguousarray(getattr(w, k))).to(cuda)
         for k in ("lam", "b_tilde", "c_tilde", "d", "log_delta")}
    if w.io == "bf16":
        t["u"] = torch.from_numpy(w.u_bf16.view(np.int16)).view(torch.bfloat16).to(cuda)
    else:
        t["u"] = torch.from_numpy(w.u).to(cuda)
    if w.delta is not None:
        t["delta"] = torch.from_numpy(w.delta).to(cuda)
    return t


def _call(s5, w, t, y):
    if w.time_varying:
        s5.forward_timevarying(t["u"], t["lam"], t["b_tilde"], t["c_tilde"], t["d"], t["delta"], y=y)
    else:
        s5.forward(t["u"], t["lam"], t["b_tilde"], t["c_tilde"], t["d"], t["log_delta"], y=y)


def test_concurrent_streams_match_serial():
    import diagonal_state_space_amd as s5
    cuda = torch.device("cuda:0")
    # different shapes, so the calls ask for scratch of different sizes
    ws = [wl.make_random(4, 3000, 128, 256, io="bf16", seed=31),
          wl.make_random(2, 5000, 96, 128, io="f32", tv=True, seed=32, kind="random_walk"),
          wl.make_random(8, 1000, 64, 64, io="f32", seed=33),
          wl.make_random(3, 2500, 256, 192, io="bf16", seed=34)]
    ts = [_inputs(w, cuda) for w in ws]
    refs = []
    for w, t in zip(ws, ts):
        y = torch.empty_like(t["u"])
        _call(s5, w, t, y)
        refs.append(y)
    torch.cuda.synchronize()
    reps = 6
    outs = [[torch.full_like(t["u"], float("nan")) for _ in range(reps)] for t in ts]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in ws]
    errors = []

    def worker(k):
        try:
            with torch.cuda.stream(streams[k]):
                for r in range(reps):
                    _call(s5, ws[k], ts[k], outs[k][r])
        except Exception as e:   # reported after the join
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(ws))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in range(len(ws)):
        for r in range(reps):
            assert torch.equal(outs[k][r], refs[k]), f"workload {k}, repetition {r}"
    print(f"[streams] {len(ws)} threads x {reps} calls on separate streams: bitwise equal", flush=True)


def test_more_streams_than_scratch_slots():
    """70 streams, two rounds of calls with growing and shrinking sizes: the
    65th stream onwards takes over buffers of earlier streams after waiting
    for the device, and every output still matches its serial reference."""
    import diagonal_state_space_amd as s5
    cuda = torch.device("cuda:0")
    ws = [wl.make_random(2, 200 + 37 * (k % 5), 64, 64, io="bf16", seed=40 + k % 5) for k in range(5)]
    ts = [_inputs(w, cuda) for w in ws]
    refs = []
    for w, t in zip(ws, ts):
        y = torch.empty_like(t["u"])
        _call(s5, w, t, y)
        refs.append(y)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(70)]
    outs = []
    for rnd in range(2):
        for k, st in enumerate(streams):
            j = (k + rnd) % len(ws)
            with torch.cuda.stream(st):   # the poison fill and the call in one stream's order
                y = torch.full_like(ts[j]["u"], float("nan"))
                _call(s5, ws[j], ts[j], y)
            outs.append((j, y))
    torch.cuda.synchronize()
    for n, (j, y) in enumerate(outs):
        assert torch.equal(y, refs[j]), f"call {n} (workload {j})"
    print(f"[streams] {len(outs)} calls over {len(streams)} streams: bitwise equal", flush=True)


def test_library_loaded_before_torch_initialises():
    """A program that loads the library before it touches torch (s5.lib()
    first) still gets working calls: the binding imports torch before it
    loads libs5.so, so both use torch's HIP runtime. (Loaded the other way
    round, the library bound to the system's runtime and every call on
    torch's stream returned S5_ERR_HIP.) Run in a child process, which must
    start with nothing imported."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import diagonal_state_space_amd as s5\n"
        "s5.lib()\n"
        "import numpy as np, torch, workloads as wl\n"
        "w = wl.make_random(1, 64, 16, 8, seed=3)\n"
        "c = torch.device('cuda:0')\n"
        "t = [torch.from_numpy(np.ascontiguousarray(getattr(w, k))).to(c) for k in "
        "('u', 'lam', 'b_tilde', 'c_tilde', 'd', 'log_delta')]\n"
        "y = s5.forward(*t)\n"
        "torch.cuda.synchronize()\n"
        "print('ok', bool(torch.isfinite(y).all()))\n"
    )
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=root, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().endswith("ok True")
