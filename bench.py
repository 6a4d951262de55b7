"""Benchmark of the S5 layer forward hot path on one MI355X.

One step = one complete s5_forward call (discretisation, drive projection,
chunked scan with carry, readout) over one batch of synthetic input that is
already resident in HBM. Default workload: B=16, L=16384, H=128, P=256 with
bf16 u/y (the Path-X-shaped configuration). The step rotates over several
input/output buffer sets whose total exceeds the 256 MB Infinity Cache.

Prints one JSON line with the contract fields plus
  roofline      dominant kernel: the state and output pass (k_scan: drive,
                scan and readout), timed with HIP events that the library
                records around that launch on the call's stream; its
                algorithmic work is the two complex projections, 8*P*H flops
                per token
  kernels       average duration of each of the three launches of one call
                (packing, aggregate pass k_reduce, k_scan)
  hbm           the layer's algorithmic bytes (u in, y out, Delta in) over the
                summed duration of the three launches
  cpu_baseline  the float64 oracle timed on this host's cores
  parity        max |y - y_oracle| / rms(y_oracle) of the benchmark's output
  step_events   the same call timed by a HIP event pair on its stream: median
                and mean of --event-steps calls after 10 warm-ups
  peaks_measured  the chip's rates measured in this run (libs5_peak.so): a
                streaming copy for HBM GB/s and a register-only MFMA loop for
                dense bf16 TF/s, beside the vendor figures; every fraction
                below is also given against them (frac_measured)
  configs       the four other workloads (tiny, medium, long, irregular),
                each measured in this run: wall time per call over rotating
                buffer sets (20 warm-up calls, then max(--steps, 100) timed:
                the first few hundred microseconds after a synchronisation
                run slower), tokens/s, per-launch kernel times, the dominant
                kernel's roofline fraction, the layer's HBM fraction and the
                parity of its output against the oracle
  device_warmup before the warm-up steps, untimed calls keep the GPU busy for
                --device-warmup seconds (default 0.5), since the chip raises
                its clocks only under sustained load: a timed region of a few
                milliseconds right after set-up measures that ramp (config 3,
                20 calls: 127-137 us per call cold, 108-109 us once warm).
                ms_per_step_without gives the same K steps timed right after
                the --warmup calls alone, before that phase

--variant times the same workload through s5_forward_ex with one option
(initial/final state, half spectrum, bilinear, GELU, bidirectional) or as a
stream of chunks with the state carried between calls (chunked:C); those
lines carry the timing only (no roofline, kernels or cpu_baseline).
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "S5 layer fwd tokens/s (B·L/s) at L=16384,H=128,P=256; % HBM roofline"
CSRC = os.path.join(ROOT, "diagonal_state_space_amd", "csrc")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "k_scan_traffic.json")
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 2500.0}   # fp32 io runs bf16x3 products
CONFIG_INDEX = 3


class HipEvents:
    """Raw hipEvent_t handles via libamdhip64 (the library records them)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        e = ctypes.c_void_p()
        rc = self.h.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        rc = self.h.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, e: int) -> None:
        self.h.hipEventDestroy(ctypes.c_void_p(e))


# sources that do not build or launch the forward passes' kernels (the
# single-step and gated-activation kernels, the host-side discretisation
# entry point, the C ABI layer's validation): edits there leave the traffic
# record valid
DIGEST_EXCLUDE = {"s5_step.hip", "s5_glu.hip", "s5_discretize.hip", "s5_api.cpp"}


def kernel_source_digest() -> str:
    """sha256 over the HIP/C++ sources that build and launch the forward
    passes' kernels (sorted by name)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".cpp")) and name not in DIGEST_EXCLUDE:
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per k_scan launch from the committed counter record, if it was
    taken on this workload with the current kernel sources; else None."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("source_sha256") != kernel_source_digest():
        return None
    return int(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"])


def calibrate_copy(mib: int, reps: int) -> int:
    """Plain device-to-device copies of a known size (for scaling the HBM byte
    counters): reads and writes mib MiB per copy."""
    import torch
    n = mib << 20
    x = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    x.fill_(1)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "reps": reps}), flush=True)
    return 0


def algorithmic_bytes(w) -> int:
    """HBM bytes the method must move: u in, y out, (time-varying) Delta in,
    parameters once."""
    s = 2 if w.io == "bf16" else 4
    tok = w.B * w.L
    b = tok * w.H * 2 * s
    if w.time_varying:
        b += tok * w.P * 4
    b += 8 * w.P + 16 * w.P * w.H + 4 * w.H + 4 * w.P
    return b


def algorithmic_flops(w) -> int:
    """Dense real-equivalent work of the two complex projections: 8*P*H per token
    (4PH for B_bar u, 4PH for Re(C~ x))."""
    return 8 * w.P * w.H * w.B * w.L


class PeakProbes:
    """The chip's rates measured in this run with libs5_peak.so: HBM GB/s of
    a streaming copy, dense bf16 TF/s of a register-only MFMA loop."""

    def __init__(self):
        from diagonal_state_space_amd import build_lib
        self.lib = ctypes.CDLL(build_lib.PEAK_LIB_PATH)
        self.lib.s5_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_void_p]
        self.lib.s5_peak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]

    def measure(self, torch, copy_mib: int = 2048, reps: int = 10) -> dict:
        stream = torch.cuda.current_stream()
        nbytes = copy_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
        src.fill_(3)
        dst = torch.empty_like(src)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]

        def timed(fn):
            for r in range(-2, reps):
                if r >= 0:
                    ev[2 * r].record()
                fn()
                if r >= 0:
                    ev[2 * r + 1].record()
            torch.cuda.synchronize()
            return float(np.median([ev[2 * r].elapsed_time(ev[2 * r + 1]) for r in range(reps)]))

        def probe(nt):
            rc = self.lib.s5_peak_copy(src.data_ptr(), dst.data_ptr(), nbytes, nt, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"s5_peak_copy failed ({rc})")

        copies = {"plain": timed(lambda: probe(0)), "nontemporal": timed(lambda: probe(1)),
                  "torch": timed(lambda: dst.copy_(src))}
        if not torch.equal(dst[:4096], src[:4096]):
            raise RuntimeError("s5_peak_copy: copy mismatch")
        del src, dst
        copy_gbs = {k: round(2 * nbytes / (v * 1e-3) / 1e9, 1) for k, v in copies.items()}
        ncu = torch.cuda.get_device_properties(0).multi_processor_count
        blocks, iters = 4 * ncu, 4000
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
        def mfma():
            rc = self.lib.s5_peak_mfma_bf16(blocks, iters, out.data_ptr(), stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"s5_peak_mfma_bf16 failed ({rc})")

        mfma_ms = timed(mfma)
        flops = blocks * 4 * 8 * iters * 16384
        return {"hbm_copy_GBs": max(copy_gbs.values()), "copies_GBs": copy_gbs,
                "mfma_bf16_TFLOPs": round(flops / (mfma_ms * 1e-3) / 1e12, 1),
                "vendor": {"hbm_GBs": HBM_PEAK_GBS, "mfma_bf16_TFLOPs": MFMA_PEAK_TFLOPS["bf16"]},
                "method": f"best of three copies of {copy_mib} MiB (16-byte vector loads/stores, plain and "
                          f"nontemporal, and torch's copy; median of {reps} each); {blocks} workgroups x 4 "
                          f"waves x 8 independent v_mfma_f32_16x16x32_bf16 chains x {iters} iterations "
                          f"(median of {reps})"}


def keep_busy(call, torch, seconds: float, batch: int = 20) -> int:
    """Untimed calls call(0), call(1), ... for `seconds` (a synchronisation
    after every `batch`): the chip raises its clocks only under sustained
    load. Returns the number of calls."""
    n = 0
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(batch):
            call(n)
            n += 1
        torch.cuda.synchronize()
    return n


def forward_timed(w, s5, torch, warmup: int, steps: int, event_steps: int = 0, device_warmup_s: float = 0.0):
    """Time s5_forward / s5_forward_timevarying on workload w: rotating input
    and output sets (> 512 MB in total, so that the 256 MB Infinity Cache
    cannot serve repeats), `warmup` untimed calls, `steps` calls between two
    synchronisations (wall clock), then per-launch HIP events on `steps` more
    calls, and (event_steps > 0) event pairs around whole calls. With
    device_warmup_s > 0 the wall-clock timing is taken twice: once right after
    the `warmup` calls (returned as cold_wall_ms), then again after calls
    have kept the GPU busy for device_warmup_s seconds and `warmup` more
    calls (wall_ms): the chip raises its clocks only under sustained load, and
    a timed region of a few milliseconds otherwise measures the ramp.
    Returns a dict of timings and the output of the last call."""
    dev = torch.device("cuda:0")
    lam = torch.from_numpy(w.lam).to(dev)
    bt = torch.from_numpy(w.b_tilde).to(dev)
    ct = torch.from_numpy(w.c_tilde).to(dev)
    d = torch.from_numpy(w.d).to(dev)
    logd = torch.from_numpy(w.log_delta).to(dev)
    if w.io == "bf16":
        u0 = torch.from_numpy(w.u_bf16.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        u0 = torch.from_numpy(w.u).to(dev)
    delta0 = torch.from_numpy(w.delta).to(dev) if w.time_varying else None
    set_bytes = u0.numel() * u0.element_size() * 2 + (delta0.numel() * 4 if delta0 is not None else 0)
    n_sets = min(64, max(2, math.ceil(512e6 / set_bytes)))
    us = [u0] + [u0.clone() for _ in range(n_sets - 1)]
    ys = [torch.empty_like(u0) for _ in range(n_sets)]
    deltas = ([delta0] + [delta0.clone() for _ in range(n_sets - 1)]) if delta0 is not None else None

    def step(i):
        k = i % n_sets
        if w.time_varying:
            s5.forward_timevarying(us[k], lam, bt, ct, d, deltas[k], y=ys[k])
        else:
            s5.forward(us[k], lam, bt, ct, d, logd, y=ys[k])
        return k

    i = 0

    def timed_steps():
        nonlocal i
        for _ in range(warmup):
            step(i)
            i += 1
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step(i)
            i += 1
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    cold_wall_ms = None
    warm_calls = 0
    if device_warmup_s > 0:
        cold_wall_ms = timed_steps()
        warm_calls = keep_busy(step, torch, device_warmup_s)
    wall_ms = timed_steps()
    ev = HipEvents()
    evs = [[ev.create() for _ in range(6)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in evs:
        s5.set_profiling_events(e)
        step(i)
        i += 1
    torch.cuda.synchronize()
    s5.set_profiling_events(None)
    launch_ms = np.array([[ev.elapsed_ms(e[2 * k], e[2 * k + 1]) for k in range(3)] for e in evs])
    for e in evs:
        for h in e:
            ev.destroy(h)
    res = {"wall_ms": wall_ms, "cold_wall_ms": cold_wall_ms, "device_warmup_calls": warm_calls,
           "launch_ms": launch_ms, "n_sets": n_sets,
           "set_last": (i - 1) % n_sets, "ys": ys, "step": step, "next": i,
           "params": (lam, bt, ct, d, logd), "us": us, "deltas": deltas}
    if event_steps > 0:
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(event_steps)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(event_steps)]
        for _ in range(10):
            step(i)
            i += 1
        for k in range(event_steps):
            e0[k].record()
            step(i)
            i += 1
            e1[k].record()
        torch.cuda.synchronize()
        call_ms = np.array([a.elapsed_time(b) for a, b in zip(e0, e1)])
        res["call_ms"] = call_ms
        res["set_last"] = (i - 1) % n_sets
    return res


def roofline_fracs(w, k_ms: float, layer_ms: float, peaks: dict):
    """Roofline of the state and output pass (k_scan, time k_ms) and of the
    whole layer (layer_ms): the bound the algorithmic work sets (MFMA: 8*P*H
    flops per token; HBM: u, y, Delta and the parameters once), against the
    vendor peaks and, when given, the rates measured in this run."""
    flops = algorithmic_flops(w)
    nbytes = algorithmic_bytes(w)
    mfma_peak = MFMA_PEAK_TFLOPS[w.io]
    bound = "mfma" if flops / (mfma_peak * 1e12) >= nbytes / (HBM_PEAK_GBS * 1e9) else "hbm"
    tf = flops / (k_ms * 1e-3) / 1e12
    gbs = nbytes / (k_ms * 1e-3) / 1e9
    lgbs = nbytes / (layer_ms * 1e-3) / 1e9
    ltf = flops / (layer_ms * 1e-3) / 1e12
    out = {"bound": bound, "k_scan_us": round(k_ms * 1e3, 2),
           "k_scan_mfma_frac": round(tf / mfma_peak, 4), "k_scan_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
           "layer_us": round(layer_ms * 1e3, 2),
           "layer_hbm_frac": round(lgbs / HBM_PEAK_GBS, 4), "layer_mfma_frac": round(ltf / mfma_peak, 4)}
    if peaks:
        mp, hp = peaks["mfma_bf16_TFLOPs"], peaks["hbm_copy_GBs"]
        out["frac_measured"] = {"k_scan_mfma": round(tf / mp, 4), "k_scan_hbm": round(gbs / hp, 4),
                                "layer_hbm": round(lgbs / hp, 4), "layer_mfma": round(ltf / mp, 4)}
    return out


def measure_config(i: int, s5, torch, wl, peaks: dict, warmup: int, steps: int, device_warmup_s: float) -> dict:
    """One of the other workloads, measured in this run (see the module
    docstring, `configs`)."""
    import oracle.s5_oracle as orc
    w = wl.make_config(i)
    r = forward_timed(w, s5, torch, warmup, steps, device_warmup_s=device_warmup_s)
    mean = r["launch_ms"].mean(axis=0)
    wall = r["wall_ms"]
    yg = r["ys"][r["set_last"]].float().cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    if w.time_varying:
        yo = orc.forward_timevarying(w.u, w.lam, w.b_tilde, w.c_tilde, w.d, w.delta)
    else:
        yo = orc.forward(w.u, w.lam, w.b_tilde, w.c_tilde, w.d, w.log_delta)
    t_orc = time.perf_counter() - t0
    rms = math.sqrt(float(np.mean(yo ** 2)))
    out = {"workload": (f"s5_fwd_{w.name}_B{w.B}_L{w.L}_H{w.H}_P{w.P}_{w.io}"
                        f"{'_timevarying' if w.time_varying else ''}"),
           "ms_per_step": round(wall, 5), "tokens_per_s": round(w.B * w.L / (wall * 1e-3), 1),
           "steps": steps, "buffer_sets": r["n_sets"],
           "ms_per_step_without_device_warmup": (round(r["cold_wall_ms"], 5)
                                                 if r["cold_wall_ms"] is not None else None),
           "kernels": {"pack_us": round(float(mean[0]) * 1e3, 2), "reduce_us": round(float(mean[1]) * 1e3, 2),
                       "scan_us": round(float(mean[2]) * 1e3, 2)},
           "roofline": roofline_fracs(w, float(mean[2]), float(mean.sum()), peaks),
           "parity": {"max_err_over_rms": float(np.max(np.abs(yg - yo)) / rms), "tol": w.tol},
           "oracle_tokens_per_s": round(w.B * w.L / t_orc, 1)}
    del r
    torch.cuda.empty_cache()
    return out


def cpu_baseline(w, repeats: int, budget_s: float):
    import oracle.s5_oracle as orc
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    times = []
    y = None
    for _ in range(repeats):
        t0 = time.perf_counter()
        if w.time_varying:
            y = orc.forward_timevarying(w.u, w.lam, w.b_tilde, w.c_tilde, w.d, w.delta)
        else:
            y = orc.forward(w.u, w.lam, w.b_tilde, w.c_tilde, w.d, w.log_delta)
        times.append(time.perf_counter() - t0)
        if sum(times) > budget_s:
            break
    t = float(np.median(times))
    return {"value": w.B * w.L / t, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"whole workload (B={w.B}, L={w.L}), float64 NumPy, median of {len(times)} "
                      f"run(s), {t:.2f} s each"}, y


def bench_step(args, w, s5, torch, us, lam, bt, ct, d, logd, deltas) -> int:
    """Single recurrent steps (s5_step) for the workload's B sequences: one
    token per sequence per call, the state carried in place."""
    n = 64
    u1 = [us[0][:, k].contiguous() for k in range(n)]
    dl = [deltas[0][:, k].contiguous() for k in range(n)] if w.time_varying else None
    x = torch.zeros(w.B, w.P, dtype=torch.complex64, device=lam.device)
    y = torch.empty_like(u1[0])

    def one(i):
        kw = {"delta": dl[i % n]} if w.time_varying else {"log_delta": logd}
        s5.step(u1[i % n], lam, bt, ct, d, x, y=y, **kw)

    steps = max(args.steps, 200)
    keep_busy(one, torch, args.device_warmup)
    for i in range(args.warmup):
        one(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    # the kernel alone: events on the stream the binding launches on
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(50)]
    e1 = [torch.cuda.Event(enable_timing=True) for _ in range(50)]
    for i in range(50):
        e0[i].record()
        one(i)
        e1[i].record()
    torch.cuda.synchronize()
    k_us = float(np.median([a.elapsed_time(b) for a, b in zip(e0, e1)])) * 1e3
    s_io = 2 if w.io == "bf16" else 4
    nbytes = (8 * w.P + 16 * w.P * w.H + 4 * w.H + 4 * w.P + 2 * w.B * w.H * s_io + 16 * w.B * w.P
              + (4 * w.B * w.P if w.time_varying else 0))
    gbs = nbytes / (k_us * 1e-6) / 1e9
    out = {"metric": "S5 single recurrent step, tokens/s (B per call)", "unit": "tokens/s",
           "value": round(w.B / (ms * 1e-3), 1), "ms_per_step": round(ms, 5), "steps": steps,
           "higher_is_better": True, "dtype": w.io, "data": "synthetic",
           "config": {"workload": f"s5_step_B{w.B}_H{w.H}_P{w.P}_{w.io}"
                                  f"{'_timevarying' if w.time_varying else ''}", "variant": "step"},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 5), "traffic": None, "kernel": "k_step",
                        "kernel_us": round(k_us, 2), "per_launch": {"bytes": nbytes}}}
    if not args.no_cpu_baseline:
        import oracle.s5_oracle as orc
        kw = {"delta": w.delta[:, :1]} if w.time_varying else {"log_delta": w.log_delta}
        x0 = np.zeros((w.B, w.P), np.complex128)
        u1 = w.u[:, :1]
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(args.cpu_budget, 5.0):
            orc.forward_ex(u1, w.lam, w.b_tilde, w.c_tilde, w.d, x0=x0, **kw)
            reps += 1
        t = (time.perf_counter() - t0) / reps
        out["cpu_baseline"] = {"value": w.B / t, "unit": "tokens/s", "cores": _blas_threads(), "kind": "oracle",
                               "sample": f"one step of B={w.B} sequences (oracle forward_ex, L = 1), "
                                         f"{reps} repetitions, {t * 1e3:.2f} ms each"}
    print(json.dumps(out), flush=True)
    return 0


def bench_glu(args, w, s5, torch, us, ys, n_sets) -> int:
    """The gated activation (s5_glu, variant 1 or 2 from "glu" / "glu2") over
    the workload's B*L tokens of H features (the layer output's shape), with
    a dense W ~ N(0, 1/H) and a bias; HBM-bound: y in, out written."""
    variant = 2 if args.variant == "glu2" else 1
    rng = np.random.default_rng(7)
    wmat = (rng.normal(size=(w.H, w.H)) / math.sqrt(w.H)).astype(np.float32)
    bias = (rng.normal(size=w.H) * 0.5).astype(np.float32)
    wd = torch.from_numpy(wmat).cuda()
    bd = torch.from_numpy(bias).cuda()
    yin = [u.view(-1, w.H) for u in us]
    outs = [y.view(-1, w.H) for y in ys]

    def one(i):
        k = i % n_sets
        s5.glu(yin[k], wd, bd, variant, out=outs[k])

    keep_busy(one, torch, args.device_warmup)
    for i in range(args.warmup):
        one(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one(args.warmup + i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    e1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        e0[i].record()
        one(i)
        e1[i].record()
    torch.cuda.synchronize()
    k_us = float(np.mean([a.elapsed_time(b) for a, b in zip(e0, e1)])) * 1e3
    T = w.B * w.L
    s_io = 2 if w.io == "bf16" else 4
    nbytes = 2 * T * w.H * s_io + 4 * w.H * w.H + 4 * w.H
    gbs = nbytes / (k_us * 1e-6) / 1e9
    out = {"metric": "S5 gated activation tokens/s (B*L tokens of H features)", "unit": "tokens/s",
           "value": round(T / (ms * 1e-3), 1), "ms_per_step": round(ms, 5), "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "dtype": w.io, "data": "synthetic",
           "config": {"workload": f"s5_glu{variant}_T{T}_H{w.H}_{w.io}", "variant": args.variant},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "k_glu",
                        "kernel_us": round(k_us, 2), "per_launch": {"bytes": nbytes, "flops": 2 * T * w.H * w.H}}}
    if not args.no_cpu_baseline:
        import oracle.s5_oracle as orc
        yv = w.u.reshape(-1, w.H)
        times = []
        while not times or (sum(times) < args.cpu_budget and len(times) < 10):
            t1 = time.perf_counter()
            orc.glu(yv, wmat, bias, variant)
            times.append(time.perf_counter() - t1)
        t = float(np.median(times))
        out["cpu_baseline"] = {"value": T / t, "unit": "tokens/s", "cores": _blas_threads(), "kind": "oracle",
                               "sample": f"whole workload ({T} tokens), oracle glu, float64 NumPy, median of "
                                         f"{len(times)} run(s), {t:.2f} s each"}
    print(json.dumps(out), flush=True)
    return 0


def bench_variant(args, w, s5, torch, us, ys, deltas, lam, bt, ct, d, logd, n_sets) -> int:
    """Time one option of s5_forward_ex, or chunked streaming, on the workload."""
    v = args.variant
    B, P = w.B, w.P
    x0 = torch.zeros(B, P, dtype=torch.complex64, device=lam.device)
    xl = torch.empty_like(x0)
    if v == "bidir":
        ct_run = torch.cat([ct, ct.conj()], dim=1).contiguous()
    else:
        ct_run = ct
    opts = {"stateful": {}, "half": {"half_spectrum": True}, "bilinear": {"bilinear": True},
            "gelu": {"gelu": True}, "bidir": {"bidirectional": True}}
    if v == "gated":
        # the gated activation (variant 1, with bias) in the same call
        gw, gb = gate_params(w.H)
        opts["gated"] = {"glu_w": torch.from_numpy(gw).to(lam.device),
                         "glu_bias": torch.from_numpy(gb).to(lam.device), "glu_variant": 1}
    chunk = int(v.split(":")[1]) if v.startswith("chunked:") else 0
    if v == "step":
        return bench_step(args, w, s5, torch, us, lam, bt, ct, d, logd, deltas)
    if v.startswith("glu"):
        return bench_glu(args, w, s5, torch, us, ys, n_sets)
    if chunk:
        if w.L % chunk:
            print("chunk must divide L", file=sys.stderr)
            return 2
        n_ck = w.L // chunk
        ucs = [[us[k][:, j * chunk:(j + 1) * chunk].contiguous() for j in range(n_ck)] for k in range(n_sets)]
        ycs = [[torch.empty_like(ucs[0][0]) for _ in range(n_ck)] for _ in range(n_sets)]
        dcs = ([[deltas[k][:, j * chunk:(j + 1) * chunk].contiguous() for j in range(n_ck)]
                for k in range(n_sets)] if w.time_varying else None)
        xs = [x0, xl]
    elif v not in opts:
        print(f"unknown variant {v}", file=sys.stderr)
        return 2

    def step(i):
        k = i % n_sets
        if chunk:
            for j in range(n_ck):
                kw = {"delta": dcs[k][j]} if w.time_varying else {"log_delta": logd}
                s5.forward_ex(ucs[k][j], lam, bt, ct, d, x0=xs[j & 1], x_last=xs[(j + 1) & 1],
                              y=ycs[k][j], **kw)
            return
        kw = {"delta": deltas[k]} if w.time_varying else {"log_delta": logd}
        extra = {"x0": x0, "x_last": xl} if v == "stateful" else {}
        s5.forward_ex(us[k], lam, bt, ct_run, d, y=ys[k], **kw, **extra, **opts[v])

    keep_busy(step, torch, args.device_warmup)   # as for the default line
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # HIP events around every launch of one call (chunked: the last call of
    # the step): packing, aggregate pass, state and output pass, and for the
    # bidirectional form the same three for the backward scan
    nl = 6 if v == "bidir" else 3
    ev = HipEvents()
    evs = [[ev.create() for _ in range(2 * nl)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        s5.set_profiling_events(evs[i])
        step(args.warmup + args.steps + i)
    torch.cuda.synchronize()
    s5.set_profiling_events(None)
    ms = np.array([[ev.elapsed_ms(e[2 * k], e[2 * k + 1]) for k in range(nl)] for e in evs]).mean(axis=0)
    for e in evs:
        for h in e:
            ev.destroy(h)
    names = ["pack_us", "reduce_us", "scan_us", "back_pack_us", "back_reduce_us", "back_scan_us"]
    kernels = {names[k]: round(float(ms[k]) * 1e3, 2) for k in range(nl)}
    # dominant kernel: the (slower) state and output pass; its algorithmic
    # work is 8 P H flops per token of the call
    k_dom = 5 if v == "bidir" and ms[5] > ms[2] else 2
    tokens_call = w.B * (chunk if chunk else w.L)
    flops = 8 * w.P * w.H * tokens_call
    achieved = flops / (float(ms[k_dom]) * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[w.io]
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": None,
            "kernel": "k_scan (backward scan)" if k_dom == 5 else "k_scan",
            "kernel_us": round(float(ms[k_dom]) * 1e3, 2), "per_launch": {"flops": flops}}
    workload = (f"s5_fwd_{w.name}_B{w.B}_L{w.L}_H{w.H}_P{w.P}_{w.io}"
                f"{'_timevarying' if w.time_varying else ''}")
    out = {"metric": METRIC, "value": round(w.B * w.L / (ms_per_step * 1e-3), 1),
           "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": w.io, "data": "synthetic",
           "config": {"workload": workload, "variant": v, "buffer_sets": n_sets},
           "roofline": roof, "kernels": kernels}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_variant(w, v, ct_run, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


def gate_params(H: int):
    """Seeded W [H, H] ~ N(0, 1/H) and bias ~ N(0, 1/4) of the gated activation, float32."""
    rng = np.random.default_rng(7)
    return ((rng.normal(size=(H, H)) / math.sqrt(H)).astype(np.float32),
            (0.5 * rng.normal(size=H)).astype(np.float32))


def cpu_baseline_variant(w, v, ct_run, budget_s: float):
    """The oracle's forward_ex with the variant's options on the whole
    workload (chunked: one call over the whole sequence, as the chunks carry
    the state exactly), median of runs within the budget."""
    import oracle.s5_oracle as orc
    c = ct_run.cpu().numpy() if v == "bidir" else w.c_tilde
    kw = {"delta": w.delta} if w.time_varying else {"log_delta": w.log_delta}
    opts = {"half": {"conj_sym": True}, "bilinear": {"method": "bilinear"}, "gelu": {"activation": "gelu"},
            "bidir": {"bidirectional": True}}.get(v, {})
    if v == "stateful" or v.startswith("chunked:"):
        kw["x0"] = np.zeros((w.B, w.P), np.complex128)
    gate = gate_params(w.H) if v == "gated" else None
    times = []
    while not times or (sum(times) < budget_s and len(times) < 25):
        t0 = time.perf_counter()
        y, _ = orc.forward_ex(w.u, w.lam, w.b_tilde, c, w.d, **kw, **opts)
        if gate is not None:
            orc.glu(y, gate[0], gate[1], 1)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": w.B * w.L / t, "unit": "tokens/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"whole workload (B={w.B}, L={w.L}), oracle forward_ex with the variant's options, "
                      f"float64 NumPy, median of {len(times)} run(s), {t:.2f} s each"}


def _blas_threads() -> int:
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        return int(max([i.get("num_threads", 1) for i in info] or [1]))
    except Exception:
        return len(os.sched_getaffinity(0))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=CONFIG_INDEX)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-repeats", type=int, default=40)
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--variant", default="plain",
                    help="plain | stateful | half | bilinear | gelu | bidir | gated | chunked:C | step | glu | glu2")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run plain device copies of MIB MiB (counter calibration)")
    ap.add_argument("--other-configs", default="0,1,2,4",
                    help="workloads measured beside the main one (comma list; empty for none)")
    ap.add_argument("--event-steps", type=int, default=100,
                    help="calls timed one by one with a HIP event pair (median reported)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the in-run peak-rate probes")
    ap.add_argument("--device-warmup", type=float, default=0.5, metavar="SECONDS",
                    help="keep the GPU busy with untimed calls this long before the warm-up and timed "
                         "steps (0: none); the timing without it is reported beside")
    args = ap.parse_args()
    if args.calibrate_copy:
        return calibrate_copy(args.calibrate_copy, 5)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the S5 forward path here runs on a single "
              "MI355X; batch sharding across GPUs needs no communication and is not "
              "benchmarked. Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    import diagonal_state_space_amd as s5
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    w = wl.make_config(args.config)
    print(f"[bench] workload {w.name}: B={w.B} L={w.L} H={w.H} P={w.P} io={w.io} "
          f"tv={w.time_varying}", file=sys.stderr, flush=True)

    if args.variant != "plain":
        # parameters (shared) and rotating input/output sets (> 512 MB in total)
        lam = torch.from_numpy(w.lam).to(dev)
        bt = torch.from_numpy(w.b_tilde).to(dev)
        ct = torch.from_numpy(w.c_tilde).to(dev)
        d = torch.from_numpy(w.d).to(dev)
        logd = torch.from_numpy(w.log_delta).to(dev)
        if w.io == "bf16":
            u0 = torch.from_numpy(w.u_bf16.view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            u0 = torch.from_numpy(w.u).to(dev)
        delta0 = torch.from_numpy(w.delta).to(dev) if w.time_varying else None
        set_bytes = u0.numel() * u0.element_size() * 2 + (delta0.numel() * 4 if delta0 is not None else 0)
        n_sets = max(4, math.ceil(512e6 / set_bytes))
        us = [u0] + [u0.clone() for _ in range(n_sets - 1)]
        ys = [torch.empty_like(u0) for _ in range(n_sets)]
        deltas = ([delta0] + [delta0.clone() for _ in range(n_sets - 1)]) if delta0 is not None else None
        return bench_variant(args, w, s5, torch, us, ys, deltas, lam, bt, ct, d, logd, n_sets)

    peaks = {}
    if not args.no_peaks:
        print("[bench] measuring the chip's peak rates (copy, MFMA loop)", file=sys.stderr, flush=True)
        peaks = PeakProbes().measure(torch)

    # warm-up, K timed calls (wall clock), K calls with per-launch events,
    # then calls timed one by one with event pairs
    r = forward_timed(w, s5, torch, args.warmup, args.steps, args.event_steps, args.device_warmup)
    launch_ms = r["launch_ms"]
    kernel_ms = launch_ms[:, 2]
    ms_per_step = r["wall_ms"]
    n_sets = r["n_sets"]
    ys = r["ys"]
    tokens = w.B * w.L
    value = tokens / (ms_per_step * 1e-3)
    k_ms = float(np.mean(kernel_ms))
    mean_ms = launch_ms.mean(axis=0)
    flops = algorithmic_flops(w)
    nbytes = algorithmic_bytes(w)
    mfma_peak = MFMA_PEAK_TFLOPS[w.io]
    achieved_tf = flops / (k_ms * 1e-3) / 1e12
    mfma_floor = flops / (mfma_peak * 1e12)
    hbm_floor = nbytes / (HBM_PEAK_GBS * 1e9)
    bound = "mfma" if mfma_floor >= hbm_floor else "hbm"
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(achieved_tf, 2), "peak": mfma_peak,
                "unit": "TFLOP/s", "frac": round(achieved_tf / mfma_peak, 4), "traffic": None}
        if peaks:
            roof["frac_measured"] = round(achieved_tf / peaks["mfma_bf16_TFLOPs"], 4)
    else:
        a_gbs = nbytes / (k_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(a_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(a_gbs / HBM_PEAK_GBS, 4), "traffic": None}
        if peaks:
            roof["frac_measured"] = round(a_gbs / peaks["hbm_copy_GBs"], 4)
    workload = (f"s5_fwd_{w.name}_B{w.B}_L{w.L}_H{w.H}_P{w.P}_{w.io}"
                f"{'_timevarying' if w.time_varying else ''}")
    roof["traffic"] = measured_traffic(workload)
    roof["kernel"] = "k_scan"
    roof["kernel_us"] = round(k_ms * 1e3, 2)
    roof["per_launch"] = {"flops": flops, "bytes": nbytes}
    kernels = {"pack_us": round(float(mean_ms[0]) * 1e3, 2),
               "reduce_us": round(float(mean_ms[1]) * 1e3, 2),
               "scan_us": round(float(mean_ms[2]) * 1e3, 2),
               "reduce_flops": flops // 2}
    fwd_ms = float(mean_ms.sum())
    achieved_gbs = nbytes / (fwd_ms * 1e-3) / 1e9
    hbm = {"achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "over": "pack + reduce + scan"}
    if peaks:
        hbm["frac_measured"] = round(achieved_gbs / peaks["hbm_copy_GBs"], 4)
    call_ms = r.get("call_ms")

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.io,
        "data": "synthetic",
        "config": {"workload": workload,
                   "B": w.B, "L": w.L, "H": w.H, "P": w.P, "io": w.io,
                   "time_varying": w.time_varying, "buffer_sets": n_sets},
        "roofline": roof,
        "kernels": kernels,
        "hbm": hbm,
    }
    if r["cold_wall_ms"] is not None:
        out["device_warmup"] = {"s": args.device_warmup, "calls": r["device_warmup_calls"],
                                "ms_per_step_without": round(r["cold_wall_ms"], 5)}
    if call_ms is not None:
        out["step_events"] = {"median_us": round(float(np.median(call_ms)) * 1e3, 2),
                              "mean_us": round(float(np.mean(call_ms)) * 1e3, 2),
                              "calls": int(call_ms.size), "warmup": 10}
    if peaks:
        out["peaks_measured"] = peaks
    yg_main = ys[r["set_last"]].float().cpu().numpy().astype(np.float64)
    del r, ys
    torch.cuda.empty_cache()
    others = [int(c) for c in args.other_configs.split(",") if c.strip() != ""]
    if others:
        out["configs"] = {}
        for c in others:
            if c == args.config:
                continue
            print(f"[bench] workload {c} (in-run measurement)", file=sys.stderr, flush=True)
            out["configs"][str(c)] = measure_config(c, s5, torch, wl, peaks, 20, max(args.steps, 100), args.device_warmup)

    if not args.no_cpu_baseline:
        print("[bench] timing the float64 oracle on the host", file=sys.stderr, flush=True)
        cb, yo = cpu_baseline(w, args.cpu_repeats, args.cpu_budget)
        out["cpu_baseline"] = cb
        rms = math.sqrt(float(np.mean(yo ** 2)))
        out["parity"] = {"max_err_over_rms": float(np.max(np.abs(yg_main - yo)) / rms), "tol": w.tol}
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
