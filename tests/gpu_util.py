"""Helpers for the GPU parity tests (device upload, error metric, tolerances)."""
import sys

import numpy as np

import synth

TOL = {"f32": 1e-4, "bf16": 2e-2}


def torch():
    import torch as _t
    return _t


def note(msg):
    """Name the case on stdout before a GPU step (survives a crash of the step)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(t, device="cuda:0"):
    """synth.Tensor (or float32 ndarray) -> device tensor in storage precision."""
    T = torch()
    if isinstance(t, synth.Tensor):
        if t.dtype == "bf16":
            return T.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).to(device).view(T.bfloat16)
        return T.from_numpy(np.ascontiguousarray(t.f32)).to(device)
    return T.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).to(device)


def dev_bf16_from_f32(a, device="cuda:0"):
    return dev(synth.Tensor(a, "bf16", synth.round_to_bf16_bits(a)), device)


def host(t):
    T = torch()
    return t.detach().to(T.float32).cpu().numpy().astype(np.float64)


def empty(shape, dtype, device="cuda:0", fill=None):
    T = torch()
    td = {"bf16": T.bfloat16, "f32": T.float32}[dtype]
    x = T.empty(shape, dtype=td, device=device)
    if fill is not None:
        x.fill_(fill)
    return x


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    return float(np.max(np.abs(gpu - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def assert_close(gpu, ref, dtype, what):
    e = rel_err(gpu, ref)
    tol = TOL[dtype]
    assert e <= tol, f"{what}: max rel err {e:.3e} > {tol:.0e}"
    return e
