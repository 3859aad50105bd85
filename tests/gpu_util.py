"""Shared helpers for the GPU parity tests: move seeded host inputs to the
device and compare device outputs with oracle values."""
import sys

import numpy as np
import torch

import gdn_inputs as gi

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x, device="cuda"):
    if x is None:
        return None
    if isinstance(x, gi.Tensor):
        if x.dtype == "bf16":
            return torch.from_numpy(x.data.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(x.data).to(device)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def f64(x):
    if x is None:
        return None
    if isinstance(x, gi.Tensor):
        return x.f64()
    return np.asarray(x, dtype=np.float64)


def relerr(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    scale = np.max(np.abs(ref))
    if scale == 0.0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / scale)


def assert_close(name, got, ref, tol):
    err = relerr(got, ref)
    say(f"    {name}: rel err {err:.3e} (tol {tol:g})")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert err <= tol, f"{name}: rel err {err:.3e} > {tol:g}"
