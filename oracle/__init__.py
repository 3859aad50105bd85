"""fp64 CPU oracle for the gated delta rule (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP library
(``gated_delta_rule_74_amd``) and never imports it.

The arithmetic lives in ``gdn_oracle.c`` (serial loops in IEEE double, see its
header for the definitions and where the pages state them); this module only
marshals numpy arrays. ``chunked.py`` holds the chunk-64 closed form, used as a
self-check of the serial loop, never by the product.

Parity status of each function:
  fwd  - pinned (brute-force sums, closed forms, invariants, chunked form,
         hand-worked fixture; see tests/test_oracle_pins.py)
  bwd  - pinned by central finite differences of fwd and the dA_log identity
  step - pinned against fwd (a chain of steps equals one forward pass)
  gates_from_logits, logit_grads - the sigmoid of the gate logits and the
         chain rule through it; pinned by central finite differences of fwd
         composed with gates_from_logits (tests/test_oracle_grad.py)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O3 keeps IEEE semantics: no fast-math,
    no FMA contraction, so every sum runs in source order)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O3", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-shared",
               "-fPIC", "-pthread", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.gdn_oracle_fwd.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, I, P, P, P, I, I]
        lib.gdn_oracle_bwd.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P, I, P, P, P, P, P,
                                       P, P, P, I, I]
        lib.gdn_oracle_step.argtypes = [I, I, I, I, P, P, P, P, P, P, P, I, P, P, I]
        for f in (lib.gdn_oracle_fwd, lib.gdn_oracle_bwd, lib.gdn_oracle_step):
            f.restype = I
        _lib = lib
    return _lib


def default_threads() -> int:
    """Cores this process may use: its affinity mask, capped by
    OMP_NUM_THREADS when that is set (a host's CPU share per job)."""
    try:
        n = max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return n


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    return None if x is None else x.ctypes.data


def _units(units):
    if units is None:
        return None, 0
    u = np.ascontiguousarray(np.asarray(units, dtype=np.int32))
    return u, int(u.size)


def fwd(q, k, v, g, beta, A_log, h0=None, delta=True, units=None, nthreads=None):
    """Serial forward. q,k [B,T,H,dk]; v [B,T,H,dv]; g,beta [B,T,H]; A_log [H];
    h0 [B,H,dk,dv] or None. Returns (o [B,T,H,dv], hT [B,H,dk,dv]) in float64.
    ``units`` (list of b*H+h) restricts the work; other units stay zero."""
    q, k, v, g, beta, A_log, h0 = map(_f64, (q, k, v, g, beta, A_log, h0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    hT = np.zeros((B, H, dk, dv))
    u, nu = _units(units)
    rc = _load().gdn_oracle_fwd(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(A_log), _ptr(h0), int(bool(delta)), _ptr(o), _ptr(hT),
                                _ptr(u), nu, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_fwd failed ({rc})")
    return o, hT


def bwd(q, k, v, g, beta, A_log, h0, do, dhT=None, delta=True, units=None, nthreads=None):
    """Manual reverse pass. Returns a dict with dq, dk, dv, dg, dbeta, dA_log
    [H] (summed over the computed units), dA_log_part [B,H] and dh0."""
    q, k, v, g, beta, A_log, h0, do, dhT = map(_f64, (q, k, v, g, beta, A_log, h0, do, dhT))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               dg=np.zeros_like(g), dbeta=np.zeros_like(beta), dA_log_part=np.zeros((B, H)),
               dh0=np.zeros((B, H, dk, dv)))
    u, nu = _units(units)
    rc = _load().gdn_oracle_bwd(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(A_log), _ptr(h0), _ptr(do), _ptr(dhT), int(bool(delta)),
                                _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                                _ptr(out["dbeta"]), _ptr(out["dA_log_part"]), _ptr(out["dh0"]),
                                _ptr(u), nu, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_bwd failed ({rc})")
    part = out["dA_log_part"]
    dA = np.zeros(H)
    for b in range(B):  # fixed order
        dA += part[b]
    out["dA_log"] = dA
    return out


def step(q, k, v, g, beta, A_log, h_in=None, delta=True, nthreads=None):
    """One token per sequence. q,k [N,H,dk]; v [N,H,dv]; g,beta [N,H];
    h_in [N,H,dk,dv] or None. Returns (o [N,H,dv], h_out [N,H,dk,dv])."""
    q, k, v, g, beta, A_log, h_in = map(_f64, (q, k, v, g, beta, A_log, h_in))
    N, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((N, H, dv))
    h_out = np.zeros((N, H, dk, dv))
    rc = _load().gdn_oracle_step(N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(A_log), _ptr(h_in), int(bool(delta)), _ptr(o), _ptr(h_out),
                                 nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_step failed ({rc})")
    return o, h_out


def gates_from_logits(x):
    """Gate values from logits: the logistic sigmoid 1 / (1 + e^-x) in
    float64 (the gate of "GDN & MLA Mechanism Deep-Dive", Step 4, is
    g = sigmoid(dt_proj(x)); the write gate beta is formed the same way)."""
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def logit_grads(d_gate, gate):
    """Gradient with respect to a logit from the gradient with respect to its
    gate value s = sigmoid(x): ds/dx = s (1 - s)."""
    gate = np.asarray(gate, dtype=np.float64)
    return np.asarray(d_gate, dtype=np.float64) * gate * (1.0 - gate)
