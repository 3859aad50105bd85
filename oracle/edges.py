"""fp64 layer edges around the recurrence (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; it shares no code with the HIP library.

Two steps that sit on either side of the gated delta rule in the GDN layer,
written as plain compositions around the serial oracle (``oracle.fwd`` /
``oracle.bwd``), each with its own derivative:

* per-token L2 normalisation of the keys: the write/erase key of the delta
  rule is a unit vector (the erase is then a projection; "GDN & MLA Mechanism
  Deep-Dive", Step 3 and Step 4, and the unit-norm key of the workload
  recipe). Per (b, t, h) row, k_hat = k / sqrt(sum_j k_j^2 + EPS), EPS = 1e-6
  (the plain reading: the norm of the row, kept away from zero by a fixed
  epsilon under the square root). Its reverse:
  dk = (dk_hat - k_hat (k_hat . dk_hat)) / sqrt(sum_j k_j^2 + EPS).
* the per-head skip term D of the layer's recurrence parameters (HyMo README,
  Architecture: the GDN recurrence is initialised with A_log, dt_bias and D),
  read as o_t += D_h v_t; its reverse adds D_h do_t to dv_t and gives
  dD_h = sum over batch, tokens and value columns of do * v.

Parity status: pinned by central finite differences of the composed forward
for every input, D included, and by the invariances in
tests/test_oracle_edges.py (scale invariance of the normalised keys, the
gradient's orthogonality to k, D = 0 reducing to the plain recurrence).
"""
from __future__ import annotations

import numpy as np

from . import bwd as _bwd
from . import fwd as _fwd

EPS = 1e-6


def l2norm_keys(k):
    """k_hat = k / sqrt(sum_j k_j^2 + EPS) for every row of the last axis."""
    k = np.asarray(k, dtype=np.float64)
    n = np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + EPS)
    return k / n


def l2norm_keys_grad(k, dk_hat):
    """Gradient with respect to k of sum(dk_hat * l2norm_keys(k))."""
    k = np.asarray(k, dtype=np.float64)
    dk_hat = np.asarray(dk_hat, dtype=np.float64)
    n = np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + EPS)
    kh = k / n
    return (dk_hat - kh * np.sum(kh * dk_hat, axis=-1, keepdims=True)) / n


def fwd(q, k, v, g, beta, A_log, h0=None, D=None, norm_k=False, delta=True, nthreads=None):
    """Forward of the recurrence with its edges: keys normalised first when
    norm_k, then o_t += D_h v_t when D [H] is given."""
    kk = l2norm_keys(k) if norm_k else k
    o, hT = _fwd(q, kk, v, g, beta, A_log, h0, delta=delta, nthreads=nthreads)
    if D is not None:
        o = o + np.asarray(D, np.float64)[None, None, :, None] * np.asarray(v, np.float64)
    return o, hT


def bwd(q, k, v, g, beta, A_log, h0, do, dhT=None, D=None, norm_k=False, delta=True, nthreads=None):
    """Reverse of fwd(): the oracle's reverse pass at the normalised keys,
    dk taken back through the normalisation, and the skip's terms (dv +=
    D_h do, dD [H]) when D is given."""
    kk = l2norm_keys(k) if norm_k else k
    r = _bwd(q, kk, v, g, beta, A_log, h0, do, dhT, delta=delta, nthreads=nthreads)
    if norm_k:
        r["dk"] = l2norm_keys_grad(k, r["dk"])
    if D is not None:
        do64 = np.asarray(do, np.float64)
        v64 = np.asarray(v, np.float64)
        r["dv"] = r["dv"] + np.asarray(D, np.float64)[None, None, :, None] * do64
        r["dD"] = np.sum(do64 * v64, axis=(0, 1, 3))
    return r
