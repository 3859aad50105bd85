"""Chunked closed form of the gated delta rule, fp64 numpy (TEST INFRASTRUCTURE).

A self-check of the serial oracle only: the tests require this and the serial
loop in ``gdn_oracle.c`` to agree. Nothing on the product path imports it.

What it follows: the chunked evaluation of "GDN & MLA Mechanism Deep-Dive",
Math derivation Step 5 (fixed-length chunks of 64 tokens, the inside of a
chunk solved at once through a small square matrix, the state handed from
one chunk to the next). The pages leave the in-chunk solution unspecified;
the one written out here is the WY/UT form of the Gated Delta Net paper that
page cites (Yang et al. 2024), for one chunk of n rows with start state h:

    lam_r   = g_r * A                       (A = -exp(A_log))
    gam_i   = sum_{r <= i} lam_r            (restarted at every chunk)
    Gam_ij  = exp(gam_i - gam_j) for i >= j, else 0
    L       = strictly-lower part of diag(beta) (K K^T o Gam)
    Tm      = (I + L)^{-1}
    U       = Tm diag(beta) V
    Kw      = Tm diag(beta * exp(gam)) K
    W       = U - Kw h
    O       = diag(exp(gam)) Q h + ((Q K^T) o Gam) W
    h_next  = exp(gam_n) h + (diag(exp(gam_n - gam)) K)^T W

With the delta term off, W = diag(beta) V directly (L = 0, Kw = 0).
"""
from __future__ import annotations

import numpy as np


def fwd_chunked(q, k, v, g, beta, A_log, h0=None, delta=True, chunk=64):
    q, k, v, g, beta, A_log = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta, A_log))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    hT = np.zeros((B, H, dk, dv))
    for b in range(B):
        for hh in range(H):
            A = -np.exp(A_log[hh])
            h = np.zeros((dk, dv)) if h0 is None else np.array(h0[b, hh], dtype=np.float64)
            for c0 in range(0, T, chunk):
                c1 = min(T, c0 + chunk)
                n = c1 - c0
                Q = q[b, c0:c1, hh]
                K = k[b, c0:c1, hh]
                V = v[b, c0:c1, hh]
                bet = beta[b, c0:c1, hh]
                gam = np.cumsum(g[b, c0:c1, hh] * A)
                diff = gam[:, None] - gam[None, :]
                low = np.tril(np.ones((n, n), dtype=bool))
                Gam = np.where(low, np.exp(np.where(low, diff, 0.0)), 0.0)
                if delta:
                    L = np.tril(bet[:, None] * (K @ K.T) * Gam, -1)
                    Tm = np.linalg.inv(np.eye(n) + L)
                    U = Tm @ (bet[:, None] * V)
                    Kw = Tm @ ((bet * np.exp(gam))[:, None] * K)
                    W = U - Kw @ h
                else:
                    W = bet[:, None] * V
                o[b, c0:c1, hh] = np.exp(gam)[:, None] * (Q @ h) + ((Q @ K.T) * Gam) @ W
                h = np.exp(gam[-1]) * h + (np.exp(gam[-1] - gam)[:, None] * K).T @ W
            hT[b, hh] = h
    return o, hT
