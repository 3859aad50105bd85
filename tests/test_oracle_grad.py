"""Pins of the oracle's manual reverse pass: central finite differences of the
oracle's forward for every input (q, k, v, g, beta, A_log, h0) with both
upstream gradients (do, dhT) non-zero, and the dA_log identity."""
import math

import numpy as np
import pytest


def _inputs(seed, B=2, T=9, H=2, dk=3, dv=2, weak=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    lo, hi = (math.log(1e-2), math.log(0.5)) if weak else (0.0, math.log(16.0))
    A_log = rng.uniform(lo, hi, H)
    h0 = rng.standard_normal((B, H, dk, dv))
    do = rng.standard_normal((B, T, H, dv))
    dhT = rng.standard_normal((B, H, dk, dv))
    return dict(q=q, k=k, v=v, g=g, beta=beta, A_log=A_log, h0=h0), do, dhT


def _loss(oracle_mod, x, do, dhT, delta):
    o, hT = oracle_mod.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["h0"],
                           delta=delta, nthreads=1)
    return float(np.sum(o * do) + np.sum(hT * dhT))


@pytest.mark.parametrize("delta", [True, False])
@pytest.mark.parametrize("weak", [True, False])
def test_reverse_pass_matches_central_differences(oracle_mod, delta, weak):
    x, do, dhT = _inputs(20 + int(delta) + 2 * int(weak), weak=weak)
    gr = oracle_mod.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["h0"], do, dhT,
                        delta=delta, nthreads=1)
    names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", A_log="dA_log", h0="dh0")
    eps = 1e-6
    for name, gname in names.items():
        base = x[name]
        fd = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = {kk: vv.copy() for kk, vv in x.items()}
            xp[name][idx] += eps
            lp = _loss(oracle_mod, xp, do, dhT, delta)
            xp[name][idx] -= 2 * eps
            lm = _loss(oracle_mod, xp, do, dhT, delta)
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(fd - gr[gname]))
        scale = max(1.0, np.max(np.abs(fd)))
        assert err < 1e-7 * scale, (name, err, scale)


def test_dA_log_equals_sum_g_dg(oracle_mod):
    """A = -exp(A_log) gives dA/dA_log = A, and lambda_t = g_t A gives
    dg_t = A dlambda_t, so dA_log[h] = sum_{b,t} g_t dg_t exactly."""
    x, do, dhT = _inputs(30, B=3, T=70, H=2, dk=4, dv=3)
    gr = oracle_mod.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["h0"], do, dhT)
    ref = np.sum(x["g"] * gr["dg"], axis=(0, 1))
    assert np.max(np.abs(ref - gr["dA_log"])) < 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_reverse_pass_over_many_checkpoint_segments(oracle_mod):
    """T spans several 64-token recompute segments; the gradient must equal a
    finite difference in a few sampled coordinates."""
    x, do, dhT = _inputs(31, B=1, T=150, H=1, dk=3, dv=2)
    gr = oracle_mod.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["h0"], do, dhT,
                        nthreads=1)
    eps = 1e-6
    for name, gname, idx in [("k", "dk", (0, 3, 0, 1)), ("v", "dv", (0, 100, 0, 0)),
                             ("g", "dg", (0, 64, 0)), ("beta", "dbeta", (0, 127, 0)),
                             ("q", "dq", (0, 149, 0, 2)), ("h0", "dh0", (0, 0, 1, 1))]:
        xp = {kk: vv.copy() for kk, vv in x.items()}
        xp[name][idx] += eps
        lp = _loss(oracle_mod, xp, do, dhT, True)
        xp[name][idx] -= 2 * eps
        lm = _loss(oracle_mod, xp, do, dhT, True)
        fd = (lp - lm) / (2 * eps)
        assert abs(fd - gr[gname][idx]) < 1e-7 * max(1.0, abs(fd)), (name, fd, gr[gname][idx])


def test_reverse_pass_thread_count_invariant(oracle_mod):
    x, do, dhT = _inputs(32, B=3, T=40, H=3, dk=4, dv=4)
    a = oracle_mod.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["h0"], do, dhT,
                       nthreads=1)
    b = oracle_mod.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["h0"], do, dhT,
                       nthreads=5)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("delta", [True, False])
def test_logit_gradients_match_central_differences(oracle_mod, delta):
    """Gates given as logits: the forward composed with the sigmoid, and the
    reverse pass composed with the chain rule through it, against central
    differences of the composed loss with respect to the logits (delta rule
    and additive form)."""
    x, do, dhT = _inputs(40, T=7)
    rng = np.random.default_rng(41)
    gl = rng.standard_normal(x["g"].shape) * 2.0
    bl = rng.standard_normal(x["beta"].shape) * 2.0

    def loss(gl_, bl_):
        xx = dict(x, g=oracle_mod.gates_from_logits(gl_), beta=oracle_mod.gates_from_logits(bl_))
        return _loss(oracle_mod, xx, do, dhT, delta)

    gs, bs = oracle_mod.gates_from_logits(gl), oracle_mod.gates_from_logits(bl)
    gr = oracle_mod.bwd(x["q"], x["k"], x["v"], gs, bs, x["A_log"], x["h0"], do, dhT, delta=delta, nthreads=1)
    dgl = oracle_mod.logit_grads(gr["dg"], gs)
    dbl = oracle_mod.logit_grads(gr["dbeta"], bs)
    eps = 1e-6
    for arr, ana, which in ((gl, dgl, "g"), (bl, dbl, "beta")):
        fd = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += eps
            a2[idx] -= eps
            lp = loss(a1, bl) if which == "g" else loss(gl, a1)
            lm = loss(a2, bl) if which == "g" else loss(gl, a2)
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(fd - ana))
        assert err < 1e-7 * max(1.0, np.max(np.abs(fd))), (which, err)
    # the sigmoid itself: sigmoid(0) = 1/2, symmetric, and matches tanh's identity
    z = np.linspace(-8, 8, 33)
    assert oracle_mod.gates_from_logits(0.0) == 0.5
    assert np.allclose(oracle_mod.gates_from_logits(z) + oracle_mod.gates_from_logits(-z), 1.0, atol=0, rtol=1e-15)
    assert np.allclose(oracle_mod.gates_from_logits(z), 0.5 * (1.0 + np.tanh(z / 2)), atol=1e-15, rtol=0)
