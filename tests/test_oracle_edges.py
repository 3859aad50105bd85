"""Pins of the oracle's layer edges (oracle/edges.py): per-token L2
normalisation of the keys and the per-head D skip term, forward and reverse.
Every gradient is checked against central finite differences of the composed
forward; the normalisation against its scale invariance and the gradient's
orthogonality to k; the skip against D = 0 and its closed form."""
import math

import numpy as np
import pytest


def _edges():
    from oracle import edges

    return edges


def _inputs(seed, B=2, T=9, H=2, dk=3, dv=2):
    rng = np.random.default_rng(seed)
    x = dict(q=rng.standard_normal((B, T, H, dk)), k=rng.standard_normal((B, T, H, dk)) * 1.7,
             v=rng.standard_normal((B, T, H, dv)), g=1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H)))),
             beta=1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H)))),
             A_log=rng.uniform(math.log(1e-2), math.log(0.5), H), h0=rng.standard_normal((B, H, dk, dv)),
             D=rng.standard_normal(H))
    return x, rng.standard_normal((B, T, H, dv)), rng.standard_normal((B, H, dk, dv))


def _loss(E, x, do, dhT, norm_k, skip, delta):
    o, hT = E.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["h0"],
                  D=x["D"] if skip else None, norm_k=norm_k, delta=delta, nthreads=1)
    return float(np.sum(o * do) + np.sum(hT * dhT))


@pytest.mark.parametrize("norm_k,skip,delta", [(True, False, True), (False, True, True), (True, True, True),
                                               (True, True, False)])
def test_edges_reverse_matches_central_differences(oracle_mod, norm_k, skip, delta):
    E = _edges()
    x, do, dhT = _inputs(40 + 2 * int(norm_k) + int(skip) + 4 * int(delta))
    r = E.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["h0"], do, dhT,
              D=x["D"] if skip else None, norm_k=norm_k, delta=delta, nthreads=1)
    names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", A_log="dA_log", h0="dh0")
    if skip:
        names["D"] = "dD"
    eps = 1e-6
    for name, gname in names.items():
        base = x[name]
        fd = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = {kk: vv.copy() for kk, vv in x.items()}
            xp[name][idx] += eps
            lp = _loss(E, xp, do, dhT, norm_k, skip, delta)
            xp[name][idx] -= 2 * eps
            lm = _loss(E, xp, do, dhT, norm_k, skip, delta)
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(fd - r[gname]))
        scale = max(1.0, np.max(np.abs(fd)))
        assert err < 1e-7 * scale, (name, err, scale)


def test_normalised_keys_are_scale_invariant(oracle_mod):
    """Scaling every key row by any positive factor leaves the outputs
    unchanged (up to the epsilon under the root) and scales dk by its
    inverse; normalised rows have unit length."""
    E = _edges()
    x, do, dhT = _inputs(50, T=20, dk=4, dv=3)
    kh = E.l2norm_keys(x["k"])
    assert np.allclose(np.linalg.norm(kh, axis=-1), 1.0, atol=1e-6)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["h0"])
    o1, h1 = E.fwd(*args, norm_k=True, nthreads=1)
    r1 = E.bwd(*args, do, dhT, norm_k=True, nthreads=1)
    c = 3.0
    args3 = (x["q"], c * x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["h0"])
    o3, h3 = E.fwd(*args3, norm_k=True, nthreads=1)
    r3 = E.bwd(*args3, do, dhT, norm_k=True, nthreads=1)
    assert np.max(np.abs(o3 - o1)) <= 1e-5 * np.max(np.abs(o1))
    assert np.max(np.abs(h3 - h1)) <= 1e-5 * np.max(np.abs(h1))
    assert np.max(np.abs(c * r3["dk"] - r1["dk"])) <= 1e-5 * np.max(np.abs(r1["dk"]))


def test_key_gradient_is_orthogonal_to_the_key(oracle_mod):
    """The normalisation discards the length of k, so the gradient with
    respect to k has (up to the epsilon) no component along k."""
    E = _edges()
    x, do, dhT = _inputs(51, T=30, dk=5, dv=3)
    r = E.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["h0"], do, dhT, norm_k=True,
              nthreads=1)
    along = np.sum(r["dk"] * x["k"], axis=-1)
    assert np.max(np.abs(along)) <= 1e-5 * np.max(np.abs(r["dk"]))


def test_skip_closed_form_and_zero(oracle_mod):
    """o with the skip minus o without it is exactly D_h v_t; D = 0 gives
    the plain recurrence and its gradients; dD_h = sum do * v."""
    E = _edges()
    x, do, dhT = _inputs(52, T=15, dk=4, dv=3)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["h0"])
    o0, _ = oracle_mod.fwd(*args, nthreads=1)
    o1, _ = E.fwd(*args, D=x["D"], nthreads=1)
    assert np.array_equal(o1, o0 + x["D"][None, None, :, None] * x["v"])
    oz, _ = E.fwd(*args, D=np.zeros_like(x["D"]), nthreads=1)
    assert np.array_equal(oz, o0)
    r0 = oracle_mod.bwd(*args, do, dhT, nthreads=1)
    rz = E.bwd(*args, do, dhT, D=np.zeros_like(x["D"]), nthreads=1)
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dA_log", "dh0"):
        assert np.array_equal(rz[name], r0[name]), name
    r1 = E.bwd(*args, do, dhT, D=x["D"], nthreads=1)
    assert np.allclose(r1["dD"], np.einsum("bthj,bthj->h", do, x["v"]), rtol=0, atol=1e-12)
