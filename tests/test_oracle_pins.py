"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics,
independent of the oracle's own code: brute-force sums, closed forms,
invariants, special cases, the chunked closed form, a hand-worked fixture.

Each pin is chosen so that a plausible slip in the serial loop (decay applied
to the wrong term, erase with the wrong key, read before the write, a sign of
A, a transposed state) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest

from oracle import chunked

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(rng, B, T, H, dk, dv, unit_k=True, weak=False, h0=True):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    if weak:
        A_log = rng.uniform(math.log(1e-3), math.log(1e-1), H)
    else:
        A_log = rng.uniform(0.0, math.log(16.0), H)
    h0a = 0.5 * rng.standard_normal((B, H, dk, dv)) if h0 else None
    return q, k, v, g, beta, A_log, h0a


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ---------------------------------------------------------------- delta off


def test_additive_form_equals_quadratic_decay_masked_sum(oracle_mod):
    """Delta term off: unrolling h_t = alpha_t h_{t-1} + beta_t k_t v_t^T gives
    o_t = sum_{s<=t} prod_{s<r<=t} alpha_r * beta_s (q_t . k_s) v_s
          + prod_{r<=t} alpha_r * h0^T q_t.
    Evaluated here by brute force, one (t, s) pair at a time, with the decay
    product multiplied out term by term (no cumulative sums)."""
    rng = np.random.default_rng(1)
    B, T, H, dk, dv = 2, 23, 2, 3, 4
    q, k, v, g, beta, A_log, h0 = rand_inputs(rng, B, T, H, dk, dv, weak=True)
    o, hT = oracle_mod.fwd(q, k, v, g, beta, A_log, h0, delta=False)
    ref = np.zeros_like(o)
    refh = np.zeros_like(hT)
    for b in range(B):
        for h in range(H):
            alpha = [math.exp(-math.exp(A_log[h]) * g[b, t, h]) for t in range(T)]
            for t in range(T):
                acc = np.zeros(dv)
                for s in range(t + 1):
                    decay = 1.0
                    for r in range(s + 1, t + 1):
                        decay *= alpha[r]
                    acc += decay * beta[b, s, h] * np.dot(q[b, t, h], k[b, s, h]) * v[b, s, h]
                decay0 = 1.0
                for r in range(t + 1):
                    decay0 *= alpha[r]
                acc += decay0 * (h0[b, h].T @ q[b, t, h])
                ref[b, t, h] = acc
            st = h0[b, h].copy()
            for t in range(T):
                st = alpha[t] * st + beta[b, t, h] * np.outer(k[b, t, h], v[b, t, h])
            refh[b, h] = st
    assert rel(o, ref) < 1e-12
    assert rel(hT, refh) < 1e-12


def test_ungated_additive_form_is_causal_linear_attention(oracle_mod):
    """g = 0 (alpha = 1) and delta off is plain causal linear attention
    ("GDN & MLA Mechanism Deep-Dive", Step 2): O = tril(Q K^T) (beta V) + Q h0,
    computed with library matrix products."""
    rng = np.random.default_rng(2)
    B, T, H, dk, dv = 1, 40, 3, 5, 6
    q, k, v, g, beta, A_log, h0 = rand_inputs(rng, B, T, H, dk, dv)
    g = np.zeros_like(g)
    o, hT = oracle_mod.fwd(q, k, v, g, beta, A_log, h0, delta=False)
    for h in range(H):
        Q, K, V = q[0, :, h], k[0, :, h], v[0, :, h] * beta[0, :, h, None]
        ref = np.tril(Q @ K.T) @ V + Q @ h0[0, h]
        assert rel(o[0, :, h], ref) < 1e-12
        assert rel(hT[0, h], h0[0, h] + K.T @ V) < 1e-12


# ----------------------------------------------------------------- delta on


@pytest.mark.parametrize("weak", [False, True])
def test_delta_rule_writes_exactly_the_new_value(oracle_mod, weak):
    """With unit-norm k and beta = 1 the erase (I - k k^T) is a projection, so
    after every token the state maps its key to its value: h_t^T k_t = v_t,
    whatever the decay. Checked at every prefix length."""
    rng = np.random.default_rng(3)
    B, T, H, dk, dv = 1, 30, 2, 6, 5
    q, k, v, g, beta, A_log, h0 = rand_inputs(rng, B, T, H, dk, dv, weak=weak)
    beta = np.ones_like(beta)
    for t in range(1, T + 1):
        _, hT = oracle_mod.fwd(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], A_log, h0)
        for h in range(H):
            got = hT[0, h].T @ k[0, t - 1, h]
            assert np.max(np.abs(got - v[0, t - 1, h])) < 1e-12


@pytest.mark.parametrize("delta", [True, False])
def test_single_token_from_zero_state(oracle_mod, delta):
    """T = 1, h0 = 0: h1 = beta k v^T and o = beta (k . q) v, for either form."""
    rng = np.random.default_rng(4)
    q, k, v, g, beta, A_log, _ = rand_inputs(rng, 3, 1, 2, 7, 3, unit_k=False)
    o, hT = oracle_mod.fwd(q, k, v, g, beta, A_log, None, delta=delta)
    for b in range(3):
        for h in range(2):
            bt = beta[b, 0, h]
            assert rel(hT[b, h], bt * np.outer(k[b, 0, h], v[b, 0, h])) < 1e-14
            assert rel(o[b, 0, h], bt * np.dot(k[b, 0, h], q[b, 0, h]) * v[b, 0, h]) < 1e-14


@pytest.mark.parametrize("delta", [True, False])
def test_beta_zero_is_pure_decay(oracle_mod, delta):
    """beta = 0 leaves only the decay: h_t = exp(A sum_{r<=t} g_r) h0 and the
    norm shrinks strictly for g > 0 (alpha in (0, 1), "GDN & MLA Mechanism
    Deep-Dive", Intuition)."""
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 2, 17, 2, 4, 3
    q, k, v, g, beta, A_log, h0 = rand_inputs(rng, B, T, H, dk, dv, weak=True)
    beta = np.zeros_like(beta)
    o, hT = oracle_mod.fwd(q, k, v, g, beta, A_log, h0, delta=delta)
    for b in range(B):
        for h in range(H):
            lam = -math.exp(A_log[h]) * g[b, :, h]
            assert rel(hT[b, h], math.exp(lam.sum()) * h0[b, h]) < 1e-13
            for t in range(T):
                ref = math.exp(lam[: t + 1].sum()) * (h0[b, h].T @ q[b, t, h])
                assert rel(o[b, t, h], ref) < 1e-13
            assert np.linalg.norm(hT[b, h]) < np.linalg.norm(h0[b, h])


@pytest.mark.parametrize("delta", [True, False])
def test_zero_decay_limit_is_memoryless(oracle_mod, delta):
    """A_log = ln 800, g = 1 gives alpha = exp(-800) = 0 in double: every
    token sees only its own write, o_t = beta_t (k_t . q_t) v_t."""
    rng = np.random.default_rng(6)
    B, T, H, dk, dv = 1, 9, 2, 3, 4
    q, k, v, g, beta, A_log, h0 = rand_inputs(rng, B, T, H, dk, dv)
    g = np.ones_like(g)
    A_log = np.full(H, math.log(800.0))
    o, hT = oracle_mod.fwd(q, k, v, g, beta, A_log, h0, delta=delta)
    for h in range(H):
        for t in range(T):
            ref = beta[0, t, h] * np.dot(k[0, t, h], q[0, t, h]) * v[0, t, h]
            assert rel(o[0, t, h], ref) < 1e-14
        assert rel(hT[0, h], beta[0, -1, h] * np.outer(k[0, -1, h], v[0, -1, h])) < 1e-14


# -------------------------------------------------- structural properties


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
@pytest.mark.parametrize("weak", [False, True])
@pytest.mark.parametrize("delta", [True, False])
def test_chunked_closed_form_matches_serial(oracle_mod, T, weak, delta):
    """The chunk-64 closed form ("GDN & MLA Mechanism Deep-Dive", Step 5) and
    the serial loop reach the same result."""
    rng = np.random.default_rng(100 + T)
    q, k, v, g, beta, A_log, h0 = rand_inputs(rng, 1, T, 2, 8, 6, weak=weak)
    o, hT = oracle_mod.fwd(q, k, v, g, beta, A_log, h0, delta=delta)
    oc, hc = chunked.fwd_chunked(q, k, v, g, beta, A_log, h0, delta=delta)
    assert rel(oc, o) < 1e-12
    assert rel(hc, hT) < 1e-12


def test_chunked_closed_form_long_sequence(oracle_mod):
    rng = np.random.default_rng(7)
    q, k, v, g, beta, A_log, h0 = rand_inputs(rng, 1, 4096, 1, 8, 8, weak=True)
    o, hT = oracle_mod.fwd(q, k, v, g, beta, A_log, h0)
    oc, hc = chunked.fwd_chunked(q, k, v, g, beta, A_log, h0)
    assert rel(oc, o) < 1e-11
    assert rel(hc, hT) < 1e-11


@pytest.mark.parametrize("delta", [True, False])
def test_segment_split_resumes_exactly(oracle_mod, delta):
    """Running T1 tokens, then T2 tokens from the returned state, equals one
    run over T1 + T2 tokens (the state hand-off is the whole carry)."""
    rng = np.random.default_rng(8)
    q, k, v, g, beta, A_log, h0 = rand_inputs(rng, 2, 50, 2, 5, 4)
    o, hT = oracle_mod.fwd(q, k, v, g, beta, A_log, h0, delta=delta)
    o1, h1 = oracle_mod.fwd(q[:, :21], k[:, :21], v[:, :21], g[:, :21], beta[:, :21], A_log, h0,
                            delta=delta)
    o2, h2 = oracle_mod.fwd(q[:, 21:], k[:, 21:], v[:, 21:], g[:, 21:], beta[:, 21:], A_log, h1,
                            delta=delta)
    assert rel(np.concatenate([o1, o2], axis=1), o) < 1e-14
    assert rel(h2, hT) < 1e-14


def test_value_columns_are_independent(oracle_mod):
    """Column j of o and of the state depends only on column j of v and h0."""
    rng = np.random.default_rng(9)
    q, k, v, g, beta, A_log, h0 = rand_inputs(rng, 1, 33, 2, 4, 5)
    o, hT = oracle_mod.fwd(q, k, v, g, beta, A_log, h0)
    v2, h02 = v.copy(), h0.copy()
    v2[..., 2] += rng.standard_normal(v2[..., 2].shape)
    h02[..., 2] += 1.0
    o2, hT2 = oracle_mod.fwd(q, k, v2, g, beta, A_log, h02)
    keep = [0, 1, 3, 4]
    assert np.array_equal(o[..., keep], o2[..., keep])
    assert np.array_equal(hT[..., keep], hT2[..., keep])
    assert not np.allclose(o[..., 2], o2[..., 2])


def _read_golden(path):
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rhs = (s.strip() for s in line.split("=", 1))
            rows = [[float(x) for x in r.split()] for r in rhs.split(";")]
            vals[key] = np.array(rows)
    return vals


@pytest.mark.parametrize("delta", [True, False])
def test_hand_worked_example(oracle_mod, delta):
    gd = _read_golden(os.path.join(GOLDEN, "handworked_T2_d2.txt"))
    T, dk = gd["q"].shape
    q = gd["q"].reshape(1, T, 1, dk)
    k = gd["k"].reshape(1, T, 1, dk)
    v = gd["v"].reshape(1, T, 1, -1)
    g = gd["g"].reshape(1, T, 1)
    beta = gd["beta"].reshape(1, T, 1)
    A_log = gd["A_log"].reshape(1)
    h0 = gd["h0"].reshape(1, 1, dk, -1)
    o, hT = oracle_mod.fwd(q, k, v, g, beta, A_log, h0, delta=delta)
    tag = "delta_on" if delta else "delta_off"
    np.testing.assert_allclose(o[0, :, 0], gd[tag + ".o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(hT[0, 0], gd[tag + ".hT"], rtol=0, atol=1e-14)


def test_unit_subset_and_thread_count_do_not_change_results(oracle_mod):
    rng = np.random.default_rng(10)
    q, k, v, g, beta, A_log, h0 = rand_inputs(rng, 3, 40, 3, 4, 4)
    o, hT = oracle_mod.fwd(q, k, v, g, beta, A_log, h0, nthreads=1)
    o4, hT4 = oracle_mod.fwd(q, k, v, g, beta, A_log, h0, nthreads=4)
    assert np.array_equal(o, o4) and np.array_equal(hT, hT4)
    os_, hs = oracle_mod.fwd(q, k, v, g, beta, A_log, h0, units=[4, 7])
    for u in (4, 7):
        b, h = divmod(u, 3)
        assert np.array_equal(os_[b, :, h], o[b, :, h])
        assert np.array_equal(hs[b, h], hT[b, h])
    assert np.all(os_[0, :, 0] == 0)


# --------------------------------------------------------------------- step


@pytest.mark.parametrize("delta", [True, False])
def test_step_chain_equals_forward(oracle_mod, delta):
    """T consecutive single-token steps from h0 equal one forward pass."""
    rng = np.random.default_rng(11)
    B, T, H, dk, dv = 3, 12, 2, 5, 4
    q, k, v, g, beta, A_log, h0 = rand_inputs(rng, B, T, H, dk, dv)
    o, hT = oracle_mod.fwd(q, k, v, g, beta, A_log, h0, delta=delta)
    st = h0
    for t in range(T):
        ot, st = oracle_mod.step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], A_log, st,
                                 delta=delta)
        assert rel(ot, o[:, t]) < 1e-13
    assert rel(st, hT) < 1e-13


def test_empty_sequence_is_zero_steps():
    """T = 0 runs no step of the recurrence (the Step 4 loop of "GDN & MLA
    Mechanism Deep-Dive" over no tokens): the final state is h0, the gradient
    of h0 is dhT, and every other gradient is empty or zero."""
    import oracle as O

    B, T, H, dk, dv = 2, 0, 3, 5, 4
    rng = np.random.default_rng(7600)
    z = lambda *s: np.zeros(s)
    h0 = rng.standard_normal((B, H, dk, dv))
    dhT = rng.standard_normal((B, H, dk, dv))
    args = (z(B, T, H, dk), z(B, T, H, dk), z(B, T, H, dv), z(B, T, H), z(B, T, H), rng.standard_normal(H))
    o, hT = O.fwd(*args, h0)
    assert o.shape == (B, 0, H, dv) and np.array_equal(hT, h0)
    _, hz = O.fwd(*args, None)
    assert np.array_equal(hz, np.zeros_like(h0))
    r = O.bwd(*args, h0, z(B, T, H, dv), dhT)
    assert np.array_equal(r["dh0"], dhT)
    assert np.array_equal(r["dA_log"], np.zeros(H))
    assert r["dq"].shape == (B, 0, H, dk) and r["dg"].shape == (B, 0, H)
