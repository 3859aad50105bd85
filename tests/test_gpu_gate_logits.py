"""Gates given as logits (GDN_FLAG_GATE_LOGITS): the HIP kernels apply the
sigmoid to g and beta where they use them and return dg, dbeta with respect
to the logits. Reference: the oracle composed with its sigmoid and the chain
rule through it (pinned by finite differences on the CPU)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_74_amd as gdn
import gdn_inputs as gi
from gpu_util import TOL, assert_close, dev, f64, host, say

pytestmark = pytest.mark.gpu


def _oracle():
    import oracle

    return oracle


def with_logits(x, seed):
    """Replace the gate values by fp32 logits drawn N(0, 1.5^2) (the oracle
    then uses the sigmoid of exactly these stored logits)."""
    rng = np.random.default_rng(seed)
    x = dict(x)
    x["gl"] = (1.5 * rng.standard_normal(x["g"].shape)).astype(np.float32)
    x["bl"] = (1.5 * rng.standard_normal(x["beta"].shape)).astype(np.float32)
    return x


def _ref_gates(x):
    O = _oracle()
    return O.gates_from_logits(f64(x["gl"])), O.gates_from_logits(f64(x["bl"]))


@pytest.mark.parametrize("T", [64, 200])
def test_fwd_bwd_with_gate_logits(T):
    say(f"gate logits fwd+bwd B2 T{T} H4 d56 bf16")
    x = with_logits(gi.gen_seq(2, T, 4, 56, 56, "bf16", seed=7420, h0="randn", with_do=True,
                               decay="weak"), 7421)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    gl, bl, A_log, h0, do = dev(x["gl"]), dev(x["bl"]), dev(x["A_log"]), dev(x["h0"]), dev(x["do"])
    o, hT, cs = gdn.fwd(q, k, v, gl, bl, A_log, h0, gate_logits=True, save_context=True)
    r = gdn.bwd(q, k, v, gl, bl, A_log, do, h0, context=cs, gate_logits=True)
    r2 = gdn.bwd(q, k, v, gl, bl, A_log, do, h0, context=None, gate_logits=True)  # recompute path
    torch.cuda.synchronize()
    gs, bs = _ref_gates(x)
    O = _oracle()
    ro, rh = O.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), gs, bs, f64(x["A_log"]), f64(x["h0"]))
    tol = TOL["bf16"]
    assert_close("o", host(o), ro, tol)
    assert_close("hT", host(hT), rh, tol)
    rg = O.bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), gs, bs, f64(x["A_log"]), f64(x["h0"]), f64(x["do"]))
    ref = dict(rg, dg=O.logit_grads(rg["dg"], gs), dbeta=O.logit_grads(rg["dbeta"], bs))
    for res in (r, r2):
        for name in ("dq", "dk", "dv", "dg", "dbeta", "dA_log", "dh0"):
            assert_close(name, host(res[name]), ref[name], tol)


def test_wide_head_bwd_with_gate_logits():
    say("gate logits fwd+bwd B1 T130 H2 d128 bf16")
    x = with_logits(gi.gen_seq(1, 130, 2, 128, 128, "bf16", seed=7422, h0="randn", with_do=True,
                               decay="weak"), 7423)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    gl, bl, A_log, h0, do = dev(x["gl"]), dev(x["bl"]), dev(x["A_log"]), dev(x["h0"]), dev(x["do"])
    _, _, cs = gdn.fwd(q, k, v, gl, bl, A_log, h0, gate_logits=True, save_context=True)
    r = gdn.bwd(q, k, v, gl, bl, A_log, do, h0, context=cs, gate_logits=True)
    torch.cuda.synchronize()
    gs, bs = _ref_gates(x)
    O = _oracle()
    rg = O.bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), gs, bs, f64(x["A_log"]), f64(x["h0"]), f64(x["do"]))
    assert_close("dg", host(r["dg"]), O.logit_grads(rg["dg"], gs), TOL["bf16"])
    assert_close("dbeta", host(r["dbeta"]), O.logit_grads(rg["dbeta"], bs), TOL["bf16"])
    assert_close("dA_log", host(r["dA_log"]), rg["dA_log"], TOL["bf16"])


@pytest.mark.parametrize("S", [1, 3])
def test_decode_with_gate_logits(S):
    say(f"gate logits step_tokens N8 H4 d56 S={S}")
    x = with_logits(gi.gen_seq(8, S, 4, 56, 56, "bf16", seed=7424, h0="randn", decay="weak"), 7425)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    gl, bl, A_log, h = dev(x["gl"]), dev(x["bl"]), dev(x["A_log"]), dev(x["h0"]).clone()
    o, hN = gdn.step_tokens(q, k, v, gl, bl, A_log, h, h, gate_logits=True)
    torch.cuda.synchronize()
    gs, bs = _ref_gates(x)
    ro, rh = _oracle().fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), gs, bs, f64(x["A_log"]), f64(x["h0"]))
    assert_close("o", host(o), ro, TOL["bf16"])
    assert_close("state", host(hN), rh, TOL["bf16"])


@pytest.mark.parametrize("dtype,d", [("bf16", 56), ("bf16", 128), ("f32", 32)])
def test_additive_with_gate_logits(dtype, d):
    """Both flags at once (erase term off, gates as logits): forward, backward
    (saved context) and a three-token decode call against the oracle's
    additive form composed with the sigmoid and its chain rule."""
    say(f"additive + gate logits fwd+bwd B2 T130 H2 d{d} {dtype}, decode S3")
    x = with_logits(gi.gen_seq(2, 130, 2, d, d, dtype, seed=7426, h0="randn", with_do=True,
                               decay="weak"), 7427)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    gl, bl, A_log, h0, do = dev(x["gl"]), dev(x["bl"]), dev(x["A_log"]), dev(x["h0"]), dev(x["do"])
    o, hT, cs = gdn.fwd(q, k, v, gl, bl, A_log, h0, additive=True, gate_logits=True, save_context=True)
    r = gdn.bwd(q, k, v, gl, bl, A_log, do, h0, context=cs, additive=True, gate_logits=True)
    tail = lambda t: t[:, -3:].contiguous()
    h = h0.clone()
    od, hd = gdn.step_tokens(tail(q), tail(k), tail(v), tail(gl), tail(bl), A_log, h, h, additive=True,
                             gate_logits=True)
    torch.cuda.synchronize()
    gs, bs = _ref_gates(x)
    O = _oracle()
    tol = TOL[dtype]
    args = (f64(x["q"]), f64(x["k"]), f64(x["v"]), gs, bs, f64(x["A_log"]), f64(x["h0"]))
    ro, rh = O.fwd(*args, delta=False)
    assert_close("o", host(o), ro, tol)
    assert_close("hT", host(hT), rh, tol)
    rg = O.bwd(*args, f64(x["do"]), delta=False)
    ref = dict(rg, dg=O.logit_grads(rg["dg"], gs), dbeta=O.logit_grads(rg["dbeta"], bs))
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dA_log", "dh0"):
        assert_close(name, host(r[name]), ref[name], tol)
    # decode: the last three tokens from h0 as a sequence of their own
    t3 = lambda a: f64(a)[:, -3:]
    rdo, rdh = O.fwd(t3(x["q"]), t3(x["k"]), t3(x["v"]), gs[:, -3:], bs[:, -3:], f64(x["A_log"]),
                     f64(x["h0"]), delta=False)
    assert_close("decode o", host(od), rdo, tol)
    assert_close("decode state", host(hd), rdh, tol)


def test_autograd_with_gate_logits():
    """GatedDeltaRule.apply with gate_logits=True: gradients reach the logits
    (through the kernels' sigmoid) and match the oracle's chain rule."""
    say("gate logits through autograd B1 T100 H2 d56 bf16")
    x = with_logits(gi.gen_seq(1, 100, 2, 56, 56, "bf16", seed=7425, h0="randn", with_do=True,
                               decay="weak"), 7426)
    ts = {n: dev(x[n]).requires_grad_(True) for n in ("q", "k", "v", "gl", "bl", "A_log", "h0")}
    o, hT = gdn.GatedDeltaRule.apply(ts["q"], ts["k"], ts["v"], ts["gl"], ts["bl"], ts["A_log"],
                                     ts["h0"], False, True)
    o.backward(dev(x["do"]))
    gs, bs = _ref_gates(x)
    O = _oracle()
    rg = O.bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), gs, bs, f64(x["A_log"]), f64(x["h0"]), f64(x["do"]))
    ref = dict(rg, dg=O.logit_grads(rg["dg"], gs), dbeta=O.logit_grads(rg["dbeta"], bs))
    for name, key in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("gl", "dg"), ("bl", "dbeta"),
                      ("A_log", "dA_log"), ("h0", "dh0")]:
        assert_close(f"autograd {key}", host(ts[name].grad), ref[key], TOL["bf16"])
