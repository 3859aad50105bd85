"""Fused layer edges on the GPU: per-token L2 normalisation of the keys
(GDN_FLAG_L2NORM_K) and the per-head skip term o_t += D[h] v_t, in the
forward, the backward (dk through the normalisation, dv + D do, dD) and the
decode calls, against the oracle's edges (oracle/edges.py, pinned on the CPU
by finite differences and invariances). Keys are drawn with per-row lengths in
[0.25, 4] so that the normalisation changes them."""
import numpy as np
import pytest
import torch

import gated_delta_rule_74_amd as gdn
import gdn_inputs as gi
from gpu_util import TOL, assert_close, dev, f64, host, say

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dA_log", "dh0", "dD")


def _edges():
    from oracle import edges

    return edges


def _seq(B, T, H, d, dtype, seed, key_spread=True):
    """Raw keys of spread lengths are for the normalised calls only: without
    the normalisation such keys would make the delta rule's erase factor
    1 - beta |k|^2 far from (-1, 1) and the state grow without bound."""
    return gi.gen_seq(B, T, H, d, d, dtype, seed=seed, h0="randn", with_do=True, decay="weak",
                      key_spread=key_spread, with_D=True)


def _check(x, dtype, norm_k=True, skip=True, additive=False, paths=("ctx", "recompute")):
    """Forward and backward on the GPU with the edges on, against the oracle's
    composition; both backward paths (saved context, recomputed forward)."""
    E = _edges()
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log, h0, do = dev(x["g"]), dev(x["beta"]), dev(x["A_log"]), dev(x["h0"]), dev(x["do"])
    D = dev(x["D"]) if skip else None
    o, hT, cs = gdn.fwd(q, k, v, g, beta, A_log, h0, additive=additive, norm_k=norm_k, D=D, save_context=True)
    res = []
    for p in paths:
        res.append(gdn.bwd(q, k, v, g, beta, A_log, do, h0, context=cs if p == "ctx" else None,
                           additive=additive, norm_k=norm_k, D=D, want_dD=True))
    torch.cuda.synchronize()
    args = (f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["g"]), f64(x["beta"]), f64(x["A_log"]),
            f64(x["h0"]))
    Dr = f64(x["D"]) if skip else None
    ro, rh = E.fwd(*args, D=Dr, norm_k=norm_k, delta=not additive)
    tol = TOL[dtype]
    assert_close("o", host(o), ro, tol)
    assert_close("hT", host(hT), rh, tol)
    ref = E.bwd(*args, f64(x["do"]), D=Dr, norm_k=norm_k, delta=not additive)
    if not skip:  # dD is the gradient at D = 0: sum of do * v
        ref["dD"] = np.einsum("bthj,bthj->h", f64(x["do"]), f64(x["v"]))
    for p, r in zip(paths, res):
        for name in GRADS:
            assert_close(f"{p} {name}", host(r[name]), ref[name], tol)
    return o, res


@pytest.mark.parametrize("dtype,d,T", [("bf16", 56, 200), ("bf16", 64, 64), ("bf16", 20, 130), ("bf16", 128, 130),
                                       ("bf16", 100, 70), ("f32", 16, 130), ("f32", 12, 70), ("f32", 32, 130),
                                       ("f32", 60, 70)])
def test_edges_fwd_bwd(dtype, d, T):
    """Every local-gradient kernel (d <= 64 in bf16 and fp32 up to 16, the
    LDS-resident 128 kernel, the fp32 wide kernel) with 16-byte and
    element-wise row access (dims not a multiple of 8), ragged last chunks."""
    say(f"edges fwd+bwd B2 T{T} H3 d{d} {dtype} norm_k + D")
    _check(_seq(2, T, 3, d, dtype, 8100 + d), dtype)


@pytest.mark.parametrize("norm_k,skip", [(True, False), (False, True)])
def test_edges_one_at_a_time(norm_k, skip):
    say(f"edges one at a time norm_k={norm_k} skip={skip} B2 T150 H2 d56 bf16")
    _check(_seq(2, 150, 2, 56, "bf16", 8200 + 2 * norm_k + skip, key_spread=norm_k), "bf16", norm_k=norm_k,
           skip=skip)


@pytest.mark.parametrize("dtype,d", [("bf16", 56), ("bf16", 128), ("f32", 32)])
def test_edges_additive(dtype, d):
    say(f"edges with the additive form B2 T130 H2 d{d} {dtype}")
    _check(_seq(2, 130, 2, d, dtype, 8300 + d), dtype, additive=True, paths=("ctx",))


def test_edges_on_the_scan_path():
    """64 chunks and more on bf16 heads past 64: the forward and backward
    serial passes run as parallel scans over chunk ranges, with the keys
    normalised inside every range's pass."""
    say("edges on the scan path B1 T4200 H2 d128 bf16")
    _check(_seq(1, 4200, 2, 128, "bf16", 8400), "bf16", paths=("ctx",))


def test_edges_off_is_bitwise_the_plain_call():
    """norm_k=False and D=None are the plain recurrence: the same bits as a
    call that never names them, and D = 0 gives the same outputs as no D."""
    say("edges off vs plain call B2 T130 H2 d56 bf16")
    x = _seq(2, 130, 2, 56, "bf16", 8500)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log, h0 = dev(x["g"]), dev(x["beta"]), dev(x["A_log"]), dev(x["h0"])
    a = gdn.fwd(q, k, v, g, beta, A_log, h0)
    b = gdn.fwd(q, k, v, g, beta, A_log, h0, norm_k=False, D=None)
    z = gdn.fwd(q, k, v, g, beta, A_log, h0, D=torch.zeros_like(A_log))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(a[0], z[0]) and torch.equal(a[1], z[1])


def test_normalised_unit_keys_match_the_plain_call():
    """Keys that are already unit rows are (up to the epsilon and one
    rounding) unchanged by the normalisation."""
    say("unit keys with norm_k B2 T130 H2 d56 bf16")
    x = gi.gen_seq(2, 130, 2, 56, 56, "bf16", seed=8501, h0="randn", decay="weak")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log, h0 = dev(x["g"]), dev(x["beta"]), dev(x["A_log"]), dev(x["h0"])
    a = gdn.fwd(q, k, v, g, beta, A_log, h0)
    b = gdn.fwd(q, k, v, g, beta, A_log, h0, norm_k=True)
    torch.cuda.synchronize()
    assert_close("o", host(b[0]), host(a[0]), TOL["bf16"])
    assert_close("hT", host(b[1]), host(a[1]), TOL["bf16"])


@pytest.mark.parametrize("d,S", [(56, 1), (56, 3), (64, 4), (128, 1), (128, 3), (100, 2)])
def test_edges_decode(d, S):
    """Decode calls (one token, the multi-token kernel for 2 to 4 tokens on
    heads up to 64 wide, the wide-head path) with the edges on, against the
    oracle's forward over the same S tokens from the same state."""
    say(f"edges decode N8 H4 d{d} S{S} bf16")
    x = _seq(8, S, 4, d, "bf16", 8600 + d + S)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log, D = dev(x["g"]), dev(x["beta"]), dev(x["A_log"]), dev(x["D"])
    h = dev(x["h0"]).clone()
    if S == 1:
        o, hN = gdn.step(q[:, 0].contiguous(), k[:, 0].contiguous(), v[:, 0].contiguous(),
                         g[:, 0].contiguous(), beta[:, 0].contiguous(), A_log, h, h, norm_k=True, D=D)
        o = o[:, None]
    else:
        o, hN = gdn.step_tokens(q, k, v, g, beta, A_log, h, h, norm_k=True, D=D)
    torch.cuda.synchronize()
    ro, rh = _edges().fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["g"]), f64(x["beta"]), f64(x["A_log"]),
                          f64(x["h0"]), D=f64(x["D"]), norm_k=True)
    assert_close("o", host(o), ro, TOL["bf16"])
    assert_close("state", host(hN), rh, TOL["bf16"])


def test_edges_through_autograd():
    """GatedDeltaRule.apply with norm_k and D: gradients reach the raw keys
    and D."""
    say("edges through autograd B1 T100 H2 d56 bf16")
    x = _seq(1, 100, 2, 56, "bf16", 8700)
    ts = {n: dev(x[n]).requires_grad_(True) for n in ("q", "k", "v", "g", "beta", "A_log", "h0", "D")}
    o, hT = gdn.GatedDeltaRule.apply(ts["q"], ts["k"], ts["v"], ts["g"], ts["beta"], ts["A_log"], ts["h0"],
                                     False, False, True, ts["D"])
    o.backward(dev(x["do"]))
    torch.cuda.synchronize()
    args = (f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["g"]), f64(x["beta"]), f64(x["A_log"]),
            f64(x["h0"]))
    ref = _edges().bwd(*args, f64(x["do"]), D=f64(x["D"]), norm_k=True)
    for n, gname in (("k", "dk"), ("v", "dv"), ("D", "dD"), ("q", "dq"), ("A_log", "dA_log")):
        assert_close(gname, host(ts[n].grad), ref[gname], TOL["bf16"])
