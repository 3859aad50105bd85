"""Decode-step parity: chains of HIP single-token steps vs the oracle's step
chain on the same seeded tokens and initial state."""
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


def run_chain(x, steps, additive=False, inplace=True, zero_start=False):
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log = dev(x["g"]), dev(x["beta"]), dev(x["A_log"])
    h = None if zero_start else dev(x["h0"]).clone()
    outs = []
    for t in range(steps):
        if inplace and h is not None:
            o, h = gdn.step(q[t], k[t], v[t], g[t], beta[t], A_log, h, h, additive=additive)
        else:
            o, h = gdn.step(q[t], k[t], v[t], g[t], beta[t], A_log, h, None, additive=additive)
        outs.append(o)
    torch.cuda.synchronize()
    return [host(o) for o in outs], host(h)


def check_chain(x, steps, dtype, additive=False, inplace=True, zero_start=False):
    got_o, got_h = run_chain(x, steps, additive, inplace, zero_start)
    h = None if zero_start else f64(x["h0"])
    tol = TOL[dtype]
    for t in range(steps):
        ro, h = _oracle().step(f64(x["q"])[t], f64(x["k"])[t], f64(x["v"])[t], f64(x["g"])[t],
                               f64(x["beta"])[t], f64(x["A_log"]), h, delta=not additive)
        if t in (0, steps // 2, steps - 1):
            assert_close(f"o step {t}", got_o[t], ro, tol)
    assert_close("final state", got_h, h, tol)


@pytest.mark.parametrize("decay", ["normal", "weak", "zero"])
def test_decode_reduced_bf16(decay):
    say(f"step bf16 N8 H16 d56 decay={decay}")
    x = gi.gen_decode(8, 16, 56, 56, 32, "bf16", decay=decay)
    check_chain(x, 32, "bf16")


def test_decode_full_width_bf16():
    """The decode workload's full width (256 sequences x 16 heads x d56)."""
    say("step bf16 N256 H16 d56, 8 steps")
    x = gi.gen_decode(256, 16, 56, 56, 8, "bf16")
    check_chain(x, 8, "bf16")


@pytest.mark.parametrize("inplace", [True, False])
def test_decode_fp32(inplace):
    x = gi.gen_decode(4, 3, 16, 16, 20, "f32", decay="weak")
    check_chain(x, 20, "f32", inplace=inplace)


def test_decode_additive_and_zero_start():
    x = gi.gen_decode(4, 3, 56, 56, 10, "bf16", decay="weak")
    check_chain(x, 10, "bf16", additive=True)
    check_chain(x, 10, "bf16", zero_start=True)


@pytest.mark.parametrize("dk,dv", [(128, 128), (100, 70), (64, 128), (5, 3)])
def test_decode_head_dims(dk, dv):
    say(f"step bf16 dk={dk} dv={dv}")
    x = gi.gen_decode(4, 2, dk, dv, 6, "bf16", decay="weak")
    check_chain(x, 6, "bf16")


def test_decode_chain_matches_forward():
    """256 consecutive in-place steps of 2 sequences x 2 heads equal one
    oracle forward pass over the same 256 tokens."""
    x = gi.gen_decode(2, 2, 56, 56, 256, "bf16", decay="weak")
    got_o, got_h = run_chain(x, 256)
    # rearrange [steps, N, H, .] -> [N, steps, H, .]
    tr = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1))
    ro, rh = _oracle().fwd(tr(f64(x["q"])), tr(f64(x["k"])), tr(f64(x["v"])), tr(f64(x["g"])),
                           tr(f64(x["beta"])), f64(x["A_log"]), f64(x["h0"]))
    assert_close("o chain vs forward", tr(np.stack(got_o)), ro, TOL["bf16"])
    assert_close("state chain vs forward", got_h, rh, TOL["bf16"])


def test_decode_graph_replay():
    """The decode chain captured in a HIP graph (the way bench.py times it)
    gives the eager result bit for bit on every replay, with eager work and
    synchronisations between the replays."""
    say("step graph replay N16 H4 d56, 12 steps")
    S = 12
    x = gi.gen_decode(16, 4, 56, 56, S, "bf16", decay="weak")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log, h0 = dev(x["g"]), dev(x["beta"]), dev(x["A_log"]), dev(x["h0"])
    o = torch.empty(16, 4, 56, dtype=torch.bfloat16, device=q.device)

    def chain(h, out):
        for t in range(S):
            gdn.step(q[t], k[t], v[t], g[t], beta[t], A_log, h, h, o=out)

    h = h0.clone()
    chain(h, o)
    torch.cuda.synchronize()
    ref_h, ref_o = h.clone(), o.clone()
    h.copy_(h0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain(h, o)
    for rep in range(3):
        h.copy_(h0)
        o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, ref_h), f"state differs on replay {rep}"
        assert torch.equal(o, ref_o), f"output differs on replay {rep}"
        # eager work of the program between replays
        h2, o2 = h0.clone(), torch.empty_like(o)
        chain(h2, o2)
        torch.cuda.synchronize()
        assert torch.equal(h2, ref_h)


def test_step_tokens_graph_replay():
    """Three-token calls (the kernel that loads all tokens first) and an
    empty call captured in a HIP graph replay the eager result bit for bit."""
    say("step_tokens graph replay N16 S3 H4 d56, 4 calls")
    calls, S = 4, 3
    x = gi.gen_decode(16, 4, 56, 56, calls * S, "bf16", decay="weak")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log, h0 = dev(x["g"]), dev(x["beta"]), dev(x["A_log"]), dev(x["h0"])
    # [steps, N, H, *] -> per call [N, S, H, *]
    tok = lambda t, c: t[c * S:(c + 1) * S].transpose(0, 1).contiguous()
    qs = [tok(q, c) for c in range(calls)]
    ks = [tok(k, c) for c in range(calls)]
    vs = [tok(v, c) for c in range(calls)]
    gs = [tok(g, c) for c in range(calls)]
    bs = [tok(beta, c) for c in range(calls)]
    o = torch.empty(calls, 16, S, 4, 56, dtype=torch.bfloat16, device=q.device)
    q0 = torch.empty((16, 0, 4, 56), dtype=torch.bfloat16, device=q.device)
    g0 = torch.empty((16, 0, 4), dtype=torch.float32, device=q.device)
    h_copy = torch.empty_like(h0)

    def chain(h, out):
        for c in range(calls):
            gdn.step_tokens(qs[c], ks[c], vs[c], gs[c], bs[c], A_log, h, h, o=out[c])
        gdn.step_tokens(q0, q0, q0, g0, g0, A_log, h, h_copy)  # S = 0: copy of the state

    h = h0.clone()
    chain(h, o)
    torch.cuda.synchronize()
    ref_h, ref_o = h.clone(), o.clone()
    assert torch.equal(h_copy, ref_h)
    h.copy_(h0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain(h, o)
    for rep in range(3):
        h.copy_(h0)
        o.zero_()
        h_copy.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, ref_h), f"state differs on replay {rep}"
        assert torch.equal(o, ref_o), f"output differs on replay {rep}"
        assert torch.equal(h_copy, ref_h), f"empty-call copy differs on replay {rep}"
        h2, o2 = h0.clone(), torch.empty_like(o)
        chain(h2, o2)
        torch.cuda.synchronize()
        assert torch.equal(h2, ref_h)


def check_tokens(N, S, H, dk, dv, dtype, decay="weak", additive=False, inplace=True, zero_start=False,
                 seed=7413):
    """step_tokens over S tokens per sequence against the oracle's serial
    forward over the same S tokens from the same state."""
    x = gi.gen_seq(N, S, H, dk, dv, dtype, seed=seed, h0="randn", decay=decay)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log = dev(x["g"]), dev(x["beta"]), dev(x["A_log"])
    h = None if zero_start else dev(x["h0"]).clone()
    o, hN = gdn.step_tokens(q, k, v, g, beta, A_log, h, h if (inplace and h is not None) else None,
                            additive=additive)
    torch.cuda.synchronize()
    ro, rh = _oracle().fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["g"]), f64(x["beta"]),
                           f64(x["A_log"]), None if zero_start else f64(x["h0"]), delta=not additive)
    tol = TOL[dtype]
    assert_close(f"o of {S} tokens", host(o), ro, tol)
    assert_close(f"state after {S} tokens", host(hN), rh, tol)


@pytest.mark.parametrize("S", [1, 2, 3, 4, 5])  # 2..4: all inputs loaded first; 5: token loop
@pytest.mark.parametrize("decay", ["normal", "weak"])
def test_step_tokens_bf16(S, decay):
    say(f"step_tokens bf16 N32 H16 d56 S={S} decay={decay}")
    check_tokens(32, S, 16, 56, 56, "bf16", decay=decay)


@pytest.mark.parametrize("dk,dv", [(128, 128), (100, 70), (64, 64), (65, 64), (64, 65), (5, 3)])
def test_step_tokens_head_dims(dk, dv):
    """Wide heads (state read and written per token) and narrow ones."""
    say(f"step_tokens bf16 dk={dk} dv={dv} S=3")
    check_tokens(4, 3, 2, dk, dv, "bf16")


def test_step_tokens_fp32_additive_zero_start_out_of_place():
    check_tokens(4, 4, 3, 16, 16, "f32", inplace=False)
    check_tokens(4, 3, 3, 56, 56, "bf16", additive=True)
    check_tokens(4, 3, 3, 56, 56, "bf16", zero_start=True)
    check_tokens(4, 3, 2, 128, 128, "bf16", zero_start=True)


def test_step_tokens_one_token_equals_step():
    """S = 1 is gdn_step: the same outputs bit for bit."""
    x = gi.gen_decode(8, 4, 56, 56, 1, "bf16", decay="weak")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log, h0 = dev(x["g"]), dev(x["beta"]), dev(x["A_log"]), dev(x["h0"])
    o1, h1 = gdn.step(q[0], k[0], v[0], g[0], beta[0], A_log, h0, None)
    o2, h2 = gdn.step_tokens(q[0][:, None], k[0][:, None], v[0][:, None], g[0][:, None],
                             beta[0][:, None], A_log, h0, None)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2[:, 0]) and torch.equal(h1, h2)


def test_step_tokens_empty():
    """S = 0 carries the state over (h_out = the oracle's zero-token forward
    from h_in, i.e. h_in; zeros without h_in; in place nothing changes);
    N = 0 gives empty results. Outputs start as NaN so every element is seen
    to be written."""
    import oracle as O

    say("step_tokens empty: N4 S0 H3 d56, N0 S3")
    N, H, d = 4, 3, 56
    rng = np.random.default_rng(7620)
    h_n = rng.standard_normal((N, H, d, d)).astype(np.float32)
    A_n = rng.standard_normal(H).astype(np.float32)
    cuda = torch.device("cuda")
    q = torch.empty((N, 0, H, d), dtype=torch.bfloat16, device=cuda)
    k, v = torch.empty_like(q), torch.empty_like(q)
    g = torch.empty((N, 0, H), dtype=torch.float32, device=cuda)
    beta = torch.empty_like(g)
    A_log, h_in = torch.from_numpy(A_n).to(cuda), torch.from_numpy(h_n).to(cuda)
    nan = lambda: torch.full((N, H, d, d), float("nan"), device=cuda)
    o, h_out = gdn.step_tokens(q, k, v, g, beta, A_log, h_in, nan())
    _, hz = gdn.step_tokens(q, k, v, g, beta, A_log, None, nan())
    h2 = h_in.clone()
    gdn.step_tokens(q, k, v, g, beta, A_log, h2, h2)
    qe = torch.empty((0, 3, H, d), dtype=torch.bfloat16, device=cuda)
    ge = torch.empty((0, 3, H), dtype=torch.float32, device=cuda)
    oe, he = gdn.step_tokens(qe, qe, qe, ge, ge, A_log, None)
    torch.cuda.synchronize()
    z = lambda *s: np.zeros(s)
    _, ref = O.fwd(z(N, 0, H, d), z(N, 0, H, d), z(N, 0, H, d), z(N, 0, H), z(N, 0, H),
                   A_n.astype(np.float64), h_n.astype(np.float64))
    assert o.shape == (N, 0, H, d)
    assert np.array_equal(host(h_out), ref)
    assert np.array_equal(host(hz), np.zeros((N, H, d, d)))
    assert np.array_equal(host(h2), ref)
    assert oe.shape == (0, 3, H, d) and he.shape == (0, H, d, d)


def test_prefill_then_decode():
    """A state-only forward over a 200-token prompt, then three decode tokens
    in one call from its final state (in place), equal the oracle's forward
    over all 203 tokens: the decode outputs and the final state."""
    say("prefill T200 then step_tokens S3, N4 H4 d56 bf16")
    N, H, d, T0, S = 4, 4, 56, 200, 3
    x = gi.gen_seq(N, T0 + S, H, d, d, "bf16", seed=7650, h0="randn", decay="weak")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log, h0 = dev(x["g"]), dev(x["beta"]), dev(x["A_log"]), dev(x["h0"])
    pre = lambda t: t[:, :T0].contiguous()
    new = lambda t: t[:, T0:].contiguous()
    _, h, _ = gdn.fwd(pre(q), pre(k), pre(v), pre(g), pre(beta), A_log, h0, want_o=False)
    o, h = gdn.step_tokens(new(q), new(k), new(v), new(g), new(beta), A_log, h, h)
    torch.cuda.synchronize()
    ro, rh = _oracle().fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["g"]), f64(x["beta"]),
                           f64(x["A_log"]), f64(x["h0"]))
    assert_close("decode o", host(o), ro[:, T0:], TOL["bf16"])
    assert_close("final state", host(h), rh, TOL["bf16"])


def test_draft_rollback():
    """Verification of a three-token draft out of place: h_in is left bit for
    bit; with only the first two tokens accepted, a second call over them
    from h_in gives the state the oracle reaches after those two tokens."""
    say("draft rollback N8 H4 d56 S3 -> accept 2")
    x = gi.gen_seq(8, 3, 4, 56, 56, "bf16", seed=7670, h0="randn", decay="weak")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log, h_in = dev(x["g"]), dev(x["beta"]), dev(x["A_log"]), dev(x["h0"])
    keep = h_in.clone()
    _, h3 = gdn.step_tokens(q, k, v, g, beta, A_log, h_in)
    two = lambda t: t[:, :2].contiguous()
    o2, h2 = gdn.step_tokens(two(q), two(k), two(v), two(g), two(beta), A_log, h_in)
    torch.cuda.synchronize()
    assert torch.equal(h_in, keep)
    t2 = lambda a: f64(a)[:, :2]
    ro, rh = _oracle().fwd(t2(x["q"]), t2(x["k"]), t2(x["v"]), t2(x["g"]), t2(x["beta"]), f64(x["A_log"]),
                           f64(x["h0"]))
    assert_close("o of the accepted tokens", host(o2), ro, TOL["bf16"])
    assert_close("state after the accepted tokens", host(h2), rh, TOL["bf16"])
    _, r3 = _oracle().fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["g"]), f64(x["beta"]), f64(x["A_log"]),
                          f64(x["h0"]))
    assert_close("state after the whole draft", host(h3), r3, TOL["bf16"])


@pytest.mark.parametrize("decay", ["normal", "weak"])
def test_decode_step_as_configured(decay):
    """The decode workload as configured: 256 sequences x 16 heads x d56,
    bf16 tokens, fp32 state from 0.1 N(0,1), 1024 consecutive in-place
    steps. Every output of every step and the final state are compared with
    the oracle's serial forward over the same 1024 tokens per sequence (a
    chain of oracle steps equals that forward; pinned on the CPU)."""
    c = gi.CONFIGS["decode_step"]
    N, H, dk, dv, S = c.B, c.H, c.dk, c.dv, c.steps
    say(f"step as configured N{N} H{H} d{dk} {S} steps decay={decay}")
    x = gi.gen_decode(N, H, dk, dv, S, c.dtype, seed=c.seed, decay=decay)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log = dev(x["g"]), dev(x["beta"]), dev(x["A_log"])
    h = dev(x["h0"]).clone()
    o = torch.empty((S, N, H, dv), dtype=torch.bfloat16, device=q.device)
    for t in range(S):
        gdn.step(q[t], k[t], v[t], g[t], beta[t], A_log, h, h, o=o[t])
    torch.cuda.synchronize()
    del q, k, v
    # [steps, N, H, .] -> [N, steps, H, .], one array at a time
    tr = lambda a: np.ascontiguousarray(np.swapaxes(f64(a), 0, 1))
    ro, rh = _oracle().fwd(tr(x["q"]), tr(x["k"]), tr(x["v"]), tr(x["g"]), tr(x["beta"]),
                           f64(x["A_log"]), f64(x["h0"]))
    got = np.swapaxes(host(o), 0, 1)
    assert_close(f"o, all {S} steps", got, ro, TOL["bf16"])
    assert_close("final state", host(h), rh, TOL["bf16"])
