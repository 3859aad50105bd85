"""Backward parity: HIP reverse-chunk backward vs the oracle's manual reverse
pass of the serial loop, for every gradient, on the same seeded inputs."""
import numpy as np
import pytest
import torch

import gated_delta_rule_74_amd as gdn
import gdn_inputs as gi
from gpu_util import TOL, assert_close, dev, f64, host, say

pytestmark = pytest.mark.gpu

GRADS = ["dq", "dk", "dv", "dg", "dbeta", "dh0"]


def _oracle():
    import oracle

    return oracle


def with_dhT(x, seed):
    B, _, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    rng = np.random.default_rng(seed)
    x = dict(x)
    x["dhT"] = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    if x["h0"] is None:
        x["h0"] = (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32)
    return x


def run_bwd(x, additive=False, use_saved=True, want_hT=False):
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log = dev(x["g"]), dev(x["beta"]), dev(x["A_log"])
    h0, do, dhT = dev(x["h0"]), dev(x["do"]), dev(x.get("dhT"))
    cs = None
    if use_saved:
        _, _, cs = gdn.fwd(q, k, v, g, beta, A_log, h0, additive=additive, save_context=True,
                           want_hT=False)
    r = gdn.bwd(q, k, v, g, beta, A_log, do, h0, dhT, context=cs, additive=additive,
                want_hT=want_hT)
    torch.cuda.synchronize()
    return r


def check_bwd(x, dtype, additive=False, units=None, tol=None, use_saved=True):
    tol = tol or TOL[dtype]
    r = run_bwd(x, additive, use_saved)
    ref = _oracle().bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["g"]), f64(x["beta"]),
                        f64(x["A_log"]), f64(x["h0"]), f64(x["do"]), f64(x.get("dhT")),
                        delta=not additive, units=units)
    got = {kk: host(vv) for kk, vv in r.items() if vv is not None}
    if units is None:
        for name in GRADS:
            assert_close(name, got[name], ref[name], tol)
        assert_close("dA_log", got["dA_log"], ref["dA_log"], tol)
    else:
        H = got["dq"].shape[2]
        for u in units:
            b, h = divmod(u, H)
            for name in ["dq", "dk", "dv", "dg", "dbeta"]:
                assert_close(f"{name}[{b},:,{h}]", got[name][b, :, h], ref[name][b, :, h], tol)
            assert_close(f"dh0[{b},{h}]", got["dh0"][b, h], ref["dh0"][b, h], tol)
        # dA_log[h] = sum_{b,t} g dg holds for any size; check it on the GPU outputs
        ident = np.sum(f64(x["g"]) * got["dg"], axis=(0, 1))
        assert_close("dA_log vs sum g*dg", got["dA_log"], ident, 1e-3)
    return r


def test_pr1_shape_fp32():
    say("bwd fp32 B1 H2 T128 d16")
    x = gi.gen_config("pr1_ref", decay="weak", h0="randn", with_do=True)
    check_bwd(with_dhT(x, 1), "f32")


@pytest.mark.parametrize("decay", ["normal", "weak", "zero"])
def test_fp32_decays(decay):
    say(f"bwd fp32 d16 decay={decay}")
    x = gi.gen_seq(2, 150, 2, 16, 16, "f32", seed=1001, h0="randn", with_do=True, decay=decay)
    check_bwd(with_dhT(x, 2), "f32")


@pytest.mark.parametrize("decay", ["normal", "weak", "zero"])
def test_model_shape_reduced_bf16(decay):
    say(f"bwd bf16 B2 T200 H3 d56 decay={decay}")
    x = gi.gen_seq(2, 200, 3, 56, 56, "bf16", seed=1002, h0="randn", with_do=True, decay=decay)
    check_bwd(with_dhT(x, 3), "bf16")


def test_additive_fp32_and_bf16():
    x = gi.gen_seq(1, 140, 2, 16, 16, "f32", seed=1003, h0="randn", with_do=True, decay="weak")
    check_bwd(with_dhT(x, 4), "f32", additive=True)
    x = gi.gen_seq(1, 140, 2, 56, 56, "bf16", seed=1004, h0="randn", with_do=True, decay="weak")
    check_bwd(with_dhT(x, 5), "bf16", additive=True)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 130])
def test_ragged_lengths_bf16(T):
    say(f"bwd bf16 T={T}")
    x = gi.gen_seq(1, T, 2, 56, 56, "bf16", seed=1100 + T, h0="randn", with_do=True, decay="weak")
    check_bwd(with_dhT(x, 6), "bf16")


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 64), (48, 24), (5, 9)])
def test_head_dims_bf16(dk, dv):
    say(f"bwd bf16 dk={dk} dv={dv}")
    x = gi.gen_seq(1, 130, 2, dk, dv, "bf16", seed=1200 + dk, h0="randn", with_do=True, decay="weak")
    check_bwd(with_dhT(x, 7), "bf16")


@pytest.mark.parametrize("dk,dv", [(128, 128), (100, 70), (72, 128)])
def test_wide_head_dims_bf16(dk, dv):
    """Head dims past 64 (bf16): the local gradients run in the wide-head
    kernel, the reverse state pass in the LDS-staged chain kernel."""
    say(f"bwd bf16 wide dk={dk} dv={dv}")
    x = gi.gen_seq(1, 150, 2, dk, dv, "bf16", seed=1250 + dk, h0="randn", with_do=True, decay="weak")
    check_bwd(with_dhT(x, 11), "bf16")


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 64), (40, 24)])
def test_wide_head_dims_fp32(dk, dv):
    say(f"bwd fp32 wide dk={dk} dv={dv}")
    x = gi.gen_seq(1, 140, 2, dk, dv, "f32", seed=1260 + dk, h0="randn", with_do=True, decay="weak")
    check_bwd(with_dhT(x, 12), "f32")


def test_wide_head_additive_and_recompute():
    x = with_dhT(gi.gen_seq(1, 100, 2, 128, 128, "bf16", seed=1270, h0="randn", with_do=True,
                            decay="weak"), 13)
    check_bwd(x, "bf16", additive=True)
    a = run_bwd(x, use_saved=True)
    b = run_bwd(x, use_saved=False)
    for name in GRADS + ["dA_log"]:
        assert torch.equal(a[name], b[name]), name


def test_recompute_path_equals_saved_states_path():
    x = with_dhT(gi.gen_seq(2, 200, 2, 56, 56, "bf16", seed=1300, h0="randn", with_do=True,
                            decay="weak"), 8)
    a = run_bwd(x, use_saved=True)
    b = run_bwd(x, use_saved=False, want_hT=True)
    for name in GRADS + ["dA_log"]:
        assert torch.equal(a[name], b[name]), name
    _, rh = _oracle().fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["g"]), f64(x["beta"]),
                          f64(x["A_log"]), f64(x["h0"]))
    assert_close("recomputed hT", host(b["hT"]), rh, TOL["bf16"])


def test_bitwise_deterministic():
    x = with_dhT(gi.gen_seq(2, 300, 3, 56, 56, "bf16", seed=1301, h0="randn", with_do=True,
                            decay="weak"), 9)
    a = run_bwd(x)
    b = run_bwd(x)
    for name in GRADS + ["dA_log"]:
        assert torch.equal(a[name], b[name]), name


def test_autograd_function():
    x = gi.gen_seq(1, 100, 2, 56, 56, "bf16", seed=1302, h0="randn", with_do=True, decay="weak")
    ts = {kk: dev(x[kk]).requires_grad_(kk not in ("do",)) for kk in
          ("q", "k", "v", "g", "beta", "A_log", "h0")}
    o, hT = gdn.GatedDeltaRule.apply(ts["q"], ts["k"], ts["v"], ts["g"], ts["beta"], ts["A_log"],
                                     ts["h0"])
    o.backward(dev(x["do"]))
    ref = _oracle().bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["g"]), f64(x["beta"]),
                        f64(x["A_log"]), f64(x["h0"]), f64(x["do"]), None)
    for name, key in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
                      ("A_log", "dA_log"), ("h0", "dh0")]:
        assert_close(f"autograd {key}", host(ts[name].grad), ref[key], TOL["bf16"])


@pytest.mark.parametrize("decay", ["normal", "weak"])
def test_full_size_long_context_fwdbwd(decay):
    """B1 H16 T32768 d128 bf16, nonzero initial state (the long-context
    configuration; with weak decay the 512-step chain matters): every
    gradient of every head, and dA_log, against the oracle."""
    say(f"bwd full long_ctx decay={decay}")
    x = gi.gen_config("long_ctx", decay=decay)
    check_bwd(x, "bf16")


@pytest.mark.parametrize("decay", ["normal", "weak"])
def test_full_size_fwdbwd(decay):
    """B8 H16 T4096 d56 bf16 at full size with the launch configuration the
    benchmark times (saved context): every gradient of every (b, h) unit, and
    dA_log, against the oracle."""
    say(f"bwd full fwdbwd_model decay={decay}")
    x = gi.gen_config("fwdbwd_model", decay=decay)
    check_bwd(x, "bf16")


@pytest.mark.parametrize("dtype,d", [("bf16", 56), ("f32", 16)])
def test_beta_zero(dtype, d):
    """beta = 0: nothing is written, yet dbeta is not zero (every write's
    effect is still differentiated); all gradients against the oracle."""
    say(f"bwd beta = 0 {dtype} d{d}")
    x = gi.gen_seq(2, 200, 3, d, d, dtype, seed=7720 + d, h0="randn", with_do=True, decay="weak")
    x["beta"] = np.zeros_like(x["beta"])
    check_bwd(with_dhT(x, 14), dtype)


def test_fwd_bwd_graph_replay():
    """One forward (context saved, the prep of later chunk ranges on a second
    stream) plus backward captured in a HIP graph gives the eager results bit
    for bit on every replay, with eager work and synchronisations between
    replays."""
    say("fwd+bwd graph replay B1 T2048 H4 d56 (two chunk ranges, so both streams)")
    x = gi.gen_seq(1, 2048, 4, 56, 56, "bf16", seed=7430, h0="randn", with_do=True, decay="weak")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log, h0, do = dev(x["g"]), dev(x["beta"]), dev(x["A_log"]), dev(x["h0"]), dev(x["do"])
    o = torch.empty_like(v)
    hT = torch.empty_like(h0)
    ctx = torch.empty(gdn.context_size(q, v), dtype=torch.uint8, device=q.device)
    fws = torch.empty(gdn.fwd_workspace_size(q, v), dtype=torch.uint8, device=q.device)
    bws = torch.empty(gdn.bwd_workspace_size(q, v), dtype=torch.uint8, device=q.device)
    grads = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
             "dg": torch.empty_like(g), "dbeta": torch.empty_like(beta), "dA_log": torch.empty_like(A_log),
             "dh0": torch.empty_like(h0)}

    def step():
        gdn.fwd(q, k, v, g, beta, A_log, h0, o=o, hT=hT, context=ctx, workspace=fws)
        gdn.bwd(q, k, v, g, beta, A_log, do, h0, None, context=ctx, workspace=bws, out=grads)

    step()
    torch.cuda.synchronize()
    outs = {"o": o, "hT": hT, **{kk: vv for kk, vv in grads.items() if vv is not None}}
    ref = {kk: vv.clone() for kk, vv in outs.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in outs.values():
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t in outs.items():
            assert torch.equal(t, ref[name]), f"{name} differs on replay {rep}"
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o, ref["o"])


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 56), (torch.bfloat16, 128), (torch.float32, 16)])
def test_empty_sequence(dtype, d):
    """T = 0: no step runs. Forward: hT = h0 (zeros without h0); backward:
    dh0 = dhT (zeros without dhT), dA_log = 0, the recomputed hT = h0, all
    against the oracle's zero-step results. Outputs start as NaN so that every
    element is seen to be written."""
    say(f"empty sequence B2 T0 H3 d{d} {dtype}")
    O = _oracle()
    B, H = 2, 3
    rng = np.random.default_rng(7610)
    h0n = rng.standard_normal((B, H, d, d)).astype(np.float32)
    dhTn = rng.standard_normal((B, H, d, d)).astype(np.float32)
    A_logn = rng.standard_normal(H).astype(np.float32)
    cuda = torch.device("cuda")
    q = torch.empty((B, 0, H, d), dtype=dtype, device=cuda)
    k, v, do = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    g = torch.empty((B, 0, H), dtype=torch.float32, device=cuda)
    beta = torch.empty_like(g)
    A_log, h0, dhT = (torch.from_numpy(x).to(cuda) for x in (A_logn, h0n, dhTn))
    nan = lambda: torch.full((B, H, d, d), float("nan"), device=cuda)
    o, hT, cs = gdn.fwd(q, k, v, g, beta, A_log, h0, hT=nan(), save_context=True)
    _, hz, _ = gdn.fwd(q, k, v, g, beta, A_log, None, hT=nan())
    out = {"dA_log": torch.full((H,), float("nan"), device=cuda), "dh0": nan(), "hT": nan()}
    r = gdn.bwd(q, k, v, g, beta, A_log, do, h0, dhT, want_hT=True, out=out)
    r0 = gdn.bwd(q, k, v, g, beta, A_log, do, h0, None, context=cs,
                 out={"dA_log": torch.full((H,), float("nan"), device=cuda), "dh0": nan()})
    torch.cuda.synchronize()
    z = lambda *s: np.zeros(s)
    args = (z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H), z(B, 0, H), A_logn.astype(np.float64))
    _, ref_hT = O.fwd(*args, h0n.astype(np.float64))
    rg = O.bwd(*args, h0n.astype(np.float64), z(B, 0, H, d), dhTn.astype(np.float64))
    assert o.shape == (B, 0, H, d)
    assert np.array_equal(host(hT), ref_hT)
    assert np.array_equal(host(hz), np.zeros((B, H, d, d)))
    assert np.array_equal(host(r["dh0"]), rg["dh0"])
    assert np.array_equal(host(r["dA_log"]), rg["dA_log"])
    assert np.array_equal(host(r["hT"]), ref_hT)
    assert np.array_equal(host(r0["dh0"]), np.zeros((B, H, d, d)))
    assert np.array_equal(host(r0["dA_log"]), np.zeros(H))
    assert r["dq"].shape == (B, 0, H, d) and r["dg"].shape == (B, 0, H)


def test_max_size_fwdbwd():
    """Tensors just below the 2^31-element limit: B1 H8 T2097088 d128 bf16
    (q holds 2,147,418,112 elements; ~91 GB of device memory in all). The
    inputs repeat a seeded block of P = 4099 tokens (not a power of two, so
    an address that wrapped by any power of two would read other values).
    The gate of token r = T - 129 is 200 (A <= -1 here), so its decay
    exp(g A) underflows to 0: the state is reset there and the tokens from r
    on are a sequence of their own, which the oracle computes from a zero
    state; do is zero before r. Checked against the oracle: o on the first 128 tokens (from
    h0), o, hT and every gradient from r on; before r every gradient, and
    dh0, must vanish."""
    O = _oracle()
    B, H, d, P = 1, 8, 128, 4099
    T = (1 << 21) - 64
    r = T - 129
    say(f"max size B{B} T{T} H{H} d{d} bf16, reset at token {r}")
    x = gi.gen_seq(1, P, H, d, d, "bf16", seed=7630, h0="randn", with_do=True, decay="normal")
    reps = -(-T // P)

    def big(t):
        t = dev(t)
        return t.repeat(1, reps, *([1] * (t.dim() - 2)))[:, :T]

    q, k, v, beta = big(x["q"]), big(x["k"]), big(x["v"]), big(x["beta"])
    g = big(x["g"]).clone()
    g[0, r, :] = 200.0
    A_log, h0 = dev(x["A_log"]), dev(x["h0"])
    tail = np.arange(r, T) % P
    do = torch.zeros_like(q)
    do[0, r:] = dev(x["do"])[0, torch.from_numpy(tail).to(q.device)]
    torch.cuda.synchronize()
    o, hT, cs = gdn.fwd(q, k, v, g, beta, A_log, h0, save_context=True)
    res = gdn.bwd(q, k, v, g, beta, A_log, do, h0, context=cs)
    torch.cuda.synchronize()
    tol = TOL["bf16"]
    # head: the first 128 tokens from h0
    head = lambda a: f64(a)[:, :128]
    ro, _ = O.fwd(head(x["q"]), head(x["k"]), head(x["v"]), head(x["g"]), head(x["beta"]),
                  f64(x["A_log"]), f64(x["h0"]))
    assert_close("o head", host(o[:, :128]), ro, tol)
    # tail: tokens r.. from a zero state
    tl = lambda a: f64(a)[:, tail]
    gt = tl(x["g"])
    gt[0, 0, :] = 200.0
    args = (tl(x["q"]), tl(x["k"]), tl(x["v"]), gt, tl(x["beta"]), f64(x["A_log"]))
    ro, rh = O.fwd(*args, None)
    assert_close("o tail", host(o[:, r:]), ro, tol)
    assert_close("hT", host(hT), rh, tol)
    rg = O.bwd(*args, None, tl(x["do"]), None)
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        assert_close(f"{name} tail", host(res[name][:, r:]), rg[name], tol)
    assert_close("dA_log", host(res["dA_log"]), rg["dA_log"], tol)
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        m = res[name][:, :r].abs().max().item()
        assert m <= 1e-30, f"{name} before the reset: max |.| = {m}"
    assert res["dh0"].abs().max().item() <= 1e-30
    del q, k, v, g, beta, do, o, hT, cs, res
    torch.cuda.empty_cache()


def test_caller_stream():
    """Work goes on the caller's current stream: forward (two chunk ranges,
    so the second internal stream forks from and joins the caller's), backward
    and a decode call issued on a side stream, on inputs written by that
    stream just before, equal the default-stream results bit for bit."""
    say("caller stream: fwd+bwd B1 T2048 H4 d56, step_tokens S3")
    x = gi.gen_seq(1, 2048, 4, 56, 56, "bf16", seed=7660, h0="randn", with_do=True, decay="weak")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log, h0, do = dev(x["g"]), dev(x["beta"]), dev(x["A_log"]), dev(x["h0"]), dev(x["do"])
    t3 = lambda t: t[:, -3:].contiguous()

    def run(q, k, v, g, beta, h0, do):
        o, hT, cs = gdn.fwd(q, k, v, g, beta, A_log, h0, save_context=True)
        r = gdn.bwd(q, k, v, g, beta, A_log, do, h0, context=cs)
        h = hT.clone()
        od, _ = gdn.step_tokens(t3(q), t3(k), t3(v), t3(g), t3(beta), A_log, h, h)
        return dict(r, o=o, hT=hT, od=od, hd=h)

    ref = run(q, k, v, g, beta, h0, do)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ins = [t.clone() for t in (q, k, v, g, beta, h0, do)]
        got = run(*ins)
    torch.cuda.synchronize()
    for name, t in ref.items():
        if t is not None:
            assert torch.equal(got[name], t), name


@pytest.mark.parametrize("dtype,d,T,decay", [("f32", 32, 4100, "weak"), ("f32", 16, 8192, "zero"),
                                             ("bf16", 128, 4160, "weak"), ("bf16", 72, 6000, "normal")])
def test_scan_over_chunk_ranges(dtype, d, T, decay):
    """The reverse pass as a parallel scan over chunk ranges (mirror of the
    forward's): every gradient, dh0 and dA_log against the oracle, with a
    nonzero upstream dhT; the recomputing path equals the saved-context path
    bit for bit."""
    say(f"bwd scan over chunk ranges {dtype} d{d} T{T} decay={decay}")
    x = with_dhT(gi.gen_seq(1, T, 2, d, d, dtype, seed=7920 + d, h0="randn", with_do=True, decay=decay), 15)
    check_bwd(x, dtype)
    a = run_bwd(x, use_saved=True)
    b = run_bwd(x, use_saved=False)
    for name in GRADS + ["dA_log"]:
        assert torch.equal(a[name], b[name]), name


def test_scan_additive_bwd():
    x = with_dhT(gi.gen_seq(1, 4096, 2, 32, 32, "f32", seed=7930, h0="randn", with_do=True, decay="weak"), 16)
    check_bwd(x, "f32", additive=True)
