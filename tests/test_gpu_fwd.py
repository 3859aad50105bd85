"""Forward parity: HIP chunked forward vs the fp64 oracle's serial loop, on the
same seeded inputs (bf16/fp32 values upcast exactly)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_74_amd as gdn
import gdn_inputs as gi
from gpu_util import TOL, assert_close, dev, f64, host, say

pytestmark = pytest.mark.gpu


def run_fwd(x, additive=False, with_h0=True):
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log = dev(x["g"]), dev(x["beta"]), dev(x["A_log"])
    h0 = dev(x["h0"]) if with_h0 else None
    o, hT, cs = gdn.fwd(q, k, v, g, beta, A_log, h0, additive=additive, save_context=True)
    torch.cuda.synchronize()
    return o, hT, cs


def check_fwd(x, dtype, additive=False, units=None, tol=None):
    tol = tol or TOL[dtype]
    o, hT, _ = run_fwd(x, additive)
    ro, rh = _oracle().fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["g"]), f64(x["beta"]),
                           f64(x["A_log"]), f64(x["h0"]), delta=not additive, units=units)
    go, gh = host(o), host(hT)
    if units is not None:
        H = go.shape[2]
        for u in units:
            b, h = divmod(u, H)
            assert_close(f"o[{b},:,{h}]", go[b, :, h], ro[b, :, h], tol)
            assert_close(f"hT[{b},{h}]", gh[b, h], rh[b, h], tol)
    else:
        assert_close("o", go, ro, tol)
        assert_close("hT", gh, rh, tol)


def _oracle():
    import oracle

    return oracle


def test_pr1_ref_fp32_as_configured():
    """B1 H2 T128 d16 fp32, zero initial state, chunk 64."""
    say("fwd pr1_ref fp32 as configured")
    x = gi.gen_config("pr1_ref")
    assert x["h0"] is None
    check_fwd(x, "f32")


@pytest.mark.parametrize("decay", ["normal", "weak", "zero"])
@pytest.mark.parametrize("additive", [False, True])
def test_pr1_ref_fp32(decay, additive):
    say(f"fwd pr1_ref fp32 decay={decay} additive={additive}")
    x = gi.gen_config("pr1_ref", decay=decay, h0="randn")
    check_fwd(x, "f32", additive)


@pytest.mark.parametrize("decay", ["normal", "weak", "zero"])
def test_model_shape_reduced_bf16(decay):
    say(f"fwd bf16 B2 T200 H3 d56 decay={decay}")
    x = gi.gen_seq(2, 200, 3, 56, 56, "bf16", seed=500, h0="randn", decay=decay)
    check_fwd(x, "bf16")


def test_additive_bf16():
    x = gi.gen_seq(2, 150, 2, 56, 56, "bf16", seed=501, h0="randn", decay="weak")
    check_fwd(x, "bf16", additive=True)


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 129])
def test_ragged_lengths_bf16(T):
    say(f"fwd bf16 T={T}")
    x = gi.gen_seq(1, T, 2, 56, 56, "bf16", seed=600 + T, h0="randn", decay="weak")
    check_fwd(x, "bf16")


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 32), (64, 64), (100, 100), (128, 128), (64, 40),
                                   (24, 72), (5, 9), (64, 16), (40, 56)])
def test_head_dims_bf16(dk, dv):
    """Head widths of every forward kernel; heads up to 64 wide run the
    serial pass in 32-column value blocks, including a single narrow block
    (64, 16), a partial second block (64, 40) and keys narrower than the
    values (40, 56)."""
    say(f"fwd bf16 dk={dk} dv={dv}")
    x = gi.gen_seq(1, 130, 2, dk, dv, "bf16", seed=700 + dk + dv, h0="randn", decay="weak")
    check_fwd(x, "bf16")


@pytest.mark.parametrize("dk,dv", [(16, 16), (33, 33), (64, 64), (16, 24), (3, 7)])
def test_head_dims_fp32(dk, dv):
    say(f"fwd fp32 dk={dk} dv={dv}")
    x = gi.gen_seq(1, 130, 2, dk, dv, "f32", seed=800 + dk + dv, h0="randn", decay="weak")
    check_fwd(x, "f32")


def test_zero_initial_state_and_null_outputs():
    x = gi.gen_seq(1, 100, 2, 56, 56, "bf16", seed=900, h0="none", decay="weak")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log = dev(x["g"]), dev(x["beta"]), dev(x["A_log"])
    o, hT, cs = gdn.fwd(q, k, v, g, beta, A_log, None, want_hT=False)
    assert hT is None and cs is None
    o2, hT2, _ = gdn.fwd(q, k, v, g, beta, A_log, torch.zeros(1, 2, 56, 56, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o, o2)


def test_bitwise_deterministic():
    x = gi.gen_seq(2, 300, 3, 56, 56, "bf16", seed=901, h0="randn", decay="weak")
    a = run_fwd(x)
    b = run_fwd(x)
    for u, w in zip(a, b):
        assert torch.equal(u, w)


def test_chunk_states_match_oracle_prefix_states():
    """The saved state at the start of chunk c equals the oracle's final state
    after the first 64*c tokens."""
    x = gi.gen_seq(1, 200, 2, 56, 56, "bf16", seed=902, h0="randn", decay="weak")
    o, _, ctx = run_fwd(x)
    cs = host(gdn.context_states(ctx, dev(x["q"]), dev(x["v"])))
    for c in range(4):
        t = 64 * c
        if t == 0:
            ref = f64(x["h0"])
        else:
            _, ref = _oracle().fwd(f64(x["q"])[:, :t], f64(x["k"])[:, :t], f64(x["v"])[:, :t],
                                   f64(x["g"])[:, :t], f64(x["beta"])[:, :t], f64(x["A_log"]),
                                   f64(x["h0"]))
        assert_close(f"chunk state {c}", cs[:, :, c], ref, TOL["bf16"])


@pytest.mark.parametrize("decay", ["normal", "weak"])
def test_full_size_model_forward(decay):
    """B8 H16 T4096 d56 bf16 at full size: every output and the whole final
    state against the oracle."""
    say(f"fwd full fwd_model decay={decay}")
    x = gi.gen_config("fwd_model", decay=decay)
    check_fwd(x, "bf16")


@pytest.mark.parametrize("decay", ["normal", "weak"])
def test_full_size_long_context_forward(decay):
    """B1 H16 T32768 d128 bf16, initial state 0.1 N(0,1): all 16 heads."""
    say(f"fwd full long_ctx decay={decay}")
    x = gi.gen_config("long_ctx", decay=decay)
    check_fwd(x, "bf16")


@pytest.mark.parametrize("dtype,d", [("bf16", 56), ("f32", 32)])
def test_beta_zero(dtype, d):
    """beta = 0 writes nothing: the state only decays, h_t = e^{Lambda_t} h0,
    and o_t = e^{Lambda_t} h0^T q_t (weak decay keeps h0 visible across the
    chunks)."""
    say(f"fwd beta = 0 {dtype} d{d}")
    x = gi.gen_seq(2, 200, 3, d, d, dtype, seed=7700 + d, h0="randn", decay="weak")
    x["beta"] = np.zeros_like(x["beta"])
    check_fwd(x, dtype)


@pytest.mark.parametrize("decay", ["normal", "weak", "zero"])
def test_unit_key_invariant_fp32(decay):
    """Unit-norm keys (fp32) and beta = 1: the erase is a projection, so
    h_t^T k_t = v_t after every token. Reading with q_t = k_t therefore gives
    o_t = v_t exactly (up to rounding) for every decay, through every chunk
    boundary; the final state satisfies it for the last token."""
    say(f"fwd unit-key invariant fp32 decay={decay}")
    x = gi.gen_seq(2, 200, 2, 32, 32, "f32", seed=7710, h0="randn", decay=decay)
    x["q"] = x["k"]
    x["beta"] = np.ones_like(x["beta"])
    o, hT, _ = run_fwd(x)
    v = f64(x["v"])
    assert_close("o vs v", host(o), v, TOL["f32"])
    kl = f64(x["k"])[:, -1]                                  # [B, H, dk]
    hk = np.einsum("bhij,bhi->bhj", host(hT), kl)           # hT^T k_last
    assert_close("hT^T k_last vs v_last", hk, v[:, -1], TOL["f32"])
    check_fwd(x, "f32")


@pytest.mark.parametrize("dtype,T,d", [("bf16", 2048, 56), ("bf16", 200, 128), ("f32", 130, 32)])
def test_state_only_forward(dtype, T, d):
    """o = NULL (a state-only pass, e.g. a prefill): the final state and the
    saved context equal those of the full forward bit for bit (2048 tokens
    at d 56 run two chunk ranges on two streams), and the state matches the
    oracle."""
    say(f"state-only forward B2 T{T} H4 d{d} {dtype}")
    x = gi.gen_seq(2, T, 4, d, d, dtype, seed=7640, h0="randn", decay="weak")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log, h0 = dev(x["g"]), dev(x["beta"]), dev(x["A_log"]), dev(x["h0"])
    _, hT, cs = gdn.fwd(q, k, v, g, beta, A_log, h0, save_context=True)
    o2, hT2, cs2 = gdn.fwd(q, k, v, g, beta, A_log, h0, save_context=True, want_o=False)
    torch.cuda.synchronize()
    assert o2 is None
    assert torch.equal(hT, hT2)
    assert torch.equal(cs, cs2)
    _, rh = _oracle().fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["g"]), f64(x["beta"]),
                          f64(x["A_log"]), f64(x["h0"]))
    assert_close("hT", host(hT2), rh, TOL[dtype])


@pytest.mark.parametrize("dtype,d,T,decay", [("f32", 32, 4100, "weak"), ("f32", 16, 8192, "zero"),
                                             ("f32", 64, 4096, "normal"), ("bf16", 128, 4160, "weak"),
                                             ("bf16", 100, 6000, "zero")])
def test_scan_over_chunk_ranges(dtype, d, T, decay):
    """Sequences of 64 chunks or more on the general serial pass (fp32 heads,
    bf16 heads past 64) run as a parallel scan over chunk ranges: each
    range's affine map from a zero start, the start states composed from
    them, every range rerun from its start. Outputs, final state and the
    saved chunk states against the oracle (weak and zero decay carry the
    state across every range boundary)."""
    say(f"fwd scan over chunk ranges {dtype} d{d} T{T} decay={decay}")
    x = gi.gen_seq(1, T, 2, d, d, dtype, seed=7900 + d, h0="randn", decay=decay)
    check_fwd(x, dtype)
    o, _, ctx = run_fwd(x)
    cs = host(gdn.context_states(ctx, dev(x["q"]), dev(x["v"])))
    c = 40  # a chunk inside the second range
    _, ref = _oracle().fwd(f64(x["q"])[:, :64 * c], f64(x["k"])[:, :64 * c], f64(x["v"])[:, :64 * c],
                           f64(x["g"])[:, :64 * c], f64(x["beta"])[:, :64 * c], f64(x["A_log"]),
                           f64(x["h0"]))
    assert_close(f"chunk state {c}", cs[:, :, c], ref, TOL[dtype])


def test_scan_additive_and_bitwise():
    """The scan in the additive form, and twice the same call bit for bit."""
    x = gi.gen_seq(2, 4096, 2, 32, 32, "f32", seed=7910, h0="randn", decay="weak")
    check_fwd(x, "f32", additive=True)
    a = run_fwd(x)
    b = run_fwd(x)
    for u, w in zip(a, b):
        assert torch.equal(u, w)
