"""The allocation-free forward (gdn_fwd_noalloc, workspace in a static device
array) against gdn_fwd on the same inputs: two calls in a row, the second on
a smaller input, so the second call reuses the scratch the first one left
behind; outputs, final state and saved context must agree."""
import numpy as np
import pytest
import torch

import gated_delta_rule_74_amd as gdn
import gdn_inputs as gi
from gpu_util import TOL, assert_close, dev, host, say

pytestmark = pytest.mark.gpu


def both(x, dtype):
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    g, beta, A_log, h0 = dev(x["g"]), dev(x["beta"]), dev(x["A_log"]), dev(x["h0"])
    o, hT, cs = gdn.fwd(q, k, v, g, beta, A_log, h0, save_context=True)
    o2 = torch.full_like(o, float("nan"))
    hT2 = torch.full_like(hT, float("nan"))
    cs2 = torch.zeros_like(cs)
    gdn.fwd_noalloc(q, k, v, g, beta, A_log, h0, o=o2, hT=hT2, context=cs2)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert_close("o noalloc vs gdn_fwd", host(o2), host(o), tol)
    assert_close("hT noalloc vs gdn_fwd", host(hT2), host(hT), tol)
    # one stream or two, the forward computes the same values bit for bit
    assert torch.equal(o2, o) and torch.equal(hT2, hT) and torch.equal(cs2, cs)


def test_noalloc_matches_fwd_twice():
    say("fwd_noalloc: B2 T2048 H8 d56 bf16, then B1 T300 H2 d56 bf16")
    big = gi.gen_seq(2, 2048, 8, 56, 56, "bf16", seed=7800, h0="randn", decay="weak")
    both(big, "bf16")
    small = gi.gen_seq(1, 300, 2, 56, 56, "bf16", seed=7801, h0="randn", decay="weak")
    both(small, "bf16")


def test_noalloc_fp32_and_too_large():
    say("fwd_noalloc: B1 T200 H2 d32 fp32; a shape beyond the scratch is refused")
    x = gi.gen_seq(1, 200, 2, 32, 32, "f32", seed=7802, h0="randn", decay="weak")
    both(x, "f32")
    q = torch.zeros((8, 4096, 16, 56), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((8, 4096, 16), device="cuda")
    with pytest.raises(gdn.GdnError) as e:
        gdn.fwd_noalloc(q, q, q, g, g, torch.zeros(16, device="cuda"), o=torch.empty_like(q))
    assert e.value.status == 3
