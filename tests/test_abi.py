"""C-ABI checks that need no GPU: the library loads, exports every function
include/gdn.h declares, and rejects bad arguments before launching anything
(every call here returns during validation, so no device is touched)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_74_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EINVAL, EUNSUPPORTED, EWORKSPACE = 1, 2, 3


def header_functions():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gdn.LIB_PATH):
        pytest.skip("libgdn.so not built (run __graft_entry__.build())")
    return gdn.lib()


def test_exports_every_declared_function(L):
    names = header_functions()
    assert set(names) == set(gdn.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in range(5):
        assert L.gdn_status_string(code)
    assert L.gdn_status_string(99) == b"unknown status"


# fake, suitably aligned device addresses; validation never dereferences them
def fake(i, size=1 << 30):
    return ctypes.c_void_p(0x7F0000000000 + i * size)


def fwd_call(L, shape, **over):
    args = dict(q=fake(1), k=fake(2), v=fake(3), g=fake(4), beta=fake(5), A_log=fake(6), D=None, h0=None,
                o=fake(7), hT=None, cs=None, ws=fake(30), ws_bytes=1 << 30)
    args.update(over)
    return L.gdn_fwd(ctypes.byref(shape), args["q"], args["k"], args["v"], args["g"], args["beta"],
                     args["A_log"], args["D"], args["h0"], args["o"], args["hT"], args["cs"], args["ws"],
                     args["ws_bytes"], None)


def test_fwd_rejects_bad_shapes(L):
    good = dict(B=1, T=8, H=2, dk=16, dv=16, dtype=1, chunk=64, flags=0)
    for key, val, code in [("B", 0, EINVAL), ("T", -1, EINVAL), ("H", -1, EINVAL), ("dk", 0, EINVAL),
                           ("dv", 129, EINVAL), ("dtype", 7, EINVAL), ("chunk", 32, EUNSUPPORTED),
                           ("flags", 8, EINVAL)]:
        d = dict(good, **{key: val})
        s = gdn.Shape(*[d[f] for f, _ in gdn.Shape._fields_])
        assert fwd_call(L, s) == code, key
        assert L.gdn_last_error_detail()
    s = gdn.Shape(1, 8, 2, 65, 16, 0, 64, 0)  # fp32 above 64
    assert fwd_call(L, s) == EUNSUPPORTED
    assert L.gdn_fwd(None, *[None] * 11, None, 0, None) == EINVAL
    s = gdn.Shape(1, 8, 2, 16, 16, 1, 64, 0)
    assert fwd_call(L, s, ws=None) == EWORKSPACE
    assert fwd_call(L, s, ws_bytes=16) == EWORKSPACE
    assert fwd_call(L, s, cs=ctypes.c_void_p(fake(8).value + 16)) == EINVAL  # ctx misaligned


def test_fwd_rejects_null_misaligned_and_aliased(L):
    s = gdn.Shape(1, 8, 2, 16, 16, 1, 64, 0)
    assert fwd_call(L, s, q=None) == EINVAL
    assert fwd_call(L, s, A_log=None) == EINVAL
    assert fwd_call(L, s, o=None, hT=fake(4)) == EINVAL  # state-only pass still checks aliasing
    assert fwd_call(L, s, k=ctypes.c_void_p(fake(2).value + 2)) == EINVAL
    assert fwd_call(L, s, o=fake(1)) == EINVAL  # o aliases q
    assert b"overlaps" in L.gdn_last_error_detail()
    assert fwd_call(L, s, hT=fake(4)) == EINVAL  # hT aliases g
    assert fwd_call(L, s, D=ctypes.c_void_p(fake(9).value + 2)) == EINVAL  # D misaligned
    assert fwd_call(L, s, D=fake(7)) == EINVAL  # D inside o
    assert b"overlaps" in L.gdn_last_error_detail()


def test_edge_flag_and_skip_pass_validation(L):
    """The key-normalisation flag is a known bit and a separate D array is
    accepted; what fails then is only the missing workspace."""
    s = gdn.Shape(1, 8, 2, 16, 16, 1, 64, gdn.GDN_FLAG_L2NORM_K | gdn.GDN_FLAG_ADDITIVE)
    assert fwd_call(L, s, D=fake(9), ws=None) == EWORKSPACE
    s = gdn.Shape(2, 100, 3, 56, 56, 1, 64, gdn.GDN_FLAG_L2NORM_K)
    need = L.gdn_bwd_workspace_size(ctypes.byref(s))
    assert bwd_call(L, s, D=fake(17), dD=fake(18)) == EWORKSPACE
    assert bwd_call(L, s, ws=fake(20), ws_bytes=need, dD=fake(14)) == EINVAL  # dD aliases dA_log
    assert bwd_call(L, s, ws=fake(20), ws_bytes=need, D=fake(12)) == EINVAL  # D inside dg


def bwd_call(L, shape, ws=None, ws_bytes=0, **over):
    a = dict(q=fake(1), k=fake(2), v=fake(3), g=fake(4), beta=fake(5), A_log=fake(6), D=None, h0=None,
             cs=None, do=fake(8), dhT=None, dq=fake(9), dk=fake(10), dv=fake(11), dg=fake(12),
             dbeta=fake(13), dA=fake(14), dD=None, dh0=None, hT=None)
    a.update(over)
    return L.gdn_bwd(ctypes.byref(shape), a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"],
                     a["D"], a["h0"], a["cs"], a["do"], a["dhT"], a["dq"], a["dk"], a["dv"], a["dg"],
                     a["dbeta"], a["dA"], a["dD"], a["dh0"], a["hT"], ws, ws_bytes, None)


def test_bwd_validation(L):
    s = gdn.Shape(2, 100, 3, 56, 56, 1, 64, 0)
    need = L.gdn_bwd_workspace_size(ctypes.byref(s))
    assert need > 0
    assert bwd_call(L, s) == EWORKSPACE
    assert bwd_call(L, s, ws=fake(20), ws_bytes=need - 1) == EWORKSPACE
    assert bwd_call(L, s, ws=fake(20), ws_bytes=need, dq=None) == EINVAL
    assert bwd_call(L, s, ws=fake(20), ws_bytes=need, cs=fake(15), hT=fake(16)) == EINVAL
    assert bwd_call(L, gdn.Shape(1, 8, 2, 100, 100, 0, 64, 0), ws=fake(20), ws_bytes=need) == EUNSUPPORTED
    assert bwd_call(L, s, ws=fake(20), ws_bytes=need, dq=fake(1)) == EINVAL  # dq aliases q
    assert bwd_call(L, s, ws=fake(20), ws_bytes=need, dk=fake(20)) == EINVAL  # dk in workspace


def test_workspace_and_context_sizes(L):
    s = gdn.Shape(8, 4096, 16, 56, 56, 1, 64, 0)
    states = 8 * 16 * 64 * 56 * 56 * 2
    blocks = 8 * 16 * 64 * 64 * 56 * 2
    tms = 8 * 16 * 64 * 64 * 64 * 2
    ctx = L.gdn_fwd_context_size(ctypes.byref(s))
    # chunk-start states, -Kw and U of every chunk, and (I + L)^{-1} per chunk
    assert ctx >= states + 2 * blocks + tms and ctx < states + 2 * blocks + tms + 1024
    assert L.gdn_fwd_workspace_size(ctypes.byref(s)) >= 2 * blocks
    assert L.gdn_bwd_workspace_size(ctypes.byref(s)) >= ctx + states + 8 * 16 * 64 * 4
    empty = gdn.Shape(2, 0, 3, 16, 16, 1, 64, 0)  # T = 0: no chunk, no context
    assert L.gdn_fwd_context_size(ctypes.byref(empty)) == 0
    bad = gdn.Shape(0, 1, 1, 1, 1, 1, 64, 0)
    assert L.gdn_fwd_context_size(ctypes.byref(bad)) == 0
    assert L.gdn_fwd_workspace_size(ctypes.byref(bad)) == 0


def test_step_validation(L):
    P = fake
    ok = (P(1), P(2), P(3), P(4), P(5), P(6), None, None, P(7), P(8))  # D, h_in NULL
    assert L.gdn_step(-1, 16, 56, 56, 1, 0, *ok, None) == EINVAL
    assert L.gdn_step(4, 16, 0, 56, 1, 0, *ok, None) == EINVAL
    assert L.gdn_step(4, 16, 56, 56, 3, 0, *ok, None) == EINVAL
    assert L.gdn_step(4, 16, 56, 56, 1, 8, *ok, None) == EINVAL
    bad = list(ok)
    bad[8] = P(1)  # h_out aliases q
    assert L.gdn_step(4, 16, 56, 56, 1, 0, *bad, None) == EINVAL
    bad = list(ok)
    bad[7] = ctypes.c_void_p(P(7).value + 64)  # h_in partially overlaps h_out
    assert L.gdn_step(4, 16, 56, 56, 1, 0, *bad, None) == EINVAL
    bad = list(ok)
    bad[6] = P(8)  # D inside o
    assert L.gdn_step(4, 16, 56, 56, 1, gdn.GDN_FLAG_L2NORM_K, *bad, None) == EINVAL


def test_step_tokens_validation(L):
    P = fake
    ok = (P(1), P(2), P(3), P(4), P(5), P(6), None, None, P(7), P(8))  # D, h_in NULL
    assert L.gdn_step_tokens(4, -1, 16, 56, 56, 1, 0, *ok, None) == EINVAL  # S < 0
    assert L.gdn_step_tokens(-1, 3, 16, 56, 56, 1, 0, *ok, None) == EINVAL
    assert L.gdn_step_tokens(4, 3, 16, 56, 129, 1, 0, *ok, None) == EINVAL
    assert L.gdn_step_tokens(4, 3, 16, 56, 56, 1, 8, *ok, None) == EINVAL
    bad = list(ok)
    bad[9] = P(3)  # o aliases v
    assert L.gdn_step_tokens(4, 3, 16, 56, 56, 1, 0, *bad, None) == EINVAL
    # o of S tokens runs into h_out when placed S - 1 token rows below it
    bad = list(ok)
    bad[9] = ctypes.c_void_p(P(7).value - 2 * 4 * 16 * 56)
    assert L.gdn_step_tokens(4, 3, 16, 56, 56, 1, 0, *bad, None) == EINVAL


def test_product_path_has_no_cpu_fallback():
    """The binding must not reach the oracle or any host implementation."""
    src = open(os.path.join(ROOT, "gated_delta_rule_74_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("no fallback", "")
    assert "import numpy" not in src


def test_empty_sequence_host_logic(L):
    """T = 0 needs neither the T-sized arrays nor a workspace; with no state
    output requested nothing is launched (so this runs without a GPU), and
    the backward still requires dA_log and rejects aliasing of its outputs."""
    s = gdn.Shape(2, 0, 3, 16, 16, 1, 64, 0)
    assert L.gdn_fwd(ctypes.byref(s), *[None] * 8, None, None, None, None, 0, None) == 0
    assert L.gdn_fwd(ctypes.byref(s), *[None] * 7, fake(1), None, fake(1), None, None, 0, None) == EINVAL
    args = [None] * 21 + [0, None]
    assert L.gdn_bwd(ctypes.byref(s), *args) == EINVAL  # dA_log NULL
    a = list(args)
    a[16], a[18] = fake(2), fake(2)  # dA_log and dh0 overlap
    assert L.gdn_bwd(ctypes.byref(s), *a) == EINVAL
    a = list(args)
    a[16], a[17] = fake(2), ctypes.c_void_p(fake(2).value + 4)  # dA_log and dD overlap
    assert L.gdn_bwd(ctypes.byref(s), *a) == EINVAL


def test_empty_decode_host_logic(L):
    """N = 0 does nothing; S = 0 carries the state over (in place: nothing to
    launch, so this runs without a GPU) and still needs h_out and rejects a
    partial overlap of the states."""
    assert L.gdn_step_tokens(0, 3, 16, 56, 56, 1, 0, *[None] * 11) == 0
    assert L.gdn_step(0, 16, 56, 56, 1, 0, *[None] * 11) == 0
    h = fake(3)
    assert L.gdn_step_tokens(4, 0, 16, 56, 56, 1, 0, *[None] * 7, h, h, None, None) == 0
    assert L.gdn_step_tokens(4, 0, 16, 56, 56, 1, 0, *[None] * 7, h, None, None, None) == EINVAL
    shifted = ctypes.c_void_p(h.value + 4)
    assert L.gdn_step_tokens(4, 0, 16, 56, 56, 1, 0, *[None] * 7, h, shifted, None, None) == EINVAL


def test_fwd_noalloc_validation(L):
    """The allocation-free forward rejects a shape whose workspace exceeds its
    static scratch, and bad arguments, before any device call."""
    s = gdn.Shape(8, 4096, 16, 56, 56, 1, 64, 0)  # the layer shape: far beyond 64 MiB
    need = L.gdn_fwd_workspace_size(ctypes.byref(s))
    assert need > gdn.NOALLOC_SCRATCH_BYTES
    args = [fake(i) for i in range(1, 7)] + [None, None, fake(7), None, None, None]
    assert L.gdn_fwd_noalloc(ctypes.byref(s), *args) == EWORKSPACE
    assert b"static scratch" in L.gdn_last_error_detail()
    small = gdn.Shape(1, 256, 4, 56, 56, 1, 64, 0)
    assert L.gdn_fwd_workspace_size(ctypes.byref(small)) <= gdn.NOALLOC_SCRATCH_BYTES
    bad = list(args)
    bad[0] = None  # q
    assert L.gdn_fwd_noalloc(ctypes.byref(small), *bad) == EINVAL
    bad = list(args)
    bad[8] = args[0]  # o aliases q
    assert L.gdn_fwd_noalloc(ctypes.byref(small), *bad) == EINVAL
    assert L.gdn_fwd_noalloc(ctypes.byref(gdn.Shape(1, 8, 2, 16, 16, 1, 32, 0)), *args) == EUNSUPPORTED


def test_exports_only_declared_c_symbols():
    """The library's exported C-linkage functions are exactly the ones
    include/gdn.h declares (internal helpers stay out of the ABI)."""
    import shutil
    import subprocess
    if not shutil.which("nm"):
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if len(ln.split()) == 3 and ln.split()[1] == "T"}
    c_syms = {x for x in syms if not x.startswith("_Z") and not x.startswith("_")}
    assert c_syms == set(header_functions())
