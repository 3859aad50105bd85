"""Seeded synthetic inputs for the gated delta rule, shared by the oracle side
and the HIP side (this module holds none of the method's arithmetic: only
random draws, the per-token L2 normalisation of k that the workload recipe
asks for, and the float32 -> bfloat16 round-to-nearest-even cast).

Recipe (numpy ``Generator(PCG64(seed))``; normals drawn in float64):
  draw order q, k, v, beta-logits, g-logits, A_log, h0, do
  q, v, do ~ N(0, 1);  k ~ N(0, 1) then L2-normalised per (b, t, h) row
  beta = sigmoid(N(0, 1)), g = sigmoid(N(0, 1))          (float32)
  A_log ~ U(0, ln 16) per head                              (float32)
  weak-decay variant: A_log ~ U(ln 1e-3, ln 1e-1) and seed + 100
  g-zero variant: g == 0 exactly (no decay)
  h0 = 0.1 * N(0, 1) when requested (float32)
  layer-edge variants, drawn after everything above so the other draws stay
  the same: raw keys (key_spread) = the unit rows times a per-row length
  drawn U(0.25, 4); skip weights (with_D) D ~ N(0, 1) per head (float32)
  q, k, v, do are then rounded to the workload dtype (bf16: RNE).

The decode workload draws its per-step tokens in blocks of steps, each block
in the order q, k, v, beta-logits, g-logits, so memory stays bounded.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# ------------------------------------------------------------------ bf16 cast


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).
    Returns the 16-bit patterns as uint16. Inputs here are finite."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    bits = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Tensor:
    """A host array in its storage dtype: 'bf16' (uint16 bit patterns) or 'f32'."""

    data: np.ndarray
    dtype: str

    @property
    def shape(self):
        return self.data.shape

    def f64(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.data).astype(np.float64)
        return self.data.astype(np.float64)

    def f32(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.data)
        return self.data.astype(np.float32)


def _cast(x64: np.ndarray, dtype: str) -> Tensor:
    x32 = x64.astype(np.float32)
    if dtype == "bf16":
        return Tensor(f32_to_bf16_bits(x32), "bf16")
    if dtype == "f32":
        return Tensor(x32, "f32")
    raise ValueError(dtype)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _l2norm_rows(x):
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / n


# ------------------------------------------------------------ configurations


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    kind: str  # 'seq' (fwd / fwd+bwd over a sequence) or 'step' (decode)
    B: int
    T: int
    H: int
    dk: int
    dv: int
    dtype: str
    seed: int
    h0: str  # 'none' | 'zero' | 'randn'
    with_do: bool = False
    steps: int = 0  # decode only: consecutive steps


CONFIGS = {
    "pr1_ref": Config("pr1_ref", "seq", 1, 128, 2, 16, 16, "f32", 7401, "none"),
    "fwd_model": Config("fwd_model", "seq", 8, 4096, 16, 56, 56, "bf16", 7402, "none"),
    "decode_step": Config("decode_step", "step", 256, 1, 16, 56, 56, "bf16", 7403, "randn",
                          steps=1024),
    "fwdbwd_model": Config("fwdbwd_model", "seq", 8, 4096, 16, 56, 56, "bf16", 7404, "zero",
                           with_do=True),
    "long_ctx": Config("long_ctx", "seq", 1, 32768, 16, 128, 128, "bf16", 7405, "randn",
                       with_do=True),
}


def gen_seq(B, T, H, dk, dv, dtype="bf16", seed=0, h0="none", with_do=False, decay="normal",
            key_spread=False, with_D=False):
    """Inputs for one sequence workload. decay: 'normal' | 'weak' | 'zero'.
    Returns a dict: q, k, v, do (Tensor or None); g, beta, A_log, h0, D
    (float32 numpy or None). key_spread: keys of per-row lengths in
    [0.25, 4] instead of unit rows (inputs for the fused key normalisation)."""
    if decay == "weak":
        seed = seed + 100
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, T, H, dk))
    k = _l2norm_rows(rng.standard_normal((B, T, H, dk)))
    v = rng.standard_normal((B, T, H, dv))
    beta = _sigmoid(rng.standard_normal((B, T, H))).astype(np.float32)
    g = _sigmoid(rng.standard_normal((B, T, H))).astype(np.float32)
    if decay == "weak":
        A_log = rng.uniform(math.log(1e-3), math.log(1e-1), H).astype(np.float32)
    else:
        A_log = rng.uniform(0.0, math.log(16.0), H).astype(np.float32)
    if decay == "zero":
        g = np.zeros_like(g)
    if h0 == "randn":
        h0a = (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32)
    elif h0 == "zero":
        h0a = np.zeros((B, H, dk, dv), np.float32)
    else:
        h0a = None
    do = _cast(rng.standard_normal((B, T, H, dv)), dtype) if with_do else None
    if key_spread:
        k = k * rng.uniform(0.25, 4.0, (B, T, H, 1))
    D = rng.standard_normal(H).astype(np.float32) if with_D else None
    return dict(q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype), g=g, beta=beta,
                A_log=A_log, h0=h0a, do=do, D=D)


def gen_config(name, decay="normal", **override):
    c = CONFIGS[name]
    if c.kind != "seq":
        raise ValueError(f"{name} is a decode workload; use gen_decode")
    kw = dict(B=c.B, T=c.T, H=c.H, dk=c.dk, dv=c.dv, dtype=c.dtype, seed=c.seed, h0=c.h0,
              with_do=c.with_do)
    kw.update(override)
    return gen_seq(decay=decay, **kw)


def gen_decode(N, H, dk, dv, steps, dtype="bf16", seed=7403, block=64, decay="normal"):
    """Decode workload: initial state h0 [N,H,dk,dv] = 0.1 N(0,1) and fresh
    per-step tokens q,k [steps,N,H,dk], v [steps,N,H,dv], g,beta [steps,N,H].
    The initial state and A_log are drawn first, then tokens in blocks of
    ``block`` steps."""
    if decay == "weak":
        seed = seed + 100
    rng = np.random.Generator(np.random.PCG64(seed))
    if decay == "weak":
        A_log = rng.uniform(math.log(1e-3), math.log(1e-1), H).astype(np.float32)
    else:
        A_log = rng.uniform(0.0, math.log(16.0), H).astype(np.float32)
    h0 = (0.1 * rng.standard_normal((N, H, dk, dv))).astype(np.float32)
    qs, ks, vs, gs, bs = [], [], [], [], []
    for s0 in range(0, steps, block):
        n = min(block, steps - s0)
        qs.append(_cast(rng.standard_normal((n, N, H, dk)), dtype).data)
        ks.append(_cast(_l2norm_rows(rng.standard_normal((n, N, H, dk))), dtype).data)
        vs.append(_cast(rng.standard_normal((n, N, H, dv)), dtype).data)
        bs.append(_sigmoid(rng.standard_normal((n, N, H))).astype(np.float32))
        gs.append(_sigmoid(rng.standard_normal((n, N, H))).astype(np.float32))
    g = np.concatenate(gs)
    if decay == "zero":
        g = np.zeros_like(g)
    return dict(q=Tensor(np.concatenate(qs), dtype), k=Tensor(np.concatenate(ks), dtype),
                v=Tensor(np.concatenate(vs), dtype), g=g, beta=np.concatenate(bs), A_log=A_log,
                h0=h0)
