"""Seeded synthetic inputs for the KDA forward pass (shared by the tests, the smoke check and
the benchmark; holds none of the method's arithmetic -- the gate and the recurrence live in
the HIP library and, separately, in the fp64 reference).

The pages describe the workloads only qualitatively (prefill of contexts up to a million tokens,
a recurrent decode step); these generators stand in for them with the shapes and value
distributions below.  Every draw comes from ``torch.Generator('cpu')`` seeded with
``1000 + config.seed_index``, in the fixed order q, k, v, beta-logits, A, z, S0, all fp32:

* q, k ~ N(0, 1), then L2-normalised per (token, head) over d_k in fp32;
* v ~ N(0, 1); beta = sigmoid(N(0, 1)) (a recipe for inputs, not a step of the method);
* A ~ N(0, 0.5^2) per (head, key channel); z ~ N(0, z_std^2) per (token, head, key channel);
* S0 ~ N(0, s0_std^2) per (sequence, head) state, or no initial state when s0_std == 0;
* every tensor is then cast (round-to-nearest-even) to the config's input dtype; A and S0
  stay fp32.

Variable-length batches draw their lengths first from a second generator seeded
``2000 + seed_index``: U_i ~ Uniform(ln lo, ln hi), then a scale s found by bisection so that
sum_i clamp(round(s * e^U_i), lo, hi) equals the requested total, with the rounding residue
spread over sequences that still have room.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class KDAConfig:
    name: str
    seed_index: int
    B: int = 1
    T: int = 0
    H: int = 1
    dk: int = 128
    dv: int = 128
    dtype: str = "bf16"            # input dtype of q, k, v, beta, z: "bf16" or "f32"
    z_std: float = 1.0
    s0_std: float = 0.0            # 0 -> no initial state
    # variable-length packing (B must be 1; T is then the total)
    n_seqs: Optional[int] = None
    len_lo: int = 0
    len_hi: int = 0
    total: int = 0
    # decode
    decode_steps: int = 0

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


# The five workloads (sizes and distributions as stated for this benchmark).
CONFIGS = {
    "prefill_f32_small": KDAConfig("prefill_f32_small", 0, B=1, T=256, H=2, dk=64, dv=64,
                                   dtype="f32", z_std=1.0, s0_std=0.0),
    "prefill_bf16": KDAConfig("prefill_bf16", 1, B=4, T=4096, H=16, dk=128, dv=128,
                              dtype="bf16", z_std=1.0, s0_std=0.1),
    "prefill_long": KDAConfig("prefill_long", 2, B=1, T=65536, H=32, dk=128, dv=128,
                              dtype="bf16", z_std=2.0, s0_std=0.1),
    "decode": KDAConfig("decode", 3, B=256, T=1, H=32, dk=128, dv=128, dtype="bf16",
                        z_std=1.0, s0_std=0.1, decode_steps=64),
    "prefill_varlen": KDAConfig("prefill_varlen", 4, B=1, H=8, dk=128, dv=128, dtype="bf16",
                                z_std=1.0, s0_std=0.1, n_seqs=8, len_lo=1024,
                                len_hi=262144, total=1 << 20),
}


def config(name: str, **overrides) -> KDAConfig:
    """A named workload, optionally resized (same recipe and seed, smaller or ragged shape)."""
    return dataclasses.replace(CONFIGS[name], **overrides)


def varlen_lengths(n: int, lo: int, hi: int, total: int, seed: int) -> list[int]:
    """Log-uniform lengths in [lo, hi] rescaled to sum exactly to total (see module doc)."""
    if not (n * lo <= total <= n * hi):
        raise ValueError("total out of reach for n lengths in [lo, hi]")
    gen = torch.Generator("cpu").manual_seed(seed)
    u = torch.empty(n, dtype=torch.float64).uniform_(math.log(lo), math.log(hi), generator=gen)
    base = [math.exp(x) for x in u.tolist()]

    def lens(s):
        return [min(hi, max(lo, int(round(s * b)))) for b in base]

    s_lo, s_hi = 0.0, 1.0
    while sum(lens(s_hi)) < total:
        s_hi *= 2.0
    for _ in range(200):
        mid = 0.5 * (s_lo + s_hi)
        if sum(lens(mid)) < total:
            s_lo = mid
        else:
            s_hi = mid
    out = lens(s_lo)
    resid = total - sum(out)
    i = n - 1
    while resid != 0:
        room = (hi - out[i]) if resid > 0 else (lo - out[i])
        step = min(resid, room) if resid > 0 else max(resid, room)
        out[i] += step
        resid -= step
        i = (i - 1) % n
    return out


def _normal(shape, gen, std=1.0):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    return x * std if std != 1.0 else x


def _l2norm(x):
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def make_prefill(cfg: KDAConfig, seqlens: Optional[list[int]] = None) -> dict:
    """Inputs for a prefill call: q, k, z [B, T, H, dk]; v [B, T, H, dv]; beta [B, T, H];
    A [H, dk] fp32; S0 [N, H, dk, dv] fp32 or None; cu_seqlens int32 [N+1] or None."""
    gen = torch.Generator("cpu").manual_seed(1000 + cfg.seed_index)
    cu = None
    B, T = cfg.B, cfg.T
    if seqlens is None and cfg.n_seqs is not None:
        seqlens = varlen_lengths(cfg.n_seqs, cfg.len_lo, cfg.len_hi, cfg.total,
                                 2000 + cfg.seed_index)
    if seqlens is not None:
        B, T = 1, int(sum(seqlens))
        cu = torch.tensor([0] + list(_cumsum(seqlens)), dtype=torch.int32)
    N = B if cu is None else len(cu) - 1
    H, dk, dv, dt = cfg.H, cfg.dk, cfg.dv, cfg.torch_dtype
    q = _l2norm(_normal((B, T, H, dk), gen)).to(dt)
    k = _l2norm(_normal((B, T, H, dk), gen)).to(dt)
    v = _normal((B, T, H, dv), gen).to(dt)
    beta = torch.sigmoid(_normal((B, T, H), gen)).to(dt)
    A = _normal((H, dk), gen, 0.5)
    z = _normal((B, T, H, dk), gen, cfg.z_std).to(dt)
    S0 = _normal((N, H, dk, dv), gen, cfg.s0_std) if cfg.s0_std > 0 else None
    return dict(q=q, k=k, v=v, beta=beta, A=A, z=z, S0=S0, cu_seqlens=cu, B=B, T=T, N=N,
                H=H, dk=dk, dv=dv)


def make_decode(cfg: KDAConfig, steps: Optional[int] = None) -> dict:
    """Inputs for `steps` consecutive decode steps of cfg.B sequences: q, k, z
    [steps, N, H, dk]; v [steps, N, H, dv]; beta [steps, N, H]; A [H, dk]; S0 [N, H, dk, dv]."""
    gen = torch.Generator("cpu").manual_seed(1000 + cfg.seed_index)
    steps = cfg.decode_steps if steps is None else steps
    N, H, dk, dv, dt = cfg.B, cfg.H, cfg.dk, cfg.dv, cfg.torch_dtype
    q = _l2norm(_normal((steps, N, H, dk), gen)).to(dt)
    k = _l2norm(_normal((steps, N, H, dk), gen)).to(dt)
    v = _normal((steps, N, H, dv), gen).to(dt)
    beta = torch.sigmoid(_normal((steps, N, H), gen)).to(dt)
    A = _normal((H, dk), gen, 0.5)
    z = _normal((steps, N, H, dk), gen, cfg.z_std).to(dt)
    S0 = _normal((N, H, dk, dv), gen, cfg.s0_std) if cfg.s0_std > 0 else \
        torch.zeros((N, H, dk, dv), dtype=torch.float32)
    return dict(q=q, k=k, v=v, beta=beta, A=A, z=z, S0=S0, N=N, H=H, dk=dk, dv=dv,
                steps=steps)


def _cumsum(xs):
    s = 0
    for x in xs:
        s += x
        yield s
