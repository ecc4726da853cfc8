"""GPU parity at the edges of the input contract, against the fp64 oracle.

* Inputs outside the usual KDA recipe, on both input dtypes: beta ~ U[-0.5, 1.5] (the pages give
  the write strength no range), q and k of norm 3 with output scale 4, |v| ~ 30 and initial
  states 30x larger.  The recurrence stays bounded here (the gate's decay damps it), so every
  staged operand of the bf16 path stays far inside the fp16 range the kernels rely on.
* fp32 inputs (16-token records, split-bf16 operands) at lengths around the 16-token record and
  64-token chunk edges, and as a packed batch with empty sequences.
* The binding on a stream other than the current one.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_60_amd import kda as K
from kda_testutil import DEV, oracle_g, prefill_case, rel_err, say

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-4}


def widen(d, seed):
    """The same draws, rescaled outside the usual ranges; beta redrawn from its own generator."""
    gen = torch.Generator().manual_seed(seed)
    dt = d["q"].dtype
    out = dict(d)
    out["q"] = (d["q"].float() * 3.0).to(dt)
    out["k"] = (d["k"].float() * 3.0).to(dt)
    out["v"] = (d["v"].float() * 30.0).to(dt)
    out["beta"] = (torch.rand(d["beta"].shape, generator=gen, dtype=torch.float32) * 2.0 - 0.5).to(dt)
    if d["S0"] is not None:
        out["S0"] = d["S0"] * 30.0
    return out


def check(d, g, tol, scale=1.0, label="", o_dtype=torch.float32, stream=None):
    h0 = d["S0"].to(DEV) if d["S0"] is not None else None
    cu = d["cu_seqlens"].to(DEV) if d["cu_seqlens"] is not None else None
    o, hT = K.kda_chunk_fwd(*(d[x].to(DEV) for x in ("q", "k", "v", "beta")), g.to(DEV),
                            initial_state=h0, cu_seqlens=cu, o_dtype=o_dtype, scale=scale,
                            stream=stream)
    torch.cuda.synchronize()
    cun = d["cu_seqlens"].numpy() if d["cu_seqlens"] is not None else None
    o_ref, S_ref, _ = oracle.forward(d["q"], d["k"], d["v"], d["beta"], g, S0=d["S0"],
                                     cu_seqlens=cun, scale=scale)
    eo, es = rel_err(o, o_ref), rel_err(hT, S_ref)
    say(f"  {label} o err {eo:.2e}  S err {es:.2e}  max|o| {np.abs(o_ref).max():.3g}  "
        f"max|S| {np.abs(S_ref).max():.3g}")
    assert torch.isfinite(o).all() and torch.isfinite(hT).all()
    assert eo <= tol and es <= tol, (eo, es)
    return o, hT


@pytest.mark.parametrize("case", ["bf16_d128", "bf16_d64", "f32_d64", "f32_d128"])
def test_prefill_outside_usual_range(case):
    dt, dd = case.split("_d")
    dim = int(dd)
    if dt == "bf16":
        d = prefill_case("prefill_bf16", B=2, H=2, T=300, dk=dim, dv=dim)
    else:
        d = prefill_case("prefill_f32_small", B=2, H=2, T=300, dk=dim, dv=dim, s0_std=0.1)
    w = widen(d, seed=31)
    say("chunk outside usual range", case)
    check(w, oracle_g(w), TOL[dt], scale=4.0, label=case)


def test_prefill_outside_usual_range_packed():
    lens = [0, 5, 64, 1, 0, 200, 17, 128]
    d = prefill_case("prefill_varlen", seqlens=lens, H=3)
    w = widen(d, seed=32)
    say("chunk outside usual range, packed", lens)
    check(w, oracle_g(w), TOL["bf16"], scale=4.0, label="packed")


def test_prefill_outside_usual_range_mild_decay():
    """The same with the gates scaled down 20x, so the state carries over hundreds of tokens
    (the oracle's state grows to about 10x the usual recipe's)."""
    d = prefill_case("prefill_bf16", B=1, H=2, T=520)
    w = widen(d, seed=33)
    say("chunk outside usual range, mild decay")
    check(w, oracle_g(w) / 20.0, TOL["bf16"], scale=4.0, label="mild")


@pytest.mark.parametrize("T", [15, 17, 63, 65, 300])
def test_prefill_f32_ragged_lengths(T):
    """fp32 inputs (16-token records, 32-token chunks) at lengths around their edges."""
    d = prefill_case("prefill_f32_small", B=2, H=2, T=T, s0_std=0.1)
    say("chunk f32 ragged", T)
    check(d, oracle_g(d), TOL["f32"], label=f"f32 T={T}")


def test_prefill_f32_packed_with_empty_sequences():
    lens = [0, 5, 64, 1, 0, 200, 17, 128, 33]
    d = prefill_case("prefill_f32_small", seqlens=lens, H=2, s0_std=0.1, n_seqs=None)
    say("chunk f32 packed", lens)
    check(d, oracle_g(d), TOL["f32"], label="f32 packed")
    # the bf16-emitted o of the same call is the rounded fp32 one
    h0, cu = d["S0"].to(DEV), d["cu_seqlens"].to(DEV)
    args = [d[x].to(DEV) for x in ("q", "k", "v", "beta")] + [oracle_g(d).to(DEV)]
    o32, h32 = K.kda_chunk_fwd(*args, initial_state=h0, cu_seqlens=cu, o_dtype=torch.float32)
    o16, h16 = K.kda_chunk_fwd(*args, initial_state=h0, cu_seqlens=cu, o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(h16, h32)


def test_binding_on_a_side_stream():
    """Work enqueued on a stream that is not the current one (outputs and workspace allocated
    by the binding on that stream) equals the same call on the current stream bit for bit."""
    d = prefill_case("prefill_bf16", B=2, H=4, T=700)
    g = oracle_g(d).to(DEV)
    args = [d[x].to(DEV) for x in ("q", "k", "v", "beta")]
    h0 = d["S0"].to(DEV)
    o_ref, h_ref = K.kda_chunk_fwd(*args, g, initial_state=h0, o_dtype=torch.float32)
    A, z = d["A"].to(DEV), d["z"].to(DEV)
    og_ref, hg_ref = K.kda_chunk_fwd_gated(*args, A, z, initial_state=h0, o_dtype=torch.float32)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):   # allocations and frees on the side stream between calls
        o, h = K.kda_chunk_fwd(*args, g, initial_state=h0, o_dtype=torch.float32, stream=side)
        o2, h2 = K.kda_chunk_fwd_gated(*args, A, z, initial_state=h0, o_dtype=torch.float32,
                                       stream=side.cuda_stream)
    side.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(h, h_ref)
    assert torch.equal(o2, og_ref) and torch.equal(h2, hg_ref)


def test_decode_outside_usual_range():
    """The decode step (fp32 arithmetic throughout) with beta ~ U[-0.5, 1.5], |q| = |k| = 3,
    scale 4 and |v| ~ 30, over 8 steps."""
    from gated_delta_rule_60_amd import inputs
    cfg = inputs.config("decode", B=8, H=4)
    dd = inputs.make_decode(cfg, steps=8)
    gen = torch.Generator().manual_seed(34)
    bf = torch.bfloat16
    q, k = (dd["q"].float() * 3).to(bf), (dd["k"].float() * 3).to(bf)
    v = (dd["v"].float() * 30).to(bf)
    beta = (torch.rand(dd["beta"].shape, generator=gen) * 2 - 0.5).to(bf)
    g = torch.from_numpy(oracle.gate(dd["A"], dd["z"])).to(bf)
    S = dd["S0"].to(DEV).clone()
    S_ref = dd["S0"].double().numpy().copy()
    worst = 0.0
    for t in range(8):
        o = K.kda_decode_step(q[t].to(DEV), k[t].to(DEV), v[t].to(DEV), beta[t].to(DEV),
                              g[t].to(DEV), S, o_dtype=torch.float32, scale=4.0)
        o_ref = oracle.decode_step(q[t], k[t], v[t], beta[t], g[t], S_ref, scale=4.0)
        torch.cuda.synchronize()
        worst = max(worst, rel_err(o, o_ref))
    es = rel_err(S, S_ref)
    say(f"  decode outside range: o err {worst:.2e}  S err {es:.2e}")
    assert worst <= 1e-4 and es <= 1e-4
