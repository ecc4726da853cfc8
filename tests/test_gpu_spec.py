"""GPU parity: speculative decoding -- kda_decode_verify (K draft tokens from a read-only state)
and kda_decode_commit (the accepted prefix applied in place) against the fp64 oracle and against
successive kda_decode_step calls.  Commit must equal them bit for bit; verify (drafts of up to 8
tokens run batched from one pass over the state) equals them bit for bit on the first token and
up to fp32 rounding on the others."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_60_amd import inputs, kda as K
from kda_testutil import DEV, rel_err, say

pytestmark = pytest.mark.gpu


def _draft(cfg, n_draft):
    """Draft inputs [N, K, H, d] from the decode generator's [K, N, H, d] steps, with g from the
    oracle gate rounded to the input dtype."""
    d = inputs.make_decode(cfg, steps=n_draft)
    gdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    g = torch.from_numpy(oracle.gate(d["A"], d["z"])).to(gdt)
    steps = {x: d[x] for x in ("q", "k", "v", "beta")}
    steps["g"] = g
    draft = {x: t.transpose(0, 1).contiguous() for x, t in steps.items()}
    return d, steps, draft


def _step_states(steps, S0, n_draft):
    """o of each draft token and the state after each prefix, from kda_decode_step."""
    S = S0.clone()
    states, outs = [S0.clone()], []
    for t in range(n_draft):
        outs.append(K.kda_decode_step(*(steps[x][t].to(DEV) for x in ("q", "k", "v", "beta", "g")),
                                      S, o_dtype=torch.float32))
        states.append(S.clone())
    torch.cuda.synchronize()
    return outs, states


def _check(cfg, n_draft, accepted, n_oracle=None):
    d, steps, draft = _draft(cfg, n_draft)
    N = cfg.B
    S0 = d["S0"].to(DEV)
    dev = {x: t.to(DEV) for x, t in draft.items()}
    args = [dev[x] for x in ("q", "k", "v", "beta", "g")]
    # verify: every draft token's output, state untouched
    S_v = S0.clone()
    o = K.kda_decode_verify(*args, S_v, o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(S_v, S0)
    outs, states = _step_states(steps, S0, n_draft)
    assert torch.equal(o[:, 0], outs[0])
    for t in range(1, n_draft):
        if n_draft > 8:                          # token by token: the step kernel's arithmetic
            assert torch.equal(o[:, t], outs[t]), t
            continue
        diff = (o[:, t] - outs[t]).abs().max().item()
        assert diff <= 1e-5 * max(outs[t].abs().max().item(), 1e-30), (t, diff)
    # against the oracle (all sequences, or a sample)
    sel = np.arange(N) if n_oracle is None else np.unique(
        np.random.default_rng(1).choice(N, n_oracle, replace=False))
    S_ref = d["S0"][sel].double().numpy().copy()
    worst = 0.0
    for t in range(n_draft):
        o_ref = oracle.decode_step(*(steps[x][t][sel] for x in ("q", "k", "v", "beta", "g")), S_ref)
        worst = max(worst, rel_err(o[torch.from_numpy(sel).to(DEV), t], o_ref))
    # commit: each sequence advanced by its (clamped) accepted count
    acc = torch.tensor(accepted, dtype=torch.int32, device=DEV)
    S_c = S0.clone()
    K.kda_decode_commit(*args, S_c, acc)
    torch.cuda.synchronize()
    for n in range(N):
        a = min(max(int(accepted[n]), 0), n_draft)
        assert torch.equal(S_c[n], states[a][n]), (n, a)
    say(f"  verify o err {worst:.2e} over {len(sel)} sequences x {n_draft} tokens")
    assert worst <= 1e-5


@pytest.mark.parametrize("dk,dv,dtype,n_draft", [(128, 128, "bf16", 4), (64, 64, "f32", 3),
                                                 (128, 64, "bf16", 1), (64, 128, "f32", 6),
                                                 (128, 128, "bf16", 8), (128, 128, "f32", 9),
                                                 (128, 64, "bf16", 5), (64, 64, "bf16", 8)])
def test_verify_commit_small(dk, dv, dtype, n_draft):
    cfg = inputs.config("decode", B=6, H=3, dk=dk, dv=dv, dtype=dtype)
    accepted = [0, 1, n_draft, n_draft // 2, n_draft + 3, -1]     # the last two clamp
    say("spec decode", cfg.B, cfg.H, dk, dv, dtype, n_draft)
    _check(cfg, n_draft, accepted)


def test_verify_commit_full_size():
    """The decode workload's shape (256 sequences x 32 heads, d = 128, bf16) with 4-token drafts;
    every output against the step kernel, 8 sequences against the oracle."""
    cfg = inputs.config("decode")
    rng = np.random.default_rng(3)
    accepted = rng.integers(0, 5, size=cfg.B).tolist()
    say("spec decode full size", cfg.B, cfg.H)
    _check(cfg, 4, accepted, n_oracle=8)
