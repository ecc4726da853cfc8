"""GPU: the optional debug check of device-resident preconditions (KDA_DEBUG_VALIDATE).

With the variable set, a call whose g leaves [-5, 0] or whose cu_seqlens do not end at the token
count returns KDA_ERR_INVALID_ARGUMENT with nothing else enqueued (its outputs keep their sentinel
values); valid inputs give the same bits as with the check off.  Every invalid input used here
would also be memory-safe for the kernels themselves (g only changes arithmetic; a last offset
below the token count keeps every sequence inside the buffers)."""
import pytest
import torch

import oracle
from gated_delta_rule_60_amd import inputs, kda as K
from kda_testutil import DEV, oracle_g, prefill_case, say

pytestmark = pytest.mark.gpu

KDA_ERR_INVALID_ARGUMENT = 1


@pytest.fixture
def validate(monkeypatch):
    monkeypatch.setenv("KDA_DEBUG_VALIDATE", "1")


def _prefill(d, g, cu=None):
    dev = {x: d[x].to(DEV) for x in ("q", "k", "v", "beta")}
    B, T, H, _ = d["q"].shape
    o = torch.full((B, T, H, d["v"].shape[-1]), 7.0, device=DEV)
    hT = torch.full((d["S0"].shape[0] if cu is not None else B, H, d["q"].shape[-1],
                     d["v"].shape[-1]), 7.0, device=DEV)
    K.kda_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["beta"], g.to(DEV),
                    initial_state=d["S0"].to(DEV), final_state=hT, cu_seqlens=cu, o=o)
    torch.cuda.synchronize()
    return o, hT


def _rejected(fn):
    with pytest.raises(K.KDAError) as e:
        fn()
    assert e.value.status == KDA_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()


def test_validate_accepts_valid_inputs(monkeypatch):
    """Packed batch at the gate's bounds (g = -5 and 0 in places): same bits with the check on."""
    lens = [0, 5, 64, 1, 200, 17]
    d = prefill_case("prefill_varlen", seqlens=lens, H=2)
    g = oracle_g(d)
    g[0, :8] = -5.0
    g[0, 8:16] = 0.0
    cu = d["cu_seqlens"].to(DEV)
    say("validate valid", lens)
    o_off, h_off = _prefill(d, g, cu)
    monkeypatch.setenv("KDA_DEBUG_VALIDATE", "1")
    o_on, h_on = _prefill(d, g, cu)
    assert torch.equal(o_on, o_off) and torch.equal(h_on, h_off)


@pytest.mark.parametrize("bad", [-5.5, 0.25, float("nan")])
def test_validate_rejects_g_out_of_range(validate, bad):
    d = prefill_case("prefill_bf16", B=2, H=2, T=100)
    g = oracle_g(d)
    g[1, 77, 1, 5] = bad
    say("validate g", bad)
    dev = {x: d[x].to(DEV) for x in ("q", "k", "v", "beta")}
    o = torch.full(d["v"].shape, 7.0, device=DEV)
    hT = torch.full((2, 2, d["q"].shape[-1], d["v"].shape[-1]), 7.0, device=DEV)
    _rejected(lambda: K.kda_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["beta"], g.to(DEV),
                                      initial_state=d["S0"].to(DEV), final_state=hT, o=o))
    assert bool((o == 7.0).all()) and bool((hT == 7.0).all())


def test_validate_rejects_cu_seqlens_short_of_total(validate):
    lens = [40, 64, 30]
    d = prefill_case("prefill_varlen", seqlens=lens, H=2)
    cu = d["cu_seqlens"].clone()
    cu[-1] -= 16                     # ends 16 tokens before T (still in bounds)
    cu = cu.to(DEV)
    dev = {x: d[x].to(DEV) for x in ("q", "k", "v", "beta")}
    o = torch.full(d["v"].shape, 7.0, device=DEV)
    hT = torch.full(tuple(d["S0"].shape), 7.0, device=DEV)
    say("validate cu_seqlens", cu.tolist())
    _rejected(lambda: K.kda_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["beta"],
                                      oracle_g(d).to(DEV), initial_state=d["S0"].to(DEV),
                                      final_state=hT, cu_seqlens=cu, o=o))
    assert bool((o == 7.0).all()) and bool((hT == 7.0).all())


def test_validate_decode_and_spec(validate):
    """Decode step, verify and commit: valid g passes, g below -5 is rejected, state untouched."""
    cfg = inputs.config("decode", B=8, H=2)
    d = inputs.make_decode(cfg, steps=3)
    g = torch.from_numpy(oracle.gate(d["A"], d["z"])).to(torch.bfloat16)
    say("validate decode", cfg)
    S = d["S0"].to(DEV)
    S_ref = S.clone()
    step = [d[x][0].to(DEV) for x in ("q", "k", "v", "beta")]
    K.kda_decode_step(*step, g[0].to(DEV), S_ref.clone())      # valid: accepted
    bad = g[0].clone()
    bad[3, 1, 7] = -6.0
    _rejected(lambda: K.kda_decode_step(*step, bad.to(DEV), S))
    assert torch.equal(S, S_ref)
    draft = [d[x].transpose(0, 1).contiguous().to(DEV) for x in ("q", "k", "v", "beta")]
    g_bad = g.transpose(0, 1).contiguous()
    g_bad[5, 2, 0, 0] = 0.5
    g_bad = g_bad.to(DEV)
    _rejected(lambda: K.kda_decode_verify(*draft, g_bad, S))
    acc = torch.full((8,), 3, dtype=torch.int32, device=DEV)
    _rejected(lambda: K.kda_decode_commit(*draft, g_bad, S, acc))
    assert torch.equal(S, S_ref)
