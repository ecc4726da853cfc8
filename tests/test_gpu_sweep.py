"""GPU parity over a seeded sweep of small shapes mixing the options each dispatch path takes:
input dtype, head dims, fixed-length or packed batches (empty sequences included), initial state
or none, output scale, g given (fp32 or bf16) or the gate fused, and batches whose (sequence, head)
units reach the fused kernel's threshold.  Every case is compared with the fp64 oracle, per tensor
and per (sequence, head) unit, at the tolerances of the other parity tests."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_60_amd import inputs
from gated_delta_rule_60_amd import kda as K
from kda_testutil import DEV, rel_err, say, worst_unit_errs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-4}


def _cases(n=64, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fused = i % 4 == 3                                 # every fourth case: >= 256 units
        dtype = "bf16" if fused or rng.random() < 0.7 else "f32"
        dk, dv = (128, 128) if fused else tuple(int(x) for x in rng.choice([64, 128], size=2))
        packed = bool(rng.random() < 0.4)
        if fused:
            H = int(rng.choice([2, 4]))
            B = 256 // H + int(rng.integers(0, 8))
            T = int(rng.integers(1, 80))
        else:
            H = int(rng.integers(1, 5))
            B = int(rng.integers(1, 4))
            T = int(rng.integers(1, 300))
        seqlens = None
        if packed:
            seqlens = [int(x) if rng.random() > 0.15 else 0
                       for x in rng.integers(1, max(2, T), size=B)]
        out.append(dict(i=i, fused=fused, dtype=dtype, dk=dk, dv=dv, B=B, H=H, T=T,
                        seqlens=seqlens, s0=bool(rng.random() < 0.7),
                        scale=float(rng.choice([1.0, 0.5])),
                        gmode=str(rng.choice(["fused_gate", "g_f32", "g_bf16"]))))
    return out


CASES = _cases()


@pytest.mark.parametrize("c", CASES, ids=[f"case{c['i']}" for c in CASES])
def test_sweep(c):
    say("sweep", {k: v for k, v in c.items() if k != "seqlens"},
        "packed" if c["seqlens"] is not None else "fixed")
    cfg = inputs.config("prefill_bf16" if c["dtype"] == "bf16" else "prefill_f32_small",
                        B=c["B"], H=c["H"], T=c["T"], dk=c["dk"], dv=c["dv"],
                        s0_std=0.1 if c["s0"] else 0.0)
    d = inputs.make_prefill(cfg, seqlens=c["seqlens"])
    cu = d["cu_seqlens"]
    N = d["N"]
    if c["fused"]:
        assert K.kda_chunk_fwd_workspace_size(N, d["B"] * d["T"], c["H"], 128, 128) == 0 or N * c["H"] < 256
    qkvb = [d[x].to(DEV) for x in ("q", "k", "v", "beta")]
    h0 = d["S0"].to(DEV) if d["S0"] is not None else None
    cu_d = cu.to(DEV) if cu is not None else None
    if c["gmode"] == "fused_gate":
        o, hT = K.kda_chunk_fwd_gated(*qkvb, d["A"].to(DEV), d["z"].to(DEV), initial_state=h0,
                                      cu_seqlens=cu_d, o_dtype=torch.float32, scale=c["scale"])
        g_ref = oracle.gate(d["A"], d["z"])
    else:
        gdt = torch.float32 if c["gmode"] == "g_f32" else torch.bfloat16
        g = torch.from_numpy(oracle.gate(d["A"], d["z"])).to(gdt)
        o, hT = K.kda_chunk_fwd(*qkvb, g.to(DEV), initial_state=h0, cu_seqlens=cu_d,
                                o_dtype=torch.float32, scale=c["scale"])
        g_ref = g
    torch.cuda.synchronize()
    cu_np = cu.numpy() if cu is not None else None
    o_ref, S_ref, _ = oracle.forward(d["q"], d["k"], d["v"], d["beta"], g_ref, S0=d["S0"],
                                     cu_seqlens=cu_np, scale=c["scale"])
    tol = TOL[c["dtype"]]
    eo, es = rel_err(o, o_ref), rel_err(hT, S_ref)
    uo, us = worst_unit_errs(o, o_ref, hT, S_ref, cu_np)
    say(f"  o err {eo:.2e}  S err {es:.2e}  (worst unit: o {uo:.2e}  S {us:.2e})")
    assert eo <= tol and es <= tol, (eo, es)
    assert uo <= tol and us <= tol, (uo, us)
