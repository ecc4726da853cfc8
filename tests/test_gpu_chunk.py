"""GPU parity: kda_chunk_fwd (chunked prefill) against the fp64 token-by-token oracle.

Parity metric: max|x - ref| / max|ref| per tensor, on o emitted in fp32 and on the fp32 final
state; 2e-3 for bf16 inputs, 1e-4 for fp32 inputs.  (Rounding o to bf16 alone costs up to
2^-8 relative, so the bf16-emitted o is checked to equal the rounded fp32-emitted o bit for bit.)
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_60_amd import kda as K
from kda_testutil import DEV, oracle_g, prefill_case, rel_err, say, worst_unit_errs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-4}


def run_gpu(d, g, o_dtype=torch.float32, S0="given", scale=1.0):
    h0 = d["S0"].to(DEV) if (S0 == "given" and d["S0"] is not None) else None
    cu = d["cu_seqlens"].to(DEV) if d["cu_seqlens"] is not None else None
    o, hT = K.kda_chunk_fwd(d["q"].to(DEV), d["k"].to(DEV), d["v"].to(DEV), d["beta"].to(DEV),
                            g.to(DEV), initial_state=h0, cu_seqlens=cu, o_dtype=o_dtype,
                            scale=scale)
    torch.cuda.synchronize()
    return o, hT


def check_full(d, g, tol, scale=1.0, label=""):
    o, hT = run_gpu(d, g, scale=scale)
    cu = d["cu_seqlens"].numpy() if d["cu_seqlens"] is not None else None
    o_ref, S_ref, _ = oracle.forward(d["q"], d["k"], d["v"], d["beta"], g, S0=d["S0"],
                                     cu_seqlens=cu, scale=scale)
    eo, es = rel_err(o, o_ref), rel_err(hT, S_ref)
    uo, us = worst_unit_errs(o, o_ref, hT, S_ref, cu)
    say(f"  {label} o err {eo:.2e}  S err {es:.2e}  (worst unit: o {uo:.2e}  S {us:.2e})")
    assert eo <= tol and es <= tol, (eo, es)
    assert uo <= tol and us <= tol, (uo, us)
    return o, hT


def test_prefill_f32_small_config():
    """Config: fp32, B=1, H=2, T=256, d=64, zero initial state (tolerance 1e-4)."""
    d = prefill_case("prefill_f32_small")
    say("chunk parity", d["cfg"])
    check_full(d, oracle_g(d), TOL["f32"], label="f32 small")


@pytest.mark.parametrize("T", [1, 15, 16, 63, 64, 65, 130, 300])
def test_prefill_ragged_lengths(T):
    """bf16 recipe at lengths around chunk and 16-token block edges."""
    d = prefill_case("prefill_bf16", B=2, H=2, T=T)
    say("chunk ragged", T)
    check_full(d, oracle_g(d), TOL["bf16"], label=f"T={T}")


def test_prefill_bf16_config_full_size():
    """Config: bf16, B=4, H=16, T=4096, d=128, random initial state; every unit checked."""
    d = prefill_case("prefill_bf16")
    say("chunk parity full size", d["cfg"])
    check_full(d, oracle_g(d), TOL["bf16"], label="bf16 full")


def _sampled(d, g, units, tol, label):
    o, hT = run_gpu(d, g)
    cu = d["cu_seqlens"].numpy() if d["cu_seqlens"] is not None else None
    ref = oracle.forward_units(d["q"], d["k"], d["v"], d["beta"], g, units, S0=d["S0"],
                               cu_seqlens=cu)
    T = d["T"]
    for (n, h), (o_u, S_u) in ref.items():
        t0 = int(cu[n]) if cu is not None else 0
        length = o_u.shape[0]
        ob = 0 if cu is not None else n
        got_o = o[ob, t0:t0 + length, h] if length else o[ob, :0, h]
        eo = rel_err(got_o, o_u) if length else 0.0
        es = rel_err(hT[n, h], S_u)
        say(f"  {label} unit ({n},{h}) len {length}: o err {eo:.2e}  S err {es:.2e}")
        assert eo <= tol and es <= tol, (n, h, eo, es)
    assert T >= 0


def test_prefill_long_config_sampled():
    """Config: bf16, B=1, H=32, T=65536, z ~ N(0, 2^2) (many channels at the e^-5 floor and
    near 1); the whole batch runs, three heads are checked against the oracle."""
    d = prefill_case("prefill_long")
    say("chunk long sampled", d["cfg"])
    _sampled(d, oracle_g(d), [(0, 0), (0, 13), (0, 31)], TOL["bf16"], "long")


def test_prefill_varlen_config_sampled():
    """Config: 8 packed sequences, lengths log-uniform in [1K, 256K] summing to 2^20, H=8."""
    d = prefill_case("prefill_varlen")
    lens = np.diff(d["cu_seqlens"].numpy())
    say("chunk varlen sampled, lengths", lens.tolist())
    order = np.argsort(lens)
    units = [(int(order[0]), 0), (int(order[1]), 7), (int(order[4]), 3), (int(order[-1]), 5)]
    _sampled(d, oracle_g(d), units, TOL["bf16"], "varlen")


def test_prefill_varlen_small_all_units():
    """Packed batch with empty, sub-block, exact-chunk and ragged sequences; every unit."""
    lens = [0, 5, 64, 1, 0, 200, 17, 128]
    d = prefill_case("prefill_varlen", seqlens=lens, H=3)
    say("chunk varlen small", lens)
    check_full(d, oracle_g(d), TOL["bf16"], label="varlen small")


# ---- whole sequences in the fused kernel: 16-bit inputs at d_k = d_v = 128 when the (sequence,
# head) units fill 256 workgroups --------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 47, 300])
def test_fused_whole_sequences(T):
    """256 (sequence, head) units of one, 47 (a ragged second sub-block) and 300 tokens, random
    initial states; every unit."""
    d = prefill_case("prefill_bf16", B=64, H=4, T=T)
    assert K.kda_chunk_fwd_workspace_size(64, 64 * T, 4, 128, 128) == 0
    say("fused whole", T)
    check_full(d, oracle_g(d), TOL["bf16"], label=f"fused whole T={T}")


def test_fused_whole_packed_and_gated():
    """A packed batch of 130 sequences x 2 heads (empty, single-token, chunk-exact and ragged
    lengths) through kda_chunk_fwd and through the fused gate; every unit."""
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.choice([0, 1, 16, 32, 33, 64, 150, 257], size=130)]
    d = prefill_case("prefill_varlen", seqlens=lens, H=2)
    say("fused whole packed", sum(lens))
    check_full(d, oracle_g(d), TOL["bf16"], label="fused whole packed")
    o, hT = _gated(d)
    cu = d["cu_seqlens"].numpy()
    o_ref, S_ref, _ = oracle.forward(d["q"], d["k"], d["v"], d["beta"], oracle.gate(d["A"], d["z"]),
                                     S0=d["S0"], cu_seqlens=cu)
    eo, es = rel_err(o, o_ref), rel_err(hT, S_ref)
    say(f"  fused whole gated: o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_fused_whole_input_and_output_dtypes():
    """The fused kernel's other variants: g given in bf16, z given in fp32 through the fused gate,
    and bf16 o, which must be the RNE rounding of the fp32 o; two runs agree bit for bit."""
    d = prefill_case("prefill_bf16", B=64, H=4, T=100)
    say("fused whole dtypes")
    h0 = d["S0"].to(DEV)
    qkvb = [d[x].to(DEV) for x in ("q", "k", "v", "beta")]
    g = oracle_g(d, torch.bfloat16)
    o1, h1 = K.kda_chunk_fwd(*qkvb, g.to(DEV), initial_state=h0, o_dtype=torch.float32)
    o2, h2 = K.kda_chunk_fwd(*qkvb, g.to(DEV), initial_state=h0, o_dtype=torch.float32)
    o3, h3 = K.kda_chunk_fwd(*qkvb, g.to(DEV), initial_state=h0, o_dtype=torch.bfloat16)
    z32 = d["z"].to(torch.float32)
    o4, h4 = K.kda_chunk_fwd_gated(*qkvb, d["A"].to(DEV), z32.to(DEV), initial_state=h0,
                                   o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    assert torch.equal(o3, o1.to(torch.bfloat16)) and torch.equal(h3, h1)
    for (o, hT), g_ref, lab in (((o1, h1), g, "g bf16"), ((o4, h4), oracle.gate(d["A"], z32), "z f32")):
        o_ref, S_ref, _ = oracle.forward(d["q"], d["k"], d["v"], d["beta"], g_ref, S0=d["S0"])
        eo, es = rel_err(o, o_ref), rel_err(hT, S_ref)
        say(f"  fused whole {lab}: o err {eo:.2e}  S err {es:.2e}")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("gmode", ["floor", "one"])
def test_prefill_gate_extremes(gmode):
    """g = -5 in every channel (the decay floor: diagonal-block factors reach e^80) and g = 0
    (no decay, the DeltaNet limit)."""
    d = prefill_case("prefill_bf16", B=2, H=2, T=256)
    g = torch.full(d["q"].shape, -5.0 if gmode == "floor" else 0.0, dtype=torch.float32)
    say("chunk gate extreme", gmode)
    o, hT = check_full(d, g, TOL["bf16"], label=gmode)
    assert torch.isfinite(o).all() and torch.isfinite(hT).all()


@pytest.mark.parametrize("div", [20.0, 5.0])
def test_prefill_mild_decay(div):
    """Gates scaled down (mean decay about e^-0.125 and e^-0.5 per token): across the 16-token
    halves of a 32-token state step both the decay factors and the cross terms between the halves
    are far from 0 and from 1, which neither the standard recipe (cross terms vanish) nor g = 0
    (every factor is 1) exercises."""
    d = prefill_case("prefill_bf16", B=2, H=2, T=300)
    g = oracle_g(d) / div
    say("chunk mild decay", div)
    check_full(d, g, TOL["bf16"], label=f"g/{div:g}")


def test_prefill_mild_decay_f32():
    """fp32 inputs (16-token records, split-bf16 operands) with gates scaled down 20x: the state
    carries across blocks and chunks at full weight."""
    d = prefill_case("prefill_f32_small")
    say("chunk mild decay f32", d["cfg"])
    check_full(d, oracle_g(d) / 20.0, TOL["f32"], label="f32 g/20")


@pytest.mark.parametrize("bval", [0.0, 1.0])
def test_prefill_beta_extremes(bval):
    """beta = 0 (nothing written: pure decay of the initial state) and beta = 1 (full
    overwrite).  For beta = 0 the gates are scaled down 50x: at the recipe's mean decay
    (about e^-2.5 per token) the state would fall below the fp32 range within 40 tokens, where
    the GPU's fp32 state is legitimately zero and a relative comparison is meaningless."""
    d = prefill_case("prefill_bf16", B=1, H=2, T=200)
    d["beta"] = torch.full_like(d["beta"], bval)
    g = oracle_g(d) if bval else oracle_g(d) / 50.0
    say("chunk beta", bval)
    check_full(d, g, TOL["bf16"], label=f"beta={bval}")


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_prefill_head_dims(dk, dv):
    d = prefill_case("prefill_bf16", B=2, H=2, T=150, dk=dk, dv=dv)
    say("chunk dims", dk, dv)
    check_full(d, oracle_g(d), TOL["bf16"], label=f"dk={dk} dv={dv}")


def test_prefill_scale():
    d = prefill_case("prefill_bf16", B=1, H=2, T=100)
    check_full(d, oracle_g(d), TOL["bf16"], scale=0.125, label="scale")


def _split_run(d, g, T1):
    """[0, T1) then [T1, T) through the emitted state, the second call updating it in place."""
    first = {k: (v[:, :T1] if isinstance(v, torch.Tensor) and v.dim() >= 3 and k != "S0" else v)
             for k, v in d.items()}
    o1, h1 = run_gpu(first, g[:, :T1])
    qs = [d[k][:, T1:].contiguous().to(DEV) for k in ("q", "k", "v", "beta")]
    o2, h2 = K.kda_chunk_fwd(*qs, g[:, T1:].contiguous().to(DEV), initial_state=h1,
                             final_state=h1, o_dtype=torch.float32)
    torch.cuda.synchronize()
    return torch.cat([o1, o2], 1), h2


def test_split_invariance_and_inplace_state():
    """[0, T) in one call equals [0, T1) then [T1, T) through the emitted state (the second call
    updating the state in place): the state carries the whole history.  A split on a chunk
    boundary keeps every record's tokens, so the two runs agree bit for bit; a split inside a
    record changes the blocking, and they agree to the kernels' rounding (the state much more
    closely than o, whose error the fp16-staged products dominate)."""
    d = prefill_case("prefill_bf16", B=2, H=3, T=320)
    g = oracle_g(d)
    o_full, h_full = run_gpu(d, g)
    o_s, h_s = _split_run(d, g, 128)
    assert torch.equal(o_s, o_full) and torch.equal(h_s, h_full)
    o_s, h_s = _split_run(d, g, 100)
    eo = rel_err(o_s, o_full.double().cpu().numpy())
    es = rel_err(h_s, h_full.double().cpu().numpy())
    say(f"  split at 100 vs whole: o {eo:.2e}  S {es:.2e}")
    assert eo <= TOL["bf16"] and es <= 1e-4


def test_decode_steps_equal_prefill():
    d = prefill_case("prefill_bf16", B=2, H=2, T=40)
    g = oracle_g(d)
    o_p, h_p = run_gpu(d, g)
    S = d["S0"].to(DEV).clone()
    outs = []
    for t in range(d["T"]):
        outs.append(K.kda_decode_step(*(d[k][:, t].contiguous().to(DEV) for k in ("q", "k", "v", "beta")),
                                      g[:, t].contiguous().to(DEV), S, o_dtype=torch.float32))
    torch.cuda.synchronize()
    o_d = torch.stack(outs, 1)
    assert rel_err(o_d, o_p.double().cpu().numpy()) <= 2e-3
    assert rel_err(S, h_p.double().cpu().numpy()) <= 2e-3


def test_deterministic_and_bf16_output_rounding():
    d = prefill_case("prefill_bf16", B=2, H=4, T=513)
    g = oracle_g(d)
    o1, h1 = run_gpu(d, g)
    o2, h2 = run_gpu(d, g)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    o3, h3 = run_gpu(d, g, o_dtype=torch.bfloat16)
    assert torch.equal(o3, o1.to(torch.bfloat16)) and torch.equal(h3, h1)


def test_zero_initial_state_and_empty_batch():
    d = prefill_case("prefill_bf16", B=2, H=2, T=70)
    g = oracle_g(d)
    d0 = dict(d, S0=None)
    check_full(d0, g, TOL["bf16"], label="no S0")
    # T = 0: final state = initial state
    e = prefill_case("prefill_bf16", B=2, H=2, T=0)
    o, hT = run_gpu(e, torch.zeros(e["q"].shape))
    assert o.numel() == 0 and torch.equal(hT.cpu(), e["S0"])


def test_end_to_end_gate_then_chunk():
    """Gate and prefill both on the GPU versus both in the oracle (fp64 g, unrounded)."""
    d = prefill_case("prefill_bf16", B=2, H=4, T=257)
    g_gpu = K.kda_gate(d["A"].to(DEV), d["z"].to(DEV))
    o, hT = K.kda_chunk_fwd(*(d[k].to(DEV) for k in ("q", "k", "v", "beta")), g_gpu,
                            initial_state=d["S0"].to(DEV), o_dtype=torch.float32)
    torch.cuda.synchronize()
    g64 = oracle.gate(d["A"], d["z"])
    o_ref, S_ref, _ = oracle.forward(d["q"], d["k"], d["v"], d["beta"], g64, S0=d["S0"])
    assert rel_err(o, o_ref) <= TOL["bf16"] and rel_err(hT, S_ref) <= TOL["bf16"]


def _gated(d, o_dtype=torch.float32):
    cu = d["cu_seqlens"].to(DEV) if d["cu_seqlens"] is not None else None
    h0 = d["S0"].to(DEV) if d["S0"] is not None else None
    o, hT = K.kda_chunk_fwd_gated(*(d[x].to(DEV) for x in ("q", "k", "v", "beta", "A", "z")),
                                  initial_state=h0, cu_seqlens=cu, o_dtype=o_dtype)
    torch.cuda.synchronize()
    return o, hT


@pytest.mark.parametrize("case", ["fixed", "varlen", "f32"])
def test_fused_gate_equals_gate_then_chunk(case):
    """kda_chunk_fwd_gated = kda_gate (fp32 g) then kda_chunk_fwd, bit for bit (same gate
    arithmetic, including the g = 0 padding of partial blocks)."""
    if case == "fixed":
        d = prefill_case("prefill_bf16", B=2, H=4, T=300)
    elif case == "varlen":
        d = prefill_case("prefill_varlen", seqlens=[0, 5, 64, 1, 200, 17], H=3)
    else:
        d = prefill_case("prefill_f32_small")
    say("fused gate vs gate + chunk", case)
    o1, h1 = _gated(d)
    g = K.kda_gate(d["A"].to(DEV), d["z"].to(DEV))
    o2, h2 = run_gpu(d, g)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_fused_gate_parity_full_size():
    """The bf16 prefill workload through the fused entry point against the fp64 oracle."""
    d = prefill_case("prefill_bf16")
    say("fused gate parity full size", d["cfg"])
    o, hT = _gated(d)
    o_ref, S_ref, _ = oracle.forward(d["q"], d["k"], d["v"], d["beta"], oracle.gate(d["A"], d["z"]),
                                     S0=d["S0"])
    eo, es = rel_err(o, o_ref), rel_err(hT, S_ref)
    say(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("case", ["g_bf16", "g_bf16_dk64", "z_f32", "z_f32_dk64"])
def test_prefill_gate_input_dtypes(case):
    """bf16 q, k, v, beta with g given in bf16 (kda_chunk_fwd), or with z given in fp32 through the
    fused gate; both sides consume the same stored values."""
    dk = 64 if case.endswith("dk64") else 128
    d = prefill_case("prefill_bf16", B=2, H=3, T=300, dk=dk, dv=128)
    say("gate input dtypes", case)
    h0 = d["S0"].to(DEV)
    qkvb = [d[x].to(DEV) for x in ("q", "k", "v", "beta")]
    if case.startswith("g_bf16"):
        g = oracle_g(d, torch.bfloat16)
        o, hT = K.kda_chunk_fwd(*qkvb, g.to(DEV), initial_state=h0, o_dtype=torch.float32)
        g_ref = g
    else:
        z32 = d["z"].to(torch.float32)
        o, hT = K.kda_chunk_fwd_gated(*qkvb, d["A"].to(DEV), z32.to(DEV), initial_state=h0,
                                      o_dtype=torch.float32)
        g_ref = oracle.gate(d["A"], z32)
    torch.cuda.synchronize()
    o_ref, S_ref, _ = oracle.forward(d["q"], d["k"], d["v"], d["beta"], g_ref, S0=d["S0"])
    eo, es = rel_err(o, o_ref), rel_err(hT, S_ref)
    say(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("g_min", [-1.0, -2.5])
def test_fused_gate_other_g_min(g_min):
    """The gate bound g_min is a parameter (any value in [-5, 0)): the fused prefill with a milder
    bound, and the standalone gate with it, against the fp64 oracle; the fused path still equals
    kda_gate followed by kda_chunk_fwd bit for bit."""
    d = prefill_case("prefill_bf16", B=2, H=3, T=200)
    say("fused gate g_min", g_min)
    qkvb = [d[x].to(DEV) for x in ("q", "k", "v", "beta")]
    A, z, h0 = d["A"].to(DEV), d["z"].to(DEV), d["S0"].to(DEV)
    o, hT = K.kda_chunk_fwd_gated(*qkvb, A, z, g_min=g_min, initial_state=h0, o_dtype=torch.float32)
    g = K.kda_gate(A, z, g_min=g_min)
    o2, h2 = K.kda_chunk_fwd(*qkvb, g, initial_state=h0, o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(hT, h2)
    g64 = oracle.gate(d["A"], d["z"], g_min=g_min)
    assert rel_err(g, g64) <= 1e-6
    o_ref, S_ref, _ = oracle.forward(d["q"], d["k"], d["v"], d["beta"], g64, S0=d["S0"])
    eo, es = rel_err(o, o_ref), rel_err(hT, S_ref)
    say(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_fused_gate_f32_config():
    d = prefill_case("prefill_f32_small")
    o, hT = _gated(d)
    o_ref, S_ref, _ = oracle.forward(d["q"], d["k"], d["v"], d["beta"], oracle.gate(d["A"], d["z"]),
                                     S0=d["S0"])
    assert rel_err(o, o_ref) <= TOL["f32"] and rel_err(hT, S_ref) <= TOL["f32"]


# ---- checkpoint emission (kda_chunk_fwd_checkpointed) ------------------------------------------
def _ckpt_bases(d, every):
    """First slot and count of each sequence's checkpoints, from the layout kda.h specifies."""
    if d["cu_seqlens"] is None:
        B, T = d["q"].shape[:2]
        return [(n * (T // every), T // every) for n in range(B)]
    cu = d["cu_seqlens"].numpy()
    return [(int(cu[n]) // every + n, int(cu[n + 1] - cu[n]) // every) for n in range(len(cu) - 1)]


def _check_checkpoints(d, every, tol, gated=False, units=None, label=""):
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    cu = d["cu_seqlens"].to(DEV) if d["cu_seqlens"] is not None else None
    N = B if cu is None else cu.numel() - 1
    h0 = d["S0"].to(DEV) if d["S0"] is not None else None
    slots = (B * (T // every)) if cu is None else (T // every + N)
    ck = torch.full((slots, H, dk, dv), float("nan"), dtype=torch.float32, device=DEV)
    args = [d[x].to(DEV) for x in ("q", "k", "v", "beta")]
    if gated:
        gz = dict(A=d["A"].to(DEV), z=d["z"].to(DEV))
        g = oracle_g(d)
    else:
        g = oracle_g(d)
        gz = dict(g=g.to(DEV))
    o, hT, ck = K.kda_chunk_fwd_checkpointed(*args, every, initial_state=h0, cu_seqlens=cu,
                                             o_dtype=torch.float32, checkpoints=ck, **gz)
    torch.cuda.synchronize()
    # the prefill outputs are those of the plain entry points, bit for bit
    if gated:
        o2, h2 = K.kda_chunk_fwd_gated(*args, gz["A"], gz["z"], initial_state=h0, cu_seqlens=cu,
                                       o_dtype=torch.float32)
    else:
        o2, h2 = K.kda_chunk_fwd(*args, gz["g"], initial_state=h0, cu_seqlens=cu, o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(hT, h2)
    # every mapped slot against the oracle's state at that boundary; the other slots untouched
    bases = _ckpt_bases(d, every)
    if units is None:
        units = [(n, h) for n in range(N) for h in range(H)]
    ref = oracle.forward_checkpoints(d["q"], d["k"], d["v"], d["beta"], g, every, units=units,
                                     S0=d["S0"], cu_seqlens=d["cu_seqlens"].numpy() if cu is not None else None)
    ck_host = ck.cpu()
    worst = 0.0
    for (n, h), states in ref.items():
        base, count = bases[n]
        assert len(states) == count
        for j, S_j in enumerate(states):
            worst = max(worst, rel_err(ck_host[base + j, h], S_j))
    say(f"  {label} checkpoints: worst S err {worst:.2e}")
    assert worst <= tol
    mapped = set()
    for base, count in bases:
        mapped.update(range(base, base + count))
    for s in range(slots):
        if s not in mapped:
            assert torch.isnan(ck_host[s]).all(), s


@pytest.mark.parametrize("case", ["fixed", "varlen", "f32", "gated", "fused_whole"])
def test_checkpoints_parity(case):
    """States stored every k tokens equal the oracle's states at those boundaries; o and the
    final state equal the plain entry points' bit for bit; slots between packed sequences keep
    their contents."""
    if case == "fixed":
        d, every, tol = prefill_case("prefill_bf16", B=2, H=2, T=300), 64, TOL["bf16"]
    elif case == "varlen":
        d, every, tol = prefill_case("prefill_varlen", seqlens=[0, 5, 64, 130, 200, 17, 256], H=3), 64, TOL["bf16"]
    elif case == "f32":
        d, every, tol = prefill_case("prefill_f32_small"), 64, TOL["f32"]
    elif case == "gated":
        d, every, tol = prefill_case("prefill_bf16", B=2, H=2, T=257), 128, TOL["bf16"]
    else:   # 256 (sequence, head) units: whole sequences in the fused kernel, checkpoints from LDS
        d, every, tol = prefill_case("prefill_bf16", B=64, H=4, T=200), 64, TOL["bf16"]
    say("checkpoints", case, every)
    _check_checkpoints(d, every, tol, gated=(case in ("gated", "fused_whole")), label=case)


def test_checkpoints_full_size_sampled():
    """The bf16 prefill workload (B=4, H=16, T=4096) with a checkpoint every 512 tokens, fused
    gate; four units checked at all eight boundaries."""
    d = prefill_case("prefill_bf16")
    say("checkpoints full size", d["cfg"])
    _check_checkpoints(d, 512, TOL["bf16"], gated=True, units=[(0, 0), (1, 5), (2, 11), (3, 15)],
                       label="full")


# ---- long sequences split into 8192-token segments ----------------------------------------------
# A launch is segmented when its state pass would use at most 128 column blocks of 64 state
# columns and sequences average 16384 tokens or more: pass 1 (the (M, B) pairs of every segment
# but each sequence's last; at d_k != d_v segment 0 from the initial state and the middle
# segments' pairs), the scan of the pairs, pass 2 (longest segments first).  These shapes are
# segmented; every unit is checked.
@pytest.mark.parametrize("T", [2 * 8192, 2 * 8192 + 64, 3 * 8192 + 100, 4 * 8192 - 17])
def test_segmented_prefill_lengths(T):
    """Two segments (no middle one), a one-chunk last segment, a ragged last segment, four
    segments; random initial state."""
    d = prefill_case("prefill_bf16", B=1, H=2, T=T)
    say("segmented prefill", T)
    check_full(d, oracle_g(d), TOL["bf16"], label=f"seg T={T}")


def test_segmented_prefill_batch_and_packed():
    """Two fixed-length sequences, then a packed batch mixing long, short and empty sequences."""
    d = prefill_case("prefill_bf16", B=2, H=2, T=3 * 8192 + 5)
    say("segmented prefill, B=2")
    check_full(d, oracle_g(d), TOL["bf16"], label="seg B=2")
    lens = [40000, 200, 0, 25000, 18000]
    d = prefill_case("prefill_varlen", seqlens=lens, H=2)
    say("segmented prefill, packed", lens)
    check_full(d, oracle_g(d), TOL["bf16"], label="seg packed")


def test_segmented_prefill_packed_equal_last_segments():
    """Pass 2 runs the sequences' last segments by decreasing length: a packed batch whose last
    segments tie (16 tokens twice, 200 tokens twice) next to a full one, a long one and an empty
    sequence."""
    lens = [16400, 200, 24592, 0, 200, 3 * 8192, 60000]
    d = prefill_case("prefill_varlen", seqlens=lens, H=2)
    say("segmented prefill, packed, tied last segments", lens)
    check_full(d, oracle_g(d), TOL["bf16"], label="seg packed ties")


def test_segmented_prefill_most_sequences():
    """The most sequences a segmented launch takes (128 (sequence, head, 64-column) units at
    d_k = d_v = 64, one head), lengths spread around 16 K tokens so that every last segment
    differs: pass 2 ranks 128 last segments."""
    lens = [16400 + (37 * i) % 2000 for i in range(128)]
    d = prefill_case("prefill_varlen", seqlens=lens, H=1, dk=64, dv=64)
    say("segmented prefill, 128 packed sequences", sum(lens))
    check_full(d, oracle_g(d), TOL["bf16"], label="seg 128 seqs")


def test_segmented_prefill_mild_decay():
    """Gates scaled down 20x (mean decay about e^-0.125 per token): every channel carries state
    across segment boundaries, so each segment's transition M is far from 0 and the pair scan
    decides the later segments' outputs."""
    d = prefill_case("prefill_bf16", B=1, H=2, T=3 * 8192 + 5)
    say("segmented prefill, mild decay")
    check_full(d, oracle_g(d) / 20.0, TOL["bf16"], label="seg g/20")


def test_segmented_prefill_f32_and_fused_gate():
    """fp32 inputs (32-token chunks, tolerance 1e-4) and the fused gate on segmented launches."""
    d = prefill_case("prefill_f32_small", T=20000)
    say("segmented prefill f32")
    check_full(d, oracle_g(d), TOL["f32"], label="seg f32")
    d = prefill_case("prefill_bf16", B=1, H=2, T=3 * 8192 + 33)
    o, hT = _gated(d)
    o_ref, S_ref, _ = oracle.forward(d["q"], d["k"], d["v"], d["beta"], oracle.gate(d["A"], d["z"]),
                                     S0=d["S0"])
    eo, es = rel_err(o, o_ref), rel_err(hT, S_ref)
    say(f"  seg fused gate: o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_segmented_checkpoints():
    """Checkpoints every 4096 tokens on a segmented launch (boundaries inside and at the ends of
    segments), fixed-length and packed."""
    d = prefill_case("prefill_bf16", B=1, H=2, T=3 * 8192 + 300)
    say("segmented checkpoints")
    _check_checkpoints(d, 4096, TOL["bf16"], label="seg")
    d = prefill_case("prefill_varlen", seqlens=[40000, 200, 0, 25000, 18000], H=2)
    _check_checkpoints(d, 4096, TOL["bf16"], gated=True, label="seg packed")


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128)])
def test_segmented_prefill_head_dims(dk, dv):
    """Segmented launches whose segment passes run 4-wave workgroups (d_k != d_v): the M column
    blocks (d_k) and B column blocks (d_v) differ in number."""
    d = prefill_case("prefill_bf16", B=1, H=2, T=3 * 8192 + 77, dk=dk, dv=dv)
    say("segmented prefill dims", dk, dv)
    check_full(d, oracle_g(d), TOL["bf16"], label=f"seg dk={dk} dv={dv}")
