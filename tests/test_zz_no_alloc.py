"""kda_chunk_fwd_gated_noalloc, the prefill entry point that allocates nothing (its workspace is
the library's static device array), against kda_chunk_fwd_gated with a caller workspace: two
calls in a row, the second on a smaller input, each bit-equal to the allocating entry point and
within the parity tolerance of the fp64 oracle; and the size limit refused before any device
work."""
import pytest
import torch

import oracle
from gated_delta_rule_60_amd import kda as K
from kda_testutil import DEV, prefill_case, rel_err, say

pytestmark = pytest.mark.gpu


def _inputs(d):
    return [d[x].to(DEV) for x in ("q", "k", "v", "beta", "A", "z")]


def _check_pair(d, cu=None):
    q, k, v, beta, A, z = _inputs(d)
    h0 = d["S0"].to(DEV)
    cu_d = cu.to(DEV) if cu is not None else None
    o_ref, h_ref = K.kda_chunk_fwd_gated(q, k, v, beta, A, z, initial_state=h0, cu_seqlens=cu_d,
                                         o_dtype=torch.float32)
    o = torch.full_like(o_ref, float("nan"))
    hT = torch.full_like(h_ref, float("nan"))
    K.kda_chunk_fwd_gated_noalloc(q, k, v, beta, A, z, o, final_state=hT, initial_state=h0,
                                  cu_seqlens=cu_d)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(hT, h_ref)
    g64 = oracle.gate(d["A"], d["z"])
    o64, S64, _ = oracle.forward(d["q"], d["k"], d["v"], d["beta"], g64, S0=d["S0"],
                                 cu_seqlens=cu.numpy() if cu is not None else None)
    eo, es = rel_err(o, o64), rel_err(hT, S64)
    say(f"  o err {eo:.2e}  S err {es:.2e}")
    tol = 1e-4 if d["q"].dtype == torch.float32 else 2e-3
    assert eo <= tol and es <= tol


def test_noalloc_matches_gated_on_two_calls():
    """16-bit inputs: a long sequence in 8192-token segments (the array holds the records and the
    segment buffers), then a smaller input run whole (records only)."""
    for c in (dict(B=1, H=2, T=20000), dict(B=1, H=4, T=3000)):
        d = prefill_case("prefill_bf16", **c)
        need = K.kda_chunk_fwd_workspace_size(c["B"], c["B"] * c["T"], c["H"], 128, 128)
        say("noalloc", c, "workspace", need)
        assert need > 0
        _check_pair(d)


def test_noalloc_fp32_inputs_two_calls():
    """fp32 inputs (the array holds the intra-block records), then a smaller input."""
    for c in (dict(B=2, H=2, T=300), dict(B=1, H=2, T=70)):
        d = prefill_case("prefill_f32_small", s0_std=0.1, **c)
        say("noalloc fp32", c)
        _check_pair(d)


def test_noalloc_packed_batch():
    lens = [0, 33, 2048, 1, 1300]
    d = prefill_case("prefill_varlen", seqlens=lens, H=3)
    say("noalloc packed", lens)
    _check_pair(d, cu=d["cu_seqlens"])


def test_noalloc_refuses_sizes_beyond_the_array():
    """A workspace need above the array's size returns KDA_ERR_WORKSPACE before any device work
    (the pointers below are never used)."""
    lib = K.load_library()
    H, dk, dv, T = 16, 128, 128, 8192
    # fp32 inputs keep their records in the workspace: 4 x 8192 tokens x 16 heads do not fit
    need = K.kda_chunk_fwd_workspace_size(4, 4 * T, H, dk, dv, in_dtype=torch.float32)
    assert need > K.NOALLOC_SCRATCH_BYTES
    p = 1 << 40
    args = [p, p + (1 << 32), p + (2 << 32), p + (3 << 32), 0, p + (4 << 32), p + (5 << 32), 0,
            -5.0, None, None, None, p + (6 << 32), 0, 4, T, 4, H, dk, dv, 64, 1.0, None]
    st = lib.kda_chunk_fwd_gated_noalloc(*args)
    assert st == 3, K.kda_status_string(st)
    # the bf16 prefill workload (4 x 4096 tokens, 16 heads) fits
    assert K.kda_chunk_fwd_workspace_size(4, 4 * 4096, H, dk, dv) <= K.NOALLOC_SCRATCH_BYTES
