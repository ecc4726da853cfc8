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


def test_noalloc_matches_gated_on_two_calls():
    cases = [dict(B=3, H=4, T=1000), dict(B=1, H=2, T=129)]
    for c in cases:
        d = prefill_case("prefill_bf16", **c)
        q, k, v, beta, A, z = _inputs(d)
        h0 = d["S0"].to(DEV)
        say("noalloc", c)
        o_ref, h_ref = K.kda_chunk_fwd_gated(q, k, v, beta, A, z, initial_state=h0,
                                             o_dtype=torch.float32)
        o = torch.full_like(o_ref, float("nan"))
        hT = torch.full_like(h_ref, float("nan"))
        K.kda_chunk_fwd_gated_noalloc(q, k, v, beta, A, z, o, final_state=hT, initial_state=h0)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(hT, h_ref)
        g64 = oracle.gate(d["A"], d["z"])
        o64, S64, _ = oracle.forward(d["q"], d["k"], d["v"], d["beta"], g64, S0=d["S0"])
        eo, es = rel_err(o, o64), rel_err(hT, S64)
        say(f"  o err {eo:.2e}  S err {es:.2e}")
        assert eo <= 2e-3 and es <= 2e-3


def test_noalloc_packed_batch():
    lens = [0, 33, 64, 1, 300]
    d = prefill_case("prefill_varlen", seqlens=lens, H=3)
    q, k, v, beta, A, z = _inputs(d)
    h0, cu = d["S0"].to(DEV), d["cu_seqlens"].to(DEV)
    o_ref, h_ref = K.kda_chunk_fwd_gated(q, k, v, beta, A, z, initial_state=h0, cu_seqlens=cu,
                                         o_dtype=torch.float32)
    o = torch.empty_like(o_ref)
    hT = torch.empty_like(h_ref)
    K.kda_chunk_fwd_gated_noalloc(q, k, v, beta, A, z, o, final_state=hT, initial_state=h0,
                                  cu_seqlens=cu)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(hT, h_ref)


def test_noalloc_refuses_sizes_beyond_the_array():
    """A workspace need above the array's size returns KDA_ERR_WORKSPACE before any device work
    (the pointers below are never used)."""
    lib = K.load_library()
    H, dk, dv, T = 16, 128, 128, 8192
    need = K.kda_chunk_fwd_workspace_size(4, 4 * T, H, dk, dv)
    assert need > K.NOALLOC_SCRATCH_BYTES
    p = 1 << 40
    args = [p, p + (1 << 32), p + (2 << 32), p + (3 << 32), 1, p + (4 << 32), p + (5 << 32), 1,
            -5.0, None, None, None, p + (6 << 32), 0, 4, T, 4, H, dk, dv, 64, 1.0, None]
    st = lib.kda_chunk_fwd_gated_noalloc(*args)
    assert st == 3, K.kda_status_string(st)
    # the bf16 prefill workload (4 x 4096 tokens, 16 heads) fits
    assert K.kda_chunk_fwd_workspace_size(4, 4 * 4096, H, dk, dv) <= K.NOALLOC_SCRATCH_BYTES
