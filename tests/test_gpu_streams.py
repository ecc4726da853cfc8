"""Segmented 16-bit prefills at d_k = d_v = 128 run their two head groups on the caller's stream
and a side stream the library keeps per device, forked and joined by events.  The call must keep
its ordering on the caller's stream: from a non-default stream, and captured into a graph whose
replays (with eager work between them) each equal the eager call bit for bit."""
import pytest
import torch

from gated_delta_rule_60_amd import kda as K
from kda_testutil import DEV, prefill_case, say

pytestmark = pytest.mark.gpu


def _setup():
    # one 20,000-token sequence, 2 heads: 8192-token segments, one head per group
    d = prefill_case("prefill_bf16", B=1, H=2, T=20000)
    x = {n: d[n].to(DEV) for n in ("q", "k", "v", "beta", "A", "z", "S0")}
    ws = torch.empty(K.kda_chunk_fwd_workspace_size(1, 20000, 2, 128, 128), dtype=torch.uint8,
                     device=DEV)
    o = torch.empty((1, 20000, 2, 128), dtype=torch.float32, device=DEV)
    hT = torch.empty_like(x["S0"])
    return x, ws, o, hT


def _call(x, ws, o, hT, stream=None):
    K.kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["beta"], x["A"], x["z"], initial_state=x["S0"],
                          final_state=hT, o=o, workspace=ws, stream=stream)


def test_split_prefill_on_a_side_stream_of_the_caller():
    x, ws, o, hT = _setup()
    _call(x, ws, o, hT)
    torch.cuda.synchronize()
    o_ref, h_ref = o.clone(), hT.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    o.fill_(float("nan")); hT.fill_(float("nan"))
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _call(x, ws, o, hT)
        o2, h2 = o.clone(), hT.clone()      # ordered after the call on s
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ref) and torch.equal(h2, h_ref)


def test_split_prefill_graph_replays():
    x, ws, o, hT = _setup()
    _call(x, ws, o, hT)                     # eager (creates the side stream before the capture)
    torch.cuda.synchronize()
    o_ref, h_ref = o.clone(), hT.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(x, ws, o, hT)
    torch.cuda.synchronize()
    for r in range(3):
        o.fill_(float("nan")); hT.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"replay {r}")
        assert torch.equal(o, o_ref) and torch.equal(hT, h_ref), r
