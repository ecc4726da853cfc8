"""GPU, white box: the workspace records of the intra-block kernel (16-bit inputs) against their
definitions, evaluated in fp64 from the same inputs.

A record covers 32 tokens, two 16-token sub-blocks, with G the per-channel cumsum of g from the
record's first token [habr § Последовательность: the bounded gate keeps every factor in range]:
  Kt = e^G k,  Qt = e^G q (times the output scale),  Kb = e^{G_31 - G} k      (per sub-block)
  A[i, j] = beta_i sum_c k_ic k_jc e^{G_ic - G_jc} (j < i),  P[i, j] = the same with q_i, j <= i
  T' = (I + A)^{-1} Diag(beta),  and e^{G_31} - 1 per channel.
The record stores them in fp16 MFMA fragment order (Kt, Qt: 16x16x32 A operands; Kb^T: 16x16x16
A operand, channel-major; T', P: [16][16] tiles), so each field is checked to fp16 precision.
The gates are scaled down 20x so that every field, the cross-sub-block tiles included, is O(1).
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_60_amd import kda as K
from kda_testutil import DEV, oracle_g, prefill_case, say

pytestmark = pytest.mark.gpu

DK = 128
E2 = 16 * DK * 2                     # bytes of one fp16 [16][DK] array
OFF_T = 6 * E2                       # T'_00, T'_10, T'_11
OFF_P = OFF_T + 3 * 512              # P_00, P_10, P_11
OFF_G = OFF_P + 3 * 512              # e^{G_31} - 1, DK fp32
REC = OFF_G + 4 * DK
TOL = 2e-3                           # fp16 storage is 2^-11 relative


def frag32(r, c):
    """Half index of (token r, channel c) in a 16x16x32 A-operand array: fragment c // 32, lane
    (r, (c % 16) // 4), slot 4 * ((c % 32) // 16) + c % 4."""
    return ((c >> 5) * 64 + r + 16 * ((c & 15) >> 2)) * 8 + ((c & 16) >> 2) + (c & 3)


def frag16(c, t):
    """Half index of (channel c, token t) in a 16x16x16 A-operand array (tile c // 16)."""
    return ((c >> 4) * 64 + (c & 15) + 16 * (t >> 2)) * 4 + (t & 3)


def fragT(r, s):
    """Half index of (row r, column s) in a [16][16] 16x16x16 A-operand tile."""
    return (r + 16 * (s >> 2)) * 4 + (s & 3)


def decode(rec):
    h = lambda off, n: rec[off:off + 2 * n].view(np.float16).astype(np.float64)
    r16, c16 = np.meshgrid(np.arange(16), np.arange(DK), indexing="ij")

    def tok_major(off):
        return h(off, 16 * DK)[frag32(r16, c16)]

    def chan_major(off):
        return h(off, 16 * DK)[frag16(c16, r16)]

    rr, ss = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    tile = lambda off: h(off, 256)[fragT(rr, ss)]
    out = {}
    for s in range(2):
        base = 3 * s * E2
        out[f"Kt{s}"], out[f"Qt{s}"], out[f"Kb{s}"] = (tok_major(base), tok_major(base + E2),
                                                       chan_major(base + 2 * E2))
    for name, off in (("T", OFF_T), ("P", OFF_P)):
        out[name + "00"], out[name + "10"], out[name + "11"] = (tile(off), tile(off + 512),
                                                                tile(off + 1024))
    out["gamma"] = rec[OFF_G:OFF_G + 4 * DK].view(np.float32).astype(np.float64)
    return out


def expected(g, k, q, beta, t0, n):
    """The record's fields in fp64 for tokens t0 .. t0 + n - 1 (zero past the sequence)."""
    gx, kx, qx, bx = (np.zeros((32, DK)), np.zeros((32, DK)), np.zeros((32, DK)), np.zeros(32))
    gx[:n], kx[:n], qx[:n], bx[:n] = g[t0:t0 + n], k[t0:t0 + n], q[t0:t0 + n], beta[t0:t0 + n]
    G = np.cumsum(gx, axis=0)
    A = np.zeros((32, 32))
    P = np.zeros((32, 32))
    for i in range(32):
        for j in range(i + 1):
            e = np.exp(G[i] - G[j])
            if j < i:
                A[i, j] = bx[i] * np.sum(kx[i] * e * kx[j])
            P[i, j] = np.sum(qx[i] * e * kx[j])
    T = np.linalg.solve(np.eye(32) + A, np.diag(bx))
    Kt, Qt, Kb = np.exp(G) * kx, np.exp(G) * qx, np.exp(G[31] - G) * kx
    out = {"gamma": np.expm1(G[31])}
    for s in range(2):
        sl = slice(16 * s, 16 * s + 16)
        out[f"Kt{s}"], out[f"Qt{s}"], out[f"Kb{s}"] = Kt[sl], Qt[sl], Kb[sl]
    for name, M in (("T", T), ("P", P)):
        out[name + "00"], out[name + "10"], out[name + "11"] = M[:16, :16], M[16:, :16], M[16:, 16:]
    return out


@pytest.mark.parametrize("T", [63, 96])
def test_intra_records_match_definitions(T):
    """T = 63: a full record and one with 31 tokens (the tail reads zeros); T = 96: three."""
    d = prefill_case("prefill_bf16", B=1, H=1, T=T)
    g = oracle_g(d) / 20.0
    say("records", T)
    ws = torch.zeros(K.kda_chunk_fwd_workspace_size(1, T, 1, DK, DK), dtype=torch.uint8, device=DEV)
    K.kda_chunk_fwd(d["q"].to(DEV), d["k"].to(DEV), d["v"].to(DEV), d["beta"].to(DEV), g.to(DEV),
                    initial_state=d["S0"].to(DEV), workspace=ws)
    torch.cuda.synchronize()
    W = ws.cpu().numpy()
    f64 = lambda x: x.double().numpy().reshape(T, -1)
    g64, k64, q64, b64 = f64(g), f64(d["k"]), f64(d["q"]), d["beta"].double().numpy().reshape(T)
    nrec = (T + 31) // 32
    assert W.size >= nrec * REC
    for slot in range(nrec):
        got = decode(W[slot * REC:(slot + 1) * REC])
        ref = expected(g64, k64, q64, b64, 32 * slot, min(T - 32 * slot, 32))
        for name, r in ref.items():
            err = np.abs(got[name] - r).max() / max(np.abs(r).max(), 1e-30)
            say(f"  record {slot} {name}: max|ref| {np.abs(r).max():.3e}  rel err {err:.2e}")
            assert err <= TOL, (slot, name, err)
