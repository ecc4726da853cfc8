"""GPU, white box: the workspace records of the intra-block kernel (16-bit inputs, head sizes 64
and 128) against their definitions, evaluated in fp64 from the same inputs.  The fused kernel
(whole sequences at d_k = d_v = 128 when the (sequence, head) units fill the chip) builds the same
records in LDS, where they are checked only through its outputs.

A record covers 32 tokens, two 16-token sub-blocks, with G the per-channel cumsum of g from the
record's first token [habr § Последовательность: the bounded gate keeps every factor in range]:
  Kt = e^G k,  Qt = e^G q (times the output scale),  Kb = e^{G_31 - G} k      (per sub-block)
  A[i, j] = beta_i sum_c k_ic k_jc e^{G_ic - G_jc} (j < i),  P[i, j] = the same with q_i, j <= i
  T' = (I + A)^{-1} Diag(beta) (its diagonal blocks T'_00, T'_11),  C[i, j] = sum_c k_{16+i,c}
  k_jc e^{G_{16+i,c} - G_jc} (the cross block of A without beta, stored negated),
  and e^{G_31} - 1 per channel.
The record stores them in fp16 MFMA fragment order (-Kt, Qt: 16x16x32 A operands, Kt negated;
Kb^T of both sub-blocks: one 16x16x32 A operand, channel-major, a lane's tokens of sub-block 0 then
the same tokens of sub-block 1; T', P: [16][16] tiles), so each field is checked to fp16 precision.
The gates are scaled down 20x so that every field, the cross-sub-block tiles included, is O(1).
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_60_amd import kda as K
from kda_testutil import DEV, oracle_g, prefill_case, say

pytestmark = pytest.mark.gpu

TOL = 2e-3                           # fp16 storage is 2^-11 relative


def layout(dk):
    """Byte offsets of a record at head size dk.  First what every state pass reads: -Kt_0, Kb^T
    (tiles below dk / 32), -Kt_1, Kb^T (the other tiles) -- fp16 [16][dk] arrays -- then T'_00,
    -C, T'_11 (fp16 16 x 16 tiles) and e^{G_31} - 1 (dk fp32); then Qt_0, Qt_1 and P_00, P_10,
    P_11.  Returns (array bytes, -Kt_0, -Kt_1, Qt_0, Qt_1, T', P, decay, record bytes)."""
    e2 = 16 * dk * 2
    off_t = 4 * e2
    off_g = off_t + 3 * 512
    head = off_g + 4 * dk
    off_p = head + 2 * e2
    return e2, 0, 2 * e2, head, head + e2, off_t, off_p, off_g, off_p + 3 * 512


def frag32(r, c):
    """Half index of (token r, channel c) in a 16x16x32 A-operand array: fragment c // 32, lane
    (r, (c % 16) // 4), slot 4 * ((c % 32) // 16) + c % 4."""
    return ((c >> 5) * 64 + r + 16 * ((c & 15) >> 2)) * 8 + ((c & 16) >> 2) + (c & 3)


def fragkb(c, s, t, dk):
    """Half index of (channel c, sub-block s, token t) of Kb^T in a record: tile c // 16 (1 KB;
    tiles below dk / 32 in the array after -Kt_0, the others in the one after -Kt_1), lane
    (c % 16, t // 4), slot 4 * s + t % 4."""
    ct, e2 = dk // 16, 16 * dk * 2
    tile = c >> 4
    off = np.where(tile < ct // 2, e2 + 1024 * tile, 3 * e2 + 1024 * (tile - ct // 2)) // 2
    return off + ((c & 15) + 16 * (t >> 2)) * 8 + 4 * s + (t & 3)


def fragT(r, s):
    """Half index of (row r, column s) in a [16][16] 16x16x16 A-operand tile."""
    return (r + 16 * (s >> 2)) * 4 + (s & 3)


def decode(rec, dk):
    E2, OFF_KT0, OFF_KT1, OFF_QT0, OFF_QT1, OFF_T, OFF_P, OFF_G, _ = layout(dk)
    h = lambda off, n: rec[off:off + 2 * n].view(np.float16).astype(np.float64)
    r16, c16 = np.meshgrid(np.arange(16), np.arange(dk), indexing="ij")

    def tok_major(off):
        return h(off, 16 * dk)[frag32(r16, c16)]


    rr, ss = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    tile = lambda off: h(off, 256)[fragT(rr, ss)]
    out = {}
    whole = rec[:OFF_T].view(np.float16).astype(np.float64)
    for s, (kt, qt) in enumerate(((OFF_KT0, OFF_QT0), (OFF_KT1, OFF_QT1))):
        out[f"Kt{s}"], out[f"Qt{s}"] = -tok_major(kt), tok_major(qt)
        out[f"Kb{s}"] = whole[fragkb(c16, s, r16, dk)]
    out["T00"], out["negC"], out["T11"] = tile(OFF_T), tile(OFF_T + 512), tile(OFF_T + 1024)
    out["P00"], out["P10"], out["P11"] = tile(OFF_P), tile(OFF_P + 512), tile(OFF_P + 1024)
    out["gamma"] = rec[OFF_G:OFF_G + 4 * dk].view(np.float32).astype(np.float64)
    return out


def expected(g, k, q, beta, t0, n):
    """The record's fields in fp64 for tokens t0 .. t0 + n - 1 (zero past the sequence)."""
    dk = k.shape[1]
    gx, kx, qx, bx = (np.zeros((32, dk)), np.zeros((32, dk)), np.zeros((32, dk)), np.zeros(32))
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
    C = np.zeros((16, 16))
    for i in range(16):
        for j in range(16):
            C[i, j] = np.sum(kx[16 + i] * np.exp(G[16 + i] - G[j]) * kx[j])
    out["T00"], out["negC"], out["T11"] = T[:16, :16], -C, T[16:, 16:]
    out["P00"], out["P10"], out["P11"] = P[:16, :16], P[16:, :16], P[16:, 16:]
    return out


def _check_records(W, base, slots, T, d, g, dk):
    rec_bytes = layout(dk)[-1]
    f64 = lambda x: x.double().numpy().reshape(T, -1)
    g64, k64, q64, b64 = f64(g), f64(d["k"]), f64(d["q"]), d["beta"].double().numpy().reshape(T)
    assert W.size >= (base + max(slots) + 1) * rec_bytes
    for j in slots:
        got = decode(W[(base + j) * rec_bytes:(base + j + 1) * rec_bytes], dk)
        ref = expected(g64, k64, q64, b64, 32 * j, min(T - 32 * j, 32))
        for name, r in ref.items():
            err = np.abs(got[name] - r).max() / max(np.abs(r).max(), 1e-30)
            say(f"  record {j} {name}: max|ref| {np.abs(r).max():.3e}  rel err {err:.2e}")
            assert err <= TOL, (j, name, err)


@pytest.mark.parametrize("T,DK", [(63, 64), (96, 64), (63, 128), (96, 128)])
def test_intra_records_match_definitions(T, DK):
    """T = 63: a full record and one with 31 tokens (the tail reads zeros); T = 96: three."""
    d = prefill_case("prefill_bf16", B=1, H=1, T=T, dk=DK, dv=DK)
    g = oracle_g(d) / 20.0
    say("records", T, DK)
    ws = torch.zeros(K.kda_chunk_fwd_workspace_size(1, T, 1, DK, DK), dtype=torch.uint8, device=DEV)
    K.kda_chunk_fwd(d["q"].to(DEV), d["k"].to(DEV), d["v"].to(DEV), d["beta"].to(DEV), g.to(DEV),
                    initial_state=d["S0"].to(DEV), workspace=ws)
    torch.cuda.synchronize()
    _check_records(ws.cpu().numpy(), 0, range((T + 31) // 32), T, d, g, DK)
