"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix, written so
that none of them re-types the oracle's own loop.  Each check takes the path of an oracle
library build (None = the real one) so the same checks can be run against deliberately broken
builds (tests/test_oracle_mutants.py) to show that a plausible mistake fails at least one.

Pages cited: [habr] "Как устроена Kimi K3: 2,8 трлн параметров, линейное внимание и агенты на
миллион токенов" (savepearlharbor.com); [bagrov] "Архитектура Kimi K3: как открытая модель с
миллионным контекстом конкурирует с лидерами рынка" (bagrov.by).
"""
from __future__ import annotations

import math

import numpy as np
import scipy.special

import oracle

G_MIN = -5.0


def _rand_unit_rows(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# --------------------------------------------------------------------------------- gate
def check_gate_closed_forms(lib=None):
    """Gate g = g_min * sigmoid(exp(A) z) [habr, § Последовательность]."""
    rng = np.random.default_rng(1)
    H, dk = 3, 7
    A = rng.normal(0, 0.5, (H, dk))
    # z = 0: sigmoid(0) = 1/2 exactly, whatever A is
    g = oracle.gate(A, np.zeros((4, H, dk)), G_MIN, lib_path=lib)
    assert np.all(g == G_MIN / 2), "gate(z=0) must be g_min/2"
    # A = 0, z = ln 3: sigmoid(ln 3) = 3/4
    g = oracle.gate(np.zeros((H, dk)), np.full((2, H, dk), math.log(3.0)), G_MIN, lib_path=lib)
    assert np.allclose(g, 0.75 * G_MIN, rtol=0, atol=1e-14), "gate(A=0, z=ln3) must be 3/4 g_min"
    # symmetry sigmoid(x) + sigmoid(-x) = 1
    z = rng.normal(0, 2, (5, H, dk))
    gp = oracle.gate(A, z, G_MIN, lib_path=lib)
    gm = oracle.gate(A, -z, G_MIN, lib_path=lib)
    assert np.allclose(gp + gm, G_MIN, rtol=0, atol=1e-14), "g(z) + g(-z) must equal g_min"
    # saturation limits
    assert np.all(oracle.gate(A, np.full((1, H, dk), 1e5), G_MIN, lib_path=lib) == G_MIN)
    assert np.all(oracle.gate(A, np.full((1, H, dk), -1e5), G_MIN, lib_path=lib) == 0.0)
    # a library sigmoid (scipy's expit) on the same inputs
    ref = G_MIN * scipy.special.expit(np.exp(A)[None] * z)
    assert np.allclose(gp, ref, rtol=1e-14, atol=1e-300), "gate disagrees with expit"
    # strictly decreasing in z (exp(A) > 0), bounded: alpha = exp(g) in [e^-5, 1]
    zs = np.linspace(-30, 30, 601)[:, None, None] * np.ones((1, H, dk))
    gs = oracle.gate(A, zs, G_MIN, lib_path=lib)
    assert np.all(np.diff(gs, axis=0) <= 0), "gate must not increase with z"
    alpha = np.exp(gs)
    assert alpha.min() >= math.exp(G_MIN) and alpha.max() <= 1.0


def check_gate_dtypes(lib=None):
    """bf16/fp32 z are upcast exactly: same values in fp64 give bit-identical g."""
    import torch
    rng = np.random.default_rng(2)
    A = torch.tensor(rng.normal(0, 0.5, (2, 8)), dtype=torch.float32)
    z = torch.tensor(rng.normal(0, 1, (6, 2, 8)), dtype=torch.float32).to(torch.bfloat16)
    g1 = oracle.gate(A, z, lib_path=lib)
    g2 = oracle.gate(A.double(), z.double(), lib_path=lib)
    assert np.array_equal(g1, g2)


# ------------------------------------------------------------------ recurrence (forward)
def _fwd(lib, q, k, v, beta, g, S0=None, cu=None, scale=1.0):
    o, S, _ = oracle.forward(q, k, v, beta, g, S0=S0, cu_seqlens=cu, scale=scale, nthreads=1,
                             lib_path=lib)
    return o, S


def check_worked_example(lib=None):
    """Two tokens worked by hand (d_k = 2, d_v = 1, S0 = [1, 2]^T):
    t=1: alpha=(1/2, 1), k=(1, 0), v=3, beta=1/2, q=(0, 1)
         decay S=(1/2, 2); u = 3 - 1/2 = 5/2; S += 1/2*(1,0)*5/2 -> S=(7/4, 2); o = 2
    t=2: alpha=(1, 1/4), k=(3/5, 4/5), v=-1, beta=1, q=(1, 1)
         decay S=(7/4, 1/2); S^T k = 21/20 + 2/5 = 29/20; u = -1 - 29/20 = -49/20
         S += (3/5, 4/5)*(-49/20) -> S=(7/25, -73/50); o = 7/25 - 73/50 = -59/50
    """
    q = np.array([[0.0, 1.0], [1.0, 1.0]]).reshape(1, 2, 1, 2)
    k = np.array([[1.0, 0.0], [0.6, 0.8]]).reshape(1, 2, 1, 2)
    v = np.array([3.0, -1.0]).reshape(1, 2, 1, 1)
    beta = np.array([0.5, 1.0]).reshape(1, 2, 1)
    g = np.log(np.array([[0.5, 1.0], [1.0, 0.25]])).reshape(1, 2, 1, 2)
    S0 = np.array([1.0, 2.0]).reshape(1, 1, 2, 1)
    o, S = _fwd(lib, q, k, v, beta, g, S0)
    assert np.allclose(o.ravel(), [2.0, -59 / 50], rtol=0, atol=1e-14), o.ravel()
    assert np.allclose(S.ravel(), [7 / 25, -73 / 50], rtol=0, atol=1e-14), S.ravel()


def check_retrieval(lib=None):
    """Delta rule, beta = 1, |k| = 1: right after the write the state returns v for k
    ([bagrov, § Как архитектура … миллион токенов]: the token erases what is stored along k
    and writes v there).  Holds for any forget factor only if the forget comes first
    [habr, § Последовательность]; q = k reads the updated state, so o_t = v_t."""
    rng = np.random.default_rng(3)
    T, dk, dv = 24, 8, 5
    k = _rand_unit_rows(rng, (1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    beta = np.ones((1, T, 1))
    S0 = rng.standard_normal((1, 1, dk, dv))
    for g in (rng.uniform(-5, 0, (1, T, 1, dk)), np.zeros((1, T, 1, dk))):
        o, _ = _fwd(lib, k, k, v, beta, g, S0)
        assert np.allclose(o, v, rtol=0, atol=1e-12), "retrieval invariant broken"


def check_pure_decay(lib=None):
    """beta = 0: nothing is written, the state only decays channel-wise:
    S_T = Diag(exp(sum_t g_t)) S0 and o_t = S0^T (exp(G_t) * q_t), G_t = sum_{tau<=t} g_tau."""
    rng = np.random.default_rng(4)
    T, dk, dv = 17, 6, 4
    q = rng.standard_normal((1, T, 1, dk))
    k = rng.standard_normal((1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    g = rng.uniform(-5, 0, (1, T, 1, dk))
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, S = _fwd(lib, q, k, v, np.zeros((1, T, 1)), g, S0)
    G = np.cumsum(g[0, :, 0, :], axis=0)                   # [T, dk], inclusive
    exp_S = np.exp(G[-1])[:, None] * S0[0, 0]
    exp_o = (np.exp(G) * q[0, :, 0, :]) @ S0[0, 0]         # [T, dv]
    assert np.allclose(S[0, 0], exp_S, rtol=1e-13, atol=1e-300)
    assert np.allclose(o[0, :, 0, :], exp_o, rtol=1e-12, atol=1e-14)


def check_deltanet_limit(lib=None):
    """alpha = 1 (g = 0), orthonormal keys, S0 = 0: every write lands on an empty direction,
    so S_T = sum_t beta_t k_t v_t^T, and querying with an earlier key k_j returns beta_j v_j."""
    rng = np.random.default_rng(5)
    T, dk, dv = 6, 8, 3
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:, :T].T.reshape(1, T, 1, dk)
    v = rng.standard_normal((1, T, 1, dv))
    beta = rng.uniform(0.1, 1.0, (1, T, 1))
    perm = [0, 0, 1, 2, 1, 4]                               # query t asks for key perm[t] <= t
    q = k[:, perm]
    o, S = _fwd(lib, q, k, v, beta, np.zeros((1, T, 1, dk)))
    exp_S = sum(beta[0, t, 0] * np.outer(k[0, t, 0], v[0, t, 0]) for t in range(T))
    assert np.allclose(S[0, 0], exp_S, rtol=0, atol=1e-13)
    for t, j in enumerate(perm):
        assert np.allclose(o[0, t, 0], beta[0, j, 0] * v[0, j, 0], rtol=0, atol=1e-13)


def check_unrolled_product(lib=None):
    """Brute force with explicit transition matrices: M_t = (I - beta_t k_t k_t^T) Diag(alpha_t),
    S_t = M_t S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t, on general inputs (unnormalised k,
    beta outside [0, 1], d_k != d_v, scale != 1)."""
    rng = np.random.default_rng(6)
    T, dk, dv, scale = 9, 5, 3, 0.7
    q = rng.standard_normal((1, T, 1, dk))
    k = rng.standard_normal((1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    beta = rng.uniform(-0.5, 1.5, (1, T, 1))
    g = rng.uniform(-5, 0, (1, T, 1, dk))
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, S = _fwd(lib, q, k, v, beta, g, S0, scale=scale)
    St = S0[0, 0].copy()
    for t in range(T):
        kt, b = k[0, t, 0], beta[0, t, 0]
        M = (np.eye(dk) - b * np.outer(kt, kt)) @ np.diag(np.exp(g[0, t, 0]))
        # closed product form, accumulated explicitly
        St = M @ St + b * np.outer(kt, v[0, t, 0])
        assert np.allclose(o[0, t, 0], scale * St.T @ q[0, t, 0], rtol=1e-11, atol=1e-12)
    # and the fully unrolled sum: S_T = (prod M) S0 + sum_t (prod_{j>t} M_j) beta_t k_t v_t^T
    Ms = [(np.eye(dk) - beta[0, t, 0] * np.outer(k[0, t, 0], k[0, t, 0]))
          @ np.diag(np.exp(g[0, t, 0])) for t in range(T)]

    def prod(a, b):  # M_{b-1} ... M_a
        P = np.eye(dk)
        for j in range(a, b):
            P = Ms[j] @ P
        return P
    unrolled = prod(0, T) @ S0[0, 0] + sum(
        prod(t + 1, T) @ (beta[0, t, 0] * np.outer(k[0, t, 0], v[0, t, 0])) for t in range(T))
    assert np.allclose(S[0, 0], unrolled, rtol=1e-11, atol=1e-12)


def check_pair_scan(lib=None):
    """Segments combine as affine pairs (M, B) with (M2, B2) o (M1, B1) = (M2 M1, M2 B1 + B2)
    ([habr, § Инфраструктура триллионной MoE]: a segment is its accumulated transform plus the
    state it builds from zero).  M of a segment = its final state from S0 = I with v = 0."""
    rng = np.random.default_rng(7)
    T, dk, dv = 30, 6, 4
    q = rng.standard_normal((1, T, 1, dk))
    k = _rand_unit_rows(rng, (1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    beta = rng.uniform(0, 1, (1, T, 1))
    g = rng.uniform(-1, 0, (1, T, 1, dk))
    S0 = rng.standard_normal((1, 1, dk, dv))
    _, S_full = _fwd(lib, q, k, v, beta, g, S0)
    cuts = [0, 7, 19, T]
    Mtot, Btot = np.eye(dk), np.zeros((dk, dv))
    for a, b in zip(cuts[:-1], cuts[1:]):
        sl = slice(a, b)
        qs, ks, bs, gs = q[:, sl], k[:, sl], beta[:, sl], g[:, sl]
        _, M = _fwd(lib, qs, ks, np.zeros((1, b - a, 1, dk)), bs, gs,
                    np.eye(dk).reshape(1, 1, dk, dk))
        _, Bm = _fwd(lib, qs, ks, v[:, sl], bs, gs, None)
        Mtot, Btot = M[0, 0] @ Mtot, M[0, 0] @ Btot + Bm[0, 0]
    assert np.allclose(Mtot @ S0[0, 0] + Btot, S_full[0, 0], rtol=1e-11, atol=1e-12)


def check_linearity(lib=None):
    """For fixed q, k, beta, g the map (v, S0) -> (o, S_T) is linear."""
    rng = np.random.default_rng(8)
    T, dk, dv = 11, 5, 4
    q = rng.standard_normal((1, T, 1, dk))
    k = rng.standard_normal((1, T, 1, dk))
    beta = rng.uniform(0, 1, (1, T, 1))
    g = rng.uniform(-5, 0, (1, T, 1, dk))
    v1, v2 = rng.standard_normal((2, 1, T, 1, dv))
    s1, s2 = rng.standard_normal((2, 1, 1, dk, dv))
    a, b = 0.75, -1.5
    o1, S1 = _fwd(lib, q, k, v1, beta, g, s1)
    o2, S2 = _fwd(lib, q, k, v2, beta, g, s2)
    o3, S3 = _fwd(lib, q, k, a * v1 + b * v2, beta, g, a * s1 + b * s2)
    assert np.allclose(o3, a * o1 + b * o2, rtol=1e-12, atol=1e-12)
    assert np.allclose(S3, a * S1 + b * S2, rtol=1e-12, atol=1e-12)


def check_nonexpansive(lib=None):
    """|k| = 1, beta in [0, 1], alpha <= 1: each transition has spectral norm <= 1, so with
    nothing written (v = 0) the state's spectral norm never grows."""
    rng = np.random.default_rng(9)
    T, dk, dv = 40, 8, 8
    k = _rand_unit_rows(rng, (1, T, 1, dk))
    beta = rng.uniform(0, 1, (1, T, 1))
    g = rng.uniform(-0.2, 0, (1, T, 1, dk))
    S0 = rng.standard_normal((1, 1, dk, dv))
    _, S = _fwd(lib, k, k, np.zeros((1, T, 1, dv)), beta, g, S0)
    assert np.linalg.norm(S[0, 0], 2) <= np.linalg.norm(S0[0, 0], 2) * (1 + 1e-12)


def check_batch_layouts(lib=None):
    """Packed variable-length batches, fixed-length batches and a split at any token all give
    the same per-sequence results as separate single-sequence runs (state carried across)."""
    rng = np.random.default_rng(10)
    H, dk, dv = 2, 4, 3
    lens = [5, 1, 9, 3]
    T = sum(lens)
    q = rng.standard_normal((1, T, H, dk))
    k = _rand_unit_rows(rng, (1, T, H, dk))
    v = rng.standard_normal((1, T, H, dv))
    beta = rng.uniform(0, 1, (1, T, H))
    g = rng.uniform(-5, 0, (1, T, H, dk))
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    cu = np.cumsum([0] + lens).astype(np.int32)
    o, S = _fwd(lib, q, k, v, beta, g, S0, cu)
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        sl = slice(int(a), int(b))
        o1, S1 = _fwd(lib, q[:, sl], k[:, sl], v[:, sl], beta[:, sl], g[:, sl], S0[n:n + 1])
        assert np.array_equal(o[:, sl], o1) and np.array_equal(S[n], S1[0])
        # split after the first token, carrying the emitted state
        if b - a > 1:
            sa, sb = slice(int(a), int(a) + 1), slice(int(a) + 1, int(b))
            oa, Sa = _fwd(lib, q[:, sa], k[:, sa], v[:, sa], beta[:, sa], g[:, sa], S0[n:n + 1])
            ob, Sb = _fwd(lib, q[:, sb], k[:, sb], v[:, sb], beta[:, sb], g[:, sb], Sa)
            assert np.array_equal(np.concatenate([oa, ob], 1), o1) and np.array_equal(Sb, S1)
    # fixed-length batch of 2 equals two single runs
    qb = rng.standard_normal((2, 4, H, dk))
    kb, vb = _rand_unit_rows(rng, (2, 4, H, dk)), rng.standard_normal((2, 4, H, dv))
    bb, gb = rng.uniform(0, 1, (2, 4, H)), rng.uniform(-5, 0, (2, 4, H, dk))
    ob, Sb = _fwd(lib, qb, kb, vb, bb, gb, S0[:2])
    for n in range(2):
        o1, S1 = _fwd(lib, qb[n:n + 1], kb[n:n + 1], vb[n:n + 1], bb[n:n + 1], gb[n:n + 1],
                      S0[n:n + 1])
        assert np.array_equal(ob[n:n + 1], o1) and np.array_equal(Sb[n], S1[0])


def check_dtype_upcast(lib=None):
    """bf16 and fp32 inputs are consumed exactly: same values passed as fp64 give identical bits."""
    import torch
    rng = np.random.default_rng(11)
    T, H, dk, dv = 7, 2, 4, 3
    t = lambda a, dt: torch.tensor(a, dtype=torch.float32).to(dt)  # noqa: E731
    for dt in (torch.bfloat16, torch.float32):
        q, k = t(rng.standard_normal((1, T, H, dk)), dt), t(rng.standard_normal((1, T, H, dk)), dt)
        v, beta = t(rng.standard_normal((1, T, H, dv)), dt), t(rng.uniform(0, 1, (1, T, H)), dt)
        g = t(rng.uniform(-5, 0, (1, T, H, dk)), dt)
        S0 = t(rng.standard_normal((1, H, dk, dv)), torch.float32)
        o1, S1 = _fwd(lib, q, k, v, beta, g, S0)
        o2, S2 = _fwd(lib, q.double(), k.double(), v.double(), beta.double(), g.double(),
                      S0.double())
        assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def check_decode(lib=None):
    """The decode step on N independent states equals one token of the forward pass for each,
    and obeys the retrieval invariant on its own."""
    rng = np.random.default_rng(12)
    N, H, dk, dv = 3, 2, 6, 4
    q = rng.standard_normal((N, H, dk))
    k = _rand_unit_rows(rng, (N, H, dk))
    v = rng.standard_normal((N, H, dv))
    beta = rng.uniform(0, 1, (N, H))
    g = rng.uniform(-5, 0, (N, H, dk))
    S = rng.standard_normal((N, H, dk, dv))
    S_dec = S.copy()
    o = oracle.decode_step(q, k, v, beta, g, S_dec, scale=0.5, lib_path=lib)
    for n in range(N):
        o1, S1 = _fwd(lib, q[n][None, None], k[n][None, None], v[n][None, None],
                      beta[n][None, None], g[n][None, None], S[n][None], scale=0.5)
        assert np.allclose(o[n], o1[0, 0], rtol=1e-14, atol=1e-15)
        assert np.allclose(S_dec[n], S1[0], rtol=1e-14, atol=1e-15)
    S_r = S.copy()
    o_r = oracle.decode_step(k, k, v, np.ones((N, H)), g, S_r, lib_path=lib)
    assert np.allclose(o_r, v, rtol=0, atol=1e-12)


def check_forward_units(lib=None, forward_units=None):
    """oracle.forward_units, the reference the sampled parity tests of the long and packed
    workloads compare against, returns for each chosen (sequence, head) unit exactly the rows of
    o and the final state that oracle.forward (pinned above) gives for the whole batch: a
    fixed-length batch with bf16 inputs, fp32 S0 and scale != 1, and a packed batch with empty
    and unequal sequences, per-sequence S0 and without one.  `forward_units` replaces the
    function under test (the mutation tests pass deliberately broken copies)."""
    import torch
    fu = forward_units or oracle.forward_units
    rng = np.random.default_rng(13)
    t = lambda a, dt: torch.tensor(a, dtype=torch.float32).to(dt)  # noqa: E731
    # fixed-length batch: B = 3 sequences of T tokens, bf16 inputs, fp32 initial states
    B, T, H, dk, dv, scale = 3, 11, 3, 5, 4, 0.5
    bf = torch.bfloat16
    q, k = t(rng.standard_normal((B, T, H, dk)), bf), t(_rand_unit_rows(rng, (B, T, H, dk)), bf)
    v, beta = t(rng.standard_normal((B, T, H, dv)), bf), t(rng.uniform(0, 1, (B, T, H)), bf)
    g = t(rng.uniform(-5, 0, (B, T, H, dk)), torch.float32)
    S0 = t(rng.standard_normal((B, H, dk, dv)), torch.float32)
    o, S = _fwd(lib, q, k, v, beta, g, S0, scale=scale)
    units = [(0, 0), (2, 1), (1, 2), (2, 2), (0, 1)]
    res = fu(q, k, v, beta, g, units, S0=S0, scale=scale, lib_path=lib)
    assert set(res) == set(units)
    for (n, h), (o_u, S_u) in res.items():
        assert o_u.shape == (T, dv) and S_u.shape == (dk, dv)
        assert np.array_equal(o_u, o[n, :, h]), f"o of unit {(n, h)}"
        assert np.array_equal(S_u, S[n, h]), f"final state of unit {(n, h)}"
    # packed batch with an empty first sequence and unequal lengths
    lens = [0, 7, 13, 1, 9]
    N, tot = len(lens), sum(lens)
    cu = np.cumsum([0] + lens).astype(np.int32)
    q = rng.standard_normal((1, tot, H, dk))
    k = _rand_unit_rows(rng, (1, tot, H, dk))
    v = rng.standard_normal((1, tot, H, dv))
    beta = rng.uniform(0, 1, (1, tot, H))
    g = rng.uniform(-5, 0, (1, tot, H, dk))
    S0 = rng.standard_normal((N, H, dk, dv))
    everything = [(n, h) for n in range(N) for h in range(H)]
    for s0 in (S0, None):
        o, S = _fwd(lib, q, k, v, beta, g, s0, cu, scale=scale)
        res = fu(q, k, v, beta, g, everything, S0=s0, cu_seqlens=cu, scale=scale, lib_path=lib)
        assert set(res) == set(everything)
        for (n, h), (o_u, S_u) in res.items():
            a, b = int(cu[n]), int(cu[n + 1])
            assert o_u.shape == (b - a, dv), f"rows of unit {(n, h)}"
            assert np.array_equal(o_u, o[0, a:b, h]), f"o of unit {(n, h)}"
            assert np.array_equal(S_u, S[n, h]), f"final state of unit {(n, h)}"
        if s0 is not None:   # an empty sequence passes its initial state through
            assert np.array_equal(res[(0, 1)][1], S0[0, 1])


ALL_CHECKS = [
    check_gate_closed_forms, check_gate_dtypes, check_worked_example, check_retrieval,
    check_pure_decay, check_deltanet_limit, check_unrolled_product, check_pair_scan,
    check_linearity, check_nonexpansive, check_batch_layouts, check_dtype_upcast, check_decode,
    check_forward_units,
]
