"""The fp64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(None)


def test_checkpoints_equal_prefix_final_states():
    """oracle.forward_checkpoints: checkpoint j of a unit is the final state of the oracle run on
    that unit's first j * every tokens (same fp64 loop, so equal bit for bit), for fixed-length
    and packed batches, with and without an initial state; a length that is a multiple of
    `every` ends on the full run's final state."""
    import torch
    g = torch.Generator().manual_seed(7)
    B, T, H, dk, dv, every = 2, 150, 2, 8, 6, 32
    q = torch.nn.functional.normalize(torch.randn(B, T, H, dk, generator=g, dtype=torch.float64), dim=-1)
    k = torch.nn.functional.normalize(torch.randn(B, T, H, dk, generator=g, dtype=torch.float64), dim=-1)
    v = torch.randn(B, T, H, dv, generator=g, dtype=torch.float64)
    beta = torch.sigmoid(torch.randn(B, T, H, generator=g, dtype=torch.float64))
    gg = -5.0 * torch.sigmoid(torch.randn(B, T, H, dk, generator=g, dtype=torch.float64))
    S0 = 0.1 * torch.randn(B, H, dk, dv, generator=g, dtype=torch.float64)
    ck = oracle.forward_checkpoints(q, k, v, beta, gg, every, S0=S0)
    assert set(ck) == {(n, h) for n in range(B) for h in range(H)}
    for j in range(1, T // every + 1):
        t = j * every
        _, S_t, _ = oracle.forward(q[:, :t].contiguous(), k[:, :t].contiguous(), v[:, :t].contiguous(),
                                   beta[:, :t].contiguous(), gg[:, :t].contiguous(), S0=S0)
        for (n, h), states in ck.items():
            assert len(states) == T // every
            assert np.array_equal(states[j - 1], S_t[n, h])
    # packed batch, zero initial state; the third length is a multiple of `every`
    lens = [0, 20, 64, 66]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tot = int(cu[-1])
    qp, kp, vp, bp, gp = (x[:1, :tot].contiguous() for x in (q, k, v, beta, gg))
    ck = oracle.forward_checkpoints(qp, kp, vp, bp, gp, every, cu_seqlens=cu)
    _, S_full, _ = oracle.forward(qp, kp, vp, bp, gp, cu_seqlens=cu)
    for (n, h), states in ck.items():
        assert len(states) == lens[n] // every
        for j, S_j in enumerate(states, start=1):
            s, t = int(cu[n]), int(cu[n]) + j * every
            _, S_pre, _ = oracle.forward(qp[:, s:t].contiguous(), kp[:, s:t].contiguous(),
                                         vp[:, s:t].contiguous(), bp[:, s:t].contiguous(),
                                         gp[:, s:t].contiguous())
            assert np.array_equal(S_j, S_pre[0, h])
        if lens[n] % every == 0 and lens[n]:
            assert np.array_equal(states[-1], S_full[n, h])
