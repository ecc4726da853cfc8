"""Shared helpers for the GPU parity tests (inputs from the seeded generators, expected values
from the fp64 oracle only)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from gated_delta_rule_60_amd import inputs

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def rel_err(x, ref) -> float:
    """max_i |x_i - ref_i| / max_i |ref_i| (the parity metric), in fp64."""
    x = np.asarray(x.detach().double().cpu().numpy() if isinstance(x, torch.Tensor) else x,
                   dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.abs(ref).max()
    return float(np.abs(x - ref).max() / (denom if denom > 0 else 1.0))


def _np64(x):
    return np.asarray(x.detach().double().cpu().numpy() if isinstance(x, torch.Tensor) else x,
                      dtype=np.float64)


def worst_unit_errs(o, o_ref, S, S_ref, cu=None):
    """The parity metric per (sequence, head) unit -- each unit's o rows and final state
    normalised by that unit's own max|ref| -- and the worst over units: (o err, state err)."""
    o, o_ref, S, S_ref = _np64(o), _np64(o_ref), _np64(S), _np64(S_ref)
    N, H = S_ref.shape[:2]
    eo = es = 0.0
    for n in range(N):
        b, rows = (0, slice(int(cu[n]), int(cu[n + 1]))) if cu is not None else (n, slice(None))
        for h in range(H):
            ref = o_ref[b, rows, h]
            if ref.size:
                eo = max(eo, rel_err(o[b, rows, h], ref))
            es = max(es, rel_err(S[n, h], S_ref[n, h]))
    return eo, es


def oracle_g(d, g_dtype=torch.float32):
    """Gate values from the fp64 oracle, rounded to the dtype both sides consume."""
    g64 = oracle.gate(d["A"], d["z"])
    return torch.from_numpy(g64).to(g_dtype)


def to_dev(d, keys=("q", "k", "v", "beta", "g", "S0", "cu_seqlens", "A", "z")):
    out = dict(d)
    for key in keys:
        if key in d and isinstance(d[key], torch.Tensor):
            out[key] = d[key].to(DEV)
    return out


def prefill_case(name, **over):
    cfg = inputs.config(name, **{k: v for k, v in over.items() if k != "seqlens"})
    d = inputs.make_prefill(cfg, seqlens=over.get("seqlens"))
    d["cfg"] = cfg
    return d
