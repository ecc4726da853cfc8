"""fp64 CPU reference ("oracle") for the KDA forward pass -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of ``bench.py`` may import this
package.  It wraps ``kda_oracle.c`` (plain C, fp64, one token at a time) through ctypes and
shares nothing with the HIP library.  What each function computes, and which passage of the
pages it follows, is stated in ``kda_oracle.c``.

Parity status of every function here: pinned by ``tests/test_oracle_pins.py`` (closed forms,
invariants and brute-force transition products on small inputs).  ``forward_units`` and
``forward_checkpoints`` are pinned to the pinned ``forward`` bit for bit (``check_forward_units``,
``test_checkpoints_equal_prefix_final_states``); ``tests/test_oracle_mutants.py`` shows that
broken copies of ``forward_units`` (a shifted first token, a short unit, the wrong initial-state
row or head, no scale) fail that pin.

Inputs may be numpy arrays or CPU torch tensors in float32, bfloat16 or float64; they are
handed to C in their stored dtype and upcast exactly there.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .build import build_oracle, oracle_lib_path

_F32, _BF16, _F64 = 0, 1, 2
_libs: dict = {}


def _load(path: str | None = None):
    """Load (building on first use) the oracle library at `path` (default: the built one)."""
    path = path or oracle_lib_path()
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        if path != oracle_lib_path():
            raise FileNotFoundError(path)
        build_oracle()
    lib = ctypes.CDLL(path)
    vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.kda_oracle_gate.argtypes = [vp, i32, vp, i32, vp, i64, i32, i32, dbl]
    lib.kda_oracle_gate.restype = None
    lib.kda_oracle_unit.argtypes = [vp, vp, vp, vp, vp, i32, i32, i64, i64, i32, i32, i32, i32,
                                    dbl, vp, vp, i64]
    lib.kda_oracle_unit.restype = None
    lib.kda_oracle_forward.argtypes = [vp, vp, vp, vp, vp, i32, i32, vp, i32, vp, vp, vp, i32,
                                       i64, i32, i32, i32, i32, dbl, i32]
    lib.kda_oracle_forward.restype = i32
    lib.kda_oracle_decode_step.argtypes = [vp, vp, vp, vp, vp, i32, i32, vp, vp, i32, i32, i32,
                                           i32, dbl, i32]
    lib.kda_oracle_decode_step.restype = None
    _libs[path] = lib
    return lib


def _host(x):
    """Return (contiguous numpy array, dtype code) holding x's stored bits."""
    try:
        import torch
    except ImportError:  # pragma: no cover
        torch = None
    if torch is not None and isinstance(x, torch.Tensor):
        x = x.detach().cpu().contiguous()
        if x.dtype == torch.bfloat16:
            return np.ascontiguousarray(x.view(torch.int16).numpy().view(np.uint16)), _BF16
        if x.dtype == torch.float32:
            return np.ascontiguousarray(x.numpy()), _F32
        if x.dtype == torch.float64:
            return np.ascontiguousarray(x.numpy()), _F64
        raise TypeError(f"oracle: unsupported torch dtype {x.dtype}")
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, _F32
    if x.dtype == np.float64:
        return x, _F64
    raise TypeError(f"oracle: unsupported numpy dtype {x.dtype}")


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def gate(A, z, g_min: float = -5.0, lib_path: str | None = None) -> np.ndarray:
    """g = g_min * sigmoid(exp(A) * z) in fp64.  A: [H, dk]; z: [..., H, dk] -> g like z."""
    a, adt = _host(A)
    zz, zdt = _host(z)
    H, dk = a.shape[-2], a.shape[-1]
    if zz.shape[-2:] != (H, dk):
        raise ValueError("gate: z must end in [H, dk] matching A")
    n_tokens = zz.size // (H * dk)
    g = np.empty(zz.shape, dtype=np.float64)
    _load(lib_path).kda_oracle_gate(_p(a), adt, _p(zz), zdt, _p(g), n_tokens, H, dk, float(g_min))
    return g


def _shapes(q, v, cu_seqlens):
    if q.ndim != 4 or v.ndim != 4:
        raise ValueError("q/k/g must be [B, T, H, dk] and v [B, T, H, dv]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        return B, T, B, H, dk, dv, None
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    if B != 1:
        raise ValueError("cu_seqlens requires B == 1")
    return B, T, len(cu) - 1, H, dk, dv, cu


def forward(q, k, v, beta, g, S0=None, cu_seqlens=None, scale: float = 1.0, nthreads: int = 0,
            want_o: bool = True, lib_path: str | None = None):
    """Token-by-token fp64 forward over every (sequence, head) unit.

    q, k, g: [B, T, H, dk]; v: [B, T, H, dv]; beta: [B, T, H]; S0: [N, H, dk, dv] or None;
    cu_seqlens: host int array [N+1] (B must be 1) or None.
    Returns (o [B, T, H, dv] float64 or None, S_final [N, H, dk, dv] float64, threads_used).
    """
    qq, idt = _host(q)
    kk, kdt = _host(k)
    vv, vdt = _host(v)
    bb, bdt = _host(beta)
    gg, gdt = _host(g)
    if not (idt == kdt == vdt == bdt):
        raise TypeError("q, k, v, beta must share one dtype")
    B, T, N, H, dk, dv, cu = _shapes(qq, vv, cu_seqlens)
    s0, sdt = (None, _F32) if S0 is None else _host(S0)
    o = np.zeros((B, T, H, dv), dtype=np.float64) if want_o else None
    S_final = np.empty((N, H, dk, dv), dtype=np.float64)
    used = _load(lib_path).kda_oracle_forward(_p(qq), _p(kk), _p(vv), _p(bb), _p(gg), idt, gdt, _p(s0),
                                      sdt, _p(cu), _p(o), _p(S_final), B, T, N, H, dk, dv,
                                      float(scale), int(nthreads))
    return o, S_final, used


def forward_units(q, k, v, beta, g, units, S0=None, cu_seqlens=None, scale: float = 1.0,
                  max_workers: int | None = None, lib_path: str | None = None):
    """Forward for a chosen list of (sequence, head) units only (for sampling large batches).

    Returns {(n, h): (o_unit [len, dv] float64, S_final_unit [dk, dv] float64)}.
    """
    qq, idt = _host(q)
    kk, _ = _host(k)
    vv, _ = _host(v)
    bb, _ = _host(beta)
    gg, gdt = _host(g)
    B, T, N, H, dk, dv, cu = _shapes(qq, vv, cu_seqlens)
    s0, sdt = (None, _F32) if S0 is None else _host(S0)
    lib = _load(lib_path)

    def run(unit):
        n, h = unit
        tok0 = int(cu[n]) if cu is not None else n * T
        length = int(cu[n + 1] - cu[n]) if cu is not None else T
        if s0 is None:
            S = np.zeros((dk, dv), dtype=np.float64)
        else:
            S = np.array(s0[n, h], dtype=np.float64) if sdt != _BF16 else None
            if S is None:
                raise TypeError("forward_units: bf16 S0 not supported")
        o_u = np.empty((length, dv), dtype=np.float64)
        lib.kda_oracle_unit(_p(qq), _p(kk), _p(vv), _p(bb), _p(gg), idt, gdt, tok0, length, H, h,
                            dk, dv, float(scale), _p(S), _p(o_u), dv)
        return unit, (o_u, S)

    workers = max_workers or min(len(units), os.cpu_count() or 1) or 1
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return dict(ex.map(run, list(units)))


def forward_checkpoints(q, k, v, beta, g, every: int, units=None, S0=None, cu_seqlens=None,
                        scale: float = 1.0, max_workers: int | None = None,
                        lib_path: str | None = None):
    """States after every `every` tokens of each chosen (sequence, head) unit (all units when
    `units` is None): {(n, h): [S after every, 2 every, ... tokens] (float64 [dk, dv] each)}.

    The token loop of kda_oracle.c runs segment by segment on one fp64 state, so each value is
    exactly the state a single pass holds at that position -- the prefix-cache checkpoints of a
    chunked prefill (state kept at fixed boundaries so a shared prefix is not recomputed).
    """
    qq, idt = _host(q)
    kk, _ = _host(k)
    vv, _ = _host(v)
    bb, _ = _host(beta)
    gg, gdt = _host(g)
    B, T, N, H, dk, dv, cu = _shapes(qq, vv, cu_seqlens)
    s0, sdt = (None, _F32) if S0 is None else _host(S0)
    if s0 is not None and sdt == _BF16:
        raise TypeError("forward_checkpoints: bf16 S0 not supported")
    lib = _load(lib_path)
    if units is None:
        units = [(n, h) for n in range(N) for h in range(H)]

    def run(unit):
        n, h = unit
        tok0 = int(cu[n]) if cu is not None else n * T
        length = int(cu[n + 1] - cu[n]) if cu is not None else T
        S = np.zeros((dk, dv)) if s0 is None else np.array(s0[n, h], dtype=np.float64)
        o_seg = np.empty((every, dv), dtype=np.float64)
        states = []
        for j in range(length // every):
            lib.kda_oracle_unit(_p(qq), _p(kk), _p(vv), _p(bb), _p(gg), idt, gdt, tok0 + j * every,
                                every, H, h, dk, dv, float(scale), _p(S), _p(o_seg), dv)
            states.append(S.copy())
        return unit, states

    workers = max_workers or min(len(units), os.cpu_count() or 1) or 1
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return dict(ex.map(run, list(units)))


def decode_step(q, k, v, beta, g, S: np.ndarray, scale: float = 1.0, nthreads: int = 0,
                lib_path: str | None = None):
    """One token per sequence: q, k, g [N, H, dk]; v [N, H, dv]; beta [N, H];
    S float64 [N, H, dk, dv] updated in place.  Returns o [N, H, dv] float64."""
    qq, idt = _host(q)
    kk, _ = _host(k)
    vv, _ = _host(v)
    bb, _ = _host(beta)
    gg, gdt = _host(g)
    if S.dtype != np.float64 or not S.flags.c_contiguous:
        raise TypeError("decode_step: S must be a C-contiguous float64 array")
    N, H, dk = qq.shape
    dv = vv.shape[-1]
    o = np.empty((N, H, dv), dtype=np.float64)
    _load(lib_path).kda_oracle_decode_step(_p(qq), _p(kk), _p(vv), _p(bb), _p(gg), idt, gdt, _p(S), _p(o),
                                   N, H, dk, dv, float(scale), int(nthreads))
    return o
