"""Thin ctypes binding of libkda.so: the C ABI in include/kda.h, called with torch tensors.

Argument marshalling only -- every step of the computation runs in the HIP library.  The
functions keep the C names and raise ``KDAError`` for any status other than KDA_OK.  Loading
fails loudly when the built library is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from .build import lib_path

KDA_F32, KDA_BF16 = 0, 1
KDA_OK = 0
_DT = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}


class KDAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {kda_status_string(status)} ({status})")
        self.status = status


_lib = None


def load_library(path: Optional[str] = None):
    """Load libkda.so (default: the in-tree build).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libkda.so not found at {path}; build it first "
                           "(python -m gated_delta_rule_60_amd.build or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ctypes.c_int
    lib.kda_gate.argtypes = [vp, vp, ctypes.c_int, vp, ctypes.c_int, i64, i32, i32, f32, vp]
    lib.kda_gate.restype = ctypes.c_int
    lib.kda_chunk_fwd_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, ctypes.c_int]
    lib.kda_chunk_fwd_workspace_size.restype = sz
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, vp, vp,
                                  ctypes.c_int, i32, i64, i32, i32, i32, i32, i32, f32, vp, sz, vp]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd_gated.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int, f32,
                                        vp, vp, vp, vp, ctypes.c_int, i32, i64, i32, i32, i32,
                                        i32, i32, f32, vp, sz, vp]
    lib.kda_chunk_fwd_gated.restype = ctypes.c_int
    lib.kda_chunk_fwd_checkpointed.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int,
                                               f32, vp, vp, vp, vp, ctypes.c_int, i32, i64, i32,
                                               i32, i32, i32, i32, f32, vp, i32, i64, vp, sz, vp]
    lib.kda_chunk_fwd_checkpointed.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, ctypes.c_int, vp, vp,
                                    ctypes.c_int, i32, i32, i32, i32, f32, vp]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_decode_verify.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, ctypes.c_int, vp, vp,
                                      ctypes.c_int, i32, i32, i32, i32, i32, f32, vp]
    lib.kda_decode_verify.restype = ctypes.c_int
    lib.kda_decode_commit.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, ctypes.c_int, vp, vp,
                                      i32, i32, i32, i32, i32, vp]
    lib.kda_decode_commit.restype = ctypes.c_int
    if path == lib_path():
        _lib = lib
    return lib


EXPORTED = ["kda_status_string", "kda_version", "kda_gate", "kda_chunk_fwd_workspace_size",
            "kda_chunk_fwd", "kda_chunk_fwd_gated", "kda_chunk_fwd_checkpointed", "kda_decode_step",
            "kda_decode_verify", "kda_decode_commit"]


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libkda must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dt(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)") from None


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(fn: str, status: int):
    if status != KDA_OK:
        raise KDAError(fn, status)


def kda_status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def kda_version() -> int:
    return int(load_library().kda_version())


def kda_gate(A: torch.Tensor, z: torch.Tensor, g: Optional[torch.Tensor] = None,
             g_dtype: torch.dtype = torch.float32, g_min: float = -5.0, stream=None) -> torch.Tensor:
    """g = g_min * sigmoid(exp(A) * z); A [H, dk] fp32, z [..., H, dk] -> g like z (g_dtype)."""
    H, dk = A.shape
    if z.shape[-2:] != (H, dk):
        raise ValueError("z must end in [H, dk]")
    if g is None:
        g = torch.empty(z.shape, dtype=g_dtype, device=z.device)
    n_tokens = z.numel() // (H * dk)
    _check("kda_gate", load_library().kda_gate(_ptr(A), _ptr(z), _dt(z), _ptr(g), _dt(g),
                                               n_tokens, H, dk, float(g_min), _stream(stream)))
    return g


def kda_chunk_fwd_workspace_size(n_seqs: int, total_tokens: int, H: int, dk: int, dv: int,
                                 chunk: int = 64, in_dtype: torch.dtype = torch.bfloat16) -> int:
    return int(load_library().kda_chunk_fwd_workspace_size(n_seqs, total_tokens, H, dk, dv,
                                                            chunk, _DT[in_dtype]))


def kda_chunk_fwd(q, k, v, beta, g, initial_state=None, final_state=None, cu_seqlens=None,
                  o=None, o_dtype=None, scale: float = 1.0, output_final_state: bool = True,
                  workspace=None, stream=None):
    """Chunked prefill.  q, k, g [B, T, H, dk]; v [B, T, H, dv]; beta [B, T, H];
    initial_state [N, H, dk, dv] fp32 or None; cu_seqlens device int32 [N+1] or None (B == 1).
    Returns (o, final_state); final_state is allocated when output_final_state and not given."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    N, o, final_state, workspace, ws_bytes = _chunk_outputs(
        q, v, cu_seqlens, o, o_dtype, final_state, output_final_state, workspace)
    _check("kda_chunk_fwd", load_library().kda_chunk_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _dt(q), _ptr(g), _dt(g), _ptr(initial_state),
        _ptr(final_state), _ptr(cu_seqlens), _ptr(o), _dt(o), B, T, N, H, dk, dv, 64,
        float(scale), _ptr(workspace), ws_bytes, _stream(stream)))
    return o, final_state


def _chunk_outputs(q, v, cu_seqlens, o, o_dtype, final_state, output_final_state, workspace):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=o_dtype or q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    need = kda_chunk_fwd_workspace_size(N, B * T, H, dk, dv, in_dtype=q.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return N, o, final_state, workspace, ws_bytes


def kda_chunk_fwd_gated(q, k, v, beta, A, z, g_min: float = -5.0, initial_state=None,
                        final_state=None, cu_seqlens=None, o=None, o_dtype=None,
                        scale: float = 1.0, output_final_state: bool = True, workspace=None,
                        stream=None):
    """Chunked prefill with the gate fused: A [H, dk] fp32 and z [B, T, H, dk] replace g.
    Same outputs as kda_gate followed by kda_chunk_fwd (fp32 g)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    N, o, final_state, workspace, ws_bytes = _chunk_outputs(
        q, v, cu_seqlens, o, o_dtype, final_state, output_final_state, workspace)
    _check("kda_chunk_fwd_gated", load_library().kda_chunk_fwd_gated(
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _dt(q), _ptr(A), _ptr(z), _dt(z), float(g_min),
        _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens), _ptr(o), _dt(o), B, T, N, H,
        dk, dv, 64, float(scale), _ptr(workspace), ws_bytes, _stream(stream)))
    return o, final_state


def checkpoint_layout(every: int, T: int, B: int = 1, seqlens=None):
    """Host-side slot layout of kda_chunk_fwd_checkpointed: ([(first slot, count) per sequence],
    slots needed).  seqlens (host ints) describe a packed batch of total length T, else B
    sequences of T tokens."""
    if seqlens is None:
        per = T // every
        return [(n * per, per) for n in range(B)], B * per
    out, start = [], 0
    for n, length in enumerate(seqlens):
        out.append((start // every + n, int(length) // every))
        start += int(length)
    return out, T // every + len(seqlens)


def kda_chunk_fwd_checkpointed(q, k, v, beta, every: int, g=None, A=None, z=None,
                               g_min: float = -5.0, initial_state=None, final_state=None,
                               cu_seqlens=None, o=None, o_dtype=None, scale: float = 1.0,
                               output_final_state: bool = True, checkpoints=None, workspace=None,
                               stream=None):
    """Chunked prefill that also stores the state after every `every` tokens (a multiple of
    64) of each sequence.  Give g (as kda_chunk_fwd) or A and z (as kda_chunk_fwd_gated).
    Returns (o, final_state, checkpoints [slots, H, dk, dv] fp32); slot layout as
    checkpoint_layout; a new checkpoints buffer starts zeroed."""
    if (g is None) == (A is None or z is None):
        raise ValueError("give either g, or A and z")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    N, o, final_state, workspace, ws_bytes = _chunk_outputs(
        q, v, cu_seqlens, o, o_dtype, final_state, output_final_state, workspace)
    need = (B * (T // every)) if cu_seqlens is None else (T // every + N)
    if checkpoints is None:
        checkpoints = torch.zeros((need, H, dk, dv), dtype=torch.float32, device=q.device)
    gz = g if g is not None else z
    _check("kda_chunk_fwd_checkpointed", load_library().kda_chunk_fwd_checkpointed(
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _dt(q), _ptr(A), _ptr(gz), _dt(gz), float(g_min),
        _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens), _ptr(o), _dt(o), B, T, N, H,
        dk, dv, 64, float(scale), _ptr(checkpoints), int(every), checkpoints.shape[0],
        _ptr(workspace), ws_bytes, _stream(stream)))
    return o, final_state, checkpoints


def kda_decode_step(q, k, v, beta, g, state, o=None, o_dtype=None, scale: float = 1.0,
                    stream=None):
    """One token per sequence: q, k, g [N, H, dk]; v [N, H, dv]; beta [N, H]; state
    [N, H, dk, dv] fp32 updated in place.  Returns o [N, H, dv]."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((N, H, dv), dtype=o_dtype or q.dtype, device=q.device)
    _check("kda_decode_step", load_library().kda_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _dt(q), _ptr(g), _dt(g), _ptr(state), _ptr(o),
        _dt(o), N, H, dk, dv, float(scale), _stream(stream)))
    return o


def kda_decode_verify(q, k, v, beta, g, state, o=None, o_dtype=None, scale: float = 1.0,
                      stream=None):
    """K draft tokens per sequence from a read-only state: q, k, g [N, K, H, dk]; v [N, K, H, dv];
    beta [N, K, H]; state [N, H, dk, dv] fp32 (not modified).  Returns o [N, K, H, dv]."""
    N, Kd, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((N, Kd, H, dv), dtype=o_dtype or q.dtype, device=q.device)
    _check("kda_decode_verify", load_library().kda_decode_verify(
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _dt(q), _ptr(g), _dt(g), _ptr(state), _ptr(o),
        _dt(o), N, Kd, H, dk, dv, float(scale), _stream(stream)))
    return o


def kda_decode_commit(q, k, v, beta, g, state, accepted, stream=None):
    """Advance each state in place by its first accepted[n] draft tokens (device int32 [N]);
    inputs as kda_decode_verify.  Returns state."""
    N, Kd, H, dk = q.shape
    dv = v.shape[-1]
    if accepted.dtype != torch.int32:
        raise TypeError("accepted must be int32")
    _check("kda_decode_commit", load_library().kda_decode_commit(
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _dt(q), _ptr(g), _dt(g), _ptr(state),
        _ptr(accepted), N, Kd, H, dk, dv, _stream(stream)))
    return state
