"""The C ABI on the CPU: the library loads, exports every symbol include/kda.h declares, and
rejects host-checkable argument errors before enqueuing any device work.  The pointers passed
here are never dereferenced: each call below fails validation first."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_60_amd import kda as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "kda.h")

FAKE = 1 << 40          # a host-side address-like integer; validation fails before any use
INV, UNS, WS = 1, 2, 3


def declared_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return K.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(K.EXPORTED), names
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert K.kda_status_string(0) == "KDA_OK"
    assert K.kda_status_string(1) == "KDA_ERR_INVALID_ARGUMENT"
    assert K.kda_status_string(2) == "KDA_ERR_UNSUPPORTED"
    assert K.kda_status_string(3) == "KDA_ERR_WORKSPACE"
    assert K.kda_status_string(4) == "KDA_ERR_HIP"
    assert K.kda_status_string(99) == "KDA_UNKNOWN_STATUS"
    assert K.kda_version() >= 200


def P(x):
    return ctypes.c_void_p(x) if x else None


def chunk(lib, q=FAKE, k=FAKE + 0x10000000, v=FAKE + 0x20000000, beta=FAKE + 0x30000000,
          in_dt=1, g=FAKE + 0x40000000, g_dt=0, h0=0, hT=0, cu=0, o=FAKE + 0x50000000, o_dt=1,
          B=1, T=128, N=1, H=2, dk=128, dv=128, chunk=64, scale=1.0, ws=FAKE + 0x80000000,
          ws_bytes=1 << 30):
    return lib.kda_chunk_fwd(P(q), P(k), P(v), P(beta), in_dt, P(g), g_dt, P(h0), P(hT), P(cu),
                             P(o), o_dt, B, T, N, H, dk, dv, chunk, scale, P(ws), ws_bytes, None)


def test_chunk_fwd_rejects(lib):
    # 4096 tokens and 2 heads run in segments, whose buffers live in the workspace
    ws_need = K.kda_chunk_fwd_workspace_size(1, 4096, 2, 128, 128)
    assert ws_need > 0
    assert chunk(lib, T=4096, ws=FAKE + 0x80000000, ws_bytes=ws_need - 1) == WS   # undersized
    assert chunk(lib, T=4096, ws=0, ws_bytes=0) == WS                             # missing
    f32_need = K.kda_chunk_fwd_workspace_size(1, 128, 2, 128, 128, in_dtype=__import__("torch").float32)
    assert chunk(lib, in_dt=0, ws=FAKE + 0x80000000, ws_bytes=f32_need - 1) == WS   # fp32 records
    assert chunk(lib, ws=FAKE + 0x20000000 + 64) == INV                   # workspace overlaps v
    assert chunk(lib, in_dt=7) == INV
    assert chunk(lib, g_dt=-1) == INV
    assert chunk(lib, o_dt=2) == INV
    assert chunk(lib, B=0) == INV
    assert chunk(lib, T=-1) == INV
    assert chunk(lib, H=0) == INV
    assert chunk(lib, N=2) == INV                       # fixed-length: N must equal B
    assert chunk(lib, B=2, N=2, cu=FAKE + 0x60000000) == INV   # packed batch needs B == 1
    assert chunk(lib, dk=96) == UNS
    assert chunk(lib, dv=256) == UNS
    assert chunk(lib, chunk=32) == UNS
    assert chunk(lib, q=0) == INV
    assert chunk(lib, o=0) == INV
    assert chunk(lib, scale=float("nan")) == INV
    assert chunk(lib, o=FAKE + 0x100) == INV            # o overlaps q
    assert chunk(lib, h0=FAKE + 0x70000000, hT=FAKE + 0x70000000 + 4096) == INV  # partial overlap
    assert chunk(lib, hT=FAKE + 0x10000010) == INV      # final state overlaps k


def gated(lib, q=FAKE, k=FAKE + 0x10000000, v=FAKE + 0x20000000, beta=FAKE + 0x30000000,
          in_dt=1, A=FAKE + 0x48000000, z=FAKE + 0x40000000, z_dt=1, gmin=-5.0, h0=0, hT=0, cu=0,
          o=FAKE + 0x50000000, o_dt=1, B=1, T=128, N=1, H=2, dk=128, dv=128, chunk=64, scale=1.0,
          ws=FAKE + 0x80000000, ws_bytes=1 << 30):
    return lib.kda_chunk_fwd_gated(P(q), P(k), P(v), P(beta), in_dt, P(A), P(z), z_dt, gmin,
                                   P(h0), P(hT), P(cu), P(o), o_dt, B, T, N, H, dk, dv, chunk,
                                   scale, P(ws), ws_bytes, None)


def test_chunk_fwd_gated_rejects(lib):
    assert gated(lib, gmin=-6.0) == UNS                 # outside [-5, 0)
    assert gated(lib, gmin=0.0) == UNS
    assert gated(lib, gmin=float("nan")) == UNS
    assert gated(lib, A=0) == INV                       # A required
    assert gated(lib, z=0) == INV                       # z required
    assert gated(lib, z_dt=4) == INV
    assert gated(lib, o=FAKE + 0x48000000 + 64) == INV  # o overlaps A
    assert gated(lib, ws=FAKE + 0x40000000 + 64) == INV  # workspace overlaps z
    assert gated(lib, dk=96) == UNS
    assert gated(lib, T=4096, ws_bytes=16) == WS


def two_kernel_workspace(n, tok, H, dk, dv, tpr, rec):
    """One fixed-size record per (head, slot) -- 32 tokens for 16-bit inputs (two 16-token
    sub-blocks), 16 for fp32 -- with slots <= tokens / tpr + sequences + 1 and the area rounded up
    to 256 bytes.  Launches that cut long sequences into 8192-token segments (when n * H * dv / 64
    <= 128 and sequences average at least 16384 tokens) add, per (segment slot, head), a start
    state, B (d_k x d_v) and M (d_k x d_k) in fp32, with segment slots <= tokens / 8192 +
    sequences + 1."""
    area = (tok // tpr + n + 1) * H * rec
    area = (area + 255) // 256 * 256
    if n * H * (dv // 64) <= 128 and tok >= 2 * 8192 * n:
        area += (tok // 8192 + n + 1) * H * dk * (2 * dv + dk) * 4
    return area


def test_workspace_size(lib):
    import torch
    # 16-bit records at d_k = 128: 6 fp16 [16][128] arrays, 3 + 3 fp16 16 x 16 tiles, 128 fp32 decays
    rec128 = 6 * 16 * 128 * 2 + 3072 + 512
    # 16-bit inputs at d_k = d_v = 128: no workspace when the (sequence, head) units fill 256
    # workgroups (the fused kernel runs whole sequences); otherwise the two-kernel layout (its
    # segment pass 1 is the fused kernel, which writes the same records)
    for n, tok, H in [(4, 4 * 4096, 16), (8, 1 << 20, 8), (1, 1 << 16, 32), (3, 17, 5), (1, 15, 1),
                      (16, 16 * 4096, 16), (1, 4096, 2), (2, 32768, 2), (64, 64 * 1024, 16), (256, 256, 1)]:
        want = 0 if n * H >= 256 else two_kernel_workspace(n, tok, H, 128, 128, 32, rec128)
        assert K.kda_chunk_fwd_workspace_size(n, tok, H, 128, 128) == want, (n, tok, H)
    # the bf16 prefill workload runs whole sequences; the long and packed ones in 8192-token segments
    assert K.kda_chunk_fwd_workspace_size(4, 4 * 4096, 16, 128, 128) == (512 + 5) * 16 * rec128
    assert K.kda_chunk_fwd_workspace_size(8, 1 << 20, 8, 128, 128) == \
        (32768 + 9) * 8 * rec128 + (128 + 9) * 8 * 128 * 384 * 4
    assert K.kda_chunk_fwd_workspace_size(1, 1 << 16, 32, 128, 128) == \
        (2048 + 2) * 32 * rec128 + (8 + 2) * 32 * 128 * 384 * 4
    # fp32 inputs, or 16-bit inputs with a head size of 64
    for dt, tpr, dk in ((torch.bfloat16, 32, 64), (torch.float32, 16, 128), (torch.float32, 16, 64)):
        rec = K.kda_chunk_fwd_workspace_size(1, 0, 1, dk, dk, in_dtype=dt) // 2
        assert rec > 0 and rec % 16 == 0
        for n, tok, H in [(4, 4 * 4096, 16), (8, 1 << 20, 8), (1, 1 << 16, 32), (3, 17, 5), (1, 15, 1)]:
            got = K.kda_chunk_fwd_workspace_size(n, tok, H, dk, dk, in_dtype=dt)
            assert got == two_kernel_workspace(n, tok, H, dk, dk, tpr, rec), (n, tok, H, got)
    # 16-bit records at d_k = 64: 6 fp16 [16][64] arrays, 3 + 3 fp16 16 x 16 tiles, 64 fp32 decays
    assert K.kda_chunk_fwd_workspace_size(1, 0, 1, 64, 64) == 2 * (6 * 16 * 64 * 2 + 3072 + 256)
    f32 = K.kda_chunk_fwd_workspace_size(4, 4 * 4096, 16, 128, 128, in_dtype=torch.float32)
    assert f32 > K.kda_chunk_fwd_workspace_size(4, 4 * 4096, 16, 128, 128)
    assert K.kda_chunk_fwd_workspace_size(1, 4096, 16, 96, 128) == 0
    assert K.kda_chunk_fwd_workspace_size(0, 4096, 16, 128, 128) == 0
    assert lib.kda_chunk_fwd_workspace_size(1, 64, 1, 128, 128, 64, 7) == 0


def test_gate_rejects(lib):
    g = lambda **kw: lib.kda_gate(P(kw.get("A", FAKE)), P(kw.get("z", FAKE + 0x1000000)),  # noqa: E731
                                  kw.get("zdt", 1), P(kw.get("g", FAKE + 0x2000000)),
                                  kw.get("gdt", 0), kw.get("n", 10), kw.get("H", 2),
                                  kw.get("dk", 8), kw.get("gmin", -5.0), None)
    assert g(zdt=3) == INV
    assert g(n=-1) == INV
    assert g(H=0) == INV
    assert g(gmin=-6.0) == UNS
    assert g(gmin=0.0) == UNS
    assert g(gmin=float("inf")) == UNS
    assert g(A=0) == INV
    assert g(g=FAKE + 0x1000000 + 8) == INV             # g overlaps z
    assert g(n=0, A=0, z=0, g=0) == 0                   # nothing to do


def test_decode_rejects(lib):
    d = lambda **kw: lib.kda_decode_step(  # noqa: E731
        P(kw.get("q", FAKE)), P(FAKE + 0x1000000), P(FAKE + 0x2000000), P(FAKE + 0x3000000),
        kw.get("idt", 1), P(FAKE + 0x4000000), kw.get("gdt", 1), P(kw.get("S", FAKE + 0x10000000)),
        P(kw.get("o", FAKE + 0x5000000)), kw.get("odt", 1), kw.get("N", 4), kw.get("H", 2),
        kw.get("dk", 128), kw.get("dv", 128), 1.0, None)
    assert d(idt=5) == INV
    assert d(N=-1) == INV
    assert d(dk=32) == UNS
    assert d(q=0) == INV
    assert d(o=FAKE + 0x10000000 + 64) == INV           # o overlaps the state
    assert d(N=0, q=0) == 0                              # nothing to do


def ckpt(lib, q=FAKE, k=FAKE + 0x10000000, v=FAKE + 0x20000000, beta=FAKE + 0x30000000,
         in_dt=1, A=0, gz=FAKE + 0x40000000, gz_dt=0, gmin=-5.0, h0=0, hT=0, cu=0,
         o=FAKE + 0x50000000, o_dt=1, B=1, T=128, N=1, H=2, dk=128, dv=128, chunk=64, scale=1.0,
         ck=FAKE + 0x90000000, every=64, slots=2, ws=FAKE + 0x80000000, ws_bytes=1 << 30):
    return lib.kda_chunk_fwd_checkpointed(P(q), P(k), P(v), P(beta), in_dt, P(A), P(gz), gz_dt,
                                          gmin, P(h0), P(hT), P(cu), P(o), o_dt, B, T, N, H, dk,
                                          dv, chunk, scale, P(ck), every, slots, P(ws), ws_bytes,
                                          None)


def test_chunk_fwd_checkpointed_rejects(lib):
    assert ckpt(lib, ck=0) == INV                        # buffer required
    assert ckpt(lib, every=0) == INV
    assert ckpt(lib, every=32) == INV                    # not a multiple of the 64-token chunk
    assert ckpt(lib, every=96) == INV
    assert ckpt(lib, slots=1) == INV                     # T=128, every=64: two slots needed
    assert ckpt(lib, B=2, N=2, T=256, slots=7) == INV    # 2 * 4 needed
    assert ckpt(lib, cu=FAKE + 0x60000000, N=3, slots=4) == INV   # packed: 128/64 + 3 needed
    assert ckpt(lib, ck=FAKE + 0x50000000 + 64) == INV   # checkpoints overlap o
    assert ckpt(lib, ck=FAKE + 0x80000000 + 64) == INV   # checkpoints overlap the workspace
    assert ckpt(lib, ck=FAKE + 0x40000000 - 64) == INV   # checkpoints run into g
    assert ckpt(lib, A=FAKE + 0x48000000, gmin=1.0) == UNS   # fused gate: g_min checked as usual
    assert ckpt(lib, dk=96) == UNS
    # otherwise kda_chunk_fwd's checks (4096 tokens in two or three sequences need segment buffers)
    assert ckpt(lib, T=4096, slots=64, ws_bytes=16) == WS
    assert ckpt(lib, T=4096, cu=FAKE + 0x60000000, N=3, slots=67, ws_bytes=16) == WS


def test_checkpoint_layout_helper():
    # fixed-length: sequence n starts at n * floor(T / every)
    bases, need = K.checkpoint_layout(64, 300, B=2)
    assert bases == [(0, 4), (4, 4)] and need == 8
    # packed: base(n) = floor(cu[n] / every) + n, count floor(len / every)
    lens = [0, 5, 64, 130, 200, 17]
    bases, need = K.checkpoint_layout(64, sum(lens), seqlens=lens)
    cu = [0, 0, 5, 69, 199, 399]
    assert bases == [(cu[n] // 64 + n, lens[n] // 64) for n in range(6)]
    assert need == sum(lens) // 64 + 6
    ends = [b + c for b, c in bases]
    assert all(ends[n] <= bases[n + 1][0] for n in range(5)) and ends[-1] <= need


def verify(lib, q=FAKE, k=FAKE + 0x10000000, v=FAKE + 0x20000000, beta=FAKE + 0x30000000,
           in_dt=1, g=FAKE + 0x40000000, g_dt=1, S=FAKE + 0x70000000, o=FAKE + 0x50000000,
           o_dt=1, N=4, Kd=3, H=2, dk=128, dv=128, scale=1.0):
    return lib.kda_decode_verify(P(q), P(k), P(v), P(beta), in_dt, P(g), g_dt, P(S), P(o), o_dt,
                                 N, Kd, H, dk, dv, scale, None)


def commit(lib, q=FAKE, k=FAKE + 0x10000000, v=FAKE + 0x20000000, beta=FAKE + 0x30000000,
           in_dt=1, g=FAKE + 0x40000000, g_dt=1, S=FAKE + 0x70000000, acc=FAKE + 0x60000000,
           N=4, Kd=3, H=2, dk=128, dv=128):
    return lib.kda_decode_commit(P(q), P(k), P(v), P(beta), in_dt, P(g), g_dt, P(S), P(acc), N, Kd,
                                 H, dk, dv, None)


def test_decode_verify_commit_reject(lib):
    assert verify(lib, Kd=0) == INV
    assert verify(lib, N=-1) == INV
    assert verify(lib, H=0) == INV
    assert verify(lib, in_dt=5) == INV
    assert verify(lib, o_dt=3) == INV
    assert verify(lib, scale=float("inf")) == INV
    assert verify(lib, dk=96) == UNS
    assert verify(lib, S=0) == INV
    assert verify(lib, o=0) == INV
    assert verify(lib, o=FAKE + 0x100) == INV              # o overlaps q
    assert verify(lib, o=FAKE + 0x70000000 + 64) == INV    # o overlaps the state
    assert verify(lib, N=0, q=0, o=0) == 0                 # nothing to do
    assert commit(lib, Kd=0) == INV
    assert commit(lib, acc=0) == INV
    assert commit(lib, dv=32) == UNS
    assert commit(lib, S=FAKE + 0x40000000 + 64) == INV    # state overlaps g
    assert commit(lib, acc=FAKE + 0x70000000 + 128) == INV  # accepted inside the state
    assert commit(lib, N=0, q=0, S=0) == 0
