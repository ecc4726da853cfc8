"""Benchmark of the KDA forward pass on one MI355X.

One step = one pass of the prefill hot path over the bf16 prefill workload (B=4, H=16, T=4096,
d_k=d_v=128, chunk 64, random fp32 initial state): kda_chunk_fwd_gated, i.e. the forget gate,
the intra-block work and the state pass, from A and z (bf16) to o (bf16) and the final state
(fp32).  The same step through the separate kda_gate + kda_chunk_fwd entry points is timed too
and reported under "unfused".  Inputs are synthetic (seeded generators, the workload's shapes
and distributions) and resident in HBM before the timed region starts.  The decode workload
(256 sequences x 32 heads, 64 in-place steps, plus speculative-decode verify and commit) is
timed in the same run and reported under "decode", the long workload (1 x 65536 tokens, 32
heads, run in 8192-token segments) under "long_prefill", and the packed workload (8 sequences of
seeded log-uniform lengths summing to 2^20 tokens, 8 heads, cu_seqlens) under "packed_prefill".

Prints ONE JSON line.  ``value`` is prefill tokens/s (B*T tokens per step / step time).
``roofline`` describes the step's one operation, kda_chunk_fwd_gated (its two kernels: the
intra-block kernel with the gate fused, and the state-passing kernel, launched back to back on
one stream), with its algorithmic bytes per call divided by its mean call time: HIP events on
the launch stream around the timed region's K steps.
``cpu_baseline`` is the fp64 oracle (test infrastructure) timed on this host's cores on the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import torch

HBM_PEAK = 8.0e12           # B/s, MI355X HBM3E
BF16_PEAK = 2516.6e12       # FLOP/s dense
# Algorithmic work per (token, head) at d_k = d_v = 128, chunk 64 (what the method must move and
# compute, not what the kernels execute):
#   bytes, gate fused: q, k, v, z bf16 (4*256) + beta bf16 (2) + o bf16 (256) = 1282
#   bytes, g given   : q, k, v bf16 (3*256) + g fp32 (512) + beta bf16 (2) + o bf16 (256) = 1538
#   FLOP : 6 dk dv + C (3 dk + 2 dv) + C^2 / 3 = 140,629
FUSED_BYTES_PER_TH = 1282
PREFILL_BYTES_PER_TH = 1538
PREFILL_FLOP_PER_TH = 6 * 128 * 128 + 64 * (3 * 128 + 2 * 128) + 64 * 64 / 3
STATE_BYTES = 128 * 128 * 4
# Decode per (sequence, head, step): state read + write (2 * 64 KiB) + q, k, v, g bf16 + beta + o
DECODE_BYTES_PER_UNIT = 2 * STATE_BYTES + 4 * 128 * 2 + 2 + 128 * 2


ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "gated_delta_rule_60_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--decode-passes", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long", action="store_true", help="skip the long-sequence prefill leg")
    ap.add_argument("--no-packed", action="store_true", help="skip the packed-batch prefill leg")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--mode", choices=("all", "prefill", "decode", "packed"), default="all",
                    help="prefill / decode: run only that workload and print no JSON line "
                         "(for profiler counter passes)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first copy this many MiB device-to-device (a plain copy kernel of known "
                         "size, the calibration for HBM byte counters)")
    return ap.parse_args()


def source_digest(*names):
    """sha256 over the kernel sources a counter measurement was taken with."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(summary: str, digest: str):
    """HBM bytes per launch from a committed counter summary (FETCH_SIZE + WRITE_SIZE scaled by a
    copy kernel of known size), or None when the summary is missing or was taken with other
    kernel sources than the ones built now."""
    path = os.path.join(PROFILES, summary)
    if not os.path.exists(path):
        return None
    m = re.search(r"<!-- traffic (\{.*?\}) -->", open(path).read())
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_sha256") != digest:
        return None
    return int(rec["hbm_bytes_per_launch"])


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def copy_ceiling(dev, stream, mib=1024, reps=10):
    """Device-to-device copy of `mib` MiB (torch copy_), the practical HBM ceiling: bytes read
    plus bytes written per second, best of `reps` timed with HIP events on the stream."""
    src = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del src, dst
    return 2 * (mib << 20) / (best * 1e-3)


def run_decode(args, dev, inputs, K, stream):
    """The decode workload: 64 in-place steps over 256 sequences x 32 heads, timed with HIP events
    on the launch stream over args.decode_passes passes."""
    dcfg = inputs.config("decode")
    log("generating", dcfg)
    dd = inputs.make_decode(dcfg)
    N, steps = dcfg.B, dcfg.decode_steps
    dq, dk_, dv_, db, dz = (dd[x].to(dev) for x in ("q", "k", "v", "beta", "z"))
    dA = dd["A"].to(dev)
    dg = K.kda_gate(dA, dz, g_dtype=torch.bfloat16)     # inputs prepared before timing
    Sd = dd["S0"].to(dev)
    od = torch.empty((N, dcfg.H, dcfg.dv), dtype=torch.bfloat16, device=dev)

    def decode_pass():
        for t in range(steps):
            K.kda_decode_step(dq[t], dk_[t], dv_[t], db[t], dg[t], Sd, o=od, stream=stream)

    decode_pass()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.decode_passes):
        decode_pass()
    e1.record(stream)
    e1.synchronize()
    dec_ms_step = e0.elapsed_time(e1) / (args.decode_passes * steps)
    dec_units = N * dcfg.H
    dec_gbs = dec_units * DECODE_BYTES_PER_UNIT / (dec_ms_step * 1e-3)

    # speculative decoding on the same state: verify a 4-token draft (state read once, every
    # token's output written), then commit 2 accepted tokens (state read and written once)
    n_draft, n_acc = 4, 2
    draft = [t[:n_draft].transpose(0, 1).contiguous() for t in (dq, dk_, dv_, db, dg)]
    od4 = torch.empty((N, n_draft, dcfg.H, dcfg.dv), dtype=torch.bfloat16, device=dev)
    acc = torch.full((N,), n_acc, dtype=torch.int32, device=dev)
    K.kda_decode_verify(*draft, Sd, o=od4, stream=stream)
    K.kda_decode_commit(*draft, Sd, acc, stream=stream)
    torch.cuda.synchronize()
    reps = 20
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(stream)
    for _ in range(reps):
        K.kda_decode_verify(*draft, Sd, o=od4, stream=stream)
    ev[1].record(stream)
    for _ in range(reps):
        K.kda_decode_commit(*draft, Sd, acc, stream=stream)
    ev[2].record(stream)
    ev[2].synchronize()
    ver_ms = ev[0].elapsed_time(ev[1]) / reps
    com_ms = ev[1].elapsed_time(ev[2]) / reps
    units = N * dcfg.H
    state_b = dcfg.dk * dcfg.dv * 4
    tok_in_b = 3 * dcfg.dk * 2 + dcfg.dv * 2 + 2            # q, k, g, v, beta (bf16)
    ver_b = units * (state_b + n_draft * (tok_in_b + dcfg.dv * 2))
    com_b = units * (2 * state_b + n_acc * tok_in_b)
    spec = {"draft_tokens": n_draft, "accepted": n_acc,
            "verify_ms": round(ver_ms, 4), "commit_ms": round(com_ms, 4),
            "verify_gbs": round(ver_b / (ver_ms * 1e-3) / 1e9, 1),
            "commit_gbs": round(com_b / (com_ms * 1e-3) / 1e9, 1),
            "verify_frac_hbm": round(ver_b / (ver_ms * 1e-3) / HBM_PEAK, 4),
            "commit_frac_hbm": round(com_b / (com_ms * 1e-3) / HBM_PEAK, 4),
            "step_by_step_ms": round(n_draft * dec_ms_step, 4),
            "note": "verify + commit against 4 kda_decode_step calls on state copies"}

    return {"seq_steps_per_s": round(N / (dec_ms_step * 1e-3), 1),
            "ms_per_step": round(dec_ms_step, 4),
            "spec_decode": spec,
            "roofline": {"bound": "hbm", "achieved": round(dec_gbs / 1e9, 1),
                         "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                         "frac": round(dec_gbs / HBM_PEAK, 4),
                         "traffic": measured_traffic("decode_kernel_256x32_d128.md",
                                                     source_digest("kda_decode.hip", "kda_common.hpp")),
                         "kernel": "decode_kernel",
                         "bytes_per_launch": dec_units * DECODE_BYTES_PER_UNIT},
            "config": "256 sequences x 32 heads, d_k=d_v=128, fp32 state in place, "
                      "bf16 q/k/v/beta/g, 64 steps"}


def run_long(args, dev, inputs, K, stream):
    """The long workload: 1 sequence x 65536 tokens, 32 heads, z ~ N(0, 2^2).  With few
    (sequence, head) units the library cuts the sequence into 8192-token segments (pass 1, the
    scan of segment pairs, pass 2).  kda_chunk_fwd_gated, timed with HIP events over 5 calls."""
    cfg = inputs.config("prefill_long")
    log("generating", cfg)
    d = inputs.make_prefill(cfg)
    q, k, v, beta, z = (d[x].to(dev) for x in ("q", "k", "v", "beta", "z"))
    A, S0 = d["A"].to(dev), d["S0"].to(dev)
    del d
    B, T, H, dk, dv = cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dv
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    hT = torch.empty_like(S0)
    ws = torch.empty(K.kda_chunk_fwd_workspace_size(B, B * T, H, dk, dv), dtype=torch.uint8,
                     device=dev)

    def call():
        K.kda_chunk_fwd_gated(q, k, v, beta, A, z, initial_state=S0, final_state=hT, o=o,
                              workspace=ws, stream=stream)

    call()
    torch.cuda.synchronize()
    reps = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    alg = B * T * H * FUSED_BYTES_PER_TH + H * dk * 4 + 2 * B * H * dk * dv * 4
    return {"config": "1 x 65536 tokens, 32 heads, d_k=d_v=128, bf16, gate fused; "
                      "split into 8192-token segments",
            "ms_per_call": round(ms, 4),
            "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "algorithmic_gbs": round(alg / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(alg / (ms * 1e-3) / HBM_PEAK, 4)}


def run_packed(args, dev, inputs, K, stream, reps=5):
    """The packed workload: 8 sequences of seeded log-uniform lengths summing to 2^20 tokens, 8
    heads, per-sequence initial states, packed with cu_seqlens (every sequence runs in 8192-token
    segments).  kda_chunk_fwd_gated, timed with HIP events over `reps` calls."""
    cfg = inputs.config("prefill_varlen")
    log("generating", cfg)
    d = inputs.make_prefill(cfg)
    q, k, v, beta, z = (d[x].to(dev) for x in ("q", "k", "v", "beta", "z"))
    A, S0, cu = d["A"].to(dev), d["S0"].to(dev), d["cu_seqlens"].to(dev)
    lens = d["cu_seqlens"].diff().tolist()
    del d
    T, H, dk, dv = q.shape[1], cfg.H, cfg.dk, cfg.dv
    N = len(lens)
    o = torch.empty((1, T, H, dv), dtype=torch.bfloat16, device=dev)
    hT = torch.empty_like(S0)
    ws = torch.empty(K.kda_chunk_fwd_workspace_size(N, T, H, dk, dv), dtype=torch.uint8,
                     device=dev)

    def call():
        K.kda_chunk_fwd_gated(q, k, v, beta, A, z, initial_state=S0, final_state=hT,
                              cu_seqlens=cu, o=o, workspace=ws, stream=stream)

    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    alg = T * H * FUSED_BYTES_PER_TH + H * dk * 4 + 2 * N * H * dk * dv * 4
    return {"config": f"{N} packed sequences (lengths {', '.join(str(x) for x in lens)}), "
                      f"{T} tokens, {H} heads, d_k=d_v={dk}, bf16, gate fused",
            "ms_per_call": round(ms, 4),
            "tokens_per_s": round(T / (ms * 1e-3), 1),
            "algorithmic_gbs": round(alg / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(alg / (ms * 1e-3) / HBM_PEAK, 4)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1 "
              "(sequences and heads are independent: several GPUs would each run their own share)",
              file=sys.stderr)
        sys.exit(2)

    from gated_delta_rule_60_amd import inputs
    from gated_delta_rule_60_amd import kda as K

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K.load_library()

    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.mode == "decode":
        r = run_decode(args, dev, inputs, K, torch.cuda.current_stream())
        log(f"decode: {r['ms_per_step']:.4f} ms/step; spec decode {r['spec_decode']}")
        return
    if args.mode == "packed":
        r = run_packed(args, dev, inputs, K, torch.cuda.current_stream(), reps=args.steps)
        log(f"packed prefill: {r['ms_per_call']:.4f} ms/call, {r['tokens_per_s']:.0f} tokens/s")
        return

    # ------------------------------------------------------------------ prefill workload
    cfg = inputs.config("prefill_bf16")
    log("generating", cfg)
    d = inputs.make_prefill(cfg)
    B, T, H, dk, dv = cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dv
    q, k, v, beta, z = (d[x].to(dev) for x in ("q", "k", "v", "beta", "z"))
    A, S0 = d["A"].to(dev), d["S0"].to(dev)
    g = torch.empty(z.shape, dtype=torch.float32, device=dev)
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    hT = torch.empty_like(S0)
    ws = torch.empty(K.kda_chunk_fwd_workspace_size(B, B * T, H, dk, dv, in_dtype=q.dtype),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def fused_step():
        K.kda_chunk_fwd_gated(q, k, v, beta, A, z, initial_state=S0, final_state=hT, o=o,
                              workspace=ws, stream=stream)

    def unfused_step():
        K.kda_gate(A, z, g=g, stream=stream)
        K.kda_chunk_fwd(q, k, v, beta, g, initial_state=S0, final_state=hT, o=o, workspace=ws,
                        stream=stream)

    for _ in range(args.warmup):
        fused_step()
        unfused_step()
    torch.cuda.synchronize()
    # exactly K steps: wall clock, and HIP events on the launch stream around the same region
    e_beg, e_end = ev(), ev()
    t0 = time.perf_counter()
    e_beg.record(stream)
    for _ in range(args.steps):
        fused_step()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    fused_ms = [e_beg.elapsed_time(e_end) / args.steps]
    # the unfused pair for reference: K pairs back to back, events between the calls
    evs = [ev() for _ in range(2 * args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        K.kda_gate(A, z, g=g, stream=stream)
        evs[2 * i + 1].record(stream)
        K.kda_chunk_fwd(q, k, v, beta, g, initial_state=S0, final_state=hT, o=o, workspace=ws,
                        stream=stream)
        evs[2 * i + 2].record(stream)
    torch.cuda.synchronize()
    gate_ms = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(args.steps)]
    chunk_ms = [evs[2 * i + 1].elapsed_time(evs[2 * i + 2]) for i in range(args.steps)]
    fused_avg = sum(fused_ms) / len(fused_ms)
    chunk_avg = sum(chunk_ms) / len(chunk_ms)
    gate_avg = sum(gate_ms) / len(gate_ms)
    if args.mode == "prefill":
        log(f"prefill: {ms_per_step:.4f} ms/step, kda_chunk_fwd_gated {fused_avg:.4f} ms, "
            f"kda_gate {gate_avg:.4f} ms + kda_chunk_fwd {chunk_avg:.4f} ms")
        return

    tokens = B * T
    th = tokens * H
    state_io = 2 * B * H * STATE_BYTES
    fused_bytes = th * FUSED_BYTES_PER_TH + H * dk * 4 + state_io
    chunk_bytes = th * PREFILL_BYTES_PER_TH + state_io
    chunk_flop = th * PREFILL_FLOP_PER_TH
    achieved = fused_bytes / (fused_avg * 1e-3)
    value = tokens / (ms_per_step * 1e-3)

    dec = run_decode(args, dev, inputs, K, stream)
    long_ = None if args.no_long else run_long(args, dev, inputs, K, stream)
    packed = None if args.no_packed else run_packed(args, dev, inputs, K, stream)
    copy_bps = copy_ceiling(dev, stream)
    dec["roofline"]["frac_of_copy"] = round(dec["roofline"]["achieved"] * 1e9 / copy_bps, 4)

    # ------------------------------------------------------------------ CPU baseline (oracle)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("oracle baseline on host cores")
        t1 = time.perf_counter()
        g64 = oracle.gate(d["A"], d["z"])
        _, _, used = oracle.forward(d["q"], d["k"], d["v"], d["beta"], g64, S0=d["S0"],
                                    nthreads=args.cpu_threads, want_o=True)
        cpu_s = time.perf_counter() - t1
        cpu = {"value": round(tokens / cpu_s, 1), "unit": "tokens/s", "cores": int(used),
               "kind": "oracle",
               "sample": f"the whole prefill workload (gate + token loop, fp64), {cpu_s:.1f} s"}

    out = {
        "metric": "KDA prefill tokens/s (% bf16 MFMA peak) + decode state GB/s (% HBM peak)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "KDA chunked prefill, bf16 inputs / fp32 state, B=4 H=16 T=4096 "
                               "d_k=d_v=128 chunk=64, gate fused (A, z in)",
                   "global_batch": B, "seq_len": T, "heads": H, "head_dim": dk,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved / 1e9, 1),
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK, 4),
                     "traffic": measured_traffic(
                         "chunk_fwd_gated_prefill_bf16_B4_H16_T4096.md",
                         source_digest("kda_chunk.hip", "kda_common.hpp", "kda_internal.hpp")),
                     "kernel": "kda_chunk_fwd_gated = chunk_intra_tok_kernel (gate fused) + "
                               "chunk_state_kernel",
                     "kernel_ms": round(fused_avg, 4), "bytes_per_launch": fused_bytes,
                     "workspace_bytes": ws.numel()},
        "mfma": {"canonical_tflops": round(chunk_flop / (fused_avg * 1e-3) / 1e12, 2),
                 "frac_bf16_peak": round(chunk_flop / (fused_avg * 1e-3) / BF16_PEAK, 4)},
        "unfused": {"kda_gate_ms": round(gate_avg, 4), "kda_chunk_fwd_ms": round(chunk_avg, 4),
                    "kda_chunk_fwd_bytes": chunk_bytes,
                    "kda_chunk_fwd_frac_hbm": round(chunk_bytes / (chunk_avg * 1e-3) / HBM_PEAK, 4),
                    "tokens_per_s": round(tokens / ((gate_avg + chunk_avg) * 1e-3), 1)},
        "decode": dec,
        "long_prefill": long_,
        "packed_prefill": packed,
        "copy_ceiling_gbs": round(copy_bps / 1e9, 1),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
