"""Benchmark of the KDA forward pass on one MI355X.

One step = one pass of the prefill hot path over the largest single-GPU workload: 8 packed
sequences whose seeded log-uniform lengths in [1K, 256K] sum to 2^20 tokens, 8 heads,
d_k = d_v = 128, chunk 64, per-sequence fp32 initial states, cu_seqlens offsets.  The step is
kda_chunk_fwd_gated -- the forget gate, the intra-block work and the state pass (in segments
for these long sequences), from A and z (bf16) to o (bf16) and the final states (fp32).  Inputs
are synthetic (seeded generators, the workload's shapes and distributions) and resident in HBM
before the timed region starts.

The other workloads are timed in the same run, each with its own roofline: the bf16 prefill
workload (B=4, H=16, T=4096) under "prefill_bf16" (with the separate kda_gate + kda_chunk_fwd
pair under "unfused"), the same workload at B=16 (256 (sequence, head) units: the whole-sequence
fused kernel, no workspace) under "prefill_bf16_b16_fused", the long workload (1 x 65536 tokens,
32 heads) under "long_prefill", the decode workload (256 sequences x 32 heads, 64 in-place steps, plus speculative-decode verify and
commit) under "decode".

Prints ONE JSON line.  ``value`` is prefill tokens/s (tokens per step / wall-clock step time
over exactly K steps).  ``roofline`` describes the step's one operation, kda_chunk_fwd_gated
(its kernels launched back to back on one stream), with its algorithmic bytes per call divided
by its mean call time: HIP events on the launch stream around the timed region's K steps.
``cpu_baseline`` is the fp64 oracle (test infrastructure) timed on this host's cores on the
whole headline workload.
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
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-passes", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long", action="store_true", help="skip the long-sequence prefill leg")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--mode", choices=("all", "packed", "prefill", "fused", "long", "decode"),
                    default="all",
                    help="packed (the headline workload) / prefill / long / decode: run only that "
                         "workload and print no JSON line (for profiler passes)")
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


def mfma_executed(summary: str, call_ms: float):
    """Executed MFMA work per call from a committed counter summary (SQ_INSTS_VALU_MFMA_MOPS_*
    counters, 512 FLOP per unit), over the call time measured now; None when the summary is
    missing or was taken with other kernel sources."""
    path = os.path.join(PROFILES, summary)
    if not os.path.exists(path):
        return None
    m = re.search(r"<!-- mfma (\{.*?\}) -->", open(path).read())
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_sha256") != chunk_digest():
        return None
    flop = float(rec["flop_per_call"])
    return {"flop_per_call": flop, "tflops": round(flop / (call_ms * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(flop / (call_ms * 1e-3) / BF16_PEAK, 4),
            "by_type": rec.get("by_type"),
            "note": "counter-measured MFMA work (fp32 and fp16 MFMAs together) over the call time"}


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


def _median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def load_prefill(name, inputs, dev, keep_host=False, overrides=None):
    """Device copies of a prefill workload's inputs (and, when asked, the host tensors)."""
    cfg = inputs.config(name, **(overrides or {}))
    log("generating", cfg)
    d = inputs.make_prefill(cfg)
    w = {x: d[x].to(dev) for x in ("q", "k", "v", "beta", "z", "A", "S0")}
    w["cu"] = d["cu_seqlens"].to(dev) if d["cu_seqlens"] is not None else None
    w["lens"] = d["cu_seqlens"].diff().tolist() if d["cu_seqlens"] is not None else [d["T"]] * d["B"]
    w["cfg"], w["B"], w["T"], w["N"] = cfg, d["B"], d["T"], d["N"]
    return w, (d if keep_host else None)


def gated_call(K, w, stream, o, hT, ws):
    def call():
        K.kda_chunk_fwd_gated(w["q"], w["k"], w["v"], w["beta"], w["A"], w["z"],
                              initial_state=w["S0"], final_state=hT, cu_seqlens=w["cu"], o=o,
                              workspace=ws, stream=stream)
    return call


def prefill_buffers(K, w, dev):
    cfg = w["cfg"]
    B, T, H, dk, dv = w["B"], w["T"], cfg.H, cfg.dk, cfg.dv
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    hT = torch.empty_like(w["S0"])
    ws = torch.empty(K.kda_chunk_fwd_workspace_size(w["N"], B * T, H, dk, dv), dtype=torch.uint8,
                     device=dev)
    return o, hT, ws


def time_calls(call, stream, reps):
    """(mean, median) ms per call, HIP events on the launch stream: the mean over `reps` calls
    back to back between two events, the median over another `reps` calls with an event between
    consecutive calls (whose own cost the mean leaves out)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    e1.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    evs[0].record(stream)
    for i in range(reps):
        call()
        evs[i + 1].record(stream)
    evs[-1].synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(reps)]
    return e0.elapsed_time(e1) / reps, _median(per)


def prefill_alg_bytes(w):
    cfg = w["cfg"]
    th = w["B"] * w["T"] * cfg.H
    return th * FUSED_BYTES_PER_TH + cfg.H * cfg.dk * 4 + 2 * w["N"] * cfg.H * STATE_BYTES


def prefill_leg(name, K, inputs, dev, stream, reps, traffic_summary=None, label="", overrides=None):
    """A prefill workload other than the headline one: kda_chunk_fwd_gated timed with HIP events
    over `reps` calls after one untimed call; its own HBM roofline."""
    w, _ = load_prefill(name, inputs, dev, overrides=overrides)
    o, hT, ws = prefill_buffers(K, w, dev)
    call = gated_call(K, w, stream, o, hT, ws)
    call()
    torch.cuda.synchronize()
    mean, med = time_calls(call, stream, reps)
    alg = prefill_alg_bytes(w)
    cfg = w["cfg"]
    tokens = w["B"] * w["T"]
    th = tokens * cfg.H
    out = {"config": label,
           "ms_per_call": round(mean, 4), "ms_per_call_median": round(med, 4),
           "tokens_per_s": round(tokens / (mean * 1e-3), 1),
           "roofline": {"bound": "hbm", "achieved": round(alg / (mean * 1e-3) / 1e9, 1),
                        "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                        "frac": round(alg / (mean * 1e-3) / HBM_PEAK, 4),
                        "traffic": measured_traffic(traffic_summary, chunk_digest())
                        if traffic_summary else None,
                        "bytes_per_launch": alg},
           "mfma": {"canonical_tflops": round(th * PREFILL_FLOP_PER_TH / (mean * 1e-3) / 1e12, 2),
                    "frac_bf16_peak": round(th * PREFILL_FLOP_PER_TH / (mean * 1e-3) / BF16_PEAK, 4)}}
    return out, (w, o, hT, ws)


def chunk_digest():
    """The prefill kernels' sources: both prefill paths, their shared helpers and the gate."""
    return source_digest("kda_chunk.hip", "kda_fused.hip", "kda_chunk_util.hpp", "kda_common.hpp",
                         "kda_internal.hpp")


def cpu_baseline(args, d, lens):
    """The fp64 oracle (gate + token loop) on the whole headline workload on this host's cores,
    plus one thread on two (sequence, head) units of the bf16 prefill workload."""
    import oracle
    from gated_delta_rule_60_amd import inputs
    log("oracle baseline on host cores (whole headline workload)")
    t1 = time.perf_counter()
    g64 = oracle.gate(d["A"], d["z"])
    _, _, used = oracle.forward(d["q"], d["k"], d["v"], d["beta"], g64, S0=d["S0"],
                                cu_seqlens=d["cu_seqlens"].numpy(), nthreads=args.cpu_threads,
                                want_o=True)
    cpu_s = time.perf_counter() - t1
    del g64
    tokens = int(sum(lens))
    # one thread, one unit at a time: the per-token rate that bounds the longest sequence
    c1 = inputs.config("prefill_bf16")
    s = inputs.make_prefill(inputs.config("prefill_bf16", B=1, H=2))
    g1 = oracle.gate(s["A"], s["z"])
    t2 = time.perf_counter()
    oracle.forward(s["q"], s["k"], s["v"], s["beta"], g1, S0=s["S0"], nthreads=1)
    one_s = time.perf_counter() - t2
    per_th = one_s / (c1.T * 2)                  # seconds per token-head on one thread
    return {"value": round(tokens / cpu_s, 1), "unit": "tokens/s", "cores": int(used),
            "nproc": os.cpu_count(), "kind": "oracle",
            "sample": f"the whole headline workload ({tokens} tokens x 8 heads: gate + fp64 token "
                      f"loop, OpenMP over the 64 (sequence, head) units), {cpu_s:.1f} s",
            "seconds": round(cpu_s, 2),
            "single_thread": {"tokens_per_s_per_head": round(1.0 / per_th, 1),
                              "sample": "one thread, 2 units of 4096 tokens of the bf16 "
                                        f"prefill workload, {one_s:.2f} s"},
            "critical_path_s": round(max(lens) * per_th, 2),
            "critical_path_note": "the longest sequence's one unit at the single-thread rate: "
                                  "no thread count makes the oracle faster than this"}


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
    stream = torch.cuda.current_stream()

    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.mode == "decode":
        r = run_decode(args, dev, inputs, K, stream)
        log(f"decode: {r['ms_per_step']:.4f} ms/step; spec decode {r['spec_decode']}")
        return
    if args.mode in ("prefill", "fused", "long"):
        name = "prefill_long" if args.mode == "long" else "prefill_bf16"
        r, _ = prefill_leg(name, K, inputs, dev, stream, args.steps,
                           overrides={"B": 16} if args.mode == "fused" else None)
        log(f"{args.mode} ({name}): {r['ms_per_call']:.4f} ms/call "
            f"(median {r['ms_per_call_median']:.4f})")
        return

    # ------------------------------------------------------------------ headline: packed workload
    w, host = load_prefill("prefill_varlen", inputs, dev,
                           keep_host=(args.mode == "all" and not args.no_cpu_baseline))
    cfg = w["cfg"]
    o, hT, ws = prefill_buffers(K, w, dev)
    step = gated_call(K, w, stream, o, hT, ws)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # exactly K steps: wall clock, and HIP events on the launch stream around the same region
    e_beg, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e_beg.record(stream)
    for _ in range(args.steps):
        step()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    call_ms = e_beg.elapsed_time(e_end) / args.steps
    # per-call spread: the same K calls again with an event between consecutive calls
    _, call_med = time_calls(step, stream, max(args.steps, 20))
    if args.mode == "packed":
        log(f"packed prefill: {ms_per_step:.4f} ms/step, events {call_ms:.4f} ms/call "
            f"(median {call_med:.4f})")
        return

    lens = w["lens"]
    T, H, dk = w["T"], cfg.H, cfg.dk
    tokens = T
    th = tokens * H
    alg = prefill_alg_bytes(w)
    achieved = alg / (call_ms * 1e-3)
    flop = th * PREFILL_FLOP_PER_TH
    value = tokens / (ms_per_step * 1e-3)
    del o, hT, ws, w, step
    torch.cuda.empty_cache()

    # ------------------------------------------------------------------ other workloads
    leg1, (w1, o1, h1, ws1) = prefill_leg(
        "prefill_bf16", K, inputs, dev, stream, max(args.steps, 20),
        traffic_summary="chunk_fwd_gated_prefill_bf16_B4_H16_T4096.md",
        label="B=4 H=16 T=4096 d_k=d_v=128, bf16, random initial states, gate fused")
    g1 = torch.empty(w1["z"].shape, dtype=torch.float32, device=dev)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    K.kda_gate(w1["A"], w1["z"], g=g1, stream=stream)
    torch.cuda.synchronize()
    reps = max(args.steps, 20)
    evs[0].record(stream)
    for _ in range(reps):
        K.kda_gate(w1["A"], w1["z"], g=g1, stream=stream)
    evs[1].record(stream)
    for _ in range(reps):
        K.kda_chunk_fwd(w1["q"], w1["k"], w1["v"], w1["beta"], g1, initial_state=w1["S0"],
                        final_state=h1, o=o1, workspace=ws1, stream=stream)
    evs[2].record(stream)
    evs[2].synchronize()
    gate_ms, chunk_ms = evs[0].elapsed_time(evs[1]) / reps, evs[1].elapsed_time(evs[2]) / reps
    th1 = w1["B"] * w1["T"] * w1["cfg"].H
    chunk_bytes = th1 * PREFILL_BYTES_PER_TH + 2 * w1["N"] * w1["cfg"].H * STATE_BYTES
    leg1["unfused"] = {"kda_gate_ms": round(gate_ms, 4), "kda_chunk_fwd_ms": round(chunk_ms, 4),
                       "kda_chunk_fwd_bytes": chunk_bytes,
                       "kda_chunk_fwd_frac_hbm": round(chunk_bytes / (chunk_ms * 1e-3) / HBM_PEAK, 4),
                       "tokens_per_s": round(w1["B"] * w1["T"] / ((gate_ms + chunk_ms) * 1e-3), 1)}
    del w1, o1, h1, ws1, g1
    torch.cuda.empty_cache()
    # 256 (sequence, head) units: the whole-sequence fused kernel (no workspace round trip)
    leg16, bufs = prefill_leg("prefill_bf16", K, inputs, dev, stream, max(args.steps, 20),
                              traffic_summary="chunk_fwd_gated_fused_B16_H16_T4096.md",
                              label="B=16 H=16 T=4096 d_k=d_v=128, bf16, random initial states, "
                                    "gate fused: the whole-sequence fused kernel",
                              overrides={"B": 16})
    del bufs
    torch.cuda.empty_cache()
    long_ = None
    if not args.no_long:
        long_, bufs = prefill_leg("prefill_long", K, inputs, dev, stream, max(args.steps, 20),
                                  traffic_summary="chunk_fwd_gated_long_B1_H32_T65536.md",
                                  label="1 x 65536 tokens, 32 heads, d_k=d_v=128, bf16, "
                                        "z ~ N(0, 2^2), gate fused")
        del bufs
        torch.cuda.empty_cache()
    dec = run_decode(args, dev, inputs, K, stream)
    copy_bps = copy_ceiling(dev, stream)
    dec["roofline"]["frac_of_copy"] = round(dec["roofline"]["achieved"] * 1e9 / copy_bps, 4)

    cpu = None if args.no_cpu_baseline else cpu_baseline(args, host, lens)

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
        "config": {"workload": "KDA variable-length packed prefill, bf16 inputs / fp32 state: "
                               f"{len(lens)} sequences (lengths {', '.join(str(x) for x in lens)}), "
                               f"{tokens} tokens, H={H}, d_k=d_v={dk}, chunk=64, per-sequence "
                               "initial states, cu_seqlens, gate fused (A, z in)",
                   "global_batch": len(lens), "seq_len": max(lens), "total_tokens": tokens,
                   "heads": H, "head_dim": dk, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved / 1e9, 1),
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK, 4),
                     "traffic": measured_traffic("chunk_fwd_gated_varlen_8seq_1M_H8.md",
                                                 chunk_digest()),
                     "kernel": "kda_chunk_fwd_gated (the call's kernels back to back)",
                     "kernel_ms": round(call_ms, 4), "kernel_ms_median": round(call_med, 4),
                     "bytes_per_launch": alg},
        "mfma": {"canonical_tflops": round(flop / (call_ms * 1e-3) / 1e12, 2),
                 "frac_bf16_peak": round(flop / (call_ms * 1e-3) / BF16_PEAK, 4),
                 "executed": mfma_executed("chunk_fwd_gated_varlen_8seq_1M_H8.md", call_ms)},
        "prefill_bf16": leg1,
        "prefill_bf16_b16_fused": leg16,
        "long_prefill": long_,
        "decode": dec,
        "copy_ceiling_gbs": round(copy_bps / 1e9, 1),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
