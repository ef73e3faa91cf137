#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet core on one MI355X.

A step is one gdn_chunk_fwd call (gate preparation fused with the chunk-local
WY auxiliaries, then the inter-chunk state scan with output) over the Qwen3.5-shaped prefill: B=1,
T=4096, 16 key / 64 value heads, d_k = d_v = 128, bf16 q/k/v, fp32 gates and
state, chunk 64, zero initial state, synthetic seeded inputs already resident
in HBM.  The timed region rotates over several full copies of the inputs,
outputs and workspace so that no call finds its working set in the 256 MB
Infinity Cache left behind by the previous one.

Also measured (in the same JSON line): the decode step (B=256 sequences, same
heads, 1 GiB fp32 state updated in place, 64 consecutive steps) as HBM GB/s,
per-kernel durations from HIP events recorded between the kernels on the
launch stream, the roofline position of the dominant kernels, and the float64
CPU oracle timed on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s at T=4096 (16k/64v heads, d=128) + decode-step HBM GB/s"
PEAK_MFMA_F16_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix peak
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E

# Algorithmic work per (token, value head) at d_k = d_v = 128, chunk C = 64, G = 4
# value heads per key head (flop = 2 x multiply-accumulate):
#   whole prefill:  3 dk dv + C (dk/G + (dk+dv)/2 + dv/2)  MAC  = 63,488 MAC
#   state scan:     3 dk dv + C dv/2 (A_qk Delta) + C dv/2 (A R)  = 57,344 MAC
def prefill_flop_per_token_head(dk, dv, C, G):
    return 2 * (3 * dk * dv + C * (dk // G + (dk + dv) // 2 + dv // 2))


def scan_flop_per_token_head(dk, dv, C):
    return 2 * (3 * dk * dv + C * dv // 2 + C * dv // 2)


def prefill_bytes(B, T, Hk, Hv, Dk, Dv, es, init_state):
    qk = 2 * B * T * Hk * Dk * es
    vo = 2 * B * T * Hv * Dv * es
    ab = 2 * B * T * Hv * 4
    st = (2 if init_state else 1) * B * Hv * Dk * Dv * 4
    return qk + vo + ab + st + 2 * Hv * 4


def decode_bytes(B, Hk, Hv, Dk, Dv, es):
    return (2 * B * Hv * Dk * Dv * 4 + 2 * B * Hk * Dk * es + 2 * B * Hv * Dv * es
            + 2 * B * Hv * 4 + 2 * Hv * 4)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def bench_prefill(args, torch, gdn, synth):
    spec = synth.WORKLOADS["prefill_t4096"]
    log(f"[bench] prefill workload {spec}")
    inp = synth.make_inputs(spec)
    dims = gdn.make_dims(spec.B, spec.T, spec.Hk, spec.Hv, spec.Dk, spec.Dv, spec.torch_dtype)
    sets = []
    for _ in range(args.rotate):
        d = {k: (None if v is None else v.cuda().contiguous()) for k, v in inp.items()}
        d["out"] = torch.empty((spec.B, spec.T, spec.Hv, spec.Dv), dtype=spec.torch_dtype, device="cuda")
        d["ST"] = torch.empty((spec.B, spec.Hv, spec.Dk, spec.Dv), dtype=torch.float32, device="cuda")
        d["ws"] = gdn.alloc_workspace(dims)
        sets.append(d)

    def step(d, ev=None):
        gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["S0"],
                          out=d["out"], final_state=d["ST"], workspace=d["ws"], stage_events=ev)

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    evs = [gdn.StageEvents() for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(sets[i % len(sets)], evs[i].handles)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    per = [e.stage_ms() for e in evs]
    stage_ms = [sum(p[j] for p in per) / len(per) for j in range(gdn.GDN_CHUNK_FWD_STAGES)]
    for e in evs:
        e.close()
    ms = total_ms / args.steps
    toks = spec.B * spec.T
    G = spec.Hv // spec.Hk
    units = spec.B * spec.T * spec.Hv
    path_flop = prefill_flop_per_token_head(spec.Dk, spec.Dv, spec.chunk, G) * units
    scan_flop = scan_flop_per_token_head(spec.Dk, spec.Dv, spec.chunk) * units
    nbytes = prefill_bytes(spec.B, spec.T, spec.Hk, spec.Hv, spec.Dk, spec.Dv, 2, False)
    scan_ms = stage_ms[1]
    res = dict(
        spec=spec, ms=ms, tokens_per_s=toks / (ms * 1e-3), stage_ms=stage_ms,
        roofline=dict(
            kernel="state_scan_kernel", bound="mfma",
            achieved=round(scan_flop / (scan_ms * 1e-3) / 1e12, 2), peak=PEAK_MFMA_F16_TFLOPS,
            unit="TFLOP/s", frac=round(scan_flop / (scan_ms * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4),
            traffic=None, flop_per_launch=scan_flop, avg_launch_ms=round(scan_ms, 5)),
        path=dict(flop=path_flop, bytes=nbytes,
                  tflops=round(path_flop / (ms * 1e-3) / 1e12, 2),
                  mfma_frac=round(path_flop / (ms * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4),
                  hbm_gbs=round(nbytes / (ms * 1e-3) / 1e9, 1),
                  hbm_frac=round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)),
        inp=inp)
    log(f"[bench] prefill {ms * 1e3:.1f} us/step, stages (us) "
        + ", ".join(f"{n}={s * 1e3:.1f}" for n, s in zip(gdn.STAGE_NAMES, stage_ms)))
    del sets
    torch.cuda.empty_cache()
    return res


def bench_decode(args, torch, gdn, synth):
    spec = synth.WORKLOADS["decode_b256"]
    log(f"[bench] decode workload {spec}")
    inp = synth.make_inputs(spec)
    steps = spec.T
    per_step = []
    for t in range(steps):
        per_step.append({k: inp[k][:, t].contiguous().cuda() for k in ("q", "k", "v", "a", "b")})
    A_log, dt_bias = inp["A_log"].cuda(), inp["dt_bias"].cuda()
    state = inp["S0"].cuda()
    out = torch.empty((spec.B, spec.Hv, spec.Dv), dtype=spec.torch_dtype, device="cuda")

    def step(t):
        x = per_step[t % steps]
        gdn.gdn_recurrent_step(x["q"], x["k"], x["v"], x["a"], x["b"], A_log, dt_bias, state, out=out)

    for t in range(min(args.warmup, 8)):
        step(t)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for t in range(steps):
        step(t)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    nbytes = decode_bytes(spec.B, spec.Hk, spec.Hv, spec.Dk, spec.Dv, 2)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] decode {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s")
    res = dict(
        value=round(gbs, 1), unit="GB/s", ms_per_step=round(ms, 5), steps=steps,
        tokens_per_s=round(spec.B / (ms * 1e-3), 1),
        config=dict(workload="decode_b256", B=spec.B, Hk=spec.Hk, Hv=spec.Hv, Dk=spec.Dk,
                    Dv=spec.Dv, input_dtype="bf16", state_dtype="f32", consecutive_steps=steps),
        roofline=dict(kernel="decode_kernel", bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS,
                      unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 4), traffic=None,
                      bytes_per_launch=nbytes, avg_launch_ms=round(ms, 5)))
    del per_step, state
    torch.cuda.empty_cache()
    return res


def cpu_baseline(pre):
    """The float64 oracle on this host's cores, over the whole prefill workload."""
    import numpy as np
    import oracle
    spec, inp = pre["spec"], pre["inp"]
    x = {k: (None if v is None else oracle.f64(v)) for k, v in inp.items()}
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    out, ST = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["a"], x["b"], x["A_log"], x["dt_bias"], S0=x["S0"])
    dt = time.perf_counter() - t0
    assert np.isfinite(out).all()
    return dict(value=round(spec.B * spec.T / dt, 1), unit="tokens/s", cores=threads, kind="oracle",
                seconds=round(dt, 3),
                sample=f"whole prefill workload once (B={spec.B}, T={spec.T}, {spec.Hv} value heads, "
                       f"d={spec.Dk}), float64 token loop, OpenMP over (sequence, value head)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rotate", type=int, default=3, help="buffer sets rotated in the timed region")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (got --gpus {args.gpus}); the multi-GPU "
              f"sharding of the path is a design note, not implemented", file=sys.stderr)
        sys.exit(2)
    import torch
    import gated_deltanet_sequence_amd as gdn
    import synth
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    gdn.lib()

    pre = bench_prefill(args, torch, gdn, synth)
    dec = None if args.no_decode else bench_decode(args, torch, gdn, synth)
    cpu = None if args.no_cpu_baseline else cpu_baseline(pre)
    spec = pre["spec"]
    line = {
        "metric": METRIC,
        "value": round(pre["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "prefill_t4096", "B": spec.B, "T": spec.T, "Hk": spec.Hk, "Hv": spec.Hv,
                   "Dk": spec.Dk, "Dv": spec.Dv, "chunk": spec.chunk, "input_dtype": "bf16",
                   "state_dtype": "f32", "matrix_operands": "f16", "accumulate": "f32",
                   "rotated_buffer_sets": args.rotate},
        "roofline": pre["roofline"],
        "stages_us": {n: round(s * 1e3, 2) for n, s in zip(gdn.STAGE_NAMES, pre["stage_ms"])},
        "path": pre["path"],
        "decode": dec,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
