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

HBM traffic of the dominant kernels comes from rocprofv3 counter runs
(FETCH_SIZE and WRITE_SIZE, one pass each) summarised under profiles/ together
with a hash of the kernel sources; it is reported only while the sources still
match that hash.

Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W]
  python bench.py --calibration-copy ...       (also run a 256 MiB device copy,
                                                the counter calibration kernel)
  python bench.py --summarize-stats DIR OUT CMD (rocprofv3 --stats CSVs -> profiles/OUT)
  python bench.py --summarize-pmc FETCH_DIR WRITE_DIR
                                               (two counter passes -> traffic summaries)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s at T=4096 (16k/64v heads, d=128) + decode-step HBM GB/s"
PEAK_MFMA_F16_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix peak
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
PEAK_MFMA_F32_TFLOPS = 157.3    # MI355X fp32 matrix peak, equal to the packed fp32 vector peak:
                                # 256 CUs x 4 SIMDs x 16 lanes x 2 (FMA) x 2 (packed) x 2.4 GHz

# Algorithmic work per (token, value head) at d_k = d_v = 128, chunk C = 64, G = 4
# value heads per key head (flop = 2 x multiply-accumulate):
#   whole prefill:  3 dk dv + C (dk/G + (dk+dv)/2 + dv/2)  MAC  = 63,488 MAC
#   state scan:     3 dk dv + C dv/2 (A_qk Delta) + C dv/2 (A R)  = 57,344 MAC
def prefill_flop_per_token_head(dk, dv, C, G):
    return 2 * (3 * dk * dv + C * (dk // G + (dk + dv) // 2 + dv // 2))


def scan_flop_per_token_head(dk, dv, C):
    return 2 * (3 * dk * dv + C * dv // 2 + C * dv // 2)


# Gated DeltaNet-2 (channel-wise decay): no sharing of the chunk-local products
# across value heads: 3 dk dv + C (dk + (dk+dv)/2 + dv/2) MAC per (token, value head)
# (= 139,264 flop at d = 128, C = 64).  Its minimum traffic: q, k, v, the three
# gate-logit tensors and the output once each, plus the state(s).
def gdn2_flop_per_token_head(dk, dv, C):
    return 2 * (3 * dk * dv + C * (dk + (dk + dv) // 2 + dv // 2))


# Algorithmic work of the Gated DeltaNet-2 backward per (token, value head) and launch
# (flop = 2 x multiply-accumulate; triangular products counted as triangles):
#   g2b_prep      M and A_qk over the channels, (C + 1)/2 pairs each; A = (I + M)^{-1}: C^2/6
#   g2b_fwd_scan  R = Z - Et S, S update (dk dv each); U = A R (C dv / 2)
#   g2b_bwd_scan  Kh dS, Qt^T dO, Et^T dR (dk dv each); A_qk^T dO, A^T dU (C dv / 2 each)
#   g2b_products  dEt, dQt, dKh (dk dv each); tril(dO U^T) (C dv / 2); dU R^T (C dv);
#                 A^T dA and X A^T (C^2 / 2 each)
#   g2b_local     the three pairwise decay sums over (C + 1)/2 partners per channel
def bwd2_flop_per_token_head(dk, dv, C):
    return {
        "g2b_prep": 2 * (C + 1) * dk + C * C // 3,
        "g2b_fwd_scan": 2 * (2 * dk * dv + C * dv // 2),
        "g2b_bwd_scan": 2 * (3 * dk * dv + C * dv),
        "g2b_products": 2 * (3 * dk * dv + 3 * C * dv // 2 + C * C),
        "g2b_local": 3 * (C + 1) * dk,
        "g2b_reduce": 0,
    }


def gdn2_bytes(B, T, Hk, Hv, Dk, Dv, es, init_state):
    return (2 * B * T * Hk * Dk * es + 2 * B * T * Hv * Dv * es + 2 * B * T * Hv * Dk * es
            + B * T * Hv * Dv * es + Hv * Dk * 4 + (2 if init_state else 1) * B * Hv * Dk * Dv * 4)


def prefill_bytes(B, T, Hk, Hv, Dk, Dv, es, init_state):
    qk = 2 * B * T * Hk * Dk * es
    vo = 2 * B * T * Hv * Dv * es
    ab = 2 * B * T * Hv * 4
    st = (2 if init_state else 1) * B * Hv * Dk * Dv * 4
    return qk + vo + ab + st + 2 * Hv * 4


def decode_bytes(B, Hk, Hv, Dk, Dv, es):
    return (2 * B * Hv * Dk * Dv * 4 + 2 * B * Hk * Dk * es + 2 * B * Hv * Dv * es
            + 2 * B * Hv * 4 + 2 * Hv * 4)


def decode_gdn2_bytes(B, Hk, Hv, Dk, Dv, es):
    return (2 * B * Hv * Dk * Dv * 4 + 2 * B * Hk * Dk * es + 3 * B * Hv * Dv * es
            + 2 * B * Hv * Dk * es + Hv * Dk * 4)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Counter-based HBM traffic (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE).
# ---------------------------------------------------------------------------
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "gated_deltanet_sequence_amd", "csrc")
COPY_MIB = 256                      # calibration copy: 256 MiB read + 256 MiB written
# kernel key -> (regex on the demangled kernel name, summary file, source file)
TRAFFIC_FILES = {
    # (names with float16 template arguments come out mangled: Lb0E / Lb1E is the bool)
    "scan_split_kernel": (r"scan_split_kernel(<[^>]*false>|I.*Lb0E)", "scan_split_kernel_prefill_t4096_traffic.md",
                          "state_scan.hip"),
    "chunk_local_kernel": (r"chunk_local_kernel", "chunk_local_kernel_prefill_t4096_traffic.md", "chunk_local.hip"),
    "decode_kernel": (r"decode_kernel<[^>]*false>", "decode_kernel_decode_b256_traffic.md", "decode.hip"),
    "decode_kernel_gdn2": (r"decode_kernel<[^>]*true>", "decode_kernel_gdn2_decode_b256_traffic.md", "decode.hip"),
    "scan_split_kernel_gdn2": (r"scan_split_kernel(<[^>]*true>|I.*Lb1E)", "scan_split_kernel_gdn2_t8192_traffic.md",
                               "state_scan.hip"),
    "chunk_local2_kernel": (r"chunk_local2_kernel", "chunk_local2_kernel_gdn2_t8192_traffic.md", "chunk_local2.hip"),
    "g2b_local": (r"g2b_local", "g2b_local_gdn2_bwd_t8192_traffic.md", "bwd2.hip"),
    "gated_rmsnorm_kernel": (r"gated_rmsnorm_kernel", "gated_rmsnorm_kernel_t4096_traffic.md", "epilogue.hip"),
    "causal_conv1d_kernel": (r"causal_conv1d_kernel", "causal_conv1d_kernel_t4096_traffic.md", "prologue.hip"),
}


def _source_closure(src):
    """The HIP source and the local headers it includes, transitively."""
    seen, todo = set(), [os.path.join(CSRC, src)]
    while todo:
        f = todo.pop()
        if f in seen or not os.path.exists(f):
            continue
        seen.add(f)
        for inc in re.findall(r'^#include\s+"([^"]+)"', open(f).read(), re.M):
            for d in (os.path.dirname(f), CSRC, os.path.join(ROOT, "include")):
                if os.path.exists(os.path.join(d, inc)):
                    todo.append(os.path.join(d, inc))
                    break
    return sorted(seen)


def kernel_sources_sha256(kernel):
    """Hash of the source file a kernel is built from and the headers it includes."""
    h = hashlib.sha256()
    for f in _source_closure(TRAFFIC_FILES[kernel][2]):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def stored_traffic(kernel):
    """Bytes per launch from the committed counter summary, or None if the
    summary is missing or the kernel's sources changed since it was taken."""
    path = os.path.join(PROFILES, TRAFFIC_FILES.get(kernel, ("", "-", ""))[1])
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"^source_sha256:\s*([0-9a-f]{64})", text, re.M)
    m_b = re.search(r"^traffic_bytes_per_launch:\s*([0-9]+)", text, re.M)
    if not (m_sha and m_b) or m_sha.group(1) != kernel_sources_sha256(kernel):
        return None
    return int(m_b.group(1))


def calibration_copy(torch):
    """A plain streaming kernel of known traffic (reads and writes COPY_MIB MiB:
    an elementwise multiply, which has a kernel of its own, unlike a device copy
    that shares the runtime's blit kernel with the input uploads), profiled
    beside the kernels so the counters can be scaled to bytes."""
    n = COPY_MIB * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def _read_counter_csv(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _per_dispatch(rows, counter, name_rx):
    """Mean over dispatches of kernels matching name_rx of the counter (summed over dimensions)."""
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter or not re.search(name_rx, r["Kernel_Name"]):
            continue
        per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return (sum(per.values()) / len(per), len(per)) if per else (None, 0)


def summarize_pmc(fetch_dir, write_dir):
    """Write profiles/<kernel>_..._traffic.md: FETCH_SIZE / WRITE_SIZE per
    dispatch of the dominant kernels, scaled by the calibration copy, with the
    source hash."""
    f_rows, w_rows = _read_counter_csv(fetch_dir), _read_counter_csv(write_dir)
    copy_rx = r"MulFunctor"
    cf, ncf = _per_dispatch(f_rows, "FETCH_SIZE", copy_rx)
    cw, ncw = _per_dispatch(w_rows, "WRITE_SIZE", copy_rx)
    kib = COPY_MIB * 1024
    f_scale, w_scale = kib / cf, kib / cw
    for kernel, (rx, fname, _src) in TRAFFIC_FILES.items():
        sha = kernel_sources_sha256(kernel)
        kf, nkf = _per_dispatch(f_rows, "FETCH_SIZE", rx)
        kw, nkw = _per_dispatch(w_rows, "WRITE_SIZE", rx)
        if kf is None or kw is None:
            continue
        fetch_b = kf * f_scale * 1024
        write_b = kw * w_scale * 1024
        lines = [
            f"# HBM traffic of {kernel} (rocprofv3 counters; kernel names matching `{rx}`)", "",
            "Two counter passes over the same bench command, one counter each:", "",
            "```",
            "cd /tmp && export TMPDIR=/tmp",
            f"timeout -s KILL 200 rocprofv3 --pmc FETCH_SIZE -d <dir_fetch> -o pmc --output-format csv -- python3 <repo>/bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-long --calibration-copy",
            f"timeout -s KILL 200 rocprofv3 --pmc WRITE_SIZE -d <dir_write> -o pmc --output-format csv -- python3 <repo>/bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-long --calibration-copy",
            "python3 bench.py --summarize-pmc <dir_fetch> <dir_write>",
            "```", "",
            "| quantity | value |", "|---|---|",
            f"| {kernel} FETCH_SIZE per dispatch (KiB, mean of {nkf}) | {kf:.0f} |",
            f"| {kernel} WRITE_SIZE per dispatch (KiB, mean of {nkw}) | {kw:.0f} |",
            f"| calibration: elementwise multiply, {COPY_MIB} MiB in + {COPY_MIB} MiB out, FETCH_SIZE per dispatch (KiB, mean of {ncf}) | {cf:.0f} |",
            f"| calibration: same kernel, WRITE_SIZE per dispatch (KiB, mean of {ncw}) | {cw:.0f} |",
            f"| scale factors (known KiB / counted KiB): fetch, write | {f_scale:.4f}, {w_scale:.4f} |",
            f"| {kernel} HBM read bytes per launch | {fetch_b:.0f} |",
            f"| {kernel} HBM write bytes per launch | {write_b:.0f} |", "",
            f"traffic_bytes_per_launch: {int(round(fetch_b + write_b))}",
            f"sources: {', '.join(os.path.basename(f) for f in _source_closure(_src))}",
            f"source_sha256: {sha}", ""]
        path = os.path.join(PROFILES, fname)
        open(path, "w").write("\n".join(lines))
        print(f"wrote {path}")


def summarize_stats(d, out_name, command):
    """profiles/<out_name>: per-kernel durations from rocprofv3 --kernel-trace --stats."""
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(files[0])))
    lines = [f"# Kernel durations (rocprofv3 --kernel-trace --stats)", "", "```", command, "```", "",
             "| kernel | calls | total ms | average us | min us | max us | % |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        short = re.sub(r"\(.*", "", name.replace("(anonymous namespace)::", ""))[:90]
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    path = os.path.join(PROFILES, out_name)
    open(path, "w").write("\n".join(lines) + "\n")
    print(f"wrote {path}")


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
    # the headline: exactly K steps and nothing else in the timed region
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(sets[i % len(sets)])
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    # per-kernel durations: a second pass of K steps with HIP events recorded
    # between the kernels on the launch stream (each event pair also brackets
    # a launch, and the events lengthen the step by ~10 us, so they stay out
    # of the headline)
    evs = [gdn.StageEvents() for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(sets[i % len(sets)], evs[i].handles)
    torch.cuda.synchronize()
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
    scan_kernel = "scan_split_kernel" if spec.dtype == "bf16" else "state_scan_kernel"
    res = dict(
        spec=spec, ms=ms, tokens_per_s=toks / (ms * 1e-3), stage_ms=stage_ms,
        roofline=dict(
            kernel=scan_kernel, bound="mfma",
            achieved=round(scan_flop / (scan_ms * 1e-3) / 1e12, 2), peak=PEAK_MFMA_F16_TFLOPS,
            unit="TFLOP/s", frac=round(scan_flop / (scan_ms * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4),
            traffic=stored_traffic(scan_kernel), flop_per_launch=scan_flop, avg_launch_ms=round(scan_ms, 5)),
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


def bench_prefill_long(args, torch, gdn, synth):
    """The long-context prefill (B=2, T=65536, 16/64 heads, d=128, bf16, initial state ~ N(0, 0.02)):
    the same call and protocol as the headline leg, on fewer steps (each call is ~1 ms)."""
    spec = synth.WORKLOADS["prefill_long"]
    log(f"[bench] long-context prefill workload {spec}")
    inp = synth.make_inputs(spec)
    dims = gdn.make_dims(spec.B, spec.T, spec.Hk, spec.Hv, spec.Dk, spec.Dv, spec.torch_dtype)
    sets = []
    for _ in range(args.rotate):
        d = {k: (None if v is None else v.cuda().contiguous()) for k, v in inp.items()}
        d["out"] = torch.empty((spec.B, spec.T, spec.Hv, spec.Dv), dtype=spec.torch_dtype, device="cuda")
        d["ST"] = torch.empty((spec.B, spec.Hv, spec.Dk, spec.Dv), dtype=torch.float32, device="cuda")
        d["ws"] = gdn.alloc_workspace(dims)
        sets.append(d)
    del inp
    steps, warmup = max(1, min(args.steps, 5)), max(1, min(args.warmup, 2))

    def step(d, ev=None):
        gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["S0"],
                          out=d["out"], final_state=d["ST"], workspace=d["ws"], stage_events=ev)

    for i in range(warmup):
        step(sets[i % len(sets)])
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        step(sets[i % len(sets)])
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    evs = [gdn.StageEvents() for _ in range(steps)]
    for i in range(steps):
        step(sets[i % len(sets)], evs[i].handles)
    torch.cuda.synchronize()
    stage_ms = [sum(e.stage_ms()[j] for e in evs) / steps for j in range(gdn.GDN_CHUNK_FWD_STAGES)]
    for e in evs:
        e.close()
    G = spec.Hv // spec.Hk
    units = spec.B * spec.T * spec.Hv
    path_flop = prefill_flop_per_token_head(spec.Dk, spec.Dv, spec.chunk, G) * units
    scan_flop = scan_flop_per_token_head(spec.Dk, spec.Dv, spec.chunk) * units
    nbytes = prefill_bytes(spec.B, spec.T, spec.Hk, spec.Hv, spec.Dk, spec.Dv, 2, True)
    scan_tf = scan_flop / (stage_ms[1] * 1e-3) / 1e12
    path_tf = path_flop / (ms * 1e-3) / 1e12
    log(f"[bench] long-context prefill {ms * 1e3:.1f} us/step, stages (us) "
        + ", ".join(f"{n}={t * 1e3:.1f}" for n, t in zip(gdn.STAGE_NAMES, stage_ms)))
    del sets
    torch.cuda.empty_cache()
    return dict(value=round(spec.B * spec.T / (ms * 1e-3), 1), unit="tokens/s", ms_per_step=round(ms, 5),
                steps=steps, warmup=warmup,
                config=dict(workload="prefill_long", B=spec.B, T=spec.T, Hk=spec.Hk, Hv=spec.Hv, Dk=spec.Dk,
                            Dv=spec.Dv, chunk=spec.chunk, input_dtype="bf16", state_dtype="f32",
                            initial_state=True, rotated_buffer_sets=args.rotate),
                stages_us={n: round(t * 1e3, 2) for n, t in zip(gdn.STAGE_NAMES, stage_ms)},
                roofline=dict(kernel="scan_split_kernel", bound="mfma", achieved=round(scan_tf, 2),
                              peak=PEAK_MFMA_F16_TFLOPS, unit="TFLOP/s", frac=round(scan_tf / PEAK_MFMA_F16_TFLOPS, 4),
                              flop_per_launch=scan_flop, avg_launch_ms=round(stage_ms[1], 5)),
                path=dict(flop=path_flop, bytes=nbytes, tflops=round(path_tf, 2),
                          mfma_frac=round(path_tf / PEAK_MFMA_F16_TFLOPS, 4),
                          hbm_gbs=round(nbytes / (ms * 1e-3) / 1e9, 1),
                          hbm_frac=round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)))


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
                      unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 4), traffic=stored_traffic("decode_kernel"),
                      bytes_per_launch=nbytes, avg_launch_ms=round(ms, 5)))
    del per_step, state
    torch.cuda.empty_cache()
    return res


def bench_decode_gdn2(args, torch, gdn, synth):
    """Gated DeltaNet-2 decode: B=256, 16/64 heads, d=128, bf16, 1 GiB state updated in place;
    the 16 distinct seeded tokens are fed 4 times over (64 steps in the timed region)."""
    spec = synth.WORKLOADS["decode_gdn2_b256"]
    log(f"[bench] gdn2 decode workload {spec}")
    inp = synth.make_inputs(spec)
    per_step = [{k: inp[k][:, t].contiguous().cuda() for k in ("q", "k", "v", "a", "erase", "write")}
                for t in range(spec.T)]
    A_log = inp["A_log"].cuda()
    state = inp["S0"].cuda()
    del inp
    out = torch.empty((spec.B, spec.Hv, spec.Dv), dtype=spec.torch_dtype, device="cuda")

    def step(t):
        x = per_step[t % spec.T]
        gdn.gdn2_recurrent_step(x["q"], x["k"], x["v"], x["a"], A_log, x["erase"], x["write"], state, out=out)

    for t in range(min(args.warmup, 8)):
        step(t)
    steps = 64
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for t in range(steps):
        step(t)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    nbytes = decode_gdn2_bytes(spec.B, spec.Hk, spec.Hv, spec.Dk, spec.Dv, 2)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] gdn2 decode {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s")
    del per_step, state
    torch.cuda.empty_cache()
    return dict(value=round(gbs, 1), unit="GB/s", ms_per_step=round(ms, 5), steps=steps,
                tokens_per_s=round(spec.B / (ms * 1e-3), 1),
                config=dict(workload="decode_gdn2_b256", B=spec.B, Hk=spec.Hk, Hv=spec.Hv, Dk=spec.Dk,
                            Dv=spec.Dv, input_dtype="bf16", state_dtype="f32", distinct_tokens=spec.T),
                roofline=dict(kernel="decode_kernel<G2>", bound="hbm", achieved=round(gbs, 1),
                              peak=PEAK_HBM_GBS, unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 4),
                              traffic=stored_traffic("decode_kernel_gdn2"),
                              bytes_per_launch=nbytes, avg_launch_ms=round(ms, 5)))


def graph_timed(args, torch, step, sets, outputs):
    """Milliseconds per step of a kernel too short to time through per-call Python:
    args.steps calls of step (rotating over sets) captured in one HIP graph, so the
    timed replay holds the kernels back to back with no host work between them.
    The replay's outputs (names in `outputs`) must equal an eager run's bit for bit;
    the captured calls record no memset."""
    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    n = args.steps
    used = sorted({i % len(sets) for i in range(n)})
    for i in range(n):  # eager reference: each set's outputs as its last step leaves them
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    ref = {j: {k: sets[j][k].clone() for k in outputs} for j in used}
    for d in sets:
        for k in outputs:
            d[k].zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            step(sets[i % len(sets)])
    for r in range(2):  # each replay against the eager outputs, eager work between replays
        for d in sets:
            for k in outputs:
                d[k].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j in used:
            for k in outputs:
                if not torch.equal(sets[j][k], ref[j][k]):
                    raise RuntimeError(f"graph replay {r}: {k} of buffer set {j} differs from the eager run")
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    g.replay()
    stop.record()
    torch.cuda.synchronize()
    del g
    return start.elapsed_time(stop) / n


def bench_epilogue(args, torch, gdn, synth):
    """The gated RMS normalisation on the prefill output's shape (B=1, T=4096, 64 value heads,
    d=128, bf16): read x and z, write y, over rotated buffer sets."""
    shape = (1, 4096, 64, 128)
    log(f"[bench] gated rmsnorm workload {shape} bf16")
    x, z, w = synth.make_norm_inputs(shape, "bf16", seed=620)
    sets = [dict(x=x.cuda(), z=z.cuda(), y=torch.empty(shape, dtype=torch.bfloat16, device="cuda"))
            for _ in range(args.rotate)]
    w = w.cuda()

    def step(d):
        gdn.gdn_gated_rmsnorm(d["x"], d["z"], w, eps=1e-6, gate="silu", out=d["y"])

    ms = graph_timed(args, torch, step, sets, ["y"])
    nbytes = 3 * x.numel() * 2 + 128 * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] gated rmsnorm {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s")
    del sets
    torch.cuda.empty_cache()
    return dict(value=round(gbs, 1), unit="GB/s", ms_per_step=round(ms, 5), timing="hip graph of the steps",
                config=dict(workload="gated_rmsnorm_t4096", rows=4096 * 64, d=128, dtype="bf16", gate="silu"),
                roofline=dict(kernel="gated_rmsnorm_kernel", bound="hbm", achieved=round(gbs, 1),
                              peak=PEAK_HBM_GBS, unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 4),
                              traffic=stored_traffic("gated_rmsnorm_kernel"),
                              bytes_per_launch=nbytes, avg_launch_ms=round(ms, 5)))


def bench_prologue(args, torch, gdn, synth):
    """The causal conv1d + SiLU prologue on the prefill's shape: x [1, 4096, 12288] bf16
    (q | k | v channels of 16/64 heads, d=128) -> q, k, v, plus the new conv state."""
    B, T, Hk, Hv, D = 1, 4096, 16, 64, 128
    C = 2 * Hk * D + Hv * D
    log(f"[bench] causal conv1d workload B={B} T={T} C={C} bf16")
    x, w, b, s0 = synth.make_conv_inputs(B, T, C, "bf16", seed=630)
    w, b = w.cuda(), b.cuda()
    mk = lambda H: torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    sets = [dict(x=x.cuda(), s=s0.cuda(), so=torch.empty_like(s0, device="cuda"), q=mk(Hk), k=mk(Hk), v=mk(Hv))
            for _ in range(args.rotate)]

    def step(d):
        gdn.gdn_causal_conv1d(d["x"], w, b, d["s"], Hk=Hk, Hv=Hv, Dk=D, Dv=D, conv_state_out=d["so"],
                              q=d["q"], k=d["k"], v=d["v"])

    ms = graph_timed(args, torch, step, sets, ["q", "k", "v", "so"])
    nbytes = 2 * B * T * C * 2 + 2 * B * 3 * C * 2 + C * 5 * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] causal conv1d {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s")
    del sets
    torch.cuda.empty_cache()
    return dict(value=round(gbs, 1), unit="GB/s", ms_per_step=round(ms, 5), timing="hip graph of the steps",
                config=dict(workload="causal_conv1d_t4096", B=B, T=T, C=C, kernel_size=4, dtype="bf16",
                            activation="silu"),
                roofline=dict(kernel="causal_conv1d_kernel", bound="hbm", achieved=round(gbs, 1),
                              peak=PEAK_HBM_GBS, unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 4),
                              traffic=stored_traffic("causal_conv1d_kernel"),
                              bytes_per_launch=nbytes, avg_launch_ms=round(ms, 5)))


def bench_gdn2(args, torch, gdn, synth):
    """The Gated DeltaNet-2 prefill (B=1, T=8192, 16/64 heads, d=128, bf16): K steps of
    gdn2_chunk_fwd over rotated buffer sets, nothing else in the timed region."""
    spec = synth.WORKLOADS["gdn2_t8192"]
    log(f"[bench] gdn2 workload {spec}")
    inp = synth.make_inputs(spec)
    sets = []
    for _ in range(args.rotate):
        d = {k: (None if v is None else v.cuda().contiguous()) for k, v in inp.items()}
        d["out"] = torch.empty((spec.B, spec.T, spec.Hv, spec.Dv), dtype=spec.torch_dtype, device="cuda")
        d["ST"] = torch.empty((spec.B, spec.Hv, spec.Dk, spec.Dv), dtype=torch.float32, device="cuda")
        d["ws"] = gdn.alloc_workspace_gdn2(
            gdn.make_dims(spec.B, spec.T, spec.Hk, spec.Hv, spec.Dk, spec.Dv, spec.torch_dtype))
        sets.append(d)
    del inp

    def step(d):
        gdn.gdn2_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["A_log"], d["erase"], d["write"], d["S0"],
                           out=d["out"], final_state=d["ST"], workspace=d["ws"])

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(sets[i % len(sets)])
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    units = spec.B * spec.T * spec.Hv
    flop = gdn2_flop_per_token_head(spec.Dk, spec.Dv, spec.chunk) * units
    nbytes = gdn2_bytes(spec.B, spec.T, spec.Hk, spec.Hv, spec.Dk, spec.Dv, 2, spec.init_state)
    tf = flop / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] gdn2 {ms * 1e3:.1f} us/step")
    del sets
    torch.cuda.empty_cache()
    return dict(value=round(spec.B * spec.T / (ms * 1e-3), 1), unit="tokens/s", ms_per_step=round(ms, 5),
                config=dict(workload="gdn2_t8192", B=spec.B, T=spec.T, Hk=spec.Hk, Hv=spec.Hv, Dk=spec.Dk,
                            Dv=spec.Dv, chunk=spec.chunk, input_dtype="bf16", state_dtype="f32",
                            matrix_operands="f16", accumulate="f32"),
                roofline=dict(kernel="whole step (chunk_local2_kernel + scan_split_kernel<G2>)", bound="hbm",
                              achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                              frac=round(gbs / PEAK_HBM_GBS, 4), bytes_per_step=nbytes,
                              traffic=(None if stored_traffic("chunk_local2_kernel") is None
                                       or stored_traffic("scan_split_kernel_gdn2") is None else
                                       stored_traffic("chunk_local2_kernel") + stored_traffic("scan_split_kernel_gdn2"))),
                path=dict(flop=flop, tflops=round(tf, 2), mfma_frac=round(tf / PEAK_MFMA_F16_TFLOPS, 4)))


def bench_gdn2_bwd(args, torch, gdn, synth):
    """The Gated DeltaNet-2 backward on the same workload (B=1, T=8192, 16/64 heads, d=128):
    K calls of gdn2_chunk_bwd (output and final-state gradients given), each launch
    bracketed by HIP events on the call's stream."""
    spec = synth.WORKLOADS["gdn2_t8192"]
    log(f"[bench] gdn2 backward workload {spec}")
    inp = synth.make_inputs(spec)
    inp.update(synth.make_grad_inputs(spec))
    nsets = 2
    sets = []
    for _ in range(nsets):
        d = {k: (None if v is None else v.cuda().contiguous()) for k, v in inp.items()}
        d["ws"] = torch.empty(gdn.gdn2_chunk_bwd_workspace_bytes(
            gdn.make_dims(spec.B, spec.T, spec.Hk, spec.Hv, spec.Dk, spec.Dv, spec.torch_dtype)),
            dtype=torch.uint8, device="cuda")
        d["g"] = None
        sets.append(d)
    del inp
    stream = torch.cuda.current_stream()
    events = [gdn.StageEvents(gdn.GDN2_CHUNK_BWD_STAGES) for _ in range(args.steps)]

    def step(d, ev=None):
        d["g"] = gdn.gdn2_chunk_bwd(d["q"], d["k"], d["v"], d["a"], d["A_log"], d["erase"], d["write"],
                                    d["S0"], d["d_out"], d["d_ST"], workspace=d["ws"], grads=d["g"],
                                    stream=stream, stage_events=ev)

    for i in range(args.warmup):
        step(sets[i % nsets])
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(sets[i % nsets], events[i])
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    stage = [sum(e.stage_ms()[j] for e in events) / args.steps for j in range(gdn.GDN2_CHUNK_BWD_STAGES)]
    for e in events:
        e.close()
    units = spec.B * spec.T * spec.Hv
    fl = bwd2_flop_per_token_head(spec.Dk, spec.Dv, spec.chunk)
    names = gdn.BWD2_STAGE_NAMES
    dom = max(range(len(names)), key=lambda j: stage[j])
    dflop = fl[names[dom]] * units
    tf = dflop / (stage[dom] * 1e-3) / 1e12
    total_flop = sum(fl.values()) * units
    log(f"[bench] gdn2 backward {ms * 1e3:.1f} us/step; "
        + ", ".join(f"{n} {t * 1e3:.1f} us" for n, t in zip(names, stage)))
    del sets
    torch.cuda.empty_cache()
    return dict(value=round(spec.B * spec.T / (ms * 1e-3), 1), unit="tokens/s", ms_per_step=round(ms, 5),
                config=dict(workload="gdn2_t8192_backward", B=spec.B, T=spec.T, Hk=spec.Hk, Hv=spec.Hv,
                            Dk=spec.Dk, Dv=spec.Dv, chunk=spec.chunk, input_dtype="bf16",
                            grad_dtype="f32", arithmetic="f32"),
                stages_us={n: round(t * 1e3, 2) for n, t in zip(names, stage)},
                roofline=dict(kernel=names[dom], bound=("alu" if names[dom] in ("g2b_local", "g2b_prep") else "mfma"),
                              achieved=round(tf, 2), peak=PEAK_MFMA_F32_TFLOPS,
                              unit="TFLOP/s", frac=round(tf / PEAK_MFMA_F32_TFLOPS, 4), flop_per_launch=dflop,
                              avg_launch_ms=round(stage[dom], 5), traffic=stored_traffic(names[dom])),
                path=dict(flop=total_flop, tflops=round(total_flop / (ms * 1e-3) / 1e12, 2),
                          f32_frac=round(total_flop / (ms * 1e-3) / 1e12 / PEAK_MFMA_F32_TFLOPS, 4)))


def cpu_baseline(pre, min_seconds=10.0):
    """The float64 oracle on this host's cores: the whole prefill workload,
    repeated until at least min_seconds of CPU time have passed."""
    import numpy as np
    import oracle
    spec, inp = pre["spec"], pre["inp"]
    x = {k: (None if v is None else oracle.f64(v)) for k, v in inp.items()}
    threads = oracle.num_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        out, ST = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["a"], x["b"], x["A_log"], x["dt_bias"], S0=x["S0"])
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    assert np.isfinite(out).all()
    return dict(value=round(reps * spec.B * spec.T / dt, 1), unit="tokens/s", cores=threads, kind="oracle",
                seconds=round(dt, 3),
                sample=f"the whole prefill workload (B={spec.B}, T={spec.T}, {spec.Hv} value heads, "
                       f"d={spec.Dk}) {reps} times, float64 token loop, OpenMP over (sequence, value head)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rotate", type=int, default=3, help="buffer sets rotated in the timed region")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-gdn2", action="store_true")
    ap.add_argument("--no-bwd", action="store_true", help="skip the Gated DeltaNet-2 backward leg")
    ap.add_argument("--no-long", action="store_true", help="skip the long-context prefill leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run a 256 MiB device copy (counter calibration)")
    ap.add_argument("--summarize-stats", nargs=3, metavar=("DIR", "OUT", "COMMAND"))
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args()
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (got --gpus {args.gpus}); the multi-GPU "
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
    lng = None if args.no_long else bench_prefill_long(args, torch, gdn, synth)
    dec = None if args.no_decode else bench_decode(args, torch, gdn, synth)
    g2 = None if args.no_gdn2 else bench_gdn2(args, torch, gdn, synth)
    g2d = None if args.no_gdn2 or args.no_decode else bench_decode_gdn2(args, torch, gdn, synth)
    g2b = None if args.no_gdn2 or args.no_bwd else bench_gdn2_bwd(args, torch, gdn, synth)
    epi = bench_epilogue(args, torch, gdn, synth)
    pro = bench_prologue(args, torch, gdn, synth)
    if args.calibration_copy:
        calibration_copy(torch)
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
        "prefill_long": lng,
        "decode": dec,
        "gdn2": g2,
        "gdn2_decode": g2d,
        "gdn2_backward": g2b,
        "gated_rmsnorm": epi,
        "causal_conv1d": pro,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
