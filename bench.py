#!/usr/bin/env python3
"""Throughput of the bounded-decay KDA chunked forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 64k] [--gpus 1]

A step is one whole forward (gate, intra-chunk stage, inter-chunk state and
output) over the workload's synthetic inputs, which are resident in HBM before
timing starts.  Prints one JSON line: tokens/s (B*T per step), the path's
algorithmic TFLOP/s as a fraction of the bf16 MFMA peak, per-kernel HIP-event
times measured on the launch stream inside the timed region, the roofline of
the dominant kernel, and the CPU oracle's throughput on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA chunked fwd tokens/s at T=64K,H=32,d=128; % of bf16 MFMA peak"
PEAK_BF16_FLOPS = 2.5e15     # MI355X dense bf16 MFMA
PEAK_FP32_FLOPS = 157.3e12   # MI355X fp32 matrix
PEAK_HBM = 8.0e12            # MI355X HBM3E bytes/s


def flops_per_token_head(dk, dv, C):
    """Algorithmic flops of the chunked form per (token, head): the causal 16x16
    sub-tiles of M and A, the UT solve, W, U~, W S, K^T U, Q S and M U."""
    return (3 * dk + 2 * dv) * (C + 16) + 6 * dk * dv + C * C / 3.0


def path_bytes_per_token_head(dk, dv, es):
    """q, k, a, v and beta read once, out written once."""
    return (3 * dk + dv + dv) * es + es


# the sources the forward's chunk and state kernels are compiled from (the translation unit and
# every header it includes): counters taken on other sources are not reported
FWD_SOURCES = ("kda_kernels.hip", "kda_device.h", "kda_intra.h", "kda_state.h", "kda_state_seg.h", "kda_layout.h",
               "kda_launch.h", "kda_varlen.h", "kda_decode.h")

# the forward's two stages and the kernels each dispatches once per step
STAGES = {"kda_intra_kernel": ("kda_intra_kernel",),
          "state_stage": ("kda_seg_state_kernel", "kda_seg_scan_kernel", "kda_state_kernel")}


def record_layout(dk, dv, C, es):
    """Byte sizes of one chunk record (kda_layout.h): region 1 (W^T, Qbar^T, K^, gamma, exponents),
    one value slice (exponents, U~, Oi^T), and the record stride."""
    nt, ndk, ndv = C // 16, dk // 16, dv // 16
    tile = 256 * es
    wt = ndk * nt * tile
    kh = 2 * ((nt + 1) // 2) * ndk * tile
    region1 = 2 * wt + kh + dk * 4 + 16
    slice_ = 16 + 2 * nt * tile
    stride = (region1 + ndv * slice_ + 255) // 256 * 256
    return {"wt": wt, "kh": kh, "region1": region1, "slice": slice_, "ut_part": 16 + nt * tile, "stride": stride}


def seg_count(units, nc):
    """Segments per head of the state stage (kda_seg_count in kda_layout.h): enough (head, segment)
    work-groups for 256 compute units, at least 8 chunks each, none empty."""
    if units <= 0 or units >= 256 or nc < 16:
        return 1
    s = max(1, min(256 // units, nc // 8))
    ln = -(-nc // s)
    return -(-nc // ln)


def use_segmented(units, dv, dk, C, es):
    """Whether the state stage runs segmented (kda_use_segmented in kda_layout.h): where the
    per-slice stage's (head, value slice) work-groups do not fill 256 compute units, or with 256
    heads or more -- and only where the segmented stage's LDS ring holds two chunks."""
    L = record_layout(dk, dv, C, es)
    # the two passes' ring parts: pass 0 W^T, then K^, gamma and the exponents; pass 1 region 1
    rings = ((L["wt"], L["region1"] - 2 * L["wt"]), (L["region1"], 0))
    lds = 160 * 1024

    def ok(p1, p2):
        slot = (p1 + p2 + 15) // 16 * 16
        depth = 4 if 4 * slot <= lds else 3 if 3 * slot <= lds else 2 if 2 * slot <= lds else 0
        ndma = -(-p1 // 1024) + -(-p2 // 1024)
        return depth >= 2 and ((ndma + 3) // 4) * (depth - 2) <= 63

    return all(ok(*r) for r in rings) and (units * (dv // 16) < 256 or units >= 256)


def state_stage_bytes(B, H, T, dk, dv, C, es):
    """Design bytes of the state stage per step: pass 0 reads W^T, K^, gamma, the exponents and every
    slice's U~ of the chunks in all segments but the last and writes two float32 maps per segment;
    the scan reads and writes them; pass 1 reads region 1 and every slice of every chunk and writes
    out (one segment: pass 1 alone)."""
    L = record_layout(dk, dv, C, es)
    units, nc = B * H, T // C
    nseg = seg_count(units, nc) if use_segmented(units, dv, dk, C, es) else 1
    seglen = -(-nc // nseg) if nc else 0
    p1 = units * nc * (L["region1"] + (dv // 16) * L["slice"]) + units * T * dv * es
    if nseg == 1:
        return p1
    nc0 = units * min(nc, (nseg - 1) * seglen)
    p0 = nc0 * (L["wt"] + L["kh"] + dk * 4 + 16 + (dv // 16) * L["ut_part"])
    maps = units * (nseg - 1) * (dv * dk + dk * dk) * 4
    return p0 + maps + 3 * units * (nseg - 1) * dv * dk * 4 + p1


def _src_sha():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "chunked_gated_linear_bounded_amd", "csrc")
    for f in FWD_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    with open(os.path.join(ROOT, "chunked_gated_linear_bounded_amd", "build.py"), "rb") as fh:  # the flags
        h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(kernel + "@" + workload)
    except Exception:
        return None
    if not rec or rec.get("src_sha") != _src_sha():
        return None
    return rec.get("bytes_per_launch")


def _counter_rows(d):
    """(kernel name, counter, value) rows of every rocprofv3 counter CSV under `d`."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    return rows


def record_traffic(fetch_dir, write_dir, workload, copy_bytes):
    """HBM bytes per launch of the path's kernels from two rocprofv3 --pmc runs of
    this script (FETCH_SIZE, then WRITE_SIZE, both KiB per dispatch), each scaled
    by the factor that makes the same counter read the known size of the
    calibration copy (a float32 negation over `copy_bytes`, which reads and writes
    `copy_bytes` once).  Writes profiles/traffic.json keyed kernel@workload with
    the hash of the kernel sources the counters were taken on."""
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(d) if r[1] == counter]
        if not rows:
            raise SystemExit("no %s rows under %s" % (counter, d))
        cal = [v for (k, _, v) in rows if "neg" in k]
        if not cal:
            raise SystemExit("no calibration copy dispatch under %s" % d)
        factor = copy_bytes / (sum(cal) / len(cal) * 1024.0)
        for stage, pats in STAGES.items():
            # per step: the mean over its dispatches of every kernel the stage launches, summed
            names = sorted({k for (k, _, _) in rows if any(p in k for p in pats)})
            if not names:
                raise SystemExit("no %s dispatches under %s" % (stage, d))
            kib = 0.0
            for n in names:
                vals = [v for (k, _, v) in rows if k == n]
                kib += sum(vals) / len(vals)
            rec = out.setdefault(stage + "@" + workload, {"src_sha": _src_sha()})
            rec[counter.lower() + "_kib_raw"] = kib
            rec[counter.lower() + "_factor"] = factor
            rec[counter.lower() + "_bytes"] = kib * 1024.0 * factor
            rec["kernels"] = len(names)
    for rec in out.values():
        rec["bytes_per_launch"] = rec["fetch_size_bytes"] + rec["write_size_bytes"]
    p = os.path.join(ROOT, "profiles", "traffic.json")
    old = json.load(open(p)) if os.path.exists(p) else {}
    old.update(out)
    with open(p, "w") as fh:
        json.dump(old, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(out, indent=1))


def decode_bench(args):
    """Decode throughput: one token per (sequence, head) per step through kda_decode_step, a batch of
    sequences with the heads of the throughput workload (H=32, dk=dv=128, bf16 I/O), the float32
    state resident in HBM.  Algorithmic bytes per token-head: the state read and written once
    (2 dv dk 4) plus q, k, a, v, beta and out."""
    import torch
    import chunked_gated_linear_bounded_amd as kda
    import kda_inputs as KI
    B, H, d = args.decode_batch, 32, 128
    w = KI.Workload("decode", B, H, 16, d, d, 16, "bf16", 4.0, False, 9)
    dev = torch.device("cuda:0")
    inp = KI.make_inputs(w, device=dev)
    tok = {n: t[:, :, 0].contiguous() for n, t in inp.items()}
    gen = torch.Generator(device=dev)
    gen.manual_seed(9)
    S = torch.randn((B, H, d, d), generator=gen, device=dev, dtype=torch.float32) * 0.5
    out = torch.empty((B, H, d), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        kda.decode_step(tok["q"], tok["k"], tok["v"], tok["a"], tok["beta"], S, out=out, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = e0.elapsed_time(e1) / args.steps
    bph = 2 * d * d * 4 + (3 * d + d + d) * 2 + 2
    alg = bph * B * H
    print(json.dumps({
        "metric": "KDA decode tokens/s (one token per sequence and head, H=32, d=128, bf16 I/O, fp32 state)",
        "value": B / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "wall_ms_per_step": (t1 - t0) * 1e3 / args.steps, "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode", "B": B, "H": H, "dk": d, "dv": d, "state_bytes": B * H * d * d * 4},
        "roofline": {"kernel": "kda_decode_kernel", "bound": "hbm", "achieved": alg / (ms * 1e-3) / 1e9,
                     "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": alg / (ms * 1e-3) / PEAK_HBM,
                     "bytes_per_token_head": bph}}), flush=True)


def packed_bench(args):
    """Packed documents: the 64k stream of 32 heads holding documents of log-uniform lengths in
    [32, 4096] tokens (seeded), one kda_chunk_fwd_varlen call per step (plan, chunk stage and state
    stage), inputs and boundaries resident in HBM.  Algorithmic bytes: inputs read and outputs
    written once, each chunk record written once and read once."""
    import torch
    import chunked_gated_linear_bounded_amd as kda
    import kda_inputs as KI
    w = KI.PACKED
    lengths = KI.packed_lengths(w.T, w.seed)
    dev = torch.device("cuda:0")
    print("bench: generating %s inputs (%d documents)" % (w.name, len(lengths)), file=sys.stderr, flush=True)
    inp = KI.make_packed_inputs(w, device=dev)
    cu = torch.from_numpy(KI.cu_seqlens(lengths)).to(dev)
    N = len(lengths)
    ws = torch.empty(kda.varlen_workspace_bytes(N, w.H, w.T, w.dk, w.dv, w.chunk, w.torch_dtype),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((w.H, w.T, w.dv), dtype=w.torch_dtype, device=dev)
    fs = torch.empty((N, w.H, w.dv, w.dk), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        kda.chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], cu, w.g_min, w.chunk, out=out,
                             final_state=fs, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = e0.elapsed_time(e1) / args.steps
    assert torch.isfinite(out.float()).all().item(), "non-finite output"
    es = 2
    chunks = sum((n + w.chunk - 1) // w.chunk for n in lengths)
    rec = kda.workspace_bytes(1, 1, w.chunk, w.dk, w.dv, w.chunk, w.torch_dtype)
    th = w.H * w.T
    alg = th * ((3 * w.dk + 2 * w.dv) * es + es) + 2 * w.H * chunks * rec + N * w.H * w.dv * w.dk * 4
    print(json.dumps({
        "metric": "KDA chunked fwd tokens/s over packed documents (T=64K stream, H=32, d=128, bf16 I/O)",
        "value": w.T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "wall_ms_per_step": (t1 - t0) * 1e3 / args.steps, "higher_is_better": True,
        "dtype": w.io, "data": "synthetic",
        "config": {"workload": w.name, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv, "chunk": w.chunk,
                   "documents": N, "doc_len_min": min(lengths), "doc_len_max": max(lengths), "chunks_per_head": chunks},
        "mfma_peak_frac": flops_per_token_head(w.dk, w.dv, w.chunk) * th / (ms * 1e-3) / PEAK_BF16_FLOPS,
        "roofline": {"kernel": "kda_chunk_fwd_varlen (plan + chunk stage + state stage)", "bound": "hbm",
                     "achieved": alg / (ms * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": alg / (ms * 1e-3) / PEAK_HBM, "bytes_per_step": alg}}), flush=True)


def lowrank_bench(args):
    """The 64k workload with the gate pre-activation formed in the chunk kernel from a rank-R factor
    (kda_chunk_fwd_lowrank): one call per step, inputs resident in HBM.  Algorithmic bytes per
    token-head: q, k, v, beta read and out written once, plus R/H factor values per token-head (h is
    shared by the heads), with each chunk record written once and read once."""
    import torch
    import chunked_gated_linear_bounded_amd as kda
    import kda_inputs as KI
    w = KI.BY_NAME["64k"]
    R = args.lowrank
    dev = torch.device("cuda:0")
    print("bench: generating %s inputs with a rank-%d gate factor" % (w.name, R), file=sys.stderr, flush=True)
    inp = KI.make_inputs(w, device=dev)
    del inp["a"]
    lr = KI.make_lowrank_factors(w, R, device=dev)
    ws = torch.empty(kda.workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, w.torch_dtype), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((w.B, w.H, w.T, w.dv), dtype=w.torch_dtype, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        kda.chunk_fwd_lowrank(inp["q"], inp["k"], inp["v"], lr["h"], lr["z"], lr["A_log"], inp["beta"], w.g_min,
                              w.chunk, out=out, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = e0.elapsed_time(e1) / args.steps
    assert torch.isfinite(out.float()).all().item(), "non-finite output"
    es = 2
    th = w.B * w.H * w.T
    bph = (2 * w.dk + 2 * w.dv) * es + es + R * es / w.H
    alg = th * bph + 2 * ws.numel()
    print(json.dumps({
        "metric": "KDA chunked fwd tokens/s, gate pre-activation from a rank-%d factor (T=64K, H=32, d=128, bf16 I/O)"
                  % R,
        "value": w.B * w.T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "wall_ms_per_step": (t1 - t0) * 1e3 / args.steps,
        "higher_is_better": True, "dtype": w.io, "data": "synthetic",
        "config": {"workload": w.name + "-lowrank", "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
                   "chunk": w.chunk, "rank": R},
        "mfma_peak_frac": (flops_per_token_head(w.dk, w.dv, w.chunk) + 2 * R * w.dk) * th / (ms * 1e-3)
                          / PEAK_BF16_FLOPS,
        "path": {"bytes_per_token_head": bph,
                 "gbps_algorithmic": th * bph / (ms * 1e-3) / 1e9},
        "roofline": {"kernel": "kda_chunk_fwd_lowrank (chunk stage + state stage)", "bound": "hbm",
                     "achieved": alg / (ms * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": alg / (ms * 1e-3) / PEAK_HBM, "bytes_per_step": alg}}), flush=True)


def backward_bench(args):
    """The backward pass (kda_chunk_bwd) over the 64k workload with seeded incoming gradients (dout and
    a final-state gradient), inputs resident in HBM; one call per step.  Its bytes per step as this
    design moves them: inputs and dout read, float32 gradients written, the 16-token chunk records
    written once and read by the state and reverse passes, and the float32 chunk states and their
    gradients each written once and read once."""
    import torch
    import chunked_gated_linear_bounded_amd as kda
    import kda_inputs as KI
    w = KI.BY_NAME["64k"]
    dev = torch.device("cuda:0")
    print("bench: generating %s inputs and gradients" % w.name, file=sys.stderr, flush=True)
    inp = KI.make_inputs(w, device=dev)
    dout, dF = KI.make_grads(w, device=dev)
    ws = torch.empty(kda.bwd_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.torch_dtype), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        return kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], dout, w.g_min, dfinal_state=dF,
                             workspace=ws, stream=stream)

    for _ in range(args.warmup):
        g = step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        g = step()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = e0.elapsed_time(e1) / args.steps
    for key in ("dq", "dk", "dv", "da", "dbeta"):
        assert torch.isfinite(g[key]).all().item(), "non-finite " + key
    es = 2
    th = w.B * w.H * w.T
    nch = th // 16
    rec = kda.workspace_bytes(1, 1, 16, w.dk, w.dv, 16, w.torch_dtype)
    st = w.dk * w.dv * 4
    io = th * ((3 * w.dk + 2 * w.dv) * es + es)            # q, k, a, v, dout, beta
    grads = th * ((3 * w.dk + w.dv) * 4 + 4)               # dq, dk, da, dv, dbeta (float32)
    alg = io + grads + 3 * nch * rec + 4 * nch * st
    print(json.dumps({
        "metric": "KDA chunked backward tokens/s (T=64K, H=32, d=128, bf16 inputs, float32 gradients)",
        "value": w.B * w.T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "wall_ms_per_step": (t1 - t0) * 1e3 / args.steps,
        "higher_is_better": True, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name + "-backward", "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
                   "bwd_chunk": 16, "io": w.io},
        "roofline": {"kernel": "kda_chunk_bwd (all stages)", "bound": "hbm", "achieved": alg / (ms * 1e-3) / 1e9,
                     "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": alg / (ms * 1e-3) / PEAK_HBM,
                     "bytes_per_step": alg}}), flush=True)


def cpu_baseline(inputs, w, seconds):
    """The float64 oracle on whole heads of the same workload, all host threads, until `seconds`
    have passed: whole-job tokens/s extrapolated from the sampled heads.  Beside it, the same
    oracle on one thread over the first 16,384 tokens of head (0, 0)."""
    import kda_inputs as KI
    from oracle import native
    done, t_used = 0, 0.0
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    for (b, h) in heads:
        hs = KI.head_slice(inputs, b, h)
        t0 = time.perf_counter()
        native.recurrent(hs["q"], hs["k"], hs["v"], hs["a"], hs["beta"], w.g_min)
        t_used += time.perf_counter() - t0
        done += 1
        if t_used >= seconds:
            break
    per_head = t_used / done
    job_time = per_head * len(heads)
    threads = native.threads()
    t1n = min(w.T, 16384)
    hs = KI.head_slice(inputs, 0, 0, t1n)
    old = native.set_threads(1)
    try:
        t0 = time.perf_counter()
        native.recurrent(hs["q"], hs["k"], hs["v"], hs["a"], hs["beta"], w.g_min)
        one = time.perf_counter() - t0
    finally:
        native.set_threads(old)
    return {"value": w.B * w.T / job_time, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d heads (%d tokens each), float64 token recurrence, %.1f s on %d threads; "
                      "whole job extrapolated per head" % (done, len(heads), w.T, t_used, threads),
            "cpu_model": native.cpu_model(),
            "one_core": {"value": t1n / one / (w.B * w.H), "unit": "tokens/s",
                         "sample": "%d tokens of one head on 1 thread, %.2f s; whole job extrapolated" % (t1n, one),
                         "token_heads_per_s": t1n / one}}


def ablation_bench(args):
    """The 1m workload (B=1, H=8, T=1,048,576, d=128, bf16) with the bounded gate and with the
    unbounded log-sigmoid gate it replaces, one forward each: the device counters of non-finite
    Gamma-scaled bf16 key operands of the diagonal 16-token tiles and of non-finite outputs."""
    import torch
    import chunked_gated_linear_bounded_amd as kda
    import kda_inputs as KI
    w = KI.BY_NAME["1m"]
    dev = torch.device("cuda:0")
    print("bench: generating %s inputs" % w.name, file=sys.stderr, flush=True)
    inp = KI.make_inputs(w, device=dev)
    out = torch.empty((w.B, w.H, w.T, w.dv), dtype=w.torch_dtype, device=dev)
    ws = torch.empty(kda.workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, w.torch_dtype), dtype=torch.uint8,
                     device=dev)
    res = {}
    for gate in ("bounded", "logsigmoid"):
        cnt = torch.zeros(2, dtype=torch.int64, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        stream = torch.cuda.current_stream(dev)
        e0.record(stream)
        kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], w.g_min, w.chunk, out=out, workspace=ws,
                      stream=stream, gate=gate, counts=cnt)
        e1.record(stream)
        torch.cuda.synchronize()
        c = cnt.tolist()
        res[gate] = {"nonfinite_operands": c[0], "nonfinite_outputs": c[1], "ms": e0.elapsed_time(e1)}
    th = w.B * w.H * w.T
    print(json.dumps({
        "metric": "bf16 overflow count, bounded vs unbounded gate (1m workload)", "unit": "count",
        "dtype": w.io, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv, "chunk": w.chunk,
                   "a": "0.9 N(0,1) + 0.1 (+-12)"},
        "operands_checked": th * w.dk, "outputs": th * w.dv, "bounded": res["bounded"],
        "logsigmoid": res["logsigmoid"]}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="64k", help="tiny, 8k, 64k, 256k or 1m")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, run one float32 negation over MIB MiB (the counter calibration copy)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: turn two rocprofv3 --pmc output folders of this script into "
                         "profiles/traffic.json (needs --copy-calibration as used in those runs)")
    ap.add_argument("--decode-batch", type=int, default=0, metavar="B",
                    help="instead of the chunked forward, time kda_decode_step on B sequences x 32 heads")
    ap.add_argument("--packed", action="store_true",
                    help="instead of the fixed-length workload, time kda_chunk_fwd_varlen on the 64k packed stream")
    ap.add_argument("--lowrank", type=int, default=0, metavar="R",
                    help="instead of reading a, form the gate pre-activation from a rank-R factor (64k workload)")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the forward, time the backward pass (kda_chunk_bwd) on the 64k workload")
    ap.add_argument("--ablation", action="store_true",
                    help="instead of timing, count non-finite operands and outputs of the 1m workload with the "
                         "bounded and the unbounded gate")
    args = ap.parse_args()
    if args.decode_batch > 0:
        decode_bench(args)
        return
    if args.packed:
        packed_bench(args)
        return
    if args.lowrank > 0:
        lowrank_bench(args)
        return
    if args.backward:
        backward_bench(args)
        return
    if args.ablation:
        ablation_bench(args)
        return
    if args.traffic_from:
        if args.copy_calibration <= 0:
            raise SystemExit("--traffic-from needs --copy-calibration MIB")
        record_traffic(args.traffic_from[0], args.traffic_from[1], args.workload, args.copy_calibration << 20)
        return
    if args.gpus != 1:
        print("bench.py: measures one GPU only (the path shards over heads with no "
              "communication); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import chunked_gated_linear_bounded_amd as kda
    import kda_inputs as KI

    w = KI.BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("bench: generating %s inputs on %s" % (w.name, torch.cuda.get_device_name(dev)), file=sys.stderr,
          flush=True)
    inp = KI.make_inputs(w, device=dev)
    es = 4 if w.io == "fp32" else 2
    ws = torch.empty(kda.workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, w.torch_dtype), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((w.B, w.H, w.T, w.dv), dtype=w.torch_dtype, device=dev)
    fs = torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device=dev) if w.final_state else None
    stream = torch.cuda.current_stream(dev)

    def step(e=None):
        if e is not None:
            e[0].record(stream)
        kda.chunk_intra(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], ws, w.g_min, w.chunk, stream=stream)
        if e is not None:
            e[1].record(stream)
        kda.chunk_state(ws, out, fs, w.chunk, dk=w.dk, stream=stream)
        if e is not None:
            e[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    print("bench: timing %d steps" % args.steps, file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    intra_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    state_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    assert torch.isfinite(out.float()).all().item(), "non-finite output"
    if args.copy_calibration > 0:
        cx = torch.ones(args.copy_calibration << 18, dtype=torch.float32, device=dev)
        cy = torch.empty_like(cx)
        torch.neg(cx, out=cy)
        torch.cuda.synchronize()
        del cx, cy

    th = w.B * w.H * w.T
    flops = flops_per_token_head(w.dk, w.dv, w.chunk) * th
    peak = PEAK_BF16_FLOPS if w.io == "bf16" else PEAK_FP32_FLOPS
    tokens_per_s = w.B * w.T / (ms_step * 1e-3)
    alg_bytes = path_bytes_per_token_head(w.dk, w.dv, es) * th  # each input read once, out written once
    rec_bytes = w.B * w.H * (w.T // w.chunk) * record_layout(w.dk, w.dv, w.chunk, es)["stride"]
    in_bytes = th * ((3 * w.dk + w.dv) * es + es)
    kern = {  # the chunk stage writes every record once; the state stage's passes read them
        "kda_intra_kernel": {"ms": intra_ms, "bytes": in_bytes + rec_bytes},
        "state_stage": {"ms": state_ms, "bytes": state_stage_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, es)},
    }
    dom = max(kern, key=lambda k: kern[k]["ms"])
    # the roofline of the dominant kernel on the path's algorithmic bytes (inputs read once, out
    # written once): what the whole path has to move, over the time this one kernel takes
    ach = alg_bytes / (kern[dom]["ms"] * 1e-3)
    traffic = _traffic(dom, w.name)
    step_traffic = [_traffic(k, w.name) for k in kern]
    step_traffic = None if None in step_traffic else sum(step_traffic)
    t_floor = max(flops / peak, alg_bytes / PEAK_HBM)
    res = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.io,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv, "chunk": w.chunk,
                   "io": w.io, "g_min": w.g_min},
        "mfma_peak_frac": flops / (ms_step * 1e-3) / peak,
        "path": {"tflops_algorithmic": flops / (ms_step * 1e-3) / 1e12,
                 "gbps_algorithmic": alg_bytes / (ms_step * 1e-3) / 1e9,
                 "hbm_peak_frac": alg_bytes / (ms_step * 1e-3) / PEAK_HBM,
                 "attainable_frac": t_floor / (ms_step * 1e-3),
                 "flop_per_token_head": flops_per_token_head(w.dk, w.dv, w.chunk),
                 "bytes_per_token_head": path_bytes_per_token_head(w.dk, w.dv, es),
                 "traffic_counters": step_traffic,
                 "traffic_over_algorithmic": None if step_traffic is None else step_traffic / alg_bytes},
        "kernels_ms": {k: v["ms"] for k, v in kern.items()},
        "kernels_design_bytes": {k: v["bytes"] for k, v in kern.items()},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": ach / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": ach / PEAK_HBM, "algorithmic_bytes": alg_bytes, "traffic": traffic,
                     "traffic_over_algorithmic": None if traffic is None else traffic / alg_bytes},
    }
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(inp, w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
