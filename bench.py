#!/usr/bin/env python3
"""Benchmark of libm3scan on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

A step is one m3_scan_fwd call (the whole chunked prefill: prefix scans,
data-RoPE, intra-chunk tiles, state passing, outputs and final state) over one
batch of the prefill_bf16 workload (batch 4, 16 heads, L = 2048, P = 64,
N = 64, R = 1, bf16 I/O, fp32 state), inputs resident in HBM.  Prints one
JSON line: whole-job tokens/s, the roofline of the scan kernel (algorithmic
bytes per launch / its average launch time from HIP events on the launch
stream, against 8 TB/s), the fp64 oracle's rate on this host's cores, and
secondary lines for the MIMO, long-context and decode workloads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Mamba-3 scan tokens/s (chunked prefill) + decode step/s; % MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PROFILE_DIR = os.path.join(ROOT, "profiles")


def io_bytes(w):
    return 4 if w.io_dtype == "f32" else 2


def scan_algorithmic_bytes(w, L=None, ngroups=0, a_tok=False, phase="native", premix=False):
    """Minimum HBM bytes of one m3_scan_fwd: every input read once, y and the
    final state record written once.  Options: B and C read once per head
    group, A per token, no theta with the zero phase, the pre-mixer's
    parameters (and the shuffle permutation) once."""
    L = w.seqlen if L is None else L
    e = io_bytes(w)
    R, P, N, H = w.rank, w.headdim, w.dstate, w.heads
    G = ngroups or H
    per_tok = e * 2 * R * P + 4 * 2 + (0 if phase == "zero" else 4 * (N // 2)) + (4 if a_tok else 0)
    per_grp_tok = e * 2 * R * N
    per_bh = 4 * N * P + e * (R * N + R * P)
    extra = 0 if a_tok else 4 * H
    if phase == "shuffle":
        extra += 4 * (N // 2)
    if premix:
        extra += 4 * (2 * N + 2 * H * R * N + H)
    return w.batch * (L * (H * per_tok + G * per_grp_tok) + H * per_bh) + extra


def bwd_algorithmic_bytes(w, ngroups=0, premix=False):
    """One m3_scan_bwd: x, B, C, dy, dt, theta, lam read once; dx, dB, dC,
    ddt, dtheta, dlam written once in float32 (checkpoint traffic excluded).
    With head groups B, C and their gradients are per group; the pre-mixer
    adds its parameters read and their gradients written."""
    e = io_bytes(w)
    R, P, N, H = w.rank, w.headdim, w.dstate, w.heads
    G = ngroups or H
    per_head_tok = e * 2 * R * P + 4 * (N // 2 + 2) + 4 * (R * P + N // 2 + 2)
    per_grp_tok = e * 2 * R * N + 4 * 2 * R * N
    extra = 2 * 4 * (2 * N + 2 * H * R * N + H) if premix else 0
    return w.batch * w.seqlen * (H * per_head_tok + G * per_grp_tok) + 8 * H + extra


def decode_algorithmic_bytes(w, premix=False):
    """One m3_decode_step: state h read and written, record (B, X) read and
    written, step inputs read, y written (plus the pre-mixer's parameters)."""
    e = io_bytes(w)
    R, P, N, H = w.rank, w.headdim, w.dstate, w.heads
    per_bh = 8 * N * P + 2 * e * (R * N + R * P) + e * (2 * R * N + R * P) + 4 * (N // 2 + 2) \
        + e * R * P
    extra = 4 * (2 * N + 2 * H * R * N + H) if premix else 0
    return w.batch * H * per_bh + 4 * H + extra


def _counter_rows(path, kernel_regex=None):
    import csv
    import re
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel_regex and not re.search(kernel_regex, r["Kernel_Name"]):
                continue
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def traffic_summary(name, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_mib,
                    kernel_regex, call_regex):
    """HBM bytes per call of the library entry point from rocprofv3 FETCH_SIZE
    and WRITE_SIZE runs (KiB per dispatch, summed over the dispatches a call
    makes), each scaled by copy_bytes / counter reading of a plain device copy
    of `copy_mib` MiB.  Writes profiles/<name>_traffic.json."""
    import collections
    copy_bytes = copy_mib * (1 << 20)

    def per_dispatch(path, regex):
        d = collections.defaultdict(float)
        for did, k, v in _counter_rows(path, regex):
            d[did] += v
        return d

    cf = per_dispatch(copy_fetch_csv, "copyBuffer|copy")
    cw = per_dispatch(copy_write_csv, "copyBuffer|copy")
    big_f = [v for v in cf.values() if v > copy_bytes / 1024 / 8]
    big_w = [v for v in cw.values() if v > copy_bytes / 1024 / 8]
    ffac = copy_bytes / (sum(big_f) / len(big_f) * 1024)
    wfac = copy_bytes / (sum(big_w) / len(big_w) * 1024)
    f = per_dispatch(fetch_csv, kernel_regex)
    w = per_dispatch(write_csv, kernel_regex)
    ncalls_f = len({d for d, k, v in _counter_rows(fetch_csv, call_regex)})
    ncalls_w = len({d for d, k, v in _counter_rows(write_csv, call_regex)})
    fetch = sum(f.values()) * 1024 * ffac / ncalls_f
    write = sum(w.values()) * 1024 * wfac / ncalls_w
    out = {"workload": name, "bytes_per_launch": round(fetch + write),
           "fetch_bytes": round(fetch), "write_bytes": round(write),
           "fetch_scale": round(ffac, 4), "write_scale": round(wfac, 4),
           "calls": ncalls_f, "source_hash": kernel_source_hash(_kind(name))}
    os.makedirs(PROFILE_DIR, exist_ok=True)
    with open(os.path.join(PROFILE_DIR, "%s_traffic.json" % name), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


# Device sources each measured kernel is compiled from.
KERNEL_SOURCES = {
    "scan": ["m3_device.hpp", "m3_scan_kernel.hpp", "m3_scan_inst.hpp", "m3_scan_f32.hip",
             "m3_scan_bf16_a.hip", "m3_scan_bf16_b.hip"],
    "decode": ["m3_device.hpp", "m3_decode.hip"],
}


def kernel_source_hash(kind):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mamba_selective_ssm_amd", "csrc")
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _kind(name):
    return "decode" if name == "decode" else "scan"


def load_traffic(name):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources; else None."""
    path = os.path.join(PROFILE_DIR, "%s_traffic.json" % name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash(_kind(name)):
        return None
    return d.get("bytes_per_launch")


def time_launches(fn, steps, warmup, torch):
    """Run fn() warmup + steps times; returns (total seconds, mean kernel ms).
    Two HIP events on the launch stream bracket the timed region, so the mean
    step duration is their span over the steps: the steps' kernels and the
    gaps between them, with no other work queued in between (an event record
    per step would add its own barrier to every step)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        fn()
    ev1.record(stream)
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    kms = ev0.elapsed_time(ev1) / max(steps, 1)
    return total, kms


def bench_prefill(w, steps, warmup, torch, m3, synth, seed=1001):
    inp = synth.make_scan_inputs(w, seed, "cuda")
    # Arguments, outputs and workspace are prepared once; each step is one
    # m3_scan_fwd call on the same resident inputs.
    step = m3.ScanCall(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"],
                       inp["lam"], chunk=w.chunk)
    total, kms = time_launches(step, steps, warmup, torch)
    tokens = w.batch * w.seqlen
    nbytes = scan_algorithmic_bytes(w)
    return dict(tokens_per_s=tokens * steps / total, ms_per_step=1e3 * total / steps,
                kernel_ms=kms, bytes=nbytes, gbs=nbytes / (kms * 1e-3) / 1e9, inputs=inp)


# Option workloads measured beside the plain mixer, at the prefill_bf16 shape.
OPTION_CASES = {
    "prefill_bf16+premix": dict(premix=True),
    "prefill_bf16+groups4+A_t": dict(ngroups=4, a_tok=True),
    "prefill_bf16+phase_zero": dict(phase="zero"),
    "prefill_bf16+phase_shuffle": dict(phase="shuffle"),
    # the same 8192 tokens per head as 8 packed sequences of mixed lengths
    "prefill_bf16+packed8": dict(packed=[1536, 256, 1024, 768, 2048, 512, 640, 1408]),
}


def _premix(m3, extras):
    pm = extras["premix"]
    return m3.Premix(pm["B_norm_w"], pm["C_norm_w"], pm["B_bias"], pm["C_bias"], pm["dt_bias"],
                     pm["eps"])


def bench_prefill_options(w, opts, steps, warmup, torch, m3, synth, seed=1002):
    ngroups, a_tok = opts.get("ngroups", 0), opts.get("a_tok", False)
    phase, premix = opts.get("phase", "native"), opts.get("premix", False)
    lens = opts.get("packed")
    cu = None
    if lens is not None:
        assert sum(lens) == w.batch * w.seqlen
        w = w.with_(batch=1, seqlen=sum(lens))
        cu = torch.tensor([0] + [sum(lens[:i + 1]) for i in range(len(lens))], dtype=torch.int32,
                          device="cuda")
    inp, ex = synth.make_option_inputs(w, seed, "cuda", ngroups=ngroups, a_per_token=a_tok,
                                       phase=phase, premix=premix)
    step = m3.ScanCall(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"],
                       None if phase == "zero" else inp["theta"], inp["lam"], chunk=w.chunk,
                       ngroups=ngroups, phase=phase, perm=ex.get("perm"),
                       premix=_premix(m3, ex) if premix else None, cu_seqlens=cu,
                       max_seqlen=max(lens) if lens else None)
    total, kms = time_launches(step, steps, warmup, torch)
    nbytes = scan_algorithmic_bytes(w, ngroups=ngroups, a_tok=a_tok, phase=phase, premix=premix)
    if lens is not None:   # one state record per sequence instead of per batch row
        e = io_bytes(w)
        nbytes += (len(lens) - 1) * w.heads * (4 * w.dstate * w.headdim
                                               + e * w.rank * (w.dstate + w.headdim)) + 4 * (len(lens) + 1)
    return dict(tokens_per_s=w.batch * w.seqlen * steps / total, kernel_ms=kms, bytes=nbytes,
                gbs=nbytes / (kms * 1e-3) / 1e9)


def bench_backward(w, steps, warmup, torch, m3, synth, seed=1003, method="auto", ngroups=0,
                   phase="native", premix=False):
    """One m3_scan_bwd call per step on resident inputs and dy ("auto" picks
    the chunked method where it is supported), optionally with head groups, a
    phase mode and the pre-mixer."""
    inp, ex = synth.make_option_inputs(w, seed, "cuda", ngroups=ngroups, phase=phase,
                                       premix=premix)
    g = torch.Generator(device="cuda").manual_seed(seed)
    dy = torch.randn(inp["x"].shape, generator=g, device="cuda").to(w.torch_dtype)
    step = m3.ScanBwdCall(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"],
                          inp["lam"], dy, state_grads=False, method=method, ngroups=ngroups,
                          phase=phase, perm=ex.get("perm"),
                          premix=_premix(m3, ex) if premix else None)
    total, kms = time_launches(step, steps, warmup, torch)
    nbytes = bwd_algorithmic_bytes(w, ngroups=ngroups, premix=premix)
    return dict(tokens_per_s=w.batch * w.seqlen * steps / total, kernel_ms=kms, bytes=nbytes,
                gbs=nbytes / (kms * 1e-3) / 1e9)


def bench_decode(w, steps, warmup, torch, m3, synth, seed=1004, premix=False):
    """Decode workload: a 1024-token prefill builds the resident state, then
    `steps` single-token steps with fresh inputs, one launch each."""
    pre = synth.make_scan_inputs(w, seed, "cuda")
    _, st = m3.m3_scan_fwd(pre["x"], pre["B"], pre["C"], pre["dt"], pre["A"], pre["theta"],
                           pre["lam"], chunk=w.chunk)
    A = pre["A"]
    del pre
    pm = None
    if premix:
        # the pre-mixer's parameters as the option generator draws them
        _, ex = synth.make_option_inputs(w.with_(seqlen=1, batch=1), seed, "cuda", premix=True)
        pm = _premix(m3, ex)
    nsteps = warmup + steps
    ins = [synth.make_decode_inputs(w, seed, s, A, "cuda") for s in range(nsteps)]
    y = torch.empty(w.batch, w.heads, w.rank, w.headdim, dtype=w.torch_dtype, device="cuda")
    calls = iter([m3.DecodeCall(s["x"], s["B"], s["C"], s["dt"], s["A"], s["theta"], s["lam"],
                                st, y=y, premix=pm) for s in ins])

    def step():
        next(calls)()

    total, kms = time_launches(step, steps, warmup, torch)
    nbytes = decode_algorithmic_bytes(w, premix=premix)
    return dict(steps_per_s=steps / total, tokens_per_s=w.batch * steps / total,
                ms_per_step=1e3 * total / steps, kernel_ms=kms, bytes=nbytes,
                gbs=nbytes / (kms * 1e-3) / 1e9)


def cpu_baseline(w, inp, budget_s, torch):
    """fp64 oracle on this host's cores over the same inputs (whole workload,
    repeated until about budget_s seconds have been spent)."""
    import oracle
    from mamba_selective_ssm_amd.synth import to_f64_numpy
    args = [to_f64_numpy(inp[k]) for k in ("x", "B", "C", "dt", "A", "theta", "lam")]
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.scan(*args, threads=threads)
        reps += 1
        if time.perf_counter() - t0 >= budget_s or reps >= 1000:
            break
    el = time.perf_counter() - t0
    return {"value": w.batch * w.seqlen * reps / el, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": "whole %s workload (%d x %d tokens, %d heads) x %d repetitions, %.1f s"
                      % (w.name, w.batch, w.seqlen, w.heads, reps, el)}


def progress(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def backward_lines(steps, torch, m3, synth):
    """Backward secondary lines: the chunked method (what "auto" picks) and
    the step-by-step adjoint, on prefill_bf16 and mimo_prefill_bf16."""
    sec = {}
    for name in ("prefill_bf16", "mimo_prefill_bf16"):
        for method, tag, n in (("chunked", "backward", min(steps, 10)), ("step", "backward_step", 3)):
            progress("timing the %s backward on %s" % (method, name))
            rb = bench_backward(synth.WORKLOADS[name], n, 1, torch, m3, synth, method=method)
            sec[tag + ":" + name] = {"tokens_per_s": round(rb["tokens_per_s"], 1),
                                     "kernel_ms": round(rb["kernel_ms"], 4),
                                     "hbm_gbs": round(rb["gbs"], 1),
                                     "hbm_frac": round(rb["gbs"] / HBM_PEAK_GBS, 4)}
            torch.cuda.empty_cache()
    # the option maps around the chunked gradient: 8 head groups of 2, shuffled
    # phases and the pre-mixer
    w = synth.WORKLOADS["prefill_bf16"]
    progress("timing the chunked backward with options on prefill_bf16")
    rb = bench_backward(w, min(steps, 10), 1, torch, m3, synth, method="chunked",
                        ngroups=w.heads // 2, phase="shuffle", premix=True)
    sec["backward_options:prefill_bf16"] = {"tokens_per_s": round(rb["tokens_per_s"], 1),
                                            "kernel_ms": round(rb["kernel_ms"], 4),
                                            "hbm_gbs": round(rb["gbs"], 1),
                                            "hbm_frac": round(rb["gbs"] / HBM_PEAK_GBS, 4),
                                            "options": "ngroups=8 phase=shuffle premix"}
    torch.cuda.empty_cache()
    return sec


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_bf16")
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-options", action="store_true",
                    help="skip the option workloads (pre-mixer, groups, phase modes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only time the decode workload (for per-kernel counter runs)")
    ap.add_argument("--backward-only", action="store_true",
                    help="only time the backward (both methods) on prefill_bf16 and "
                         "mimo_prefill_bf16, one JSON line each (for per-kernel traces)")
    ap.add_argument("--traffic-summary", nargs=5,
                    metavar=("NAME", "FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="turn rocprofv3 FETCH_SIZE/WRITE_SIZE csv files into "
                         "profiles/NAME_traffic.json (no GPU needed)")
    ap.add_argument("--copy-mib", type=int, default=1024)
    args = ap.parse_args(argv)

    if args.traffic_summary:
        name = args.traffic_summary[0]
        regex, call = (("decode_kernel", "decode_kernel") if name == "decode"
                       else ("scan_kernel", "scan_kernel.*Lb1E"))
        traffic_summary(name, *args.traffic_summary[1:], args.copy_mib, regex, call)
        return 0

    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the mixer needs no exchange "
              "between GPUs; batch and heads shard without communication).", file=sys.stderr)
        return 2

    import torch
    import mamba_selective_ssm_amd as m3
    from mamba_selective_ssm_amd import synth

    if args.backward_only:
        for k, v in backward_lines(args.steps, torch, m3, synth).items():
            print(json.dumps({"line": k, **v}), flush=True)
        return 0

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        a = torch.ones(n, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n * 4, "launches": 3}))
        return 0

    if args.decode_only:
        wd = synth.WORKLOADS["decode"]
        progress("timing decode only: prefill + %d steps" % args.decode_steps)
        rd = bench_decode(wd, args.decode_steps, 2, torch, m3, synth)
        print(json.dumps({"workload": "decode", "steps_per_s": round(rd["steps_per_s"], 1),
                          "kernel_ms": round(rd["kernel_ms"], 5),
                          "hbm_gbs": round(rd["gbs"], 1)}), flush=True)
        return 0

    w = synth.WORKLOADS[args.workload]
    if args.chunk:
        w = w.with_(chunk=args.chunk)
    progress("timing %s: %d warmup + %d steps" % (w.name, args.warmup, args.steps))
    r = bench_prefill(w, args.steps, args.warmup, torch, m3, synth)
    traffic = load_traffic(w.name)
    roof = {"bound": "hbm", "achieved": round(r["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(r["gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "m3::scan_kernel", "kernel_ms": round(r["kernel_ms"], 5),
            "algorithmic_bytes_per_launch": r["bytes"]}
    out = {"metric": METRIC, "value": round(r["tokens_per_s"], 1), "unit": "tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(r["ms_per_step"], 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": w.io_dtype, "data": "synthetic",
           "config": {"workload": w.name, "batch": w.batch, "heads": w.heads,
                      "seqlen": w.seqlen, "headdim": w.headdim, "dstate": w.dstate,
                      "rank": w.rank, "chunk": w.chunk, "state": "fp32",
                      "accumulate": "fp32"},
           "roofline": roof}
    inp = r.pop("inputs")

    if not args.no_secondary:
        sec = {}
        for name in ("mimo_prefill_bf16", "long_prefill_bf16"):
            ws = synth.WORKLOADS[name]
            progress("timing %s" % name)
            rs = bench_prefill(ws, 5, 2, torch, m3, synth)
            rs.pop("inputs")
            sec[name] = {"tokens_per_s": round(rs["tokens_per_s"], 1),
                         "kernel_ms": round(rs["kernel_ms"], 4),
                         "hbm_gbs": round(rs["gbs"], 1),
                         "hbm_frac": round(rs["gbs"] / HBM_PEAK_GBS, 4),
                         "traffic": load_traffic(name)}
            torch.cuda.empty_cache()
        wd = synth.WORKLOADS["decode"]
        progress("timing decode: prefill + %d steps" % args.decode_steps)
        rd = bench_decode(wd, args.decode_steps, 8, torch, m3, synth)
        sec["decode"] = {"steps_per_s": round(rd["steps_per_s"], 1),
                         "tokens_per_s": round(rd["tokens_per_s"], 1),
                         "kernel_ms": round(rd["kernel_ms"], 5),
                         "hbm_gbs": round(rd["gbs"], 1),
                         "hbm_frac": round(rd["gbs"] / HBM_PEAK_GBS, 4),
                         "traffic": load_traffic("decode")}
        if not args.no_options:
            progress("timing decode with the pre-mixer")
            rd = bench_decode(wd, min(args.decode_steps, 256), 8, torch, m3, synth, premix=True)
            sec["decode+premix"] = {"steps_per_s": round(rd["steps_per_s"], 1),
                                    "kernel_ms": round(rd["kernel_ms"], 5),
                                    "hbm_gbs": round(rd["gbs"], 1),
                                    "hbm_frac": round(rd["gbs"] / HBM_PEAK_GBS, 4)}
            torch.cuda.empty_cache()
        wp = synth.WORKLOADS["prefill_bf16"]
        for name, opts in ({} if args.no_options else OPTION_CASES).items():
            progress("timing %s" % name)
            ro = bench_prefill_options(wp, opts, 20, 3, torch, m3, synth)
            sec[name] = {"tokens_per_s": round(ro["tokens_per_s"], 1),
                         "kernel_ms": round(ro["kernel_ms"], 5),
                         "hbm_gbs": round(ro["gbs"], 1),
                         "hbm_frac": round(ro["gbs"] / HBM_PEAK_GBS, 4)}
        sec.update(backward_lines(args.steps, torch, m3, synth))
        out["secondary"] = sec
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        progress("timing the fp64 oracle on the host")
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_budget, torch)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
