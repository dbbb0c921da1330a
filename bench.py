#!/usr/bin/env python3
"""Benchmark of libm3scan on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

A step is one m3_scan_fwd call (the whole chunked prefill: prefix scans,
data-RoPE, intra-chunk tiles, state passing, outputs and final state) over one
batch of the MIMO prefill workload (batch 8, 32 heads, L = 4096, P = 64,
N = 128, rank 4, bf16 I/O, fp32 state), inputs resident in HBM.  Prints one
JSON line: whole-job tokens/s; the roofline of the scan kernel (algorithmic
bytes per launch over its average launch time from HIP events on the launch
stream, against 8 TB/s, and its dense-tile bf16 flops against 2.5 PFLOP/s);
the fp64 oracle's rate on this host's cores over a sample of the same
workload; and secondary lines, each with its own roofline, for the
single-layer, long-context (with its chunk sweep) and decode workloads, the
options and the gradient.
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


def scan_dense_flops(w, Q=None, L=None):
    """Dense-tile flops of one m3_scan_fwd by the chunked method at chunk Q:
    per head-token 2 Q R^2 N (score tiles C B^T) + 2 Q R^2 P ((S o M) X, both
    over whole Q R x Q R tiles, masked half included) + 4 R N P (the chunk
    state B^T X and the state term C G)."""
    Q = Q or w.chunk
    L = w.seqlen if L is None else L
    R, P, N = w.rank, w.headdim, w.dstate
    per_ht = 2 * Q * R * R * N + 2 * Q * R * R * P + 4 * R * N * P
    return w.batch * L * w.heads * per_ht


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


PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof/trace_{n} -o t "
             "-- python3 bench.py --steps 20 --warmup 3 --no-secondary --no-cpu-baseline --workload {n}",
    "trace_decode": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof/trace_decode "
                    "-o t -- python3 bench.py --decode-only --decode-steps 256",
    "pmc": "rocprofv3 --pmc {c} --kernel-include-regex scan_kernel --output-format csv "
           "-d gpurun_out/prof/{f}_{n} -o {f} -- python3 bench.py --workload {n} --steps 3 --warmup 1 "
           "--no-secondary --no-cpu-baseline",
    "pmc_decode": "rocprofv3 --pmc {c} --kernel-include-regex decode_kernel --output-format csv "
                  "-d gpurun_out/prof/{f}_decode -o {f} -- python3 bench.py --decode-only --decode-steps 64",
    "copy": "rocprofv3 --pmc {c} --output-format csv -d gpurun_out/prof/c{f} -o {f} "
            "-- python3 bench.py --copy-calibration 1024",
}


def trace_summary(name, trace_csv):
    """profiles/<kernel>_<name>.md from a rocprofv3 kernel-trace csv of
    `bench.py --workload name` (or --decode-only): per-kernel dispatch
    statistics, the per-call sum, the algorithmic rate against 8 TB/s and 2.5
    PFLOP/s, and the committed traffic summary of the same workload."""
    import collections
    import csv
    import statistics
    from mamba_selective_ssm_amd import synth
    decode = name == "decode"
    kre = "decode_kernel" if decode else "scan_kernel"
    rows = [r for r in csv.DictReader(open(trace_csv)) if kre in r["Kernel_Name"]]
    by = collections.OrderedDict()
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append(r)
    w = synth.WORKLOADS[name]
    lines = ["# %s on workload %s" % (kre, name), ""]
    lines.append("Workload: batch %d, heads %d, seqlen %d, headdim %d, dstate %d, rank %d, %s I/O, "
                 "chunk %d%s" % (w.batch, w.heads, w.seqlen, w.headdim, w.dstate, w.rank, w.io_dtype,
                                 w.chunk, ", 256 decode steps" if decode else ""))
    lines += ["", "## Kernel trace", "", "Command (repo root, `TMPDIR=/tmp`):", ""]
    cmd = PROFILE_COMMANDS["trace_decode" if decode else "trace"].format(n=name)
    lines += ["    " + cmd, "    python bench.py --trace-summary %s gpurun_out/prof/trace_%s/t_kernel_trace.csv"
              % (name, name), ""]
    lines += ["| kernel | pass | dispatches | avg us | median us | min us | max us | arch VGPR | "
              "SGPR | grid | wg |", "|---|---|---|---|---|---|---|---|---|---|---|"]
    call_avg = call_med = 0.0
    durs_all = None
    for k, rs in by.items():
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs]
        role = ("decode step" if decode else
                "output (FULL)" if "EELb1E" in k else "state (no outputs)")
        lines.append("| `%s` | %s | %d | %.1f | %.1f | %.1f | %.1f | %s | %s | %s | %s |" % (
            k[:80], role, len(d), sum(d) / len(d), statistics.median(d), min(d), max(d),
            rs[0]["VGPR_Count"], rs[0]["SGPR_Count"], rs[0]["Grid_Size_X"], rs[0]["Workgroup_Size_X"]))
        call_avg += sum(d) / len(d)
        call_med += statistics.median(d)
        if durs_all is None or "EELb1E" in k:
            durs_all = d
    nbytes = decode_algorithmic_bytes(w) if decode else scan_algorithmic_bytes(w)
    lines += ["", "Per entry-point call (sum of its passes): average %.1f us, median %.1f us." % (
        call_avg, call_med)]
    lines.append("Algorithmic bytes per call: %d -> %.0f GB/s on the average (%.1f%% of 8 TB/s), "
                 "%.0f GB/s on the median." % (nbytes, nbytes / call_avg / 1e3,
                                               nbytes / call_avg / 1e3 / HBM_PEAK_GBS * 100,
                                               nbytes / call_med / 1e3))
    if not decode:
        fl = scan_dense_flops(w)
        lines.append("Dense-tile flops per call (chunk %d): %d -> %.1f TFLOP/s on the average "
                     "(%.1f%% of 2.5 PFLOP/s)." % (w.chunk, fl, fl / call_avg / 1e6,
                                                   fl / call_avg / 1e6 / BF16_PEAK_TFLOPS * 100))
    if durs_all and len(durs_all) <= 64:
        lines.append("Dispatch durations in launch order (us): %s -- the spread is the device clock "
                     "settling under sustained load, not the kernel." % [round(x) for x in durs_all])
    tpath = os.path.join(PROFILE_DIR, "%s_traffic.json" % name)
    if os.path.exists(tpath):
        t = json.load(open(tpath))
        pk = "pmc_decode" if decode else "pmc"
        lines += ["", "## HBM traffic (FETCH_SIZE / WRITE_SIZE)", "",
                  "Commands, each pass under `timeout -s KILL 120`:", ""]
        lines += ["    " + PROFILE_COMMANDS[pk].format(c=c, f=f, n=name)
                  for c, f in (("FETCH_SIZE", "f"), ("WRITE_SIZE", "w"))]
        lines += ["    " + PROFILE_COMMANDS["copy"].format(c=c, f=f)
                  for c, f in (("FETCH_SIZE", "f"), ("WRITE_SIZE", "w"))]
        lines += ["    python bench.py --traffic-summary %s gpurun_out/prof/f_%s/f_counter_collection.csv "
                  "gpurun_out/prof/w_%s/w_counter_collection.csv gpurun_out/prof/cf/f_counter_collection.csv "
                  "gpurun_out/prof/cw/w_counter_collection.csv" % (name, name, name), ""]
        lines += ["Copy calibration: a 1 GiB device-to-device copy reads FETCH_SIZE x %.4f and WRITE_SIZE x "
                  "%.4f of its true bytes; both counters are scaled by that." % (1 / t["fetch_scale"],
                                                                                  1 / t["write_scale"]), ""]
        lines += ["| per call | bytes |", "|---|---|",
                  "| fetched (scaled) | %d |" % t["fetch_bytes"], "| written (scaled) | %d |" % t["write_bytes"],
                  "| total | %d |" % t["bytes_per_launch"], "| algorithmic | %d |" % nbytes,
                  "| ratio | %.3f |" % (t["bytes_per_launch"] / nbytes), ""]
        lines.append("Kernel sources hash at measurement: `%s` (bench.py reports traffic only while the "
                     "sources match)." % t["source_hash"])
    out = os.path.join(PROFILE_DIR, "%s_%s.md" % (kre, name))
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(out)


# Device sources each measured kernel is compiled from.
KERNEL_SOURCES = {
    "scan": ["m3_device.hpp", "m3_timeline.hpp", "m3_scan_kernel.hpp", "m3_scan_inst.hpp", "m3_scan_f32.hip",
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


SETTLE_S = 0.15      # untimed run-in of every timed workload (seconds)


def time_launches(fn, steps, warmup, torch, settle_s=None):
    """Run fn() warmup + steps times; returns (total seconds, mean kernel ms).
    Two HIP events on the launch stream bracket the timed region, so the mean
    step duration is their span over the steps: the steps' kernels and the
    gaps between them, with no other work queued in between (an event record
    per step would add its own barrier to every step).
    Before the warm-up steps, fn() runs untimed for settle_s seconds (at most
    500 calls): after an idle spell the device clock first boosts, then drops
    under sustained load and recovers over some tens of calls (MIMO prefill
    dispatches ran 687, 705, 1004 us, easing to 742 and then 690 us), so the
    timed steps see the settled rate."""
    settle_s = SETTLE_S if settle_s is None else settle_s
    t_end = time.perf_counter() + settle_s
    n = 0
    while n < 500 and time.perf_counter() < t_end:
        for _ in range(5):
            fn()
        n += 5
        torch.cuda.synchronize()
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


def bench_prefill(w, steps, warmup, torch, m3, synth, seed=1001, inp=None):
    inp = synth.make_scan_inputs(w, seed, "cuda") if inp is None else inp
    # Arguments, outputs and workspace are prepared once; each step is one
    # m3_scan_fwd call on the same resident inputs.
    step = m3.ScanCall(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"],
                       inp["lam"], chunk=w.chunk)
    total, kms = time_launches(step, steps, warmup, torch)
    tokens = w.batch * w.seqlen
    nbytes = scan_algorithmic_bytes(w)
    flops = scan_dense_flops(w)
    return dict(tokens_per_s=tokens * steps / total, ms_per_step=1e3 * total / steps,
                kernel_ms=kms, bytes=nbytes, gbs=nbytes / (kms * 1e-3) / 1e9, flops=flops,
                tflops=flops / (kms * 1e-3) / 1e12, inputs=inp)


def roofline(r, name, kernel="m3::scan_kernel", flops=True):
    """Roofline object of one measured workload: algorithmic HBM bytes per
    call over the call's average span against 8 TB/s (the binding roof of
    every workload here), the committed HBM traffic counters when they match
    the current kernel sources, and -- for the prefill -- the dense-tile bf16
    flops against the 2.5 PFLOP/s matrix-core peak."""
    roof = {"bound": "hbm", "achieved": round(r["gbs"], 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(r["gbs"] / HBM_PEAK_GBS, 4),
            "traffic": load_traffic(name), "kernel": kernel,
            "kernel_ms": round(r["kernel_ms"], 5),
            "algorithmic_bytes_per_launch": r["bytes"]}
    if flops:
        roof["mfma"] = {"achieved": round(r["tflops"], 1), "peak": BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(r["tflops"] / BF16_PEAK_TFLOPS, 4),
                        "flops_per_launch": r["flops"]}
    return roof


def chunk_sweep(w, steps, warmup, torch, m3, synth, chunks=(32, 64, 128, 256), seed=1001):
    """A prefill workload at each chunk length (tokens): time per call, HBM
    and matrix-core fractions (the dense-tile flops grow with the chunk);
    chunk lengths outside the compiled set are listed as unsupported."""
    from mamba_selective_ssm_amd import M3_BF16
    inp = synth.make_scan_inputs(w, seed, "cuda")
    out = []
    for Q in chunks:
        wq = w.with_(chunk=Q)
        if not m3.m3_scan_supported(w.dstate, w.headdim, w.rank, Q, M3_BF16):
            out.append({"chunk": Q, "status": "unsupported"})
            continue
        r = bench_prefill(wq, steps, warmup, torch, m3, synth, inp=inp)
        out.append({"chunk": Q, "kernel_ms": round(r["kernel_ms"], 4),
                    "tokens_per_s": round(r["tokens_per_s"], 1),
                    "hbm_frac": round(r["gbs"] / HBM_PEAK_GBS, 4),
                    "mfma_frac": round(r["tflops"] / BF16_PEAK_TFLOPS, 4)})
    del inp
    torch.cuda.empty_cache()
    return out


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

    # (each step takes fresh inputs, so no run-in beyond the warm-up steps;
    # the 1024 timed steps span about 0.1 s)
    total, kms = time_launches(step, steps, warmup, torch, settle_s=0.0)
    nbytes = decode_algorithmic_bytes(w, premix=premix)
    return dict(steps_per_s=steps / total, tokens_per_s=w.batch * steps / total,
                ms_per_step=1e3 * total / steps, kernel_ms=kms, bytes=nbytes,
                gbs=nbytes / (kms * 1e-3) / 1e9)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, budget_s, torch):
    """The fp64 oracle on this host's cores over a bounded sample of the same
    inputs: whole batch rows (every head, every token), taken in turn until
    about budget_s seconds are spent, on all visible cores; then one
    (batch, head) unit on one thread for the single-thread rate.  Rates are tokens/s of the
    workload (a token is one sequence position of one batch row, all heads)."""
    import oracle
    from mamba_selective_ssm_amd.synth import to_f64_numpy
    keys = ("x", "B", "C", "dt", "A", "theta", "lam")
    threads = oracle.default_threads()
    rows, el = 0, 0.0
    while el < budget_s and rows < 64 * w.batch:
        b = rows % w.batch
        args = [to_f64_numpy(inp[k] if k == "A" else inp[k][b:b + 1]) for k in keys]
        t0 = time.perf_counter()
        oracle.scan(*args, threads=threads)
        el += time.perf_counter() - t0
        rows += 1
    one = [to_f64_numpy(inp[k][0:1] if k == "A" else inp[k][0:1, :, 0:1]) for k in keys]
    t0 = time.perf_counter()
    oracle.scan(*one, threads=1)
    el1 = time.perf_counter() - t0
    return {"value": rows * w.seqlen / el, "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "single_thread_tokens_per_s": w.seqlen / w.heads / el1,
            "sample": "%d batch rows of %s in turn (each %d tokens x %d heads; the workload has %d), "
                      "%.1f s on %d threads; single thread: one (batch, head) unit of %d tokens, %.1f s"
                      % (rows, w.name, w.seqlen, w.heads, w.batch, el, threads, w.seqlen, el1)}


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
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mimo_prefill_bf16")
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
    ap.add_argument("--row-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB as 128-byte rows gathered at a 4 KiB stride (the "
                         "prefill's per-head row reads), for a second counter calibration")
    ap.add_argument("--calibration-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "MIB"),
                    help="FETCH_SIZE / WRITE_SIZE scale factors of a --copy-calibration or "
                         "--row-calibration run of MIB MiB (no GPU needed)")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--trace-summary", nargs=2, metavar=("NAME", "TRACE_CSV"),
                    help="turn a rocprofv3 kernel-trace csv into profiles/<kernel>_NAME.md "
                         "(no GPU needed)")
    args = ap.parse_args(argv)

    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return 0

    if args.calibration_summary:
        fcsv, wcsv, mib = args.calibration_summary
        total = int(mib) * (1 << 20)
        res = {}
        for tag, path in (("fetch", fcsv), ("write", wcsv)):
            # the copy dispatches of the run (3 rounds of one large copy, or of
            # 32 row copies), not the fill that initialises the source
            rows = [v for _, k, v in _counter_rows(path)
                    if "copy" in k.lower() and "fill" not in k.lower()]
            per_round = sum(rows) / 3 * 1024 if rows else 0.0
            res[tag + "_kib_per_round"] = round(per_round / 1024, 1)
            res[tag + "_scale"] = round(total / per_round, 4) if per_round else None
        print(json.dumps(res))
        return 0

    if args.traffic_summary:
        name = args.traffic_summary[0]
        # one dispatch per call: the output pass (the first template flag
        # after the configuration, FULL, is true)
        regex, call = (("decode_kernel", "decode_kernel") if name == "decode"
                       else ("scan_kernel", "scan_kernelI.*EELb1E"))
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

    if args.row_calibration:
        # src [L, 32, 64] bf16: head h's rows are 128 bytes, 4 KiB apart (the
        # layout of x at 32 heads); each head's rows are copied to a
        # contiguous destination, so every byte is read and written once.
        L = args.row_calibration * (1 << 20) // (32 * 64 * 2)
        src = torch.ones(L, 32, 64, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty(32, L, 64, dtype=torch.bfloat16, device="cuda")
        for _ in range(3):
            for h in range(32):
                dst[h].copy_(src[:, h])
        torch.cuda.synchronize()
        print(json.dumps({"row_copy_bytes_each_way": L * 32 * 64 * 2, "launches": 3 * 32}))
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
    # The secondary workloads run first: the device clock settles under
    # sustained load (in a kernel trace the first MIMO dispatches after an
    # idle spell ran 687, 705, then 1004 us, easing to 742 us over twenty
    # calls), so the headline's warm-up and timed steps follow them.
    sec = None
    if not args.no_secondary:
        sec = {}
        nsec = max(args.steps, 20)
        for name in ("prefill_bf16", "long_prefill_bf16", "mimo_prefill_bf16"):
            if name == w.name:
                continue
            ws = synth.WORKLOADS[name]
            progress("timing %s" % name)
            rs = bench_prefill(ws, nsec, 3, torch, m3, synth)
            rs.pop("inputs")
            sec[name] = {"tokens_per_s": round(rs["tokens_per_s"], 1), "calls": nsec,
                         "roofline": roofline(rs, name)}
            torch.cuda.empty_cache()
        wl = synth.WORKLOADS["long_prefill_bf16"]
        progress("long_prefill_bf16 chunk sweep")
        sec.setdefault("long_prefill_bf16", {})["chunk_sweep"] = chunk_sweep(
            wl, nsec, 3, torch, m3, synth)
        wd = synth.WORKLOADS["decode"]
        progress("timing decode: prefill + %d steps" % args.decode_steps)
        rd = bench_decode(wd, args.decode_steps, 8, torch, m3, synth)
        sec["decode"] = {"steps_per_s": round(rd["steps_per_s"], 1),
                         "tokens_per_s": round(rd["tokens_per_s"], 1),
                         "calls": args.decode_steps,
                         "roofline": roofline(rd, "decode", kernel="m3::decode_kernel",
                                              flops=False)}
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
            ro = bench_prefill_options(wp, opts, nsec, 3, torch, m3, synth)
            sec[name] = {"tokens_per_s": round(ro["tokens_per_s"], 1),
                         "kernel_ms": round(ro["kernel_ms"], 5),
                         "hbm_gbs": round(ro["gbs"], 1),
                         "hbm_frac": round(ro["gbs"] / HBM_PEAK_GBS, 4)}
        sec.update(backward_lines(args.steps, torch, m3, synth))
        torch.cuda.empty_cache()
        # the MIMO prefill at 32, 64 (the library's default) and 128 operand
        # rows per chunk (chunks of 8, 16 and 32 tokens at rank 4)
        wm = synth.WORKLOADS["mimo_prefill_bf16"]
        progress("mimo_prefill_bf16 chunk sweep")
        sec.setdefault("mimo_prefill_bf16", {})["chunk_sweep"] = chunk_sweep(
            wm, nsec, 3, torch, m3, synth, chunks=(8, 16, 32))

    progress("timing %s: %d warmup + %d steps" % (w.name, args.warmup, args.steps))
    r = bench_prefill(w, args.steps, args.warmup, torch, m3, synth)
    out = {"metric": METRIC, "value": round(r["tokens_per_s"], 1), "unit": "tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_s": SETTLE_S,
           "ms_per_step": round(r["ms_per_step"], 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": w.io_dtype, "data": "synthetic",
           "config": {"workload": w.name, "batch": w.batch, "heads": w.heads,
                      "seqlen": w.seqlen, "headdim": w.headdim, "dstate": w.dstate,
                      "rank": w.rank, "chunk": w.chunk, "state": "fp32",
                      "accumulate": "fp32"},
           "roofline": roofline(r, w.name)}
    inp = r.pop("inputs")
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle on the headline's own inputs, before they are freed
        progress("timing the fp64 oracle on the host")
        cpu = cpu_baseline(w, inp, args.cpu_budget, torch)
    del inp
    torch.cuda.empty_cache()

    if sec is not None:
        out["secondary"] = sec
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
