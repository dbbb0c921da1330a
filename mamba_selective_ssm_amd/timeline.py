"""Per-wave phase timeline of the fused chunked prefill and of the chunked
gradient's main kernel (instrumented library).

    python -m mamba_selective_ssm_amd.build --timeline
    python -m mamba_selective_ssm_amd.timeline [--workload prefill_bf16] [--calls 20] [--premix]
    python -m mamba_selective_ssm_amd.timeline --backward [--workload prefill_bf16]

Loads libm3scan_timeline.so -- the library built with M3_TIMELINE=1, whose
scan kernels stamp every wave's phase boundaries with s_memtime -- in place of
libm3scan.so, runs m3_scan_fwd on the workload `calls` times (inputs resident
in HBM), keeps the stamps of the last call and prints a markdown summary: for
each pass (state, output) and wave role (operand prep, matrix core), the
prologue's milestones from the workgroup's start and the steady-state phases
of one chunk (median over waves and chunks, in microseconds).  The stamps add
a little time of their own (one scalar clock read and one store per event).
"""
from __future__ import annotations

import argparse
import ctypes
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

SLOTS = 256            # 64-bit entries per wave (kTlSlots in the kernel)
REALTIME_MHZ = 100.0   # s_memrealtime's constant clock

EV = {5: "set-up done (workgroup barrier passed)", 1: "first loads issued", 2: "first angle/decay inputs in", 3: "first chunk prepared",
      4: "prologue barrier passed", 10: "prep start", 11: "angle totals published",
      12: "decay scan (A0)", 13: "X rows", 14: "wait for the other waves' totals",
      15: "rotation of B, C + next loads", 16: "chunk barrier", 20: "record fold / initial state",
      17: "angle inputs in hand (the wait for this chunk's loads)", 18: "angle scan across the wave's lanes",
      21: "state staged", 22: "phase C (outputs)", 23: "phase D (state update)",
      24: "state staged for the next chunk", 30: "exit"}
PREP_STEPS = [(10, 17), (17, 18), (18, 11), (11, 12), (12, 13), (13, 14), (14, 15), (15, 16)]
MATH_STEPS = [(16, 22), (22, 23), (23, 24), (24, 16)]      # output pass
MATH_STEPS_STATE = [(16, 23), (23, 16)]                    # state pass: no outputs
BWD_STEPS = [(40, 41, "staging (inputs in, rotation into LDS)"), (41, 42, "phase 1: S, dS tiles"),
             (42, 43, "phase 2a: dX"), (43, 44, "phase 2b: dBbar products"),
             (44, 49, "phase 2b: angle terms, back-rotation and stores of dB"),
             (49, 50, "phase 2c: dCbar products"),
             (50, 45, "phase 2c: back-rotation and stores of dC, barrier"), (45, 46, "phase 3a: angle suffix sums"),
             (46, 47, "phase 3b: dtheta"), (47, 48, "phase 3c: decay and weight gradients (wave 0)")]
BACKWARD_BIT = 1 << 61


def parse(rows):
    """rows: list of SLOTS-long lists of ints (waves that ran).  Returns dicts
    with the wave's header and its events as (code, ticks from entry)."""
    waves = []
    for r in rows:
        if r[0] == 0:
            continue
        hdr = r[2]
        t0 = r[1]
        ev = []
        for v in r[3:SLOTS - 2]:
            code = v >> 56
            if code == 0:
                break
            if code == 30:
                break
            ev.append((code, (v & ((1 << 56) - 1)) - t0))
        rt_span = r[SLOTS - 1] - r[0]
        tk_span = r[SLOTS - 2] - t0
        waves.append(dict(full=bool(hdr >> 63), math=bool((hdr >> 62) & 1), wv=(hdr >> 48) & 0xff,
                          bwd=bool(hdr & BACKWARD_BIT),
                          seg=(hdr >> 32) & 0xffff, unit=hdr & 0xffffffff, rt0=r[0], ev=ev,
                          rt_span=rt_span, tk_span=tk_span))
    return waves


def summarize(waves, name):
    # s_memtime ticks per microsecond, from the waves' own entry/exit pairs
    rates = [w["tk_span"] / (w["rt_span"] / REALTIME_MHZ) for w in waves if w["rt_span"] > 0]
    tpu = statistics.median(rates)
    out = ["# Per-wave timeline of scan_kernel on workload %s" % name, ""]
    out.append("s_memtime runs at %.0f ticks per us here (median over waves, against s_memrealtime's "
               "100 MHz)." % tpu)
    out.append("")
    for full in (False, True):
        pw = [w for w in waves if w["full"] == full and not w["bwd"]]
        if not pw:
            continue
        start = min(w["rt0"] for w in pw)
        end = max(w["rt0"] + w["rt_span"] for w in pw)
        life = [w["rt_span"] / REALTIME_MHZ for w in pw]
        starts = [(w["rt0"] - start) / REALTIME_MHZ for w in pw]
        out.append("## %s pass" % ("output" if full else "state"))
        out.append("")
        out.append("%d waves; pass span %.1f us (first wave start to last wave exit); waves start "
                   "within %.2f us of each other; wave lifetime median %.1f us." % (
                       len(pw), (end - start) / REALTIME_MHZ, max(starts), statistics.median(life)))
        out.append("")
        for math in (False, True):
            rw = [w for w in pw if w["math"] == math]
            if not rw:
                continue
            role = "matrix-core waves" if math else "prep waves"
            out.append("**%s** (%d): prologue milestones, us from the wave's start (median):" % (role, len(rw)))
            out.append("")
            out.append("| milestone | median us |")
            out.append("|---|---|")
            codes = (5, 1, 2, 3, 4) if not math else (5, 20, 21, 4)
            for c in codes:
                # milestones up to the prologue barrier (event 4)
                ts = []
                for w in rw:
                    for cc, t in w["ev"]:
                        if cc == c:
                            ts.append(t)
                            break
                        if cc == 4:
                            break
                if ts:
                    out.append("| %s | %.2f |" % (EV[c], statistics.median(ts) / tpu))
            out.append("")
            steps = (MATH_STEPS if full else MATH_STEPS_STATE) if math else PREP_STEPS
            out.append("steady state, per chunk (events after the prologue barrier):")
            out.append("")
            out.append("| phase | median us | mean us | samples |")
            out.append("|---|---|---|---|")
            tot = 0.0
            for a, b in steps:
                ds = []
                for w in rw:
                    ev = w["ev"]
                    k0 = next((i for i, (c, _) in enumerate(ev) if c == 4), None)
                    if k0 is None:
                        continue
                    for i in range(k0, len(ev) - 1):
                        if ev[i][0] == a and ev[i + 1][0] == b:
                            ds.append((ev[i + 1][1] - ev[i][1]) / tpu)
                        elif math and a == 16 and ev[i][0] == 4 and ev[i + 1][0] == b:
                            ds.append((ev[i + 1][1] - ev[i][1]) / tpu)
                if ds:
                    tot += statistics.mean(ds)
                    label = "wait at the chunk barrier" if b == 16 else EV[b]
                    out.append("| %s | %.2f | %.2f | %d |" % (label, statistics.median(ds),
                                                              statistics.mean(ds), len(ds)))
            out.append("| sum of means | | %.2f | |" % tot)
            out.append("")
            # by wave index: the barrier wait and the work before it, per chunk
            per = {}
            for w in rw:
                ev = w["ev"]
                k0 = next((i for i, (c, _) in enumerate(ev) if c == 4), None)
                if k0 is None:
                    continue
                marks = [t for (c, t) in ev[k0:] if c in (4, 16)]
                last = [t for (c, t) in ev[k0:] if c == (15 if not math else (24 if full else 23))]
                d = per.setdefault(w["wv"], [[], []])
                for i in range(len(marks) - 1):
                    ends = [t for t in last if marks[i] < t < marks[i + 1]]
                    if ends:
                        d[0].append((ends[-1] - marks[i]) / tpu)
                        d[1].append((marks[i + 1] - ends[-1]) / tpu)
            if per:
                out.append("by wave index: work before the chunk barrier / wait at it (mean us per chunk): " +
                           ", ".join("w%d %.2f/%.2f" % (k, statistics.mean(v[0]), statistics.mean(v[1]))
                                     for k, v in sorted(per.items()) if v[0]))
                out.append("")
    return "\n".join(out)


def summarize_backward(waves, name):
    """bc_grad_kernel rows: per unit (one chunk of one (b, h)), the phases
    between its barriers, over all waves and the units they stamped."""
    waves = [w for w in waves if w["bwd"]]
    rates = [w["tk_span"] / (w["rt_span"] / REALTIME_MHZ) for w in waves if w["rt_span"] > 0]
    tpu = statistics.median(rates)
    start = min(w["rt0"] for w in waves)
    end = max(w["rt0"] + w["rt_span"] for w in waves)
    out = ["# Per-wave timeline of bc_grad_kernel (chunked gradient) on workload %s" % name, ""]
    out.append("s_memtime runs at %.0f ticks per us here (median over waves, against s_memrealtime's "
               "100 MHz)." % tpu)
    out.append("")
    out.append("%d waves of a persistent grid; kernel span %.1f us; wave lifetime median %.1f us." % (
        len(waves), (end - start) / REALTIME_MHZ, statistics.median(w["rt_span"] / REALTIME_MHZ for w in waves)))
    out.append("")
    out.append("Per unit (one 64-row chunk), between the kernel's barriers:")
    out.append("")
    out.append("| phase | median us | mean us | samples |")
    out.append("|---|---|---|---|")
    tot = 0.0
    for a, b, label in BWD_STEPS:
        ds = []
        for w in waves:
            ev = w["ev"]
            for i in range(len(ev) - 1):
                if ev[i][0] == a and ev[i + 1][0] == b:
                    ds.append((ev[i + 1][1] - ev[i][1]) / tpu)
        if ds:
            tot += statistics.mean(ds)
            out.append("| %s | %.2f | %.2f | %d |" % (label, statistics.median(ds), statistics.mean(ds), len(ds)))
    out.append("| sum of means (one unit) | | %.2f | |" % tot)
    out.append("")
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="prefill_bf16")
    ap.add_argument("--calls", type=int, default=20)
    ap.add_argument("--seed", type=int, default=7)
    ap.add_argument("--premix", action="store_true", help="with the fused pre-mixer")
    ap.add_argument("--backward", action="store_true", help="the chunked gradient (m3_scan_bwd)")
    ap.add_argument("--raw", default=None, help="also save the stamped rows (uint64, one per wave) to this .npy file")
    args = ap.parse_args(argv)

    import torch
    from mamba_selective_ssm_amd import binding, build, synth
    if not os.path.exists(build.LIB_TIMELINE):
        raise RuntimeError("libm3scan_timeline.so is not built; run "
                           "`python -m mamba_selective_ssm_amd.build --timeline`")
    binding.LIB_PATH = build.LIB_TIMELINE
    lib = binding.load_library()
    lib.m3_timeline_buffer.restype = None
    lib.m3_timeline_buffer.argtypes = [ctypes.c_void_p, ctypes.c_int64]

    w = synth.WORKLOADS[args.workload]
    keys = ("x", "B", "C", "dt", "A", "theta", "lam")
    pm = None
    if args.premix:
        inp, ex = synth.make_option_inputs(w, args.seed, "cuda", premix=True)
        q = ex["premix"]
        pm = binding.Premix(q["B_norm_w"], q["C_norm_w"], q["B_bias"], q["C_bias"], q["dt_bias"], q["eps"])
    else:
        inp = synth.make_scan_inputs(w, args.seed, "cuda")
    nrows = 32768                       # waves of both passes (a call needing more is not stamped)
    buf = torch.zeros(nrows * SLOTS, dtype=torch.int64, device="cuda")
    if args.backward:
        gen = torch.Generator(device="cuda").manual_seed(args.seed + 1)
        dy = torch.randn(inp["x"].shape, generator=gen, device="cuda").to(inp["x"].dtype)
        call = binding.ScanBwdCall(*[inp[k] for k in keys], dy, method="chunked")
    else:
        call = binding.ScanCall(*[inp[k] for k in keys], chunk=w.chunk, premix=pm)
    lib.m3_timeline_buffer(ctypes.c_void_p(buf.data_ptr()), nrows)
    for _ in range(args.calls - 1):
        call()
    torch.cuda.synchronize()
    buf.zero_()
    torch.cuda.synchronize()
    call()
    torch.cuda.synchronize()
    lib.m3_timeline_buffer(None, 0)
    rows = buf.view(nrows, SLOTS).cpu().tolist()
    mask = (1 << 64) - 1
    rows = [[v & mask for v in r] for r in rows]
    if args.raw:
        import numpy as np
        np.save(args.raw, np.array([r for r in rows if r[0] != 0], dtype=np.uint64))
    if args.backward:
        print(summarize_backward(parse(rows), w.name))
    else:
        print(summarize(parse(rows), w.name + (" with the pre-mixer" if pm is not None else "")))
    return 0


if __name__ == "__main__":
    sys.exit(main())
