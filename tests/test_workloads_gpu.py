"""Parity at the measured workloads' full sizes, in the launch configuration
bench.py times (library defaults for chunk, headdim split and segments).

The GPU computes every (batch, head); the fp64 oracle checks a sample of
(batch, head) units whole (all tokens, all ranks, all columns) -- each unit is
independent, so a sampled unit is checked exactly.  Metric per tensor sample:
max |gpu - oracle| / max |oracle| <= 2e-2 (bf16 I/O).
"""
import numpy as np
import pytest
import torch

import oracle
from mamba_selective_ssm_amd import m3_decode_step, m3_scan_fwd, synth
from helpers import TOL, f64, rel_err, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda"


def oracle_units(inp, units, threads=None):
    """Oracle on each sampled unit (own head's A); returns stacked results."""
    ys, hs, bs, xs = [], [], [], []
    for b, h in units:
        sub = {k: (inp[k][h:h + 1] if k == "A" else inp[k][b:b + 1, :, h:h + 1]) for k in inp}
        y, hL, bL, xL = oracle.scan(*[f64(sub[k]) for k in ("x", "B", "C", "dt", "A", "theta", "lam")],
                                    threads=threads)
        ys.append(y); hs.append(hL); bs.append(bL); xs.append(xL)
    return ys, hs, bs, xs


def run_and_check(name, units, seed):
    w = synth.WORKLOADS[name]
    say("case %s full size: %s; sampled units %s" % (name, w, units))
    inp = synth.make_scan_inputs(w, seed, DEV)
    y, st = m3_scan_fwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"],
                        inp["lam"], chunk=w.chunk)
    torch.cuda.synchronize()
    ys, hs, bs, xs = oracle_units(inp, units)
    ey = max(rel_err(f64(y[b:b + 1, :, h:h + 1]), yr) for (b, h), yr in zip(units, ys))
    eh = max(rel_err(f64(st.h[b:b + 1, h:h + 1]), hr) for (b, h), hr in zip(units, hs))
    say("   max rel err over samples: y %.3e  state %.3e" % (ey, eh))
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
    for (b, h), br, xr in zip(units, bs, xs):
        np.testing.assert_array_equal(f64(st.B_prev[b:b + 1, h:h + 1]), br)
        np.testing.assert_array_equal(f64(st.x_prev[b:b + 1, h:h + 1]), xr)
    assert torch.isfinite(y).all()
    return inp, y, st


def test_prefill_bf16_full_every_head():
    """batch 4, 16 heads, L=2048, P=64, N=64, R=1: every (b, h) checked."""
    w = synth.WORKLOADS["prefill_bf16"]
    units = [(b, h) for b in range(w.batch) for h in range(w.heads)]
    say("case prefill_bf16 full: %s" % (w,))
    inp = synth.make_scan_inputs(w, 2001, DEV)
    y, st = m3_scan_fwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"],
                        inp["lam"], chunk=w.chunk)
    torch.cuda.synchronize()
    yr, hr, br, xr = oracle.scan(*[f64(inp[k]) for k in ("x", "B", "C", "dt", "A", "theta", "lam")])
    ey, eh = rel_err(f64(y), yr), rel_err(f64(st.h), hr)
    say("   rel err y %.3e  state %.3e (%d units)" % (ey, eh, len(units)))
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
    np.testing.assert_array_equal(f64(st.B_prev), br)
    np.testing.assert_array_equal(f64(st.x_prev), xr)


def test_mimo_prefill_bf16_full_sampled():
    """batch 8, 32 heads, L=4096, P=64, N=128, R=4."""
    run_and_check("mimo_prefill_bf16", [(0, 0), (3, 17), (5, 9), (7, 31)], 2002)


def test_long_prefill_bf16_full_sampled():
    """batch 1, 32 heads, L=65536, P=64, N=128, R=1 (slow decay)."""
    run_and_check("long_prefill_bf16", [(0, 0), (0, 13), (0, 31)], 2003)


def test_decode_workload_full_sampled():
    """batch 256, 32 heads, P=64, N=128, R=4: 1024-token prefill, then 1024
    decode steps with fresh inputs each step; sampled units checked at every
    step against the oracle's decode step from the oracle's own prefill."""
    w = synth.WORKLOADS["decode"]
    units = [(0, 0), (101, 7), (255, 31)]
    say("case decode full: %s; sampled units %s" % (w, units))
    pre = synth.make_scan_inputs(w, 2004, DEV)
    _, st = m3_scan_fwd(pre["x"], pre["B"], pre["C"], pre["dt"], pre["A"], pre["theta"],
                        pre["lam"], chunk=w.chunk)
    A = pre["A"]
    _, hs, bs, xs = oracle_units(pre, units)
    ref = [(h, b, x) for h, b, x in zip(hs, bs, xs)]
    del pre
    torch.cuda.synchronize()
    worst_y = worst_h = 0.0
    for step in range(w.decode_steps):
        s = synth.make_decode_inputs(w, 2004, step, A, DEV)
        y = m3_decode_step(s["x"], s["B"], s["C"], s["dt"], s["A"], s["theta"], s["lam"], st)
        torch.cuda.synchronize()
        # advance the oracle for the sampled units every step
        for i, (b, h) in enumerate(units):
            sub = {k: (s[k][h:h + 1] if k == "A" else s[k][b:b + 1, h:h + 1]) for k in s}
            yr, hr, br, xr = oracle.decode_step(*[f64(sub[k]) for k in
                                                  ("x", "B", "C", "dt", "A", "theta", "lam")],
                                                *ref[i])
            ref[i] = (hr, br, xr)
            if step % 64 == 63 or step == 0:
                worst_y = max(worst_y, rel_err(f64(y[b:b + 1, h:h + 1]), yr))
                worst_h = max(worst_h, rel_err(f64(st.h[b:b + 1, h:h + 1]), hr))
        if step % 256 == 255:
            say("   step %d: worst rel err so far y %.3e state %.3e" % (step, worst_y, worst_h))
    assert worst_y <= TOL["bf16"] and worst_h <= TOL["bf16"]
