"""Parity at the measured workloads' full sizes, in the launch configuration
bench.py times (library defaults for chunk, headdim split and segments).

Every (batch, head) unit is checked against the fp64 oracle, which is run in
pieces (a batch row or a group of heads at a time) to bound host memory.
Metric per tensor: max |gpu - oracle| / max |oracle| <= 2e-2 (bf16 I/O); the
state record's (B_prev, x_prev) must match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from mamba_selective_ssm_amd import M3_BF16, m3_decode_step, m3_scan_fwd, m3_scan_supported, synth
from helpers import TOL, f64, rel_err, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda"
KEYS = ("x", "B", "C", "dt", "A", "theta", "lam")


def oracle_piece(inp, bsel, hsel, state=None):
    """Oracle on batch rows bsel and heads hsel (slices) of a scan input."""
    sub = [f64(inp[k][hsel] if k == "A" else inp[k][bsel, :, hsel]) for k in KEYS]
    kw = {}
    if state is not None:
        kw = dict(h0=state[0], Bprev=state[1], xprev=state[2])
    return oracle.scan(*sub, **kw)


def check_every_unit(w, inp, y, st, pieces):
    """Compare y and the state record with the oracle piece by piece; returns
    the worst relative errors of y and h over all pieces."""
    ey = eh = 0.0
    for bsel, hsel in pieces:
        yr, hr, br, xr = oracle_piece(inp, bsel, hsel)
        ey = max(ey, rel_err(f64(y[bsel, :, hsel]), yr))
        eh = max(eh, rel_err(f64(st.h[bsel, hsel]), hr))
        np.testing.assert_array_equal(f64(st.B_prev[bsel, hsel]), br)
        np.testing.assert_array_equal(f64(st.x_prev[bsel, hsel]), xr)
    return ey, eh


def run_workload(name, seed, pieces, chunk=None):
    w = synth.WORKLOADS[name]
    say("case %s full size, every unit: %s" % (name, w))
    inp = synth.make_scan_inputs(w, seed, DEV)
    y, st = m3_scan_fwd(*[inp[k] for k in KEYS], chunk=chunk or w.chunk)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    ey, eh = check_every_unit(w, inp, y, st, pieces(w))
    say("   rel err over all %d units: y %.3e  state %.3e" % (w.batch * w.heads, ey, eh))
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def by_batch_row(w):
    return [(slice(b, b + 1), slice(None)) for b in range(w.batch)]


def by_head_group(w, size=16):
    return [(slice(None), slice(h, h + size)) for h in range(0, w.heads, size)]


def test_prefill_bf16_full_every_unit():
    """batch 4, 16 heads, L=2048, P=64, N=64, R=1."""
    run_workload("prefill_bf16", 2001, by_batch_row)


@pytest.mark.parametrize("chunk", [16, 32])
def test_mimo_prefill_bf16_full_every_unit(chunk):
    """batch 8, 32 heads, L=4096, P=64, N=128, R=4: all 256 units, at the
    benchmark's chunk (16 tokens, 64 operand rows) and at 32 (128 rows)."""
    run_workload("mimo_prefill_bf16", 2002, by_batch_row, chunk=chunk)


def test_long_prefill_bf16_every_unit_at_each_chunk():
    """batch 1, 32 heads, L=65536, P=64, N=128, R=1 (slow decay): y and the
    final state of every head at every compiled chunk length of the sweep
    (the oracle, which does not chunk, runs once)."""
    w = synth.WORKLOADS["long_prefill_bf16"]
    chunks = [q for q in (32, 64, 128, 256)
              if m3_scan_supported(w.dstate, w.headdim, w.rank, q, M3_BF16)]
    say("case long_prefill_bf16 full size, every unit, chunks %s" % chunks)
    assert 64 in chunks
    inp = synth.make_scan_inputs(w, 2003, DEV)
    outs = {}
    for q in chunks:
        y, st = m3_scan_fwd(*[inp[k] for k in KEYS], chunk=q)
        torch.cuda.synchronize()
        assert torch.isfinite(y).all()
        outs[q] = (y, st)
    worst = {q: [0.0, 0.0] for q in chunks}
    for bsel, hsel in by_head_group(w):
        yr, hr, br, xr = oracle_piece(inp, bsel, hsel)
        for q, (y, st) in outs.items():
            worst[q][0] = max(worst[q][0], rel_err(f64(y[bsel, :, hsel]), yr))
            worst[q][1] = max(worst[q][1], rel_err(f64(st.h[bsel, hsel]), hr))
            np.testing.assert_array_equal(f64(st.B_prev[bsel, hsel]), br)
            np.testing.assert_array_equal(f64(st.x_prev[bsel, hsel]), xr)
    for q in chunks:
        say("   chunk %d: rel err y %.3e  state %.3e" % (q, *worst[q]))
        assert worst[q][0] <= TOL["bf16"] and worst[q][1] <= TOL["bf16"], q


def test_decode_workload_256_units_every_step():
    """batch 256, 32 heads, P=64, N=128, R=4: a 1024-token prefill, then 1024
    decode steps with fresh inputs.  256 units (batch rows 0..7, every head)
    are checked against the oracle: the prefill's y and record; then y at
    every step and the whole state every 64 steps.  The oracle advances those
    units through the decode steps as a scan over the step inputs from the
    prefill's record (a scan is the step applied token by token, the same
    arithmetic as its decode step).  The record of every unit (all 8192) must
    hold the step's B and x bit for bit after every step."""
    w = synth.WORKLOADS["decode"]
    nb, blk = 8, 64
    bs = slice(0, nb)
    say("case decode full: %s; units: batch rows 0..%d x %d heads" % (w, nb - 1, w.heads))
    pre = synth.make_scan_inputs(w, 2004, DEV)
    ypre, st = m3_scan_fwd(*[pre[k] for k in KEYS], chunk=w.chunk)
    torch.cuda.synchronize()
    A = pre["A"]
    yr, hr, br, xr = oracle_piece(pre, bs, slice(None))
    ey, eh = rel_err(f64(ypre[bs]), yr), rel_err(f64(st.h[bs]), hr)
    say("   prefill: rel err y %.3e  state %.3e" % (ey, eh))
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
    np.testing.assert_array_equal(f64(st.B_prev[bs]), br)
    np.testing.assert_array_equal(f64(st.x_prev[bs]), xr)
    ref = (hr, br, xr)
    del pre, ypre
    worst_y = worst_h = 0.0
    for b0 in range(0, w.decode_steps, blk):
        ys, steps = [], []
        for step in range(b0, b0 + blk):
            s = synth.make_decode_inputs(w, 2004, step, A, DEV)
            y = m3_decode_step(*[s[k] for k in KEYS], st)
            assert torch.equal(st.B_prev, s["B"]) and torch.equal(st.x_prev, s["x"]), step
            ys.append(y[bs].clone())
            steps.append({k: (s[k] if k == "A" else s[k][bs].unsqueeze(1)) for k in KEYS})
        torch.cuda.synchronize()
        seq = {k: (A if k == "A" else torch.cat([t[k] for t in steps], 1)) for k in KEYS}
        yr, hr, br, xr = oracle.scan(*[f64(seq[k]) for k in KEYS], h0=ref[0], Bprev=ref[1],
                                     xprev=ref[2])
        got = torch.stack(ys, 1)
        worst_y = max(worst_y, rel_err(f64(got), yr))
        worst_h = max(worst_h, rel_err(f64(st.h[bs]), hr))
        np.testing.assert_array_equal(f64(st.B_prev[bs]), br)
        ref = (hr, br, xr)
        if b0 % 256 == 256 - blk:
            say("   step %d: worst rel err so far y %.3e state %.3e" % (b0 + blk - 1, worst_y,
                                                                        worst_h))
    assert worst_y <= TOL["bf16"] and worst_h <= TOL["bf16"]
