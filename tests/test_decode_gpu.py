"""Parity of the HIP decode step (m3_decode_step) against the fp64 oracle, and
prefill-then-decode == one scan."""
import numpy as np
import pytest
import torch

import oracle
from mamba_selective_ssm_amd import State, m3_decode_step, m3_scan_fwd, synth
from helpers import TOL, f64, oracle_scan, random_state, rel_err, say, workload

pytestmark = pytest.mark.gpu
DEV = "cuda"


def step_inputs(inp, t):
    return {k: (v if k == "A" else v[:, t].contiguous()) for k, v in inp.items()}


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N,P,R", [(128, 64, 4), (64, 64, 1), (16, 16, 2), (32, 128, 1)])
def test_decode_steps_match_oracle(io, N, P, R):
    w = workload(3, 6, 5, R, P, N, io=io, dt_mu=0.0, theta="uniform_pi")
    say("case decode: %s" % (w,))
    inp = synth.make_scan_inputs(w, 40 + N + R, DEV)
    h, Bp, xp = random_state(w, 41, DEV)
    st = State(h.clone(), Bp.clone(), xp.clone())
    ref = (f64(h), f64(Bp), f64(xp))
    for t in range(w.seqlen):
        s = step_inputs(inp, t)
        y = m3_decode_step(s["x"], s["B"], s["C"], s["dt"], s["A"], s["theta"], s["lam"], st)
        torch.cuda.synchronize()
        yr, hr, br, xr = oracle.decode_step(f64(s["x"]), f64(s["B"]), f64(s["C"]), f64(s["dt"]),
                                            f64(s["A"]), f64(s["theta"]), f64(s["lam"]), *ref)
        ref = (hr, br, xr)
        ey, eh = rel_err(f64(y), yr), rel_err(f64(st.h), hr)
        say("   step %d rel err y %.3e state %.3e" % (t, ey, eh))
        assert ey <= TOL[io] and eh <= TOL[io]
        np.testing.assert_array_equal(f64(st.B_prev), br)
        np.testing.assert_array_equal(f64(st.x_prev), xr)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_then_decode_equals_full_scan(io):
    w = workload(2, 200, 4, 4, 64, 128, io=io, chunk=16)
    say("case prefill+decode: %s" % (w,))
    inp = synth.make_scan_inputs(w, 91, DEV)
    y_full, s_full = m3_scan_fwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"],
                                 inp["theta"], inp["lam"])
    L1 = 150
    part = {k: (v if k == "A" else v[:, :L1].contiguous()) for k, v in inp.items()}
    y1, st = m3_scan_fwd(part["x"], part["B"], part["C"], part["dt"], part["A"],
                         part["theta"], part["lam"])
    ys = [y1]
    for t in range(L1, w.seqlen):
        s = step_inputs(inp, t)
        ys.append(m3_decode_step(s["x"], s["B"], s["C"], s["dt"], s["A"], s["theta"],
                                 s["lam"], st).unsqueeze(1).clone())
    torch.cuda.synchronize()
    y_mix = torch.cat(ys, 1)
    yr, hr, _, _ = oracle_scan(inp)
    tol = TOL[io]
    assert rel_err(f64(y_mix), yr) <= tol
    assert rel_err(f64(st.h), hr) <= tol
    assert rel_err(f64(y_mix), f64(y_full)) <= tol
    assert rel_err(f64(st.h), f64(s_full.h)) <= tol
