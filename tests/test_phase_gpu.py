"""Parity of the accumulated rotation angle (phase_in / phase_out of both
entry points) and of the decode step with the rotation removed from writing,
readout or both, against the fp64 oracle (oracle.accumulated_phase,
oracle.decode_step_rotation_removed).

Angles are compared modulo 2 pi: |wrap(got - ref)| <= 1e-5 rad (the library
sums dt theta in float64 from the same float32 inputs).  y and the state:
max |got - ref| / max |ref| <= 1e-4 for float32 I/O, <= 2e-2 for bfloat16.
"""
import numpy as np
import pytest
import torch

import oracle
from mamba_selective_ssm_amd import Premix, State, m3_decode_step, m3_scan_fwd, synth
from helpers import TOL, f64, random_state, rel_err, say, workload

pytestmark = pytest.mark.gpu
DEV = "cuda"
ANGLE_TOL = 1e-5


def angle_err(got, ref):
    return float(np.max(np.abs(oracle.wrap_angle(f64(got) - ref)))) if ref.size else 0.0


def effective_dt_theta(inp, ex, phase, premix):
    """dt and theta as the recurrence uses them (the oracle's transforms)."""
    dt = f64(inp["dt"])
    if premix:
        dt = oracle.premix_dt_lam(dt, f64(inp["lam"]), f64(ex["premix"]["dt_bias"]))[0]
    theta = oracle.phase_transform(f64(inp["theta"]), phase,
                                   ex["perm"].cpu().numpy() if "perm" in ex else None)
    return dt, theta


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("phase,premix", [("native", False), ("zero", False), ("reverse", False),
                                          ("shuffle", False), ("native", True)])
def test_scan_accumulated_phase(io, phase, premix):
    """phase_out of a scan (several 64-token blocks and a ragged tail) from a
    random phase_in, y unchanged by asking for it."""
    w = workload(2, 150, 3, 2, 32, 64, io=io, dt_mu=-1.0, theta="uniform_pi")
    seed = 700 + len(phase) + 3 * premix
    say("case scan phase_out %s phase=%s premix=%s seed=%d" % (io, phase, premix, seed))
    inp, ex = synth.make_option_inputs(w, seed, DEV, phase=phase, premix=premix)
    pm = ex.get("premix")
    pmo = Premix(pm["B_norm_w"], pm["C_norm_w"], pm["B_bias"], pm["C_bias"], pm["dt_bias"],
                 pm["eps"]) if pm else None
    g = torch.Generator(device=DEV).manual_seed(seed)
    ph_in = (torch.rand((w.batch, w.heads, w.dstate // 2), generator=g, device=DEV) * 2 - 1) * np.pi
    ph_out = torch.empty_like(ph_in)
    theta = None if phase == "zero" else inp["theta"]
    kw = dict(phase=phase, perm=ex.get("perm"), premix=pmo)
    y1, _ = m3_scan_fwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], theta, inp["lam"],
                        phase_in=ph_in, phase_out=ph_out, **kw)
    y0, _ = m3_scan_fwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], theta, inp["lam"], **kw)
    torch.cuda.synchronize()
    dt, th = effective_dt_theta(inp, ex, phase, premix)
    ref = oracle.accumulated_phase(dt, th, f64(ph_in))
    e = angle_err(ph_out, ref)
    say("   angle err %.2e (tol %.0e)" % (e, ANGLE_TOL))
    assert e <= ANGLE_TOL, e
    assert torch.equal(y0, y1)


def test_scan_accumulated_phase_packed_and_in_place():
    """Packed sequences: one angle per sequence; phase_in and phase_out the
    same tensor (updated in place); an empty sequence keeps its angle."""
    w = workload(1, 230, 2, 1, 32, 32, io="f32", dt_mu=-1.0, theta="uniform_pi")
    inp = synth.make_scan_inputs(w, 720, DEV)
    cu = torch.tensor([0, 70, 70, 161, 230], dtype=torch.int32, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(721)
    ph = (torch.rand((4, w.heads, w.dstate // 2), generator=g, device=DEV) * 2 - 1) * np.pi
    ph0 = f64(ph)
    say("case scan phase_out packed, in place")
    m3_scan_fwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"], inp["lam"],
                cu_seqlens=cu, max_seqlen=91, phase_in=ph, phase_out=ph)
    torch.cuda.synchronize()
    cuh = cu.cpu().tolist()
    dt, th = f64(inp["dt"]), f64(inp["theta"])
    for s in range(4):
        a, b = cuh[s], cuh[s + 1]
        ref = oracle.accumulated_phase(dt[:, a:b], th[:, a:b], ph0[s:s + 1])
        e = angle_err(ph[s:s + 1], ref)
        say("   sequence %d (%d tokens): angle err %.2e" % (s, b - a, e))
        assert e <= ANGLE_TOL, (s, e)


def decode_case(w, seed, mode, in_place=False, label=""):
    say("case decode %s %s: B%d H%d R%d P%d N%d %s seed=%d in_place=%s" % (
        label, mode, w.batch, w.heads, w.rank, w.headdim, w.dstate, w.io_dtype, seed, in_place))
    g = torch.Generator(device=DEV).manual_seed(seed)
    A = -torch.exp(torch.rand((w.heads,), generator=g, device=DEV) * 2 - 1)
    s = synth.make_decode_inputs(w, seed, 0, A, DEV)
    st = random_state(w, seed + 1, DEV)
    ph_in = (torch.rand((w.batch, w.heads, w.dstate // 2), generator=g, device=DEV) * 2 - 1) * np.pi
    ph0 = f64(ph_in)
    ph_out = ph_in if in_place else torch.empty_like(ph_in)
    h0, Bp0, xp0 = f64(st[0]), f64(st[1]), f64(st[2])
    state = State(*st)
    y = m3_decode_step(s["x"], s["B"], s["C"], s["dt"], s["A"], s["theta"], s["lam"], state,
                       phase=mode, phase_in=ph_in, phase_out=ph_out)
    torch.cuda.synchronize()
    args = (f64(s["x"]), f64(s["B"]), f64(s["C"]), f64(s["dt"]), f64(s["A"]), f64(s["theta"]),
            f64(s["lam"]), h0, Bp0, xp0)
    if mode == "native":
        yr, hr, _, _ = oracle.decode_step(*args)
        phr = oracle.wrap_angle(ph0 + f64(s["dt"])[..., None] * f64(s["theta"]))
    else:
        yr, hr, _, _, phr = oracle.decode_step_rotation_removed(*args, mode, ph0)
    tol = TOL[w.io_dtype]
    ey, eh, ep = rel_err(f64(y), yr), rel_err(f64(state.h), hr), angle_err(ph_out, phr)
    say("   rel err y %.2e  state %.2e  angle %.2e (tol %.0e, %.0e)" % (ey, eh, ep, tol, ANGLE_TOL))
    assert ey <= tol and eh <= tol and ep <= ANGLE_TOL, (ey, eh, ep)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["native", "no_write", "no_read", "no_write_read"])
@pytest.mark.parametrize("N,P,R", [(16, 16, 1), (64, 32, 2), (128, 64, 4)])
def test_decode_rotation_removed(io, mode, N, P, R):
    w = workload(3, 1, 5, R, P, N, io=io, dt_mu=-1.0, theta="uniform_pi")
    decode_case(w, 730 + N + P + R, mode, label="shapes")


@pytest.mark.parametrize("mode", ["no_write", "no_read"])
def test_decode_rotation_removed_in_place(mode):
    w = workload(2, 1, 4, 4, 64, 128, io="f32", dt_mu=-1.0, theta="uniform_pi")
    decode_case(w, 760, mode, in_place=True, label="in-place")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["no_write", "no_read", "no_write_read"])
def test_native_context_then_intervened_steps(io, mode):
    """The protocol of the pages: a native prefill of the context (its
    accumulated angle carried out), then prediction steps with the rotation
    removed, against the oracle run the same way."""
    w = workload(2, 96, 3, 2, 64, 64, io=io, dt_mu=-1.0, theta="uniform_pi")
    seed = 770 + len(mode)
    say("case context + %s steps %s" % (mode, io))
    inp = synth.make_scan_inputs(w, seed, DEV)
    ph = torch.empty((w.batch, w.heads, w.dstate // 2), device=DEV)
    _, st = m3_scan_fwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"],
                        inp["lam"], phase_out=ph)
    _, hr, br, xr = oracle.scan(f64(inp["x"]), f64(inp["B"]), f64(inp["C"]), f64(inp["dt"]),
                                f64(inp["A"]), f64(inp["theta"]), f64(inp["lam"]))
    phr = oracle.accumulated_phase(f64(inp["dt"]), f64(inp["theta"]))
    tol = TOL[w.io_dtype]
    for k in range(6):
        s = synth.make_decode_inputs(w, seed, k, inp["A"], DEV)
        y = m3_decode_step(s["x"], s["B"], s["C"], s["dt"], s["A"], s["theta"], s["lam"], st,
                           phase=mode, phase_in=ph, phase_out=ph)
        torch.cuda.synchronize()
        yr, hr, br, xr, phr = oracle.decode_step_rotation_removed(
            f64(s["x"]), f64(s["B"]), f64(s["C"]), f64(s["dt"]), f64(s["A"]), f64(s["theta"]),
            f64(s["lam"]), hr, br, xr, mode, phr)
        ey, eh, ep = rel_err(f64(y), yr), rel_err(f64(st.h), hr), angle_err(ph, phr)
        say("   step %d: rel err y %.2e  state %.2e  angle %.2e" % (k, ey, eh, ep))
        assert ey <= tol and eh <= tol and ep <= ANGLE_TOL, (k, ey, eh, ep)
