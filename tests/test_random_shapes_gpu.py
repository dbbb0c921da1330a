"""Seeded random shapes and option combinations for m3_scan_fwd and
m3_decode_step against the fp64 oracle: dstate, headdim, rank, I/O type,
sequence length (ragged last chunks included), batch, heads, head groups,
per-token decay, phase mode, pre-mixer, initial state and (scan) forced
segment counts, each case drawn from its own seed.  Tolerances as for the
plain mixer (max |got - ref| / max |ref| <= 1e-4 for float32 I/O, <= 2e-2 for
bfloat16) on y and the final state (and the record's B_prev).
"""
import random

import pytest

import test_options_gpu as opt
from helpers import workload
from mamba_selective_ssm_amd import m3_scan_supported

pytestmark = pytest.mark.gpu


def draw(case):
    rnd = random.Random(9000 + case)
    N = rnd.choice([16, 32, 64, 128])
    R = rnd.choice([1, 2, 4])
    P = rnd.choice([16, 32, 48, 64])
    io = rnd.choice(["f32", "bf16"])
    L = rnd.randint(1, 420)
    Bt = rnd.randint(1, 3)
    H = rnd.choice([1, 2, 3, 4, 6])
    groups = rnd.choice([0] + [g for g in (1, 2, 3) if H % g == 0 and g < H])
    a_tok = rnd.random() < 0.3
    phase = rnd.choice(["native", "native", "zero", "reverse", "shuffle"])
    premix = rnd.random() < 0.25
    with_state = rnd.random() < 0.7
    segments = rnd.choice([0, 0, 1, 2, 3, 7])
    dt_mu = rnd.choice([-2.0, -1.0, 0.0])
    return dict(N=N, R=R, P=P, io=io, L=L, Bt=Bt, H=H, groups=groups, a_tok=a_tok, phase=phase,
                premix=premix, with_state=with_state, segments=segments, dt_mu=dt_mu)


@pytest.mark.parametrize("case", range(96))
def test_random_scan_case(case):
    c = draw(case)
    if not m3_scan_supported(c["N"], c["P"], c["R"], 0, 0 if c["io"] == "f32" else 1):
        pytest.skip("shape outside the compiled set: %s" % (c,))
    w = workload(c["Bt"], c["L"], c["H"], c["R"], c["P"], c["N"], io=c["io"], dt_mu=c["dt_mu"],
                 theta="uniform_pi")
    opt.run_case(w, 9100 + case, ngroups=c["groups"], a_tok=c["a_tok"], phase=c["phase"],
                 premix=c["premix"], with_state=c["with_state"], segments=c["segments"],
                 label="random %d" % case)


def draw_decode(case):
    rnd = random.Random(9500 + case)
    N = rnd.choice([2, 6, 16, 30, 64, 96, 128, 200, 256])
    P = rnd.choice([4, 8, 16, 32, 64, 128])
    R = rnd.choice([1, 2, 4])
    io = rnd.choice(["f32", "bf16"])
    Bt = rnd.randint(1, 4)
    H = rnd.choice([1, 2, 3, 4, 6])
    groups = rnd.choice([0] + [g for g in (1, 2, 3) if H % g == 0 and g < H])
    a_tok = rnd.random() < 0.3
    phase = rnd.choice(["native", "native", "zero", "reverse", "shuffle"])
    premix = rnd.random() < 0.3
    return dict(N=N, P=P, R=R, io=io, Bt=Bt, H=H, groups=groups, a_tok=a_tok, phase=phase,
                premix=premix)


@pytest.mark.parametrize("case", range(48))
def test_random_decode_case(case):
    """Three decode steps from a random state record, each against the
    oracle's decode step continued from the library's record."""
    import numpy as np
    import torch

    import oracle
    from helpers import TOL, f64, random_state, rel_err, say
    from mamba_selective_ssm_amd import State, m3_decode_step, m3_decode_supported, synth

    c = draw_decode(case)
    if not m3_decode_supported(c["N"], c["P"], c["R"], 0 if c["io"] == "f32" else 1):
        pytest.skip("shape outside the supported set: %s" % (c,))
    w = workload(c["Bt"], 3, c["H"], c["R"], c["P"], c["N"], io=c["io"], dt_mu=0.0, theta="uniform_pi")
    say("case random decode %d: %s" % (case, c))
    inp, ex = synth.make_option_inputs(w, 9600 + case, "cuda", ngroups=c["groups"],
                                       a_per_token=c["a_tok"], phase=c["phase"], premix=c["premix"])
    h, Bp, xp = random_state(w, 9700 + case, "cuda")
    st = State(h.clone(), Bp.clone(), xp.clone())
    ref = (f64(h), f64(Bp), f64(xp))
    okw = opt.oracle_kw(ex, c["groups"], c["phase"])
    for t in range(w.seqlen):
        # one step's tensors as fresh allocations (a batch-1 slice is a view
        # at an offset that need not meet the library's 16-byte alignment)
        s = {k: (v if (k == "A" and not c["a_tok"]) else v[:, t].clone()) for k, v in inp.items()}
        theta = None if c["phase"] == "zero" else s["theta"]
        y = m3_decode_step(s["x"], s["B"], s["C"], s["dt"], s["A"], theta, s["lam"], st,
                           ngroups=c["groups"], phase=c["phase"], perm=ex.get("perm"),
                           premix=opt.premix_obj(ex))
        torch.cuda.synchronize()
        yr, hr, br, xr = oracle.decode_step(f64(s["x"]), f64(s["B"]), f64(s["C"]), f64(s["dt"]),
                                            f64(s["A"]), f64(s["theta"]), f64(s["lam"]), *ref,
                                            **okw)
        ref = (hr, f64(st.B_prev), xr)
        tol = TOL[c["io"]]
        ey, eh, eb = rel_err(f64(y), yr), rel_err(f64(st.h), hr), rel_err(f64(st.B_prev), br)
        say("   step %d rel err y %.3e state %.3e B_prev %.3e" % (t, ey, eh, eb))
        assert ey <= tol and eh <= tol and eb <= tol, (ey, eh, eb)
        np.testing.assert_array_equal(f64(st.x_prev), xr)


def draw_bwd(case):
    rnd = random.Random(9800 + case)
    N, P, R = rnd.choice([(16, 16, 1), (32, 32, 2), (32, 64, 4), (64, 32, 1), (64, 64, 2),
                          (128, 64, 1), (128, 32, 4), (64, 16, 2)])
    io = rnd.choice(["f32", "bf16"])
    return dict(N=N, P=P, R=R, io=io, L=rnd.randint(1, 160), Bt=rnd.randint(1, 2),
                H=rnd.randint(1, 3), with_state=rnd.random() < 0.7, with_dh=rnd.random() < 0.7,
                dt_mu=rnd.choice([-2.0, -1.0, 0.0]))


@pytest.mark.parametrize("case", range(24))
def test_random_bwd_case(case):
    """The scan gradient by both methods (where the chunked one supports the
    shape) against the fp64 gradient oracle."""
    import test_bwd_gpu as bwd

    c = draw_bwd(case)
    w = workload(c["Bt"], c["L"], c["H"], c["R"], c["P"], c["N"], io=c["io"], dt_mu=c["dt_mu"],
                 theta="uniform_pi")
    methods = ["step"] + (["chunked"] if bwd.chunked_ok(c["io"], c["N"], c["P"], c["R"]) else [])
    for m in methods:
        bwd.grads_case(w, 9900 + case, with_state=c["with_state"], with_dh=c["with_dh"],
                       label="random bwd %d" % case, method=m)
