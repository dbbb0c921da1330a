"""Seeded random shapes and option combinations for m3_scan_fwd against the
fp64 oracle: dstate, headdim, rank, I/O type, sequence length (ragged last
chunks included), batch, heads, head groups, per-token decay, phase mode,
pre-mixer, initial state and forced segment counts, each case drawn from its
own seed.  Tolerances as for the plain mixer (max |got - ref| / max |ref| <=
1e-4 for float32 I/O, <= 2e-2 for bfloat16) on y and the final state.
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
