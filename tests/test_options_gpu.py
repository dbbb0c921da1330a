"""Parity of the library's options against the fp64 oracle: per-token decay
A_t, B/C shared by head groups, the phase interventions (zero, reverse,
shuffle) and the pre-mixer (softplus/sigmoid of raw dt/lam, RMSNorm with
gains and biases on B and C), in m3_scan_fwd and m3_decode_step.

Tolerances as for the plain mixer: max |got - ref| / max |ref| <= 1e-4 for
float32 I/O and <= 2e-2 for bfloat16 I/O, for y, the final state and (with
the pre-mixer, where the record holds a computed B) the record's B_prev.
"""
import numpy as np
import pytest
import torch

import oracle
from mamba_selective_ssm_amd import Premix, State, m3_decode_step, m3_scan_fwd, synth
from helpers import TOL, f64, random_state, rel_err, say, workload

pytestmark = pytest.mark.gpu
DEV = "cuda"


def premix_obj(extras):
    pm = extras.get("premix")
    if pm is None:
        return None
    return Premix(pm["B_norm_w"], pm["C_norm_w"], pm["B_bias"], pm["C_bias"], pm["dt_bias"], pm["eps"])


def oracle_kw(extras, ngroups, phase):
    kw = dict(ngroups=ngroups or None, phase=phase)
    if "perm" in extras:
        kw["perm"] = extras["perm"].cpu().numpy()
    pm = extras.get("premix")
    if pm is not None:
        kw["premix"] = {k: (f64(v) if torch.is_tensor(v) else v) for k, v in pm.items()}
    return kw


def run_case(w, seed, ngroups=0, a_tok=False, phase="native", premix=False, with_state=True,
             segments=0, chunk=0, label=""):
    say("case %s: B%d L%d H%d R%d P%d N%d %s groups=%d a_tok=%s phase=%s premix=%s seg=%d seed=%d"
        % (label, w.batch, w.seqlen, w.heads, w.rank, w.headdim, w.dstate, w.io_dtype, ngroups,
           a_tok, phase, premix, segments, seed))
    inp, ex = synth.make_option_inputs(w, seed, DEV, ngroups=ngroups, a_per_token=a_tok,
                                       phase=phase, premix=premix)
    st = random_state(w, seed + 7, DEV) if with_state else None
    theta = None if phase == "zero" else inp["theta"]
    y, so = m3_scan_fwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], theta, inp["lam"],
                        State(*st) if st else None, segments=segments, chunk=chunk,
                        ngroups=ngroups, phase=phase, perm=ex.get("perm"), premix=premix_obj(ex))
    torch.cuda.synchronize()
    skw = {} if st is None else dict(h0=f64(st[0]), Bprev=f64(st[1]), xprev=f64(st[2]))
    yr, hr, br, xr = oracle.scan(f64(inp["x"]), f64(inp["B"]), f64(inp["C"]), f64(inp["dt"]),
                                 f64(inp["A"]), f64(inp["theta"]), f64(inp["lam"]),
                                 **skw, **oracle_kw(ex, ngroups, phase))
    tol = TOL[w.io_dtype]
    ey, eh = rel_err(f64(y), yr), rel_err(f64(so.h), hr)
    say("   rel err y %.3e  state %.3e  (tol %.0e)" % (ey, eh, tol))
    assert ey <= tol and eh <= tol, (ey, eh)
    if premix:
        eb = rel_err(f64(so.B_prev), br)
        say("   rel err B_prev %.3e" % eb)
        assert eb <= tol
    else:
        np.testing.assert_array_equal(f64(so.B_prev), br)
    np.testing.assert_array_equal(f64(so.x_prev), xr)
    return inp, ex, y, so


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N,R,G", [(64, 1, 2), (128, 4, 4), (16, 2, 1)])
def test_groups_and_per_token_decay(io, N, R, G):
    w = workload(2, 203, 4, R, 32, N, io=io, dt_mu=-1.0)
    run_case(w, 300 + N + R, ngroups=G, a_tok=True, label="groups+A_t")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("phase", ["zero", "reverse", "shuffle"])
def test_phase_interventions(io, phase):
    w = workload(2, 190, 3, 2, 32, 64, io=io, dt_mu=-1.0, theta="uniform_pi")
    run_case(w, 320, phase=phase, label="phase")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N,R", [(64, 1), (128, 4), (16, 2), (32, 1)])
def test_premix(io, N, R):
    w = workload(2, 171, 3, R, 32, N, io=io, dt_mu=-1.0)
    run_case(w, 340 + N + R, premix=True, label="premix")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("segments", [2, 5])
def test_all_options_with_segments(io, segments):
    """Every option at once, through the state pass and the record fold."""
    w = workload(2, 900, 4, 2, 32, 64, io=io, dt_mu=-1.5)
    run_case(w, 360 + segments, ngroups=2, a_tok=True, phase="shuffle", premix=True,
             segments=segments, label="all+segments")


@pytest.mark.slow
@pytest.mark.parametrize("opts", [dict(ngroups=4, a_tok=True), dict(phase="zero"), dict(phase="shuffle"),
                                  dict(premix=True)],
                         ids=["groups4+A_t", "phase_zero", "phase_shuffle", "premix"])
def test_option_workloads_full_every_unit(opts):
    """The benchmark's option workloads at the single-layer prefill's full
    shape (batch 4, 16 heads, 2048 tokens, P = N = 64, bf16, chunk 64) from
    a random state record, in the launch the library picks (segments, the
    pre-mixer's own variant): every (b, h) unit's y and final state against
    the oracle."""
    run_case(synth.WORKLOADS["prefill_bf16"], 470, label="option workload, full size", **opts)


def test_premix_prefill_workload_sampled():
    """prefill_bf16 shapes with the pre-mixer and head groups (segmented
    launch as the library picks it): sampled (b, h) units against the oracle."""
    w = synth.WORKLOADS["prefill_bf16"]
    say("case premix prefill_bf16 full size")
    inp, ex = synth.make_option_inputs(w, 380, DEV, ngroups=4, premix=True)
    y, so = m3_scan_fwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"],
                        inp["lam"], ngroups=4, premix=premix_obj(ex))
    torch.cuda.synchronize()
    H, G = w.heads, 4
    for b, h in [(0, 0), (1, 5), (3, 15)]:
        g = h // (H // G)
        sub = lambda t, ax=2, i=h: f64(t[b:b + 1].narrow(ax, i, 1))
        pm = {k: (f64(v) if torch.is_tensor(v) else v) for k, v in ex["premix"].items()}
        pm["B_bias"] = pm["B_bias"][h:h + 1]
        pm["C_bias"] = pm["C_bias"][h:h + 1]
        pm["dt_bias"] = pm["dt_bias"][h:h + 1]
        yr, hr, _, _ = oracle.scan(sub(inp["x"]), sub(inp["B"], i=g), sub(inp["C"], i=g),
                                   sub(inp["dt"]), f64(inp["A"][h:h + 1]), sub(inp["theta"]),
                                   sub(inp["lam"]), premix=pm)
        ey = rel_err(f64(y[b:b + 1, :, h:h + 1]), yr)
        eh = rel_err(f64(so.h[b:b + 1, h:h + 1]), hr)
        say("   unit (%d, %d): rel err y %.3e state %.3e" % (b, h, ey, eh))
        assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def step_of(inp, t, a_tok):
    return {k: (v if (k == "A" and not a_tok) else v[:, t].contiguous()) for k, v in inp.items()}


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("opts", [
    dict(ngroups=2, a_tok=True),
    dict(phase="zero"), dict(phase="reverse"), dict(phase="shuffle"),
    dict(premix=True),
    dict(ngroups=4, a_tok=True, phase="shuffle", premix=True),
])
def test_decode_options(io, opts):
    ngroups, a_tok = opts.get("ngroups", 0), opts.get("a_tok", False)
    phase, premix = opts.get("phase", "native"), opts.get("premix", False)
    w = workload(3, 5, 4, 4, 64, 128, io=io, dt_mu=0.0, theta="uniform_pi")
    say("case decode options %s %s" % (io, opts))
    inp, ex = synth.make_option_inputs(w, 400, DEV, ngroups=ngroups, a_per_token=a_tok,
                                       phase=phase, premix=premix)
    h, Bp, xp = random_state(w, 401, DEV)
    st = State(h.clone(), Bp.clone(), xp.clone())
    ref = (f64(h), f64(Bp), f64(xp))
    okw = oracle_kw(ex, ngroups, phase)
    for t in range(w.seqlen):
        s = step_of(inp, t, a_tok)
        theta = None if phase == "zero" else s["theta"]
        y = m3_decode_step(s["x"], s["B"], s["C"], s["dt"], s["A"], theta, s["lam"], st,
                           ngroups=ngroups, phase=phase, perm=ex.get("perm"),
                           premix=premix_obj(ex))
        torch.cuda.synchronize()
        yr, hr, br, xr = oracle.decode_step(f64(s["x"]), f64(s["B"]), f64(s["C"]), f64(s["dt"]),
                                            f64(s["A"]), f64(s["theta"]), f64(s["lam"]), *ref,
                                            **okw)
        # continue the oracle from the GPU's record (B_prev rounded to the io dtype)
        ref = (hr, f64(st.B_prev), xr)
        ey, eh, eb = rel_err(f64(y), yr), rel_err(f64(st.h), hr), rel_err(f64(st.B_prev), br)
        say("   step %d rel err y %.3e state %.3e B_prev %.3e" % (t, ey, eh, eb))
        assert ey <= TOL[io] and eh <= TOL[io] and eb <= TOL[io]
        if not premix:
            np.testing.assert_array_equal(f64(st.B_prev), br)
        np.testing.assert_array_equal(f64(st.x_prev), xr)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_then_decode_with_options(io):
    """All options: scan(L1) then single decode steps == the oracle's one scan."""
    w = workload(2, 120, 4, 4, 64, 128, io=io, chunk=16, dt_mu=-1.0)
    say("case prefill+decode options %s" % io)
    inp, ex = synth.make_option_inputs(w, 420, DEV, ngroups=2, a_per_token=True, phase="shuffle",
                                       premix=True)
    kw = dict(ngroups=2, phase="shuffle", perm=ex["perm"], premix=premix_obj(ex))
    L1 = 77
    part = {k: v[:, :L1].contiguous() for k, v in inp.items()}
    y1, st = m3_scan_fwd(part["x"], part["B"], part["C"], part["dt"], part["A"], part["theta"],
                         part["lam"], **kw)
    ys = [y1]
    for t in range(L1, w.seqlen):
        s = step_of(inp, t, True)
        ys.append(m3_decode_step(s["x"], s["B"], s["C"], s["dt"], s["A"], s["theta"], s["lam"],
                                 st, **kw).unsqueeze(1).clone())
    torch.cuda.synchronize()
    yr, hr, _, _ = oracle.scan(f64(inp["x"]), f64(inp["B"]), f64(inp["C"]), f64(inp["dt"]),
                               f64(inp["A"]), f64(inp["theta"]), f64(inp["lam"]),
                               **oracle_kw(ex, 2, "shuffle"))
    ey, eh = rel_err(f64(torch.cat(ys, 1)), yr), rel_err(f64(st.h), hr)
    say("   rel err y %.3e state %.3e" % (ey, eh))
    assert ey <= TOL[io] and eh <= TOL[io]


PACKED_LENGTHS = [0, 1, 63, 64, 65, 300, 17, 129, 2, 200]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("segments,opts", [
    (0, {}), (3, {}),
    (2, dict(ngroups=2, a_tok=True, premix=True, phase="reverse")),
])
def test_packed_sequences(io, segments, opts):
    """Sequences of different lengths (one empty) packed along the token axis,
    each with its own state record."""
    lens = PACKED_LENGTHS
    T = sum(lens)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=DEV)
    ngroups, a_tok = opts.get("ngroups", 0), opts.get("a_tok", False)
    phase, premix = opts.get("phase", "native"), opts.get("premix", False)
    w = workload(1, T, 4, 2, 32, 64, io=io, dt_mu=-1.0)
    say("case packed %s seg=%d %s lengths=%s" % (io, segments, opts, lens))
    inp, ex = synth.make_option_inputs(w, 440 + segments, DEV, ngroups=ngroups, a_per_token=a_tok,
                                       phase=phase, premix=premix)
    st = random_state(w.with_(batch=len(lens)), 441, DEV)
    y, so = m3_scan_fwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"],
                        inp["lam"], State(*st), segments=segments, ngroups=ngroups, phase=phase,
                        perm=ex.get("perm"), premix=premix_obj(ex), cu_seqlens=cu,
                        max_seqlen=max(lens))
    torch.cuda.synchronize()
    yr, hr, br, xr = oracle.scan_packed(f64(inp["x"]), f64(inp["B"]), f64(inp["C"]),
                                        f64(inp["dt"]), f64(inp["A"]), f64(inp["theta"]),
                                        f64(inp["lam"]), cu.cpu().numpy(), h0=f64(st[0]),
                                        Bprev=f64(st[1]), xprev=f64(st[2]),
                                        **oracle_kw(ex, ngroups, phase))
    tol = TOL[io]
    ey, eh = rel_err(f64(y), yr), rel_err(f64(so.h), hr)
    say("   rel err y %.3e state %.3e" % (ey, eh))
    assert ey <= tol and eh <= tol
    if premix:
        assert rel_err(f64(so.B_prev), br) <= tol
    else:
        np.testing.assert_array_equal(f64(so.B_prev), br)
    np.testing.assert_array_equal(f64(so.x_prev), xr)


def test_packed_many_sequences_per_sequence_segments():
    """100 packed sequences -- 99 short ones (0 to 40 tokens, some empty) and
    one of 3000 tokens at index 70 -- in the library's segmentation: the long
    sequence takes many segments, so each workgroup finds its (sequence,
    segment) among more than 64 sequences (two rounds of the wave-wide
    search).  Against the oracle per sequence."""
    g = np.random.default_rng(470)
    lens = [int(v) for v in g.integers(0, 41, size=100)]
    lens[70] = 3000
    lens[3] = 0
    T = sum(lens)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=DEV)
    w = workload(1, T, 2, 1, 32, 32, io="bf16", dt_mu=-1.0)
    say("case packed many: %d sequences, %d tokens" % (len(lens), T))
    inp = synth.make_scan_inputs(w, 471, DEV)
    st = random_state(w.with_(batch=len(lens)), 472, DEV)
    y, so = m3_scan_fwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"],
                        inp["lam"], State(*st), cu_seqlens=cu, max_seqlen=max(lens))
    torch.cuda.synchronize()
    yr, hr, br, xr = oracle.scan_packed(f64(inp["x"]), f64(inp["B"]), f64(inp["C"]),
                                        f64(inp["dt"]), f64(inp["A"]), f64(inp["theta"]),
                                        f64(inp["lam"]), cu.cpu().numpy(), h0=f64(st[0]),
                                        Bprev=f64(st[1]), xprev=f64(st[2]))
    ey, eh = rel_err(f64(y), yr), rel_err(f64(so.h), hr)
    say("   rel err y %.3e state %.3e" % (ey, eh))
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
    np.testing.assert_array_equal(f64(so.B_prev), br)
    np.testing.assert_array_equal(f64(so.x_prev), xr)


def test_packed_equal_lengths_match_dense_batch():
    """Packing equal-length sequences gives the dense batch's results bit for bit."""
    w = workload(3, 257, 4, 1, 64, 64, io="bf16")
    say("case packed == dense")
    inp = synth.make_scan_inputs(w, 450, DEV)
    y, so = m3_scan_fwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"],
                        inp["lam"], segments=3)
    pk = {k: (v if k == "A" else v.reshape((1, -1) + tuple(v.shape[2:])).contiguous())
          for k, v in inp.items()}
    cu = torch.arange(0, 4 * 257, 257, dtype=torch.int32, device=DEV)
    yp, sp = m3_scan_fwd(pk["x"], pk["B"], pk["C"], pk["dt"], pk["A"], pk["theta"], pk["lam"],
                         segments=3, cu_seqlens=cu, max_seqlen=257)
    torch.cuda.synchronize()
    assert torch.equal(yp.reshape(y.shape), y)
    assert torch.equal(sp.h, so.h)


def test_packed_bench_lengths_per_sequence_segments():
    """The benchmark's packed case: the single-layer prefill's 8192 tokens as
    8 sequences of 1536, 256, 1024, 768, 2048, 512, 640 and 1408 tokens (16
    heads, dstate 64, headdim 64, bf16), in the library's segmentation (a
    fixed number of chunks per segment, so short sequences take fewer
    segments), against the oracle per sequence, every head."""
    lens = [1536, 256, 1024, 768, 2048, 512, 640, 1408]
    T = sum(lens)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=DEV)
    w = workload(1, T, 16, 1, 64, 64, io="bf16", dt_mu=-2.0)
    say("case packed bench lengths %s" % (lens,))
    inp = synth.make_scan_inputs(w, 460, DEV)
    st = random_state(w.with_(batch=len(lens)), 461, DEV)
    y, so = m3_scan_fwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"],
                        inp["lam"], State(*st), cu_seqlens=cu, max_seqlen=max(lens))
    torch.cuda.synchronize()
    yr, hr, br, xr = oracle.scan_packed(f64(inp["x"]), f64(inp["B"]), f64(inp["C"]),
                                        f64(inp["dt"]), f64(inp["A"]), f64(inp["theta"]),
                                        f64(inp["lam"]), cu.cpu().numpy(), h0=f64(st[0]),
                                        Bprev=f64(st[1]), xprev=f64(st[2]))
    ey, eh = rel_err(f64(y), yr), rel_err(f64(so.h), hr)
    say("   rel err y %.3e state %.3e" % (ey, eh))
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
    np.testing.assert_array_equal(f64(so.B_prev), br)
    np.testing.assert_array_equal(f64(so.x_prev), xr)
