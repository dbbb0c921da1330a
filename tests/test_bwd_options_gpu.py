"""Parity of m3_scan_bwd with options -- a decay rate per token, head groups,
the phase modes of a scan (theta zeroed, negated, shuffled) and the pre-mixer
(RMSNorm + biases on B and C, softplus and sigmoid of the raw step and
weight) -- against the fp64
gradient oracle with the same options, by both methods.  With the pre-mixer
the gradients are those of the raw inputs, plus the parameter gradients
dB_norm_w, dC_norm_w, dB_bias, dC_bias and ddt_bias.

Metric as for the plain gradient: max |got - ref| / max |ref| per tensor,
tolerance 1e-4 for float32 inputs, 2e-2 for bfloat16; dA and ddt_bias, which
sum per-token terms over batch and tokens, against the sum of the terms'
magnitudes (for ddt_bias: sum over (b, t) of |ddt_raw| of the head); dA per
token (A per token) elementwise like the other gradients.
"""
import random

import numpy as np
import pytest
import torch

import test_bwd_gpu as bwd
import test_options_gpu as opt
from oracle.backward import PREMIX_GRADS, scan_backward, scan_backward_packed
from mamba_selective_ssm_amd import State, m3_scan_bwd, synth
from helpers import TOL, f64, random_state, rel_err, say, workload

pytestmark = pytest.mark.gpu
DEV = "cuda"


def option_grads_case(w, seed, ngroups=0, phase="native", premix=False, with_state=True,
                      with_dh=True, method="auto", label="", a_tok=False):
    say("case %s [%s]: B%d L%d H%d R%d P%d N%d %s groups=%d phase=%s premix=%s a_tok=%s state=%s "
        "seed=%d" % (label, method, w.batch, w.seqlen, w.heads, w.rank, w.headdim, w.dstate,
                     w.io_dtype, ngroups, phase, premix, a_tok, with_state, seed))
    inp, ex = synth.make_option_inputs(w, seed, DEV, ngroups=ngroups, phase=phase, premix=premix,
                                       a_per_token=a_tok)
    g = torch.Generator(device=DEV).manual_seed(seed + 1)
    dy = torch.randn(inp["x"].shape, generator=g, device=DEV).to(w.torch_dtype)
    dh = torch.randn(w.batch, w.heads, w.dstate, w.headdim, generator=g, device=DEV) if with_dh else None
    st = random_state(w, seed + 2, DEV) if with_state else None
    theta = None if phase == "zero" else inp["theta"]
    got = m3_scan_bwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], theta, inp["lam"], dy,
                      State(*st) if st else None, dh, method=method, ngroups=ngroups, phase=phase,
                      perm=ex.get("perm"), premix=opt.premix_obj(ex), A_per_token=a_tok)
    torch.cuda.synchronize()
    ref = scan_backward(f64(inp["x"]), f64(inp["B"]), f64(inp["C"]), f64(inp["dt"]),
                        f64(inp["A"]), f64(inp["theta"]), f64(inp["lam"]), f64(dy),
                        None if dh is None else f64(dh),
                        h0=None if st is None else f64(st[0]),
                        Bprev=None if st is None else f64(st[1]),
                        xprev=None if st is None else f64(st[2]),
                        **opt.oracle_kw(ex, ngroups, phase))
    return check_grads(got, ref, w.io_dtype, a_tok, premix, phase)


def check_grads(got, ref, io, a_tok, premix, phase):
    tol = TOL[io]
    errs = {}
    for n in bwd.NAMES:
        if n == "dA" and not a_tok:
            errs[n] = float(np.max(np.abs(f64(got.dA) - ref["dA"])) / max(np.max(ref["dA_scale"]), 1e-300))
        else:
            errs[n] = rel_err(f64(getattr(got, n)), ref[bwd.ORACLE.get(n, n)])
    if premix:
        for n in PREMIX_GRADS:
            gv = f64(getattr(got.premix, n[1:]))
            if n == "ddt_bias":
                scale = np.abs(ref["ddt"]).sum(axis=(0, 1))
                errs[n] = float(np.max(np.abs(gv - ref[n])) / max(np.max(scale), 1e-300))
            else:
                errs[n] = rel_err(gv, ref[n])
    if phase == "zero":
        assert torch.count_nonzero(got.dtheta) == 0
    say("   " + "  ".join("%s %.2e" % (n, e) for n, e in errs.items()) + "  (tol %.0e)" % tol)
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, bad
    return got


COMBOS = [(2, "native", False, False), (0, "reverse", False, False), (0, "shuffle", False, False),
          (0, "zero", False, False), (0, "native", True, False), (2, "shuffle", True, False),
          (1, "zero", True, False), (4, "reverse", True, False), (0, "native", False, True),
          (2, "shuffle", True, True)]


@pytest.mark.parametrize("method", ["step", "chunked"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("ngroups,phase,premix,a_tok", COMBOS)
def test_bwd_options(ngroups, phase, premix, a_tok, io, method):
    """Several chunks (32 tokens at rank 2) and checkpoints, ragged tail."""
    w = workload(2, 70, 4, 2, 32, 64, io=io, dt_mu=-1.0, theta="uniform_pi")
    option_grads_case(w, 1200 + 10 * COMBOS.index((ngroups, phase, premix, a_tok)) + (io == "bf16"),
                      ngroups, phase, premix, method=method, label="bwd-options", a_tok=a_tok)


@pytest.mark.parametrize("method", ["step", "chunked"])
def test_bwd_options_longer_dstate128(method):
    """bf16, dstate 128, rank 4 (16-token chunks), 300 tokens, per-token decay,
    head groups, shuffled phases and the pre-mixer together."""
    w = workload(1, 300, 4, 4, 64, 128, io="bf16", dt_mu=-2.0)
    option_grads_case(w, 1300, 2, "shuffle", True, method=method, label="bwd-options-long",
                      a_tok=True)


def test_bwd_options_without_state_or_final_gradient():
    w = workload(2, 40, 2, 1, 64, 64, io="f32", dt_mu=-1.0)
    option_grads_case(w, 1310, 1, "reverse", True, with_state=False, with_dh=False,
                      label="bwd-options-plain")


def test_bwd_options_empty_sequence():
    """seqlen 0: the state-record gradients pass through, the parameter
    gradients are zero."""
    w = workload(2, 0, 2, 1, 32, 32, io="f32", dt_mu=-1.0)
    got = option_grads_case(w, 1320, 1, "shuffle", True, label="bwd-options-empty", a_tok=True)
    for n in PREMIX_GRADS:
        assert torch.count_nonzero(getattr(got.premix, n[1:])) == 0, n


@pytest.mark.parametrize("method", ["step", "chunked"])
def test_bwd_options_deterministic(method):
    w = workload(2, 90, 4, 2, 64, 128, io="bf16")
    inp, ex = synth.make_option_inputs(w, 1330, DEV, ngroups=2, phase="shuffle", premix=True)
    dy = torch.randn(inp["x"].shape, device=DEV,
                     generator=torch.Generator(device=DEV).manual_seed(2)).to(torch.bfloat16)
    run = lambda: m3_scan_bwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"],
                              inp["lam"], dy, method=method, ngroups=2, phase="shuffle",
                              perm=ex["perm"], premix=opt.premix_obj(ex))
    a, b = run(), run()
    torch.cuda.synchronize()
    for n in bwd.NAMES:
        assert torch.equal(getattr(a, n), getattr(b, n)), n
    for n in PREMIX_GRADS:
        assert torch.equal(getattr(a.premix, n[1:]), getattr(b.premix, n[1:])), n


def draw_bwd_options(case):
    rnd = random.Random(9850 + case)
    N, P, R = rnd.choice([(16, 16, 1), (32, 32, 2), (32, 64, 4), (64, 32, 1), (64, 64, 2),
                          (128, 64, 1), (128, 32, 4), (64, 16, 2)])
    H = rnd.choice([1, 2, 3, 4, 6])
    return dict(N=N, P=P, R=R, io=rnd.choice(["f32", "bf16"]), L=rnd.randint(1, 140),
                Bt=rnd.randint(1, 2), H=H,
                groups=rnd.choice([0] + [g for g in (1, 2, 3) if H % g == 0 and g < H]),
                phase=rnd.choice(["native", "zero", "reverse", "shuffle"]),
                premix=rnd.random() < 0.5, a_tok=rnd.random() < 0.3, with_state=rnd.random() < 0.7,
                dt_mu=rnd.choice([-2.0, -1.0, 0.0]))


@pytest.mark.parametrize("case", range(16))
def test_random_bwd_options_case(case):
    """Seeded random shapes and option combinations, both methods where the
    chunked one supports the shape."""
    c = draw_bwd_options(case)
    w = workload(c["Bt"], c["L"], c["H"], c["R"], c["P"], c["N"], io=c["io"], dt_mu=c["dt_mu"],
                 theta="uniform_pi")
    methods = ["step"] + (["chunked"] if bwd.chunked_ok(c["io"], c["N"], c["P"], c["R"]) else [])
    for m in methods:
        option_grads_case(w, 9950 + case, c["groups"], c["phase"], c["premix"],
                          with_state=c["with_state"], method=m, label="random bwd options %d" % case,
                          a_tok=c["a_tok"])


PACKED_LENGTHS = [3, 0, 70, 1, 33, 64]


@pytest.mark.parametrize("method", ["step", "chunked"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("opts,max_len", [
    ({}, True), ({}, False),
    (dict(ngroups=2, a_tok=True, premix=True, phase="shuffle"), True),
])
def test_bwd_packed(opts, max_len, io, method):
    """Packed sequences of different lengths (one empty, one of a single
    token), each with its own state record and final-state gradient: the
    gradient runs on the padded batch (max_seqlen = the longest sequence, or
    by default the packed length) and comes back to the packed tokens."""
    lens = PACKED_LENGTHS
    nseq, T = len(lens), sum(lens)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=DEV)
    ngroups, a_tok = opts.get("ngroups", 0), opts.get("a_tok", False)
    phase, premix = opts.get("phase", "native"), opts.get("premix", False)
    w = workload(1, T, 4, 2, 32, 64, io=io, dt_mu=-1.0, theta="uniform_pi")
    say("case bwd packed [%s] %s %s lengths=%s max_seqlen=%s" % (method, io, opts, lens,
                                                               max(lens) if max_len else T))
    inp, ex = synth.make_option_inputs(w, 1400, DEV, ngroups=ngroups, a_per_token=a_tok,
                                       phase=phase, premix=premix)
    g = torch.Generator(device=DEV).manual_seed(1401)
    dy = torch.randn(inp["x"].shape, generator=g, device=DEV).to(w.torch_dtype)
    dh = torch.randn(nseq, w.heads, w.dstate, w.headdim, generator=g, device=DEV)
    st = random_state(w.with_(batch=nseq), 1402, DEV)
    got = m3_scan_bwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"],
                      None if phase == "zero" else inp["theta"], inp["lam"], dy, State(*st), dh,
                      method=method, ngroups=ngroups, phase=phase, perm=ex.get("perm"),
                      premix=opt.premix_obj(ex), A_per_token=a_tok, cu_seqlens=cu,
                      max_seqlen=max(lens) if max_len else None)
    torch.cuda.synchronize()
    ref = scan_backward_packed(f64(inp["x"]), f64(inp["B"]), f64(inp["C"]), f64(inp["dt"]),
                               f64(inp["A"]), f64(inp["theta"]), f64(inp["lam"]),
                               cu.cpu().numpy(), f64(dy), f64(dh), h0=f64(st[0]),
                               Bprev=f64(st[1]), xprev=f64(st[2]),
                               **opt.oracle_kw(ex, ngroups, phase))
    check_grads(got, ref, io, a_tok, premix, phase)


def test_bwd_packed_equal_lengths_match_dense_batch():
    """Four sequences of 64 tokens packed = the dense batch of four: the same
    gradients to rounding (the padded batch is the dense batch)."""
    w = workload(4, 64, 2, 1, 64, 64, io="bf16", dt_mu=-1.0)
    inp = synth.make_scan_inputs(w, 1410, DEV)
    dy = torch.randn(inp["x"].shape, device=DEV,
                     generator=torch.Generator(device=DEV).manual_seed(1411)).to(torch.bfloat16)
    dense = m3_scan_bwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"],
                        inp["lam"], dy)
    flat = lambda t: t.reshape(1, -1, *t.shape[2:]).contiguous()
    cu = torch.arange(0, 257, 64, dtype=torch.int32, device=DEV)
    packed = m3_scan_bwd(flat(inp["x"]), flat(inp["B"]), flat(inp["C"]), flat(inp["dt"]),
                         inp["A"], flat(inp["theta"]), flat(inp["lam"]), flat(dy), cu_seqlens=cu,
                         max_seqlen=64)
    torch.cuda.synchronize()
    for n in bwd.NAMES:
        a, b = getattr(dense, n), getattr(packed, n)
        if n in ("dx", "dB", "dC", "ddt", "dtheta", "dlam"):
            a = a.reshape(b.shape)
        assert torch.equal(a, b), n


def test_bwd_options_prefill_workload_sampled():
    """The prefill_bf16 shapes (4 x 2048 tokens, 16 heads: 32 chunks of 64
    tokens per head) with 8 head groups of 2, shuffled phases,
    the pre-mixer and A per token, chunked method: every per-token gradient
    of batch row 1 and group 3 (heads 6 and 7) against the oracle run on that
    slice with the same options (one group of two heads, the group's biases)."""
    w = synth.WORKLOADS["prefill_bf16"]
    say("case bwd options prefill_bf16 full size [chunked]")
    inp, ex = synth.make_option_inputs(w, 1500, DEV, ngroups=8, a_per_token=True, phase="shuffle",
                                       premix=True)
    dy = torch.randn(inp["x"].shape, device=DEV,
                     generator=torch.Generator(device=DEV).manual_seed(1501)).to(torch.bfloat16)
    got = m3_scan_bwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"], inp["lam"],
                      dy, method="chunked", ngroups=8, phase="shuffle", perm=ex["perm"],
                      premix=opt.premix_obj(ex), A_per_token=True)
    torch.cuda.synchronize()
    b, g = 1, 3
    hs = slice(2 * g, 2 * g + 2)
    tok = lambda t: f64(t[b:b + 1, :, hs])
    grp = lambda t: f64(t[b:b + 1, :, g:g + 1])
    pm = dict(ex["premix"])
    kw = opt.oracle_kw(ex, 1, "shuffle")
    kw["premix"] = {k: (f64(v[hs]) if k in ("B_bias", "C_bias", "dt_bias") else
                        (f64(v) if torch.is_tensor(v) else v)) for k, v in pm.items()}
    ref = scan_backward(tok(inp["x"]), grp(inp["B"]), grp(inp["C"]), tok(inp["dt"]), tok(inp["A"]),
                        tok(inp["theta"]), tok(inp["lam"]), tok(dy), **kw)
    for n, sel in (("dx", tok), ("dB", grp), ("dC", grp), ("ddt", tok), ("dA", tok),
                   ("dtheta", tok), ("dlam", tok)):
        e = rel_err(sel(getattr(got, n)), ref[n])
        say("   row %d group %d %s rel err %.2e" % (b, g, n, e))
        assert e <= TOL["bf16"], (n, e)


@pytest.mark.parametrize("method", ["step", "chunked"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("opts", [{}, dict(ngroups=2, premix=True, phase="reverse")])
def test_bwd_split_sequence_chains_record_gradients(opts, io, method):
    """A sequence of 150 tokens run as two calls (70 + 80) with the state
    record carried between them: the second call's gradient of its input
    record (dh_in, dB_prev, dx_prev) goes into the first call as dh_out and
    the output record's gradient; the two calls' gradients together are the
    whole sequence's (the oracle on all 150 tokens)."""
    from mamba_selective_ssm_amd import m3_scan_fwd
    ngroups, phase, premix = opts.get("ngroups", 0), opts.get("phase", "native"), opts.get("premix", False)
    w = workload(2, 150, 4, 2, 32, 64, io=io, dt_mu=-1.0, theta="uniform_pi")
    say("case bwd split 70+80 [%s] %s %s" % (method, io, opts))
    inp, ex = synth.make_option_inputs(w, 1600, DEV, ngroups=ngroups, phase=phase, premix=premix)
    g = torch.Generator(device=DEV).manual_seed(1601)
    dy = torch.randn(inp["x"].shape, generator=g, device=DEV).to(w.torch_dtype)
    dh = torch.randn(w.batch, w.heads, w.dstate, w.headdim, generator=g, device=DEV)
    st = random_state(w, 1602, DEV)
    kw = dict(ngroups=ngroups, phase=phase, perm=ex.get("perm"), premix=opt.premix_obj(ex))
    part = lambda t, a, b: t[:, a:b].contiguous()
    cut = 70
    args = lambda a, b: [part(inp[k], a, b) for k in ("x", "B", "C", "dt")] + [inp["A"]] + \
        [part(inp[k], a, b) for k in ("theta", "lam")]
    _, rec = m3_scan_fwd(*args(0, cut), State(*st), **kw)
    g2 = m3_scan_bwd(*args(cut, 150), part(dy, cut, 150), rec, dh, method=method, **kw)
    g1 = m3_scan_bwd(*args(0, cut), part(dy, 0, cut), State(*st), g2.dh_in, method=method,
                     record_grad=(g2.dB_prev, g2.dx_prev), **kw)
    torch.cuda.synchronize()
    ref = scan_backward(f64(inp["x"]), f64(inp["B"]), f64(inp["C"]), f64(inp["dt"]),
                        f64(inp["A"]), f64(inp["theta"]), f64(inp["lam"]), f64(dy), f64(dh),
                        h0=f64(st[0]), Bprev=f64(st[1]), xprev=f64(st[2]),
                        **opt.oracle_kw(ex, ngroups, phase))
    tol = TOL[io]
    cat = lambda n: np.concatenate([f64(getattr(g1, n)), f64(getattr(g2, n))], axis=1)
    errs = {n: rel_err(cat(n), ref[n]) for n in ("dx", "dB", "dC", "ddt", "dtheta", "dlam")}
    errs["dA"] = float(np.max(np.abs(f64(g1.dA) + f64(g2.dA) - ref["dA"])) / np.max(ref["dA_scale"]))
    for n, o in (("dh_in", "dh0"), ("dB_prev", "dBprev"), ("dx_prev", "dxprev")):
        errs[n] = rel_err(f64(getattr(g1, n)), ref[o])
    if premix:
        for n in PREMIX_GRADS:
            s = f64(getattr(g1.premix, n[1:])) + f64(getattr(g2.premix, n[1:]))
            errs[n] = (float(np.max(np.abs(s - ref[n])) / np.max(np.abs(ref["ddt"]).sum(axis=(0, 1))))
                       if n == "ddt_bias" else rel_err(s, ref[n]))
    say("   " + "  ".join("%s %.2e" % (n, e) for n, e in errs.items()) + "  (tol %.0e)" % tol)
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, bad


def test_bwd_record_gradient_without_tokens_reaches_the_input_record():
    """seqlen 0: the output record is the input record, so its gradient is
    the input record's."""
    w = workload(2, 0, 3, 2, 32, 64, io="bf16", dt_mu=-1.0)
    inp = synth.make_scan_inputs(w, 1610, DEV)
    st = random_state(w, 1611, DEV)
    g = torch.Generator(device=DEV).manual_seed(1612)
    dBL = torch.randn(2, 3, 2, 64, generator=g, device=DEV)
    dxL = torch.randn(2, 3, 2, 32, generator=g, device=DEV)
    got = m3_scan_bwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"], inp["lam"],
                      torch.empty_like(inp["x"]), State(*st), record_grad=(dBL, dxL))
    torch.cuda.synchronize()
    assert torch.equal(got.dB_prev, dBL) and torch.equal(got.dx_prev, dxL)
    assert torch.count_nonzero(got.dh_in) == 0


@pytest.mark.parametrize("method", ["step", "chunked"])
def test_bwd_record_gradient_follows_the_max_seqlen_cap(method):
    """Packed sequences of 5 and 12 tokens with max_seqlen = 8: the forward
    scans only the first 8 tokens of the second sequence, so its output record
    holds token 8 (packed row 12), and the record's gradient belongs there,
    not on the sequence's last packed row.  With dy = 0 and dh_out = 0 the
    record gradient is the only gradient: dx and dB equal it on each
    sequence's recorded token and vanish on every other scanned token."""
    lens, cap = [5, 12], 8
    cu = torch.tensor([0, 5, 17], dtype=torch.int32, device=DEV)
    w = workload(1, sum(lens), 2, 2, 32, 64, io="f32", dt_mu=-1.0)
    inp = synth.make_scan_inputs(w, 1620, DEV)
    g = torch.Generator(device=DEV).manual_seed(1621)
    dBL = torch.randn(2, 2, 2, 64, generator=g, device=DEV)
    dxL = torch.randn(2, 2, 2, 32, generator=g, device=DEV)
    say("case bwd record gradient with a max_seqlen cap [%s] lengths=%s cap=%d" % (method, lens, cap))
    got = m3_scan_bwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"], inp["lam"],
                      torch.zeros_like(inp["x"]), method=method, cu_seqlens=cu, max_seqlen=cap,
                      record_grad=(dBL, dxL))
    torch.cuda.synchronize()
    rec_row = {0: 4, 1: 5 + cap - 1}
    scanned = list(range(0, 5)) + list(range(5, 5 + cap))
    for s, row in rec_row.items():
        assert torch.equal(got.dx[0, row], dxL[s]), (s, row)
        assert torch.equal(got.dB[0, row], dBL[s]), (s, row)
    others = [r for r in scanned if r not in rec_row.values()]
    assert torch.count_nonzero(got.dx[0, others]) == 0
    assert torch.count_nonzero(got.dB[0, others]) == 0
