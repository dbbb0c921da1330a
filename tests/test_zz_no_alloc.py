"""m3_scan_fwd_noalloc (the scan for callers that cannot allocate: its scratch
is the library's static device array) against m3_scan_fwd with a workspace,
through the C ABI.

Both entry points run the same kernels in the same decomposition, so their
outputs must agree bit for bit; each call is also checked against the fp64
oracle at the usual tolerances (1e-4 float32, 2e-2 bfloat16).  Consecutive
calls share the array and it keeps the last call's contents, so the tests make
several calls in a row, a smaller one after a larger one.
"""
import numpy as np
import pytest
import torch

from mamba_selective_ssm_amd import State, m3_scan_fwd, m3_scan_fwd_noalloc, synth
from helpers import TOL, f64, oracle_scan, random_state, rel_err, say, workload

pytestmark = pytest.mark.gpu
DEV = "cuda"
KEYS = ("x", "B", "C", "dt", "A", "theta", "lam")


def empty_like_state(st):
    return State(torch.empty_like(st.h), torch.empty_like(st.B_prev), torch.empty_like(st.x_prev))


def check_call(w, seed, segments, label):
    say("case noalloc %s: %s segments=%d seed=%d" % (label, w, segments, seed))
    inp = synth.make_scan_inputs(w, seed, DEV)
    st0 = random_state(w, seed + 1, DEV)
    args = [inp[k] for k in KEYS]
    y_ref, s_ref = m3_scan_fwd(*args, State(*st0), segments=segments)
    y = torch.full_like(y_ref, float("nan"))
    so = empty_like_state(s_ref)
    y_got, s_got = m3_scan_fwd_noalloc(*args, State(*st0), segments=segments, y=y, state_out=so)
    torch.cuda.synchronize()
    assert y_got is y and s_got is so
    assert torch.equal(y, y_ref)
    assert torch.equal(so.h, s_ref.h)
    assert torch.equal(so.B_prev, s_ref.B_prev) and torch.equal(so.x_prev, s_ref.x_prev)
    yr, hr, br, xr = oracle_scan(inp, st0)
    ey, eh = rel_err(f64(y), yr), rel_err(f64(so.h), hr)
    say("   bitwise equal to m3_scan_fwd; vs oracle: y %.3e  state %.3e" % (ey, eh))
    assert ey <= TOL[w.io_dtype] and eh <= TOL[w.io_dtype]
    np.testing.assert_array_equal(f64(so.B_prev), br)


def test_noalloc_two_calls_second_smaller():
    """A segmented bf16 call (six segments: records in the scratch array), then
    a smaller float32 call with three segments that reuses the same array."""
    check_call(workload(2, 1500, 3, 1, 64, 64, io="bf16", dt_mu=-1.0), 801, 6, "large")
    check_call(workload(1, 700, 2, 2, 32, 64, io="f32", dt_mu=-1.0), 802, 3, "smaller")


def test_noalloc_in_place_record_and_accumulated_angle():
    """The scratch also holds the copy of an in-place state record and the
    accumulated angle's partial sums."""
    w = workload(2, 900, 4, 1, 64, 64, io="bf16", dt_mu=-1.0)
    say("case noalloc in-place record + phase_out: %s segments=4" % (w,))
    inp = synth.make_scan_inputs(w, 803, DEV)
    args = [inp[k] for k in KEYS]
    st0 = random_state(w, 804, DEV)
    rec_a = State(*(t.clone() for t in st0))
    rec_b = State(*(t.clone() for t in st0))
    ph_a = torch.zeros(w.batch, w.heads, w.dstate // 2, device=DEV)
    ph_b = torch.zeros_like(ph_a)
    for part in (slice(0, 500), slice(500, 900)):
        sub = [a if k == "A" else a[:, part].contiguous() for k, a in zip(KEYS, args)]
        y_a, _ = m3_scan_fwd(*sub, rec_a, state_out=rec_a, segments=4, phase_in=ph_a, phase_out=ph_a)
        y_b = torch.empty_like(y_a)
        m3_scan_fwd_noalloc(*sub, rec_b, state_out=rec_b, segments=4, y=y_b, phase_in=ph_b,
                            phase_out=ph_b)
        torch.cuda.synchronize()
        assert torch.equal(y_a, y_b)
    for a, b in zip(rec_a, rec_b):
        assert torch.equal(a, b)
    assert torch.equal(ph_a, ph_b)
    yr, hr, br, xr = oracle_scan(inp, st0)
    eh = rel_err(f64(rec_b.h), hr)
    say("   in-place record after 500 + 400 tokens vs oracle: state %.3e" % eh)
    assert eh <= TOL["bf16"]


def test_noalloc_single_layer_workload():
    """The single-layer prefill workload in the library's own segmentation
    (about 7.5 MB of segment records), then a small call, then the workload
    again: every call bit for bit equal to m3_scan_fwd."""
    w = synth.WORKLOADS["prefill_bf16"]
    say("case noalloc prefill_bf16 full size")
    inp = synth.make_scan_inputs(w, 805, DEV)
    args = [inp[k] for k in KEYS]
    y_ref, s_ref = m3_scan_fwd(*args)
    for i in range(2):
        y, so = m3_scan_fwd_noalloc(*args)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(so.h, s_ref.h), i
        if i == 0:
            check_call(workload(1, 300, 2, 4, 16, 32, io="f32", dt_mu=0.0), 806, 2, "between")
