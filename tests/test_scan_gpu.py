"""Parity of the HIP prefill (m3_scan_fwd) against the fp64 oracle.

Tolerances (max |y_gpu - y_ref| / max |y_ref| over the tensor, same metric for
the final state): 1e-4 for float32 I/O, 2e-2 for bfloat16 I/O.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from mamba_selective_ssm_amd import State, m3_scan_fwd, m3_scan_workspace_bytes, synth
from helpers import TOL, f64, oracle_scan, random_state, rel_err, say, workload

pytestmark = pytest.mark.gpu
DEV = "cuda"


def check_scan(w, seed, with_state=False, chunk=0, p_split=0, segments=0, label=""):
    say("case %s: B%d L%d H%d R%d P%d N%d %s chunk=%d p_split=%d seg=%d state=%s seed=%d" % (
        label, w.batch, w.seqlen, w.heads, w.rank, w.headdim, w.dstate, w.io_dtype, chunk,
        p_split, segments, with_state, seed))
    inp = synth.make_scan_inputs(w, seed, DEV)
    st = random_state(w, seed + 7, DEV) if with_state else None
    y, so = m3_scan_fwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"],
                        inp["lam"], State(*st) if st else None, chunk=chunk, p_split=p_split,
                        segments=segments)
    torch.cuda.synchronize()
    yr, hr, br, xr = oracle_scan(inp, st)
    tol = TOL[w.io_dtype]
    ey, eh = rel_err(f64(y), yr), rel_err(f64(so.h), hr)
    say("   rel err y %.3e  state %.3e  (tol %.0e)" % (ey, eh, tol))
    assert ey <= tol and eh <= tol, (ey, eh)
    np.testing.assert_array_equal(f64(so.B_prev), br)
    np.testing.assert_array_equal(f64(so.x_prev), xr)
    return y, so


def test_tiny_f32_workload():
    """1 x 1 head, L=64, P=16, N=16, R=1, fp32: the oracle-sized workload."""
    w = synth.WORKLOADS["tiny_f32"]
    check_scan(w, 1000, label="tiny_f32")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N,R", [(16, 1), (32, 2), (64, 4), (128, 1), (128, 4), (64, 1), (16, 4)])
def test_shapes_ragged_with_state(io, N, R):
    """Several chunks plus a ragged tail, random initial state record."""
    w = workload(2, 157, 3, R, 32, N, io=io, dt_mu=0.0, theta="uniform_pi")
    check_scan(w, 11 + N + R, with_state=True, label="ragged")


@pytest.mark.parametrize("L", [0, 1, 2, 63, 64, 65])
def test_short_and_empty_sequences(L):
    w = workload(1, L, 2, 2, 16, 32, io="f32", dt_mu=0.0, theta="uniform_pi")
    check_scan(w, 30 + L, with_state=True, label="short")


@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_chunk_invariance_bf16(chunk):
    w = workload(1, 700, 4, 1, 64, 64, io="bf16")
    check_scan(w, 5, with_state=True, chunk=chunk, label="chunk")


@pytest.mark.parametrize("R,chunk", [(1, 128), (4, 32)])
@pytest.mark.parametrize("segments", [0, 3])
def test_one_chunk_buffer_variants(R, chunk, segments):
    """128 operand rows per chunk at dstate 128 (one LDS chunk buffer, the
    prepared rows held in registers across a second barrier per chunk): a
    ragged tail, a random state record, with and without segments."""
    w = workload(2, 1000 + 37, 3, R, 64, 128, io="bf16", dt_mu=-1.0)
    check_scan(w, 90 + R + segments, with_state=True, chunk=chunk, segments=segments,
               label="one-buffer")


@pytest.mark.parametrize("p_split", [1, 4])
def test_headdim_split_invariance(p_split):
    w = workload(2, 300, 2, 1, 64, 64, io="bf16")
    check_scan(w, 6, with_state=True, p_split=p_split, label="psplit")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("segments", [2, 3, 5])
def test_sequence_segments(io, segments):
    """Segmented scans (state pass + output pass) with ragged chunk counts."""
    w = workload(2, 1000, 3, 2, 32, 64, io=io, dt_mu=-1.0)
    check_scan(w, 50 + segments, with_state=True, segments=segments, label="segments")


def test_sequence_segments_fast_rotation_slow_decay():
    """Large angles and slow decay carry the state across many segments."""
    w = workload(1, 2000, 2, 1, 16, 32, io="f32", dt_mu=-4.0, theta="uniform_pi")
    check_scan(w, 61, with_state=True, segments=7, label="segments-slow")


def test_split_scan_equals_one_scan():
    """The state record carries everything: scan(L1) then scan(L2) == scan(L1+L2)."""
    w = workload(2, 320, 3, 2, 32, 64, io="f32", dt_mu=-1.0)
    say("case split: %s" % (w,))
    inp = synth.make_scan_inputs(w, 77, DEV)
    y, so = m3_scan_fwd(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["theta"], inp["lam"])
    L1 = 131
    part = lambda sl: [inp[k][:, sl].contiguous() if k != "A" else inp[k]
                       for k in ("x", "B", "C", "dt", "A", "theta", "lam")]
    y1, s1 = m3_scan_fwd(*part(slice(0, L1)))
    y2, s2 = m3_scan_fwd(*part(slice(L1, None)), s1)
    torch.cuda.synchronize()
    assert rel_err(f64(torch.cat([y1, y2], 1)), f64(y)) < 1e-5
    assert rel_err(f64(s2.h), f64(so.h)) < 1e-5


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("segments,p_split", [(1, 0), (1, 4), (5, 0), (3, 4)])
def test_split_scan_with_the_record_in_place(io, segments, p_split):
    """A sequence of 1000 tokens run as calls of 333, 1, 400 and 266 tokens
    that update one state record in place (state_out is state_in), with
    forced sequence segments and headdim slices: y of every call and the final
    record against the oracle on the whole sequence."""
    w = workload(2, 1000, 3, 1, 64, 64, io=io, dt_mu=-1.0)
    say("case in-place record split: %s segments=%d p_split=%d" % (w, segments, p_split))
    inp = synth.make_scan_inputs(w, 78, DEV)
    st0 = random_state(w, 79, DEV)
    rec = State(st0[0].clone(), st0[1].clone(), st0[2].clone())
    ys, a = [], 0
    for b in (333, 334, 734, 1000):
        part = [inp[k][:, a:b].contiguous() if k != "A" else inp[k]
                for k in ("x", "B", "C", "dt", "A", "theta", "lam")]
        y, out = m3_scan_fwd(*part, rec, state_out=rec, segments=segments, p_split=p_split)
        assert out is rec
        ys.append(y)
        a = b
    torch.cuda.synchronize()
    yr, hr, br, xr = oracle_scan(inp, st0)
    tol = TOL[io]
    ey, eh = rel_err(f64(torch.cat(ys, 1)), yr), rel_err(f64(rec.h), hr)
    say("   rel err y %.3e  state %.3e" % (ey, eh))
    assert ey <= tol and eh <= tol
    np.testing.assert_array_equal(f64(rec.B_prev), br)
    np.testing.assert_array_equal(f64(rec.x_prev), xr)


def test_hand_set_parity_tracking_exact_sign():
    """theta_t = pi * bit_t, A = 0, dt = 1, lam = 1, B = 0, h0 = C = e_1:
    y_t = (-1)^(number of ones so far), for 4096 tokens through 64 chunks."""
    L, N, P = 4096, 16, 16
    g = torch.Generator().manual_seed(3)
    bits = torch.randint(0, 2, (L,), generator=g)
    x = torch.zeros(1, L, 1, 1, P, device=DEV)
    Bm = torch.zeros(1, L, 1, 1, N, device=DEV)
    Cm = torch.zeros(1, L, 1, 1, N, device=DEV)
    Cm[..., 0] = 1.0
    dt = torch.ones(1, L, 1, device=DEV)
    lam = torch.ones(1, L, 1, device=DEV)
    A = torch.zeros(1, device=DEV)
    theta = torch.zeros(1, L, 1, N // 2, device=DEV)
    theta[0, :, 0, 0] = math.pi * bits.float().to(DEV)
    h0 = torch.zeros(1, 1, N, P, device=DEV)
    h0[0, 0, 0, :] = 1.0
    st = State(h0, torch.zeros(1, 1, 1, N, device=DEV), torch.zeros(1, 1, 1, P, device=DEV))
    y, _ = m3_scan_fwd(x, Bm, Cm, dt, A, theta, lam, st)
    torch.cuda.synchronize()
    parity = torch.cumsum(bits, 0) % 2
    expect = 1.0 - 2.0 * parity.double()
    got = y[0, :, 0, 0, :].double().cpu()
    assert torch.all(torch.sign(got) == expect[:, None])
    assert float((got - expect[:, None]).abs().max()) < 1e-3


def test_segment_workspace_reused_and_uncleared():
    """The workspace of a segmented call holds only that call's records: one
    filled with arbitrary bytes and reused across calls gives the same result
    every time."""
    w = workload(2, 1500, 3, 1, 64, 64, io="bf16", dt_mu=-1.0)
    say("case workspace reuse: %s segments=6" % (w,))
    inp = synth.make_scan_inputs(w, 71, DEV)
    args = [inp[k] for k in ("x", "B", "C", "dt", "A", "theta", "lam")]
    need = m3_scan_workspace_bytes(inp["x"], inp["B"], segments=6)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)
    outs = []
    for _ in range(3):
        y, so = m3_scan_fwd(*args, segments=6, workspace=ws)
        outs.append((y.clone(), so.h.clone()))
    torch.cuda.synchronize()
    yr, hr, _, _ = oracle_scan(inp, None)
    for y, h in outs:
        assert rel_err(f64(y), yr) <= TOL["bf16"] and rel_err(f64(h), hr) <= TOL["bf16"]
        assert torch.equal(y, outs[0][0]) and torch.equal(h, outs[0][1])


def test_segment_workspace_reused_with_new_inputs():
    """One workspace (filled with arbitrary bytes first) reused by segmented
    calls on different inputs, with shapes that change the record layout
    between calls: each call reads only the records it wrote, so each matches
    the oracle on its own inputs."""
    shapes = [(2, 1500, 3, 6), (2, 1500, 3, 6), (1, 2100, 4, 9), (2, 1500, 3, 5), (3, 800, 2, 4)]
    ws = torch.full((1 << 22,), 0x5A, dtype=torch.uint8, device=DEV)
    for i, (Bt, L, H, seg) in enumerate(shapes):
        w = workload(Bt, L, H, 1, 64, 64, io="bf16", dt_mu=-1.0)
        say("case workspace reuse %d: %s segments=%d" % (i, w, seg))
        inp = synth.make_scan_inputs(w, 500 + i, DEV)
        args = [inp[k] for k in ("x", "B", "C", "dt", "A", "theta", "lam")]
        assert m3_scan_workspace_bytes(inp["x"], inp["B"], segments=seg) <= ws.numel()
        y, so = m3_scan_fwd(*args, segments=seg, workspace=ws)
        torch.cuda.synchronize()
        yr, hr, _, _ = oracle_scan(inp, None)
        ey, eh = rel_err(f64(y), yr), rel_err(f64(so.h), hr)
        say("   rel err y %.3e  state %.3e" % (ey, eh))
        assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_segmented_scan_graph_replays():
    """A segmented scan captured in a HIP graph: every replay (with eager work
    and synchronisation between replays) equals the eager call."""
    w = workload(2, 1200, 4, 1, 64, 64, io="bf16", dt_mu=-1.0)
    say("case graph replay: %s segments=5" % (w,))
    inp = synth.make_scan_inputs(w, 72, DEV)
    args = [inp[k] for k in ("x", "B", "C", "dt", "A", "theta", "lam")]
    need = m3_scan_workspace_bytes(inp["x"], inp["B"], segments=5)
    ws = torch.zeros((need,), dtype=torch.uint8, device=DEV)
    y_ref, s_ref = m3_scan_fwd(*args, segments=5, workspace=ws)
    y = torch.empty_like(y_ref)
    st = State(torch.empty_like(s_ref.h), torch.empty_like(s_ref.B_prev), torch.empty_like(s_ref.x_prev))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            m3_scan_fwd(*args, segments=5, workspace=ws, y=y, state_out=st)
    torch.cuda.synchronize()
    for i in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), i
        assert torch.equal(st.h, s_ref.h), i
        _ = (inp["x"].float() * 2).sum().item()      # eager work between replays
