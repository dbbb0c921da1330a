"""Pins for the fp64 oracle: each test checks it against something other than
itself -- a closed form, a library routine, an independent formulation of the
same method from the pages, an exact worked example, or brute force.

Sources (pages, by title and section):
  [KO]  Mamba-3 summary on b-lab.team (Korean): section 1 "Exponential-
        Trapezoidal Discretization" (recurrence, alpha/beta/gamma, lam limits,
        two-band mask), section 2 "Complex-Valued SSM" (complex SSM, real
        block-rotation form = Proposition 2, RoPE trick = Proposition 3),
        section 3 "MIMO".
  [TAI] Towards AI explainer of Mamba-3: section II (trapezoid error orders,
        "decay mask times a size-two convolutional mask"), section III (parity
        tracking with data-dependent RoPE).
  [OSC] Summary of "Understanding Mamba-3 Through Oscillatory Dynamics":
        section 3 (each decay-rotation step is the exact flow of a fixed
        generator), appendix on accumulation under persistent forcing, and the
        learned phase increments of about 180 deg (parity) and 120 deg (mod 3).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.signal

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(rng, Bt, L, H, R, P, N, lam=None, theta_scale=1.0):
    x = rng.standard_normal((Bt, L, H, R, P))
    Bm = rng.standard_normal((Bt, L, H, R, N))
    Cm = rng.standard_normal((Bt, L, H, R, N))
    dt = np.log1p(np.exp(rng.standard_normal((Bt, L, H))))
    A = -np.exp(rng.uniform(-1, 1, size=H))
    theta = rng.uniform(-math.pi, math.pi, size=(Bt, L, H, N // 2)) * theta_scale
    if lam is None:
        lam = 1.0 / (1.0 + np.exp(-rng.standard_normal((Bt, L, H))))
    else:
        lam = np.full((Bt, L, H), float(lam))
    return x, Bm, Cm, dt, A, theta, lam


def rel_err(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------------------
# [KO] s1: lam = 1 is Mamba-2's exponential-Euler rule.  With theta = 0 and
# constant B, C, dt the system is LTI, and the output is a first-order IIR
# filter of x: y = lfilter([dt * C.B], [1, -alpha], x).
def test_lambda_one_is_euler_lti_lfilter():
    rng = np.random.default_rng(1)
    L, P, N = 200, 3, 6
    b = rng.standard_normal(N)
    c = rng.standard_normal(N)
    d, A = 0.37, -0.8
    x = rng.standard_normal((1, L, 1, 1, P))
    Bm = np.broadcast_to(b, (1, L, 1, 1, N))
    Cm = np.broadcast_to(c, (1, L, 1, 1, N))
    dt = np.full((1, L, 1), d)
    lam = np.ones((1, L, 1))
    theta = np.zeros((1, L, 1, N // 2))
    y, h, _, _ = oracle.scan(x, Bm, Cm, dt, np.array([A]), theta, lam)
    alpha = math.exp(d * A)
    for p in range(P):
        ref = scipy.signal.lfilter([d * float(c @ b)], [1.0, -alpha], x[0, :, 0, 0, p])
        np.testing.assert_allclose(y[0, :, 0, 0, p], ref, rtol=1e-12, atol=1e-12)


# [KO] s1: lam = 1, theta = 0 with time-varying inputs is the Mamba-2 recurrence
# h_t = exp(dt_t A) h_{t-1} + dt_t B_t x_t^T (no previous-endpoint term, no
# rotation), including MIMO input summation and per-rank readout.
def test_lambda_one_theta_zero_is_mamba2_time_varying():
    rng = np.random.default_rng(2)
    Bt, L, H, R, P, N = 2, 37, 3, 2, 4, 8
    x, Bm, Cm, dt, A, theta, lam = rand_inputs(rng, Bt, L, H, R, P, N, lam=1.0)
    theta[:] = 0.0
    h0 = rng.standard_normal((Bt, H, N, P))
    y, hL, _, _ = oracle.scan(x, Bm, Cm, dt, A, theta, lam, h0=h0,
                              Bprev=rng.standard_normal((Bt, H, R, N)),
                              xprev=rng.standard_normal((Bt, H, R, P)))
    for b in range(Bt):
        for hh in range(H):
            h = h0[b, hh].copy()
            for t in range(L):
                h = math.exp(dt[b, t, hh] * A[hh]) * h + dt[b, t, hh] * (Bm[b, t, hh].T @ x[b, t, hh])
                np.testing.assert_allclose(y[b, t, hh], Cm[b, t, hh] @ h, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(hL[b, hh], h, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# [KO] s1 / [TAI] s.II: the trapezoid (lam = 1/2) has global error O(dt^2), the
# Euler rule (lam = 1) and the left-endpoint rule (lam = 0) O(dt).  Pinned
# against the closed-form solution of the continuous complex SSM
# z' = (a + i w) z + b u(t), u = cos(nu t), over [0, T]:
#   z(T) = b/2 [ (e^{i nu T} - e^{sT})/(i nu - s) + (e^{-i nu T} - e^{sT})/(-i nu - s) ],
# s = a + i w.  The sample u(0) enters through the state record (B_prev, x_prev).
def _trapezoid_error(n, lam_value, a=-0.7, w=2.3, nu=1.7, T=3.0, b=(0.8, -0.5)):
    d = T / n
    t = d * np.arange(1, n + 1)
    x = np.cos(nu * t).reshape(1, n, 1, 1, 1)
    Bm = np.broadcast_to(np.array(b), (1, n, 1, 1, 2))
    Cm = np.zeros((1, n, 1, 1, 2))
    dt = np.full((1, n, 1), d)
    theta = np.full((1, n, 1, 1), w)
    lam = np.full((1, n, 1), lam_value)
    _, hL, _, _ = oracle.scan(x, Bm, Cm, dt, np.array([a]), theta, lam,
                              h0=np.zeros((1, 1, 2, 1)),
                              Bprev=np.array(b).reshape(1, 1, 1, 2),
                              xprev=np.ones((1, 1, 1, 1)))
    s = complex(a, w)
    bc = complex(*b)
    e = complex(0, nu)
    zT = bc * 0.5 * ((np.exp(e * T) - np.exp(s * T)) / (e - s)
                     + (np.exp(-e * T) - np.exp(s * T)) / (-e - s))
    return abs(complex(hL[0, 0, 0, 0], hL[0, 0, 1, 0]) - zT)


@pytest.mark.parametrize("lam_value,order", [(0.5, 2.0), (1.0, 1.0), (0.0, 1.0)])
def test_discretization_order(lam_value, order):
    ns = [100, 200, 400, 800]
    errs = [_trapezoid_error(n, lam_value) for n in ns]
    slope = -np.polyfit(np.log(ns), np.log(errs), 1)[0]
    assert abs(slope - order) < 0.05, (lam_value, slope, errs)


# ---------------------------------------------------------------------------
# [KO] s2, Proposition 2: the complex SSM with h in C^{N/2},
#   h' = Diag(A + i theta) h + (B + i B^) x,   y = Re((C + i C^)^T h),
# discretised with the exponential-trapezoidal rule of s1 (each step's flow is
# exp(dt (A + i theta)), applied to the state and to the previous endpoint),
# equals the real N-state SSM with block rotations.  Real rows (2i, 2i+1) stack
# (Re, Im) of B, and (Re, -Im) of (C + i C^) because the readout is a plain
# transpose.  Native complex128 arithmetic here.
def complex_form(x, Bm, Cm, dt, A, theta, lam, h0, Bprev, xprev):
    Bt, L, H, R, P = x.shape
    N = Bm.shape[-1]
    y = np.zeros((Bt, L, H, R, P))
    hL = np.zeros((Bt, H, N, P))
    for b in range(Bt):
        for hh in range(H):
            z = h0[b, hh, 0::2] + 1j * h0[b, hh, 1::2]                  # [N/2, P]
            Bc = Bprev[b, hh, :, 0::2] + 1j * Bprev[b, hh, :, 1::2]     # [R, N/2]
            Uprev = Bc.T @ xprev[b, hh]                                 # [N/2, P]
            for t in range(L):
                E = np.exp(dt[b, t, hh] * (A[hh] + 1j * theta[b, t, hh]))[:, None]
                Bc = Bm[b, t, hh, :, 0::2] + 1j * Bm[b, t, hh, :, 1::2]
                U = Bc.T @ x[b, t, hh]
                z = (E * z + (1 - lam[b, t, hh]) * dt[b, t, hh] * E * Uprev
                     + lam[b, t, hh] * dt[b, t, hh] * U)
                Cc = Cm[b, t, hh, :, 0::2] - 1j * Cm[b, t, hh, :, 1::2]
                y[b, t, hh] = np.real(Cc @ z)
                Uprev = U
            hL[b, hh, 0::2] = z.real
            hL[b, hh, 1::2] = z.imag
    return y, hL


def test_complex_real_equivalence_mimo():
    rng = np.random.default_rng(3)
    Bt, L, H, R, P, N = 2, 23, 2, 3, 5, 6
    x, Bm, Cm, dt, A, theta, lam = rand_inputs(rng, Bt, L, H, R, P, N)
    h0 = rng.standard_normal((Bt, H, N, P))
    Bp = rng.standard_normal((Bt, H, R, N))
    xp = rng.standard_normal((Bt, H, R, P))
    y, hL, BL, xL = oracle.scan(x, Bm, Cm, dt, A, theta, lam, h0=h0, Bprev=Bp, xprev=xp)
    yc, hc = complex_form(x, Bm, Cm, dt, A, theta, lam, h0, Bp, xp)
    assert rel_err(y, yc) < 1e-12
    assert rel_err(hL, hc) < 1e-12
    np.testing.assert_array_equal(BL, Bm[:, -1])
    np.testing.assert_array_equal(xL, x[:, -1])


# ---------------------------------------------------------------------------
# [KO] s2, Proposition 3 ("RoPE trick"): rotating B and C by the cumulative
# phase Phi_t = sum_{s<=t} dt_s theta_s turns the scan into a rotation-free
# scalar-decay scan: Bbar_t = R(Phi_t)^T B_t, Cbar_t = R(Phi_t)^T C_t,
#   hbar_t = alpha_t hbar_{t-1} + beta_t Bbar_{t-1} X_{t-1} + gamma_t Bbar_t X_t,
#   y_t = Cbar_t^T hbar_t,  and the true state is h_L = R(Phi_L) hbar_L.
def rot_pairs(v, ang, transpose):
    """Apply R(ang) (or its transpose) to adjacent pairs of the last axis of v."""
    c, s = np.cos(ang), np.sin(ang)
    if transpose:
        s = -s
    out = np.empty_like(v)
    out[..., 0::2] = c * v[..., 0::2] - s * v[..., 1::2]
    out[..., 1::2] = s * v[..., 0::2] + c * v[..., 1::2]
    return out


def rope_form(x, Bm, Cm, dt, A, theta, lam, h0, Bprev, xprev):
    Bt, L, H, R, P = x.shape
    N = Bm.shape[-1]
    y = np.zeros((Bt, L, H, R, P))
    hL = np.zeros((Bt, H, N, P))
    for b in range(Bt):
        for hh in range(H):
            Phi = np.cumsum(dt[b, :, hh, None] * theta[b, :, hh], axis=0)   # [L, N/2]
            Bbar = rot_pairs(Bm[b, :, hh], Phi[:, None, :], True)            # [L, R, N]
            Cbar = rot_pairs(Cm[b, :, hh], Phi[:, None, :], True)
            hb = h0[b, hh].copy()
            Uprev = Bprev[b, hh].T @ xprev[b, hh]
            for t in range(L):
                alpha = math.exp(dt[b, t, hh] * A[hh])
                U = Bbar[t].T @ x[b, t, hh]
                hb = (alpha * hb + (1 - lam[b, t, hh]) * dt[b, t, hh] * alpha * Uprev
                      + lam[b, t, hh] * dt[b, t, hh] * U)
                y[b, t, hh] = Cbar[t] @ hb
                Uprev = U
            hL[b, hh] = rot_pairs(hb.T, Phi[-1], False).T
    return y, hL


def test_rope_rewrite():
    rng = np.random.default_rng(4)
    Bt, L, H, R, P, N = 2, 31, 2, 2, 3, 8
    x, Bm, Cm, dt, A, theta, lam = rand_inputs(rng, Bt, L, H, R, P, N)
    h0 = rng.standard_normal((Bt, H, N, P))
    Bp = rng.standard_normal((Bt, H, R, N))
    xp = rng.standard_normal((Bt, H, R, P))
    y, hL, _, _ = oracle.scan(x, Bm, Cm, dt, A, theta, lam, h0=h0, Bprev=Bp, xprev=xp)
    yr, hr = rope_form(x, Bm, Cm, dt, A, theta, lam, h0, Bp, xp)
    assert rel_err(y, yr) < 1e-12
    assert rel_err(hL, hr) < 1e-12


# ---------------------------------------------------------------------------
# [KO] s1 and [TAI] s.II: the trapezoid makes the SSD mask a product of the
# 1-semiseparable decay mask and a size-two (lower bidiagonal) convolution
# mask.  Brute force for a zero initial state:
#   Ldec[t, s] = prod_{k=s+1..t} alpha_k  (s <= t),  0 otherwise
#   D2[s, s] = gamma_s,  D2[s+1, s] = beta_{s+1}
#   y_t = sum_s (Ldec @ D2)[t, s] * Cbar_t^T Bbar_s X_s
def test_two_band_quadratic_form():
    rng = np.random.default_rng(5)
    Bt, L, H, R, P, N = 1, 16, 2, 3, 4, 6
    x, Bm, Cm, dt, A, theta, lam = rand_inputs(rng, Bt, L, H, R, P, N)
    y, _, _, _ = oracle.scan(x, Bm, Cm, dt, A, theta, lam)
    for hh in range(H):
        d, lm = dt[0, :, hh], lam[0, :, hh]
        alpha = np.exp(d * A[hh])
        Ldec = np.zeros((L, L))
        for t in range(L):
            for s in range(t + 1):
                Ldec[t, s] = np.prod(alpha[s + 1:t + 1])
        D2 = np.diag(lm * d) + np.diag(((1 - lm) * d * alpha)[1:], k=-1)
        M = Ldec @ D2
        Phi = np.cumsum(d[:, None] * theta[0, :, hh], axis=0)
        Bbar = rot_pairs(Bm[0, :, hh], Phi[:, None, :], True).reshape(L * R, N)
        Cbar = rot_pairs(Cm[0, :, hh], Phi[:, None, :], True).reshape(L * R, N)
        G = Cbar @ Bbar.T                                      # [(t,r1), (s,r2)]
        Mx = np.kron(M, np.ones((R, R)))                       # mask per token pair
        Y = (Mx * G) @ x[0, :, hh].reshape(L * R, P)
        assert rel_err(y[0, :, hh].reshape(L * R, P), Y) < 1e-12
        # the mask is exactly two-band-structured: zero above the diagonal
        assert np.all(np.triu(M, 1) == 0)


# ---------------------------------------------------------------------------
# [OSC] s3: one homogeneous step (no input) is the exact flow of the generator
# blockdiag([[A, -theta_i], [theta_i, A]]) over dt: exp(dt A) R(dt theta_i).
def test_step_is_generator_exponential():
    rng = np.random.default_rng(6)
    N = 10
    A = np.array([-0.43])
    dt = np.array([[[0.71]]])
    theta = rng.uniform(-3, 3, size=(1, 1, 1, N // 2))
    h0 = np.eye(N).reshape(1, 1, N, N)                        # P = N identity columns
    _, hL, _, _ = oracle.scan(np.zeros((1, 1, 1, 1, N)), np.zeros((1, 1, 1, 1, N)),
                              np.zeros((1, 1, 1, 1, N)), dt, A, theta,
                              np.full((1, 1, 1), 0.5), h0=h0)
    G = np.zeros((N, N))
    for i in range(N // 2):
        G[2 * i:2 * i + 2, 2 * i:2 * i + 2] = [[A[0], -theta[0, 0, 0, i]],
                                               [theta[0, 0, 0, i], A[0]]]
    np.testing.assert_allclose(hL[0, 0], scipy.linalg.expm(dt[0, 0, 0] * G), atol=1e-14)


# ---------------------------------------------------------------------------
# [TAI] s.III and [OSC] (learned increments near 180 deg for parity, 120 deg for
# mod 3): a hand-set data-dependent rotation tracks parity exactly.  A = 0,
# dt = 1, lam = 1, B = 0, h_0 = e_1, C = e_1, theta_t = pi b_t
#   => y_t = cos(pi sum_{s<=t} b_s) = (-1)^{parity}.
@pytest.mark.parametrize("modulus", [2, 3])
def test_hand_set_rotation_tracks_parity_and_mod3(modulus):
    rng = np.random.default_rng(7 + modulus)
    L = 4096
    bits = rng.integers(0, 2, size=L)
    theta = (2 * math.pi / modulus * bits).reshape(1, L, 1, 1)
    y, _, _, _ = oracle.scan(np.zeros((1, L, 1, 1, 1)), np.zeros((1, L, 1, 1, 2)),
                             np.broadcast_to(np.array([1.0, 0.0]), (1, L, 1, 1, 2)),
                             np.ones((1, L, 1)), np.zeros(1), theta, np.ones((1, L, 1)),
                             h0=np.array([1.0, 0.0]).reshape(1, 1, 2, 1))
    count = np.cumsum(bits) % modulus
    expect = np.cos(2 * math.pi / modulus * count)
    np.testing.assert_allclose(y[0, :, 0, 0, 0], expect, atol=1e-9)
    if modulus == 2:
        assert np.array_equal(np.sign(y[0, :, 0, 0, 0]), np.where(count == 0, 1.0, -1.0))


# ---------------------------------------------------------------------------
# [OSC] appendix (accumulation under persistent forcing): with constant U,
# alpha, phase phi and lam, the state converges to the fixed point of
# h = alpha R h + beta R U + gamma U, i.e. per pair in complex form
#   h_inf = (beta e^{i phi} + gamma) U / (1 - alpha e^{i phi}).
def test_persistent_forcing_steady_state():
    N, P, L = 6, 2, 3000
    rng = np.random.default_rng(8)
    b = rng.standard_normal(N)
    xv = rng.standard_normal(P)
    d, A, lm = 0.3, -0.35, 0.6
    th = rng.uniform(-2, 2, size=N // 2)
    _, hL, _, _ = oracle.scan(np.broadcast_to(xv, (1, L, 1, 1, P)),
                              np.broadcast_to(b, (1, L, 1, 1, N)),
                              np.zeros((1, L, 1, 1, N)), np.full((1, L, 1), d),
                              np.array([A]), np.broadcast_to(th, (1, L, 1, N // 2)),
                              np.full((1, L, 1), lm))
    alpha = math.exp(d * A)
    beta, gamma = (1 - lm) * d * alpha, lm * d
    for i in range(N // 2):
        e = np.exp(1j * d * th[i])
        U = (b[2 * i] + 1j * b[2 * i + 1]) * xv
        hinf = (beta * e + gamma) * U / (1 - alpha * e)
        np.testing.assert_allclose(hL[0, 0, 2 * i], hinf.real, atol=1e-12)
        np.testing.assert_allclose(hL[0, 0, 2 * i + 1], hinf.imag, atol=1e-12)


# ---------------------------------------------------------------------------
# [KO] s3 (MIMO): the input term B_t X_t sums the R ranks and the readout gives
# one output per rank, so by linearity a rank-R scan is the sum of R x R
# single-rank scans (input rank r, readout rank r').
def test_mimo_is_superposition_of_siso():
    rng = np.random.default_rng(9)
    Bt, L, H, R, P, N = 1, 19, 2, 3, 4, 6
    x, Bm, Cm, dt, A, theta, lam = rand_inputs(rng, Bt, L, H, R, P, N)
    y, hL, _, _ = oracle.scan(x, Bm, Cm, dt, A, theta, lam)
    ysum = np.zeros_like(y)
    hsum = np.zeros_like(hL)
    for r in range(R):
        for r2 in range(R):
            yy, hh, _, _ = oracle.scan(x[..., r:r + 1, :], Bm[..., r:r + 1, :],
                                       Cm[..., r2:r2 + 1, :], dt, A, theta, lam)
            ysum[..., r2, :] += yy[..., 0, :]
            if r2 == 0:
                hsum += hh
    assert rel_err(y, ysum) < 1e-12
    assert rel_err(hL, hsum) < 1e-12


# ---------------------------------------------------------------------------
# The state record (h, B_prev, x_prev) is a checkpoint: a scan split in two,
# or a scan followed by single decode steps, equals one scan.
def test_split_scan_and_decode_equal_one_scan():
    rng = np.random.default_rng(10)
    Bt, L, H, R, P, N = 2, 40, 2, 2, 3, 8
    x, Bm, Cm, dt, A, theta, lam = rand_inputs(rng, Bt, L, H, R, P, N)
    h0 = rng.standard_normal((Bt, H, N, P))
    Bp = rng.standard_normal((Bt, H, R, N))
    xp = rng.standard_normal((Bt, H, R, P))
    args = lambda sl: (x[:, sl], Bm[:, sl], Cm[:, sl], dt[:, sl], A, theta[:, sl], lam[:, sl])
    y, hL, BL, xL = oracle.scan(*args(slice(0, L)), h0=h0, Bprev=Bp, xprev=xp)
    L1 = 17
    y1, h1, B1, x1 = oracle.scan(*args(slice(0, L1)), h0=h0, Bprev=Bp, xprev=xp)
    y2, h2, B2, x2 = oracle.scan(*args(slice(L1, L)), h0=h1, Bprev=B1, xprev=x1)
    np.testing.assert_array_equal(np.concatenate([y1, y2], axis=1), y)
    np.testing.assert_array_equal(h2, hL)
    h, Bs, xs = h1, B1, x1
    for t in range(L1, L):
        yt, h, Bs, xs = oracle.decode_step(x[:, t], Bm[:, t], Cm[:, t], dt[:, t], A,
                                           theta[:, t], lam[:, t], h, Bs, xs)
        np.testing.assert_array_equal(yt, y[:, t])
    np.testing.assert_array_equal(h, hL)
    np.testing.assert_array_equal(Bs, BL)
    np.testing.assert_array_equal(xs, xL)


def test_empty_sequence_passes_state_through():
    rng = np.random.default_rng(11)
    Bt, H, R, P, N = 2, 3, 2, 4, 6
    z = lambda *s: np.zeros(s)
    h0 = rng.standard_normal((Bt, H, N, P))
    Bp = rng.standard_normal((Bt, H, R, N))
    xp = rng.standard_normal((Bt, H, R, P))
    y, hL, BL, xL = oracle.scan(z(Bt, 0, H, R, P), z(Bt, 0, H, R, N), z(Bt, 0, H, R, N),
                                z(Bt, 0, H), -np.ones(H), z(Bt, 0, H, N // 2), z(Bt, 0, H),
                                h0=h0, Bprev=Bp, xprev=xp)
    assert y.shape == (Bt, 0, H, R, P)
    np.testing.assert_array_equal(hL, h0)
    np.testing.assert_array_equal(BL, Bp)
    np.testing.assert_array_equal(xL, xp)


# ---------------------------------------------------------------------------
# A worked example derived by hand (tests/golden/worked_example.json holds the
# inputs, the derivation and the exact expected values).
def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    L = len(g["x"])
    y, hL, BL, xL = oracle.scan(np.array(g["x"], float).reshape(1, L, 1, 1, 1),
                                np.array(g["B"], float).reshape(1, L, 1, 1, 2),
                                np.array(g["C"], float).reshape(1, L, 1, 1, 2),
                                np.array(g["dt"], float).reshape(1, L, 1),
                                np.array([g["A"]], float),
                                np.array(g["theta"], float).reshape(1, L, 1, 1),
                                np.array(g["lam"], float).reshape(1, L, 1))
    np.testing.assert_allclose(y.ravel(), g["expect_y"], atol=1e-12)
    np.testing.assert_allclose(hL.ravel(), g["expect_h"], atol=1e-12)
    np.testing.assert_array_equal(BL.ravel(), g["B"][-1])
    np.testing.assert_array_equal(xL.ravel(), [g["x"][-1]])


# ===========================================================================
# Oracle options: per-token decay, head groups, phase interventions and the
# pre-mixer.  Each is pinned to an independent formulation or a library routine.

# [KO] s1 writes the decay as exp(dt_t A_t).  With lam = 1 and theta = 0 the
# recurrence is Mamba-2's with a time-varying rate, stepped here directly.
# B and C come per head group (head h reads group h // (H/G)) to pin the group
# indexing in the same loop.
def test_per_token_decay_and_groups_are_mamba2_time_varying():
    rng = np.random.default_rng(21)
    Bt, L, H, G, R, P, N = 2, 23, 4, 2, 2, 3, 6
    x = rng.standard_normal((Bt, L, H, R, P))
    Bg = rng.standard_normal((Bt, L, G, R, N))
    Cg = rng.standard_normal((Bt, L, G, R, N))
    dt = np.log1p(np.exp(rng.standard_normal((Bt, L, H))))
    At = -np.exp(rng.uniform(-1, 1, size=(Bt, L, H)))
    theta = rng.uniform(-3, 3, size=(Bt, L, H, N // 2))
    lam = np.ones((Bt, L, H))
    y, hL, BL, _ = oracle.scan(x, Bg, Cg, dt, At, theta, lam, ngroups=G, phase="zero")
    for b in range(Bt):
        for hh in range(H):
            g = hh // (H // G)
            h = np.zeros((N, P))
            for t in range(L):
                h = math.exp(dt[b, t, hh] * At[b, t, hh]) * h + dt[b, t, hh] * (Bg[b, t, g].T @ x[b, t, hh])
                np.testing.assert_allclose(y[b, t, hh], Cg[b, t, g] @ h, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(hL[b, hh], h, rtol=1e-11, atol=1e-12)
            np.testing.assert_array_equal(BL[b, hh], Bg[b, L - 1, g])


def test_per_token_decay_decode_matches_scan():
    rng = np.random.default_rng(22)
    Bt, L, H, G, R, P, N = 2, 9, 4, 2, 2, 3, 6
    x = rng.standard_normal((Bt, L, H, R, P))
    Bg = rng.standard_normal((Bt, L, G, R, N))
    Cg = rng.standard_normal((Bt, L, G, R, N))
    dt = np.log1p(np.exp(rng.standard_normal((Bt, L, H))))
    At = -np.exp(rng.uniform(-1, 1, size=(Bt, L, H)))
    theta = rng.uniform(-3, 3, size=(Bt, L, H, N // 2))
    lam = rng.uniform(0, 1, size=(Bt, L, H))
    y, hL, BL, xL = oracle.scan(x, Bg, Cg, dt, At, theta, lam, ngroups=G)
    z = np.zeros
    h, Bs, xs = z((Bt, H, N, P)), z((Bt, H, R, N)), z((Bt, H, R, P))
    for t in range(L):
        yt, h, Bs, xs = oracle.decode_step(x[:, t], Bg[:, t], Cg[:, t], dt[:, t], At[:, t],
                                           theta[:, t], lam[:, t], h, Bs, xs, ngroups=G)
        np.testing.assert_array_equal(yt, y[:, t])
    np.testing.assert_array_equal(h, hL)
    np.testing.assert_array_equal(Bs, BL)


# [OSC] s5.3: reversing the phase increments.  R(-phi) = D R(phi) D with
# D = diag(1, -1) on every pair, so the reversed system is the native one
# conjugated by D: y_rev(B, C) = y(DB, DC) and h_rev = D h(DB, DC).
def test_reverse_phase_is_reflection_conjugate():
    rng = np.random.default_rng(23)
    Bt, L, H, R, P, N = 2, 31, 2, 2, 3, 8
    x, Bm, Cm, dt, A, theta, lam = rand_inputs(rng, Bt, L, H, R, P, N)
    h0 = rng.standard_normal((Bt, H, N, P))
    Bp = rng.standard_normal((Bt, H, R, N))
    xp = rng.standard_normal((Bt, H, R, P))
    d = np.tile([1.0, -1.0], N // 2)
    y_rev, h_rev, _, _ = oracle.scan(x, Bm, Cm, dt, A, theta, lam, h0=h0, Bprev=Bp, xprev=xp,
                                     phase="reverse")
    y_ref, h_ref, _, _ = oracle.scan(x, Bm * d, Cm * d, dt, A, theta, lam, h0=h0 * d[:, None],
                                     Bprev=Bp * d, xprev=xp)
    assert rel_err(y_rev, y_ref) < 1e-12
    assert rel_err(h_rev, h_ref * d[:, None]) < 1e-12
    # and reversal is not the identity on these inputs
    y_nat, _, _, _ = oracle.scan(x, Bm, Cm, dt, A, theta, lam, h0=h0, Bprev=Bp, xprev=xp)
    assert rel_err(y_rev, y_nat) > 1e-2


# [OSC] App. D.4: shuffling the increments across rotary pairs.  Relabelling
# the pairs is a change of basis: pair i driven by theta[perm[i]] is pair
# perm[i] of a native system whose B, C pairs are moved to position perm[i].
def test_shuffled_phase_is_pair_relabelling():
    rng = np.random.default_rng(24)
    Bt, L, H, R, P, N = 1, 29, 3, 2, 3, 10
    x, Bm, Cm, dt, A, theta, lam = rand_inputs(rng, Bt, L, H, R, P, N)
    perm = rng.permutation(N // 2)
    y_sh, h_sh, _, _ = oracle.scan(x, Bm, Cm, dt, A, theta, lam, phase="shuffle", perm=perm)

    def move(M):   # pair i of M goes to pair perm[i]
        out = np.empty_like(M)
        for i in range(N // 2):
            out[..., 2 * perm[i]:2 * perm[i] + 2] = M[..., 2 * i:2 * i + 2]
        return out
    y_ref, h_ref, _, _ = oracle.scan(x, move(Bm), move(Cm), dt, A, theta, lam)
    assert rel_err(y_sh, y_ref) < 1e-12
    h_back = np.empty_like(h_sh)
    for i in range(N // 2):
        h_back[:, :, 2 * i:2 * i + 2] = h_ref[:, :, 2 * perm[i]:2 * perm[i] + 2]
    assert rel_err(h_sh, h_back) < 1e-12


# [OSC] s5.3: zeroing the phase leaves a rotation-free trapezoid; the output no
# longer depends on theta, and equals the complex SSM with theta = 0.
def test_zero_phase_ignores_theta():
    rng = np.random.default_rng(25)
    Bt, L, H, R, P, N = 1, 17, 2, 1, 3, 6
    x, Bm, Cm, dt, A, theta, lam = rand_inputs(rng, Bt, L, H, R, P, N)
    y0, _, _, _ = oracle.scan(x, Bm, Cm, dt, A, theta, lam, phase="zero")
    y1, _, _, _ = oracle.scan(x, Bm, Cm, dt, A, rng.standard_normal(theta.shape), lam, phase="zero")
    z = np.zeros
    yc, _ = complex_form(x, Bm, Cm, dt, A, np.zeros_like(theta), lam, z((Bt, H, N, P)),
                         z((Bt, H, R, N)), z((Bt, H, R, P)))
    np.testing.assert_array_equal(y0, y1)
    assert rel_err(y0, yc) < 1e-12


# Pre-mixer ([TAI] s.II: QKNorm-style RMSNorm and channel-wise biases on B and
# C; dt and lam through softplus and sigmoid).  Each map against torch's own.
def test_premix_maps_match_torch():
    import torch
    rng = np.random.default_rng(26)
    v = rng.standard_normal((5, 3, 2, 16)) * 3.0
    w = rng.standard_normal(16)
    for eps in (1e-6, 0.5):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(v), (16,), torch.from_numpy(w), eps)
        np.testing.assert_allclose(oracle.rms_norm(v, w, eps), ref.numpy(), rtol=1e-13, atol=1e-14)
    z = np.concatenate([rng.standard_normal(100) * 10.0, [-800.0, -50.0, 0.0, 50.0, 800.0]])
    small = z <= 20.0   # torch returns z itself above its threshold of 20
    np.testing.assert_allclose(oracle.softplus(z[small]),
                               torch.nn.functional.softplus(torch.from_numpy(z[small])).numpy(),
                               rtol=1e-13, atol=1e-300)
    big = z[~small]     # log(1 + e^z) = z + log(1 + e^-z), within e^-z of z
    assert np.all(np.abs(oracle.softplus(big) - big) <= np.exp(-big) + 1e-15 * big)
    np.testing.assert_allclose(oracle.sigmoid(z), torch.sigmoid(torch.from_numpy(z)).numpy(),
                               rtol=1e-13, atol=1e-300)


def _premix_params(rng, H, R, N, eps=1e-5):
    return dict(B_norm_w=rng.uniform(0.5, 1.5, N), C_norm_w=rng.uniform(0.5, 1.5, N),
                B_bias=0.3 * rng.standard_normal((H, R, N)),
                C_bias=0.3 * rng.standard_normal((H, R, N)),
                dt_bias=rng.uniform(-2.0, 0.0, H), eps=eps)


# With the pre-mixer the scan consumes RMSNorm(B)*w + b (torch's rms_norm),
# softplus(dt + dt_bias) and sigmoid(lam).  RMS normalisation also makes the
# output invariant to a positive rescaling of each B or C row.
def test_premix_scan_consumes_torch_maps():
    import torch
    rng = np.random.default_rng(27)
    Bt, L, H, G, R, P, N = 2, 13, 4, 2, 2, 3, 8
    x = rng.standard_normal((Bt, L, H, R, P))
    Bg = rng.standard_normal((Bt, L, G, R, N))
    Cg = rng.standard_normal((Bt, L, G, R, N))
    dt_raw = rng.standard_normal((Bt, L, H))
    lam_raw = rng.standard_normal((Bt, L, H))
    A = -np.exp(rng.uniform(-1, 1, size=H))
    theta = rng.uniform(-3, 3, size=(Bt, L, H, N // 2))
    pm = _premix_params(rng, H, R, N)
    y, hL, BL, _ = oracle.scan(x, Bg, Cg, dt_raw, A, theta, lam_raw, ngroups=G, premix=pm)

    T = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    Bh = np.repeat(Bg, H // G, axis=2)
    Ch = np.repeat(Cg, H // G, axis=2)
    Bn = (torch.nn.functional.rms_norm(T(Bh), (N,), T(pm["B_norm_w"]), pm["eps"]) + T(pm["B_bias"])).numpy()
    Cn = (torch.nn.functional.rms_norm(T(Ch), (N,), T(pm["C_norm_w"]), pm["eps"]) + T(pm["C_bias"])).numpy()
    dt = torch.nn.functional.softplus(T(dt_raw) + T(pm["dt_bias"])).numpy()
    lam = torch.sigmoid(T(lam_raw)).numpy()
    y_ref, h_ref, B_ref, _ = oracle.scan(x, Bn, Cn, dt, A, theta, lam)
    assert rel_err(y, y_ref) < 1e-12
    assert rel_err(hL, h_ref) < 1e-12
    assert rel_err(BL, B_ref) < 1e-13

    scale = rng.uniform(0.2, 5.0, size=(Bt, L, G, R, 1))
    pm0 = dict(pm, eps=0.0)
    ya, _, _, _ = oracle.scan(x, Bg, Cg, dt_raw, A, theta, lam_raw, ngroups=G, premix=pm0)
    yb, _, _, _ = oracle.scan(x, Bg * scale, Cg / scale, dt_raw, A, theta, lam_raw, ngroups=G,
                              premix=pm0)
    assert rel_err(yb, ya) < 1e-12


# Packed sequences are independent scans: equal lengths give the dense batch,
# and reordering the sequences reorders the outputs and records.
def test_packed_sequences_match_dense_batch_and_reorder():
    rng = np.random.default_rng(28)
    Bt, L, H, R, P, N = 3, 11, 2, 2, 3, 6
    x, Bm, Cm, dt, A, theta, lam = rand_inputs(rng, Bt, L, H, R, P, N)
    h0 = rng.standard_normal((Bt, H, N, P))
    Bp = rng.standard_normal((Bt, H, R, N))
    xp = rng.standard_normal((Bt, H, R, P))
    pack = lambda a: a.reshape((1, Bt * L) + a.shape[2:])
    cu = np.arange(Bt + 1) * L
    yd, hd, Bd, xd = oracle.scan(x, Bm, Cm, dt, A, theta, lam, h0=h0, Bprev=Bp, xprev=xp)
    yp, hp, Bpk, xpk = oracle.scan_packed(pack(x), pack(Bm), pack(Cm), pack(dt), A, pack(theta),
                                          pack(lam), cu, h0=h0, Bprev=Bp, xprev=xp)
    np.testing.assert_array_equal(yp.reshape(yd.shape), yd)
    np.testing.assert_array_equal(hp, hd)
    np.testing.assert_array_equal(Bpk, Bd)
    # ragged lengths (one empty), then the same sequences in reverse order
    lens = [5, 0, 9, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    xx, BB, CC, dd, _, tt, ll = rand_inputs(rng, 1, T, H, R, P, N)
    hh = rng.standard_normal((4, H, N, P))
    y1, h1, _, _ = oracle.scan_packed(xx, BB, CC, dd, A, tt, ll, cu, h0=hh,
                                      Bprev=np.zeros((4, H, R, N)), xprev=np.zeros((4, H, R, P)))
    order = [3, 2, 1, 0]
    idx = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in order]).astype(int)
    cu_r = np.concatenate([[0], np.cumsum([lens[i] for i in order])])
    y2, h2, _, _ = oracle.scan_packed(xx[:, idx], BB[:, idx], CC[:, idx], dd[:, idx], A,
                                      tt[:, idx], ll[:, idx], cu_r, h0=hh[order],
                                      Bprev=np.zeros((4, H, R, N)), xprev=np.zeros((4, H, R, P)))
    np.testing.assert_array_equal(y2, y1[:, idx])
    np.testing.assert_array_equal(h2, h1[order])
    np.testing.assert_array_equal(h1[1], hh[1])      # the empty sequence passes its state through


# ===========================================================================
# Gradient oracle (oracle/backward.py): its forward equals the C oracle, and
# every gradient matches central finite differences of the C oracle's loss.
def _bwd_case(rng, Bt=1, L=7, H=2, R=2, P=3, N=4):
    x, Bm, Cm, dt, A, theta, lam = rand_inputs(rng, Bt, L, H, R, P, N)
    h0 = rng.standard_normal((Bt, H, N, P))
    Bp = rng.standard_normal((Bt, H, R, N))
    xp = rng.standard_normal((Bt, H, R, P))
    dy = rng.standard_normal((Bt, L, H, R, P))
    dh = rng.standard_normal((Bt, H, N, P))
    return [x, Bm, Cm, dt, A, theta, lam, h0, Bp, xp], dy, dh


def test_backward_forward_matches_c_oracle():
    import torch
    from oracle.backward import forward_torch
    rng = np.random.default_rng(31)
    ins, _, _ = _bwd_case(rng, Bt=2, L=13, H=2, R=2, P=3, N=6)
    y_c, h_c, _, _ = oracle.scan(*ins[:7], h0=ins[7], Bprev=ins[8], xprev=ins[9])
    y_t, h_t = forward_torch(*[torch.tensor(a) for a in ins])
    assert rel_err(y_t.numpy(), y_c) < 1e-13
    assert rel_err(h_t.numpy(), h_c) < 1e-13


def test_backward_matches_finite_differences():
    from oracle.backward import scan_backward
    rng = np.random.default_rng(32)
    ins, dy, dh = _bwd_case(rng)
    g = scan_backward(*ins[:7], dy, dh, h0=ins[7], Bprev=ins[8], xprev=ins[9])

    def loss(args):
        y, hL, _, _ = oracle.scan(*args[:7], h0=args[7], Bprev=args[8], xprev=args[9])
        return float(np.sum(y * dy) + np.sum(hL * dh))
    names = ["dx", "dB", "dC", "ddt", "dA", "dtheta", "dlam", "dh0", "dBprev", "dxprev"]
    eps = 1e-6
    for k, name in enumerate(names):
        fd = np.zeros_like(ins[k])
        it = np.nditer(ins[k], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [a.copy() for a in ins]
            minus = [a.copy() for a in ins]
            plus[k][idx] += eps
            minus[k][idx] -= eps
            fd[idx] = (loss(plus) - loss(minus)) / (2 * eps)
        err = np.max(np.abs(fd - g[name])) / max(np.max(np.abs(g[name])), 1e-12)
        assert err < 1e-6, (name, err)


def test_backward_dA_terms_match_finite_differences():
    """dA is the sum over (b, t) of the loss's derivative with respect to a
    per-token decay rate: with A given per token to the C oracle, central
    differences of its loss reproduce each term, their sum is dA and the sum
    of their absolute values is dA_scale."""
    from oracle.backward import scan_backward
    rng = np.random.default_rng(33)
    ins, dy, dh = _bwd_case(rng, Bt=2, L=5, H=2, R=1, P=3, N=4)
    g = scan_backward(*ins[:7], dy, dh, h0=ins[7], Bprev=ins[8], xprev=ins[9])
    Bt, L, H = ins[3].shape
    A_tok = np.broadcast_to(ins[4], (Bt, L, H)).copy()

    def loss(At):
        y, hL, _, _ = oracle.scan(*ins[:4], At, *ins[5:7], h0=ins[7], Bprev=ins[8], xprev=ins[9])
        return float(np.sum(y * dy) + np.sum(hL * dh))
    eps = 1e-6
    terms = np.zeros((Bt, L, H))
    for idx in np.ndindex(Bt, L, H):
        plus, minus = A_tok.copy(), A_tok.copy()
        plus[idx] += eps
        minus[idx] -= eps
        terms[idx] = (loss(plus) - loss(minus)) / (2 * eps)
    scale = np.abs(terms).sum(axis=(0, 1))
    assert np.max(np.abs(terms.sum(axis=(0, 1)) - g["dA"])) / np.max(scale) < 1e-6
    assert np.max(np.abs(scale - g["dA_scale"])) / np.max(scale) < 1e-6
    assert np.all(g["dA_scale"] >= np.abs(g["dA"]) - 1e-9)


def _bwd_option_case(rng, ngroups, phase, premix, Bt=1, L=5, H=2, R=2, P=2, N=4, a_tok=False):
    """A gradient case with options: B, C per group, a permutation for
    "shuffle", with the pre-mixer raw dt, lam and its parameters, and A per
    token."""
    ins, dy, dh = _bwd_case(rng, Bt, L, H, R, P, N)
    if a_tok:
        ins[4] = -np.exp(rng.uniform(-1.0, 1.0, (Bt, L, H)))
    if ngroups:
        ins[1] = rng.standard_normal((Bt, L, ngroups, R, N))
        ins[2] = rng.standard_normal((Bt, L, ngroups, R, N))
    kw = dict(ngroups=ngroups or None, phase=phase)
    if phase == "shuffle":
        kw["perm"] = rng.permutation(N // 2)
    pm = None
    if premix:
        ins[3] = rng.standard_normal((Bt, L, H))
        ins[6] = rng.standard_normal((Bt, L, H))
        pm = dict(B_norm_w=rng.uniform(0.5, 1.5, N), C_norm_w=rng.uniform(0.5, 1.5, N),
                  B_bias=0.3 * rng.standard_normal((H, R, N)),
                  C_bias=0.3 * rng.standard_normal((H, R, N)),
                  dt_bias=rng.uniform(-1.0, 0.0, H), eps=1e-5)
    return ins, dy, dh, kw, pm


OPTION_GRAD_CASES = [(1, "shuffle", True), (2, "reverse", False), (0, "zero", True),
                     (1, "native", False), (0, "reverse", True)]


def test_backward_per_token_decay_matches_finite_differences():
    """A per token (the decay exp(dt_t A_t)), with groups, shuffled phases
    and the pre-mixer: dA is the per-token gradient, every other gradient as
    before; central differences of the C oracle's loss."""
    from oracle.backward import scan_backward
    rng = np.random.default_rng(41)
    ins, dy, dh, kw, pm = _bwd_option_case(rng, 1, "shuffle", True, a_tok=True)
    g = scan_backward(*ins[:7], dy, dh, h0=ins[7], Bprev=ins[8], xprev=ins[9], premix=pm, **kw)
    assert g["dA"].shape == ins[4].shape

    def loss(args):
        y, hL, _, _ = oracle.scan(*args[:7], h0=args[7], Bprev=args[8], xprev=args[9],
                                  premix=pm, **kw)
        return float(np.sum(y * dy) + np.sum(hL * dh))
    names = ["dx", "dB", "dC", "ddt", "dA", "dtheta", "dlam", "dh0", "dBprev", "dxprev"]
    eps = 1e-6
    for k, name in enumerate(names):
        fd = np.zeros_like(ins[k])
        for idx in np.ndindex(ins[k].shape):
            plus, minus = [a.copy() for a in ins], [a.copy() for a in ins]
            plus[k][idx] += eps
            minus[k][idx] -= eps
            fd[idx] = (loss(plus) - loss(minus)) / (2 * eps)
        err = np.max(np.abs(fd - g[name])) / max(np.max(np.abs(g[name])), 1e-12)
        assert err < 1e-6, (name, err)


def test_backward_packed_matches_finite_differences():
    """Packed sequences (one empty) with head groups and the pre-mixer:
    every gradient against central differences of oracle.scan_packed's loss,
    the record gradients one row per sequence and the parameter gradients
    summed over the sequences."""
    from oracle.backward import PREMIX_GRADS, scan_backward_packed
    rng = np.random.default_rng(42)
    cu = np.array([0, 3, 3, 7])
    ins, dy, _, kw, pm = _bwd_option_case(rng, 1, "reverse", True, Bt=1, L=7, H=2, R=1, P=2, N=4)
    nseq = len(cu) - 1
    ins[7] = rng.standard_normal((nseq, 2, 4, 2))
    ins[8] = rng.standard_normal((nseq, 2, 1, 4))
    ins[9] = rng.standard_normal((nseq, 2, 1, 2))
    dh = rng.standard_normal((nseq, 2, 4, 2))
    g = scan_backward_packed(*ins[:7], cu, dy, dh, h0=ins[7], Bprev=ins[8], xprev=ins[9],
                             premix=pm, **kw)
    pnames = list(PREMIX_GRADS)
    params = [pm[n[1:]] for n in pnames]

    def loss(args, prm):
        pmx = dict(zip([n[1:] for n in pnames], prm), eps=pm["eps"])
        y, hs, _, _ = oracle.scan_packed(*args[:7], cu, h0=args[7], Bprev=args[8], xprev=args[9],
                                         premix=pmx, **kw)
        return float(np.sum(y * dy) + np.sum(hs * dh))
    names = ["dx", "dB", "dC", "ddt", "dA", "dtheta", "dlam", "dh0", "dBprev", "dxprev"]
    eps = 1e-6
    for k, name in enumerate(names + pnames):
        base = ins[k] if k < len(names) else params[k - len(names)]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = [a.copy() for a in ins], [a.copy() for a in ins]
            pp, pmn = [a.copy() for a in params], [a.copy() for a in params]
            (plus[k] if k < len(names) else pp[k - len(names)])[idx] += eps
            (minus[k] if k < len(names) else pmn[k - len(names)])[idx] -= eps
            fd[idx] = (loss(plus, pp) - loss(minus, pmn)) / (2 * eps)
        err = np.max(np.abs(fd - g[name])) / max(np.max(np.abs(g[name])), 1e-12)
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("ngroups,phase,premix", OPTION_GRAD_CASES)
def test_backward_options_forward_matches_c_oracle(ngroups, phase, premix):
    """The gradient oracle's option maps (group repeat, phase transform,
    pre-mixer) give the C oracle's forward with the same options."""
    import torch
    from oracle.backward import forward_torch
    rng = np.random.default_rng(34)
    ins, _, _, kw, pm = _bwd_option_case(rng, ngroups, phase, premix, Bt=2, L=9, H=4, N=8,
                                         a_tok=premix)
    y_c, h_c, _, _ = oracle.scan(*ins[:7], h0=ins[7], Bprev=ins[8], xprev=ins[9], premix=pm, **kw)
    tpm = None if pm is None else {k: (v if k == "eps" else torch.tensor(v)) for k, v in pm.items()}
    y_t, h_t = forward_torch(*[torch.tensor(a) for a in ins], premix=tpm, **kw)
    assert rel_err(y_t.numpy(), y_c) < 1e-13
    assert rel_err(h_t.numpy(), h_c) < 1e-13


@pytest.mark.parametrize("ngroups,phase,premix", OPTION_GRAD_CASES)
def test_backward_options_match_finite_differences(ngroups, phase, premix):
    """Every gradient with options, the pre-mixer's parameters included,
    against central differences of the C oracle's loss with those options:
    the group gradients sum over the heads of a group, dtheta follows the
    phase map back (zero, negated, permuted), and the raw inputs' gradients
    pass through RMSNorm, softplus and sigmoid."""
    from oracle.backward import PREMIX_GRADS, scan_backward
    rng = np.random.default_rng(35 + OPTION_GRAD_CASES.index((ngroups, phase, premix)))
    ins, dy, dh, kw, pm = _bwd_option_case(rng, ngroups, phase, premix)
    g = scan_backward(*ins[:7], dy, dh, h0=ins[7], Bprev=ins[8], xprev=ins[9], premix=pm, **kw)
    pnames = list(PREMIX_GRADS) if pm is not None else []
    params = [pm[n[1:]] for n in pnames]

    def loss(args, prm):
        pmx = None if pm is None else dict(zip([n[1:] for n in pnames], prm), eps=pm["eps"])
        y, hL, _, _ = oracle.scan(*args[:7], h0=args[7], Bprev=args[8], xprev=args[9],
                                  premix=pmx, **kw)
        return float(np.sum(y * dy) + np.sum(hL * dh))
    names = ["dx", "dB", "dC", "ddt", "dA", "dtheta", "dlam", "dh0", "dBprev", "dxprev"]
    eps = 1e-6
    for k, name in enumerate(names + pnames):
        base = ins[k] if k < len(names) else params[k - len(names)]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = [a.copy() for a in ins], [a.copy() for a in ins]
            pp, pmn = [a.copy() for a in params], [a.copy() for a in params]
            (plus[k] if k < len(names) else pp[k - len(names)])[idx] += eps
            (minus[k] if k < len(names) else pmn[k - len(names)])[idx] -= eps
            fd[idx] = (loss(plus, pp) - loss(minus, pmn)) / (2 * eps)
        assert g[name].shape == base.shape, name
        err = np.max(np.abs(fd - g[name])) / max(np.max(np.abs(g[name])), 1e-12)
        if phase == "zero" and name == "dtheta":
            assert np.all(g[name] == 0) and np.max(np.abs(fd)) < 1e-8
            continue
        assert err < 1e-6, (name, err)


# ---------------------------------------------------------------------------
# Accumulated angle and the write / read phase interventions.

def _draw_tokens(rng, Bt, L, H, R, P, N):
    return dict(x=rng.standard_normal((Bt, L, H, R, P)), B=rng.standard_normal((Bt, L, H, R, N)),
                C=rng.standard_normal((Bt, L, H, R, N)), dt=np.log1p(np.exp(rng.standard_normal((Bt, L, H)))),
                A=-np.exp(rng.uniform(-1, 1, H)), theta=rng.uniform(-np.pi, np.pi, (Bt, L, H, N // 2)),
                lam=1.0 / (1.0 + np.exp(-rng.standard_normal((Bt, L, H)))))


def test_accumulated_phase_is_the_composed_rotation():
    """R(phase_out) = R(phi_L) ... R(phi_1) R(phase_in), multiplied out as
    2x2 matrices (commuting plane rotations compose by adding angles)."""
    rng = np.random.default_rng(40)
    d = _draw_tokens(rng, 2, 37, 3, 1, 2, 6)
    ph_in = rng.uniform(-10, 10, (2, 3, 3))
    out = oracle.accumulated_phase(d["dt"], d["theta"], ph_in)
    assert np.all(out >= -np.pi) and np.all(out < np.pi)
    for b in range(2):
        for h in range(3):
            for i in range(3):
                M = np.array([[math.cos(ph_in[b, h, i]), -math.sin(ph_in[b, h, i])],
                              [math.sin(ph_in[b, h, i]), math.cos(ph_in[b, h, i])]])
                for t in range(37):
                    a = d["dt"][b, t, h] * d["theta"][b, t, h, i]
                    M = np.array([[math.cos(a), -math.sin(a)], [math.sin(a), math.cos(a)]]) @ M
                assert abs(M[0, 0] - math.cos(out[b, h, i])) < 1e-12
                assert abs(M[1, 0] - math.sin(out[b, h, i])) < 1e-12


@pytest.mark.parametrize("mode", ["no_write", "no_read", "no_write_read"])
def test_rotation_removal_without_rotation_is_native(mode):
    """theta = 0: there is no rotation to remove, every intervention is the
    native step (the C oracle) and the angle does not move."""
    rng = np.random.default_rng(41)
    Bt, H, R, P, N = 2, 3, 2, 4, 8
    x, Bm, Cm = (rng.standard_normal((Bt, H, R, k)) for k in (P, N, N))
    dt = np.log1p(np.exp(rng.standard_normal((Bt, H))))
    lam = rng.uniform(0, 1, (Bt, H))
    A = -np.exp(rng.uniform(-1, 1, H))
    th = np.zeros((Bt, H, N // 2))
    h = rng.standard_normal((Bt, H, N, P))
    Bp, xp = rng.standard_normal((Bt, H, R, N)), rng.standard_normal((Bt, H, R, P))
    ph = rng.uniform(-3, 3, (Bt, H, N // 2))
    y0, h0, _, _ = oracle.decode_step(x, Bm, Cm, dt, A, th, lam, h, Bp, xp)
    y1, h1, _, _, ph1 = oracle.decode_step_rotation_removed(x, Bm, Cm, dt, A, th, lam, h, Bp, xp,
                                                            mode, ph)
    # with theta = 0 the removed rotations are R(phase_in), applied to writes
    # (no_write) or reads (no_read); phase_in = 0 makes them the identity
    y2, h2, _, _, _ = oracle.decode_step_rotation_removed(x, Bm, Cm, dt, A, th, lam, h, Bp, xp,
                                                          mode, np.zeros_like(ph))
    assert np.allclose(y2, y0, rtol=1e-12, atol=1e-12) and np.allclose(h2, h0, rtol=1e-12, atol=1e-12)
    assert np.allclose(ph1, oracle.wrap_angle(ph), atol=1e-12)


@pytest.mark.parametrize("mode", ["no_write", "no_read", "no_write_read"])
def test_rotation_removal_matches_rotating_frame_sum(mode):
    """A native scan of T tokens from the sequence start, then K decode steps
    with the rotation removed, against an independent O(L^2) sum in the frame
    that turns with the accumulated angle Phi_t: there the state never
    rotates, token s is written as R(Phi_s)^T B_s X_s (natively) or B_s X_s
    (write rotation removed at that step) with weight gamma_s at step s and
    beta_{s+1} at step s+1, decays by e^{Lambda_t - Lambda_k} after step k,
    and is read with R(Phi_t)^T C_t or C_t."""
    no_write, no_read = oracle.ROTATION_REMOVED[mode]
    rng = np.random.default_rng(42)
    Bt, H, R, P, N, T, K = 1, 2, 2, 3, 8, 6, 5
    d = _draw_tokens(rng, Bt, T + K, H, R, P, N)
    y_nat, h, Bp, xp = oracle.scan(d["x"][:, :T], d["B"][:, :T], d["C"][:, :T], d["dt"][:, :T],
                                   d["A"], d["theta"][:, :T], d["lam"][:, :T])
    ph = oracle.accumulated_phase(d["dt"][:, :T], d["theta"][:, :T])
    got = [y_nat[:, t] for t in range(T)]
    for t in range(T, T + K):
        y, h, Bp, xp, ph = oracle.decode_step_rotation_removed(
            d["x"][:, t], d["B"][:, t], d["C"][:, t], d["dt"][:, t], d["A"], d["theta"][:, t],
            d["lam"][:, t], h, Bp, xp, mode, ph)
        got.append(y)
    # the rotating-frame sum
    Phi = np.cumsum(d["dt"][..., None] * d["theta"], axis=1)      # [Bt, L, H, N/2]
    Lam = np.cumsum(d["dt"] * d["A"][None, None, :], axis=1)       # [Bt, L, H]
    beta = (1 - d["lam"]) * d["dt"] * np.exp(d["dt"] * d["A"][None, None, :])
    gamma = d["lam"] * d["dt"]

    def rotT(v, ang):                                               # R(ang)^T on pairs of v [..., N]
        c, s = np.cos(ang), np.sin(ang)
        out = np.empty_like(v)
        out[..., 0::2] = c * v[..., 0::2] + s * v[..., 1::2]
        out[..., 1::2] = -s * v[..., 0::2] + c * v[..., 1::2]
        return out

    for b in range(Bt):
        for hh in range(H):
            for t in range(T + K):
                hr = np.zeros((N, P))
                for s in range(t + 1):
                    for k, wgt in ((s, gamma[b, s, hh]), (s + 1, beta[b, s + 1, hh] if s + 1 <= t else 0.0)):
                        if k > t or wgt == 0.0:
                            continue
                        Bs = d["B"][b, s, hh]                       # [R, N]
                        W = Bs if (no_write and k >= T) else rotT(Bs, Phi[b, s, hh])
                        hr += math.exp(Lam[b, t, hh] - Lam[b, k, hh]) * wgt * W.T @ d["x"][b, s, hh]
                Ct = d["C"][b, t, hh]
                Cr = Ct if (no_read and t >= T) else rotT(Ct, Phi[b, t, hh])
                ref = Cr @ hr                                       # [R, P]
                assert np.allclose(got[t][b, hh], ref, rtol=1e-10, atol=1e-10), (mode, b, hh, t)
