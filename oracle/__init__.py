"""fp64 CPU oracle for the Mamba-3 sequence mixer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and
shares no code with it.  The arithmetic lives in ``m3_oracle.c`` (plain C,
double precision, one POSIX thread per worker over independent (batch, head)
units); this module only builds it with gcc and marshals numpy arrays.

Every function takes and returns float64 numpy arrays in the library's layouts:
    x [Bt,L,H,R,P]   Bm, Cm [Bt,L,H,R,N]   dt, lam [Bt,L,H]   theta [Bt,L,H,N/2]
    A [H]            h [Bt,H,N,P]          Bprev [Bt,H,R,N]   xprev [Bt,H,R,P]

Options of ``scan`` and ``decode_step`` (each one a plain transform of the
inputs, applied before the recurrence, written out below):
    A per token      A of shape [Bt,L,H] (scan) or [Bt,H] (decode) instead of [H]
    ngroups=G        Bm, Cm given per head group, [Bt,L,G,R,N]; head h reads
                     group h // (H/G)
    phase            "native", "zero", "reverse" or "shuffle" (with ``perm``);
                     for a decode step also "no_write", "no_read" or
                     "no_write_read" (``decode_step_rotation_removed``)
    premix           dict of pre-mixer parameters: dt and lam are then the raw
                     projections, and B, C are RMS-normalised with gains and
                     biases
The accumulated rotation angle (``accumulated_phase``) is a plain sum.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "m3_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libm3oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile m3_oracle.c into libm3oracle.so with gcc (IEEE double, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.m3o_scan.restype = ctypes.c_int
        lib.m3o_scan.argtypes = [_i64] * 6 + [_dp] * 14 + [ctypes.c_int]
        lib.m3o_decode_step.restype = ctypes.c_int
        lib.m3o_decode_step.argtypes = [_i64] * 5 + [_dp] * 11
        _lib = lib
    return _lib


def _arr(a, shape):
    out = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if out.shape != tuple(shape):
        raise ValueError("oracle: expected shape %s, got %s" % (tuple(shape), out.shape))
    return out


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


# ---------------------------------------------------------------------------
# Input transforms.  Each returns new float64 arrays; the recurrence itself is
# the C code's.

def expand_groups(M, H):
    """B or C given per head group, [..., G, R, N], to per head, [..., H, R, N].

    Head h reads group h // (H // G): contiguous blocks of H/G heads share one
    B and one C (the grouping of the pages' predecessor Mamba-2, whose heads
    share parameters in groups; the Mamba-3 pages are silent on grouping)."""
    M = np.asarray(M, dtype=np.float64)
    G = M.shape[-3]
    if G <= 0 or H % G != 0:
        raise ValueError("oracle: %d heads cannot be split into %d groups" % (H, G))
    return np.repeat(M, H // G, axis=-3)


def phase_transform(theta, mode, perm=None):
    """Phase interventions of "Understanding Mamba-3 Through Oscillatory
    Dynamics" (section 5.3 and appendix D.4): the per-pair phase increments are
    zeroed, reversed in sign, or shuffled across the rotary pairs (the same
    permutation at every step, so each step keeps its set of increments); the
    decay is left alone.  ``shuffle``: pair i takes the increment of pair
    perm[i]."""
    theta = np.asarray(theta, dtype=np.float64)
    if mode in (None, "native"):
        return theta
    if mode == "zero":
        return np.zeros_like(theta)
    if mode == "reverse":
        return -theta
    if mode == "shuffle":
        perm = np.asarray(perm)
        if sorted(perm.tolist()) != list(range(theta.shape[-1])):
            raise ValueError("oracle: perm must be a permutation of the pairs")
        return theta[..., perm]
    raise ValueError("oracle: unknown phase mode %r" % (mode,))


def softplus(z):
    """log(1 + e^z), evaluated without overflow."""
    return np.logaddexp(0.0, np.asarray(z, dtype=np.float64))


def sigmoid(z):
    """1 / (1 + e^-z)."""
    z = np.asarray(z, dtype=np.float64)
    return np.exp(-np.logaddexp(0.0, -z))


def rms_norm(v, weight, eps):
    """v / sqrt(mean(v^2) + eps) * weight over the last axis (dstate)."""
    v = np.asarray(v, dtype=np.float64)
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps) * np.asarray(weight, np.float64)


def premix_bc(M, weight, bias, eps):
    """Pre-mixer of B or C: RMS normalisation over dstate with a gain per
    state channel, then a bias per (head, rank, state channel).  The Towards AI
    explainer of Mamba-3 (section II) pairs the mixer with QKNorm-style RMSNorm
    and learnable channel-wise biases on the B and C projections; the pages
    give no formula, so the plain RMSNorm-then-bias reading is taken.
    ``M`` is per head, [..., H, R, N]; ``bias`` is [H, R, N]; ``weight`` [N]."""
    return rms_norm(M, weight, eps) + np.asarray(bias, dtype=np.float64)


def premix_dt_lam(dt_raw, lam_raw, dt_bias):
    """dt = softplus(dt_raw + dt_bias[h]) and lam = sigmoid(lam_raw): the
    positive step and the trapezoid weight in [0, 1] from raw projections
    (the workload recipes draw dt and lam through the same two maps)."""
    return softplus(np.asarray(dt_raw, np.float64) + np.asarray(dt_bias, np.float64)), sigmoid(lam_raw)


def _apply_options(Bm, Cm, dt, A, theta, lam, H, ngroups, phase, perm, premix, per_token_shape):
    if ngroups:
        Bm = expand_groups(Bm, H)
        Cm = expand_groups(Cm, H)
    theta = phase_transform(theta, phase, perm)
    if premix is not None:
        eps = float(premix.get("eps", 1e-6))
        Bm = premix_bc(Bm, premix["B_norm_w"], premix["B_bias"], eps)
        Cm = premix_bc(Cm, premix["C_norm_w"], premix["C_bias"], eps)
        dt, lam = premix_dt_lam(dt, lam, premix["dt_bias"])
    A = np.asarray(A, dtype=np.float64)
    if A.shape == (H,):
        A = np.broadcast_to(A, per_token_shape)
    return Bm, Cm, dt, A, theta, lam


def scan(x, Bm, Cm, dt, A, theta, lam, h0=None, Bprev=None, xprev=None, threads=None, *,
         ngroups=None, phase="native", perm=None, premix=None):
    """Run the recurrence over all L steps.

    Returns (y [Bt,L,H,R,P], h_L [Bt,H,N,P], B_L [Bt,H,R,N], x_L [Bt,H,R,P]).
    ``h0``/``Bprev``/``xprev`` may be None (zero state, zero previous endpoint).
    B_L is the last token's B as the recurrence used it (after the group
    expansion and the pre-mixer): the previous endpoint a later call needs.
    """
    x = np.asarray(x)
    Bt, L, H, R, P = x.shape
    N = np.asarray(Bm).shape[-1]
    Bm, Cm, dt, A, theta, lam = _apply_options(Bm, Cm, dt, A, theta, lam, H, ngroups, phase,
                                               perm, premix, (Bt, L, H))
    x = _arr(x, (Bt, L, H, R, P))
    Bm = _arr(Bm, (Bt, L, H, R, N))
    Cm = _arr(Cm, (Bt, L, H, R, N))
    dt = _arr(dt, (Bt, L, H))
    lam = _arr(lam, (Bt, L, H))
    theta = _arr(theta, (Bt, L, H, N // 2))
    A = _arr(A, (Bt, L, H))
    h0 = None if h0 is None else _arr(h0, (Bt, H, N, P))
    if (Bprev is None) != (xprev is None):
        raise ValueError("oracle: Bprev and xprev must be given together")
    Bprev = None if Bprev is None else _arr(Bprev, (Bt, H, R, N))
    xprev = None if xprev is None else _arr(xprev, (Bt, H, R, P))
    y = np.empty((Bt, L, H, R, P))
    h_out = np.empty((Bt, H, N, P))
    Bp_out = np.empty((Bt, H, R, N))
    xp_out = np.empty((Bt, H, R, P))
    nthreads = int(threads) if threads else default_threads()
    rc = _load().m3o_scan(Bt, L, H, P, N, R, _ptr(x), _ptr(Bm), _ptr(Cm), _ptr(dt),
                          _ptr(A), _ptr(theta), _ptr(lam), _ptr(h0), _ptr(Bprev),
                          _ptr(xprev), _ptr(y), _ptr(h_out), _ptr(Bp_out), _ptr(xp_out),
                          nthreads)
    if rc != 0:
        raise RuntimeError("m3o_scan failed with code %d" % rc)
    return y, h_out, Bp_out, xp_out


def decode_step(x, Bm, Cm, dt, A, theta, lam, h, Bprev, xprev, *, ngroups=None,
                phase="native", perm=None, premix=None):
    """One step on a state record; returns (y_t, h', Bprev', xprev') as new arrays.

    The record's Bprev is taken as the recurrence uses it (already through the
    pre-mixer); Bprev' is this step's B after group expansion and pre-mixer."""
    x = np.asarray(x)
    Bt, H, R, P = x.shape
    N = np.asarray(Bm).shape[-1]
    Bm, Cm, dt, A, theta, lam = _apply_options(Bm, Cm, dt, A, theta, lam, H, ngroups, phase,
                                               perm, premix, (Bt, H))
    x = _arr(x, (Bt, H, R, P))
    Bm = _arr(Bm, (Bt, H, R, N))
    Cm = _arr(Cm, (Bt, H, R, N))
    dt = _arr(dt, (Bt, H))
    lam = _arr(lam, (Bt, H))
    theta = _arr(theta, (Bt, H, N // 2))
    A = _arr(A, (Bt, H))
    h = _arr(h, (Bt, H, N, P)).copy()
    Bprev = _arr(Bprev, (Bt, H, R, N)).copy()
    xprev = _arr(xprev, (Bt, H, R, P)).copy()
    y = np.empty((Bt, H, R, P))
    rc = _load().m3o_decode_step(Bt, H, P, N, R, _ptr(x), _ptr(Bm), _ptr(Cm), _ptr(dt),
                                 _ptr(A), _ptr(theta), _ptr(lam), _ptr(h), _ptr(Bprev),
                                 _ptr(xprev), _ptr(y))
    if rc != 0:
        raise RuntimeError("m3o_decode_step failed with code %d" % rc)
    return y, h, Bprev, xprev


def scan_packed(x, Bm, Cm, dt, A, theta, lam, cu_seqlens, h0=None, Bprev=None, xprev=None,
                threads=None, **options):
    """Packed sequences: sequence i is tokens cu_seqlens[i] .. cu_seqlens[i+1]-1
    of token arrays with a leading dimension of 1 ([1, T, ...]; A per token is
    [1, T, H]).  Each sequence is an independent scan from its own state record
    (h0, Bprev, xprev have one row per sequence); returns y [1, T, H, R, P] and
    the per-sequence records, as ``scan`` does for a dense batch."""
    cu = [int(v) for v in np.asarray(cu_seqlens).ravel()]
    nseq = len(cu) - 1
    x = np.asarray(x, dtype=np.float64)
    _, T, H, R, P = x.shape
    N = np.asarray(Bm).shape[-1]
    if cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("oracle: cu_seqlens must rise from 0 to the packed length")
    A = np.asarray(A, dtype=np.float64)
    y = np.empty((1, T, H, R, P))
    hs = np.empty((nseq, H, N, P))
    Bs = np.empty((nseq, H, R, N))
    xs = np.empty((nseq, H, R, P))
    for i in range(nseq):
        sl = slice(cu[i], cu[i + 1])
        take = lambda a: None if a is None else np.asarray(a)[i:i + 1]
        yi, hs[i:i + 1], Bs[i:i + 1], xs[i:i + 1] = scan(
            x[:, sl], np.asarray(Bm)[:, sl], np.asarray(Cm)[:, sl], np.asarray(dt)[:, sl],
            A[:, sl] if A.ndim == 3 else A,
            np.asarray(theta)[:, sl], np.asarray(lam)[:, sl],
            h0=take(h0), Bprev=take(Bprev), xprev=take(xprev), threads=threads, **options)
        y[:, sl] = yi
    return y, hs, Bs, xs


# ---------------------------------------------------------------------------
# Accumulated rotation angle and the write / read phase interventions.

def wrap_angle(a):
    """An angle reduced into [-pi, pi)."""
    return (np.asarray(a, dtype=np.float64) + np.pi) % (2.0 * np.pi) - np.pi


def accumulated_phase(dt, theta, phase_in=None):
    """The accumulated rotation angle per (batch, head, pair) after a scan:
    phase_in + sum over the call's tokens of dt_t theta_t[i], reduced mod 2 pi.

    Mamba-3 summary on b-lab.team, section 2 (the RoPE trick, Proposition 3):
    the product of the per-step rotations R(dt_s theta_s) up to step t is the
    rotation by the running sum Phi_t of the step angles; the frame that turns
    with Phi_t carries B and C as R(Phi_t)^T B_t, R(Phi_t)^T C_t.  ``dt`` and
    ``theta`` are the values the recurrence uses (after any option
    transforms): dt [Bt, L, H], theta [Bt, L, H, N/2]; phase_in [Bt, H, N/2]
    (None: zero, the sequence start)."""
    dt = np.asarray(dt, dtype=np.float64)
    theta = np.asarray(theta, dtype=np.float64)
    total = np.einsum("blh,blhi->bhi", dt, theta)
    if phase_in is not None:
        total = total + np.asarray(phase_in, dtype=np.float64)
    return wrap_angle(total)


ROTATION_REMOVED = {"no_write": (True, False), "no_read": (False, True),
                    "no_write_read": (True, True)}


def _rotate_rows(M, c, s):
    """R(angle) applied to the pairs (2i, 2i+1) along axis -2 of M [..., N, P];
    c, s [..., N/2] are the cosine and sine of the angle per pair."""
    M = np.asarray(M, dtype=np.float64)
    c = c[..., None]
    s = s[..., None]
    out = np.empty_like(M)
    out[..., 0::2, :] = c * M[..., 0::2, :] - s * M[..., 1::2, :]
    out[..., 1::2, :] = s * M[..., 0::2, :] + c * M[..., 1::2, :]
    return out


def decode_step_rotation_removed(x, Bm, Cm, dt, A, theta, lam, h, Bprev, xprev, phase,
                                 phase_in=None):
    """One decode step with the rotation removed from writing ("no_write"),
    from readout ("no_read") or from both ("no_write_read"); returns (y_t, h',
    Bprev', xprev', phase_out).

    "Understanding Mamba-3 Through Oscillatory Dynamics", section 5.3 (Table 7)
    removes the rotation from the write or the readout of a pretrained model,
    and appendix D.4 applies these interventions to prediction steps after a
    native context.  In the frame that turns with the accumulated angle Phi_t
    (Mamba-3 summary, section 2, Proposition 3) the native model writes
    R(Phi_s)^T B_s and reads R(Phi_t)^T C_t; the interventions use B_s, C_t
    unrotated instead (the reading taken here).  In the state's own frame,
    h = R(Phi) h_rot, that is, with Phi_t = phase_in + dt_t theta_t (the angle
    after this step), U = B_t X_t, Uprev = Bprev Xprev (N x P, summed over the
    ranks) and phi_t = dt_t theta_t:
        h' = alpha R(phi_t) h + beta Wp + gamma W
        W  = R(Phi_t) U       (write rotation removed)   else U
        Wp = R(Phi_t) Uprev   (write rotation removed)   else R(phi_t) Uprev
        y  = (R(Phi_t) C_t)^T h'  (read rotation removed)  else C_t^T h'
    with alpha, beta, gamma as in the native step (Mamba-3 summary, section 1).
    Shapes as ``decode_step`` without options; phase_in [Bt, H, N/2] (None:
    zero).  phase_out = Phi_t reduced mod 2 pi."""
    no_write, no_read = ROTATION_REMOVED[phase]
    x = np.asarray(x, dtype=np.float64)
    Bt, H, R, P = x.shape
    Bm = np.asarray(Bm, dtype=np.float64)
    Cm = np.asarray(Cm, dtype=np.float64)
    N = Bm.shape[-1]
    dt = np.asarray(dt, dtype=np.float64)
    A = np.broadcast_to(np.asarray(A, dtype=np.float64), (Bt, H)) if np.ndim(A) == 1 \
        else np.asarray(A, dtype=np.float64)
    theta = np.asarray(theta, dtype=np.float64)
    lam = np.asarray(lam, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    Bprev = np.asarray(Bprev, dtype=np.float64)
    xprev = np.asarray(xprev, dtype=np.float64)
    ph_in = np.zeros((Bt, H, N // 2)) if phase_in is None else np.asarray(phase_in, np.float64)
    phi = dt[..., None] * theta                          # this step's angle per pair
    Phi = ph_in + phi                                    # accumulated angle after the step
    alpha = np.exp(dt * A)[..., None, None]
    beta = ((1.0 - lam) * dt)[..., None, None] * alpha
    gamma = (lam * dt)[..., None, None]
    U = np.einsum("bhrn,bhrp->bhnp", Bm, x)
    Uprev = np.einsum("bhrn,bhrp->bhnp", Bprev, xprev)
    cp, sp = np.cos(phi), np.sin(phi)
    cP, sP = np.cos(Phi), np.sin(Phi)
    W = _rotate_rows(U, cP, sP) if no_write else U
    Wp = _rotate_rows(Uprev, cP, sP) if no_write else _rotate_rows(Uprev, cp, sp)
    h_new = alpha * _rotate_rows(h, cp, sp) + beta * Wp + gamma * W
    if no_read:
        # (R(Phi) C)^T h = C^T R(Phi)^T h = C^T R(-Phi) h
        y = np.einsum("bhrn,bhnp->bhrp", Cm, _rotate_rows(h_new, cP, -sP))
    else:
        y = np.einsum("bhrn,bhnp->bhrp", Cm, h_new)
    return y, h_new, Bm.copy(), x.copy(), wrap_angle(Phi)
