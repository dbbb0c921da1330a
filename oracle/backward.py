"""fp64 oracle for the gradient of the Mamba-3 scan -- TEST INFRASTRUCTURE ONLY
(loaded only by tests/, the smoke check and the benchmark's CPU leg).

The forward recurrence is written out step by step in plain float64 PyTorch
on the CPU (the same definition as m3_oracle.c: Mamba-3 summary on
b-lab.team, section 1 recurrence, section 2 block rotations R(dt theta_i) on
adjacent rows, section 3 MIMO; the rotation also carries the previous
endpoint), and its gradient is taken by reverse-mode automatic
differentiation of that loop: the gradient of L = sum(dy * y) + sum(dh * h_L)
with respect to every input, the decay rate A and the state record.

Layouts as the scan: x [Bt,L,H,R,P], Bm/Cm [Bt,L,H,R,N], dt/lam [Bt,L,H],
theta [Bt,L,H,N/2], A [H] or per token [Bt,L,H] (the decay exp(dt_t A_t) of
the Mamba-3 summary's section 1);
h0 [Bt,H,N,P], Bprev [Bt,H,R,N], xprev [Bt,H,R,P].

Options (the same maps as oracle.scan applies before the recurrence, here on
float64 tensors so that autograd carries the gradient back through them):
head groups (B, C given per group of nheads/ngroups heads and repeated per
head), the phase interventions of "Understanding Mamba-3 Through Oscillatory
Dynamics" (section 5.3: theta zeroed, negated or shuffled across the pairs)
and the pre-mixer of the Towards AI explainer (section II: RMSNorm with a gain
per state channel and a bias per head, rank and channel on B and C; softplus
of the raw step plus its bias; sigmoid of the raw trapezoid weight).  With the
pre-mixer the gradients are those of the raw inputs and of its parameters.

dA is a sum over batch and tokens of per-token terms (the decay rate enters
every step's alpha_t = exp(dt_t A)); scan_backward differentiates with
respect to A repeated per token, so that it can also return the size of what
that sum adds up: dA_scale[h] = sum over (b, t) of |dL/dA_{b,t,h}|.
"""
from __future__ import annotations

import numpy as np
import torch


def options_torch(Bm, Cm, dt, theta, lam, H, ngroups=None, phase="native", perm=None,
                  premix=None):
    """(B, C, dt, theta, lam) as the recurrence uses them.  ``premix`` holds
    float64 tensors B_norm_w, C_norm_w [N], B_bias, C_bias [H,R,N], dt_bias
    [H] and the float eps."""
    if ngroups:
        Bm = torch.repeat_interleave(Bm, H // Bm.shape[2], dim=2)
        Cm = torch.repeat_interleave(Cm, H // Cm.shape[2], dim=2)
    if phase == "zero":
        theta = torch.zeros_like(theta)
    elif phase == "reverse":
        theta = -theta
    elif phase == "shuffle":
        theta = theta[..., torch.as_tensor(np.asarray(perm), dtype=torch.long)]
    elif phase not in (None, "native"):
        raise ValueError("oracle: unknown phase mode %r" % (phase,))
    if premix is not None:
        eps = float(premix["eps"])

        def norm(M, w, b):
            return M / torch.sqrt(torch.mean(M * M, dim=-1, keepdim=True) + eps) * w + b
        Bm = norm(Bm, premix["B_norm_w"], premix["B_bias"])
        Cm = norm(Cm, premix["C_norm_w"], premix["C_bias"])
        dt = torch.logaddexp(torch.zeros_like(dt), dt + premix["dt_bias"])
        lam = torch.sigmoid(lam)
    return Bm, Cm, dt, theta, lam


def forward_torch(x, Bm, Cm, dt, A, theta, lam, h0, Bprev, xprev, **options):
    """y [Bt,L,H,R,P] and h_L, stepping the recurrence on float64 tensors
    (``options`` as options_torch takes them)."""
    Bt, L, H, R, P = x.shape
    N = Bm.shape[-1]
    if options:
        Bm, Cm, dt, theta, lam = options_torch(Bm, Cm, dt, theta, lam, H, **options)
    h = h0                                               # [Bt,H,N,P]
    Uprev = torch.einsum("bhrn,bhrp->bhnp", Bprev, xprev)
    ys = []
    for t in range(L):
        d = dt[:, t]                                     # [Bt,H]
        alpha = torch.exp(d * (A if A.dim() == 1 else A[:, t]))
        beta = (1.0 - lam[:, t]) * d * alpha
        gamma = lam[:, t] * d
        U = torch.einsum("bhrn,bhrp->bhnp", Bm[:, t], x[:, t])
        a = alpha[..., None, None] * h + beta[..., None, None] * Uprev
        phi = d[..., None] * theta[:, t]                 # [Bt,H,N/2]
        c, s = torch.cos(phi)[..., None], torch.sin(phi)[..., None]
        a0, a1 = a[:, :, 0::2], a[:, :, 1::2]
        r0 = c * a0 - s * a1                             # R(phi) on rows (2i, 2i+1)
        r1 = s * a0 + c * a1
        ra = torch.stack([r0, r1], dim=3).reshape(Bt, H, N, P)
        h = ra + gamma[..., None, None] * U
        ys.append(torch.einsum("bhrn,bhnp->bhrp", Cm[:, t], h))
        Uprev = U
    y = torch.stack(ys, dim=1) if ys else x.new_zeros((Bt, 0, H, R, P))
    return y, h


PREMIX_GRADS = ("dB_norm_w", "dC_norm_w", "dB_bias", "dC_bias", "ddt_bias")


def scan_backward(x, Bm, Cm, dt, A, theta, lam, dy, dh=None, h0=None, Bprev=None, xprev=None, *,
                  ngroups=None, phase="native", perm=None, premix=None):
    """Gradients of sum(dy * y) + sum(dh * h_L).  Returns a dict of float64
    numpy arrays: dx, dB, dC, ddt, dA, dtheta, dlam, dh0, dBprev, dxprev,
    dA_scale [H] (the sum of |per-token terms| that dA adds up; with A given
    per token, [Bt,L,H], dA is per token and dA_scale its magnitude) and, with
    ``premix`` (a dict of arrays B_norm_w, C_norm_w, B_bias, C_bias, dt_bias
    and eps), the parameter gradients dB_norm_w, dC_norm_w, dB_bias, dC_bias,
    ddt_bias."""
    t64 = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    x, Bm, Cm, dt, theta, lam = map(t64, (x, Bm, Cm, dt, theta, lam))
    Bt, L, H, R, P = x.shape
    N = Bm.shape[-1]
    # A repeated per (b, t) (or given per token): its gradient holds the
    # per-token terms of dA
    A_in = np.asarray(A, dtype=np.float64)
    A = t64(np.broadcast_to(A_in, (Bt, L, H)))
    z = lambda *s: np.zeros(s)
    h0 = t64(z(Bt, H, N, P) if h0 is None else h0)
    Bprev = t64(z(Bt, H, R, N) if Bprev is None else Bprev)
    xprev = t64(z(Bt, H, R, P) if xprev is None else xprev)
    pm = None
    if premix is not None:
        pm = {k: t64(premix[k]) for k in ("B_norm_w", "C_norm_w", "B_bias", "C_bias", "dt_bias")}
        pm["eps"] = float(premix.get("eps", 1e-6))
    y, hL = forward_torch(x, Bm, Cm, dt, A, theta, lam, h0, Bprev, xprev, ngroups=ngroups,
                          phase=phase, perm=perm, premix=pm)
    loss = (y * torch.as_tensor(np.asarray(dy, dtype=np.float64))).sum()
    if dh is not None:
        loss = loss + (hL * torch.as_tensor(np.asarray(dh, dtype=np.float64))).sum()
    names = ["dx", "dB", "dC", "ddt", "dA", "dtheta", "dlam", "dh0", "dBprev", "dxprev"]
    leaves = [x, Bm, Cm, dt, A, theta, lam, h0, Bprev, xprev]
    if pm is not None:
        names += list(PREMIX_GRADS)
        leaves += [pm[n[1:]] for n in PREMIX_GRADS]
    grads = torch.autograd.grad(loss, leaves, allow_unused=True)
    out = {n: (np.zeros(v.shape) if g is None else g.detach().numpy())
           for n, v, g in zip(names, leaves, grads)}
    terms = out["dA"]                                    # [Bt, L, H]
    if np.ndim(A_in) == 3:
        # a decay rate per token: each term is its own gradient
        out["dA_scale"] = np.abs(terms)
        return out
    out["dA"] = terms.sum(axis=(0, 1))
    out["dA_scale"] = np.abs(terms).sum(axis=(0, 1))
    return out


def scan_backward_packed(x, Bm, Cm, dt, A, theta, lam, cu_seqlens, dy, dh=None, h0=None,
                         Bprev=None, xprev=None, **options):
    """Gradients for packed sequences (oracle.scan_packed's layout: token arrays
    [1, T, ...], sequence i = tokens cu_seqlens[i] .. cu_seqlens[i+1]-1, one
    state record and one dh row per sequence).  Each sequence is an independent
    scan, so its gradients are scan_backward's on its own tokens and record;
    the token gradients are placed back at the sequence's tokens, the decay
    rate's and the pre-mixer's parameter gradients add over the sequences."""
    cu = [int(v) for v in np.asarray(cu_seqlens).ravel()]
    nseq = len(cu) - 1
    x = np.asarray(x, dtype=np.float64)
    _, T, H, R, P = x.shape
    N = np.asarray(Bm).shape[-1]
    A = np.asarray(A, dtype=np.float64)
    z = lambda *s: np.zeros(s)
    h0 = z(nseq, H, N, P) if h0 is None else np.asarray(h0, dtype=np.float64)
    Bprev = z(nseq, H, R, N) if Bprev is None else np.asarray(Bprev, dtype=np.float64)
    xprev = z(nseq, H, R, P) if xprev is None else np.asarray(xprev, dtype=np.float64)
    tok_names = {"dx": x, "dB": Bm, "dC": Cm, "ddt": dt, "dtheta": theta, "dlam": lam}
    out = {n: np.zeros(np.shape(v)) for n, v in tok_names.items()}
    out["dA"] = np.zeros(A.shape)
    out["dA_scale"] = np.zeros(A.shape)
    out["dh0"], out["dBprev"], out["dxprev"] = z(nseq, H, N, P), z(nseq, H, R, N), z(nseq, H, R, P)
    for i in range(nseq):
        sl = slice(cu[i], cu[i + 1])
        g = scan_backward(x[:, sl], np.asarray(Bm)[:, sl], np.asarray(Cm)[:, sl],
                          np.asarray(dt)[:, sl], A[:, sl] if A.ndim == 3 else A,
                          np.asarray(theta)[:, sl], np.asarray(lam)[:, sl],
                          np.asarray(dy)[:, sl], None if dh is None else np.asarray(dh)[i:i + 1],
                          h0=h0[i:i + 1], Bprev=Bprev[i:i + 1], xprev=xprev[i:i + 1], **options)
        for n in tok_names:
            out[n][:, sl] = g[n]
        if A.ndim == 3:
            out["dA"][:, sl] = g["dA"]
            out["dA_scale"][:, sl] = g["dA_scale"]
        else:
            out["dA"] += g["dA"]
            out["dA_scale"] += g["dA_scale"]
        for n in ("dh0", "dBprev", "dxprev"):
            out[n][i:i + 1] = g[n]
        for n in PREMIX_GRADS:
            if n in g:
                out[n] = out.get(n, 0.0) + g[n]
    if options.get("premix") is not None:
        pm = options["premix"]
        for n in PREMIX_GRADS:
            if n not in out:
                out[n] = np.zeros(np.shape(pm[n[1:]]))
    return out
