"""Seeded synthetic inputs for the Mamba-3 mixer workloads.

This module only draws random tensors; it holds none of the mixer's arithmetic.
Both the HIP library's callers (tests, bench) and the fp64 oracle consume the
exact tensors produced here (the oracle receives them upcast to float64), so
the two sides always see byte-identical inputs.

Distributions (the five workloads the library is measured on):
    x, B, C ~ N(0, 1)
    dt      = softplus(N(mu_dt, 1))          mu_dt = 0, -2 or -3
    A       = -exp(U(-1, 1))                  one value per head
    theta   ~ U(-pi, pi)  or  N(0, 0.5)       one angle per state pair per step
    lam     = sigmoid(N(0, 1))
N(m, s) means mean m and standard deviation s.  Random numbers are drawn in
float32 from a torch generator seeded with ``seed`` on ``device`` (draw order
A, x, B, C, dt, theta, lam), then x/B/C are cast to the I/O dtype with
round-to-nearest-even.  dt, theta, lam and A stay float32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seqlen: int
    headdim: int      # P
    dstate: int       # N (even)
    rank: int         # MIMO rank R
    io_dtype: str     # "f32" or "bf16"
    chunk: int
    dt_mu: float
    theta_dist: str   # "uniform_pi" or "normal_0.5"
    decode_steps: int = 0

    @property
    def torch_dtype(self):
        return torch.float32 if self.io_dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # Tiny fp32 single-head scan (oracle finishes instantly).
    "tiny_f32": Workload("tiny_f32", 1, 1, 64, 16, 16, 1, "f32", 32, 0.0, "uniform_pi"),
    # Single-layer prefill, bf16 I/O, fp32 state and accumulation.
    "prefill_bf16": Workload("prefill_bf16", 4, 16, 2048, 64, 64, 1, "bf16", 64, -2.0,
                             "normal_0.5"),
    # MIMO prefill, rank 4.
    "mimo_prefill_bf16": Workload("mimo_prefill_bf16", 8, 32, 4096, 64, 128, 4, "bf16", 16,
                                  -2.0, "normal_0.5"),
    # Long-context prefill with slow decay.
    "long_prefill_bf16": Workload("long_prefill_bf16", 1, 32, 65536, 64, 128, 1, "bf16", 64,
                                  -3.0, "normal_0.5"),
    # Decode: 1024-token MIMO prefill at batch 256, then 1024 single-token steps.
    "decode": Workload("decode", 256, 32, 1024, 64, 128, 4, "bf16", 16, -2.0, "normal_0.5",
                       decode_steps=1024),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def make_scan_inputs(w: Workload, seed: int, device="cpu", A: Optional[torch.Tensor] = None):
    """Draw one prefill batch for workload ``w``: dict of tensors on ``device``.

    Keys: x [B,L,H,R,P], B/C [B,L,H,R,N] (I/O dtype), dt/lam [B,L,H],
    theta [B,L,H,N/2], A [H] (float32).  ``A`` may be supplied (decode reuses
    the prefill's per-head A).
    """
    g = _gen(seed, device)
    f32 = dict(dtype=torch.float32, device=device)
    Bt, L, H, P, N, R = w.batch, w.seqlen, w.heads, w.headdim, w.dstate, w.rank
    if A is None:
        A = -torch.exp(torch.rand((H,), generator=g, **f32) * 2.0 - 1.0)
    x = torch.randn((Bt, L, H, R, P), generator=g, **f32).to(w.torch_dtype)
    Bm = torch.randn((Bt, L, H, R, N), generator=g, **f32).to(w.torch_dtype)
    Cm = torch.randn((Bt, L, H, R, N), generator=g, **f32).to(w.torch_dtype)
    dt = torch.nn.functional.softplus(torch.randn((Bt, L, H), generator=g, **f32) + w.dt_mu)
    if w.theta_dist == "uniform_pi":
        theta = (torch.rand((Bt, L, H, N // 2), generator=g, **f32) * 2.0 - 1.0) * math.pi
    else:
        theta = torch.randn((Bt, L, H, N // 2), generator=g, **f32) * 0.5
    lam = torch.sigmoid(torch.randn((Bt, L, H), generator=g, **f32))
    return dict(x=x, B=Bm, C=Cm, dt=dt.contiguous(), A=A.to(device=device).contiguous(),
                theta=theta.contiguous(), lam=lam.contiguous())


def make_decode_inputs(w: Workload, seed: int, step: int, A: torch.Tensor, device="cpu"):
    """Fresh single-token inputs for decode step ``step``: x [B,H,R,P], B/C [B,H,R,N],
    dt/lam [B,H], theta [B,H,N/2], plus the given A [H].  Seeded by (seed, step)."""
    g = _gen(seed * 1_000_003 + step, device)
    f32 = dict(dtype=torch.float32, device=device)
    Bt, H, P, N, R = w.batch, w.heads, w.headdim, w.dstate, w.rank
    x = torch.randn((Bt, H, R, P), generator=g, **f32).to(w.torch_dtype)
    Bm = torch.randn((Bt, H, R, N), generator=g, **f32).to(w.torch_dtype)
    Cm = torch.randn((Bt, H, R, N), generator=g, **f32).to(w.torch_dtype)
    dt = torch.nn.functional.softplus(torch.randn((Bt, H), generator=g, **f32) + w.dt_mu)
    theta = torch.randn((Bt, H, N // 2), generator=g, **f32) * 0.5
    lam = torch.sigmoid(torch.randn((Bt, H), generator=g, **f32))
    return dict(x=x, B=Bm, C=Cm, dt=dt.contiguous(), A=A, theta=theta.contiguous(),
                lam=lam.contiguous())


def to_f64_numpy(t: torch.Tensor):
    """Exact upcast of a float32/bfloat16 tensor to a float64 numpy array (host)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def make_option_inputs(w: Workload, seed: int, device="cpu", *, ngroups: int = 0,
                       a_per_token: bool = False, phase: str = "native", premix: bool = False):
    """A scan batch for ``w`` with the library's options drawn as well.

    Returns (inputs, extras).  ``inputs`` has the keys of make_scan_inputs;
    with ``ngroups`` B and C are [B,L,G,R,N]; with ``a_per_token`` A is
    [B,L,H] = -exp(U(-1, 1)); with ``premix`` dt and lam are the raw
    projections dt_raw ~ N(0, 1), lam_raw ~ N(0, 1).  ``extras`` holds
    ``perm`` (int32 [N/2], a uniform random permutation, for phase "shuffle")
    and ``premix`` parameters: gains U(0.5, 1.5) [N], biases N(0, 0.3^2)
    [H,R,N], dt_bias = dt_mu + U(-0.5, 0.5) [H] (so that the mapped dt follows
    the workload's softplus(N(dt_mu, 1))), eps 1e-5.  Seeded by ``seed``;
    draws come after those of make_scan_inputs.
    """
    inp = make_scan_inputs(w, seed, device)
    g = _gen(seed * 7919 + 17, device)
    f32 = dict(dtype=torch.float32, device=device)
    Bt, L, H, P, N, R = w.batch, w.seqlen, w.heads, w.headdim, w.dstate, w.rank
    extras = {}
    if ngroups:
        inp["B"] = torch.randn((Bt, L, ngroups, R, N), generator=g, **f32).to(w.torch_dtype)
        inp["C"] = torch.randn((Bt, L, ngroups, R, N), generator=g, **f32).to(w.torch_dtype)
    if a_per_token:
        inp["A"] = -torch.exp(torch.rand((Bt, L, H), generator=g, **f32) * 2.0 - 1.0)
    if phase == "shuffle":
        extras["perm"] = torch.randperm(N // 2, generator=g, device=device).to(torch.int32)
    if premix:
        inp["dt"] = torch.randn((Bt, L, H), generator=g, **f32)
        inp["lam"] = torch.randn((Bt, L, H), generator=g, **f32)
        extras["premix"] = dict(
            B_norm_w=torch.rand((N,), generator=g, **f32) + 0.5,
            C_norm_w=torch.rand((N,), generator=g, **f32) + 0.5,
            B_bias=torch.randn((H, R, N), generator=g, **f32) * 0.3,
            C_bias=torch.randn((H, R, N), generator=g, **f32) * 0.3,
            dt_bias=w.dt_mu + torch.rand((H,), generator=g, **f32) - 0.5,
            eps=1e-5)
    return inp, extras
