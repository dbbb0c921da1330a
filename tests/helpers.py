"""Shared helpers for the parity tests: seeded inputs, oracle calls, error metric."""
import math
import sys

import numpy as np
import torch

import oracle
from mamba_selective_ssm_amd import synth

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over the whole tensor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref))) / max(den, 1e-30)


def f64(t):
    return synth.to_f64_numpy(t)


def workload(Bt, L, H, R, P, N, io="bf16", chunk=64, dt_mu=-2.0, theta="normal_0.5"):
    return synth.Workload("case", Bt, H, L, P, N, R, io, chunk, dt_mu, theta)


def random_state(w, seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    h = torch.randn(w.batch, w.heads, w.dstate, w.headdim, generator=g, device=device)
    Bp = torch.randn(w.batch, w.heads, w.rank, w.dstate, generator=g, device=device)
    xp = torch.randn(w.batch, w.heads, w.rank, w.headdim, generator=g, device=device)
    return h, Bp.to(w.torch_dtype), xp.to(w.torch_dtype)


def oracle_scan(inp, state=None, threads=None):
    """Run the fp64 oracle on exactly the tensors the GPU consumed."""
    kw = {}
    if state is not None:
        kw = dict(h0=f64(state[0]), Bprev=f64(state[1]), xprev=f64(state[2]))
    return oracle.scan(f64(inp["x"]), f64(inp["B"]), f64(inp["C"]), f64(inp["dt"]),
                       f64(inp["A"]), f64(inp["theta"]), f64(inp["lam"]), threads=threads, **kw)


def select_heads(inp, bsel, hsel):
    """Sub-problem of a scan input restricted to batch rows bsel and heads hsel."""
    out = {}
    for k, v in inp.items():
        if k == "A":
            out[k] = v[hsel]
        else:
            out[k] = v[bsel][:, :, hsel]
    return out


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
