"""Thin Python binding of libm3scan (ctypes).  Argument marshalling only:
every step of the mixer runs in the HIP library; torch provides device memory
and the current stream.  There is no fallback: if the library is missing the
calls raise.

Names follow the C ABI (include/m3scan.h): m3_scan_fwd, m3_decode_step,
m3_scan_workspace_bytes, m3_scan_supported, m3_decode_supported,
m3_status_string, m3_abi_version.

Layouts (contiguous):
    x, y [Bt, L, H, R, P]   B, C [Bt, L, H, R, N]   dt, lam [Bt, L, H]
    theta [Bt, L, H, N/2]   A [H]
    state: h [Bt, H, N, P] float32, B_prev [Bt, H, R, N], x_prev [Bt, H, R, P]

Options (the m3_options of the C ABI), keyword arguments of the scan and
decode calls:
    A of shape [Bt, L, H] (decode: [Bt, H])  per-token decay rate
    ngroups=G      B, C given per head group: [Bt, L, G, R, N] (decode [Bt, G, R, N])
    phase          "native" | "zero" | "reverse" | "shuffle"; perm: int32 [N/2]
    premix         a Premix: dt and lam are raw, B and C RMS-normalised
    cu_seqlens     (scan only) int32 [nseq + 1]: nseq sequences packed along the
                   token axis of [1, T, ...] token arrays; max_seqlen bounds
                   their lengths (default: T); the state record is per sequence
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libm3scan.so")

M3_F32, M3_BF16 = 0, 1
_STATUS = {0: "M3_OK", -1: "M3_ERR_NULL", -2: "M3_ERR_SHAPE", -3: "M3_ERR_UNSUPPORTED",
           -4: "M3_ERR_DTYPE", -5: "M3_ERR_ALIGN", -6: "M3_ERR_WORKSPACE", -7: "M3_ERR_ALIAS",
           -8: "M3_ERR_HIP", -9: "M3_ERR_OPTION", -10: "M3_ERR_SCRATCH"}
PHASE_MODES = {"native": 0, "zero": 1, "reverse": 2, "shuffle": 3,
               # decode steps only: the rotation removed from writing / readout
               "no_write": 4, "no_read": 5, "no_write_read": 6}

_vp = ctypes.c_void_p


class Options(ctypes.Structure):
    _fields_ = [("ngroups", ctypes.c_int64), ("A_per_token", ctypes.c_int32),
                ("phase_mode", ctypes.c_int32), ("phase_perm", _vp),
                ("premix", ctypes.c_int32), ("norm_eps", ctypes.c_float),
                ("B_norm_w", _vp), ("C_norm_w", _vp), ("B_bias", _vp), ("C_bias", _vp),
                ("dt_bias", _vp), ("cu_seqlens", _vp), ("max_seqlen", ctypes.c_int64),
                ("phase_in", _vp), ("phase_out", _vp)]


class Premix(NamedTuple):
    """Pre-mixer parameters (float32 device tensors; None = ones / zeros).
    dt = softplus(dt_raw + dt_bias[h]), lam = sigmoid(lam_raw),
    B' = B / sqrt(mean_n B^2 + eps) * B_norm_w[n] + B_bias[h, r, n] (C alike)."""
    B_norm_w: Optional[torch.Tensor] = None   # [N]
    C_norm_w: Optional[torch.Tensor] = None   # [N]
    B_bias: Optional[torch.Tensor] = None     # [H, R, N]
    C_bias: Optional[torch.Tensor] = None     # [H, R, N]
    dt_bias: Optional[torch.Tensor] = None    # [H]
    eps: float = 1e-5


class ScanArgs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("rank", ctypes.c_int64),
                ("chunk", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("p_split", ctypes.c_int32), ("segments", ctypes.c_int32),
                ("x", _vp), ("B", _vp), ("C", _vp),
                ("dt", _vp), ("A", _vp), ("theta", _vp), ("lam", _vp),
                ("h_in", _vp), ("B_prev_in", _vp), ("x_prev_in", _vp),
                ("y", _vp), ("h_out", _vp), ("B_prev_out", _vp), ("x_prev_out", _vp),
                ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
                ("opt", Options)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("rank", ctypes.c_int64), ("io_dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32),
                ("x", _vp), ("B", _vp), ("C", _vp),
                ("dt", _vp), ("A", _vp), ("theta", _vp), ("lam", _vp),
                ("h", _vp), ("B_prev", _vp), ("x_prev", _vp), ("y", _vp),
                ("opt", Options)]


class ScanBwdArgs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("rank", ctypes.c_int64),
                ("io_dtype", ctypes.c_int32), ("method", ctypes.c_int32),
                ("x", _vp), ("B", _vp), ("C", _vp),
                ("dt", _vp), ("A", _vp), ("theta", _vp), ("lam", _vp),
                ("h_in", _vp), ("B_prev_in", _vp), ("x_prev_in", _vp),
                ("dy", _vp), ("dh_out", _vp),
                ("dx", _vp), ("dB", _vp), ("dC", _vp), ("ddt", _vp), ("dA", _vp),
                ("dtheta", _vp), ("dlam", _vp),
                ("dh_in", _vp), ("dB_prev", _vp), ("dx_prev", _vp),
                ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
                ("opt", Options),
                ("dB_norm_w", _vp), ("dC_norm_w", _vp), ("dB_bias", _vp), ("dC_bias", _vp),
                ("ddt_bias", _vp), ("dB_prev_out", _vp), ("dx_prev_out", _vp)]


class M3Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (what, _STATUS.get(status, status),
                                                  m3_status_string(status)))


_lib = None


def load_library():
    """Load libm3scan.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libm3scan.so is not built (%s); run "
                               "`python -m mamba_selective_ssm_amd.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
        lib.m3_scan_fwd.restype = ctypes.c_int
        lib.m3_scan_fwd.argtypes = [ctypes.POINTER(ScanArgs), _vp]
        lib.m3_scan_fwd_noalloc.restype = ctypes.c_int
        lib.m3_scan_fwd_noalloc.argtypes = [ctypes.POINTER(ScanArgs), _vp]
        lib.m3_scan_bwd.restype = ctypes.c_int
        lib.m3_scan_bwd.argtypes = [ctypes.POINTER(ScanBwdArgs), _vp]
        lib.m3_scan_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.m3_scan_bwd_workspace_bytes.argtypes = [ctypes.POINTER(ScanBwdArgs)]
        lib.m3_scan_bwd_supported.restype = ctypes.c_int
        lib.m3_scan_bwd_supported.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                              ctypes.c_int32]
        lib.m3_scan_bwd_method_supported.restype = ctypes.c_int
        lib.m3_scan_bwd_method_supported.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                     ctypes.c_int32, ctypes.c_int32]
        lib.m3_decode_step.restype = ctypes.c_int
        lib.m3_decode_step.argtypes = [ctypes.POINTER(DecodeArgs), _vp]
        lib.m3_scan_workspace_bytes.restype = ctypes.c_size_t
        lib.m3_scan_workspace_bytes.argtypes = [ctypes.POINTER(ScanArgs)]
        lib.m3_scan_supported.restype = ctypes.c_int
        lib.m3_scan_supported.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int32, ctypes.c_int32]
        lib.m3_decode_supported.restype = ctypes.c_int
        lib.m3_decode_supported.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int32]
        lib.m3_status_string.restype = ctypes.c_char_p
        lib.m3_status_string.argtypes = [ctypes.c_int]
        lib.m3_last_hip_error.restype = ctypes.c_int
        lib.m3_last_hip_error.argtypes = []
        lib.m3_abi_version.restype = ctypes.c_int
        lib.m3_abi_version.argtypes = []
        _lib = lib
    return _lib


def m3_status_string(status: int) -> str:
    return load_library().m3_status_string(int(status)).decode()


def m3_abi_version() -> int:
    return load_library().m3_abi_version()


def m3_scan_supported(dstate: int, headdim: int, rank: int, chunk: int, io_dtype: int) -> bool:
    return bool(load_library().m3_scan_supported(dstate, headdim, rank, chunk, io_dtype))


def m3_decode_supported(dstate: int, headdim: int, rank: int, io_dtype: int) -> bool:
    return bool(load_library().m3_decode_supported(dstate, headdim, rank, io_dtype))


class State(NamedTuple):
    """State record: true state h plus the last token's (B, X)."""
    h: torch.Tensor        # [Bt, H, N, P] float32
    B_prev: torch.Tensor   # [Bt, H, R, N] io dtype
    x_prev: torch.Tensor   # [Bt, H, R, P] io dtype


def zero_state(batch, nheads, headdim, dstate, rank, dtype, device) -> State:
    return State(torch.zeros(batch, nheads, dstate, headdim, dtype=torch.float32, device=device),
                 torch.zeros(batch, nheads, rank, dstate, dtype=dtype, device=device),
                 torch.zeros(batch, nheads, rank, headdim, dtype=dtype, device=device))


def _io_code(dtype) -> int:
    if dtype == torch.float32:
        return M3_F32
    if dtype == torch.bfloat16:
        return M3_BF16
    raise TypeError("io dtype must be float32 or bfloat16, got %s" % dtype)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _check(t: torch.Tensor, name: str, shape, dtype):
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.dtype != dtype:
        raise TypeError("%s: expected %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)


def _options(H, N, R, A_per_token, ngroups, phase, perm, premix, device, rows=None,
             phase_in=None, phase_out=None):
    """m3_options from the keyword arguments (plus the tensors to keep alive).
    phase_in / phase_out: accumulated rotation angle [rows, H, N/2] float32
    (may be the same tensor: updated in place)."""
    mode = PHASE_MODES[phase] if isinstance(phase, str) else int(phase)
    o = Options(ngroups=int(ngroups or 0), A_per_token=int(bool(A_per_token)), phase_mode=mode)
    keep = []
    for name, t in (("phase_in", phase_in), ("phase_out", phase_out)):
        if t is not None:
            _check(t, name, (rows, H, N // 2), torch.float32)
            setattr(o, name, t.data_ptr())
            keep.append(t)
    if mode == PHASE_MODES["shuffle"]:
        if perm is None:
            raise ValueError("phase='shuffle' needs perm")
        _check(perm, "perm", (N // 2,), torch.int32)
        o.phase_perm = perm.data_ptr()
        keep.append(perm)
    if premix is not None:
        o.premix = 1
        o.norm_eps = float(premix.eps)
        for name, shape in (("B_norm_w", (N,)), ("C_norm_w", (N,)), ("B_bias", (H, R, N)),
                            ("C_bias", (H, R, N)), ("dt_bias", (H,))):
            t = getattr(premix, name)
            if t is not None:
                _check(t, "premix." + name, shape, torch.float32)
                setattr(o, name, t.data_ptr())
                keep.append(t)
    return o, keep


def _stream_handle(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _prepare_scan(x, B, C, dt, A, theta, lam, state, chunk, p_split, segments, return_state,
                  y, state_out, workspace, ngroups=0, phase="native", perm=None, premix=None,
                  cu_seqlens=None, max_seqlen=None, phase_in=None, phase_out=None,
                  alloc_workspace=True):
    lib = load_library()
    Bx, L, H, R, P = x.shape
    N = B.shape[-1]
    G = int(ngroups) if ngroups else H
    io = _io_code(x.dtype)
    if cu_seqlens is not None:
        if Bx != 1:
            raise ValueError("packed sequences: token arrays must have a leading dimension of 1")
        _check(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32)
        Bt = cu_seqlens.numel() - 1     # sequences: the state record's batch
    else:
        Bt = Bx
    _check(x, "x", (Bx, L, H, R, P), x.dtype)
    _check(B, "B", (Bx, L, G, R, N), x.dtype)
    _check(C, "C", (Bx, L, G, R, N), x.dtype)
    _check(dt, "dt", (Bx, L, H), torch.float32)
    _check(lam, "lam", (Bx, L, H), torch.float32)
    if theta is not None or phase != "zero":
        _check(theta, "theta", (Bx, L, H, N // 2), torch.float32)
    a_tok = A.dim() == 3
    _check(A, "A", (Bx, L, H) if a_tok else (H,), torch.float32)
    opt, keep = _options(H, N, R, a_tok, ngroups, phase, perm, premix, x.device, Bt,
                         phase_in, phase_out)
    if cu_seqlens is not None:
        opt.cu_seqlens = cu_seqlens.data_ptr()
        opt.max_seqlen = int(L if max_seqlen is None else max_seqlen)
        keep.append(cu_seqlens)
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", (Bx, L, H, R, P), x.dtype)
    if state is not None:
        _check(state.h, "state.h", (Bt, H, N, P), torch.float32)
        _check(state.B_prev, "state.B_prev", (Bt, H, R, N), x.dtype)
        _check(state.x_prev, "state.x_prev", (Bt, H, R, P), x.dtype)
    if return_state and state_out is None:
        state_out = State(torch.empty(Bt, H, N, P, dtype=torch.float32, device=x.device),
                          torch.empty(Bt, H, R, N, dtype=x.dtype, device=x.device),
                          torch.empty(Bt, H, R, P, dtype=x.dtype, device=x.device))
    a = ScanArgs(batch=Bt, seqlen=L, nheads=H, headdim=P, dstate=N, rank=R,
                 chunk=chunk, io_dtype=io, p_split=p_split, segments=segments,
                 x=_ptr(x), B=_ptr(B), C=_ptr(C), dt=_ptr(dt), A=_ptr(A),
                 theta=_ptr(theta), lam=_ptr(lam),
                 h_in=_ptr(state.h) if state else None,
                 B_prev_in=_ptr(state.B_prev) if state else None,
                 x_prev_in=_ptr(state.x_prev) if state else None,
                 y=_ptr(y),
                 h_out=_ptr(state_out.h) if state_out else None,
                 B_prev_out=_ptr(state_out.B_prev) if state_out else None,
                 x_prev_out=_ptr(state_out.x_prev) if state_out else None,
                 workspace=None, workspace_bytes=0, opt=opt)
    a._keep = keep
    need = lib.m3_scan_workspace_bytes(ctypes.byref(a)) if alloc_workspace else 0
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(int(need), dtype=torch.uint8, device=x.device)
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    return a, y, state_out, workspace


def m3_scan_fwd(x, B, C, dt, A, theta, lam, state: Optional[State] = None, *,
                chunk: int = 0, p_split: int = 0, segments: int = 0,
                return_state: bool = True, y: Optional[torch.Tensor] = None,
                state_out: Optional[State] = None, workspace: Optional[torch.Tensor] = None,
                ngroups: int = 0, phase="native", perm: Optional[torch.Tensor] = None,
                premix: Optional[Premix] = None, cu_seqlens: Optional[torch.Tensor] = None,
                max_seqlen: Optional[int] = None, phase_in: Optional[torch.Tensor] = None,
                phase_out: Optional[torch.Tensor] = None, stream=None):
    """Chunked prefill.  Returns (y, State after the last token or None); with
    packed sequences the State holds one record per sequence.  ``phase_out``
    (float32 [batch or sequences, H, N/2]) receives the accumulated rotation
    angle after the last token, starting from ``phase_in`` (None: zero)."""
    a, y, state_out, _ = _prepare_scan(x, B, C, dt, A, theta, lam, state, chunk, p_split,
                                       segments, return_state, y, state_out, workspace,
                                       ngroups, phase, perm, premix, cu_seqlens, max_seqlen,
                                       phase_in, phase_out)
    st = load_library().m3_scan_fwd(ctypes.byref(a), _stream_handle(stream))
    if st != 0:
        raise M3Error(st, "m3_scan_fwd")
    return y, state_out


def m3_scan_fwd_noalloc(x, B, C, dt, A, theta, lam, state: Optional[State] = None, *,
                        chunk: int = 0, p_split: int = 0, segments: int = 0,
                        return_state: bool = True, y: Optional[torch.Tensor] = None,
                        state_out: Optional[State] = None, stream=None, **options):
    """m3_scan_fwd_noalloc: the same scan as m3_scan_fwd, its scratch taken
    from the library's static device array (M3_NOALLOC_SCRATCH_BYTES) instead
    of a workspace.  ``y`` and ``state_out`` may be given so that the call
    itself allocates nothing; options as m3_scan_fwd (ngroups, phase, perm,
    premix, cu_seqlens, max_seqlen, phase_in, phase_out)."""
    a, y, state_out, _ = _prepare_scan(
        x, B, C, dt, A, theta, lam, state, chunk, p_split, segments, return_state, y, state_out,
        None, options.get("ngroups", 0), options.get("phase", "native"), options.get("perm"),
        options.get("premix"), options.get("cu_seqlens"), options.get("max_seqlen"),
        options.get("phase_in"), options.get("phase_out"), alloc_workspace=False)
    st = load_library().m3_scan_fwd_noalloc(ctypes.byref(a), _stream_handle(stream))
    if st != 0:
        raise M3Error(st, "m3_scan_fwd_noalloc")
    return y, state_out


class ScanCall:
    """An m3_scan_fwd call marshalled once: calling it re-issues the same scan
    (same tensors, outputs and workspace) on the current stream.  Repeated
    scans then cost one C call each."""

    def __init__(self, x, B, C, dt, A, theta, lam, state: Optional[State] = None, *,
                 chunk: int = 0, p_split: int = 0, segments: int = 0, return_state: bool = True,
                 y: Optional[torch.Tensor] = None, state_out: Optional[State] = None,
                 workspace: Optional[torch.Tensor] = None, ngroups: int = 0, phase="native",
                 perm: Optional[torch.Tensor] = None, premix: Optional[Premix] = None,
                 cu_seqlens: Optional[torch.Tensor] = None, max_seqlen: Optional[int] = None,
                 phase_in: Optional[torch.Tensor] = None, phase_out: Optional[torch.Tensor] = None):
        self._keep = (x, B, C, dt, A, theta, lam, state)
        self.args, self.y, self.state_out, self.workspace = _prepare_scan(
            x, B, C, dt, A, theta, lam, state, chunk, p_split, segments, return_state, y,
            state_out, workspace, ngroups, phase, perm, premix, cu_seqlens, max_seqlen,
            phase_in, phase_out)
        self._ref = ctypes.byref(self.args)
        self._fn = load_library().m3_scan_fwd

    def __call__(self, stream=None):
        st = self._fn(self._ref, _stream_handle(stream))
        if st != 0:
            raise M3Error(st, "m3_scan_fwd")
        return self.y, self.state_out


def m3_scan_workspace_bytes(x, B, *, chunk=0, p_split=0, segments=0, cu_seqlens=None,
                            max_seqlen=None) -> int:
    Bt, L, H, R, P = x.shape
    a = ScanArgs(batch=Bt, seqlen=L, nheads=H, headdim=P, dstate=B.shape[-1], rank=R,
                 chunk=chunk, io_dtype=_io_code(x.dtype), p_split=p_split, segments=segments)
    if cu_seqlens is not None:
        a.batch = cu_seqlens.numel() - 1
        a.opt.cu_seqlens = cu_seqlens.data_ptr()
        a.opt.max_seqlen = int(L if max_seqlen is None else max_seqlen)
    return int(load_library().m3_scan_workspace_bytes(ctypes.byref(a)))


def _prepare_decode(x, B, C, dt, A, theta, lam, state, y, ngroups=0, phase="native", perm=None,
                    premix=None, phase_in=None, phase_out=None):
    Bt, H, R, P = x.shape
    N = B.shape[-1]
    G = int(ngroups) if ngroups else H
    io = _io_code(x.dtype)
    _check(x, "x", (Bt, H, R, P), x.dtype)
    _check(B, "B", (Bt, G, R, N), x.dtype)
    _check(C, "C", (Bt, G, R, N), x.dtype)
    _check(dt, "dt", (Bt, H), torch.float32)
    _check(lam, "lam", (Bt, H), torch.float32)
    if theta is not None or phase != "zero":
        _check(theta, "theta", (Bt, H, N // 2), torch.float32)
    a_tok = A.dim() == 2
    _check(A, "A", (Bt, H) if a_tok else (H,), torch.float32)
    opt, keep = _options(H, N, R, a_tok, ngroups, phase, perm, premix, x.device, Bt,
                         phase_in, phase_out)
    _check(state.h, "state.h", (Bt, H, N, P), torch.float32)
    _check(state.B_prev, "state.B_prev", (Bt, H, R, N), x.dtype)
    _check(state.x_prev, "state.x_prev", (Bt, H, R, P), x.dtype)
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", (Bt, H, R, P), x.dtype)
    a = DecodeArgs(batch=Bt, nheads=H, headdim=P, dstate=N, rank=R, io_dtype=io,
                   x=_ptr(x), B=_ptr(B), C=_ptr(C), dt=_ptr(dt), A=_ptr(A),
                   theta=_ptr(theta), lam=_ptr(lam), h=_ptr(state.h),
                   B_prev=_ptr(state.B_prev), x_prev=_ptr(state.x_prev), y=_ptr(y), opt=opt)
    a._keep = keep
    return a, y


def m3_decode_step(x, B, C, dt, A, theta, lam, state: State, *,
                   y: Optional[torch.Tensor] = None, ngroups: int = 0, phase="native",
                   perm: Optional[torch.Tensor] = None, premix: Optional[Premix] = None,
                   phase_in: Optional[torch.Tensor] = None, phase_out: Optional[torch.Tensor] = None,
                   stream=None):
    """One token for every (batch, head); ``state`` is updated in place.  Returns y_t.
    ``phase_in`` / ``phase_out``: the accumulated rotation angle before / after
    this step (float32 [batch, H, N/2]; may be one tensor, updated in place);
    the phases "no_write", "no_read", "no_write_read" rotate the write / read
    terms by it."""
    a, y = _prepare_decode(x, B, C, dt, A, theta, lam, state, y, ngroups, phase, perm, premix,
                           phase_in, phase_out)
    st = load_library().m3_decode_step(ctypes.byref(a), _stream_handle(stream))
    if st != 0:
        raise M3Error(st, "m3_decode_step")
    return y


class DecodeCall:
    """An m3_decode_step call marshalled once (fixed step inputs, state record
    and y); calling it issues that step on the current stream."""

    def __init__(self, x, B, C, dt, A, theta, lam, state: State, *,
                 y: Optional[torch.Tensor] = None, ngroups: int = 0, phase="native",
                 perm: Optional[torch.Tensor] = None, premix: Optional[Premix] = None,
                 phase_in: Optional[torch.Tensor] = None, phase_out: Optional[torch.Tensor] = None):
        self._keep = (x, B, C, dt, A, theta, lam, state)
        self.args, self.y = _prepare_decode(x, B, C, dt, A, theta, lam, state, y, ngroups, phase,
                                            perm, premix, phase_in, phase_out)
        self._ref = ctypes.byref(self.args)
        self._fn = load_library().m3_decode_step

    def __call__(self, stream=None):
        st = self._fn(self._ref, _stream_handle(stream))
        if st != 0:
            raise M3Error(st, "m3_decode_step")
        return self.y


class ScanGrads(NamedTuple):
    """Gradients from m3_scan_bwd (float32, shapes of the inputs)."""
    dx: torch.Tensor
    dB: torch.Tensor
    dC: torch.Tensor
    ddt: torch.Tensor
    dA: torch.Tensor
    dtheta: torch.Tensor
    dlam: torch.Tensor
    dh_in: Optional[torch.Tensor]
    dB_prev: Optional[torch.Tensor]
    dx_prev: Optional[torch.Tensor]
    premix: Optional[Premix] = None   # the pre-mixer's parameter gradients (premix set)


BWD_METHODS = {"auto": 0, "step": 1, "chunked": 2}


def m3_scan_bwd_supported(dstate: int, headdim: int, rank: int, io_dtype: int,
                          method: str = "auto") -> bool:
    return bool(load_library().m3_scan_bwd_method_supported(dstate, headdim, rank, io_dtype,
                                                            BWD_METHODS[method]))


def _prepare_bwd(x, B, C, dt, A, theta, lam, dy, state, dh_out, state_grads, workspace,
                 method="auto", ngroups=0, phase="native", perm=None, premix=None,
                 A_per_token=False, cu_seqlens=None, max_seqlen=None, record_grad=None):
    lib = load_library()
    Bx, L, H, R, P = x.shape
    N = B.shape[-1]
    G = int(ngroups) if ngroups else H
    io = _io_code(x.dtype)
    zero = phase == "zero"
    Bt = Bx
    if cu_seqlens is not None:
        if Bx != 1:
            raise ValueError("packed sequences: token arrays must have a leading dimension of 1")
        _check(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32)
        Bt = cu_seqlens.numel() - 1     # sequences: the state record's batch
    for t, n, shp, dt_ in ((x, "x", (Bx, L, H, R, P), x.dtype), (B, "B", (Bx, L, G, R, N), x.dtype),
                           (C, "C", (Bx, L, G, R, N), x.dtype), (dt, "dt", (Bx, L, H), torch.float32),
                           (lam, "lam", (Bx, L, H), torch.float32),
                           (theta, "theta", (Bx, L, H, N // 2), torch.float32),
                           (A, "A", (Bx, L, H) if A_per_token else (H,), torch.float32),
                           (dy, "dy", (Bx, L, H, R, P), x.dtype)):
        if t is None and n == "theta" and zero:
            continue
        _check(t, n, shp, dt_)
    if state is not None:
        _check(state.h, "state.h", (Bt, H, N, P), torch.float32)
        _check(state.B_prev, "state.B_prev", (Bt, H, R, N), x.dtype)
        _check(state.x_prev, "state.x_prev", (Bt, H, R, P), x.dtype)
    if dh_out is not None:
        _check(dh_out, "dh_out", (Bt, H, N, P), torch.float32)
    opt, keep = _options(H, N, R, A_per_token, ngroups, phase, perm, premix, x.device)
    f32 = dict(dtype=torch.float32, device=x.device)
    pg = None
    if premix is not None:
        pg = Premix(torch.empty(N, **f32), torch.empty(N, **f32), torch.empty(H, R, N, **f32),
                    torch.empty(H, R, N, **f32), torch.empty(H, **f32), premix.eps)
    g = ScanGrads(torch.empty(x.shape, **f32), torch.empty(B.shape, **f32),
                  torch.empty(C.shape, **f32), torch.empty(dt.shape, **f32),
                  torch.empty(A.shape, **f32), torch.empty(Bx, L, H, N // 2, **f32),
                  torch.empty(lam.shape, **f32),
                  torch.empty(Bt, H, N, P, **f32) if state_grads else None,
                  torch.empty(Bt, H, R, N, **f32) if state_grads else None,
                  torch.empty(Bt, H, R, P, **f32) if state_grads else None, pg)
    if method not in BWD_METHODS:
        raise ValueError("method must be one of %s" % sorted(BWD_METHODS))
    a = ScanBwdArgs(batch=Bt, seqlen=L, nheads=H, headdim=P, dstate=N, rank=R, io_dtype=io,
                    method=BWD_METHODS[method], x=_ptr(x), B=_ptr(B), C=_ptr(C), dt=_ptr(dt), A=_ptr(A),
                    theta=None if zero else _ptr(theta), lam=_ptr(lam),
                    h_in=_ptr(state.h) if state else None,
                    B_prev_in=_ptr(state.B_prev) if state else None,
                    x_prev_in=_ptr(state.x_prev) if state else None,
                    dy=_ptr(dy), dh_out=_ptr(dh_out),
                    dx=_ptr(g.dx), dB=_ptr(g.dB), dC=_ptr(g.dC), ddt=_ptr(g.ddt), dA=_ptr(g.dA),
                    dtheta=_ptr(g.dtheta), dlam=_ptr(g.dlam), dh_in=_ptr(g.dh_in),
                    dB_prev=_ptr(g.dB_prev), dx_prev=_ptr(g.dx_prev), opt=opt)
    if record_grad is not None:
        dBL, dxL = record_grad
        _check(dBL, "record_grad[0] (dB_L)", (Bt, H, R, N), torch.float32)
        _check(dxL, "record_grad[1] (dx_L)", (Bt, H, R, P), torch.float32)
        a.dB_prev_out, a.dx_prev_out = dBL.data_ptr(), dxL.data_ptr()
        keep += [dBL, dxL]
    if cu_seqlens is not None:
        a.opt.cu_seqlens = cu_seqlens.data_ptr()
        a.opt.max_seqlen = int(L if max_seqlen is None else max_seqlen)
        keep.append(cu_seqlens)
    if pg is not None:
        a.dB_norm_w, a.dC_norm_w = _ptr(pg.B_norm_w), _ptr(pg.C_norm_w)
        a.dB_bias, a.dC_bias, a.ddt_bias = _ptr(pg.B_bias), _ptr(pg.C_bias), _ptr(pg.dt_bias)
    need = lib.m3_scan_bwd_workspace_bytes(ctypes.byref(a))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=x.device)
    a.workspace = workspace.data_ptr()
    a.workspace_bytes = workspace.numel() * workspace.element_size()
    return a, g, workspace, keep


def m3_scan_bwd(x, B, C, dt, A, theta, lam, dy, state: Optional[State] = None,
                dh_out: Optional[torch.Tensor] = None, *, state_grads: bool = True,
                workspace: Optional[torch.Tensor] = None, method: str = "auto",
                ngroups: int = 0, phase: str = "native", perm: Optional[torch.Tensor] = None,
                premix: Optional[Premix] = None, A_per_token: bool = False,
                cu_seqlens: Optional[torch.Tensor] = None, max_seqlen: Optional[int] = None,
                record_grad: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                stream=None) -> ScanGrads:
    """Gradients of sum(dy * y) + sum(dh_out * h_L) of m3_scan_fwd with respect
    to every input; ``state_grads`` also returns those of the input state
    record (zero record when ``state`` is None).  ``method``: "chunked"
    (reverse mode of the chunked form), "step" (adjoint recurrence step by
    step) or "auto" (chunked where supported).  Options as m3_scan_fwd takes
    them (A per token, head groups, the phase modes of a scan, the
    pre-mixer, packed sequences); with ``A_per_token`` dA is per token, with
    ``premix`` the result's ``premix`` field holds the parameter gradients.
    Packed sequences: token arrays [1, T, ...], ``cu_seqlens`` int32 [nseq+1],
    one state record, dh_out and record gradient row per sequence;
    ``max_seqlen`` (default T) sizes the padded batch the gradient runs on.
    ``record_grad`` = (dB_L, dx_L), float32 [batch, H, R, N] and [batch, H,
    R, P]: the gradient with respect to the output record (for a sequence
    split into calls, the next call's dB_prev, dx_prev)."""
    a, g, _, _keep = _prepare_bwd(x, B, C, dt, A, theta, lam, dy, state, dh_out, state_grads,
                                  workspace, method, ngroups, phase, perm, premix, A_per_token,
                                  cu_seqlens, max_seqlen, record_grad)
    st = load_library().m3_scan_bwd(ctypes.byref(a), _stream_handle(stream))
    if st != 0:
        raise M3Error(st, "m3_scan_bwd")
    return g


class ScanBwdCall:
    """An m3_scan_bwd call marshalled once; calling it re-issues it."""

    def __init__(self, x, B, C, dt, A, theta, lam, dy, state: Optional[State] = None,
                 dh_out: Optional[torch.Tensor] = None, *, state_grads: bool = True,
                 workspace: Optional[torch.Tensor] = None, method: str = "auto",
                 ngroups: int = 0, phase: str = "native", perm: Optional[torch.Tensor] = None,
                 premix: Optional[Premix] = None):
        self._keep = (x, B, C, dt, A, theta, lam, dy, state, dh_out)
        self.args, self.grads, self.workspace, self._keep_opt = _prepare_bwd(
            x, B, C, dt, A, theta, lam, dy, state, dh_out, state_grads, workspace, method,
            ngroups, phase, perm, premix)
        self._ref = ctypes.byref(self.args)
        self._fn = load_library().m3_scan_bwd

    def __call__(self, stream=None):
        st = self._fn(self._ref, _stream_handle(stream))
        if st != 0:
            raise M3Error(st, "m3_scan_bwd")
        return self.grads
