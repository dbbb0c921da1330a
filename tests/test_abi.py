"""C ABI contract, checked without a GPU: the library loads, exports every
function that include/m3scan.h declares, the ctypes structures match the C
layout, and argument validation returns its status codes before any HIP call.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "m3scan.h")

from mamba_selective_ssm_amd import binding  # noqa: E402

FAKE = 0x7F0000000000   # never dereferenced: validation fails before any device access


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(m3_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH],
                         stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = set(re.findall(r" T (m3_\w+)", out))
    assert set(names) <= exported, set(names) - exported


def test_struct_layout_matches_header(tmp_path):
    """Compile a tiny C program against the header and compare offsets."""
    fields_s = [f[0] for f in binding.ScanArgs._fields_]
    fields_d = [f[0] for f in binding.DecodeArgs._fields_]
    fields_o = [f[0] for f in binding.Options._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>', '#include "m3scan.h"', "int main(void){"]
    src.append('printf("%zu\\n", sizeof(m3_options));')
    for f in fields_o:
        src.append('printf("%%zu\\n", offsetof(m3_options, %s));' % f)
    src.append('printf("%zu\\n", sizeof(m3_scan_args));')
    for f in fields_s:
        src.append('printf("%%zu\\n", offsetof(m3_scan_args, %s));' % f)
    src.append('printf("%zu\\n", sizeof(m3_decode_args));')
    for f in fields_d:
        src.append('printf("%%zu\\n", offsetof(m3_decode_args, %s));' % f)
    src.append("return 0;}")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(c)], check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], stdout=subprocess.PIPE, text=True,
                                           check=True).stdout.split()]
    expect = [ctypes.sizeof(binding.Options)]
    expect += [getattr(binding.Options, f).offset for f in fields_o]
    expect += [ctypes.sizeof(binding.ScanArgs)]
    expect += [getattr(binding.ScanArgs, f).offset for f in fields_s]
    expect += [ctypes.sizeof(binding.DecodeArgs)]
    expect += [getattr(binding.DecodeArgs, f).offset for f in fields_d]
    assert vals == expect


def test_bwd_struct_layout_matches_header(tmp_path):
    fields = [f[0] for f in binding.ScanBwdArgs._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>', '#include "m3scan.h"', "int main(void){",
           'printf("%zu\\n", sizeof(m3_scan_bwd_args));']
    src += ['printf("%%zu\\n", offsetof(m3_scan_bwd_args, %s));' % f for f in fields]
    src.append("return 0;}")
    c = tmp_path / "layout_bwd.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout_bwd"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(c)], check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], stdout=subprocess.PIPE, text=True,
                                           check=True).stdout.split()]
    assert vals == [ctypes.sizeof(binding.ScanBwdArgs)] + \
        [getattr(binding.ScanBwdArgs, f).offset for f in fields]


def bwd_args(**kw):
    a = binding.ScanBwdArgs(batch=2, seqlen=10, nheads=3, headdim=64, dstate=64, rank=1,
                            io_dtype=1)
    ptrs = ["x", "B", "C", "dt", "A", "theta", "lam", "dy", "dx", "dB", "dC", "ddt", "dA",
            "dtheta", "dlam"]
    for i, p in enumerate(ptrs):
        setattr(a, p, FAKE + i * (1 << 32))
    a.workspace = FAKE + (30 << 32)
    a.workspace_bytes = 1 << 40
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(dstate=5), -2), (dict(headdim=0), -2), (dict(io_dtype=3), -4),
    (dict(headdim=128), -3), (dict(dstate=256), -3), (dict(rank=3), -3),
    (dict(dy=None), -1), (dict(dA=None), -1), (dict(dx=None), -1),
    (dict(h_in=FAKE + (20 << 32)), -1),                    # partial state record
    (dict(dh_in=FAKE + (21 << 32)), -1),                   # partial record gradients
    (dict(dx=FAKE + 8), -5),
    (dict(dx=FAKE), -7),                                   # dx aliases x
    (dict(dB=FAKE + (10 << 32) + 64), -7),                 # dB overlaps dC
    (dict(workspace=None), -6), (dict(workspace_bytes=16), -6),
    (dict(workspace=FAKE + (30 << 32) + 16), -5),
    (dict(method=3), -9), (dict(method=-1), -9),           # not an m3_bwd_method
    (dict(method=2, headdim=16), -3),                      # chunked: headdim 32 or 64
    (dict(method=2, dstate=48), -3),                       # chunked: dstate 32, 64, 128
    (dict(method=2, dstate=128, io_dtype=0), -3),          # chunked float32: dstate <= 64
    (dict(method=1, headdim=128), -3),
    # options of the gradient
    (dict(opt=binding.Options(A_per_token=2)), -9),
    # the output record's gradient: both or neither, aligned, not an output
    (dict(dB_prev_out=FAKE + (25 << 32)), -1),
    (dict(dB_prev_out=FAKE + (25 << 32), dx_prev_out=FAKE + (26 << 32) + 4), -5),
    (dict(dB_prev_out=FAKE + (25 << 32), dx_prev_out=FAKE + (26 << 32), dx=FAKE + (26 << 32)), -7),
    # per-token decay: A and dA are [batch, seqlen, nheads] (dA 128 bytes into A overlaps it)
    (dict(opt=binding.Options(A_per_token=1), dA=FAKE + (4 << 32) + 128), -7),
    (dict(opt=binding.Options(A_per_token=1), A=None), -1),
    (dict(opt=binding.Options(max_seqlen=11, cu_seqlens=FAKE + (23 << 32))), -9),  # > seqlen
    (dict(opt=binding.Options(max_seqlen=-1, cu_seqlens=FAKE + (23 << 32))), -9),
    (dict(opt=binding.Options(max_seqlen=4, cu_seqlens=FAKE + (23 << 32) + 4)), -5),
    (dict(opt=binding.Options(max_seqlen=4, cu_seqlens=FAKE + (23 << 32)), dx=FAKE + (23 << 32)), -7),
    (dict(opt=binding.Options(phase_out=FAKE + (23 << 32))), -3),
    (dict(opt=binding.Options(phase_mode=4)), -9),           # decode-only phase mode
    (dict(opt=binding.Options(phase_mode=7)), -9),
    (dict(opt=binding.Options(ngroups=2)), -9),              # 3 heads
    (dict(opt=binding.Options(ngroups=-1)), -9),
    (dict(opt=binding.Options(phase_mode=3)), -1),           # shuffle without a permutation
    (dict(opt=binding.Options(phase_mode=1), theta=None, dtheta=None, dx=None), -1),
    (dict(theta=None), -1),                                  # theta needed unless zeroed
    (dict(opt=binding.Options(premix=1, norm_eps=-1.0)), -9),
    (dict(opt=binding.Options(premix=2)), -9),
    (dict(dB_norm_w=FAKE + (22 << 32)), -9),                 # parameter gradient without premix
    (dict(opt=binding.Options(premix=1), dB_bias=FAKE + (10 << 32)), -7),   # overlaps dC
    (dict(opt=binding.Options(premix=1), ddt_bias=FAKE + (22 << 32) + 4), -5),
    (dict(opt=binding.Options(premix=1, B_norm_w=FAKE + (24 << 32)), dx=FAKE + (24 << 32)), -7),
])
def test_bwd_validation_codes(lib, kw, code):
    assert lib.m3_scan_bwd(ctypes.byref(bwd_args(**kw)), None) == code


def test_bwd_supported_and_workspace(lib):
    for io in (0, 1):
        for N in (16, 32, 64, 128):
            for P in (16, 32, 64):
                for R in (1, 2, 4):
                    assert lib.m3_scan_bwd_supported(N, P, R, io) == 1
                    assert lib.m3_scan_bwd_method_supported(N, P, R, io, 1) == 1
                    chunked = P in (32, 64) and N in ((32, 64, 128) if io == 1 else (32, 64))
                    assert lib.m3_scan_bwd_method_supported(N, P, R, io, 2) == int(chunked)
                    assert lib.m3_scan_bwd_method_supported(N, P, R, io, 0) == 1
    assert lib.m3_scan_bwd_supported(64, 128, 1, 1) == 0
    assert lib.m3_scan_bwd_method_supported(64, 64, 1, 1, 3) == 0
    ws = lib.m3_scan_bwd_workspace_bytes(ctypes.byref(bwd_args(seqlen=2048, method=1)))
    # one checkpoint per 32 steps per (b, h), N x P floats, plus scratch
    assert ws >= 6 * 64 * 64 * 64 * 4
    # chunked: per (b, h) the two local sums of 32 chunks and 33 states and
    # adjoints, stored in the io type (bf16: 2 bytes)
    wc = lib.m3_scan_bwd_workspace_bytes(ctypes.byref(bwd_args(seqlen=2048, method=2)))
    assert wc >= 6 * (32 * 2 + 33 * 2) * 64 * 64 * 2
    wf = lib.m3_scan_bwd_workspace_bytes(ctypes.byref(bwd_args(seqlen=2048, method=2, io_dtype=0)))
    assert wf >= 6 * (32 * 2 + 33 * 2) * 64 * 64 * 4
    assert lib.m3_scan_bwd_workspace_bytes(ctypes.byref(bwd_args(seqlen=2048))) == wc
    assert lib.m3_scan_bwd_workspace_bytes(ctypes.byref(bwd_args(method=5))) == 0


def test_bwd_option_workspace(lib):
    """The option maps' buffers follow the plain gradient's workspace: the
    pre-mixer and head groups add the materialised B, C and their gradients,
    the phase maps theta and its gradient; rejected options size nothing."""
    ws = lambda **kw: lib.m3_scan_bwd_workspace_bytes(ctypes.byref(bwd_args(seqlen=256, **kw)))
    plain = ws()
    tok, N, R = 2 * 256 * 3, 64, 1
    assert ws(opt=binding.Options(phase_mode=2)) >= plain + 2 * tok * (N // 2) * 4
    assert ws(opt=binding.Options(ngroups=1)) >= plain + tok * R * N * (2 * 2 + 2 * 4)
    assert ws(opt=binding.Options(premix=1)) > ws(opt=binding.Options(ngroups=1))
    assert ws(opt=binding.Options(ngroups=3)) == plain          # one group per head
    assert ws(opt=binding.Options(A_per_token=1)) == plain       # no maps needed
    assert ws(opt=binding.Options(A_per_token=2)) == 0
    # packed sequences (2 of them in 256 tokens): the gradient runs on a padded
    # batch of max_seqlen tokens each, its inputs and gradients moved there
    cu = FAKE + (23 << 32)
    p64, p128 = (ws(opt=binding.Options(cu_seqlens=cu, max_seqlen=m)) for m in (64, 128))
    assert p128 > p64 > 0
    assert p128 - p64 >= 2 * 64 * 3 * (2 * 64 * 2 + 2 * 64 * 2 + 64 * 4 + 2 * 64 * 4)
    assert ws(opt=binding.Options(cu_seqlens=cu, max_seqlen=257)) == 0
    assert ws(opt=binding.Options(phase_mode=5)) == 0
    assert lib.m3_scan_bwd_workspace_bytes(ctypes.byref(bwd_args(batch=0))) == 0
    assert lib.m3_scan_bwd_workspace_bytes(
        ctypes.byref(bwd_args(batch=0, opt=binding.Options(premix=1)))) == 0


def test_version_and_status_strings(lib):
    assert lib.m3_abi_version() == 6
    for code in range(-10, 1):
        s = lib.m3_status_string(code)
        assert s and s != b"unknown status"
    assert lib.m3_status_string(-99) == b"unknown status"
    assert lib.m3_last_hip_error() == 0




OPTION_FIELDS = {f[0] for f in binding.Options._fields_}


def scan_args(**kw):
    base = dict(batch=2, seqlen=10, nheads=3, headdim=32, dstate=64, rank=1, chunk=0,
                io_dtype=1, p_split=0, segments=0)
    ptrs = ["x", "B", "C", "dt", "A", "theta", "lam", "y"]
    a = binding.ScanArgs(**base)
    for i, p in enumerate(ptrs):
        setattr(a, p, FAKE + i * (1 << 32))
    for k, v in kw.items():
        setattr(a.opt if k in OPTION_FIELDS else a, k, v)
    return a


def run_scan(lib, a):
    return lib.m3_scan_fwd(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,code", [
    (dict(dstate=63), -2), (dict(headdim=0), -2), (dict(rank=0), -2), (dict(batch=-1), -2),
    (dict(seqlen=-5), -2), (dict(chunk=-1), -2),
    (dict(io_dtype=7), -4),
    (dict(dstate=48), -3), (dict(rank=3), -3), (dict(chunk=24), -3), (dict(headdim=40), -3),
    (dict(p_split=3), -3),
    (dict(seqlen=1000, segments=4), -6),                    # needs a workspace
    (dict(seqlen=1000, segments=4, workspace=FAKE + (30 << 32) + 16, workspace_bytes=1 << 40), -5),
    (dict(x=None), -1), (dict(y=None), -1), (dict(theta=None), -1), (dict(A=None), -1),
    (dict(h_in=FAKE + (20 << 32)), -1),                      # partial state record
    (dict(h_out=FAKE + (21 << 32), B_prev_out=FAKE + (22 << 32)), -1),
    (dict(x=FAKE + 8), -5), (dict(dt=FAKE + 4), -5),
    (dict(y=FAKE), -7),                                      # y aliases x
    (dict(y=FAKE + (1 << 32) + 64), -7),                     # y overlaps B
    # options
    (dict(ngroups=2), -9), (dict(ngroups=-1), -9), (dict(A_per_token=2), -9),
    (dict(phase_mode=4), -9), (dict(phase_mode=-1), -9), (dict(premix=2), -9),
    (dict(premix=1, norm_eps=-1.0), -9), (dict(premix=1, norm_eps=float("nan")), -9),
    (dict(phase_mode=3), -1),                                # shuffle without a permutation
    (dict(phase_mode=3, phase_perm=FAKE + (40 << 32) + 4), -5),
    (dict(premix=1, B_bias=FAKE + (41 << 32) + 8), -5),
    (dict(theta=None, phase_mode=1, x=FAKE + 8), -5),        # zero phase: theta may be NULL
    (dict(theta=None, phase_mode=2, x=FAKE + 8), -1),
    (dict(premix=1, C_bias=FAKE + (7 << 32)), -7),           # y overlaps the C bias
    # packed sequences
    (dict(cu_seqlens=FAKE + (42 << 32), max_seqlen=11), -9),  # longer than the packed axis
    (dict(cu_seqlens=FAKE + (42 << 32), max_seqlen=-1), -9),
    (dict(cu_seqlens=FAKE + (42 << 32) + 4, max_seqlen=10), -5),
    (dict(cu_seqlens=FAKE + (7 << 32), max_seqlen=10), -7),   # y overlaps the offsets
    # accumulated angle; rotation removed from writing / readout (decode only)
    (dict(phase_mode=5), -9), (dict(phase_mode=6), -9), (dict(phase_mode=7), -9),
    (dict(phase_in=FAKE + (43 << 32) + 4), -5),
    (dict(phase_out=FAKE + (43 << 32) + 8), -5),
    (dict(phase_out=FAKE + (7 << 32)), -7),                  # phase_out overlaps y
    (dict(phase_out=FAKE + (43 << 32)), -6),                 # needs a workspace
])
def test_scan_validation_codes(lib, kw, code):
    assert run_scan(lib, scan_args(**kw)) == code


def test_scan_state_record_in_place(lib):
    """The output state record may be exactly the input record: validation
    accepts it (the workspace then holds a copy of the input record, so it
    grows by the record's size); any partial overlap is still rejected."""
    h, bp, xp = FAKE + (20 << 32), FAKE + (21 << 32), FAKE + (22 << 32)
    rec_in = dict(h_in=h, B_prev_in=bp, x_prev_in=xp)
    ws = lambda **kw: lib.m3_scan_workspace_bytes(ctypes.byref(scan_args(**kw)))
    base = ws(**rec_in, h_out=FAKE + (23 << 32), B_prev_out=FAKE + (24 << 32),
              x_prev_out=FAKE + (25 << 32))
    inplace = ws(**rec_in, h_out=h, B_prev_out=bp, x_prev_out=xp)
    nbh, N, P, R = 2 * 3, 64, 32, 1
    assert base == 0
    assert inplace >= nbh * N * P * 4 + nbh * R * (N + P) * 2
    # in place needs that workspace
    assert run_scan(lib, scan_args(**rec_in, h_out=h, B_prev_out=bp, x_prev_out=xp)) == -6
    # partial overlaps of the two records, and a record that is only partly in place
    assert run_scan(lib, scan_args(**rec_in, h_out=h + 16, B_prev_out=bp, x_prev_out=xp)) == -7
    assert run_scan(lib, scan_args(**rec_in, h_out=h, B_prev_out=FAKE + (24 << 32),
                                   x_prev_out=xp)) == -7
    # the in-place record must still not overlap y or the workspace
    assert run_scan(lib, scan_args(**rec_in, h_out=h, B_prev_out=bp, x_prev_out=xp,
                                   workspace=h, workspace_bytes=inplace)) == -7


def test_scan_noalloc_validation(lib):
    """The allocation-free scan checks its arguments like m3_scan_fwd (before
    any HIP call), ignores the workspace fields, and rejects a call whose
    scratch exceeds M3_NOALLOC_SCRATCH_BYTES with M3_ERR_SCRATCH."""
    noalloc = lambda a: lib.m3_scan_fwd_noalloc(ctypes.byref(a), None)
    assert noalloc(scan_args(dstate=63)) == -2
    assert noalloc(scan_args(x=None)) == -1
    assert noalloc(scan_args(y=FAKE)) == -7
    # 64 x 16 heads x 64 segments of 4096-token chunks: far more than 32 MiB of records
    big = dict(batch=64, nheads=16, seqlen=1 << 16, headdim=64, dstate=64, segments=64)
    ws = lib.m3_scan_workspace_bytes(ctypes.byref(scan_args(**big)))
    assert ws > 32 << 20
    assert noalloc(scan_args(**big)) == -10
    # a caller's (bogus) workspace is ignored, not validated
    assert noalloc(scan_args(**big, workspace=FAKE + 8, workspace_bytes=1)) == -10
    assert lib.m3_status_string(-10) != b"unknown status"


def test_scan_zero_work_is_ok_without_pointers(lib):
    a = binding.ScanArgs(batch=0, seqlen=100, nheads=4, headdim=64, dstate=64, rank=1,
                         io_dtype=1)
    assert run_scan(lib, a) == 0
    a = binding.ScanArgs(batch=3, seqlen=100, nheads=0, headdim=64, dstate=64, rank=1,
                         io_dtype=0)
    assert run_scan(lib, a) == 0


def test_scan_null_args(lib):
    assert lib.m3_scan_fwd(None, None) == -1
    assert lib.m3_decode_step(None, None) == -1


def decode_args(**kw):
    a = binding.DecodeArgs(batch=4, nheads=2, headdim=64, dstate=128, rank=4, io_dtype=1)
    for i, p in enumerate(["x", "B", "C", "dt", "A", "theta", "lam", "h", "B_prev", "x_prev", "y"]):
        setattr(a, p, FAKE + i * (1 << 32))
    for k, v in kw.items():
        setattr(a.opt if k in OPTION_FIELDS else a, k, v)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(dstate=5), -2), (dict(rank=0), -2), (dict(io_dtype=2), -4),
    (dict(rank=3), -3), (dict(headdim=6), -3),
    (dict(h=None), -1), (dict(y=None), -1),
    (dict(h=FAKE + (7 << 32) + 4), -5),
    (dict(y=FAKE + (7 << 32)), -7),          # y aliases the state
    (dict(B_prev=FAKE + (1 << 32)), -7),     # state record aliases a step input
    (dict(ngroups=3), -9), (dict(phase_mode=9), -9), (dict(premix=1, norm_eps=-2.0), -9),
    (dict(phase_mode=3), -1),
    (dict(theta=None, phase_mode=1, h=FAKE + (7 << 32) + 4), -5),   # zero phase: theta may be NULL
    (dict(theta=None, h=FAKE + (7 << 32) + 4), -1),
    (dict(premix=1, dt_bias=FAKE + (10 << 32)), -7),                # y overlaps the dt bias
    (dict(premix=1, B_bias=FAKE + (7 << 32)), -7),                  # state overlaps the B bias
    (dict(cu_seqlens=FAKE + (20 << 32), max_seqlen=1), -9),         # scans only
    (dict(phase_mode=7), -9), (dict(phase_mode=-2), -9),
    (dict(theta=None, phase_mode=4, h=FAKE + (7 << 32) + 4), -1),   # removal modes read theta
    (dict(phase_in=FAKE + (12 << 32) + 4), -5),
    (dict(phase_out=FAKE + (7 << 32)), -7),                         # phase_out overlaps the state
    (dict(phase_out=FAKE + (10 << 32) + 16), -7),                   # ... or y
    (dict(phase_out=FAKE + (5 << 32)), -7),                         # ... or theta
    (dict(phase_in=FAKE + (7 << 32)), -7),                          # state overlaps phase_in
])
def test_decode_validation_codes(lib, kw, code):
    assert lib.m3_decode_step(ctypes.byref(decode_args(**kw)), None) == code


def test_supported_sets(lib):
    for io in (0, 1):
        for N in (16, 32, 64, 128):
            for R in (1, 2, 4):
                assert lib.m3_scan_supported(N, 64, R, 0, io) == 1
                assert lib.m3_decode_supported(N, 64, R, io) == 1
    assert lib.m3_scan_supported(64, 64, 1, 32, 1) == 1
    assert lib.m3_scan_supported(64, 64, 1, 128, 1) == 1
    assert lib.m3_scan_supported(96, 64, 1, 0, 1) == 0
    assert lib.m3_scan_supported(64, 24, 1, 0, 1) == 0
    assert lib.m3_scan_workspace_bytes(ctypes.byref(scan_args())) == 0
    # segmented calls need one record (N*P state + totals) per (b, h, segment boundary)
    ws = lib.m3_scan_workspace_bytes(ctypes.byref(scan_args(seqlen=1000, segments=4)))
    assert ws >= 2 * 3 * 3 * 64 * 32 * 4
    assert lib.m3_scan_workspace_bytes(ctypes.byref(scan_args(dstate=63))) == 0


def test_scan_workspace_for_the_accumulated_angle(lib):
    """phase_out needs float64 partial sums per (row, head, 64-token block, pair)."""
    base = lib.m3_scan_workspace_bytes(ctypes.byref(scan_args(seqlen=1000)))
    ws = lib.m3_scan_workspace_bytes(ctypes.byref(scan_args(seqlen=1000, phase_out=FAKE + (43 << 32))))
    assert ws >= base + 2 * 3 * 16 * 32 * 8


def test_bench_algorithmic_sizes():
    """The benchmark's per-call byte and flop counts at the workloads' sizes:
    bf16 x, B, C, y (2 bytes), float32 theta, dt, lam, A and state record; the
    per head-token bytes e (2RP + 2RN) + 4 (N/2 + 2) are 648, 3336 and 1032
    for the single-layer, MIMO and long-context workloads."""
    import bench
    from mamba_selective_ssm_amd import synth
    for name, per_ht in (("prefill_bf16", 648), ("mimo_prefill_bf16", 3336),
                         ("long_prefill_bf16", 1032)):
        w = synth.WORKLOADS[name]
        R, P, N, H = w.rank, w.headdim, w.dstate, w.heads
        rec = w.batch * H * (4 * N * P + 2 * R * (N + P))
        assert bench.scan_algorithmic_bytes(w) == w.batch * w.seqlen * H * per_ht + rec + 4 * H
        Q = w.chunk
        assert bench.scan_dense_flops(w) == w.batch * w.seqlen * H * (
            2 * Q * R * R * (N + P) + 4 * R * N * P)
    # decode: state in and out, record in and out, step inputs, y
    wd = synth.WORKLOADS["decode"]
    assert bench.decode_algorithmic_bytes(wd) == 256 * 32 * 71944 + 4 * 32


def test_bench_refuses_more_than_one_gpu():
    import bench
    assert bench.main(["--gpus", "2"]) == 2
