"""AddressSanitizer and UndefinedBehaviorSanitizer runs on the CPU: the fp64
oracle (oracle/m3_oracle.c) and the host side of libm3scan (argument
validation, variant choice and workspace sizing in csrc/m3_abi.hip), each
driven by a small program under tests/sanitize/ that checks its own results.
Device code is not sanitized (no GPU here); the library's other objects are
linked as built.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "san")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ENV = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def run(cmd, env=None):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env)
    assert r.returncode == 0, "%s\n%s" % (" ".join(cmd), r.stdout[-4000:])
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    run(["gcc", "-std=c99", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-pthread", os.path.join(SAN, "oracle_driver.c"),
         os.path.join(ROOT, "oracle", "m3_oracle.c"), "-lm", "-o", exe])
    out = run([exe], env=dict(ENV, ASAN_OPTIONS=ENV["ASAN_OPTIONS"] + ":detect_leaks=1"))
    assert "all checks passed" in out


def test_host_abi_layer_under_asan_and_ubsan():
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "lib", "llvm", "bin", "clang++")
    build = os.path.join(ROOT, "_build")
    objs = sorted(os.path.join(build, f) for f in os.listdir(build) if f.endswith(".hip.o")) \
        if os.path.isdir(build) else []
    if not (os.path.exists(hipcc) and os.path.exists(clang)) or not objs:
        pytest.skip("hipcc or the library's objects are missing (run the build first)")
    os.makedirs(OUT, exist_ok=True)
    abi_o = os.path.join(OUT, "m3_abi.o")
    # host code only is instrumented: every sanitizer flag is for the host pass
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-I" + os.path.join(ROOT, "include"),
         "-I" + os.path.join(ROOT, "mamba_selective_ssm_amd", "csrc"),
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-result"]
        + host_san + ["-c", os.path.join(ROOT, "mamba_selective_ssm_amd", "csrc", "m3_abi.hip"),
                      "-o", abi_o])
    drv_o = os.path.join(OUT, "abi_driver.o")
    run([clang, "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-I" + os.path.join(ROOT, "include"), "-c",
         os.path.join(SAN, "abi_driver.cpp"), "-o", drv_o])
    exe = os.path.join(OUT, "abi_driver")
    others = [o for o in objs if not os.path.basename(o).startswith("m3_abi")]
    run([clang, "-fsanitize=address,undefined", "-o", exe, drv_o, abi_o] + others
        + ["-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    # the HIP runtime's own allocations at load time are not this library's
    out = run([exe], env=dict(ENV, ASAN_OPTIONS=ENV["ASAN_OPTIONS"] + ":detect_leaks=0"))
    assert "all checks passed" in out
