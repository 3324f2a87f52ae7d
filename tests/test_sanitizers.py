"""The CPU oracle and the host side of the C ABI built with AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): tests/sanitize/oracle_driver.c drives every oracle entry point over small, grouped, empty and
degenerate shapes and all masks; tests/sanitize/capi_driver.cpp drives every C-ABI entry point's argument
checks, with the kernel launchers replaced by stubs (tests/sanitize/sanitize_stubs.cpp) and capi.hip's host
code compiled with the sanitizers. Any sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
SAN_FLAGS = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def run(cmd, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp"] + SAN_FLAGS +
        [os.path.join(ROOT, "oracle", "attn_oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    r = run([exe], env=env)
    assert "all checks passed" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("g++") is None, reason="needs hipcc and g++")
def test_capi_host_code_under_asan_ubsan(tmp_path):
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "transformer_scaled_dot_amd", "csrc")]
    # device code is compiled as usual (the scratch array of attn_bwd_noalloc is a device variable); the
    # sanitizers apply to the host pass only
    host = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC"]
    xs = [x for f in SAN_FLAGS for x in ("-Xarch_host", f)]
    objs = []
    for src in (os.path.join(ROOT, "transformer_scaled_dot_amd", "csrc", "capi.hip"), os.path.join(SAN, "sanitize_stubs.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        run([HIPCC] + host + xs + inc + ["-c", src, "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "capi_driver.o")
    run(["g++", "-O1", "-g", "-std=c++17"] + SAN_FLAGS + inc + ["-c", os.path.join(SAN, "capi_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "capi_san")
    run(["g++"] + SAN_FLAGS + objs + [drv, "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-o", exe])
    # leaks inside the HIP runtime at exit are not this code's
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1",
               LD_LIBRARY_PATH=os.path.join(ROCM, "lib") + ":" + os.environ.get("LD_LIBRARY_PATH", ""))
    r = run([exe], env=env)
    assert "all checks passed" in r.stdout
