"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU):
the fp64 oracle driven through every entry point on small inputs and edge
cases (tests/sanitize/orc_driver.c), and the C ABI's host side -- argument
checks, workspace sizing, error paths -- driven with arguments it must
reject (tests/sanitize/abi_driver.c), against a copy of the library whose
host code alone is instrumented (the device code cannot be)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])}...\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "orc_san")
    run(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-fsanitize=address,undefined",
         "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off",
         os.path.join(SAN, "orc_driver.c"), os.path.join(ROOT, "oracle", "orc.c"), "-o", exe,
         "-lm"])
    r = run([exe], env=ENV)
    assert "oracle sanitizer run ok" in r.stdout
    assert "runtime error" not in r.stderr


HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="ROCm compilers not installed")
def test_host_api_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    from moe_layer_zero_amd import build as B
    csrc = os.path.join(ROOT, "moe_layer_zero_amd", "csrc")
    objs = []
    for src in B.SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        built = os.path.join(B.BUILD, src.replace(".hip", ".o"))
        if (src != "api.hip" and os.path.exists(built) and
                os.path.getmtime(built) >= os.path.getmtime(os.path.join(csrc, src))):
            objs.append(built)  # device-only changes do not matter here: reuse the build
            continue
        cmd = [HIPCC, *B.COMMON, "-c", os.path.join(csrc, src), "-o", obj]
        if src == "api.hip":  # host code instrumented; device code as usual
            cmd[1:1] = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                        "-fsanitize=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
        if src in B.STRICT_FP:
            cmd.insert(1, "-ffp-contract=off")
        if src in B.NO_ATOMIC_OPT:
            cmd[1:1] = ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]
        run(cmd)
        objs.append(obj)
    lib = str(tmp_path / "libzcmoe_san.so")
    run([HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *objs, "-o", lib])
    exe = str(tmp_path / "abi_san")
    run([CLANG, "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
         os.path.join(SAN, "abi_driver.c"), lib, f"-Wl,-rpath,{tmp_path}", "-o", exe, "-lm"])
    # the HIP runtime's own allocations are not the library's: leaks off
    env = dict(ENV, ASAN_OPTIONS="detect_leaks=0")
    r = run([exe], env=env)
    assert "host API sanitizer run ok" in r.stdout
    assert "runtime error" not in r.stderr
