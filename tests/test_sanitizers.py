"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

- The CPU oracle, built with gcc and the sanitizers, runs every entry point
  on seeded random inputs and edge cases (tests/sanitize/oracle_drive.c).
- The library, with its host code instrumented (the device code is built as
  usual), is linked into the plain C client, which checks the host side of
  the boundary: argument checks, status codes, workspace sizes.  Leak
  detection is off: the HIP runtime keeps allocations until exit.

Only host code is instrumented; nothing here runs on a GPU.
"""
import importlib.util
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all".split()
CPU_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_drive")
    run(["gcc", "-std=c99", "-O1", "-g", "-ffp-contract=off", *CPU_SAN, f"-I{ROOT}/oracle",
         f"{ROOT}/tests/sanitize/oracle_drive.c", f"{ROOT}/oracle/oracle.c", "-lm", "-o", exe])
    r = run([exe], env=ENV, timeout=300)
    assert "all calls passed" in r.stdout


@pytest.mark.skipif(not shutil.which(f"{ROCM}/bin/hipcc"), reason="hipcc not installed")
def test_host_layer_under_sanitizers(tmp_path):
    spec = importlib.util.spec_from_file_location(
        "_sv_build", os.path.join(ROOT, "draft_verification_verify_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    objs = []
    for src, extra in b.SOURCES.items():
        obj = str(tmp_path / (src + ".o"))
        run([b.HIPCC, *b.COMMON, *extra, *HOST_SAN, "-c", os.path.join(b.CSRC, src), "-o", obj],
            timeout=600)
        objs.append(obj)
    lib = str(tmp_path / "libspecverify.so")
    run([b.HIPCC, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", *HOST_SAN, *objs, "-o", lib], timeout=300)
    # the client links with clang, whose sanitizer runtime the instrumented library expects
    exe = str(tmp_path / "sv_client")
    run([f"{ROCM}/llvm/bin/clang", "-std=c99", "-O1", "-g", *CPU_SAN, "-D__HIP_PLATFORM_AMD__",
         f"-I{ROOT}/include", f"-I{ROCM}/include", f"{ROOT}/tests/c_client/sv_client.c", "-o", exe,
         f"-L{tmp_path}", "-lspecverify", f"-L{ROCM}/lib", "-lamdhip64",
         f"-Wl,-rpath,{tmp_path}", f"-Wl,-rpath,{ROCM}/lib"], timeout=300)
    r = run([exe], env=ENV, timeout=300)
    assert "all checks passed" in r.stdout
