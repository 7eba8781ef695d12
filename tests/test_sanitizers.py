"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

libgattn's sources are compiled as usual for gfx950, with the host side
instrumented (every argument check, size query and planner is host code;
device code is left as it is), oracle.c likewise, and both are linked with
tests/sanitize_driver.c, which
drives every ABI entry point through its error paths and the oracle through
every option on small graphs.  A memory error, a leak or undefined
behaviour ends the run with a report.  Nothing here touches a GPU.
"""
import concurrent.futures as cf
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "graph_sparse_attention_amd", "csrc")
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain not installed")
def test_host_code_under_asan_and_ubsan(tmp_path):
    from graph_sparse_attention_amd import build as b
    def compile_lib(src):
        obj = str(tmp_path / (src + ".o"))
        _run([HIPCC, f"--offload-arch={b.ARCH}", "-std=c++17", "-fPIC", *SAN, "-Xclang", "-target-feature",
              "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
              "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    jobs = max(1, min(len(b.SOURCES), os.cpu_count() or 4, int(os.environ.get("MAX_JOBS", "16"))))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_lib, b.SOURCES))
    common = ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
              "-I", os.path.join(ROOT, "oracle")]
    for src, name in ((os.path.join(ROOT, "oracle", "oracle.c"), "oracle.o"),
                      (os.path.join(ROOT, "tests", "sanitize_driver.c"), "driver.o")):
        _run([CLANG, "-std=c11", "-ffp-contract=off", *SAN, *common, "-c", src, "-o", str(tmp_path / name)])
        objs.append(str(tmp_path / name))
    exe = str(tmp_path / "sanitize_driver")
    _run([HIPCC, f"--offload-arch={b.ARCH}", *SAN, "-o", exe, *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-lm"])
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "abort_on_error=0:halt_on_error=1:detect_leaks=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"sanitized run failed ({r.returncode}):\n{r.stdout}\n{r.stderr[-6000:]}"
    assert "all checks passed" in r.stdout
