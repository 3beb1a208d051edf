"""CPU builds under the address and undefined-behaviour sanitizers (no GPU):

* the fp64 oracle (``oracle/gqa_oracle.c``) with a driver that calls every entry point on small
  shapes and every option (``tests/sanitize/oracle_driver.c``);
* the C ABI's host-side argument validation (``csrc/gqa_attn_api.cpp``, host code instrumented,
  device code untouched) with a driver that makes every entry point refuse its arguments and
  checks the workspace queries over many shapes (``tests/sanitize/api_driver.cpp``).

Any sanitizer report aborts the driver (``-fno-sanitize-recover=all``), so a clean exit with the
driver's own "ok" line is the pass condition."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(exe, env_extra=None):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    env.update(env_extra or {})
    return subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)


def _instrumented(exe):
    deps = subprocess.run(["ldd", exe], capture_output=True, text=True).stdout
    return "libasan" in deps and "libubsan" in deps


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", "-O1", "-g", *SAN, "-fopenmp", "-std=c11",
                    os.path.join(ROOT, "oracle", "gqa_oracle.c"),
                    os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"], check=True)
    assert _instrumented(exe)
    r = _run(exe, {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1"})
    assert r.returncode == 0 and "oracle driver ok" in r.stdout, r.stdout + r.stderr


def test_abi_validation_under_sanitizers(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    lib_dir = os.path.join(ROOT, "grouped_query_softmax_amd")
    if not hipcc or not os.path.exists(os.path.join(lib_dir, "libgqa_attn.so")):
        pytest.skip("needs hipcc and the built library")
    api_obj = str(tmp_path / "api.o")
    host_san = []
    for flag in SAN:
        host_san += ["-Xarch_host", flag]
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                    f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(lib_dir, 'csrc')}",
                    *host_san, "-x", "hip", "-c",
                    os.path.join(lib_dir, "csrc", "gqa_attn_api.cpp"), "-o", api_obj],
                   check=True, capture_output=True)
    drv_obj = str(tmp_path / "driver.o")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", *SAN, f"-I{os.path.join(ROOT, 'include')}",
                    "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-c",
                    os.path.join(HERE, "api_driver.cpp"), "-o", drv_obj], check=True)
    exe = str(tmp_path / "api_driver")
    # the instrumented validation object comes first, so the driver calls it rather than the
    # library's own copy; the library supplies the launchers and split planning
    subprocess.run(["g++", *SAN, drv_obj, api_obj, f"-L{lib_dir}", "-lgqa_attn",
                    f"-Wl,-rpath,{lib_dir}", "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", exe], check=True)
    assert _instrumented(exe)
    r = _run(exe)
    assert r.returncode == 0 and "api driver ok" in r.stdout, r.stdout + r.stderr
