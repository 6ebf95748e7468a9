"""The C ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU needed).

The library's sources are compiled with the host code instrumented
(`-Xarch_host -fsanitize=...`; the device code is built as usual) and linked
with tests/sanitize/host_checks.cpp, a driver that makes every kind of invalid
call the CPU tests of the ABI make (bad shapes, pointers, dtypes, workspaces,
envelopes, gates, grids, the diagnostics and test hooks) and checks each
status. Every such call is refused on the host before any HIP call."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "associative_scan_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


@pytest.mark.timeout(900)
def test_host_validation_under_asan_and_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not found")
    srcs = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith((".hip", ".cpp"))]
    srcs.append(os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"))
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}", *SAN]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "host_checks")
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", "-o", exe, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath,/opt/rocm/lib"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "host checks ok" in r.stdout, (r.stdout + r.stderr)[-4000:]
