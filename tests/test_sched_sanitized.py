"""The admission scheduler's host C++ (pa_sched.cpp), built on its own with
AddressSanitizer and UndefinedBehaviorSanitizer and driven through its C ABI by
random traces (tests/c/sched_trace.c): every call's result and the pool's
invariants are checked after each step, and the sanitizers abort on any
out-of-bounds access, use after free, leak or undefined behaviour (CPU only)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FLAGS = ["-O1", "-g", "-Wall", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
         "-I", "/opt/rocm/include"]


def build(tmp_path):
    gcc, gxx = shutil.which("gcc"), shutil.which("g++")
    if gcc is None or gxx is None:
        pytest.skip("gcc / g++ not available")
    objs = []
    for comp, std, src in ((gcc, "-std=c11", "tests/c/sched_trace.c"),
                           (gxx, "-std=c++17", "paged_kv_cache_205_amd/csrc/pa_sched.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        res = subprocess.run([comp, std, *FLAGS, "-c", os.path.join(ROOT, src), "-o", obj],
                             capture_output=True, text=True)
        if res.returncode != 0 and "asan" in res.stderr.lower():
            pytest.skip("sanitizer runtime not available")
        assert res.returncode == 0, res.stderr[-2000:]
        objs.append(obj)
    exe = str(tmp_path / "sched_trace")
    res = subprocess.run([gxx, "-fsanitize=address,undefined", *objs, "-o", exe], capture_output=True, text=True)
    if res.returncode != 0 and "asan" in res.stderr.lower():
        pytest.skip("sanitizer runtime not available")
    assert res.returncode == 0, res.stderr[-2000:]
    return exe


@pytest.mark.parametrize("seed", [205, 7, 90210])
def test_random_traces_under_sanitizers(tmp_path, seed):
    exe = build(tmp_path)
    # other preloaded libraries may precede the sanitizer runtime: do not insist on its place
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe, "1000", "500", str(seed)], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "all checks held" in run.stdout
