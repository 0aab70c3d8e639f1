"""The C ABI's host code (argument checks, geometry, status strings) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

api.hip is compiled for the host only, with the sanitizers, and linked with
stand-ins for the kernel launchers (tests/host_sanitize/stubs.cpp) and a
driver (tests/host_sanitize/driver.cpp) that sends every entry point invalid
and extreme configurations, NULL and fake pointers on the rejection paths,
valid calls over many geometries, and calls whose launch the (stand-in)
runtime refuses, which must come back as KARA_EHIP with the HIP code kept for
kara_last_hip_error.  The program must report every status as documented and
the sanitizers must stay silent.  No GPU code is built or run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
HERE = os.path.join(ROOT, "tests", "host_sanitize")


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not found")
def test_abi_host_code_under_sanitizers(tmp_path):
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROOT, 'decode_kv_cache_amd', 'csrc')}"]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-O1", "-g"]
    objs = []
    for src in (os.path.join(ROOT, "decode_kv_cache_amd", "csrc", "api.hip"), os.path.join(HERE, "stubs.cpp"),
                os.path.join(HERE, "driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [CLANG, "-x", "hip", "--cuda-host-only", "--offload-arch=gfx950", "-std=c++17", *san, *inc, "-c", src,
               "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    exe = str(tmp_path / "abi_host")
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
    assert r.returncode == 0, r.stdout + r.stderr[-3000:]
    assert "0 failures" in r.stdout
