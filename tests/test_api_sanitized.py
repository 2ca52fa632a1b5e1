"""The C-ABI layer (csrc/api.hip: argument validation, dispatch, error
mapping) built for the host alone with AddressSanitizer and
UndefinedBehaviorSanitizer, its kernel launchers and HIP runtime calls
replaced by the stubs of tests/native/api_asan_driver.cpp, and driven through
every entry point with valid, invalid and extreme arguments.  Host code only:
no GPU code is built or run."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/bin/amdclang++"
# host-only HIP compile; each sanitizer flag applies to the host pass only
FLAGS = ["-x", "hip", "--offload-host-only", "-std=c++17", "-O1", "-g",
         "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address,undefined",
         "-Xarch_host", "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include")]


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not available")
def test_api_layer_under_asan_and_ubsan(tmp_path):
    objs = []
    for src in (os.path.join(ROOT, "sparse_memory_linear_sdm_amd", "csrc", "api.hip"),
                os.path.join(ROOT, "tests", "native", "api_asan_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run([CLANG, *FLAGS, "-c", src, "-o", obj], check=True)
        objs.append(obj)
    exe = str(tmp_path / "api_asan")
    subprocess.run([CLANG, "-Xarch_host", "-fsanitize=address,undefined", *objs, "-o", exe],
                   check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0")
    env.pop("SDM_DEBUG_SYNC", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert r.stdout.strip() == "ok"
