"""The host half of the library (block manager and work planners) under
AddressSanitizer and UndefinedBehaviorSanitizer: compiled with g++ into a
host-only library and driven by tests/host_sanitizer_driver.py in a child
process with the sanitizer runtime preloaded. Memory errors and undefined
behaviour abort the child (leak detection is off: the Python interpreter's own
allocations would drown it)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_162_amd", "csrc")


def _runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no AddressSanitizer runtime")
    lib = str(tmp_path / "libpagedkv_host_sanitized.so")
    # the prefill plan asks the prefill kernel's file for its rows per item; the
    # host-only build gets the header's formula, 8 * (16 / G) for G <= 16
    stub = tmp_path / "rows_per_item.cpp"
    stub.write_text('#include "pagedkv.h"\n'
                    'extern "C" int32_t kv_paged_attention_prefill_rows_per_item(int32_t hq, '
                    'int32_t hkv) {\n'
                    '  if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || hq / hkv > 16) return 0;\n'
                    '  return 8 * (16 / (hq / hkv));\n}\n')
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra",
           "-Werror", "-fPIC", "-shared", "-I", os.path.join(ROOT, "include"), "-o", lib,
           os.path.join(CSRC, "host_pool.cpp"), os.path.join(CSRC, "plan.cpp"), str(stub)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "host_sanitizer_driver.py"),
                          lib, "120", "162"], capture_output=True, text=True, env=env,
                         timeout=600)
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-6000:]
    assert run.stdout.startswith("ok:"), run.stdout
