"""The host library under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/sanitize/abi_sanitize.cpp is compiled with g++ together with the library's host source
(attn_api.cpp: validation, plans, workspace sizing, launch parameters); stub launchers stand
in for the kernels and check what each call hands them.  It runs the rejection matrix, the
launch-size limits, a sweep of valid plans and the kv_append / kv_keep / attn_merge calls, and
exits 0 only if every check held and no sanitizer reported an error.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_library_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "gqa_causal_attention_attn_amd", "csrc"),
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "gqa_causal_attention_attn_amd", "csrc", "attn_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "abi_sanitize.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(res.stdout, res.stderr)
    assert res.returncode == 0, res.stderr[-4000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr
    assert " 0 failed" in res.stdout
