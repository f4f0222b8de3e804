"""The C-ABI host layer under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

api.hip (argument validation, workspace sizing and layout, split plans) is built with host-side
sanitizers (device code unsanitized) together with host stubs of the kernel launchers
(host_sanitize/launch_stubs.cpp, which check each launch descriptor the way the kernels rely on
it), and host_sanitize/abi_cases.cpp drives every entry point through bad arguments, exact and
one-byte-short workspaces and a sweep of shapes up to the largest accepted sizes."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CSRC = os.path.join(ROOT, "long_context_sparse_oracle_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_layer_clean_under_asan_and_ubsan(tmp_path):
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    exe = str(tmp_path / "abi_cases")
    objs = []
    for src in (os.path.join(CSRC, "api.hip"), os.path.join(HERE, "launch_stubs.cpp"),
                os.path.join(HERE, "abi_cases.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        subprocess.run([HIPCC, *common, *san, *lang, "-c", src, "-o", obj], check=True, capture_output=True)
        objs.append(obj)
    subprocess.run([HIPCC, "--offload-arch=gfx950", *san, *objs, "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "0 failed" in r.stdout
