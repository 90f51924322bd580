"""The library's host code (argument checks, launch planning, workspace
layout, size and plan queries) built with AddressSanitizer and
UndefinedBehaviorSanitizer, and exercised on the CPU by
tests/sanitize/abi_driver.c over a grid of problem sizes, invalid
arguments and workspaces one byte short of the reported size. The
sanitizers instrument the host pass only (the device code is compiled as
usual and never runs), and the test program makes no call that reaches the GPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_draft_context_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"

sys.path.insert(0, ROOT)
from block_draft_context_amd.build import SOURCES  # noqa: E402

# host-side sanitizers only: each -fsanitize option applies to the host pass
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs hipcc and clang")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    procs = []
    objs = []
    for src in SOURCES:
        obj = str(tmp_path / (src + ".o"))
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
               "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        assert p.returncode == 0, f"{src}:\n{out[-3000:]}"
    lib = str(tmp_path / "libdspark_host_san.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN, *objs, "-o", lib],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    assert r.returncode == 0, r.stdout.decode(errors="replace")[-3000:]
    exe = str(tmp_path / "abi_driver")
    # the test program carries the sanitizer runtimes the library's host code calls into
    r = subprocess.run([CLANG, "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                        "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "sanitize", "abi_driver.c"),
                        lib, "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    assert r.returncode == 0, r.stdout.decode(errors="replace")[-3000:]
    env = dict(os.environ)
    # leaks inside the (uninstrumented) HIP runtime are not this library's;
    # no device is needed, and none is used
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["HIP_VISIBLE_DEVICES"] = "-1"
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, env=env, timeout=300)
    out = r.stdout.decode(errors="replace")
    print(out[-2000:])
    assert r.returncode == 0, out[-4000:]
    assert " 0 failures" in out
