"""The C ABI's host code under AddressSanitizer (CPU only).

``pkv_api.cpp`` (argument validation, workspace and scratch sizing, the
occupancy cache, the error text) is rebuilt with AddressSanitizer on its host
side only, linked with the library's ordinary device objects into a separate
``libpkv_asan.so``, and the ABI tests run against it in a child process with
the sanitizer runtime preloaded.  Any invalid host memory access aborts the
child and fails this test.  No GPU is touched: the ABI tests make no compute
calls.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "flashattention_paged_kv_amd", "csrc")


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return h if os.path.exists(h) else None


def test_abi_tests_pass_under_host_asan(tmp_path):
    hipcc = _hipcc()
    runtime = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if hipcc is None or not runtime:
        pytest.skip("hipcc or the clang AddressSanitizer runtime is not installed")
    from flashattention_paged_kv_amd import build as B
    flags = [f for f in B.HIPCC_FLAGS if f != "-O3"]
    objs = []
    for src in B.sources():
        obj = os.path.join(str(tmp_path), os.path.basename(src) + ".o")
        cmd = [hipcc, *flags, "-O1", "-g", "-c", src, "-o", obj]
        if src.endswith(".cpp"):
            # host code only: the sanitizer applies to the host side of this file
            cmd[1:1] = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
        objs.append((cmd, obj))
    procs = [subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True) for c, _ in objs]
    for p, (c, _) in zip(procs, objs):
        out, _ = p.communicate()
        assert p.returncode == 0, f"{' '.join(c)}\n{out}"
    lib = os.path.join(str(tmp_path), "libpkv_asan.so")
    link = [hipcc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address", "-o", lib,
            *[o for _, o in objs]]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join([runtime[-1]] + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else []))
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"  # the interpreter's own allocations are not ours
    env["PKV_LIBRARY"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "AddressSanitizer" not in out, out[-4000:]
    assert "passed" in out
