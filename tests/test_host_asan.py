"""Host-side AddressSanitizer run (CPU): the library's host code (argument checks, launch plans, workspace sizing,
the status strings) built with -fsanitize=address for the host pass only, then the ABI tests run against it in a
child process with the sanitizer runtime preloaded.  Device code is compiled as usual and never launched here.
"""
import os
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "fp4_sparse_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.hip", "pack.hip", "index.hip", "topk.hip", "attention.hip", "absorb.hip"]


def _asan_runtime():
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin", "clang")
    for c in (clang, "/opt/rocm/llvm/bin/clang"):
        if os.path.exists(c):
            p = subprocess.run([c, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
            path = p.stdout.strip()
            if p.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    return None


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_checks_under_host_address_sanitizer():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime next to the compiler")
    with tempfile.TemporaryDirectory() as d:
        flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                 "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-I", os.path.join(ROOT, "include")]
        procs = [subprocess.Popen([HIPCC, *flags, "-c", os.path.join(CSRC, s), "-o", os.path.join(d, s + ".o")],
                                  stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True) for s in SOURCES]
        for p in procs:
            out, _ = p.communicate()
            assert p.returncode == 0, out
        lib = os.path.join(d, "libcsa2_asan.so")
        r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                            "-o", lib, *[os.path.join(d, s + ".o") for s in SOURCES]],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr
        code = ("import sys; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
                "import fp4_sparse_attention_amd as F\n"
                "F.LIB_PATH = %r\n"
                "import pytest\n"
                "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r]))\n"
                % (ROOT, HERE, lib, os.path.join(HERE, "test_abi.py")))
        env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=d, timeout=600)
        assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
        assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr
