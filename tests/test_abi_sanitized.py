"""The host side of libcsa (argument checks, workspace sizing) under
AddressSanitizer and UndefinedBehaviorSanitizer.  The library is rebuilt with
the sanitizers on its host code only (the device code is compiled as usual),
loaded into a fresh interpreter with the ASan runtime preloaded, and runs the
host-only ABI tests (tests/test_abi_cpu.py, no GPU calls); any sanitizer
report fails the test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
# sanitizers on the host compilation only; each flag behind -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="needs the ROCm toolchain")
def test_host_checks_clean_under_asan_and_ubsan(tmp_path):
    srcs = sorted(glob.glob(os.path.join(ROOT, "long_context_sparse_10_amd", "csrc", "*.hip")))
    procs = []
    for s in srcs:
        obj = str(tmp_path / (os.path.basename(s)[:-4] + ".o"))
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
               "-I", os.path.join(ROOT, "include"), "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", *HOST_SAN, "-c", s, "-o", obj]
        procs.append((s, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                               stderr=subprocess.STDOUT, text=True)))
    objs = []
    for s, obj, p in procs:
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, f"{s}:\n{out[-3000:]}"
        objs.append(obj)
    lib = str(tmp_path / "libcsa_sanitized.so")
    link = [CLANG, "-shared", "-fsanitize=address,undefined", *objs, "-L/opt/rocm/lib",
            "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", lib]
    subprocess.run(link, check=True, capture_output=True, timeout=300)
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], check=True,
                        capture_output=True, text=True).stdout.strip()
    assert os.path.exists(rt), rt
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import sys; sys.path.insert(0, {root!r}); "
            "from long_context_sparse_10_amd import _lib as C; C.LIB_PATH = {lib!r}; "
            "import pytest; sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', "
            "{test!r}]))").format(root=ROOT, lib=lib,
                                  test=os.path.join(ROOT, "tests", "test_abi_cpu.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    log = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, log
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, log
    assert " passed" in r.stdout, log
