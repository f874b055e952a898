"""The C ABI's host code under AddressSanitizer (no GPU needed).

libgdn is rebuilt with the sanitizer on its host code only (`-Xarch_host`
before each `-fsanitize=`: the device code is built as usual), and a C driver
(`tests/asan/abi_driver.c`) calls every entry point on the paths that end
before a kernel launch: validation, workspace sizing, status strings, the
thread-local error message, the debug-record accessor and malformed values
of the GDN_CHECK and GDN_DEBUG_DUMP switches.  A memory error aborts the
driver with the sanitizer's report."""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, os.path.join(ROOT, "gated_deltanet_rule_amd"))
import build as gdn_build  # noqa: E402

ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _clang():
    for cand in ("/opt/rocm/llvm/bin/clang", "/opt/rocm/lib/llvm/bin/clang"):
        if os.path.exists(cand):
            return cand
    pytest.skip("ROCm clang not found")


@pytest.mark.timeout(900)
def test_abi_host_paths_under_address_sanitizer(tmp_path):
    hipcc = gdn_build.hipcc()
    common = [x for x in gdn_build.COMMON if x != "-O3"] + ["-O1"]

    def comp(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc] + common + ASAN + lang + ["-c", os.path.join(gdn_build.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(len(gdn_build.SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(comp, gdn_build.SOURCES))
    lib = str(tmp_path / "libgdn_asan.so")
    r = subprocess.run([hipcc, f"--offload-arch={gdn_build.ARCH}", "-shared", "-fPIC", "-shared-libasan"] + ASAN
                       + ["-o", lib] + objs, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    exe = str(tmp_path / "abi_driver")
    # the sanitizer's shared runtime sits in the compiler's resource directory
    rt = subprocess.run([_clang(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    r = subprocess.run([_clang(), "-std=c99", "-O1", "-g", "-fsanitize=address", "-shared-libasan",
                        "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "asan", "abi_driver.c"),
                        lib, f"-Wl,-rpath,{tmp_path}", f"-Wl,-rpath,{os.path.dirname(rt)}", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    assert "all host paths as expected" in r.stdout
