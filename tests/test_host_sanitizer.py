"""The library's host code under AddressSanitizer (CPU only).

Builds a copy of liblapattn.so with the host side of every source compiled
with -fsanitize=address (device code unchanged) into a temporary directory,
links tests/host/abi_check.c against it, and runs it: version and error
strings, argument checks, workspace sizing and the launch plan for the
workloads' shapes, and every argument error of the forward, none of which
does device work.  Any heap or stack misuse in that host code aborts the run.
"""
import os
import shlex
import shutil
import subprocess

import pytest

from nystr_linear_attention_amd import build as libbuild

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CLANG = "/opt/rocm/llvm/bin/clang"

# sanitizer flags for the host pass only: each -fsanitize= directly after
# -Xarch_host, so that no GPU code is built with it
HOST_ASAN = shlex.split("-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer")


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not found")
def test_host_abi_under_address_sanitizer(tmp_path):
    lib_dir = tmp_path / "lib"
    lib_dir.mkdir()
    lib = libbuild.build(extra=HOST_ASAN, link_extra=HOST_ASAN, out=str(lib_dir / "liblapattn.so"))
    exe = str(tmp_path / "abi_check")
    subprocess.run([CLANG, "-fsanitize=address", "-fno-omit-frame-pointer", "-g", "-O1",
                    f"-I{os.path.join(ROOT, 'include')}", os.path.join(HERE, "host", "abi_check.c"),
                    f"-L{lib_dir}", "-llapattn", f"-Wl,-rpath,{lib_dir}", "-lm", "-o", exe],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ)
    # the HIP runtime's own allocations outlive main; leaks are not the point
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "host ABI checks passed" in res.stdout
    assert "AddressSanitizer" not in res.stderr, res.stderr
    assert os.path.exists(lib)
