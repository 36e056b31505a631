"""The host code of the C ABI (argument checks, work-table and tile-index building)
built with AddressSanitizer and UndefinedBehaviorSanitizer on the host side only
(device code unchanged), and the host ABI tests run against that build in a child
process.  Runs without a GPU: every call fails validation, or reaches the first HIP
call after building its tables and returns ADA_EHIP."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from weight_merge_amd import build  # noqa: E402

ASAN_RT = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))

try:
    import torch

    _gpu = torch.cuda.is_available()
except Exception:  # pragma: no cover
    _gpu = False


@pytest.mark.skipif(not ASAN_RT, reason="clang's AddressSanitizer runtime is not installed")
@pytest.mark.skipif(_gpu, reason="the host ABI tests pass fake pointers: run where no GPU is visible")
def test_host_abi_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    lib = str(tmp_path / "libadafuse_san.so")
    host_only = []
    for f in ("address", "undefined"):
        host_only += ["-Xarch_host", f"-fsanitize={f}"]
    host_only += ["-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [build.HIPCC, *build.FLAGS, *host_only, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(build.PKG, "csrc"), *build.sources(), "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms, "the host code was not instrumented"
    driver = (
        "import sys, pytest\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "from weight_merge_amd import _lib\n"
        f"_lib.LIB_PATH = {lib!r}\n"
        f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', {os.path.join(ROOT, 'tests', 'test_abi_host.py')!r}]))\n"
    )
    env = dict(os.environ, LD_PRELOAD=ASAN_RT[-1], ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([sys.executable, "-c", driver], capture_output=True, text=True, env=env, timeout=600)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
