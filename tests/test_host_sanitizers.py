"""The host-side argument validation of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

The library is rebuilt with the sanitizers on its host code only (device code
is compiled as usual and never runs here), and tests/test_abi_host.py runs
against that build in a child Python with the ASan runtime preloaded: every
call there returns before any HIP call, so this exercises exactly the host
checks (dims, sizes, alignment, workspace bounds) with bounds and overflow
checking.  A second test plants a heap overflow in a throw-away library built
with the same flags and checks that the same setup reports it, so a silently
inactive sanitizer cannot pass the first test.
"""
import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from mixture_experts_ffn_bias_amd import build as B  # noqa: E402

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _asan_runtime():
    hits = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) or _asan_runtime() is None,
                                reason="hipcc or the ASan runtime is not installed")


def _flags():
    f = [x for x in B.FLAGS if x != "-O3"]
    return f + ["-O1", "-g"] + SAN


def _env():
    env = dict(os.environ)
    env["LD_PRELOAD"] = _asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stderr[-3000:]


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("asan_build")
    objs = []
    cmds = []
    for s in B.SOURCES:
        o = str(d / s.replace(".hip", ".o"))
        objs.append(o)
        cmds.append([HIPCC, *_flags(), "-c", os.path.join(B.CSRC, s), "-o", o])
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(_run, cmds))
    lib = str(d / "libmoe_asan.so")
    _run([HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libsan", *SAN[:4], "-o", lib, *objs])
    return lib


RUNNER = """
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import mixture_experts_ffn_bias_amd._binding as b
b.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {target!r}]))
"""


def test_abi_host_checks_under_asan_and_ubsan(sanitized_lib):
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=sanitized_lib,
                         target=os.path.join(ROOT, "tests", "test_abi_host.py"))
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=_env(), timeout=600)
    out = p.stdout + p.stderr
    print(out[-1500:])
    assert "AddressSanitizer" not in out and "runtime error" not in out
    assert p.returncode == 0
    assert " passed" in p.stdout


PLANTED = r"""
#include <cstdlib>
extern "C" int planted_overflow(int n) {
  int* a = (int*)malloc(n * sizeof(int));
  for (int i = 0; i < n; ++i) a[i] = i;
  int s = a[n];  // one past the end
  free(a);
  return s;
}
"""


def test_the_same_setup_reports_a_planted_heap_overflow(tmp_path):
    src = tmp_path / "planted.hip"
    src.write_text(PLANTED)
    lib = str(tmp_path / "libplanted.so")
    _run([HIPCC, *_flags(), "-shared", "-fPIC", "-shared-libsan", str(src), "-o", lib])
    code = f"import ctypes; ctypes.CDLL({lib!r}).planted_overflow(8)"
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=_env(), timeout=120)
    assert p.returncode != 0
    assert "heap-buffer-overflow" in p.stderr
