"""The host runtime under AddressSanitizer and UndefinedBehaviorSanitizer.

libtl_asan.so is libtl.so with its host engine (argument checks, the staging area,
the KV arena allocator, descriptors, graph capture) built by g++ with
-fsanitize=address,undefined and linked with the ordinary HIP objects.  Each test
runs other test files in a child process that preloads the sanitizer runtimes and
loads that build through TL_LIBRARY, and fails on any sanitizer report.
"""
import importlib.util
import os
import subprocess
import sys

import pytest

from looped_transformer_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_sanitized(test_args, timeout):
    rt = b.sanitizer_runtimes()
    if not rt:
        pytest.skip("g++'s sanitizer runtimes are not installed")
    if not os.path.exists(b.LIB_ASAN):
        pytest.skip("libtl_asan.so is not built (__graft_entry__.build() builds it)")
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join(rt) + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    # leak checks would report the Python interpreter's and HIP runtime's own
    # process-lifetime allocations; the runtime is not first in the preload order
    # when the environment preloads another library
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    env["TL_LIBRARY"] = b.LIB_ASAN
    # the sanitizer's dlopen interceptor hides its callers' run paths, so the
    # libraries torch opens by name at run time are found through the search path
    spec = importlib.util.find_spec("torch")
    if spec and spec.origin:
        tlib = os.path.join(os.path.dirname(spec.origin), "lib")
        env["LD_LIBRARY_PATH"] = tlib + (":" + env["LD_LIBRARY_PATH"] if env.get("LD_LIBRARY_PATH") else "")
    # the child really runs the sanitized build under the sanitizer runtime
    probe = ("import looped_transformer_amd as tl; tl.lib(); m = open('/proc/self/maps').read(); "
             "print('libtl_asan.so' in m and 'libasan.so' in m and 'libtl.so' not in m)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.stdout.strip().endswith("True"), r.stdout + r.stderr
    cmd = [sys.executable, "-u", "-m", "pytest", "-q", "-p", "no:cacheprovider", *test_args]
    print("[sanitizer] running", " ".join(test_args), flush=True)
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    out = r.stdout + r.stderr
    print(out[-3000:], flush=True)
    assert "ERROR: AddressSanitizer" not in out
    assert "runtime error:" not in out, "UndefinedBehaviorSanitizer report"
    assert r.returncode == 0
    assert "passed" in out


def test_abi_checks_under_sanitizers():
    """Argument validation, error strings and the no-allocation entry point's
    argument checks through the C ABI (no device needed)."""
    _run_sanitized(["tests/test_abi_cpu.py", "-m", "not gpu"], timeout=600)


@pytest.mark.gpu
@pytest.mark.timeout(900)
def test_device_paths_under_sanitizers():
    """Load, scoring forwards and their graph replay, cached decode with early exit
    and in every cache mode, lane forks and appends, speculative rounds, the
    no-allocation decode step, allocator failures and stream changes on the
    device, with the host engine sanitized."""
    _run_sanitized(["tests/test_gpu_errors.py", "tests/test_gpu_prefix.py", "tests/test_gpu_speculate.py",
                    "tests/test_gpu_early_exit.py", "tests/test_gpu_store_h.py", "tests/test_zz_no_alloc.py",
                    "tests/test_gpu_parity.py::test_graph_replay_matches_eager", "-m", "gpu",
                    "--timeout", "300", "--timeout-method", "thread"], timeout=900)
