"""The CPU tests of the oracle and of the C ABI's argument checks, run again with the
oracle and the library's host code built with AddressSanitizer and
UndefinedBehaviorSanitizer (clang's runtime, preloaded into a child interpreter).
Every check in test_abi.py fails validation before any launch, so no GPU is needed;
an out-of-bounds access or undefined behaviour in the host code or the oracle on
those paths ends the child with a sanitizer report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
SUITE = ["tests/test_abi.py", "tests/test_oracle_formats.py", "tests/test_oracle_compress.py",
         "tests/test_oracle_select_attend.py", "tests/test_oracle_pool.py", "tests/test_golden.py"]


def _asan_runtime():
    if not os.path.exists(CLANG):
        return None
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True)
    p = r.stdout.strip()
    return p if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    import oracle
    from compressed_sparse_attention_csa2_amd import _build
    d = tmp_path_factory.mktemp("sanitized")
    orc = oracle.build_sanitized(str(d / "libcsa2oracle.so"), cc=CLANG)
    lib = _build.build_host_sanitized(str(d / "libcsa2.so"))
    return rt, orc, lib


def _imports(path):
    r = subprocess.run(["nm", "-D", "--undefined-only", path], capture_output=True, text=True,
                       check=True)
    return r.stdout


def test_builds_are_instrumented(sanitized):
    _, orc, lib = sanitized
    for p in (orc, lib):
        syms = _imports(p)
        assert "__asan_report_" in syms, p
        assert "__ubsan_handle_" in syms, p


def test_cpu_suite_under_sanitizers(sanitized):
    rt, orc, lib = sanitized
    env = dict(os.environ)
    # the sanitizer runtime must come first among preloaded libraries
    env["LD_PRELOAD"] = rt + (" " + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["CSA2_LIB"] = lib
    env["CSA2_ORACLE_LIB"] = orc
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p",
                        "no:cacheprovider", *SUITE], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out and " failed" not in out, out[-2000:]
